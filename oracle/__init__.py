"""fp64 CPU oracle of clustered block-sparse attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the library.  It shares no code with the
HIP path.  See oracle/cbsa.py for the functions and the passages they follow.
"""

from .cbsa import (  # noqa: F401
    DOMAIN_GROUP,
    DOMAIN_HEAD,
    DOMAIN_ROW,
    NEAR_TIE_REL,
    SELECT_TIE_LOGIT_REL,
    SELECT_TIE_MASS,
    BisectNode,
    ClusterCfg,
    HeadResult,
    SelectCfg,
    attention,
    attention_backward,
    attention_lse,
    bisect,
    bisect_split,
    cluster_head,
    cluster_logits,
    cluster_means,
    dense_attention,
    domains,
    forward_head,
    head_entropy,
    kmeans,
    kmeans_assign,
    kmeans_update,
    permute,
    pool_counts,
    proxy_probs,
    raster_blocks,
    select,
    select_domains,
    stat_threshold,
    sq_dists,
    subspace_cluster,
    subspace_logits,
)
