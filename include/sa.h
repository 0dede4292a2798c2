/*
 * sa.h - C ABI of libsa, clustered block-sparse attention on MI355X (gfx950).
 *
 * The operation (per attention head) is the training-free sparse attention
 * described by
 *   [SCOPE]  "SCOPE: Subspace Clustering with Online Per-Head Top-K Estimation
 *            for Sparse Video Attention" (arXiv 2608.12780): English abstract,
 *            technical framework and key design sections;
 *   [CA]     "ClusterAttention: A training-free speedup of bidirectional
 *            attention" (arXiv 2608.26965): English and Chinese abstracts.
 * Post-RoPE queries and keys are clustered and permuted into contiguous
 * cluster order; centroid proxy scores drive a hybrid Top-p / minimum Top-k
 * choice of key clusters for every query cluster, with SCOPE's online per-head
 * Top-k; attention then runs over the selected original keys/values only,
 * optionally compensating each excluded key cluster through its mean [CA].
 *
 * Conventions for every entry point:
 *  - Tensors are row-major [heads, n, d] with token n = (t*height + h)*width + w.
 *  - All tensor pointers are DEVICE pointers, allocated and owned by the
 *    caller.  The library never allocates, frees or retains a pointer after a
 *    call returns.  Inputs are never modified.
 *  - Scratch memory is one caller-provided device workspace of at least
 *    sa_workspace_size() bytes (256-byte aligned).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues kernels on it: no device->host copy, no synchronisation.
 *    Calls on distinct workspaces are reentrant.  One exception to "only on
 *    `stream`": when Q and K are clustered with different settings,
 *    sa_cluster_qk and sa_forward enqueue K's clustering on a second stream
 *    of the current device (default priority; created with two events by the
 *    first such call on that device, kept until the process ends), ordered
 *    after the work already on `stream` and joined back to it by events, so
 *    everything enqueued on `stream` afterwards follows it.  A graph capture
 *    of `stream` captures both; make the first such call outside a capture.
 *  - Arguments are validated before anything is enqueued: a call that
 *    returns an error has done no work.  SA_ERR_HIP reports a launch failure
 *    (hipGetLastError after a launch).  No C++ exception crosses the ABI.
 *  - Results are deterministic: identical inputs give bit-identical outputs
 *    (no floating-point atomics anywhere).
 */
#ifndef SA_H_
#define SA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define SA_API __attribute__((visibility("default")))
#else
#define SA_API
#endif

typedef enum sa_status {
  SA_OK = 0,
  SA_ERR_INVALID_ARG = 1, /* null pointer, bad config value */
  SA_ERR_SHAPE = 2,       /* n != frames*height*width, unsupported d, too many clusters */
  SA_ERR_DTYPE = 3,       /* dtype not SA_F32 / SA_BF16 */
  SA_ERR_WORKSPACE = 4,   /* workspace smaller than sa_workspace_size() */
  SA_ERR_UNSUPPORTED = 5, /* valid but not implemented combination */
  SA_ERR_HIP = 6          /* a kernel launch failed */
} sa_status;

enum { SA_F32 = 0, SA_BF16 = 1 };

/* Clustering methods.
 * SA_KMEANS:   Lloyd k-means, `clusters` centroids seeded with the first
 *              `clusters` tokens (or caller centroids), `iters` rounds of
 *              assignment + update.
 * SA_BISECT:   balanced recursive 2-means down to leaves of `leaf` tokens
 *              (all leaves full except the last) [CA: recursive clustering,
 *              power-of-two cluster sizes].  C = ceil(n / leaf).
 * SA_SUBSPACE: keys only [SCOPE]: the t/h/w RoPE column slices (`sub_dims`)
 *              are k-means clustered independently with `clusters` centroids
 *              each; a key's cluster is its combo
 *              g = (a_t*clusters + a_h)*clusters + a_w, C = clusters^3.
 * SA_RASTER:   no clustering ["VMoBA: Mixture-of-Block Attention for Video
 *              Diffusion Models", English abstract, item (1): a 1D-2D-3D
 *              block partition]: the frames x height x width grid is cut
 *              into boxes of sub_dims = (bt, bh, bw) tokens (edge boxes keep
 *              what remains), numbered in raster order of their block
 *              coordinates; 1D = (bt, height, width), 2D = (frames, bh, bw),
 *              3D = cubes.  C = ceil(F/bt)*ceil(H/bh)*ceil(W/bw). */
enum { SA_KMEANS = 0, SA_BISECT = 1, SA_SUBSPACE = 2, SA_RASTER = 3 };
enum { SA_INIT_FIRST = 0, SA_INIT_GIVEN = 1 };

/* Size limits (SA_ERR_SHAPE otherwise): n <= 2^24, heads*n <= 2^31, and one
 * head's rows of a tensor, n*d*(2 for bf16, 4 for f32) bytes, below 4 GiB
 * (kernels address them with 32-bit byte offsets; bf16 at d = 128: n < 2^24). */
typedef struct sa_problem {
  int32_t heads, n, d;            /* d in {64, 128}                                 */
  int32_t frames, height, width;  /* n == frames*height*width; (1,1,n) unstructured */
  int32_t dtype;                  /* SA_F32 or SA_BF16 (Q, K, V and O)              */
} sa_problem;

typedef struct sa_cluster_cfg {
  int32_t method;      /* SA_KMEANS | SA_BISECT | SA_SUBSPACE | SA_RASTER           */
  int32_t clusters;    /* KMEANS: C (1..1024, <= n); SUBSPACE: per-slice C (<= 32)  */
  int32_t leaf;        /* BISECT leaf size (>= 4)                                   */
  int32_t tile_cap;    /* upper bound on query rows per attention tile (tiling
                          only, never changes results; 0 = 128)                    */
  int32_t iters;       /* rounds per k-means run / per bisection node (>= 1)        */
  int32_t init;        /* KMEANS / SUBSPACE: SA_INIT_FIRST, or SA_INIT_GIVEN = start
                          from the centroids already in out->centroids (SUBSPACE:
                          the expanded [3*clusters, d] layout below)               */
  int32_t sub_dims[3]; /* SUBSPACE column widths (t, h, w), summing to d;
                          RASTER block extents (bt, bh, bw)                        */
} sa_cluster_cfg;

/* Competition domains of the selection.
 * SA_DOMAIN_ROW:   every query cluster selects among its own units (the
 *                  hybrid Top-p rule above).
 * SA_DOMAIN_HEAD:  VMoBA global block selection ["VMoBA: Mixture-of-Block
 *                  Attention for Video Diffusion Models", English abstract,
 *                  item (2)]: the (query cluster, key cluster) pairs of a
 *                  whole head compete for one Top-p.
 * SA_DOMAIN_GROUP: EG-Sparse ["Competition Domains Matter: Selective Head
 *                  Globalization for Training-Free Sparse Attention in Video
 *                  Diffusion Transformers", abstract]: heads are cut into
 *                  groups of `group` consecutive heads; the heads of a group
 *                  whose entropy is below `max_entropy` share one pool, the
 *                  others select per row.
 * A pool's pairs compete by proxy probability p_ij (descending; ties by head,
 * row, unit), each with mass |Q_i| p_ij / n; the pool keeps the shortest
 * prefix whose mass reaches top_p times its number of heads, which gives each
 * query cluster its Top-p count; the floor and the online Top-k then apply
 * per row as above.  A head's entropy is the query-size-weighted mean of its
 * rows' proxy entropies divided by ln(number of non-empty units), in [0, 1].
 * Key clusters only (SUBSPACE keys: SA_ERR_UNSUPPORTED). */
enum { SA_DOMAIN_ROW = 0, SA_DOMAIN_HEAD = 1, SA_DOMAIN_GROUP = 2 };

/* Rule of a row's initial selection.
 * SA_RULE_TOP_P: the shortest prefix whose proxy mass reaches top_p.
 * SA_RULE_STAT:  BSA's statistical dynamic threshold ["Bidirectional Sparse
 *                Attention for Faster Video Diffusion Training", abstract]:
 *                the units whose proxy probability is at least the row's
 *                mean plus stat_lambda population standard deviations (over
 *                its non-empty units); top_p is ignored, the floor (>= 1) and
 *                the online Top-k apply as with Top-p.  SA_DOMAIN_ROW and key
 *                clusters only. */
enum { SA_RULE_TOP_P = 0, SA_RULE_STAT = 1 };

typedef struct sa_select_cfg {
  double top_p;         /* cumulative proxy mass to reach (>= 1: all non-empty);
                           double, so a configured 0.9 is compared as 0.9      */
  int32_t topk_floor;   /* fixed Top-k minimum in units (clusters; keys in
                           SUBSPACE mode); top_p <= 0 with floor <= 0 is invalid */
  int32_t online_topk;  /* SCOPE online per-head Top-k on/off                    */
  int32_t size_weighted;/* 1: proxy logits add ln|K_j| (softmax over per-key
                           scores); 0: plain centroid softmax                    */
  int32_t domain;       /* SA_DOMAIN_ROW (0, default), _HEAD or _GROUP          */
  int32_t group;        /* SA_DOMAIN_GROUP: heads per group (>= 1)              */
  double max_entropy;   /* SA_DOMAIN_GROUP: heads below it are pooled           */
  int32_t rule;         /* SA_RULE_TOP_P (0, default) or SA_RULE_STAT           */
  double stat_lambda;   /* SA_RULE_STAT: standard deviations above the mean     */
} sa_select_cfg;

typedef struct sa_attn_cfg {
  int32_t compensate;  /* mean compensation of excluded key clusters [CA] */
  float scale;         /* score scale; 0 = 1/sqrt(d)                      */
  /* Optional timing events (hipEvent_t passed as void*, created and owned by
   * the caller), or both NULL.  When set, this call records ev_start on its
   * stream right before the attention kernels and ev_stop right after them
   * (the call's preparation kernels and, in sa_forward, clustering and
   * selection fall outside), so hipEventElapsedTime(ev_start, ev_stop) is
   * the attention kernels' duration.  Only this call records on them.  One
   * NULL with one non-NULL is SA_ERR_INVALID_ARG. */
  void* ev_start;
  void* ev_stop;
  /* Optional output, or NULL: float [H, n] in the original token order, the
   * natural-log normaliser of each query's attention (the log of the
   * softmax denominator over its selected keys' scaled scores, plus the
   * compensation terms log|K_j| + <q, kbar_j> scale when compensate is on;
   * -inf for a query with nothing to attend).  Written by
   * sa_block_sparse_attn, its allocation-free form and sa_forward; the
   * backward takes it (from a forward without compensation) instead of
   * recomputing it. */
  void* lse;
} sa_attn_cfg;

/* Clustering of one tensor (Q or K).  Every pointer is caller-owned device
 * memory, written by sa_cluster and read by sa_select/sa_block_sparse_attn.
 *   labels    int32 [H, n]      cluster of each token (original order)
 *   perm      int32 [H, n]      perm[h][p] = original token at cluster-order
 *                               position p (ascending inside a cluster)
 *   offsets   int32 [H, C+1]    cluster c occupies positions [off[c], off[c+1])
 *   centroids f32   [H, Cc, d]  KMEANS/BISECT: Cc = C member means (an empty
 *                               k-means cluster keeps its previous centroid);
 *                               SUBSPACE: Cc = 3*clusters slice centroids, row
 *                               s*clusters+c holds slice s in its own columns
 *                               and zeros elsewhere
 *   x_perm    dtype [H, n, d]   rows of x in cluster order
 * num_clusters, method, sub_clusters and sub_dims are filled by sa_cluster. */
typedef struct sa_clusters {
  int32_t* labels;
  int32_t* perm;
  int32_t* offsets;
  float* centroids;
  void* x_perm;
  int32_t num_clusters;
  int32_t method;
  int32_t sub_clusters;
  int32_t sub_dims[3];
} sa_clusters;

/* Number of clusters C a configuration produces (BISECT: ceil(n/leaf);
 * SUBSPACE: clusters^3), or -1 for an invalid configuration. */
SA_API int32_t sa_num_clusters(const sa_problem* p, const sa_cluster_cfg* cfg);

/* Workspace bytes sufficient for sa_forward with these configurations and
 * for each component call (sa_cluster with qcfg or kcfg, sa_select,
 * sa_block_sparse_attn) on the same problem.  Any cfg may be NULL
 * only if the matching component is never called with that workspace. */
SA_API sa_status sa_workspace_size(const sa_problem* p, const sa_cluster_cfg* qcfg,
                                   const sa_cluster_cfg* kcfg, const sa_select_cfg* scfg,
                                   const sa_attn_cfg* acfg, size_t* bytes);

/* Cluster x [H, n, d] per head with `cfg` and permute it into cluster order
 * [SCOPE technical framework: clustering of post-RoPE keys; CA: recursive
 * power-of-two clustering].  Fills every field of *out. */
SA_API sa_status sa_cluster(const sa_problem* p, const sa_cluster_cfg* cfg, const void* x,
                            sa_clusters* out, void* ws, size_t ws_bytes, void* stream);

/* Cluster Q with qcfg and K with kcfg, exactly as two sa_cluster calls would
 * (bit-identical results), as sa_forward does.  When both use BISECT with
 * the same leaf and iters, the two tensors are bisected together as one
 * problem of 2H heads, so every kernel launch covers both; otherwise K's
 * clustering runs beside Q's on the device's second stream (see the stream
 * convention above), each in its own part of the workspace.  Workspace: as
 * returned by sa_workspace_size with both configurations. */
SA_API sa_status sa_cluster_qk(const sa_problem* p, const sa_cluster_cfg* qcfg,
                               const sa_cluster_cfg* kcfg, const void* q, const void* k,
                               sa_clusters* qout, sa_clusters* kout, void* ws, size_t ws_bytes,
                               void* stream);

/* Gather rows of x [H, n, d] into the cluster order of `c` (x_perm) and, if
 * `means` is not NULL, write the member mean of every cluster to means
 * f32 [H, C, d] (zeros for an empty cluster).  Used for V (the compensation
 * of [CA] needs the mean value of every key cluster).  Needs no workspace. */
SA_API sa_status sa_permute(const sa_problem* p, const sa_clusters* c, const void* x,
                            void* x_perm, float* means, void* stream);

/* Hybrid Top-p / fixed Top-k selection with SCOPE's online per-head Top-k.
 * For each query cluster i: logits l_ij = <qbar_i, kbar_j>*scale (+ ln|K_j|),
 * p_ij = softmax_j over non-empty key units, ranking by (p desc, j asc); the
 * initial prefix is the shortest reaching mass >= top_p and count >= floor
 * (n_i units); with online Top-k, k_h = ceil(sum_i |Q_i| n_i / n) and rows
 * with n_i < k_h extend along the same ranking to k_h units.  SUBSPACE keys
 * use SCOPE's lookup-table scores over combos (units = keys).
 *   mask        uint32 [H, Cq, ceil(Ck/32)]  bit j of row (h,i), LSB first
 *   counts      int32  [H, Cq]  final selected units
 *   init_counts int32  [H, Cq]  initial units n_i (may be NULL)
 *   head_topk   int32  [H]      k_h (0 when online Top-k is off)
 *   head_entropy f64   [H]      entropy of each head's proxy attention (may be
 *                               NULL; written only when cfg->domain is not
 *                               SA_DOMAIN_ROW)
 * `scale` of the proxy scores is 1/sqrt(d). */
SA_API sa_status sa_select(const sa_problem* p, const sa_select_cfg* cfg, const sa_clusters* q,
                           const sa_clusters* k, uint32_t* mask, int32_t* counts,
                           int32_t* init_counts, int32_t* head_topk, double* head_entropy, void* ws,
                           size_t ws_bytes, void* stream);

/* Block-sparse attention [SCOPE: attention over the selected original keys
 * and values; CA: block-sparse attention over power-of-two clusters, mean
 * compensation].  For a query token n of query cluster i:
 *   O_n = [sum_{m in sel} e^{s_nm} v_m + c sum_{j excl} |K_j| e^{<q_n,kbar_j>s} vbar_j]
 *       / [sum_{m in sel} e^{s_nm}     + c sum_{j excl} |K_j| e^{<q_n,kbar_j>s}]
 * with s_nm = <q_n, k_m>*scale, sel = keys of the key clusters set in mask row
 * i, excl = non-empty key clusters not set, c = cfg->compensate.
 *   v_perm  dtype [H, n, d]  V rows in the key cluster order of k
 *   v_means f32 [H, Ck, d]   member means of V per key cluster (compensation
 *                            only; NULL otherwise)
 *   o       dtype [H, n, d]  output in ORIGINAL token order
 * Compensation is not supported for SUBSPACE keys (SA_ERR_UNSUPPORTED). */
SA_API sa_status sa_block_sparse_attn(const sa_problem* p, const sa_attn_cfg* cfg,
                                      const sa_clusters* q, const sa_clusters* k,
                                      const void* v_perm, const float* v_means,
                                      const uint32_t* mask, void* o, void* ws, size_t ws_bytes,
                                      void* stream);

/* Bytes of the library-owned scratch of sa_block_sparse_attn_noalloc (one
 * array per GPU, held from library load until the process ends). */
#define SA_NOALLOC_ATTN_SCRATCH_BYTES (128u << 20)

/* sa_block_sparse_attn for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): same arguments, same kernels and bit-identical results, but
 * the scratch comes from a fixed array inside the library (the GPU's own
 * copy, SA_NOALLOC_ATTN_SCRATCH_BYTES) instead of a caller workspace.  The
 * caller still passes every input and output.  The call allocates and frees
 * nothing (no hipMalloc, no library allocation).  A problem whose attention
 * scratch exceeds the array (roughly H*Cq*(Ck/2+1)*8 bytes of range lists
 * plus, with compensation, 6*H*Ck*d bytes) returns SA_ERR_WORKSPACE before
 * any work.  Nothing in the array needs to start at zero: every call writes
 * what it reads.  All calls on one GPU share its array, so calls that can
 * overlap on one GPU (two streams, two threads) race: serialise them. */
SA_API sa_status sa_block_sparse_attn_noalloc(const sa_problem* p, const sa_attn_cfg* cfg,
                                              const sa_clusters* q, const sa_clusters* k,
                                              const void* v_perm, const float* v_means,
                                              const uint32_t* mask, void* o, void* stream);

/* Backward of sa_block_sparse_attn without compensation: the gradients of
 * Q, K and V for an output gradient dO, over the same selected key clusters
 * (the trainable use of block-sparse attention: "Bidirectional Sparse
 * Attention for Faster Video Diffusion Training", abstract; "VMoBA:
 * Mixture-of-Block Attention for Video Diffusion Models", English abstract).
 * With P_nm = softmax over the selected keys m of s_nm = <q_n, k_m> scale:
 *   dV_m = sum_n P_nm dO_n,  dS_nm = P_nm (<dO_n, v_m> - <dO_n, O_n>),
 *   dQ_n = scale sum_m dS_nm k_m,  dK_m = scale sum_n dS_nm q_n.
 *   q, k     clusters of sa_cluster (x_perm used), v_perm as for the forward
 *   mask     the selection the forward used
 *   o, d_o   bf16 [H, n, d] forward output and its gradient, original order
 *   lse      optional f32 [H, n]: the forward's normaliser (sa_attn_cfg.lse of
 *            the same forward, without compensation); NULL recomputes it
 *   dq, dk, dv  f32 [H, n, d] gradients, original order (every row written)
 * bf16 only (SA_ERR_DTYPE otherwise); compensation has no backward here.
 * Workspace: sa_block_sparse_attn_bwd_workspace_size() bytes. */
SA_API sa_status sa_block_sparse_attn_bwd_workspace_size(const sa_problem* p, int32_t q_clusters,
                                                         int32_t k_clusters, size_t* bytes);
SA_API sa_status sa_block_sparse_attn_bwd(const sa_problem* p, const sa_attn_cfg* cfg,
                                          const sa_clusters* q, const sa_clusters* k,
                                          const void* v_perm, const uint32_t* mask, const void* o,
                                          const void* d_o, const float* lse, float* dq, float* dk,
                                          float* dv, void* ws, size_t ws_bytes, void* stream);

/* The whole path: cluster Q and K, permute V, select, attend.
 * o dtype [H, n, d] original order; mask as in sa_select. */
SA_API sa_status sa_forward(const sa_problem* p, const sa_cluster_cfg* qcfg,
                            const sa_cluster_cfg* kcfg, const sa_select_cfg* scfg,
                            const sa_attn_cfg* acfg, const void* q, const void* k,
                            const void* v, void* o, uint32_t* mask, void* ws, size_t ws_bytes,
                            void* stream);

/* Static description of a status code. */
SA_API const char* sa_status_string(sa_status s);

#ifdef __cplusplus
}
#endif
#endif /* SA_H_ */
