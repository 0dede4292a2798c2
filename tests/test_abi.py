"""C ABI checks that need no GPU: the library loads, exports every entry
point include/sa.h declares, and rejects invalid arguments before doing any
work (validation touches no device)."""

import ctypes
import os
import re

import pytest

from clustered_block_sparse_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "sa.h")).read()
    return re.findall(r"SA_API\s+[\w\s\*]+?\b(sa_\w+)\s*\(", src)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libsa.so not built")
    return L.load()


def test_exports_every_declared_symbol(lib):
    names = declared_symbols()
    assert set(names) >= {"sa_cluster", "sa_cluster_qk", "sa_select", "sa_block_sparse_attn", "sa_forward",
                          "sa_workspace_size", "sa_status_string", "sa_permute", "sa_num_clusters"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert L.sa_status_string(0) == "ok"
    assert "workspace" in L.sa_status_string(4)
    assert L.sa_status_string(99) == "unknown status"


def test_num_clusters(lib):
    p = L.problem(40, 75600, 128, 21, 45, 80, "bf16")
    assert L.sa_num_clusters(p, L.cluster_cfg("bisect", leaf=128)) == 591
    assert L.sa_num_clusters(p, L.cluster_cfg("kmeans", clusters=64)) == 64
    assert L.sa_num_clusters(p, L.cluster_cfg("subspace", clusters=32, sub_dims=(32, 48, 48))) == 32768
    assert L.sa_num_clusters(p, L.cluster_cfg("subspace", clusters=32, sub_dims=(32, 48, 40))) == -1
    assert L.sa_num_clusters(p, L.cluster_cfg("kmeans", clusters=0)) == -1


def test_workspace_sizes(lib):
    p = L.problem(8, 10800, 128, 9, 30, 40, "bf16")
    q = L.cluster_cfg("kmeans", clusters=64)
    k = L.cluster_cfg("kmeans", clusters=128)
    s = L.select_cfg(0.95, 1, True)
    a = L.attn_cfg(False)
    full = L.sa_workspace_size(p, q, k, s, a)
    # at least the two permuted copies of Q and K plus V
    assert full >= 3 * 8 * 10800 * 128 * 2
    assert L.sa_workspace_size(p, q, k, s, L.attn_cfg(True)) > full
    assert L.sa_workspace_size(p, q) > 0


def call_cluster(lib, p, cfg, ws_bytes=1 << 30):
    out = L.Clusters(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, 0, (L.I32 * 3)(0, 0, 0))
    return lib.sa_cluster(ctypes.byref(p), ctypes.byref(cfg), FAKE, ctypes.byref(out), FAKE, ws_bytes, None)


def test_validation_before_work(lib):
    ok = L.problem(2, 256, 64, 4, 8, 8, "f32")
    km = L.cluster_cfg("kmeans", clusters=8)
    assert call_cluster(lib, L.problem(2, 256, 96, 4, 8, 8, "f32"), km) == 2       # d
    assert call_cluster(lib, L.problem(2, 256, 64, 4, 8, 9, "f32"), km) == 2       # n != F*H*W
    assert call_cluster(lib, L.problem(2, 256, 64, 4, 8, 8, 7), km) == 3           # dtype
    assert call_cluster(lib, ok, L.cluster_cfg("kmeans", clusters=300)) == 2       # C > n
    assert call_cluster(lib, ok, L.cluster_cfg("kmeans", clusters=8, iters=0)) == 1
    assert call_cluster(lib, ok, L.cluster_cfg("bisect", leaf=1)) == 1
    assert call_cluster(lib, ok, L.cluster_cfg("subspace", clusters=4, sub_dims=(16, 24, 20))) == 5
    assert call_cluster(lib, ok, km, ws_bytes=16) == 4                              # workspace
    # null pointers
    assert lib.sa_cluster(ctypes.byref(ok), ctypes.byref(km), None, None, FAKE, 1 << 30, None) == 1


def test_size_limits(lib):
    """n <= 2^24, heads*n <= 2^31, and one head's rows of a tensor below 4 GiB
    (32-bit byte offsets inside a head)."""
    km = L.cluster_cfg("kmeans", clusters=8)
    assert call_cluster(lib, L.problem(1, (1 << 24) + 64, 64, 1, 1, (1 << 24) + 64, "bf16"), km) == 2
    assert call_cluster(lib, L.problem(129, 1 << 24, 64, 1, 1, 1 << 24, "bf16"), km) == 2  # heads*n
    # bf16 d=128: 2^24 rows are exactly 4 GiB per head; one row fewer fits
    assert call_cluster(lib, L.problem(1, 1 << 24, 128, 1, 1, 1 << 24, "bf16"), km) == 2
    assert call_cluster(lib, L.problem(1, (1 << 24) - 1, 128, 1, 1, (1 << 24) - 1, "bf16"), km, 16) == 4
    # f32 d=128: the bound is 2^23 rows
    assert call_cluster(lib, L.problem(1, 1 << 23, 128, 1, 1, 1 << 23, "f32"), km) == 2
    assert call_cluster(lib, L.problem(1, (1 << 23) - 1, 128, 1, 1, (1 << 23) - 1, "f32"), km, 16) == 4
    assert call_cluster(lib, L.problem(1, 1 << 24, 64, 1, 1, 1 << 24, "bf16"), km, 16) == 4


def test_select_and_forward_validation(lib):
    p = L.problem(1, 256, 64, 4, 8, 8, "f32")
    km = L.cluster_cfg("kmeans", clusters=8)
    bad_sel = L.select_cfg(0.0, 0)
    a = L.attn_cfg(False)
    r = lib.sa_forward(ctypes.byref(p), ctypes.byref(km), ctypes.byref(km), ctypes.byref(bad_sel),
                       ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert r == 1
    good = L.select_cfg(0.9, 2)
    r = lib.sa_forward(ctypes.byref(p), ctypes.byref(km), ctypes.byref(km), ctypes.byref(good),
                       ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, None)
    assert r == 4
    sub = L.cluster_cfg("subspace", clusters=4, sub_dims=(16, 24, 24))
    r = lib.sa_forward(ctypes.byref(p), ctypes.byref(sub), ctypes.byref(km), ctypes.byref(good),
                       ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert r == 1  # subspace is for keys only


def test_attn_timing_events_come_in_pairs(lib):
    """The optional timing events of the attention configuration are both set
    or both null; one alone is rejected before any work."""
    p = L.problem(1, 256, 64, 4, 8, 8, "f32")
    km = L.cluster_cfg("kmeans", clusters=8)
    good = L.select_cfg(0.9, 2)
    for start, stop in ((FAKE, None), (None, FAKE)):
        a = L.AttnCfg(0, 0.0, start, stop)
        r = lib.sa_forward(ctypes.byref(p), ctypes.byref(km), ctypes.byref(km), ctypes.byref(good),
                           ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
        assert r == 1
        cl = L.Clusters(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 0, 0, (L.I32 * 3)(0, 0, 0))
        r = lib.sa_block_sparse_attn(ctypes.byref(p), ctypes.byref(a), ctypes.byref(cl), ctypes.byref(cl), FAKE,
                                     None, FAKE, FAKE, FAKE, 1 << 30, None)
        assert r == 1


def test_permute_validation(lib):
    p = L.problem(1, 256, 64, 4, 8, 8, "f32")
    cl = L.Clusters(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 0, 0, (L.I32 * 3)(0, 0, 0))
    assert lib.sa_permute(ctypes.byref(p), ctypes.byref(cl), None, FAKE, None, None) == 1
    assert lib.sa_permute(ctypes.byref(L.problem(1, 256, 96, 4, 8, 8, "f32")), ctypes.byref(cl), FAKE, FAKE,
                          None, None) == 2


def test_selection_rule_validation(lib):
    """Competition domains and the statistical threshold are validated before
    any work: unknown values, a group below one, a statistical rule without a
    floor or combined with a pooled domain, and either on subspace keys."""
    p = L.problem(1, 256, 64, 4, 8, 8, "f32")
    km = L.cluster_cfg("kmeans", clusters=8)
    a = L.attn_cfg(False)

    def fwd(sc, kc=km):
        return lib.sa_forward(ctypes.byref(p), ctypes.byref(km), ctypes.byref(kc), ctypes.byref(sc), ctypes.byref(a),
                              FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)

    assert fwd(L.select_cfg(0.9, 1, domain=7)) == 1
    assert fwd(L.select_cfg(0.9, 1, domain="group", group=0)) == 1
    assert fwd(L.select_cfg(0.9, 1, rule=5)) == 1
    assert fwd(L.select_cfg(0.0, 0, rule="stat", stat_lambda=1.0)) == 1          # no floor
    assert fwd(L.select_cfg(0.9, 1, rule="stat", stat_lambda=float("nan"))) == 1
    assert fwd(L.select_cfg(0.9, 1, rule="stat", domain="head")) == 5
    sub = L.cluster_cfg("subspace", clusters=4, sub_dims=(16, 24, 24))
    assert fwd(L.select_cfg(0.9, 1, domain="head"), sub) == 5
    assert fwd(L.select_cfg(0.9, 1, rule="stat", stat_lambda=1.0), sub) == 5


def test_backward_validation(lib):
    """The backward takes bf16 only, no compensation, a workspace of the size
    its query function reports, and non-null tensors; each is checked before
    any work."""
    p = L.problem(1, 256, 64, 4, 8, 8, "bf16")
    cl = L.Clusters(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 0, 0, (L.I32 * 3)(0, 0, 0))
    need = L.sa_block_sparse_attn_bwd_workspace_size(p, 8, 8)
    assert need > 256 * 64 * 2

    def bwd(prob=p, a=L.attn_cfg(False), ws_bytes=need, d_o=FAKE):
        return lib.sa_block_sparse_attn_bwd(ctypes.byref(prob), ctypes.byref(a), ctypes.byref(cl), ctypes.byref(cl),
                                            FAKE, FAKE, FAKE, d_o, None, FAKE, FAKE, FAKE, FAKE, ws_bytes, None)

    assert bwd(prob=L.problem(1, 256, 64, 4, 8, 8, "f32")) == 3
    assert bwd(a=L.attn_cfg(True)) == 5
    assert bwd(ws_bytes=need - 1) == 4
    assert bwd(d_o=None) == 1
    out = ctypes.c_size_t(0)
    assert lib.sa_block_sparse_attn_bwd_workspace_size(ctypes.byref(p), 0, 8, ctypes.byref(out)) == 1
