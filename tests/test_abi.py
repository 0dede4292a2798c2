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


def test_attn_events_probe_validation(lib):
    assert lib.sa_set_attn_events(None, FAKE) == 1
    assert lib.sa_set_attn_events(FAKE, None) == 1
    assert lib.sa_set_attn_events(None, None) == 0
