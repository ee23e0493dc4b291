"""Host logic of the C ABI, run on the CPU: the library loads and exports every
declared symbol; pool layout and page bookkeeping; the Partial dispatch plan
(pinned to the Figure 4 worked example); argument validation.  No call here
launches a kernel: every compute call below fails validation on the host."""

import ctypes
import json
import os
import re

import pytest

from oracle import dsa_oracle as O
from sparse_attention_09_amd import dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")

pytestmark = pytest.mark.skipif(not os.path.exists(dsa.LIB_PATH),
                                reason="libdsa.so not built (run __graft_entry__.build())")

FAKE = 0x7f0000000000  # a 256-byte aligned address that is never dereferenced on the host


def declared_functions():
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text))
    return names


def test_library_exports_every_declared_symbol():
    L = dsa.lib()
    declared = declared_functions()
    assert declared == set(dsa.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name
    assert dsa.abi_version() == 1


def test_status_strings():
    L = dsa.lib()
    assert L.dsa_status_string(0) == b"DSA_OK"
    assert L.dsa_status_string(4) == b"DSA_ERR_WORKSPACE"


@pytest.mark.parametrize("kv", [dsa.KV_BF16, dsa.KV_FP8])
def test_pool_layout_matches_the_format(kv):
    n = 37
    l = dsa.pool_layout(kv, n)
    assert (l.page_tokens, l.d_latent, l.d_rope, l.d_index) == (64, 512, 64, 128)
    if kv == dsa.KV_FP8:
        assert (l.latent_row_bytes, l.latent_row_stride, l.scale_offset) == (612, 640, 576)
    else:
        assert (l.latent_row_bytes, l.latent_row_stride, l.scale_offset) == (1152, 1152, -1)
    assert l.index_row_bytes == 256
    # the oracle's independent statement of the same format
    lat, idx, total = O.pool_plane_offsets(kv, n)
    assert (l.latent_plane_offset, l.index_plane_offset, l.total_bytes) == (lat, idx, total)


def test_fp8_row_bytes_for_a_million_token_request():
    # 1,048,576 rows of 612 algorithmic bytes ~= 0.6 GB per request per layer
    l = dsa.pool_layout(dsa.KV_FP8, 1)
    gib = (1 << 20) * l.latent_row_bytes / 2 ** 30
    assert abs(gib - 0.598) < 0.001


def _raw_pool(num_pages, kv=dsa.KV_FP8):
    L = dsa.lib()
    h = ctypes.c_void_p()
    st = L.dsa_pool_create(ctypes.c_void_p(FAKE), dsa.pool_layout(kv, num_pages).total_bytes,
                           num_pages, kv, ctypes.byref(h))
    assert st == 0
    return h


def _arr(ids):
    return (ctypes.c_int32 * max(len(ids), 1))(*ids)


def test_pool_create_validation():
    L = dsa.lib()
    h = ctypes.c_void_p()
    need = dsa.pool_layout(dsa.KV_FP8, 10).total_bytes
    assert L.dsa_pool_create(None, need, 10, 1, ctypes.byref(h)) == 1
    assert L.dsa_pool_create(ctypes.c_void_p(FAKE + 16), need, 10, 1, ctypes.byref(h)) == 1
    assert L.dsa_pool_create(ctypes.c_void_p(FAKE), need - 1, 10, 1, ctypes.byref(h)) == 1
    assert b"smaller" in L.dsa_last_error()
    assert L.dsa_pool_create(ctypes.c_void_p(FAKE), need, 10, 7, ctypes.byref(h)) == 1
    assert L.dsa_pool_create(ctypes.c_void_p(FAKE), need, 0, 1, ctypes.byref(h)) == 1
    assert L.dsa_pool_create(ctypes.c_void_p(FAKE), need, 10, 1, ctypes.byref(h)) == 0
    L.dsa_pool_destroy(h)


def test_pool_alloc_share_release():
    L = dsa.lib()
    h = _raw_pool(8)
    ids = (ctypes.c_int32 * 8)()
    assert L.dsa_pool_alloc(h, 5, ids) == 0
    got = list(ids[:5])
    assert sorted(got) == list(range(5)) and L.dsa_pool_free_pages(h) == 3
    # all-or-nothing exhaustion
    assert L.dsa_pool_alloc(h, 4, ids) == 3
    assert L.dsa_pool_free_pages(h) == 3
    # sharing raises refcounts; a page returns to the free list only at zero
    assert L.dsa_pool_share(h, _arr(got[:2]), 2) == 0
    assert L.dsa_pool_refcount(h, got[0]) == 2
    assert L.dsa_pool_release(h, _arr(got), 5) == 0
    assert L.dsa_pool_free_pages(h) == 6
    assert L.dsa_pool_refcount(h, got[0]) == 1 and L.dsa_pool_refcount(h, got[4]) == 0
    # releasing a free page, or a page more times than referenced, changes nothing
    assert L.dsa_pool_release(h, _arr([got[4]]), 1) == 1
    assert L.dsa_pool_release(h, _arr([got[0], got[0]]), 2) == 1
    assert L.dsa_pool_refcount(h, got[0]) == 1 and L.dsa_pool_free_pages(h) == 6
    assert L.dsa_pool_share(h, _arr([99]), 1) == 1
    assert L.dsa_pool_refcount(h, 99) == -1
    L.dsa_pool_destroy(h)


def test_prefix_sharing_page_count_matches_slot_formula():
    g = json.load(open(os.path.join(GOLDEN, "prefix_sharing_slots.json")))
    N, Lp, Ls, P = g["num_requests"], g["prefix_tokens"], g["suffix_tokens"], g["page_tokens"]
    prefix_pages, suffix_pages = Lp // P, -(-Ls // P)
    L = dsa.lib()
    h = _raw_pool(g["shared_pages"])
    prefix = (ctypes.c_int32 * prefix_pages)()
    assert L.dsa_pool_alloc(h, prefix_pages, prefix) == 0
    priv = (ctypes.c_int32 * suffix_pages)()
    for r in range(N):
        if r:
            assert L.dsa_pool_share(h, prefix, prefix_pages) == 0
        assert L.dsa_pool_alloc(h, suffix_pages, priv) == 0
    # exactly Lp + N*Ls token slots (in pages) are used; nothing left over
    assert L.dsa_pool_free_pages(h) == 0
    assert L.dsa_pool_refcount(h, prefix[0]) == N
    assert N * (prefix_pages + suffix_pages) == g["unshared_pages"]
    # one more request cannot get its private pages
    assert L.dsa_pool_alloc(h, 1, priv) == 3
    for r in range(N):
        assert L.dsa_pool_release(h, prefix, prefix_pages) == 0
    assert L.dsa_pool_free_pages(h) == prefix_pages
    L.dsa_pool_destroy(h)


def test_plan_matches_figure4_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "fig4_virtual_padding.json")))
    W = g["width"]
    for tile, iters in g["iterations"].items():
        p = dsa.plan_partial(1024, W, int(tile), 1)
        assert p.iters_total == iters and p.splits == 1 and p.tile == int(tile)
    p = dsa.plan_partial(1024, W, 128, 1)
    assert p.virtual_cols == g["virtual_columns"]["128"]
    assert p.padding_cols == g["padding_columns"]["128"]


def test_plan_split_columns_match_oracle_partition():
    for W in [1, 100, 2048, 2112, 5000]:
        for tile in [32, 64, 128]:
            for S in [1, 2, 3, 7, 64]:
                p = dsa.plan_partial(8, W, tile, S)
                ours = [(min(W, s * p.cols_per_split), min(W, (s + 1) * p.cols_per_split))
                        for s in range(S)]
                assert ours == O.split_bounds(W, tile, S)


def test_plan_dispatch_uses_query_parallelism():
    # enough query tokens for every CU: one split (no combine work beyond a copy)
    p = dsa.plan_partial(1024, 2048, 0, 0, 256)
    assert p.splits == 1
    assert p.tile == 32
    # few tokens: splits supply the parallelism up to one workgroup per CU,
    # with at least two tiles per split
    p = dsa.plan_partial(8, 2048, 0, 0, 256)
    assert (p.tile, p.splits, p.iters_per_split) == (64, 16, 2)
    p = dsa.plan_partial(100, 2048, 0, 0, 256)
    assert p.splits == 3 and p.splits * 100 >= 256
    # a short index row takes tile 32 and still splits
    p = dsa.plan_partial(1, 256, 0, 0, 256)
    assert (p.tile, p.splits, p.iters_per_split) == (32, 4, 2)
    p = dsa.plan_partial(1, 40, 0, 0, 256)
    assert (p.tile, p.splits) == (32, 1)
    L = dsa.lib()
    out = dsa.PartialPlan()
    assert L.dsa_plan_partial(4, 0, 0, 0, 0, ctypes.byref(out)) == 1
    assert L.dsa_plan_partial(4, 100, 48, 0, 0, ctypes.byref(out)) == 1
    assert L.dsa_plan_partial(4, 100, 32, -1, 0, ctypes.byref(out)) == 1


def test_topk_workspace_bytes():
    L = dsa.lib()
    assert L.dsa_topk_workspace_bytes(1024, 65536, 2048) == 0
    # 1M positions -> 16 segments of 65,536, candidates of (fp32, int32)
    assert L.dsa_topk_workspace_bytes(8, 1 << 20, 2048) == 8 * 16 * 2048 * 8
    # k is padded to a multiple of 4 per segment
    assert L.dsa_topk_workspace_bytes(2, 70000, 5) == 2 * 2 * 8 * 8


def test_index_topk_workspace_bytes():
    L = dsa.lib()
    T, cap = 1024, 128
    # fallback counter, fallback list, samples (one page in 32: 32 x 64 columns),
    # thresholds, and per 512-position chunk (128) a region of (score,
    # position) pairs: a count pair and cap candidates, in whole 16-pair lines
    want = 256 + 4 * T + 4 * T * 2048 + 4 * T + 8 * T * 128 * (cap + 16)
    assert L.dsa_index_topk_workspace_bytes(T, 65536, cap) == want
    want20 = want - 8 * T * 128 * (cap + 16) + 8 * T * 128 * 32
    assert L.dsa_index_topk_workspace_bytes(T, 65536, 20) == want20
    assert L.dsa_index_topk_workspace_bytes(T, 65537, cap) == 0     # rows too long
    assert L.dsa_index_topk_workspace_bytes(T, 4096, 0) == 0
    assert L.dsa_index_topk_workspace_bytes(T, 4096, 129) == 0
    assert L.dsa_index_topk_workspace_bytes(0, 4096, 128) == 0


def test_index_topk_validates_before_launch():
    L = dsa.lib()
    vp = ctypes.c_void_p
    h = _raw_pool(4)
    f = vp(FAKE)
    need = L.dsa_index_topk_workspace_bytes(1, 256, 128)

    def call(k=64, cap=128, target=0, max_ctx=256, ws=f, ws_bytes=need, T=1, pool=h):
        return L.dsa_index_topk(pool, f, 4, f, 1, 1, f, T, max_ctx, f, f, k, cap, target, f, ws,
                                ws_bytes, None)

    assert call(pool=None) == 1
    assert call(k=0) == 1
    assert call(k=20000) == 1
    assert call(cap=0) == 1 and call(cap=129) == 1
    assert call(target=-1) == 1
    assert call(max_ctx=65537) == 2
    assert call(ws=None) == 4
    assert call(ws_bytes=need - 1) == 4
    assert call(ws=vp(FAKE + 16)) == 1
    assert call(T=0) == 0
    L.dsa_pool_destroy(h)


def test_dcp_calls_validate_before_launch():
    L = dsa.lib()
    vp = ctypes.c_void_p
    f = vp(FAKE)
    assert L.dsa_dcp_merge(0, 4, 8, f, f, 64, f, f, None) == 1          # no shards
    assert L.dsa_dcp_merge(17, 4, 8, f, f, 64, f, f, None) == 1         # too many
    assert L.dsa_dcp_merge(8, 4, 4096, f, f, 4096, f, f, None) == 2     # G*k above 16384
    assert L.dsa_dcp_merge(2, 4, 0, f, f, 64, f, f, None) == 1
    assert L.dsa_dcp_merge(2, 4, 8, None, f, 64, f, f, None) == 1
    assert L.dsa_dcp_merge(2, 4, 8, f, f, 0, f, f, None) == 1
    assert L.dsa_dcp_merge(2, 0, 8, None, None, 64, None, None, None) == 0   # empty batch
    assert L.dsa_combine_shards(f, f, 1, 0, f, f, None) == 1
    assert L.dsa_combine_shards(None, f, 1, 2, f, f, None) == 1
    assert L.dsa_combine_shards(None, None, 0, 2, None, None, None) == 0


def test_compute_calls_validate_before_launch():
    L = dsa.lib()
    vp = ctypes.c_void_p
    h = _raw_pool(4)
    f = vp(FAKE)
    # null pool / pointers, bad ld
    assert L.dsa_index_scores(None, f, 4, f, 1, 1, f, 1, 64, f, f, f, 64, None) == 1
    assert L.dsa_index_scores(h, None, 4, f, 1, 1, f, 1, 64, f, f, f, 64, None) == 1
    assert L.dsa_index_scores(h, f, 4, f, 1, 1, f, 1, 64, f, f, f, 62, None) == 1
    assert L.dsa_index_scores(h, f, 4, f, 1, 1, f, 1, 64, vp(FAKE + 2), f, f, 64, None) == 1
    # top-k: k limits, workspace for long rows
    assert L.dsa_topk(f, 64, f, 1, 64, 0, f, None, 0, None) == 1
    assert L.dsa_topk(f, 64, f, 1, 64, 20000, f, None, 0, None) == 2
    assert L.dsa_topk(f, 1 << 20, f, 1, 1 << 20, 2048, f, None, 0, None) == 4
    assert L.dsa_topk(f, 1 << 20, f, 1, 1 << 20, 2048, f, f, 100, None) == 4
    assert L.dsa_topk(f, 1 << 22, f, 1, 1 << 22, 2048, f, f, 1 << 40, None) == 2
    # partial: tile and split checks
    assert L.dsa_sparse_mla_partial(h, f, 4, f, 1, f, 1, f, f, 64, ctypes.c_float(0.1), 48, 1, f, f,
                                    None) == 1
    assert L.dsa_sparse_mla_partial(h, f, 4, f, 1, f, 1, f, f, 0, ctypes.c_float(0.1), 64, 1, f, f,
                                    None) == 1
    assert L.dsa_sparse_mla_partial(h, f, 4, f, 1, f, 1, f, f, 64, ctypes.c_float(0.1), 64, 0, f, f,
                                    None) == 1
    assert L.dsa_sparse_mla_partial(h, f, 4, f, 1, f, 1, f, f, 64, ctypes.c_float(float("nan")), 64,
                                    1, f, f, None) == 1
    assert L.dsa_sparse_mla_partial(h, f, 4, f, 1, f, 1, f, f, 64, ctypes.c_float(-0.1), 64,
                                    1, f, f, None) == 1
    assert L.dsa_sparse_mla_partial(h, f, 4, f, 1, f, 1, f, f, 64, ctypes.c_float(0.1), 64,
                                    1, None, f, None) == 1
    # single-split form: same checks, outputs required
    assert L.dsa_sparse_mla(h, f, 4, f, 1, f, 1, f, f, 64, ctypes.c_float(0.1), 48, f, f, None) == 1
    assert L.dsa_sparse_mla(h, f, 4, f, 1, f, 1, f, f, 64, ctypes.c_float(0.0), 64, f, f, None) == 1
    assert L.dsa_sparse_mla(h, f, 4, f, 1, f, 1, f, f, 64, ctypes.c_float(0.1), 64, None, f, None) == 1
    assert L.dsa_sparse_mla(h, f, 4, f, 1, f, 1, f, f, 64, ctypes.c_float(0.1), 64, f, None, None) == 1
    assert L.dsa_sparse_mla(h, f, 4, f, 1, f, 0, None, None, 64, ctypes.c_float(0.1), 64, None, None,
                            None) == 0
    # combine
    assert L.dsa_combine(f, f, 1, 0, f, f, None) == 1
    assert L.dsa_combine(None, f, 1, 1, f, f, None) == 1
    # cache append: pool, sizes, pointers, alignment
    assert L.dsa_kv_append(None, f, 4, 1, f, f, 1, f, f, None) == 1
    assert L.dsa_kv_append(h, f, 4, 1, f, f, -1, f, f, None) == 1
    assert L.dsa_kv_append(h, f, 0, 1, f, f, 1, f, f, None) == 1
    assert L.dsa_kv_append(h, f, 4, 1, None, f, 1, f, f, None) == 1
    assert L.dsa_kv_append(h, f, 4, 1, f, f, 1, None, f, None) == 1
    assert L.dsa_kv_append(h, f, 4, 1, f, f, 1, vp(FAKE + 8), None, None) == 1
    assert L.dsa_kv_append(h, f, 4, 1, f, f, 1, f, vp(FAKE + 4), None) == 1
    assert L.dsa_kv_append(h, None, 4, 1, None, None, 0, None, None, None) == 0
    # read probe: pointers, size, alignment, grid bounds; 0 bytes launches nothing
    assert L.dsa_read_probe(None, 64, f, 1, None) == 1
    assert L.dsa_read_probe(f, 64, None, 1, None) == 1
    assert L.dsa_read_probe(f, 60, f, 1, None) == 1
    assert L.dsa_read_probe(f, -16, f, 1, None) == 1
    assert L.dsa_read_probe(vp(FAKE + 4), 64, f, 1, None) == 1
    assert L.dsa_read_probe(f, 64, f, 0, None) == 1
    assert L.dsa_read_probe(f, 64, f, 65537, None) == 1
    assert L.dsa_read_probe(f, 0, f, 1, None) == 0
    # empty batches are valid no-ops
    assert L.dsa_combine(None, None, 0, 1, None, None, None) == 0
    assert L.dsa_topk(None, 64, None, 0, 64, 8, None, None, 0, None) == 0
    L.dsa_pool_destroy(h)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(dsa, "_lib", None)
    monkeypatch.setattr(dsa, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        dsa.lib()
