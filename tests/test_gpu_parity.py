"""Parity of the HIP path (through the C ABI) with the CPU oracle on small
workloads that span several tiles, ragged tails and ragged contexts, plus the
edge cases.  Indexer scores and top-k indices must be bit-exact; attention
outputs within the stated tolerance of the float64 oracle."""

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from sparse_attention_09_amd import dsa, synth
from tests._harness import HostView, bf16_to_f64, check_attention, make_pool, run_path, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _gen(name, seed=0):
    say(f"[case] generate {name} seed={seed}")
    return synth.generate(synth.spec(name), seed=seed, device="cpu").to(DEV)


def _check_full_path(wl, kv_tile=0, num_splits=0, tokens=None):
    s = wl.spec
    say(f"[case] path {s.name} tile={kv_tile} splits={num_splits}")
    path, out, lse = run_path(wl, kv_tile, num_splits)
    hv = HostView(wl)
    scores = path.scores.cpu().numpy()
    idx = path.idx.cpu().numpy()
    out_h = bf16_to_f64(out)
    lse_h = lse.cpu().numpy().astype(np.float64)
    tokens = range(s.num_tokens) if tokens is None else tokens
    worst = 0.0
    for t in tokens:
        pos = int(hv.tok_pos[t])
        ref = hv.token(t, path.plan.tile, path.plan.splits)
        assert np.array_equal(scores[t, :pos + 1], ref["scores"]), f"scores differ at token {t}"
        assert np.array_equal(idx[t], ref["idx"]), f"top-k differs at token {t}"
        worst = max(worst, check_attention(out_h[t], lse_h[t], ref["o"], ref["lse"], f"token {t}"))
    return path, worst


@pytest.mark.parametrize("name", ["tiny_bf16", "tiny_fp8", "tiny_fp8_shared", "dense_fp8",
                                  "decode_bf16_4k"])
def test_full_path_small(name):
    _check_full_path(_gen(name))


def test_many_requests_some_empty():
    # 300 requests, a fifth of them with no query token (equal consecutive
    # offsets): the kernels find a token's request by counting the offsets
    # at or below it, 256 requests in the first round and 64 at a time after,
    # so tokens of requests past 256 and next to empty ones are checked
    g = np.random.default_rng(31)
    R = 300
    ctx = [int(x) for x in g.integers(40, 260, size=R)]
    q = [int(x) for x in g.integers(0, 3, size=R)]
    for b in (0, 255, 256, 257, R - 1):
        q[b] = max(q[b], 1)
    for b in (254, 258, 290):
        q[b] = 0
    spec = synth.Spec("many_reqs_fp8", synth.KV_FP8, ctx, q, 32)
    wl = synth.generate(spec, seed=5, device="cpu").to(DEV)
    assert spec.num_reqs == R and sum(1 for x in q if x == 0) > 0
    offs = np.cumsum([0] + q)
    late = [t for t in range(int(offs[255]), spec.num_tokens)]
    early = list(range(0, 12))
    for tile, splits in ((32, 1), (64, 1)):
        _check_full_path(wl, tile, splits, tokens=early + late)


@pytest.mark.parametrize("tile,splits", [(32, 1), (32, 3), (64, 1), (64, 2), (32, 40), (128, 1),
                                         (128, 3)])
def test_full_path_tiles_and_splits(tile, splits):
    _check_full_path(_gen("tiny_fp8", seed=1), tile, splits)


@pytest.mark.parametrize("tile,splits", [(128, 1), (128, 2), (64, 2)])
def test_bf16_partial_splits_against_oracle(tile, splits):
    # BF16 rows at tile 128 (the warp-specialized kernel's BF16 form, 4 value
    # waves; splits cut at multiples of 128 columns) and at tile 64, with one
    # and with several splits: every split's (o, lse) and the combined output
    # against the oracle
    wl = _gen("tiny_bf16", seed=12)
    hv = HostView(wl)
    pool = make_pool(wl)
    for width in (300, 129):
        say(f"[case] bf16 partial width={width} tile={tile} splits={splits}")
        idx = synth.random_index(wl.tok_pos, width, seed=width + 7 * tile + splits).to(DEV)
        o_p, lse_p = dsa.sparse_mla_partial(pool, wl.page_table, wl.q_offsets, wl.tok_pos, wl.q, idx,
                                            wl.spec.sm_scale, tile, splits)
        out, lse = dsa.combine(o_p, lse_p)
        torch.cuda.synchronize()
        o_p = o_p.cpu().numpy().astype(np.float64)
        lse_p = lse_p.cpu().numpy().astype(np.float64)
        out_h, lse_h = bf16_to_f64(out), lse.cpu().numpy().astype(np.float64)
        idx_h = idx.cpu().numpy()
        for t in range(wl.num_tokens):
            ref = hv.token(t, tile, splits, idx=idx_h[t])
            for s in range(splits):
                check_attention(o_p[t, s], lse_p[t, s], ref["o_part"][s], ref["lse_part"][s],
                                f"token {t} split {s}")
            check_attention(out_h[t], lse_h[t], ref["o"], ref["lse"], f"token {t}")


def test_width_2112_figure4_shape():
    # index width 2112: not a multiple of 64 at tile 64 (virtual padding of the last tile)
    wl = _gen("width2112_fp8")
    for tile in (32, 64):
        path, _ = _check_full_path(wl, tile, 1)
        assert path.plan.iters_total == O.num_iterations(2112, tile)


def test_partial_with_arbitrary_index_tensor():
    # -1 padding, positions past the token's range, repeats; ragged width
    wl = _gen("tiny_fp8", seed=2)
    hv = HostView(wl)
    pool = make_pool(wl)
    for width, tile, splits in [(77, 32, 1), (77, 64, 2), (300, 32, 4), (300, 64, 3), (5, 32, 2)]:
        say(f"[case] partial random idx width={width} tile={tile} splits={splits}")
        idx = synth.random_index(wl.tok_pos, width, seed=width + tile).to(DEV)
        o_p, lse_p = dsa.sparse_mla_partial(pool, wl.page_table, wl.q_offsets, wl.tok_pos, wl.q, idx,
                                            wl.spec.sm_scale, tile, splits)
        out, lse = dsa.combine(o_p, lse_p)
        torch.cuda.synchronize()
        o_p = o_p.cpu().numpy().astype(np.float64)
        lse_p = lse_p.cpu().numpy().astype(np.float64)
        out_h, lse_h = bf16_to_f64(out), lse.cpu().numpy().astype(np.float64)
        idx_h = idx.cpu().numpy()
        for t in range(wl.num_tokens):
            ref = hv.token(t, tile, splits, idx=idx_h[t])
            for s in range(splits):
                check_attention(o_p[t, s], lse_p[t, s], ref["o_part"][s], ref["lse_part"][s],
                                f"token {t} split {s}")
            check_attention(out_h[t], lse_h[t], ref["o"], ref["lse"], f"token {t}")


def test_partial_peaked_softmax_and_single_rows():
    # sm_scale 1.0 makes the softmax peaked; width-1 indices give a single row
    wl = _gen("tiny_bf16", seed=3)
    hv = HostView(wl)
    pool = make_pool(wl)
    for width, scale in [(1, 1 / 24), (40, 1.0), (3, 1.0)]:
        say(f"[case] partial width={width} scale={scale}")
        idx = synth.random_index(wl.tok_pos, width, seed=10 + width, frac_invalid=0.0).to(DEV)
        o_p, lse_p = dsa.sparse_mla_partial(pool, wl.page_table, wl.q_offsets, wl.tok_pos, wl.q, idx,
                                            scale, 32, 1)
        out, lse = dsa.combine(o_p, lse_p)
        torch.cuda.synchronize()
        out_h, lse_h = bf16_to_f64(out), lse.cpu().numpy().astype(np.float64)
        hv.sm_scale = scale
        idx_h = idx.cpu().numpy()
        for t in range(wl.num_tokens):
            ref = hv.token(t, 32, 1, idx=idx_h[t])
            check_attention(out_h[t], lse_h[t], ref["o"], ref["lse"], f"token {t}")


def test_partial_later_tile_far_above_first_tile():
    # One row of request 1 gets a score about 200 (natural units, sm_scale 1)
    # above everything before it in the index, and it sits at index column
    # 152: in the fifth tile at tile 32, the third at tile 64 and the second
    # at tile 128.  At tile 64 the kernel's reference max, fixed by the first
    # tile, is then far too low and the split is recomputed with the exact max;
    # at tiles 32 and 128 the warp-specialized kernel's running max grows by
    # more than its rescale threshold and O is rescaled.  Every form must
    # match the oracle.
    wl = synth.generate(synth.spec("tiny_bf16"), seed=7, device="cpu")
    b, t, p_hi = 1, 3, 120
    assert int(wl.tok_req[t]) == b and int(wl.tok_pos[t]) >= 300
    q = O.bf16_bits_to_f64(wl.q[t].view(torch.uint16).numpy())          # [64, 576]
    v = q.sum(axis=0)
    assert (q @ v).min() > 0
    k_hi = v * (250.0 / (q @ v).min())
    bits = torch.from_numpy(k_hi.astype(np.float32)).to(torch.bfloat16).view(torch.uint8)
    phys = int(wl.page_table[b, p_hi // 64]) * 64 + p_hi % 64
    stride = synth.ROW_STRIDE[wl.spec.kv_dtype]
    wl.pool[phys * stride: phys * stride + 2 * 576] = bits
    wl = wl.to(DEV)
    hv = HostView(wl)
    hv.sm_scale = 1.0
    cols = np.concatenate([np.arange(32), np.arange(200, 300), np.arange(100, 132)]).astype(np.int32)
    assert int(np.nonzero(cols == p_hi)[0][0]) == 152
    idx = torch.from_numpy(np.tile(cols, (wl.num_tokens, 1))).to(DEV)
    pool = make_pool(wl)
    for tile, splits in ((32, 1), (64, 1), (128, 1), (128, 2)):
        say(f"[case] partial tile={tile} splits={splits}: dominant row at index column 152")
        o_p, lse_p = dsa.sparse_mla_partial(pool, wl.page_table, wl.q_offsets, wl.tok_pos, wl.q,
                                            idx, 1.0, tile, splits)
        out, lse = dsa.combine(o_p, lse_p)
        torch.cuda.synchronize()
        out_h, lse_h = bf16_to_f64(out), lse.cpu().numpy().astype(np.float64)
        for tt in range(wl.num_tokens):
            ref = hv.token(tt, tile, splits, idx=cols)
            check_attention(out_h[tt], lse_h[tt], ref["o"], ref["lse"], f"tile {tile} token {tt}")
            if tt == t:   # the case is what it claims: every head's max is the planted row
                assert np.all(ref["lse"] > 200)


@pytest.mark.parametrize("name", ["tiny_fp8", "tiny_bf16"])
def test_single_split_call_equals_partial_plus_combine(name):
    # dsa_sparse_mla (final output, no Combine) against the split form with one
    # split followed by Combine: bit for bit, at every tile size
    wl = _gen(name, seed=6)
    pool = make_pool(wl)
    idx = synth.random_index(wl.tok_pos, 300, seed=66, frac_invalid=0.1).to(DEV)
    for tile in (32, 64, 128):
        say(f"[case] single-split form {name} tile={tile}")
        o_p, lse_p = dsa.sparse_mla_partial(pool, wl.page_table, wl.q_offsets, wl.tok_pos, wl.q, idx,
                                            wl.spec.sm_scale, tile, 1)
        out_a, lse_a = dsa.combine(o_p, lse_p)
        out_b, lse_b = dsa.sparse_mla(pool, wl.page_table, wl.q_offsets, wl.tok_pos, wl.q, idx,
                                      wl.spec.sm_scale, tile)
        torch.cuda.synchronize()
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
        assert torch.equal(lse_a, lse_b)


@pytest.mark.parametrize("name", ["tiny_fp8", "tiny_bf16"])
def test_kv_append_matches_oracle_bytes(name):
    # new tokens written into the pool by the GPU and by the oracle's
    # quantizer/append on a host copy: every byte of the pool must agree
    # (FP8 codes and scales bit-exact; rows with an out-of-range request,
    # position or page id write nothing)
    wl = synth.generate(synth.spec(name), seed=8, device="cpu")
    g = torch.Generator().manual_seed(88)
    B = wl.page_table.shape[0]
    n_pos = wl.page_table.shape[1] * 64
    # distinct destinations inside the requests' contexts (unused page-table
    # entries alias page 0, and two rows with one destination are unspecified)
    cand = torch.tensor([(b, p) for b, L in enumerate(wl.spec.ctx_lens) for p in range(L)])
    pick = cand[torch.randperm(cand.shape[0], generator=g)[:300]]
    req = pick[:, 0].to(torch.int32).contiguous()
    pos = pick[:, 1].to(torch.int32).contiguous()
    req[:3] = torch.tensor([B, -1, 0], dtype=torch.int32)            # bad request ids
    pos[2] = n_pos                                                     # past the page table
    n = req.numel()
    scale = torch.exp(torch.randn((n, 9), generator=g) * 4).repeat_interleave(64, dim=1)
    lat = (torch.randn((n, 576), generator=g) * scale).to(torch.bfloat16)
    lat[5, 64:128] = 0.0                                               # an all-zero group
    lat[6, :64] = -0.0                                                 # negative zeros
    lat[7, 128:192] = torch.randn(64, generator=g).to(torch.bfloat16) * 1e-30
    keys = torch.randint(-8, 9, (n, 128), generator=g).to(torch.bfloat16)
    pool_host = O.PoolView(wl.pool.numpy().copy(), wl.num_pages, wl.spec.kv_dtype)
    O.append_rows(pool_host, wl.page_table.numpy(), req.tolist(), pos.tolist(),
                  lat.float().numpy(), keys.view(torch.uint16).numpy())
    dev = wl.to(DEV)
    pool = make_pool(dev)
    say(f"[case] kv_append {name}: {n} rows")
    dsa.kv_append(pool, dev.page_table, req.to(DEV), pos.to(DEV), lat.to(DEV), keys.to(DEV))
    torch.cuda.synchronize()
    got = dev.pool.cpu().numpy()
    bad = np.nonzero(got != pool_host.buf)[0]
    assert bad.size == 0, f"{bad.size} pool bytes differ, first at {bad[:8]}"


def test_kv_append_rounds_midpoints_to_even_codes():
    # Values that land exactly halfway between two E4M3FN codes after the
    # division by the group scale, so the rounding rule decides them: each
    # group's amax is 448 * 2^e (scale exactly 2^e) and its other 63 values
    # are +-midpoints * 2^e, covering the midpoints of every adjacent pair of
    # finite codes (lower code even and odd; subnormal, subnormal-to-normal
    # and normal range).  Ties go to the even code: the GPU's bytes must equal
    # the oracle's and the hand-derived codes.
    wl = synth.generate(synth.spec("tiny_fp8"), seed=9, device="cpu")
    vals = torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).double()  # ascending
    mids = (vals[:-1] + vals[1:]) / 2                                   # 126 midpoints
    even_code = torch.where(torch.arange(126) % 2 == 0, torch.arange(126), torch.arange(126) + 1)
    g = torch.Generator().manual_seed(123)
    rows, want = [], []
    for r in range(8):
        row, wrow = [], []
        for grp in range(9):
            e = int(torch.randint(-12, 9, (1,), generator=g))
            pick = torch.randint(0, 126, (63,), generator=g)
            if r < 2:                                   # the first rows walk every midpoint
                pick = (torch.arange(63) + 63 * ((2 * r + grp) % 2)) % 126
            sign = torch.where(torch.rand(63, generator=g) < 0.5, -1.0, 1.0).double()
            x = torch.cat([torch.tensor([448.0]).double(), sign * mids[pick]]) * 2.0 ** e
            codes = torch.cat([torch.tensor([0x7E]), even_code[pick] | torch.where(sign < 0, 0x80, 0)])
            perm = torch.randperm(64, generator=g)
            row.append(x[perm])
            wrow.append(codes[perm])
        rows.append(torch.cat(row))
        want.append(torch.cat(wrow))
    lat = torch.stack(rows)
    assert torch.equal(lat.to(torch.bfloat16).double(), lat)           # exact in bf16
    n = lat.shape[0]
    req = torch.zeros(n, dtype=torch.int32)
    pos = torch.arange(100, 100 + n, dtype=torch.int32)
    pool_host = O.PoolView(wl.pool.numpy().copy(), wl.num_pages, wl.spec.kv_dtype)
    O.append_rows(pool_host, wl.page_table.numpy(), req.tolist(), pos.tolist(),
                  lat.to(torch.bfloat16).float().numpy(), None)
    dev = wl.to(DEV)
    pool = make_pool(dev)
    say(f"[case] kv_append midpoints: {n} rows")
    dsa.kv_append(pool, dev.page_table, req.to(DEV), pos.to(DEV), lat.to(torch.bfloat16).to(DEV))
    torch.cuda.synchronize()
    got = dev.pool.cpu().numpy()
    bad = np.nonzero(got != pool_host.buf)[0]
    assert bad.size == 0, f"{bad.size} pool bytes differ, first at {bad[:8]}"
    pt = wl.page_table.numpy()
    for i in range(n):
        phys = int(pt[0, int(pos[i]) // 64]) * 64 + int(pos[i]) % 64
        codes = got[phys * 640: phys * 640 + 576]
        assert np.array_equal(codes, want[i].numpy().astype(np.uint8)), f"row {i}"


def test_all_masked_token_gives_zero_and_neg_inf():
    wl = _gen("tiny_fp8", seed=4)
    pool = make_pool(wl)
    idx = torch.full((wl.num_tokens, 50), -1, dtype=torch.int32, device=DEV)
    o_p, lse_p = dsa.sparse_mla_partial(pool, wl.page_table, wl.q_offsets, wl.tok_pos, wl.q, idx,
                                        wl.spec.sm_scale, 32, 3)
    out, lse = dsa.combine(o_p, lse_p)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_shared_prefix_pool_equals_duplicated_pool():
    a = _gen("tiny_fp8_shared", seed=5)
    b = _gen("tiny_fp8_shared_dup", seed=5)
    assert b.num_pages > a.num_pages
    for tile in (32, 64):
        pa, oa, la = run_path(a, tile, 1)
        pb, ob, lb = run_path(b, tile, 1)
        for t, pos in enumerate(a.tok_pos.tolist()):
            assert torch.equal(pa.scores[t, :pos + 1], pb.scores[t, :pos + 1])
        assert torch.equal(pa.idx, pb.idx)
        assert torch.equal(oa, ob) and torch.equal(la, lb)


def test_page_permutation_invariance():
    s = synth.spec("tiny_fp8")
    w1 = synth.generate(s, seed=6).to(DEV)
    # same logical content, different physical page ids
    n = w1.num_pages
    ids = torch.randperm(n, generator=torch.Generator().manual_seed(99))
    w2 = synth.generate(s, seed=6, page_ids=ids).to(DEV)
    assert not torch.equal(w1.page_table, w2.page_table)
    p1, o1, l1 = run_path(w1, 32, 2)
    p2, o2, l2 = run_path(w2, 32, 2)
    assert torch.equal(p1.idx, p2.idx) and torch.equal(o1, o2) and torch.equal(l1, l2)


def test_tile32_vs_tile64_same_indices_close_outputs():
    wl = _gen("tiny_fp8", seed=7)
    p32, o32, l32 = run_path(wl, 32, 1)
    p64, o64, l64 = run_path(wl, 64, 1)
    assert torch.equal(p32.idx, p64.idx)
    a, b = bf16_to_f64(o32), bf16_to_f64(o64)
    assert np.max(np.abs(a - b)) < 2e-2


def test_deterministic_repeat():
    wl = _gen("tiny_fp8", seed=8)
    p, o1, l1 = run_path(wl, 32, 2)
    o2, l2 = p.step(wl.q_idx, wl.w, wl.q)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_empty_batch_is_noop():
    wl = _gen("tiny_fp8", seed=9)
    pool = make_pool(wl)
    z = torch.zeros(0, dtype=torch.int32, device=DEV)
    qo = torch.zeros(1, dtype=torch.int32, device=DEV)
    sc = dsa.index_scores(pool, wl.page_table, qo, z,
                          torch.zeros((0, 16, 128), dtype=torch.bfloat16, device=DEV),
                          torch.zeros((0, 16), device=DEV), 1, 64)
    idx = dsa.topk(sc, z, 8, 64)
    assert idx.shape == (0, 8)
    o, l = dsa.combine(torch.zeros((0, 1, 64, 512), device=DEV), torch.zeros((0, 1, 64), device=DEV))
    torch.cuda.synchronize()
    assert o.shape == (0, 64, 512)


def test_topk_ties_and_short_rows_direct():
    # hand-made score rows: many ties at the threshold, rows shorter than k
    T, ld, k = 6, 4096, 100
    g = torch.Generator().manual_seed(11)
    sc = torch.randint(0, 7, (T, ld), generator=g).float()
    sc[1] = 5.0                                            # all equal
    sc[2] = torch.arange(ld).float()                       # strictly increasing
    sc[3] = -torch.arange(ld).float()                      # negative values
    tok_pos = torch.tensor([4095, 4095, 4095, 4095, 50, 0], dtype=torch.int32)
    say("[case] topk hand-made rows")
    idx = dsa.topk(sc.to(DEV), tok_pos.to(DEV), k, ld).cpu().numpy()
    for t in range(T):
        ref = O.topk_positions(sc[t, :int(tok_pos[t]) + 1].numpy(), k)
        assert np.array_equal(idx[t], ref), t


def test_topk_long_rows_two_stage():
    # rows longer than one 65,536-element segment go through segment + merge
    T, L, k = 3, 200_000, 700
    g = torch.Generator().manual_seed(12)
    sc = torch.randint(0, 1000, (T, L), generator=g).float()
    # token 1 sees one position of its third segment and token 2 none past
    # the first, so their segment lists hold empty slots; token 1's scores
    # are negative, so an empty slot read as a score would outrank them
    sc[1] = -1.0 - sc[1]
    tok_pos = torch.tensor([L - 1, 131_072, 65_535], dtype=torch.int32)
    say("[case] topk long rows")
    idx = dsa.topk(sc.to(DEV), tok_pos.to(DEV), k, L).cpu().numpy()
    for t in range(T):
        ref = O.topk_positions(sc[t, :int(tok_pos[t]) + 1].numpy(), k)
        assert np.array_equal(idx[t], ref), t


def test_topk_full_rows_candidate_and_fallback_paths():
    # 65,536-position rows: (a) integer scores like the indexer's (threshold bin
    # small enough for the LDS candidate list), (b) three distinct values (the
    # threshold bin overflows the list: register fallback), (c) negative and
    # positive values with many exact ties, (d) a row shorter than k
    L, k = 65536, 2048
    g = torch.Generator().manual_seed(13)
    rows = [torch.randint(0, 15000, (L,), generator=g).float(),
            torch.randint(0, 3, (L,), generator=g).float() * 7.0,
            (torch.randint(-50, 50, (L,), generator=g).float() * 0.25),
            torch.randn(L, generator=g)]
    sc = torch.stack(rows)
    tok_pos = torch.tensor([L - 1, L - 1, 40000, 1000], dtype=torch.int32)
    say("[case] topk full rows")
    idx = dsa.topk(sc.to(DEV), tok_pos.to(DEV), k, L).cpu().numpy()
    for t in range(sc.shape[0]):
        ref = O.topk_positions(sc[t, :int(tok_pos[t]) + 1].numpy(), k)
        assert np.array_equal(idx[t], ref), t


@pytest.mark.parametrize("S", [1, 7, 8, 9, 64])
def test_combine_against_oracle_merge(S):
    """dsa_combine on seeded partials against the oracle's log-sum-exp merge:
    split counts around the kernel's group of eight, empty splits (lse -inf,
    o 0) mixed in, heads whose every split is empty, and lse values far
    apart.  Only the bf16 rounding of o separates the two."""
    T = 5
    g = torch.Generator().manual_seed(100 + S)
    o = torch.randn((T, S, 64, 512), generator=g, dtype=torch.float64)
    lse = torch.randn((T, S, 64), generator=g, dtype=torch.float64) * 6.0
    lse[:, :, 5] += 80.0 * torch.rand((T, S), generator=g, dtype=torch.float64)   # far apart
    empty = torch.rand((T, S, 64), generator=g) < 0.3
    empty[:, :, 7] = True                                                          # all splits empty
    lse[empty] = -np.inf
    o[empty.unsqueeze(-1).expand_as(o)] = 0.0
    o32, lse32 = o.to(torch.float32), lse.to(torch.float32)
    say(f"[case] combine S={S}")
    out, lse_out = dsa.combine(o32.to(DEV), lse32.to(DEV))
    torch.cuda.synchronize()
    got_o = bf16_to_f64(out)
    got_l = lse_out.cpu().numpy().astype(np.float64)
    for t in range(T):
        ref_o, ref_l = O.combine(o32[t].numpy(), lse32[t].numpy())
        assert np.array_equal(np.isneginf(got_l[t]), np.isneginf(ref_l))
        fin = np.isfinite(ref_l)
        assert np.all(got_o[t][~fin] == 0)
        assert np.max(np.abs(got_l[t][fin] - ref_l[fin])) <= 1e-4
        err = np.abs(got_o[t][fin] - ref_o[fin])
        assert np.all(err <= 2.0 ** -8 * np.abs(ref_o[fin]) + 1e-6), f"token {t}: max err {err.max()}"
