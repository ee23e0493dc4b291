"""Parity of the fused indexer + top-k (dsa_index_topk) with the oracle's
top-k, through the C ABI.  The selection must be bit-exact whichever way a
token goes: through the sampled threshold and its candidates, or through the
exact fallback (forced here with tiny candidate capacities or thresholds), on
ragged contexts, rows of at most k positions, heavy ties and the boundary
k / k+1 rows."""

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from sparse_attention_09_amd import dsa, synth
from tests._harness import HostView, bf16_to_f64, check_attention, make_pool, run_path, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _gen(s, seed=0):
    say(f"[case] generate {s.name} seed={seed}")
    return synth.generate(s, seed=seed, device="cpu").to(DEV)


def _oracle_idx(wl):
    hv = HostView(wl)
    out = np.empty((wl.num_tokens, wl.spec.k), dtype=np.int32)
    for t in range(wl.num_tokens):
        b, pos = int(hv.tok_req[t]), int(hv.tok_pos[t])
        keys = hv.pool.index_keys(hv.pt[b], np.arange(pos + 1))
        s = O.index_scores(O.bf16_bits_to_f64(hv.q_idx[t]), hv.w[t], keys)
        out[t] = O.topk_positions(s, wl.spec.k)
    return out


def _fused(wl, pool, cap=dsa.DEFAULT_CAP, target=0):
    T = wl.num_tokens
    ws = torch.empty(max(dsa.index_topk_workspace_bytes(T, wl.max_ctx, cap), 1), dtype=torch.uint8,
                     device=DEV)
    idx = dsa.index_topk(pool, wl.page_table, wl.q_offsets, wl.tok_pos, wl.q_idx, wl.w, wl.max_q,
                         wl.max_ctx, wl.spec.k, cap=cap, cand_target=target, workspace=ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), int(ws[:4].view(torch.int32).item())


def _long_rows(wl):
    k = wl.spec.k
    return int((wl.tok_pos.cpu().numpy() + 1 > k).sum())


@pytest.mark.parametrize("name", ["tiny_bf16", "tiny_fp8", "tiny_fp8_shared", "dense_fp8",
                                  "decode_bf16_4k"])
def test_fused_path_small(name):
    """The default path (fused selection, then sparse MLA) against the oracle."""
    wl = _gen(synth.spec(name))
    say(f"[case] fused path {name}")
    path, out, lse = run_path(wl, select="auto")
    assert path.fused_topk
    hv = HostView(wl)
    idx = path.idx.cpu().numpy()
    out_h, lse_h = bf16_to_f64(out), lse.cpu().numpy().astype(np.float64)
    for t in range(wl.num_tokens):
        ref = hv.token(t, path.plan.tile, path.plan.splits)
        assert np.array_equal(idx[t], ref["idx"]), f"top-k differs at token {t}"
        check_attention(out_h[t], lse_h[t], ref["o"], ref["lse"], f"token {t}")


@pytest.mark.parametrize("seed", [0, 3])
def test_fused_caps_and_targets(seed):
    """Every capacity / threshold setting gives the oracle's indices; cap 1
    sends every row longer than k to the fallback."""
    wl = _gen(synth.spec("tiny_fp8"), seed=seed)
    pool = make_pool(wl)
    ref = _oracle_idx(wl)
    k = wl.spec.k
    # caps around the 16-pair line of a candidate region (count pair + cap)
    for cap, target in [(128, 0), (64, 0), (32, 0), (15, 0), (17, 0), (4, 0), (1, 0),
                        (128, k // 8), (128, 4 * k), (128, 1 << 20), (16, 1 << 20),
                        (15, 1 << 20)]:
        say(f"[case] fused tiny_fp8 seed={seed} cap={cap} target={target}")
        got, nfb = _fused(wl, pool, cap, target)
        for t in range(wl.num_tokens):
            assert np.array_equal(got[t], ref[t]), f"cap={cap} target={target}: token {t} differs"
        if cap == 1:
            assert nfb == _long_rows(wl)


def test_fused_boundary_rows():
    """Rows of k-1, k and k+1 positions, a short request and a long one."""
    s = synth.Spec("edge_fp8", synth.KV_FP8, [97, 98, 40, 3000], [2, 2, 1, 3], 96)
    wl = _gen(s, seed=5)
    pool = make_pool(wl)
    ref = _oracle_idx(wl)
    for cap in (128, 1):
        say(f"[case] fused edge rows cap={cap}")
        got, _ = _fused(wl, pool, cap)
        assert np.array_equal(got, ref)


def test_fused_all_scores_tied():
    """Constant indexer keys: every visible position scores the same, so the
    top-k is the k lowest positions (a threshold tie the size of the row)."""
    wl = _gen(synth.spec("tiny_bf16"), seed=4)
    stride = synth.ROW_STRIDE[wl.spec.kv_dtype]
    keys = wl.pool[wl.num_pages * 64 * stride:].view(torch.int16)
    keys.fill_(0x3F80)   # bf16 1.0
    torch.cuda.synchronize()
    pool = make_pool(wl)
    ref = _oracle_idx(wl)
    k = wl.spec.k
    pos = wl.tok_pos.cpu().numpy()
    for t in range(wl.num_tokens):
        n = min(k, int(pos[t]) + 1)
        assert np.array_equal(ref[t][:n], np.arange(n))
    for cap, target in [(128, 0), (128, 1 << 20), (2, 0)]:
        say(f"[case] fused all-tied cap={cap} target={target}")
        got, _ = _fused(wl, pool, cap, target)
        assert np.array_equal(got, ref)


def test_fused_equals_unfused_calls():
    """The fused call and dsa_index_scores + dsa_topk agree bit for bit on a
    batch with many tokens per request (several query blocks)."""
    s = synth.Spec("many_q_fp8", synth.KV_FP8, [5000, 2100, 700], [19, 8, 3], 128)
    wl = _gen(s, seed=6)
    pool = make_pool(wl)
    sc = dsa.index_scores(pool, wl.page_table, wl.q_offsets, wl.tok_pos, wl.q_idx, wl.w, wl.max_q,
                          wl.max_ctx)
    want = dsa.topk(sc, wl.tok_pos, s.k, wl.max_ctx).cpu().numpy()
    for cap in (128, 8):
        say(f"[case] fused vs unfused cap={cap}")
        got, _ = _fused(wl, pool, cap)
        assert np.array_equal(got, want)
    ref = _oracle_idx(wl)
    assert np.array_equal(want, ref)


def test_graph_replay_equals_eager():
    """The whole step recorded on a HIP graph: every replay, with eager work
    of the program between replays, gives the eager step's bits."""
    wl = _gen(synth.spec("tiny_fp8"), seed=9)
    for select in ("auto", "scores"):
        say(f"[case] graph replay select={select}")
        pool = make_pool(wl)
        path = dsa.DsaPath(pool, wl.page_table, wl.q_offsets, wl.tok_pos, wl.max_q, wl.max_ctx,
                           wl.spec.k, kv_tile=64, num_splits=1, sm_scale=wl.spec.sm_scale,
                           select=select)
        out, lse = path.step(wl.q_idx, wl.w, wl.q)
        torch.cuda.synchronize()
        want = (out.clone(), lse.clone(), path.idx.clone())
        replay = path.capture(wl.q_idx, wl.w, wl.q)
        for i in range(4):
            path.out.fill_(0)
            path.idx.fill_(-7)
            torch.cuda.synchronize()
            replay()
            torch.cuda.synchronize()
            assert torch.equal(path.out, want[0]) and torch.equal(path.lse, want[1])
            assert torch.equal(path.idx, want[2]), f"replay {i}"
            # eager work between replays
            dsa.index_scores(pool, wl.page_table, wl.q_offsets, wl.tok_pos, wl.q_idx, wl.w,
                             wl.max_q, wl.max_ctx)


@pytest.mark.parametrize("k", [1, 7, 3000, 5000])
def test_fused_odd_k(k):
    """k = 1, a small odd k, and k large enough that most rows exceed the
    selection workgroup's candidate room and take the fallback."""
    s = synth.Spec("odd_k_fp8", synth.KV_FP8, [9000, 4100, 130], [3, 2, 2], k)
    wl = _gen(s, seed=11)
    pool = make_pool(wl)
    ref = _oracle_idx(wl)
    for cap in (128, 16):
        say(f"[case] fused k={k} cap={cap}")
        got, _ = _fused(wl, pool, cap)
        assert np.array_equal(got, ref)


def test_fused_zero_context_bound():
    """max_ctx = 0: nothing is visible, every index is -1 (as the unfused calls give)."""
    wl = _gen(synth.spec("tiny_fp8"))
    pool = make_pool(wl)
    T, k = wl.num_tokens, wl.spec.k
    ws = torch.empty(max(dsa.index_topk_workspace_bytes(T, 0, 128), 1), dtype=torch.uint8,
                     device=DEV)
    idx = dsa.index_topk(pool, wl.page_table, wl.q_offsets, wl.tok_pos, wl.q_idx, wl.w, wl.max_q,
                         0, k, workspace=ws)
    torch.cuda.synchronize()
    assert bool((idx == -1).all())
