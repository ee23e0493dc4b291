"""Parity at full workload sizes, in the launch configuration the benchmark
times (automatic plan for the device's CU count).  Sampled tokens are
checked element by element against the oracle (bit-exact scores and indices,
attention within tolerance); every token is checked for properties that hold
at any size (indices ascending, unique, visible, -1 padded only at the end;
finite outputs)."""

import numpy as np
import pytest
import torch

from sparse_attention_09_amd import dsa, synth
from tests._harness import HostView, bf16_to_f64, check_attention, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run(wl, kv_tile=0, num_splits=0, select="scores"):
    cus = torch.cuda.get_device_properties(DEV).multi_processor_count
    pool = dsa.Pool(wl.pool, wl.num_pages, wl.spec.kv_dtype)
    path = dsa.DsaPath(pool, wl.page_table, wl.q_offsets, wl.tok_pos, wl.max_q, wl.max_ctx,
                       wl.spec.k, kv_tile=kv_tile, num_splits=num_splits,
                       sm_scale=wl.spec.sm_scale, cu_count=cus, select=select)
    out, lse = path.step(wl.q_idx, wl.w, wl.q)
    torch.cuda.synchronize()
    return path, out, lse


def _check_all_tokens(wl, path, out, lse):
    """Properties of every token's indices and outputs (checked on the GPU)."""
    idx = path.idx.to(torch.int64)
    pos = wl.tok_pos.to(torch.int64)[:, None]
    k = idx.shape[1]
    valid = idx >= 0
    nvis = torch.clamp(pos[:, 0] + 1, max=k)
    # exactly min(k, visible) entries, all in front
    assert torch.equal(valid.sum(1), nvis)
    assert torch.equal(valid, torch.arange(k, device=idx.device)[None, :] < nvis[:, None])
    # ascending (so unique) and visible
    d = idx[:, 1:] - idx[:, :-1]
    assert bool(((d > 0) | ~valid[:, 1:]).all())
    assert bool(((idx <= pos) | ~valid).all())
    assert bool(torch.isfinite(out.float()).all()) and bool(torch.isfinite(lse).all())


def _check_tokens(wl, path, out, lse, tokens):
    s = wl.spec
    reqs = sorted(set(int(wl.tok_req[t]) for t in tokens))
    say(f"[case] {s.name}: oracle on tokens {list(tokens)} (requests {reqs})")
    hv = HostView(wl, reqs=reqs)
    for t in tokens:
        pos = int(hv.tok_pos[t])
        ref = hv.token(t, path.plan.tile, path.plan.splits)
        if path.scores is not None:
            scores = path.scores[t, :pos + 1].cpu().numpy()
            assert np.array_equal(scores, ref["scores"]), f"scores differ at token {t}"
        assert np.array_equal(path.idx[t].cpu().numpy(), ref["idx"]), f"top-k differs at token {t}"
        check_attention(bf16_to_f64(out[t]), lse[t].cpu().numpy().astype(np.float64), ref["o"],
                        ref["lse"], f"token {t}")


def _sample(T, n_rand, seed):
    g = np.random.default_rng(seed)
    picks = {0, T - 1} | set(int(x) for x in g.integers(0, T, size=n_rand))
    return sorted(picks)


def _gen(name, seed=0):
    say(f"[case] generate {name} on the GPU")
    wl = synth.generate(synth.spec(name), seed=seed, device=DEV)
    torch.cuda.synchronize()
    return wl


def test_decode_bf16_4k_full():
    wl = _gen("decode_bf16_4k")
    path, out, lse = _run(wl)
    _check_all_tokens(wl, path, out, lse)
    _check_tokens(wl, path, out, lse, [0])


def test_verify_fp8_64k_full():
    wl = _gen("verify_fp8_64k")
    path, out, lse = _run(wl)
    _check_all_tokens(wl, path, out, lse)
    _check_tokens(wl, path, out, lse, _sample(wl.num_tokens, 4, 1))
    del wl, path, out, lse
    torch.cuda.empty_cache()


def test_longctx_fp8_1m_full():
    wl = _gen("longctx_fp8_1m")
    path, out, lse = _run(wl)
    assert path.plan.splits > 1            # few query tokens: the plan splits the KV
    _check_all_tokens(wl, path, out, lse)
    _check_tokens(wl, path, out, lse, [0, 5])
    del wl, path, out, lse
    torch.cuda.empty_cache()


def test_prefill_fp8_32k_full():
    wl = _gen("prefill_fp8_32k")
    path, out, lse = _run(wl)
    _check_all_tokens(wl, path, out, lse)
    _check_tokens(wl, path, out, lse, _sample(wl.num_tokens, 3, 2))
    del wl, path, out, lse
    torch.cuda.empty_cache()


def test_shared_prefix_fp8_full_tiles_and_pool_layouts():
    shared = _gen("shared_prefix_fp8", seed=0)
    p32, o32, l32 = _run(shared, kv_tile=32, num_splits=1)
    _check_all_tokens(shared, p32, o32, l32)
    idx32 = p32.idx.clone()
    del p32
    p128, o128, l128 = _run(shared, kv_tile=128, num_splits=1)
    _check_all_tokens(shared, p128, o128, l128)
    # tile 32 and tile 128 select the same positions and agree within tolerance
    assert torch.equal(idx32, p128.idx)
    diff = (o32.float() - o128.float()).abs()
    assert float(diff.max()) < 2e-2
    _check_tokens(shared, p128, o128, l128, _sample(shared.num_tokens, 3, 3))
    # the same logical content with a private copy of the prefix per request
    o_ref, l_ref = o128.clone(), l128.clone()
    del p128, o32, o128, l32, l128
    dup = _gen("shared_prefix_fp8_dup", seed=0)
    assert dup.num_pages > 40 * shared.num_pages
    del shared
    torch.cuda.empty_cache()
    pd, od, ld_ = _run(dup, kv_tile=128, num_splits=1)
    assert torch.equal(idx32, pd.idx)
    assert torch.equal(od, o_ref) and torch.equal(ld_, l_ref)
    del dup, pd, od, ld_
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["verify_fp8_64k", "prefill_fp8_32k"])
def test_fused_select_full(name):
    """The fused indexer + top-k (the default path for rows up to 65,536) at
    full size: every token's indices equal the unfused calls' (which the tests
    above pin to the oracle), sampled tokens equal the oracle's, and the
    attention behind it stays within tolerance."""
    wl = _gen(name)
    path, out, lse = _run(wl, select="auto")
    assert path.fused_topk
    nfb = path.fallback_count()
    say(f"[case] {name}: fused selection, {nfb} tokens took the fallback")
    assert nfb == 0      # random scores: the sampled threshold leaves >= k candidates
    _check_all_tokens(wl, path, out, lse)
    idx_fused = path.idx.clone()
    path.index_scores(wl.q_idx, wl.w)
    path.topk()
    torch.cuda.synchronize()
    assert torch.equal(idx_fused, path.idx)
    path.scores = None
    _check_tokens(wl, path, out, lse, _sample(wl.num_tokens, 3, 4))
    del wl, path, out, lse, idx_fused
    torch.cuda.empty_cache()


def test_prefill_fp8_32k_q8_full():
    """The Q8 path on the 32K prefill chunk in the benchmark's configuration
    (the fused selection's rows, the FP8 query quantizer, the Q8 attention):
    every token finite and within the FP8-query distance of the bf16-query
    output, sampled tokens against the oracle (query codes bit for bit,
    attention within tolerance)."""
    from oracle import dsa_oracle as O
    wl = _gen("prefill_fp8_32k")
    path, out16, _ = _run(wl, select="auto")
    codes, scales = dsa.quantize_q8(wl.q)
    out, lse = dsa.sparse_mla_q8(path.pool, wl.page_table, wl.q_offsets, wl.tok_pos, codes, scales,
                                 path.idx, wl.spec.sm_scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all()) and bool(torch.isfinite(lse).all())
    assert float((out.float() - out16.float()).abs().max()) < 0.1
    tokens = _sample(wl.num_tokens, 3, 5)
    reqs = sorted(set(int(wl.tok_req[t]) for t in tokens))
    say(f"[case] prefill Q8: oracle on tokens {tokens}")
    hv = HostView(wl, reqs=reqs)
    for t in tokens:
        rc, rs = O.quantize_q8(O.bf16_bits_to_f64(hv.q[t]))
        assert np.array_equal(codes[t].cpu().numpy(), rc) and np.array_equal(scales[t].cpu().numpy(), rs)
        b, pos = int(hv.tok_req[t]), int(hv.tok_pos[t])
        ref = O.token_path_q8(hv.pool, hv.pt[b], pos, path.idx[t].cpu().numpy(), rc, rs,
                              wl.spec.sm_scale)
        check_attention(bf16_to_f64(out[t]), lse[t].cpu().numpy().astype(np.float64), ref["o"],
                        ref["lse"], f"Q8 token {t}")
    del wl, path, out16, out, lse, codes, scales
    torch.cuda.empty_cache()
