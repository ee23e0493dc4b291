"""The DCP shard layout on one GPU: G round-robin KV shards (positions
p = j*G + r on shard r), each shard's own indexer + top-k, the merge into the
global top-k (dsa_dcp_merge), each shard's partial over its share and the
LSE merge (dsa_combine_shards).  Indices must equal the oracle's top-k over
the whole row bit for bit; the attention must stay within the tolerance of
the oracle's (the shards only regroup the softmax sums)."""

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from sparse_attention_09_amd import dsa, synth
from tests._harness import HostView, bf16_to_f64, check_attention, make_pool, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _dcp(wl, G, kv_tile=64):
    shards = synth.shard_round_robin(wl, G)
    views = [(make_pool(sh), sh.page_table, sh.tok_pos, sh.max_ctx) for sh in shards]
    path = dsa.DcpPath(views, wl.q_offsets, wl.max_q, wl.spec.k, kv_tile=kv_tile,
                       sm_scale=wl.spec.sm_scale)
    out, lse = path.step(wl.q_idx, wl.w, wl.q)
    torch.cuda.synchronize()
    return path, out, lse


def _check_shard_share(path, G):
    idx = path.idx.cpu().numpy()
    sidx = path.shard_idx.cpu().numpy()
    for r in range(G):
        for t in range(idx.shape[0]):
            mine = [p // G for p in idx[t] if p >= 0 and p % G == r]
            row = sidx[r, t]
            assert row[:len(mine)].tolist() == mine, (r, t)
            assert np.all(row[len(mine):] == -1)


@pytest.mark.parametrize("name,G", [("tiny_fp8", 2), ("tiny_fp8", 3), ("tiny_bf16", 8),
                                    ("tiny_fp8_shared", 4), ("decode_bf16_4k", 8)])
def test_dcp_small_against_oracle(name, G):
    wl = synth.generate(synth.spec(name), seed=0, device="cpu").to(DEV)
    say(f"[case] dcp {name} G={G}")
    path, out, lse = _dcp(wl, G)
    hv = HostView(wl)
    idx = path.idx.cpu().numpy()
    out_h, lse_h = bf16_to_f64(out), lse.cpu().numpy().astype(np.float64)
    for t in range(wl.num_tokens):
        ref = hv.token(t, 64, 1)
        assert np.array_equal(idx[t], ref["idx"]), f"top-k differs at token {t}"
        check_attention(out_h[t], lse_h[t], ref["o"], ref["lse"], f"token {t}")
    _check_shard_share(path, G)


def test_dcp_equals_unsharded_path_and_ties():
    """Many tokens per request; then constant indexer keys (every score tied,
    the winners interleaved over the shards)."""
    s = synth.Spec("many_q_fp8", synth.KV_FP8, [5000, 2100, 700, 3], [19, 8, 3, 2], 128)
    for tied in (False, True):
        wl = synth.generate(s, seed=6, device="cpu").to(DEV)
        if tied:
            stride = synth.ROW_STRIDE[s.kv_dtype]
            wl.pool[wl.num_pages * 64 * stride:].view(torch.int16).fill_(0x3F80)
        say(f"[case] dcp vs unsharded tied={tied}")
        pool = make_pool(wl)
        ref = dsa.DsaPath(pool, wl.page_table, wl.q_offsets, wl.tok_pos, wl.max_q, wl.max_ctx,
                          s.k, kv_tile=64, num_splits=1, sm_scale=s.sm_scale, select="scores")
        o_ref, l_ref = ref.step(wl.q_idx, wl.w, wl.q)
        for G in (2, 5):
            path, out, lse = _dcp(wl, G)
            assert torch.equal(path.idx, ref.idx), f"G={G}"
            _check_shard_share(path, G)
            assert float((out.float() - o_ref.float()).abs().max()) < 2e-2
            fin = torch.isfinite(l_ref)
            assert torch.equal(fin, torch.isfinite(lse))
            assert float((lse[fin] - l_ref[fin]).abs().max()) < 2e-2
        if tied:
            pos = wl.tok_pos.cpu().numpy()
            got = path.idx.cpu().numpy()
            for t in range(wl.num_tokens):
                n = min(s.k, int(pos[t]) + 1)
                assert got[t][:n].tolist() == list(range(n))


def test_dcp_verify_64k_eight_shards():
    """The 64K verify batch over 8 shards: every token's indices equal the
    unsharded fused selection's, sampled tokens equal the oracle's."""
    say("[case] dcp verify_fp8_64k G=8: generate")
    wl = synth.generate(synth.spec("verify_fp8_64k"), seed=0, device=DEV)
    torch.cuda.synchronize()
    pool = make_pool(wl)
    ref = dsa.DsaPath(pool, wl.page_table, wl.q_offsets, wl.tok_pos, wl.max_q, wl.max_ctx,
                      wl.spec.k, kv_tile=64, num_splits=1, sm_scale=wl.spec.sm_scale)
    o_ref, _ = ref.step(wl.q_idx, wl.w, wl.q)
    idx_ref = ref.idx.clone()
    del ref
    pool.close()
    say("[case] dcp verify_fp8_64k G=8: sharded step")
    path, out, lse = _dcp(wl, 8)
    assert torch.equal(path.idx, idx_ref)
    assert float((out.float() - o_ref.float()).abs().max()) < 2e-2
    tokens = [0, 517, wl.num_tokens - 1]
    reqs = sorted(set(int(wl.tok_req[t]) for t in tokens))
    hv = HostView(wl, reqs=reqs)
    for t in tokens:
        r = hv.token(t, 64, 1)
        assert np.array_equal(path.idx[t].cpu().numpy(), r["idx"])
        check_attention(bf16_to_f64(out[t]), lse[t].cpu().numpy().astype(np.float64), r["o"],
                        r["lse"], f"token {t}")
    del wl, path, out, lse
    torch.cuda.empty_cache()
