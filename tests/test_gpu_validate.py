"""DSA_VALIDATE=1 through the C ABI on the GPU: a corrupt page table or token
position is rejected before launch with DSA_ERR_INVALID_ARG (the kernels
would otherwise clamp a bad page id into the pool), and a valid batch runs
and gives the same result as without the checks."""

import pytest
import torch

from sparse_attention_09_amd import dsa, synth
from tests._harness import make_pool, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture
def validate(monkeypatch):
    monkeypatch.setenv("DSA_VALIDATE", "1")


def _wl():
    return synth.generate(synth.spec("tiny_fp8"), seed=21, device="cpu").to(DEV)


def test_validate_accepts_a_good_batch(validate):
    wl = _wl()
    pool = make_pool(wl)
    say("[case] DSA_VALIDATE good batch")
    idx = dsa.index_topk(pool, wl.page_table, wl.q_offsets, wl.tok_pos, wl.q_idx, wl.w, wl.max_q,
                         wl.max_ctx, wl.spec.k)
    out, lse = dsa.sparse_mla(pool, wl.page_table, wl.q_offsets, wl.tok_pos, wl.q, idx,
                              wl.spec.sm_scale, 64)
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all()


@pytest.mark.parametrize("what", ["page_negative", "page_past_pool", "tok_pos", "q_offsets"])
def test_validate_rejects_corrupt_batch(validate, what):
    wl = _wl()
    pool = make_pool(wl)
    pt, tp, qo = wl.page_table.clone(), wl.tok_pos.clone(), wl.q_offsets.clone()
    if what == "page_negative":
        pt[0, 1] = -1
    elif what == "page_past_pool":
        pt[2, 0] = wl.num_pages
    elif what == "tok_pos":
        tp[0] = pt.shape[1] * 64
    else:
        qo[1] = qo[2] + 1
    idx = torch.zeros((wl.num_tokens, wl.spec.k), dtype=torch.int32, device=DEV)
    say(f"[case] DSA_VALIDATE rejects {what}")
    calls = [
        lambda: dsa.index_scores(pool, pt, qo, tp, wl.q_idx, wl.w, wl.max_q, wl.max_ctx),
        lambda: dsa.index_topk(pool, pt, qo, tp, wl.q_idx, wl.w, wl.max_q, wl.max_ctx, wl.spec.k),
        lambda: dsa.sparse_mla(pool, pt, qo, tp, wl.q, idx, wl.spec.sm_scale, 64),
        lambda: dsa.sparse_mla_partial(pool, pt, qo, tp, wl.q, idx, wl.spec.sm_scale, 32, 2),
        lambda: dsa.sparse_mla_q8(pool, pt, qo, tp, *dsa.quantize_q8(wl.q), idx, wl.spec.sm_scale),
    ]
    for call in calls:
        with pytest.raises(dsa.DsaError) as e:
            call()
        assert e.value.status == 1 and "DSA_VALIDATE" in str(e.value)
    torch.cuda.synchronize()
