"""Seeded synthetic workloads for the DSA sparse-attention path.

This module only draws random inputs and lays them out in the storage format;
it holds none of the path's arithmetic (no scoring, selection, attention or
merging).  Tests and the benchmark generate a workload once and hand the same
bytes to both the HIP library and the CPU oracle.

Shapes follow the workloads the pages discuss (GLM-5.3-Flash serving):
  * decode_bf16_4k       - batch 1, one query token, 4,096-token context,
                           BF16 latent KV, top-256;
  * verify_fp8_64k       - speculative verify: 128 requests x 8 query tokens
                           (the M1024 verification shape of the lmsys.org
                           blog, section 3), 64K context each, FP8 KV, top-2048;
  * prefill_fp8_32k      - a 32K-token prefill chunk (query i at 32,768+i) over
                           a 64K causal context (the 64K-input / 32K-chunk
                           prefill of the same blog, section 4), FP8, top-2048;
  * longctx_fp8_1m       - 8 requests x 1 token at a 1,048,576-token context
                           (the 1M context of the SGLang cookbook), FP8;
  * shared_prefix_fp8    - 132 requests sharing a 63,488-token prefix (one copy
                           of its pages) plus a private 1,024-token suffix, 8
                           query tokens each (the 99.9%-shared-prefix 64K/1K
                           decode of the blog, section 3), FP8.
Small variants of the same structure serve the parity tests.

Value recipe: indexer queries and keys are integers drawn uniformly from
[-8, 8] and stored as bf16; indexer head weights are integers from {1,..,4}
(fp32); attention queries and latent rows are N(0,1).  BF16 rows are the
round-to-nearest-even bf16 of the draws.  FP8 rows are quantized per 64
consecutive elements: scale = the smallest power of two 2^k with
amax <= 448 * 2^k (k >= -126; 1 if the group is all zero), stored as fp32,
code = E4M3FN(x / scale) via torch's float8_e4m3fn cast (x / scale is exact
and within +-448).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import torch

PAGE_TOKENS = 64
HEADS = 64
D_QK = 576
IDX_HEADS = 16
IDX_DIM = 128
KV_BF16 = 0
KV_FP8 = 1
ROW_STRIDE = {KV_BF16: 1152, KV_FP8: 640}
KEY_ROW_BYTES = 256


@dataclasses.dataclass
class Spec:
    """Structure of a synthetic batch."""
    name: str
    kv_dtype: int
    ctx_lens: Sequence[int]          # context length of each request
    q_per_req: Sequence[int]         # query tokens of each request (last positions)
    k: int
    shared_prefix: int = 0           # tokens (multiple of 64) shared by all requests
    duplicate_prefix: bool = False   # store a private copy of the prefix per request
    sm_scale: float = 1.0 / math.sqrt(D_QK)

    @property
    def num_reqs(self) -> int:
        return len(self.ctx_lens)

    @property
    def num_tokens(self) -> int:
        return int(sum(self.q_per_req))


def _uniform(name, kv_dtype, B, L, Tq, k, **kw):
    return Spec(name, kv_dtype, [L] * B, [Tq] * B, k, **kw)


def spec(name: str) -> Spec:
    """Named workloads (full sizes and small parity variants)."""
    table = {
        "decode_bf16_4k": lambda: _uniform("decode_bf16_4k", KV_BF16, 1, 4096, 1, 256),
        "verify_fp8_64k": lambda: _uniform("verify_fp8_64k", KV_FP8, 128, 65536, 8, 2048),
        "prefill_fp8_32k": lambda: _uniform("prefill_fp8_32k", KV_FP8, 1, 65536, 32768, 2048),
        "longctx_fp8_1m": lambda: _uniform("longctx_fp8_1m", KV_FP8, 8, 1 << 20, 1, 2048),
        "shared_prefix_fp8": lambda: _uniform("shared_prefix_fp8", KV_FP8, 132, 64512, 8, 2048,
                                              shared_prefix=63488),
        "shared_prefix_fp8_dup": lambda: _uniform("shared_prefix_fp8_dup", KV_FP8, 132, 64512, 8,
                                                  2048, shared_prefix=63488,
                                                  duplicate_prefix=True),
        # small structural variants: several tiles, ragged tails, ragged contexts
        "tiny_bf16": lambda: Spec("tiny_bf16", KV_BF16, [300, 1000, 77], [3, 5, 2], 96),
        "tiny_fp8": lambda: Spec("tiny_fp8", KV_FP8, [1000, 300, 4096], [4, 1, 3], 160),
        "tiny_fp8_shared": lambda: Spec("tiny_fp8_shared", KV_FP8, [1100, 1100, 1100],
                                        [2, 2, 2], 200, shared_prefix=1024),
        "tiny_fp8_shared_dup": lambda: Spec("tiny_fp8_shared_dup", KV_FP8, [1100, 1100, 1100],
                                            [2, 2, 2], 200, shared_prefix=1024,
                                            duplicate_prefix=True),
        "width2112_fp8": lambda: _uniform("width2112_fp8", KV_FP8, 2, 4096, 2, 2112),
        "dense_fp8": lambda: Spec("dense_fp8", KV_FP8, [200, 64, 129], [1, 2, 1], 256),
    }
    return table[name]()


def _gen(device, *key: int) -> torch.Generator:
    g = torch.Generator(device=device)
    h = 0x9E3779B97F4A7C15
    for v in key:
        h = (h ^ (int(v) + 0x632BE59BD9B9E5 + (h << 6) + (h >> 2))) & ((1 << 63) - 1)
    g.manual_seed(h)
    return g


def _quantize_fp8_rows(x: torch.Tensor) -> torch.Tensor:
    """[n,576] float32 -> [n,640] uint8 rows (codes | 9 fp32 scales | pad)."""
    n = x.shape[0]
    xg = x.view(n, 9, 64)
    amax = xg.abs().amax(dim=2)
    # amax = m * 2^e, m in [0.5, 1): 448 * 2^k >= amax first holds at
    # k = e - 9, or e - 8 when m > 448 / 512
    m, e = torch.frexp(amax)
    k = torch.clamp(e - 9 + (m > 0.875).to(e.dtype), min=-126)
    scale = torch.where(amax > 0, torch.ldexp(torch.ones_like(amax), k), torch.ones_like(amax))
    y = xg / scale[:, :, None]
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).view(n, 576)
    out = torch.zeros((n, 640), dtype=torch.uint8, device=x.device)
    out[:, :576] = codes
    out[:, 576:612] = scale.contiguous().view(torch.uint8).view(n, 36)
    return out


def _bf16_rows(x: torch.Tensor) -> torch.Tensor:
    n = x.shape[0]
    return x.to(torch.bfloat16).contiguous().view(torch.uint8).view(n, 2 * x.shape[1])


@dataclasses.dataclass
class Workload:
    spec: Spec
    seed: int
    num_pages: int
    pool: torch.Tensor          # uint8 [pool bytes]
    page_table: torch.Tensor    # int32 [B, pt_stride]
    q_offsets: torch.Tensor     # int32 [B+1]
    tok_pos: torch.Tensor       # int32 [T]
    tok_req: torch.Tensor       # int32 [T]
    q_idx: torch.Tensor         # bf16 [T,16,128]
    w: torch.Tensor             # float32 [T,16]
    q: torch.Tensor             # bf16 [T,64,576]

    @property
    def num_tokens(self) -> int:
        return self.spec.num_tokens

    @property
    def max_ctx(self) -> int:
        return int(max(self.spec.ctx_lens)) if self.spec.ctx_lens else 0

    @property
    def max_q(self) -> int:
        return int(max(self.spec.q_per_req)) if self.spec.q_per_req else 0

    def to(self, device) -> "Workload":
        f = {fld.name: getattr(self, fld.name) for fld in dataclasses.fields(self)}
        for key, v in f.items():
            if isinstance(v, torch.Tensor):
                f[key] = v.to(device)
        return Workload(**f)


def pool_bytes(kv_dtype: int, num_pages: int) -> int:
    return num_pages * PAGE_TOKENS * (ROW_STRIDE[kv_dtype] + KEY_ROW_BYTES)


def generate(s: Spec, seed: int = 0, device="cpu",
             page_ids: Optional[torch.Tensor] = None,
             chunk_pages: int = 2048) -> Workload:
    """Draw a workload.  Physical page ids are a seeded permutation of
    `page_ids` (default: 0..num_pages-1), so the page table is not the
    identity.  Page contents are keyed by logical page, so a duplicated-prefix
    pool holds byte-identical copies of the shared pages."""
    device = torch.device(device)
    B = s.num_reqs
    assert s.shared_prefix % PAGE_TOKENS == 0
    shared_pages = s.shared_prefix // PAGE_TOKENS
    pages_per_req = [-(-L // PAGE_TOKENS) for L in s.ctx_lens]
    private = [p - shared_pages for p in pages_per_req]
    assert all(p >= 0 for p in private)
    n_logical = shared_pages + sum(private)
    # physical pages: shared pages are stored once, or once per request
    n_phys = (shared_pages * B if s.duplicate_prefix else shared_pages) + sum(private)
    if page_ids is None:
        page_ids = torch.arange(n_phys, dtype=torch.int64)
    page_ids = torch.as_tensor(page_ids, dtype=torch.int64).cpu()
    assert page_ids.numel() == n_phys
    num_pages = int(page_ids.max().item()) + 1 if n_phys else 0
    perm = torch.randperm(n_phys, generator=_gen("cpu", seed, 1))
    phys = page_ids[perm]

    # logical page -> list of physical pages holding it; request page tables
    pt_stride = max(pages_per_req) if B else 1
    page_table = torch.zeros((B, max(pt_stride, 1)), dtype=torch.int64)
    logical_of_phys = torch.empty(n_phys, dtype=torch.int64)
    cur = 0
    if not s.duplicate_prefix:
        shared_phys = phys[cur:cur + shared_pages]
        logical_of_phys[cur:cur + shared_pages] = torch.arange(shared_pages)
        cur += shared_pages
    lcur = shared_pages
    for b in range(B):
        if s.duplicate_prefix:
            sp = phys[cur:cur + shared_pages]
            logical_of_phys[cur:cur + shared_pages] = torch.arange(shared_pages)
            cur += shared_pages
        else:
            sp = shared_phys
        pp = phys[cur:cur + private[b]]
        logical_of_phys[cur:cur + private[b]] = torch.arange(lcur, lcur + private[b])
        cur += private[b]
        lcur += private[b]
        page_table[b, :shared_pages] = sp
        page_table[b, shared_pages:shared_pages + private[b]] = pp

    stride = ROW_STRIDE[s.kv_dtype]
    lat_plane = num_pages * PAGE_TOKENS * stride
    pool = torch.zeros(pool_bytes(s.kv_dtype, num_pages), dtype=torch.uint8, device=device)
    lat = pool[:lat_plane].view(num_pages, PAGE_TOKENS * stride)
    keys = pool[lat_plane:].view(num_pages, PAGE_TOKENS * KEY_ROW_BYTES)

    # fill logical pages chunk by chunk, scatter each to its physical copies
    order = torch.argsort(logical_of_phys, stable=True)
    lsorted = logical_of_phys[order]
    psorted = phys[order]
    for c0 in range(0, n_logical, chunk_pages):
        c1 = min(n_logical, c0 + chunk_pages)
        n = c1 - c0
        g = _gen(device, seed, 2, c0)
        x = torch.randn((n * PAGE_TOKENS, D_QK), generator=g, device=device)
        rows = _quantize_fp8_rows(x) if s.kv_dtype == KV_FP8 else _bf16_rows(x)
        rows = rows.view(n, PAGE_TOKENS * stride)
        kk = torch.randint(-8, 9, (n * PAGE_TOKENS, IDX_DIM), generator=_gen(device, seed, 3, c0),
                           device=device, dtype=torch.int32).to(torch.bfloat16)
        kk = kk.view(torch.uint8).view(n, PAGE_TOKENS * KEY_ROW_BYTES)
        lo = torch.searchsorted(lsorted, torch.tensor(c0))
        hi = torch.searchsorted(lsorted, torch.tensor(c1))
        dst = psorted[lo:hi].to(device)
        src = (lsorted[lo:hi] - c0).to(device)
        lat[dst] = rows[src]
        keys[dst] = kk[src]
        del x, rows, kk

    T = s.num_tokens
    q_offsets = torch.zeros(B + 1, dtype=torch.int32)
    q_offsets[1:] = torch.cumsum(torch.tensor(list(s.q_per_req), dtype=torch.int32), 0)
    tok_pos = torch.empty(T, dtype=torch.int32)
    tok_req = torch.empty(T, dtype=torch.int32)
    for b in range(B):
        a, e = int(q_offsets[b]), int(q_offsets[b + 1])
        L = s.ctx_lens[b]
        tok_pos[a:e] = torch.arange(L - (e - a), L, dtype=torch.int32)
        tok_req[a:e] = b
    q_idx = torch.randint(-8, 9, (T, IDX_HEADS, IDX_DIM), generator=_gen(device, seed, 4),
                          device=device, dtype=torch.int32).to(torch.bfloat16)
    w = torch.randint(1, 5, (T, IDX_HEADS), generator=_gen(device, seed, 5), device=device,
                      dtype=torch.int32).to(torch.float32)
    q = torch.empty((T, HEADS, D_QK), dtype=torch.bfloat16, device=device)
    tchunk = 4096
    for t0 in range(0, T, tchunk):
        t1 = min(T, t0 + tchunk)
        q[t0:t1] = torch.randn((t1 - t0, HEADS, D_QK), generator=_gen(device, seed, 6, t0),
                               device=device).to(torch.bfloat16)
    return Workload(spec=s, seed=seed, num_pages=num_pages, pool=pool,
                    page_table=page_table.to(torch.int32).to(device),
                    q_offsets=q_offsets.to(device), tok_pos=tok_pos.to(device),
                    tok_req=tok_req.to(device), q_idx=q_idx, w=w, q=q)


def random_index(s_tok_pos: torch.Tensor, width: int, seed: int, frac_invalid: float = 0.1,
                 device="cpu") -> torch.Tensor:
    """An arbitrary index tensor [T, width] for exercising the attention step
    on its own: mostly visible positions (repeats allowed), some -1 entries and
    some positions past the token's visible range."""
    tok_pos = s_tok_pos.to("cpu", torch.int64)
    T = tok_pos.numel()
    g = _gen("cpu", seed, 7)
    u = torch.rand((T, width), generator=g)
    idx = (u * (tok_pos[:, None] + 1).double()).floor().to(torch.int64)
    r = torch.rand((T, width), generator=g)
    idx = torch.where(r < frac_invalid / 2, torch.full_like(idx, -1), idx)
    idx = torch.where((r >= frac_invalid / 2) & (r < frac_invalid),
                      tok_pos[:, None] + 1 + (u * 50).to(torch.int64), idx)
    return idx.to(torch.int32).to(device)


def shard_round_robin(wl: Workload, G: int, seed: int = 77) -> list:
    """The same batch as G round-robin KV shards (shard r holds positions
    p = j*G + r at local position j, as in a DCP deployment), each a Workload
    with its own pool and page table (a seeded permutation of its pages), the
    tokens' local positions floor((pos - r) / G) (-1 when pos < r), and the
    queries shared.  Pure data movement: rows are copied from `wl.pool`."""
    s = wl.spec
    dev = wl.pool.device
    stride = ROW_STRIDE[s.kv_dtype]
    n_rows = wl.num_pages * PAGE_TOKENS
    lat = wl.pool[: n_rows * stride].view(n_rows, stride)
    keys = wl.pool[n_rows * stride:].view(n_rows, KEY_ROW_BYTES)
    pt = wl.page_table.to(torch.int64)
    shards = []
    for r in range(G):
        lens = [max(0, -(-(L - r) // G)) for L in s.ctx_lens]
        pages = [-(-n // PAGE_TOKENS) for n in lens]
        npg = max(1, sum(pages))
        perm = torch.randperm(npg, generator=_gen("cpu", seed, G, r)).to(dev)
        local_pt = torch.zeros((s.num_reqs, max(1, max(pages) if pages else 1)), dtype=torch.int64,
                               device=dev)
        rows = torch.zeros(npg * PAGE_TOKENS, dtype=torch.int64, device=dev)
        cur = 0
        for b, (n, np_) in enumerate(zip(lens, pages)):
            if np_ == 0:
                continue
            local_pt[b, :np_] = perm[cur:cur + np_]
            cur += np_
            j = torch.arange(n, device=dev)
            p = j * G + r
            src = pt[b, p // PAGE_TOKENS] * PAGE_TOKENS + p % PAGE_TOKENS
            dst = local_pt[b, j // PAGE_TOKENS] * PAGE_TOKENS + j % PAGE_TOKENS
            rows[dst] = src
        pool = torch.cat([lat[rows].reshape(-1), keys[rows].reshape(-1)])
        tok_pos = torch.div(wl.tok_pos.to(torch.int64) - r, G, rounding_mode="floor")
        spec_r = dataclasses.replace(s, name=f"{s.name}_shard{r}of{G}", ctx_lens=lens,
                                     shared_prefix=0, duplicate_prefix=False)
        shards.append(Workload(spec_r, wl.seed, npg, pool, local_pt.to(torch.int32),
                               wl.q_offsets, tok_pos.to(torch.int32), wl.tok_req, wl.q_idx, wl.w,
                               wl.q))
    return shards
