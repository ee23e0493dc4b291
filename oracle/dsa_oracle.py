"""Plain, slow CPU oracle for the DSA sparse-attention decode/prefill path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code with the HIP library (no kernels,
headers, helpers, tables or constants are common to the two); the storage
format constants below are restated here from the format definition, not
imported.

Sources (the pages this follows):
  * "Accelerating GLM-5.3-Flash on H200" (lmsys.org blog), section 1
    "Architecture and workloads": DSA keeps historical KV and an indexer selects
    the relevant positions.
  * same page, section 3, "Larger KV tiles for DSA Partial": after the indexer
    selects KV positions, Partial loads them and computes Q K^T, an online
    softmax and the weighted value sum; KV splits produce intermediates that a
    Combine step merges; Figure 4: an index width that is not a multiple of the
    KV tile is covered by virtual padding, the physical index tensor unchanged.
  * "A million-token context on 16 H200s" (vLLM news summary), Interpretation:
    MLA's latent KV row is shared by all 64 heads.
  * "GLM-5.3-Flash" SGLang cookbook, section 2 "Size both memory pools" and
    "Extend the cache hierarchy": a paged KV pool plus a separate DSA indexer
    pool; FP8 KV cache is the default on MI355X.

The pages never write the formulas down.  Readings adopted where they are
silent (each is listed with its reason in the design notes of the repository):
  * indexer score  s[t,p] = sum_h w[t,h] * relu(q_I[t,h,:] . k_I[p,:])  over the
    visible positions p <= pos_t, one 128-d key per position shared by the 16
    indexer heads;
  * top-k keeps the k highest scores, ties going to the lower position; the
    result is returned in ascending position order and padded with -1;
  * attention:  z_j = sm_scale * q[h] . K[i_j]  over all 576 dims,
    o[h] = softmax(z) . K[i][:, :512],  lse[h] = log sum_j exp(z_j);
  * split s of S covers index columns [s*c, min(W,(s+1)*c)) with
    c = tile * ceil(ceil(W/tile)/S); an empty split yields (o=0, lse=-inf);
  * combine:  lse = logsumexp_s lse_s,  o = sum_s exp(lse_s - lse) * o_s;
  * FP8 rows: 576 OCP E4M3FN codes followed by nine little-endian fp32 scales,
    one per 64 consecutive elements; value = decode(code) * scale;
  * writing a new token into the cache (SGLang cookbook: FP8 KV cache by
    default; the quantizer itself is not spelled out): per group of 64 the
    scale is the smallest power of two 2^k with amax <= 448 * 2^k (k >= -126;
    1 if the group is all zero), stored as fp32, and code = E4M3FN(x / scale),
    rounded to the nearest finite value with ties to the even code (x / scale
    is exact and within +-448).  Power-of-two group scales are the block
    scales MI355X's FP8 conversion and matrix instructions apply themselves;
    the decode above (code times scale) reads any fp32 scale.
  * Q8 prefill (LMSYS page, section 4 "Prefill dataflow optimization", and its
    configuration table: FP8 query against the FP8 KV cache for prefill; the
    query quantizer is not spelled out): one fp32 scale per query head over
    its 576 elements, scale = amax / 448 (1 for an all-zero head) and
    code = E4M3FN(q / scale) with the cache's rounding rule.  The score is the
    product of the codes times both scales, i.e. the attention above with q
    replaced by its dequantized value decode(code) * scale; the value sum is
    unchanged.

All floating point here is float64 (numpy).  Indexer scores are returned as
float32 after an exact float64 computation (integer-valued inputs keep every
partial sum an exact integer below 2**24, so any summation order agrees).
"""

from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# Storage format, restated from its definition (page = 64 token slots).
# ---------------------------------------------------------------------------
PAGE_TOKENS = 64
HEADS = 64
D_LATENT = 512
D_ROPE = 64
D_QK = D_LATENT + D_ROPE          # 576
IDX_HEADS = 16
IDX_DIM = 128

KV_BF16 = 0
KV_FP8 = 1

FP8_GROUP = 64                    # one fp32 scale per 64 consecutive elements
FP8_NGROUPS = D_QK // FP8_GROUP   # 9
FP8_ROW_STRIDE = 640              # 576 codes + 36 scale bytes + 28 pad bytes
FP8_SCALE_OFFSET = 576
BF16_ROW_STRIDE = 2 * D_QK        # 1152
KEY_ROW_BYTES = 2 * IDX_DIM       # 256


def latent_row_stride(kv_dtype: int) -> int:
    return FP8_ROW_STRIDE if kv_dtype == KV_FP8 else BF16_ROW_STRIDE


def pool_plane_offsets(kv_dtype: int, num_pages: int) -> tuple[int, int, int]:
    """(latent plane offset, index plane offset, total bytes) of a pool buffer.

    The latent plane holds num_pages * 64 rows at the row stride; the indexer
    key plane follows it, 64 rows of 256 bytes per page, at the same page id.
    """
    latent_bytes = num_pages * PAGE_TOKENS * latent_row_stride(kv_dtype)
    index_bytes = num_pages * PAGE_TOKENS * KEY_ROW_BYTES
    return 0, latent_bytes, latent_bytes + index_bytes


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------
def e4m3fn_value(code: int) -> float:
    """Value of one OCP FP8 E4M3FN code: 1 sign, 4 exponent (bias 7), 3 mantissa
    bits; exponent field 0 encodes subnormals m/8 * 2**-6; S.1111.111 is NaN and
    there is no infinity (max finite 448)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3fn_table() -> np.ndarray:
    return np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


_E4M3 = e4m3fn_table()


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper half of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Pool addressing (paged KV pool + page table)
# ---------------------------------------------------------------------------
class PoolView:
    """Host view of pool bytes: logical (request b, position p) -> page
    page_table[b][p // 64], slot p % 64."""

    def __init__(self, pool_bytes: np.ndarray, num_pages: int, kv_dtype: int):
        self.buf = np.asarray(pool_bytes, dtype=np.uint8).reshape(-1)
        self.num_pages = int(num_pages)
        self.kv_dtype = int(kv_dtype)
        self.stride = latent_row_stride(kv_dtype)
        self.lat_off, self.idx_off, total = pool_plane_offsets(kv_dtype, num_pages)
        assert self.buf.size >= total, (self.buf.size, total)

    def _phys_rows(self, page_row: np.ndarray, positions: np.ndarray) -> np.ndarray:
        positions = np.asarray(positions, dtype=np.int64)
        pages = np.asarray(page_row, dtype=np.int64)[positions // PAGE_TOKENS]
        assert np.all((pages >= 0) & (pages < self.num_pages))
        return pages * PAGE_TOKENS + positions % PAGE_TOKENS

    def latent_rows(self, page_row, positions) -> np.ndarray:
        """Dequantized latent rows [n, 576] (float64)."""
        phys = self._phys_rows(page_row, positions)
        if phys.size == 0:
            return np.zeros((0, D_QK))
        starts = self.lat_off + phys * self.stride
        raw = self.buf[starts[:, None] + np.arange(self.stride)[None, :]]
        if self.kv_dtype == KV_BF16:
            bits = raw[:, :2 * D_QK].copy().view(np.uint16)
            return bf16_bits_to_f64(bits)
        codes = raw[:, :D_QK]
        scales = raw[:, FP8_SCALE_OFFSET:FP8_SCALE_OFFSET + 4 * FP8_NGROUPS].copy()
        scales = scales.view('<f4').astype(np.float64)            # [n, 9]
        vals = _E4M3[codes]                                        # [n, 576]
        group = np.arange(D_QK) // FP8_GROUP
        return vals * scales[:, group]

    def index_keys(self, page_row, positions) -> np.ndarray:
        """Indexer keys [n, 128] (float64)."""
        phys = self._phys_rows(page_row, positions)
        if phys.size == 0:
            return np.zeros((0, IDX_DIM))
        starts = self.idx_off + phys * KEY_ROW_BYTES
        raw = self.buf[starts[:, None] + np.arange(KEY_ROW_BYTES)[None, :]]
        return bf16_bits_to_f64(raw.copy().view(np.uint16))


# ---------------------------------------------------------------------------
# Step 1: indexer scores
# ---------------------------------------------------------------------------
def index_scores(q_idx: np.ndarray, w: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Scores of one query token against keys [n,128].

    s[p] = sum_h w[h] * max(0, q_idx[h,:] . keys[p,:]); q_idx [16,128], w [16].
    Computed in float64, returned as float32.
    """
    q_idx = np.asarray(q_idx, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dots = np.asarray(keys, dtype=np.float64) @ q_idx.T          # [n, 16]
    s = np.maximum(dots, 0.0) @ w                                 # [n]
    return s.astype(np.float32)


# ---------------------------------------------------------------------------
# Step 2: top-k
# ---------------------------------------------------------------------------
def topk_positions(scores: np.ndarray, k: int) -> np.ndarray:
    """The k visible positions with the highest score, ties to the lower
    position, returned ascending and padded with -1 to length k."""
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[0]
    pos = np.arange(n)
    order = np.lexsort((pos, -scores))        # primary: score desc; then pos asc
    keep = np.sort(order[:min(k, n)])
    out = np.full(k, -1, dtype=np.int32)
    out[:keep.size] = keep
    return out


def dcp_merge(shard_lists, k: int) -> np.ndarray:
    """Global selection from round-robin KV shards ("A million-token context on
    16 H200s", Interpretation: the cache is sharded by token, each of G ranks
    holding every G-th position).  shard_lists[r] = (global positions, scores)
    of shard r's own top-k; the result is the k best of their union under the
    same rule as topk_positions (score desc, position asc), ascending, padded
    with -1 to length k."""
    pos = np.concatenate([np.asarray(p, dtype=np.int64) for p, _ in shard_lists])
    sc = np.concatenate([np.asarray(v, dtype=np.float64) for _, v in shard_lists])
    order = np.lexsort((pos, -sc))
    keep = np.sort(pos[order[:min(k, pos.size)]])
    out = np.full(k, -1, dtype=np.int32)
    out[:keep.size] = keep
    return out


# ---------------------------------------------------------------------------
# Step 3: attention over the selected rows, split-KV partials and combine
# ---------------------------------------------------------------------------
def attend(q: np.ndarray, rows: np.ndarray, sm_scale: float):
    """Softmax attention of 64 heads over rows [m,576].

    Returns (o [64,512], lse [64]); an empty row set gives (0, -inf)."""
    q = np.asarray(q, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64)
    if rows.shape[0] == 0:
        return np.zeros((q.shape[0], D_LATENT)), np.full(q.shape[0], -np.inf)
    z = sm_scale * (q @ rows.T)                                   # [64, m]
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    denom = e.sum(axis=1, keepdims=True)
    p = e / denom
    o = p @ rows[:, :D_LATENT]
    lse = (zmax + np.log(denom))[:, 0]
    return o, lse


def num_iterations(width: int, tile: int) -> int:
    """Loop iterations that cover an index width with KV tiles of `tile`."""
    return -(-int(width) // int(tile))


def virtual_columns(width: int, tile: int) -> int:
    """Columns covered by the loop, the last tile's tail being virtual padding."""
    return num_iterations(width, tile) * int(tile)


def split_bounds(width: int, tile: int, splits: int):
    """Contiguous, tile-aligned column ranges of the S splits."""
    per = -(-num_iterations(width, tile) // int(splits))
    c = per * int(tile)
    return [(min(width, s * c), min(width, (s + 1) * c)) for s in range(int(splits))]


def valid_mask(idx_cols: np.ndarray, pos: int) -> np.ndarray:
    """Index entries outside [0, pos] (including the -1 padding) are masked."""
    idx_cols = np.asarray(idx_cols, dtype=np.int64)
    return (idx_cols >= 0) & (idx_cols <= pos)


def partial(q, idx_row, pos, rows_of, sm_scale, tile, splits):
    """Split-KV partials of one token: (o_part [S,64,512], lse_part [S,64]).

    rows_of(positions) returns the dequantized latent rows of those positions.
    """
    o_parts = np.zeros((splits, q.shape[0], D_LATENT))
    lse_parts = np.full((splits, q.shape[0]), -np.inf)
    idx_row = np.asarray(idx_row, dtype=np.int64)
    for s, (a, b) in enumerate(split_bounds(idx_row.shape[0], tile, splits)):
        cols = idx_row[a:b]
        cols = cols[valid_mask(cols, pos)]
        o_parts[s], lse_parts[s] = attend(q, rows_of(cols), sm_scale)
    return o_parts, lse_parts


def combine(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Merge split partials: lse = logsumexp_s lse_s, o = sum_s e^(lse_s-lse) o_s."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)                                     # [64]
    finite = np.isfinite(m)
    safe_m = np.where(finite, m, 0.0)
    wts = np.where(np.isfinite(lse_parts), np.exp(lse_parts - safe_m[None, :]), 0.0)
    tot = wts.sum(axis=0)
    lse = np.where(finite, safe_m + np.log(np.where(finite, tot, 1.0)), -np.inf)
    o = np.einsum('sh,shd->hd', wts, o_parts)
    o = np.where(finite[:, None], o / np.where(finite, tot, 1.0)[:, None], 0.0)
    return o, lse


# ---------------------------------------------------------------------------
# The whole per-token path
# ---------------------------------------------------------------------------
def token_path(pool: PoolView, page_row, pos: int, q_idx, w, q, k: int,
               sm_scale: float, tile: int = 64, splits: int = 1):
    """Indexer -> top-k -> partial -> combine for one query token.

    Returns dict(scores [pos+1] f32, idx [k] i32, o [64,512] f64, lse [64] f64).
    """
    visible = np.arange(pos + 1)
    keys = pool.index_keys(page_row, visible)
    scores = index_scores(q_idx, w, keys)
    idx = topk_positions(scores, k)
    o_p, lse_p = partial(np.asarray(q, np.float64), idx, pos,
                         lambda cols: pool.latent_rows(page_row, cols),
                         sm_scale, tile, splits)
    o, lse = combine(o_p, lse_p)
    return dict(scores=scores, idx=idx, o=o, lse=lse)


# ---------------------------------------------------------------------------
# Writing new tokens into the cache (quantize + append)
# ---------------------------------------------------------------------------
_E4M3_POS = _E4M3[:0x7F]          # codes 0x00..0x7E: the finite non-negative values, ascending


def e4m3fn_encode(y) -> np.ndarray:
    """Nearest E4M3FN code of each float value: the finite code whose value is
    closest to y (ties to the code with an even last bit), |y| saturated at 448,
    the sign bit taken from y (so -0.0 and small negative values give 0x80)."""
    y = np.asarray(y, dtype=np.float64)
    mag = np.minimum(np.abs(y), 448.0)
    hi = np.searchsorted(_E4M3_POS, mag, side="left")          # first value >= mag
    hi = np.minimum(hi, len(_E4M3_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(y), code | np.uint8(0x80), code).astype(np.uint8)


def fp8_group_scale(amax) -> np.ndarray:
    """Cache group scale: the smallest 2^k (k >= -126) with amax <= 448 * 2^k,
    by exact comparison; 1 for amax = 0.  float32."""
    amax = np.asarray(amax, dtype=np.float64)
    k = np.zeros(amax.shape, dtype=np.int64)
    for i, a in np.ndenumerate(amax):
        if a > 0:
            kk = -126
            while a > 448.0 * 2.0 ** kk:
                kk += 1
            k[i] = kk
    return np.ldexp(np.float32(1.0), k).astype(np.float32)


def quantize_fp8_row(x) -> tuple[np.ndarray, np.ndarray]:
    """One 576-element row (any float input; the GPU path takes bf16) -> (codes
    uint8[576], scales float32[9]); x / scale is exact (a power of two)."""
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64).reshape(FP8_NGROUPS, FP8_GROUP)
    scale = fp8_group_scale(np.abs(x64).max(axis=1))
    return e4m3fn_encode(x64 / scale[:, None].astype(np.float64)).reshape(D_QK), scale


def quantize_q8(q) -> tuple[np.ndarray, np.ndarray]:
    """Q8 query quantizer: q [..., 576] (any float input; the GPU path takes
    bf16) -> (codes uint8 [..., 576], scales float32 [...]), one scale per
    query head, formed like the cache's per-group scale: amax / 448 in fp32,
    1 when the head is all zero, codes = E4M3FN(q / scale) with q / scale in
    fp32."""
    x32 = np.asarray(q, dtype=np.float32)
    amax = np.abs(x32).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    y = (x32 / scale[..., None]).astype(np.float32)
    return e4m3fn_encode(y), scale


def dequantize_q8(codes, scales) -> np.ndarray:
    """decode(code) * scale in float64: the query the Q8 score multiplies
    (the product of two codes times the two scales equals this value times
    the dequantized cache element exactly)."""
    return _E4M3[np.asarray(codes)] * np.asarray(scales, dtype=np.float64)[..., None]


def token_path_q8(pool: PoolView, page_row, pos: int, idx, q_codes, q_scales,
                  sm_scale: float, tile: int = 64):
    """Q8 sparse attention of one query token over given index columns: the
    attention of the dequantized FP8 query, one split.
    Returns dict(o [64,512] f64, lse [64] f64)."""
    o_p, lse_p = partial(dequantize_q8(q_codes, q_scales), np.asarray(idx), pos,
                         lambda cols: pool.latent_rows(page_row, cols),
                         sm_scale, tile, 1)
    o, lse = combine(o_p, lse_p)
    return dict(o=o, lse=lse)


def append_rows(pool: PoolView, page_table: np.ndarray, req, pos, latent, keys=None):
    """Write rows into the pool bytes in place: row i goes to request req[i],
    position pos[i] (page page_table[req[i]][pos[i] // 64], slot pos[i] % 64).
    latent: [n, 576] floats (bf16 values for a BF16 pool); keys: [n, 128]
    bf16 bit patterns or None.  Rows whose request, position or page id is out
    of range are skipped."""
    pt = np.asarray(page_table)
    for i in range(len(req)):
        b, p = int(req[i]), int(pos[i])
        if not (0 <= b < pt.shape[0] and 0 <= p and p // PAGE_TOKENS < pt.shape[1]):
            continue
        page = int(pt[b, p // PAGE_TOKENS])
        if not (0 <= page < pool.num_pages):
            continue
        phys = page * PAGE_TOKENS + p % PAGE_TOKENS
        at = pool.lat_off + phys * pool.stride
        if pool.kv_dtype == KV_FP8:
            codes, scales = quantize_fp8_row(latent[i])
            row = np.zeros(pool.stride, dtype=np.uint8)
            row[:D_QK] = codes
            row[FP8_SCALE_OFFSET:FP8_SCALE_OFFSET + 4 * FP8_NGROUPS] = scales.astype('<f4').view(np.uint8)
        else:
            row = np.asarray(latent[i], dtype=np.float32).view(np.uint32) >> np.uint32(16)
            row = row.astype(np.uint16).view(np.uint8)
            assert np.array_equal(bf16_bits_to_f64(row.view(np.uint16)),
                                  np.asarray(latent[i], dtype=np.float64)), "BF16 pool takes bf16 values"
        pool.buf[at:at + pool.stride] = row
        if keys is not None:
            ka = pool.idx_off + phys * KEY_ROW_BYTES
            pool.buf[ka:ka + KEY_ROW_BYTES] = np.asarray(keys[i], dtype=np.uint16).view(np.uint8)
