/*
 * dsa.h - C ABI of the DSA (DeepSeek-style sparse attention) hot path on
 * AMD MI355X (gfx950).
 *
 * Per query token the path is: an indexer scores every visible cached
 * position, a top-k keeps the best positions, 64 attention heads attend over
 * only the selected rows of a shared MLA latent KV cache (split-KV partials),
 * and a combine step merges the partials.  Sources:
 *   [LMSYS-1] lmsys.org, "Accelerating GLM-5.3-Flash on H200", section 1
 *             "Architecture and workloads" (DSA stores historical KV; an
 *             indexer selects relevant positions).
 *   [LMSYS-2] same page, section 2 "Turning cache capacity into concurrency",
 *             "KV-only decode RadixCache" (prefix KV shared across requests;
 *             Lp + N*Ls slots instead of N*(Lp+Ls)).
 *   [LMSYS-3] same page, section 3, "Larger KV tiles for DSA Partial" and its
 *             Figure 4 (Partial = gather selected KV, QK^T, online softmax,
 *             weighted value sum; KV tile 32 or 128; index width not padded
 *             physically; splits add intermediate writes merged by Combine;
 *             dispatch from architecture, layout and query parallelism).
 *   [LMSYS-4] same page, section 4 "Prefill dataflow optimization" and the
 *             prefill configuration table (Q8 sparse attention: the DSA
 *             prefill backend takes an FP8 query over the FP8 E4M3 KV cache).
 *   [VLLM]    "A million-token context on 16 H200s", Interpretation (MLA's
 *             latent KV row is shared by all 64 heads).
 *   [SGL]     SGLang cookbook "GLM-5.3-Flash", section 2 "Size both memory
 *             pools", "Keep the KV and DSA backends paired", "Extend the cache
 *             hierarchy" (paged KV pool, separate DSA indexer pool, FP8 KV on
 *             MI355X, BF16 KV elsewhere).
 *
 * Conventions shared by every entry point:
 *   - Pointers are DEVICE pointers unless the argument says "host".
 *   - The caller owns all device memory (allocated with PyTorch or hipMalloc);
 *     the library never allocates device memory and never synchronizes (its
 *     one device buffer of its own, the scratch of dsa_topk_noalloc, is a
 *     static array of the code object, not an allocation).
 *   - Compute entry points only enqueue work on `stream` (a hipStream_t passed
 *     as void*, NULL = the default stream); DSA_OK means "enqueued".
 *   - Every argument is validated on the host before anything is enqueued; on
 *     an error nothing is launched, the status is returned and a message is
 *     kept for dsa_last_error() (thread-local).
 *   - Page ids and token positions in device memory are trusted: a kernel
 *     clamps an out-of-range page id into the pool rather than fault.  With
 *     the environment variable DSA_VALIDATE=1, the calls that read the page
 *     table (dsa_index_scores, dsa_index_topk, dsa_sparse_mla_partial,
 *     dsa_sparse_mla) first wait for the work queued on `stream`, copy
 *     q_offsets, tok_pos and the page table to the host and check that
 *     q_offsets runs from 0 to num_tokens without decreasing, that every
 *     tok_pos is in [-1, pt_stride*64) and that every page id a token can
 *     reach (logical pages 0 .. tok_pos/64 of its request) is in
 *     [0, num_pages); otherwise they return DSA_ERR_INVALID_ARG and launch
 *     nothing.  A debugging aid: it synchronizes, so it is not for graph
 *     capture or timing.
 *   - Model dimensions are fixed: 64 heads, latent 512 + rope 64 (q/k dim
 *     576, v dim 512), indexer 16 heads x 128, 64-token pages.
 *   - bf16 values are passed as uint16_t bit patterns.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 1

#define DSA_PAGE_TOKENS 64
#define DSA_HEADS 64
#define DSA_D_LATENT 512
#define DSA_D_ROPE 64
#define DSA_D_QK 576
#define DSA_IDX_HEADS 16
#define DSA_IDX_DIM 128

typedef int32_t dsa_status;
enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, negative size, bad enum */
  DSA_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels implement */
  DSA_ERR_NO_SPACE = 3,    /* pool exhausted (allocation is all-or-nothing) */
  DSA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required */
  DSA_ERR_HIP = 5          /* a HIP runtime call or launch failed */
};

/* KV element formats [SGL "Keep the KV and DSA backends paired"]. */
enum {
  DSA_KV_BF16 = 0,         /* 576 bf16 per row */
  DSA_KV_FP8_E4M3_S64 = 1  /* 576 OCP E4M3FN codes + 9 fp32 scales (one per 64) */
};
/* FP8 rows: element d = decode(code[d]) * scale[d/64].  The scales are
 * powers of two (what dsa_kv_append writes): the attention kernels apply them
 * as block scales, i.e. only their exponent, so a row written with any other
 * fp32 scale is read with that scale rounded down to a power of two. */

int32_t dsa_abi_version(void);
/* Message of the last non-OK status on this thread ("" if none). */
const char* dsa_last_error(void);
const char* dsa_status_string(dsa_status s);

/* ------------------------------------------------------------------------
 * Paged KV pool [SGL "Size both memory pools"; LMSYS-2].
 *
 * One caller-owned device buffer holds two planes addressed by the same page
 * id: the latent plane (num_pages * 64 rows at latent_row_stride bytes) and,
 * after it, the indexer-key plane (num_pages * 64 rows of 128 bf16).
 * Latent row formats:
 *   BF16: 576 bf16 (1152 bytes), stride 1152.
 *   FP8 : bytes [0,576) E4M3FN codes, [576,612) nine little-endian fp32
 *         scales (element c has value decode(code[c]) * scale[c/64]),
 *         [612,640) padding; stride 640 (five 128-byte lines).
 * Logical position p of request b lives at page page_table[b][p/64], slot
 * p%64.  Page contents are written by the caller through this layout.
 * ------------------------------------------------------------------------ */
typedef struct dsa_pool_layout {
  int32_t page_tokens;        /* 64 */
  int32_t kv_dtype;
  int32_t d_latent, d_rope, d_index;     /* 512, 64, 128 */
  int32_t latent_row_bytes;   /* algorithmic bytes per row: 612 (FP8) or 1152 */
  int32_t latent_row_stride;  /* 640 (FP8) or 1152 */
  int32_t scale_offset;       /* 576 for FP8, -1 for BF16 */
  int32_t index_row_bytes;    /* 256 */
  int32_t reserved;
  int64_t latent_plane_offset;  /* 0 */
  int64_t index_plane_offset;   /* num_pages * 64 * latent_row_stride */
  int64_t total_bytes;          /* bytes the pool buffer must hold */
} dsa_pool_layout;

/* Host-only.  Fills *out (host) for num_pages pages of kv_dtype. */
dsa_status dsa_pool_layout_query(int32_t kv_dtype, int32_t num_pages, dsa_pool_layout* out);

typedef struct dsa_pool dsa_pool; /* opaque host object owned by the library */

/* Host-only.  Wraps the caller's device buffer `dev_base` (256-byte aligned,
 * at least total_bytes long) as a pool of num_pages pages, all free.
 * *out receives a handle to release with dsa_pool_destroy. */
dsa_status dsa_pool_create(void* dev_base, int64_t bytes, int32_t num_pages,
                           int32_t kv_dtype, dsa_pool** out);
void dsa_pool_destroy(dsa_pool* pool);
/* Host-only page bookkeeping [LMSYS-2 prefix sharing]:
 *   alloc   - take n free pages (refcount 1), ids written to host array ids;
 *             all-or-nothing: DSA_ERR_NO_SPACE leaves the pool unchanged.
 *   share   - refcount++ of n live pages (a request reusing prefix pages).
 *   release - refcount-- of n live pages; a page returns to the free list at 0.
 *             Releasing a free page is DSA_ERR_INVALID_ARG and changes nothing. */
dsa_status dsa_pool_alloc(dsa_pool* pool, int32_t n, int32_t* ids /* host out */);
dsa_status dsa_pool_share(dsa_pool* pool, const int32_t* ids /* host */, int32_t n);
dsa_status dsa_pool_release(dsa_pool* pool, const int32_t* ids /* host */, int32_t n);
int32_t dsa_pool_free_pages(const dsa_pool* pool);
int32_t dsa_pool_refcount(const dsa_pool* pool, int32_t page_id); /* -1 if out of range */
int32_t dsa_pool_num_pages(const dsa_pool* pool);
int32_t dsa_pool_kv_dtype(const dsa_pool* pool);

/* ------------------------------------------------------------------------
 * Batch description shared by the compute calls.
 *   num_reqs requests; request b owns query tokens [q_offsets[b],
 *   q_offsets[b+1]) (q_offsets: device int32[num_reqs+1], nondecreasing,
 *   q_offsets[0] = 0, q_offsets[num_reqs] = num_tokens).
 *   tok_pos: device int32[num_tokens], the absolute position of each query
 *   token; it sees positions [0, tok_pos[t]] of its request (causal, itself
 *   included).
 *   page_table: device int32[num_reqs * pt_stride]; entry [b][j] is the page of
 *   logical page j of request b; entries past ceil((tok_pos+1)/64) are never
 *   read.
 *   max_q: host bound on tokens per request; max_ctx: host bound on
 *   tok_pos[t] + 1 (both size the launch grid; tokens beyond them are not
 *   processed).
 * ------------------------------------------------------------------------ */

/* Indexer scores [LMSYS-1; VLLM: the indexer stays whole across GPUs]:
 *   scores[t*ld + p] = sum_{h<16} w[t*16+h] * max(0, q_idx[t,h,:] . key(p))
 * for p in [0, min(tok_pos[t], max_ctx-1)]; entries past that are not written.
 * q_idx: bf16 [num_tokens,16,128]; w: fp32 [num_tokens,16]; key(p) is the
 * 128-d bf16 indexer key of position p of the token's request.  Products are
 * accumulated in fp32 (never rounded through bf16): integer-valued inputs
 * whose partial sums stay below 2^24 give exact results.
 * ld >= max_ctx, ld % 4 == 0; scores 16-byte aligned. */
dsa_status dsa_index_scores(const dsa_pool* pool, const int32_t* page_table, int32_t pt_stride,
                            const int32_t* q_offsets, int32_t num_reqs, int32_t max_q,
                            const int32_t* tok_pos, int32_t num_tokens, int32_t max_ctx,
                            const uint16_t* q_idx, const float* w, float* scores, int64_t ld,
                            void* stream);

/* Top-k over each token's visible scores [LMSYS-1 indexer selection; the
 * blog's "top-k v2" change]: the k positions with the highest score among
 * [0, min(tok_pos[t], max_ctx-1)], ties going to the lower position, written
 * to idx[t*k ..] in ascending position order and padded with -1 when fewer
 * than k positions are visible.  Scores are compared as fp32 (NaN unsupported).
 * Rows longer than 65,536 positions use `workspace` (device, 256-byte
 * aligned) of at least dsa_topk_workspace_bytes() bytes; 0 bytes otherwise.
 * Limits: 1 <= k <= 16384; max_ctx <= 65536 * (65536 / k) (2,097,152 at
 * k = 2048). */
size_t dsa_topk_workspace_bytes(int32_t num_tokens, int32_t max_ctx, int32_t k);
dsa_status dsa_topk(const float* scores, int64_t ld, const int32_t* tok_pos, int32_t num_tokens,
                    int32_t max_ctx, int32_t k, int32_t* idx, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Allocation-free top-k, for callers that cannot allocate device memory
 * (code under graph capture, tight serving loops, harnesses that forbid
 * allocation): dsa_topk without the workspace argument.  The long-row
 * staging (rows above 65,536 positions: dsa_topk_workspace_bytes(num_tokens,
 * max_ctx, k) bytes) lives in a library-owned device array of
 * DSA_TOPK_SCRATCH_BYTES per GPU, held until the process ends; a call that
 * needs more returns DSA_ERR_WORKSPACE (e.g. 1,048,576-position rows at
 * k = 2048 fit 64 tokens per call).  The call allocates nothing.  Every call
 * on one GPU shares that GPU's array: calls that overlap on one GPU (on
 * different streams, or from several threads) race and must be ordered by
 * the caller.  Results are bit for bit those of dsa_topk. */
#define DSA_TOPK_SCRATCH_BYTES (16u << 20)
dsa_status dsa_topk_noalloc(const float* scores, int64_t ld, const int32_t* tok_pos,
                            int32_t num_tokens, int32_t max_ctx, int32_t k, int32_t* idx,
                            void* stream);

/* Fused indexer + top-k [LMSYS-1 indexer and selection; the blog's "top-k
 * v2" change; the fused selection is this library's design]: the same idx as
 * dsa_index_scores followed by dsa_topk (bit for bit), without a score
 * matrix.  Arguments are those two calls' (scores/ld dropped), plus:
 *   cap: candidate slots per token and 512-position chunk, 1..128 (128 is
 *     ample for k = 2048 rows of 16K+ positions; denser rows overflow and
 *     take the fallback);
 *   cand_target: how many candidates per row the sampled threshold aims at,
 *     or 0 = 2k.
 * How: an indexer pass over one page in 32 gives per-token sample scores;
 * their rank statistic sets a threshold; a full indexer pass keeps only the
 * positions that reach it; an exact selection over those candidates gives the
 * top-k whenever no chunk overflowed `cap` and at least k candidates exist.
 * Other tokens are recomputed exactly by a one-workgroup-per-token fallback.
 * max_ctx <= 65536 (DSA_ERR_UNSUPPORTED above).  workspace: device, 256-byte
 * aligned, at least dsa_index_topk_workspace_bytes(num_tokens, max_ctx, cap)
 * bytes, caller-owned; after the call completes its first int32 holds the
 * number of tokens that took the fallback.  Calls sharing a workspace must
 * be ordered on one stream. */
size_t dsa_index_topk_workspace_bytes(int32_t num_tokens, int32_t max_ctx, int32_t cap);
dsa_status dsa_index_topk(const dsa_pool* pool, const int32_t* page_table, int32_t pt_stride,
                          const int32_t* q_offsets, int32_t num_reqs, int32_t max_q,
                          const int32_t* tok_pos, int32_t num_tokens, int32_t max_ctx,
                          const uint16_t* q_idx, const float* w, int32_t k, int32_t cap,
                          int32_t cand_target, int32_t* idx, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Dispatch plan of the Partial step [LMSYS-3 and Figure 4].  Host-only.
 *   kv_tile: 32, 64 or 128 KV entries per loop iteration, or 0 = choose
 *   (32 when num_tokens >= cu_count or width < 1024, else 64).  Splits are
 *   cut at multiples of the tile; tiles of 32 and 128 run the same kernel,
 *   which moves rows through LDS 32 at a time.
 *   num_splits: KV splits per token, or 0 = choose from query parallelism
 *   (num_tokens) and cu_count (0 = 256, MI355X): 1 when num_tokens >=
 *   cu_count, else about one workgroup per CU with at least two tiles per
 *   split: min(ceil(cu_count/num_tokens), iters_total/2), at least 1.
 * Output (host): tile, splits, iters_total = ceil(width/tile), iters_per_split
 * = ceil(iters_total/splits), cols_per_split = tile*iters_per_split,
 * virtual_cols = tile*iters_total, padding_cols = virtual_cols - width.
 * Split s covers index columns [s*cols_per_split, min(width,(s+1)*cols_per_split)). */
typedef struct dsa_partial_plan {
  int32_t tile, splits, iters_total, iters_per_split;
  int32_t cols_per_split, virtual_cols, padding_cols, reserved;
} dsa_partial_plan;
dsa_status dsa_plan_partial(int32_t num_tokens, int32_t width, int32_t kv_tile,
                            int32_t num_splits, int32_t cu_count, dsa_partial_plan* out);

/* Sparse MLA Partial [LMSYS-3; VLLM head sharing].  For token t, split s and
 * head h, over the valid columns j of split s:
 *   z_j = sm_scale * q[t,h,:] . K(idx[t*width + j])        (576-d)
 *   o_part[t,s,h,:] = sum_j softmax(z)_j * K(idx[..j])[0:512]   (normalized)
 *   lse_part[t,s,h] = ln sum_j exp(z_j)
 * K(p) is the dequantized latent row of position p of the token's request.
 * An index entry is valid when 0 <= idx <= tok_pos[t]; others (including -1
 * padding) are skipped, repeats count each time.  The index tensor is
 * consumed as is: width need not be a multiple of the tile (the loop's last
 * tile is padded virtually).  A split with no valid column yields o = 0,
 * lse = -inf.  sm_scale must be finite and > 0.  kv_tile and num_splits
 * must be the resolved values of a plan (kv_tile in {32, 64, 128};
 * num_splits >= 1).
 * q: bf16 [num_tokens,64,576]; idx: int32 [num_tokens,width];
 * o_part: fp32 [num_tokens,num_splits,64,512]; lse_part: fp32
 * [num_tokens,num_splits,64].  All 16-byte aligned. */
dsa_status dsa_sparse_mla_partial(const dsa_pool* pool, const int32_t* page_table,
                                  int32_t pt_stride, const int32_t* q_offsets, int32_t num_reqs,
                                  const int32_t* tok_pos, int32_t num_tokens, const uint16_t* q,
                                  const int32_t* idx, int32_t width, float sm_scale,
                                  int32_t kv_tile, int32_t num_splits, float* o_part,
                                  float* lse_part, void* stream);

/* Sparse MLA in one pass over each token's index row [LMSYS-3: with a single
 * split there are no intermediates and no Combine work]: the same attention
 * as dsa_sparse_mla_partial with num_splits = 1 followed by dsa_combine, and
 * bit for bit the same result (Combine of one split multiplies by exp(0) = 1
 * and adds log 1 = 0), without the fp32 intermediates.  Same arguments and
 * errors as dsa_sparse_mla_partial; kv_tile in {32, 64, 128}.
 * out: bf16 [num_tokens,64,512]; lse: fp32 [num_tokens,64] (natural log).
 * q 16-byte aligned; out, lse 4-byte aligned. */
dsa_status dsa_sparse_mla(const dsa_pool* pool, const int32_t* page_table, int32_t pt_stride,
                          const int32_t* q_offsets, int32_t num_reqs, const int32_t* tok_pos,
                          int32_t num_tokens, const uint16_t* q, const int32_t* idx,
                          int32_t width, float sm_scale, int32_t kv_tile, uint16_t* out,
                          float* lse, void* stream);

/* Q8 prefill [LMSYS-4 "Prefill dataflow optimization": the prefill attention
 * takes an FP8 query against the FP8 KV cache; the query quantizer is not
 * spelled out by the pages, the reading here: one fp32 scale per (token,
 * head) over its 576 elements, scale = amax/448 (1 for an all-zero head),
 * code = E4M3FN(q/scale) rounded to nearest, ties to even, saturating at 448,
 * the same rounding as the cache rows].
 *
 * dsa_quantize_q8: q bf16 [num_tokens,64,576] (2-byte aligned) -> q_codes
 * uint8 [num_tokens,64,576] and q_scales fp32 [num_tokens,64] (4-byte
 * aligned).  Caller-owned device buffers; num_tokens = 0 launches nothing.
 *
 * dsa_sparse_mla_q8: the attention of dsa_sparse_mla (one split, final bf16
 * output and natural-log lse, same index validity rules) with the score
 *   z_j = sm_scale * q_scale[t,h] * sum_d code[t,h,d] * K(idx_j)[d]
 * i.e. q replaced by its dequantized value decode(code) * q_scale; the value
 * sum uses the dequantized latent as in dsa_sparse_mla.  FP8 pools only
 * (a BF16 pool is DSA_ERR_INVALID_ARG).  Tiles of 32 rows; no kv_tile or
 * split arguments.  q_codes 16-byte aligned; q_scales, idx, out, lse 4-byte.
 * Errors as dsa_sparse_mla. */
dsa_status dsa_quantize_q8(const uint16_t* q, int32_t num_tokens, uint8_t* q_codes,
                           float* q_scales, void* stream);
dsa_status dsa_sparse_mla_q8(const dsa_pool* pool, const int32_t* page_table, int32_t pt_stride,
                             const int32_t* q_offsets, int32_t num_reqs, const int32_t* tok_pos,
                             int32_t num_tokens, const uint8_t* q_codes, const float* q_scales,
                             const int32_t* idx, int32_t width, float sm_scale, uint16_t* out,
                             float* lse, void* stream);

/* Combine [LMSYS-3]: per token and head,
 *   lse = ln sum_s exp(lse_part_s),  out = sum_s exp(lse_part_s - lse) * o_part_s
 * with splits whose lse is -inf contributing nothing (all -inf: out = 0,
 * lse = -inf).  out: bf16 [num_tokens,64,512] (round to nearest even);
 * lse: fp32 [num_tokens,64]. */
dsa_status dsa_combine(const float* o_part, const float* lse_part, int32_t num_tokens,
                       int32_t num_splits, uint16_t* out, float* lse, void* stream);

/* DCP shard layout on one GPU [VLLM Interpretation: the KV cache sharded
 * round-robin by token, each of G ranks holding every G-th position].
 * Shard r holds positions p = j*G + r at local position j; each shard runs
 * dsa_index_scores + dsa_topk on its local positions (local tok_pos
 * floor((tok_pos - r) / G), -1 when tok_pos < r).
 *
 * dsa_dcp_merge: the global top-k from the shards' local top-k lists, exactly
 * what dsa_topk gives over the whole row (same tie rule and order): the union
 * of the local lists contains it.  Inputs: local_idx [G][T][k] int32 (each
 * shard's dsa_topk output: ascending local positions, -1 padded),
 * local_scores [G][T][ld] fp32 (each shard's dsa_index_scores output).
 * Outputs: idx [T][k] (global positions ascending, -1 padded) and, unless
 * shard_idx is NULL, shard_idx [G][T][k]: the local positions of each
 * shard's selected rows, ascending, -1 padded - the index each shard's
 * dsa_sparse_mla_partial reads.  Limits: 1 <= G <= 16, G*k <= 16384.
 *
 * dsa_combine_shards: dsa_combine over shard-major partials, o_part
 * [G][T][64][512] and lse_part [G][T][64] (shard r's single-split
 * dsa_sparse_mla_partial writes the [T] slab r). */
dsa_status dsa_dcp_merge(int32_t num_shards, int32_t num_tokens, int32_t k,
                         const int32_t* local_idx, const float* local_scores, int64_t ld,
                         int32_t* idx, int32_t* shard_idx, void* stream);
dsa_status dsa_combine_shards(const float* o_part, const float* lse_part, int32_t num_tokens,
                              int32_t num_shards, uint16_t* out, float* lse, void* stream);

/* Writing new tokens into the cache [SGL "Size both memory pools": the paged
 * KV pool, FP8 by default on MI355X, and the separate DSA indexer pool].  Row i of the batch goes to
 * request req[i], position pos[i]: page page_table[req[i]*pt_stride +
 * pos[i]/64], slot pos[i] % 64, in both planes.
 *   latent: bf16 [n,576] (512 latent + 64 rope), 16-byte aligned;
 *   keys:   bf16 [n,128] indexer keys, 16-byte aligned, or NULL to leave the
 *           indexer plane untouched.
 * FP8 pools (reading of the quantizer, not spelled out by the pages): per 64
 * consecutive elements the scale is the smallest power of two 2^k
 * (k >= -126) with amax <= 448 * 2^k (1 for an all-zero group), stored as
 * fp32, and code = E4M3FN(x/scale) rounded to the nearest finite value, ties
 * to the even code (x/scale is exact and within +-448); the nine scales
 * follow the codes and the 28 pad bytes are written as 0.  BF16 pools: the
 * 576 values are copied.  Rows whose request (outside [0,num_reqs)),
 * position (negative or past the page table) or page id (outside the pool)
 * is out of range are skipped.  Two rows with one destination: unspecified
 * which lands.  Asynchronous on `stream` like every compute call. */
dsa_status dsa_kv_append(const dsa_pool* pool, const int32_t* page_table, int32_t pt_stride,
                         int32_t num_reqs, const int32_t* req, const int32_t* pos, int32_t n,
                         const uint16_t* latent, const uint16_t* keys, void* stream);

/* Measurement utility, not a step of the path: the denominator that the
 * HBM-bound kernels' rooflines are compared against beside the vendor peak.
 * Reads `bytes` of device memory at `buf` once, in 16-byte loads spread over
 * `num_blocks` workgroups of 256 threads (a grid-stride loop), and writes one
 * uint32 per workgroup (the XOR of the words it read) to out[0..num_blocks).
 * buf and out: device, buf 16-byte aligned, bytes a multiple of 16 (0: no
 * launch); num_blocks in [1, 65536].  DSA_ERR_INVALID_ARG otherwise.
 * Asynchronous on `stream`. */
dsa_status dsa_read_probe(const void* buf, int64_t bytes, uint32_t* out, int32_t num_blocks,
                          void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H_ */
