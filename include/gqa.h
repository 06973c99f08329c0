/*
 * gqa.h -- C ABI of libgqa: grouped-query attention (GQA) over a KV cache on
 * AMD Instinct MI355X (gfx950).
 *
 * Method.  Hq query heads share Hkv key/value heads in contiguous groups of
 * Gs = Hq / Hkv: query head h (0-indexed) reads KV head g = floor(h / Gs),
 * the 0-indexed form of g(h) = ceil(h / (H/G)) in "GQA reading notes"
 * (zhongzhuzhou.org), section "方法详解 > GQA 架构", where
 * head_h = softmax(q_h K_g^T * scale) V_g.  Hkv = Hq is multi-head attention
 * and Hkv = 1 multi-query attention ("从MHA到GQA", gzher.com, GQA section).
 * Hq must be a multiple of Hkv ("查询头保持不变，只减少键值头", ttlab lesson,
 * section on the three names on one axis).
 *
 * Conventions shared by every call:
 *   - All tensors are dense, row-major, contiguous device buffers; element
 *     type is given by gqa_dtype.  bf16 is the 16-bit brain float, stored as
 *     its bit pattern.  q, caches and out share one dtype.
 *   - Every data pointer must be 16-byte aligned (GQA_ERR_ALIGN otherwise).
 *   - The caller owns every buffer.  The library allocates no device memory,
 *     keeps no pointer after return and has no state beyond a per-device
 *     cache of the compute-unit count and, for gqa_decode_noalloc only, one
 *     static device array per GPU (see there).
 *   - Calls validate their arguments on the host first; a validation error
 *     returns before any device work, and nothing is written.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     default stream).  Nothing synchronises.  A launch failure returns
 *     GQA_ERR_HIP; device faults surface at the caller's next synchronisation.
 *   - Arithmetic is fp32 throughout (bf16 inputs are widened exactly; bf16
 *     products are formed exactly in fp32 by the matrix cores); bf16 outputs
 *     are rounded to nearest-even.  Results are deterministic run to run.
 *   - Calls are reentrant and thread-safe.  `out` must not alias an input.
 *   - Lengths live in device memory and are not checked on the host by
 *     default.  A kernel clamps a length to [0, Lmax] (and skips block-table
 *     entries outside the pool), so a value outside its documented range
 *     never sends a read or write past the caller's buffers; the results of
 *     that sequence are then unspecified.  With the environment variable
 *     GQA_CHECK_SEQLENS=1, the decode calls first copy seqlens (and the
 *     block-table entries of every row a sequence holds) to the host on
 *     `stream`, wait for them, and return GQA_ERR_SHAPE before any launch if
 *     one is out of range.  This debug check synchronises the stream; it is
 *     skipped while the stream is being captured into a graph.
 */
#ifndef GQA_H
#define GQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GQA_F32 = 0,
    GQA_BF16 = 1,
    GQA_FP8_E4M3 = 2, /* OCP 8-bit float E4M3 (bias 7, no infinities); KV caches of gqa_decode_ex only */
    GQA_FP8_E5M2 = 3  /* OCP 8-bit float E5M2 (bias 15, IEEE-style infinities and NaNs); KV caches of gqa_decode_ex only */
} gqa_dtype;

typedef enum {
    GQA_OK = 0,
    GQA_ERR_NULL = 1,        /* a required pointer is NULL */
    GQA_ERR_SHAPE = 2,       /* B, Hq, Hkv, Lmax or P out of range (see each call) */
    GQA_ERR_GROUP = 3,       /* Hq is not a multiple of Hkv */
    GQA_ERR_HEADDIM = 4,     /* d is not 64 or 128 */
    GQA_ERR_DTYPE = 5,       /* dtype not supported by this call */
    GQA_ERR_ALIGN = 6,       /* a data pointer is not 16-byte aligned */
    GQA_ERR_WORKSPACE = 7,   /* workspace missing or smaller than required */
    GQA_ERR_UNSUPPORTED = 8, /* group size Hq/Hkv above 64, or num_splits out of range */
    GQA_ERR_HIP = 9,         /* the HIP runtime reported an error */
    GQA_ERR_SCRATCH_LIMIT = 10 /* gqa_decode_noalloc: the split partials exceed its static scratch */
} gqa_status;

/* Human-readable name of a status code (static storage; never NULL). */
const char *gqa_status_str(gqa_status s);

/* ------------------------------------------------------------------------
 * Decode: one new query token per sequence against its cached K/V rows.
 *
 * Follows Algorithm 2 (GQA decode, step t) of "GQA reading notes", the
 * per-query-head part: for every sequence b and query head h,
 *   s_j = scale * <q[b,h,:], k_cache[b,j,g,:]>  for j < seqlens[b],
 *   out[b,h,:] = sum_j softmax(s)_j * v_cache[b,j,g,:],   g = h / (Hq/Hkv).
 * The new token's K/V must already be written at row seqlens[b]-1 (the
 * append of that algorithm happens before this call).  Each K/V row of a
 * group is read from memory once and serves all Hq/Hkv query heads of the
 * group (same page, walkthrough of Algorithm 2).
 *
 *   q        [B, Hq, d]
 *   k_cache  [B, Lmax, Hkv, d]   rows j >= seqlens[b] are never read
 *   v_cache  [B, Lmax, Hkv, d]
 *   seqlens  [B] int32, DEVICE memory; precondition 0 <= seqlens[b] <= Lmax
 *            (checked only under GQA_CHECK_SEQLENS=1, see the conventions
 *            above).  seqlens[b] == 0 gives out[b,:,:] = 0.
 *   out      [B, Hq, d]
 *   scale    softmax scale, normally 1/sqrt(d)
 *   dtype    GQA_F32 or GQA_BF16
 *   d        64 or 128;  1 <= Hq/Hkv <= 64;  B, Hq, Hkv, Lmax >= 1;
 *            (Lmax + 32) * Hkv * d * 4 must not exceed 2^31 - 1 (one
 *            sequence's cache slice is addressed with 32-bit byte offsets)
 *   num_splits  0 = choose automatically; otherwise the number of pieces
 *            the cached length is cut into (1 <= num_splits <= Lmax).  With
 *            more than one piece, partial results (running max, sum of
 *            weights, weighted sum) go to `workspace` and a second kernel
 *            merges them.
 *   workspace, workspace_bytes  caller-provided device scratch of at least
 *            gqa_decode_workspace_size() bytes; may be NULL when that size is 0.
 *
 * Returns GQA_OK or an error code; see the conventions above.
 * ------------------------------------------------------------------------ */
gqa_status gqa_decode(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *seqlens, int B, int Hq, int Hkv, int d, int Lmax,
                      float scale, gqa_dtype dtype, void *out, void *workspace,
                      size_t workspace_bytes, int num_splits, void *stream);

/* ------------------------------------------------------------------------
 * Decode that allocates nothing, for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.
 *
 * Same arguments, layouts, results and errors as gqa_decode, without the
 * workspace: when the plan cuts the cached length into several pieces, their
 * partial results go to a static device array of GQA_NOALLOC_SCRATCH_BYTES
 * that the library holds on every GPU it runs on until the process ends.
 * Plans that need more than that (B * Hq * pieces * (d + 2) * 4 bytes, see
 * gqa_decode_workspace_size) return GQA_ERR_SCRATCH_LIMIT before any device
 * work; pass num_splits to bound the pieces.  The call issues no allocation
 * and no memset.  The array's address is resolved once per device, on the
 * first call made with that device current.
 *
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (two streams, two host threads, a graph replay beside an eager
 * call) race on it and may return wrong results.  Serialise them, or use
 * gqa_decode with a workspace per stream.  Nothing in the array needs to be
 * cleared between calls: a call reads only partials it wrote itself.
 * ------------------------------------------------------------------------ */
#define GQA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
gqa_status gqa_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *seqlens, int B, int Hq, int Hkv, int d, int Lmax,
                              float scale, gqa_dtype dtype, void *out, int num_splits,
                              void *stream);

/* Number of pieces gqa_decode will cut the cached length into for these
 * arguments (num_splits = 0 asks for the automatic choice, which depends on
 * the current device's compute-unit count).  Writes it to *splits. */
gqa_status gqa_decode_num_splits(int B, int Hq, int Hkv, int d, int Lmax, gqa_dtype dtype,
                                 int num_splits, int *splits);

/* Workspace bytes gqa_decode needs for these arguments (0 when it needs
 * none).  Same argument meaning as gqa_decode.  Writes it to *bytes. */
gqa_status gqa_decode_workspace_size(int B, int Hq, int Hkv, int d, int Lmax, gqa_dtype dtype,
                                     int num_splits, size_t *bytes);

/* ------------------------------------------------------------------------
 * Prefill: the whole prompt attends to itself in parallel.
 *
 * With causal != 0, prompt position i of sequence b attends to positions
 * 0..i only (the causal mask of the prefill phase, "从MHA到GQA", section on
 * why the question becomes how KV is stored); with causal == 0 to all P.
 *   out[b,i,h,:] = sum_j softmax_j(scale * <q[b,i,h,:], k[b,j,g,:]>) v[b,j,g,:]
 *
 *   q    [B, P, Hq, d]
 *   k    [B, P, Hkv, d]
 *   v    [B, P, Hkv, d]
 *   out  [B, P, Hq, d]
 *   dtype  GQA_BF16 only (the matrix-core path); GQA_F32 -> GQA_ERR_DTYPE
 *   d      64 or 128;  1 <= Hq/Hkv <= 64;  B, P, Hq, Hkv >= 1;
 *          (P + 128) * Hkv * d * 2 must not exceed 2^31 - 1 (K/V chunk byte
 *          offsets are 32-bit), else GQA_ERR_SHAPE
 *
 * Returns GQA_OK or an error code; see the conventions above.
 * ------------------------------------------------------------------------ */
gqa_status gqa_prefill(const void *q, const void *k, const void *v, int B, int P, int Hq,
                       int Hkv, int d, int causal, float scale, gqa_dtype dtype, void *out,
                       void *stream);

/* ------------------------------------------------------------------------
 * Extended decode: several new tokens, append, FP8 cache, paged cache,
 * sliding window.
 *
 * The decode step of "GQA reading notes", Algorithm 2, with the cache update
 * (the new K/V rows are appended before attending) done by the same call,
 * and generalised in four ways the pages combine with GQA: several new query
 * tokens per sequence verified at once against one read of the cache, a
 * cache stored in FP8, a cache managed in fixed-size blocks addressed through
 * a block table, and attention restricted to the most recent keys ("GQA
 * reading notes", sections "关联工作：GQA 之后又发生了什么" and the engineering
 * notes of "复现性"; "从MHA到GQA", section on what each attention-efficiency
 * technique changes).
 *
 * For sequence b with n = seqlens[b] valid rows (the T new ones included),
 * new token t sits at position pos = n - T + t and, for every query head h
 * (KV head g = h / (Hq/Hkv)),
 *   out[b,t,h,:] = sum_j softmax_j(scale * <q[b,t,h,:], K[b,j,g,:]>) V[b,j,g,:]
 * over keys j in [lo, pos], lo = max(0, pos - window + 1) if window > 0,
 * else 0: causal among the new tokens, as in prefill.
 *
 * Fields of gqa_decode_ex_args (all pointers are DEVICE memory, 16-byte
 * aligned where they hold rows):
 *   q        [B, T, Hq, d] bf16 (dtype must be GQA_BF16)
 *   out      [B, T, Hq, d] bf16
 *   k_cache, v_cache   the cache, element type kv_dtype (GQA_BF16,
 *            GQA_FP8_E4M3 or GQA_FP8_E5M2): contiguous [B, Lmax, Hkv, d] when block_table is
 *            NULL; otherwise a pool [num_blocks, block_size, Hkv, d] and row j
 *            of sequence b is row j % block_size of block
 *            block_table[b * max_blocks + j / block_size].  Written when
 *            k_new is given; read otherwise.
 *   seqlens  [B] int32: valid rows per sequence AFTER the append.
 *            Precondition: T <= seqlens[b] <= Lmax (checked only under
 *            GQA_CHECK_SEQLENS=1, see the conventions above).
 *   block_table  [B, max_blocks] int32 or NULL.  block_size must be a multiple
 *            of 16; Lmax must equal max_blocks * block_size.  Precondition:
 *            every entry used is in [0, num_blocks) (entries outside are
 *            never followed: their rows read as zeros and take no append).
 *   k_scale, v_scale  [Hkv] fp32, the FP8 formats only (required there,
 *            ignored for bf16): K row values are fp8(byte) * k_scale[g], V
 *            likewise with v_scale[g], fp8() the value the format encodes.
 *   k_new, v_new  [B, T, Hkv, d] in kv_dtype, or both NULL.  When given they
 *            are stored, byte for byte, at rows seqlens[b] - T + t, in the
 *            same launch that attends: the attention reads those rows from
 *            k_new/v_new, never from the cache, so their cache contents
 *            before the call do not matter.  They must not overlap the cache.
 *   window   0 = every key; W > 0 = the last W keys of each token.
 *   T * (Hq/Hkv) <= 64; d 64 or 128; B, T, Hq, Hkv, Lmax >= 1;
 *            32 * Hkv * d * (bytes per cache element) <= 2^31 - 1 (the rows of
 *            one 32-key step are addressed with 32-bit offsets), else
 *            GQA_ERR_SHAPE.
 *   num_splits, workspace, workspace_bytes  as for gqa_decode; the size comes
 *            from gqa_decode_ex_workspace_size.
 *
 * Returns GQA_OK or an error code (conventions at the top of this file).
 * ------------------------------------------------------------------------ */
typedef struct {
    const void *q;
    void *k_cache;
    void *v_cache;
    const int32_t *seqlens;
    int B, T, Hq, Hkv, d, Lmax;
    float scale;
    gqa_dtype dtype;
    gqa_dtype kv_dtype;
    const float *k_scale;
    const float *v_scale;
    const int32_t *block_table;
    int block_size, max_blocks, num_blocks;
    int window;
    const void *k_new;
    const void *v_new;
    void *out;
    void *workspace;
    size_t workspace_bytes;
    int num_splits;
} gqa_decode_ex_args;

gqa_status gqa_decode_ex(const gqa_decode_ex_args *args, void *stream);

/* Workspace bytes gqa_decode_ex needs for these arguments (0 when none).
 * Only the shape, dtype, paging and num_splits fields are read. */
gqa_status gqa_decode_ex_workspace_size(const gqa_decode_ex_args *args, size_t *bytes);

/* Prefill with a sliding window: with causal != 0 and window W > 0, prompt
 * position i attends to positions max(0, i - W + 1) .. i only (attention
 * restricted to recent keys, "从MHA到GQA", section on what each
 * attention-efficiency technique changes); W = 0 is gqa_prefill.  Same
 * arguments and conventions as gqa_prefill otherwise; window > 0 without
 * causal returns GQA_ERR_UNSUPPORTED, window < 0 GQA_ERR_SHAPE. */
gqa_status gqa_prefill_ex(const void *q, const void *k, const void *v, int B, int P, int Hq,
                          int Hkv, int d, int causal, int window, float scale, gqa_dtype dtype,
                          void *out, void *stream);

/* ------------------------------------------------------------------------
 * Counts (host only, exact integers).
 *
 * KV-cache elements per layer and sequence = 2 * L * Hkv * d: the leading 2
 * is K and V ("查询头保持不变，只减少键值头", section "什么减少，什么不减少";
 * "GQA reading notes", section 3, equation S_KV).
 * ------------------------------------------------------------------------ */
uint64_t gqa_kv_cache_elems(uint64_t L, uint64_t Hkv, uint64_t d);

/* Algorithmic bytes of one gqa_decode call: every valid K and V row read
 * once per KV head, plus q read and out written once.  The K/V part is the
 * per-step cache traffic of "GQA reading notes", section 3 (KV cache) and
 * its formal definition: K and V of each cached position are read once per
 * group, not once per query head (the walkthrough of Algorithm 2 fuses the
 * group's queries for exactly that).  host_seqlens is a HOST array of B
 * lengths.  Returns 0 for an unknown dtype. */
uint64_t gqa_decode_bytes(const int32_t *host_seqlens, int B, int Hq, int Hkv, int d,
                          gqa_dtype dtype);

/* FLOP of one gqa_decode call: 2 per multiply-add, scores plus weighted sum:
 * 4 * Hq * d * sum(seqlens).  It holds no Hkv term (ttlab lesson, same
 * section: the attention multiplications have no group count). */
uint64_t gqa_decode_flops(const int32_t *host_seqlens, int B, int Hq, int d);

/* FLOP of one gqa_prefill call: 4 * B * Hq * d * pairs, where pairs =
 * P(P+1)/2 unmasked query-key pairs if causal, P*P otherwise.  Scores and
 * weighted sum each take Hq * d multiply-adds per query-key pair, with no
 * KV-head term (ttlab lesson, section "什么减少，什么不减少"); the causal mask
 * of the prefill phase ("从MHA到GQA", the prefill/decode discussion) leaves
 * position i its keys 0..i.  A multiply-add counts 2 FLOP. */
uint64_t gqa_prefill_flops(int B, int P, int Hq, int d, int causal);

/* Algorithmic bytes of one gqa_prefill call: q, k, v read once, out written
 * once.  K and V hold 2 * P * Hkv * d elements per sequence, the cache size
 * formula of the ttlab lesson (section "什么减少，什么不减少") and of "GQA
 * reading notes", section 3; q and out hold B * P * Hq * d each. */
uint64_t gqa_prefill_bytes(int B, int P, int Hq, int Hkv, int d, gqa_dtype dtype);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H */
