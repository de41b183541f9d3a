/*
 * pa.h -- C ABI of the paged KV-cache attention library for MI355X (gfx950).
 *
 * What it computes (pages cited by title and section):
 *
 *  - "PagedAttention in mistral.rs", opening section: the KV cache is cut into
 *    fixed-size blocks of tokens (default 32) taken from a pool allocated up
 *    front; each sequence reaches its blocks through a table.  Attention over
 *    such a cache for one new query token per sequence is pa_decode().
 *  - same page, section "KV Cache Quantization": the cache may hold FP8
 *    (E4M3) instead of the activation type; the slot writer quantises on
 *    write and the attention kernels dequantise on read.
 *  - "Optimization plans" (mistral.rs discussion 46), "Update" post: the slot
 *    writer reshape_and_cache stores each new token's K and V into its cache
 *    slot before attention runs; pa_reshape_and_cache() is that writer.
 *  - "Rolling buffer cache" (llama.cpp discussion 3581), opening post: with a
 *    sliding window of W tokens the cache is a ring of W rows and position i
 *    lives in row i mod W; pa_decode() with window > 0 reads such a ring,
 *    and pa_prefill_chunk_window() (pa_prefill_chunk_window_quant() for E4M3
 *    and INT8 rings) attends a prompt chunk over it.
 *  - same page, the prefix-caching note and section "FlashAttention V2/V3 +
 *    PagedAttention": prompt (prefill) tokens attend causally over cached
 *    blocks that may be shared between sequences; pa_prefill_chunk() is that
 *    causal attention over a block table.
 *  - "libmir-metal 0.2.0, src/native/trace/kv.rs", fn build: the pages are
 *    head-major (one page per block and KV head, the layout below keeps
 *    that; the order of elements inside a page is this library's own
 *    choice, made for the matrix-core operands); a quantised cache keeps
 *    packed INT8 pages with one FP32 scale per token and head and
 *    dequantises inside paged attention for prefill and decode: the *_i8
 *    entry points.
 *
 * Conventions for every entry point:
 *
 *  - Pointers named *_cache, key, value, query, out, slot_mapping,
 *    block_tables, context_lens, cu_q_lens and workspace are DEVICE pointers
 *    owned by the caller.  The library allocates nothing and keeps no state
 *    between calls.
 *  - Cache pools are head-major: one (block, KV head) page is a contiguous
 *    run of block_size * head_dim elements, pages ordered [num_blocks]
 *    [num_kv_heads].  Inside a page (t = row 0..block_size-1, d = 0..D-1),
 *    not row-major [BS][D] but tiled, as this library lays it out:
 *      key page   [D/8][block_size][8]  element (t, d) at ((d/8)*BS + t)*8 + d%8
 *      value page [BS/8][D][8]          element (t, d) at ((t/8)*D + d)*8 + t%8
 *    (so the key pool is [NB][Hkv][D/8][BS][8] and the value pool
 *    [NB][Hkv][BS/8][D][8]).  Both layouts make the attention kernels'
 *    matrix-core operands single 16-byte loads (8 dims of one key; 8 keys
 *    of one dim); the value page groups its keys by 8 so that one new row
 *    lands in D 16-byte runs rather than D scattered elements.
 *    Activations are row-major.
 *  - Identity map ("libmir-metal 0.2.0, src/native/trace/kv.rs", fn build:
 *    identity block maps are served as one contiguous K/V view).  Every
 *    attention entry point accepts block_tables == NULL: logical block j of
 *    sequence b is then physical block b*MBPS + j (the pool is a dense
 *    [B][MBPS] cache, NB >= B*MBPS by caller contract), and no table is
 *    read.  B*MBPS must fit in int32, else PA_ERR_INVALID.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL is the default
 *    stream).  The library never synchronises.
 *  - Errors are returned as pa_status; nothing is thrown and nothing aborts.
 *    Arguments the host can see are checked before anything is launched.
 *    Sizes that would exceed a launch grid dimension (B or Hkv above 65535
 *    for decode, Hkv above 65535 for the writer and the block copy) give
 *    PA_ERR_UNSUPPORTED.
 *    Device data (table entries, lengths, slots) is NOT checked: the caller
 *    contracts below must hold, or the kernels read or write out of bounds.
 *  - Supported now: block_size 32; head_dim 64, 96 or 128; act dtype PA_F16
 *    or PA_BF16; cache dtype equal to the act dtype or PA_F8E4M3; Hq/Hkv in
 *    {1, 2, 4, 8, 16} for decode and 1..16 for prefill.  Anything else
 *    returns PA_ERR_UNSUPPORTED.  PA_I8 is accepted only by the *_i8 entry
 *    points (which take the scale pools).
 *  - INT8 caches: int8 pools in the layout above plus two fp32 scale pools
 *    key_scales, value_scales [NB][Hkv][BS] (one scale per cached row and
 *    KV head), device memory owned by the caller.  A row x of D values is
 *    stored as scale = fp32(max|x|) / 127 (IEEE division) and codes
 *    clamp(round-half-even(fp32(x) / scale), -127, 127) (IEEE division; a
 *    zero row has scale 0 and zero codes); it stands for code * scale.
 *    Inputs must be finite.
 */
#ifndef PAGED_KV_PA_H
#define PAGED_KV_PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F16 = 0, PA_BF16 = 1, PA_F8E4M3 = 2, PA_I8 = 3 } pa_dtype;

/* Counters at the start of every decode workspace, at least (see pa_decode). */
#define PA_DECODE_MIN_COUNTERS 16384

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID = 1,     /* a host-visible argument is malformed             */
  PA_ERR_UNSUPPORTED = 2, /* well-formed but not built (shape, dtype)          */
  PA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required        */
  PA_ERR_HIP = 4          /* a HIP runtime call or launch failed               */
} pa_status;

/* Human-readable name of a status code.  Never NULL. */
const char* pa_status_string(pa_status s);

/* Message of the last failed call on this host thread ("" if none). */
const char* pa_last_error(void);

/*
 * pa_reshape_and_cache -- write T new tokens into the cache pools.
 *
 * key, value      [T][Hkv][D] in act_dtype.
 * key_cache,
 * value_cache     pools in cache_dtype (layout above), updated in place.
 * slot_mapping    [T] int32.  Token n goes to block slot_mapping[n] / BS,
 *                 row slot_mapping[n] % BS, for every KV head.  A negative
 *                 slot skips the token.  Caller contract: non-negative slots
 *                 are < NB*BS and unique within one call.
 * cache_dtype     act_dtype (bit copy) or PA_F8E4M3: code =
 *                 E4M3(fp32(x) / scale) with IEEE fp32 division, round to
 *                 nearest even, saturation to +-448, NaN -> 0x7F|sign,
 *                 scale = k_scale for keys and v_scale for values (must be
 *                 finite and > 0).
 * D must be a multiple of 8 and at most 512.
 * Every byte of the pools outside the written rows is left unchanged.
 * T == 0 is a no-op returning PA_OK.
 */
pa_status pa_reshape_and_cache(const void* key, const void* value, void* key_cache,
                               void* value_cache, const int32_t* slot_mapping, int32_t T,
                               int32_t Hkv, int32_t D, int32_t BS, int32_t NB,
                               pa_dtype act_dtype, pa_dtype cache_dtype, float k_scale,
                               float v_scale, void* stream);

/*
 * pa_reshape_and_cache_i8 -- pa_reshape_and_cache into an INT8 cache.
 *
 * key_cache, value_cache  int8 pools (layout above), updated in place.
 * key_scales, value_scales fp32 [NB][Hkv][BS], updated: the scale of every
 *                 written (row, KV head).
 * Everything else as pa_reshape_and_cache (act_dtype PA_F16 or PA_BF16).
 * Every byte of the pools and every scale outside the written rows is left
 * unchanged.
 */
pa_status pa_reshape_and_cache_i8(const void* key, const void* value, int8_t* key_cache,
                                  int8_t* value_cache, float* key_scales, float* value_scales,
                                  const int32_t* slot_mapping, int32_t T, int32_t Hkv,
                                  int32_t D, int32_t BS, int32_t NB, pa_dtype act_dtype,
                                  void* stream);

/*
 * pa_copy_blocks -- copy whole cache blocks, for copy-on-write of blocks
 * shared between sequences (prefix caching: "PagedAttention in mistral.rs",
 * prefix caching notes; "libmir-metal 0.2.0, src/native/trace/kv.rs", fn
 * build, copy-on-write page maps).
 *
 * block_mapping   [N][2] int32 device pairs (src, dst): block dst receives
 *                 block src's K pages and V pages of every KV head and, for
 *                 PA_I8, its key/value row scales.
 * key_scales,
 * value_scales    the [NB][Hkv][BS] fp32 scale pools of a PA_I8 cache
 *                 (ignored, may be NULL, otherwise).
 * cache_dtype     the pools' element type (PA_F16, PA_BF16, PA_F8E4M3, PA_I8).
 * Caller contract: entries lie in [0, NB); destinations are distinct and no
 * destination is also a source in the same call (copy-on-write copies into
 * fresh blocks).  N == 0 is a no-op; N <= 65535.
 */
pa_status pa_copy_blocks(void* key_cache, void* value_cache, float* key_scales,
                         float* value_scales, const int32_t* block_mapping, int32_t N,
                         int32_t Hkv, int32_t D, int32_t BS, int32_t NB, pa_dtype cache_dtype,
                         void* stream);

/*
 * pa_decode_workspace_bytes -- bytes of scratch pa_decode needs for this
 * shape.  Same arguments as pa_decode (partition_tokens 0 = automatic).
 * The automatic plan also depends on the cache format, which this query
 * does not take: it returns the larger of the workspaces the plans for
 * 16-bit and byte-format caches need.  Returns 0 when the call needs no
 * workspace, and (size_t)-1 when the arguments are invalid.
 */
size_t pa_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                 int32_t max_context_len, int32_t window,
                                 int32_t partition_tokens);

/*
 * pa_decode_workspace_bytes_for -- the same for one cache format: exactly
 * what pa_decode (and its _append / _i8 forms) needs with that cache_dtype.
 */
size_t pa_decode_workspace_bytes_for(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                     int32_t max_context_len, int32_t window,
                                     int32_t partition_tokens, pa_dtype cache_dtype);

/*
 * pa_decode -- one query token per sequence attends over its cached tokens.
 *
 * out             [B][Hq][D] act_dtype, written.
 * query           [B][Hq][D] act_dtype.
 * block_tables    [B][MBPS] int32: logical block j of sequence b lives in
 *                 physical block block_tables[b*MBPS + j]; NULL for the
 *                 identity map (b*MBPS + j).
 * context_lens    [B] int32: tokens of sequence b, the decoded token included
 *                 (write it with pa_reshape_and_cache first).
 * window == 0     full cache: rows 0..L-1 with L = context_lens[b].
 * window  > 0     rolling buffer of `window` rows (window % BS == 0,
 *                 window <= MBPS*BS); rows 0..min(L, window)-1 are read, in
 *                 any order (softmax does not depend on key order).
 * max_context_len host-side upper bound of context_lens (sizes the split).
 * softmax_scale   multiplies q.k before the softmax.
 * k_scale,v_scale dequantisation scales of an E4M3 cache (ignored otherwise).
 * partition_tokens split size hint, a multiple of BS: > 0 splits every
 *                 sequence into ceil(max_len / partition_tokens) parts whose
 *                 partial results are merged (max_len = max_context_len,
 *                 capped at window); 0 lets the library choose: one pass
 *                 without workspace below 1024 tokens (max_len); from 1024
 *                 on, enough splits for ~2048 resident waves, at most one
 *                 split per page of each of the workgroup's waves and at
 *                 most 16 splits (more if a split would exceed 64 pages
 *                 per wave); with one split per sequence and B <= 64, pair
 *                 mode: the workgroup of each shorter sequence of a pair
 *                 (the batch ranked by length, longest with shortest) also
 *                 reads the tail of the longer one, and the two partials
 *                 are merged like splits; E4M3 and INT8 caches (B <= 1024)
 *                 where pair mode does not apply: equal ranges of the
 *                 whole batch's pages, one per workgroup, whatever the mix
 *                 of context lengths (a sequence cut between ranges is
 *                 merged like the splits).  Results do not depend on the
 *                 plan beyond rounding (the summation order, which also
 *                 varies from launch to launch).
 * workspace       device scratch of pa_decode_workspace_bytes(...) bytes
 *                 (may be NULL when that is 0), 256-byte aligned, kept by
 *                 the caller across calls.  It starts with the counter
 *                 region: one int32 arrival counter per (sequence, KV head),
 *                 max(B*Hkv, PA_DECODE_MIN_COUNTERS) of them, at byte 0;
 *                 the split partials follow it.  The counter region must be
 *                 zero when a call that needs a workspace starts; the call
 *                 leaves it zero.  So a workspace zero-filled once stays
 *                 valid for every call with B*Hkv <= PA_DECODE_MIN_COUNTERS,
 *                 whatever the other arguments; a call with a larger B*Hkv
 *                 than the last call that used the workspace needs its first
 *                 4*B*Hkv bytes zeroed first (that earlier call's partials
 *                 may lie there).  Calls that share a workspace must not
 *                 overlap in time.  The last split (or range) of each
 *                 (sequence, KV head) to finish merges the partials inside
 *                 the same launch.
 * Output is out[b][h] = sum_t softmax_t(scale * q[b][h] . k_t) v_t with KV
 * head h / (Hq/Hkv); an empty context gives zeros.  Caller contract: table
 * entries read (logical blocks < ceil(L/BS)) lie in [0, NB);
 * context_lens[b] <= max_context_len and (window == 0) <= MBPS*BS.  A
 * length above max_context_len is clamped to it on the device (a wrong
 * result for that sequence, never a read past the pages the plan covers).
 */
pa_status pa_decode(void* out, const void* query, const void* key_cache,
                    const void* value_cache, const int32_t* block_tables,
                    const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                    int32_t D, int32_t BS, int32_t MBPS, int32_t max_context_len,
                    float softmax_scale, pa_dtype act_dtype, pa_dtype cache_dtype,
                    float k_scale, float v_scale, int32_t window,
                    int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the split scratch is a fixed array in the library's
 * own device memory, PA_DECODE_SCRATCH_BYTES on each GPU the library runs on
 * (held until the process ends), instead of a caller's workspace.
 *
 * Arguments, outputs and errors as pa_decode, without workspace and
 * workspace_bytes.  Allocates nothing.  The first call on a device looks up
 * that device's array and zeroes its counter region with a small kernel on
 * `stream`; every call leaves the counters zero.
 * PA_ERR_WORKSPACE (nothing launched) when the call's plan needs more than
 * PA_DECODE_SCRATCH_BYTES, or splits with B*Hkv above
 * PA_DECODE_MIN_COUNTERS; pa_decode with a workspace serves those.
 * Every call on one GPU shares that GPU's array and leaves its partials
 * there: calls that overlap in time on one GPU (two streams without
 * ordering, two host threads) race and give wrong results.
 */
#define PA_DECODE_SCRATCH_BYTES (64u << 20)

pa_status pa_decode_noalloc(void* out, const void* query, const void* key_cache,
                            const void* value_cache, const int32_t* block_tables,
                            const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                            int32_t D, int32_t BS, int32_t MBPS, int32_t max_context_len,
                            float softmax_scale, pa_dtype act_dtype, pa_dtype cache_dtype,
                            float k_scale, float v_scale, int32_t window,
                            int32_t partition_tokens, void* stream);

/*
 * pa_decode_append -- pa_reshape_and_cache of the decoded token followed by
 * pa_decode, in one launch.
 *
 * key, value      [B][Hkv][D] act_dtype: K and V of each sequence's decoded
 *                 token.  Its cache row is context_lens[b] - 1 (window == 0)
 *                 or (context_lens[b] - 1) % window (rolling buffer), in the
 *                 block that block_tables names for that row; it is stored
 *                 exactly as pa_reshape_and_cache stores it (E4M3 with
 *                 k_scale / v_scale for an FP8 cache) and is part of the
 *                 attention of this call.
 * All other arguments, outputs and errors are those of pa_decode.  Caller
 * contract: context_lens[b] >= 1 (a sequence with 0 gets zeros and no write).
 */
pa_status pa_decode_append(void* out, const void* query, const void* key, const void* value,
                           void* key_cache, void* value_cache, const int32_t* block_tables,
                           const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                           int32_t D, int32_t BS, int32_t MBPS, int32_t max_context_len,
                           float softmax_scale, pa_dtype act_dtype, pa_dtype cache_dtype,
                           float k_scale, float v_scale, int32_t window,
                           int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * pa_decode_i8 -- pa_decode over an INT8 cache: key k_t = code * key scale
 * of row t, value v_t likewise, dequantised inside the kernel.
 *
 * key_scales, value_scales fp32 [NB][Hkv][BS], 16-byte aligned (written by
 *                 pa_reshape_and_cache_i8).
 * Same workspace (pa_decode_workspace_bytes), arguments, outputs and errors
 * as pa_decode with cache dtype PA_I8 (no k_scale / v_scale).
 */
pa_status pa_decode_i8(void* out, const void* query, const int8_t* key_cache,
                       const int8_t* value_cache, const float* key_scales,
                       const float* value_scales, const int32_t* block_tables,
                       const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                       int32_t D, int32_t BS, int32_t MBPS, int32_t max_context_len,
                       float softmax_scale, pa_dtype act_dtype, int32_t window,
                       int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * pa_decode_append_i8 -- pa_decode_append over an INT8 cache: the decoded
 * token's row is quantised as pa_reshape_and_cache_i8 quantises it (codes
 * plus one fp32 scale per row for K and for V, written to key_scales /
 * value_scales) and is part of the attention of this call.
 * key, value      [B][Hkv][D] act_dtype, 2-byte aligned.
 * Other arguments, outputs and errors as pa_decode_i8; caller contract as
 * pa_decode_append.
 */
pa_status pa_decode_append_i8(void* out, const void* query, const void* key, const void* value,
                              int8_t* key_cache, int8_t* value_cache, float* key_scales,
                              float* value_scales, const int32_t* block_tables,
                              const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                              int32_t D, int32_t BS, int32_t MBPS, int32_t max_context_len,
                              float softmax_scale, pa_dtype act_dtype, int32_t window,
                              int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * pa_prefill_chunk -- causal attention of a chunk of new tokens per sequence
 * over everything cached for it (shared prefix blocks included).
 *
 * out, query      [total_q][Hq][D] act_dtype, sequences packed back to back.
 * cu_q_lens       [B+1] int32 prefix sums of the chunk lengths C_b.
 * context_lens    [B] int32: cached tokens of sequence b, chunk included (the
 *                 chunk must already be written with pa_reshape_and_cache).
 * Query j of sequence b sits at absolute position context_lens[b] - C_b + j
 * and attends to positions 0 .. that position.
 * max_chunk_len   host-side upper bound of C_b (sizes the grid).
 * softmax_scale   finite and > 0 (each lane's running maximum is taken
 *                 over raw scores and then scaled, and masked raw scores
 *                 are -inf before scaling); else PA_ERR_INVALID.
 *                 The same holds for every prefill entry point below.
 * Caller contract: C_b <= context_lens[b] <= MBPS*BS; table entries for
 * logical blocks < ceil(context_lens[b]/BS) lie in [0, NB).  A length above
 * MBPS*BS is clamped to it on the device.
 */
pa_status pa_prefill_chunk(void* out, const void* query, const int32_t* cu_q_lens,
                           const void* key_cache, const void* value_cache,
                           const int32_t* block_tables, const int32_t* context_lens,
                           int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t BS,
                           int32_t MBPS, int32_t max_chunk_len, float softmax_scale,
                           pa_dtype act_dtype, pa_dtype cache_dtype, float k_scale,
                           float v_scale, void* stream);

/*
 * pa_prefill_chunk_i8 -- pa_prefill_chunk over an INT8 cache (scales as in
 * pa_decode_i8, 4-byte aligned).  Same arguments, outputs and errors as
 * pa_prefill_chunk with cache dtype PA_I8.
 */
pa_status pa_prefill_chunk_i8(void* out, const void* query, const int32_t* cu_q_lens,
                              const int8_t* key_cache, const int8_t* value_cache,
                              const float* key_scales, const float* value_scales,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t BS,
                              int32_t MBPS, int32_t max_chunk_len, float softmax_scale,
                              pa_dtype act_dtype, void* stream);

/*
 * pa_prefill_chunk_window -- chunked prefill of a sliding-window layer whose
 * cache is a rolling buffer ("Rolling buffer cache", llama.cpp discussion
 * 3581, opening post): a ring of `window` rows, position i in ring row
 * i mod window, reached through block_tables[b][0 .. window/BS - 1].
 *
 * key, value      [total_q][Hkv][D] act_dtype, the chunk's own K and V,
 *                 packed like the queries, 16-byte aligned.
 * key_cache, value_cache  the ring pools in act_dtype (16-bit caches only).
 * context_lens    [B] int32: positions of sequence b, chunk included.  The
 *                 ring holds the positions before the chunk,
 *                 max(0, ctx - C_b - window) .. ctx - C_b - 1, and not yet
 *                 the chunk itself: write it after this call (only its last
 *                 min(C_b, window) tokens land; earlier ones would be
 *                 overwritten within the chunk).
 * Query j of sequence b sits at position i = context_lens[b] - C_b + j and
 * attends to positions max(0, i - window + 1) .. i: those before the chunk
 * from the ring, the chunk's own from key / value.
 * Other arguments as pa_prefill_chunk (cache dtype = act_dtype).
 * Errors: PA_ERR_INVALID for window <= 0, not a multiple of 32, or needing
 * more than MBPS table entries; otherwise as pa_prefill_chunk.
 * Caller contract: C_b <= context_lens[b]; ring table entries that hold
 * positions of that range lie in [0, NB).
 */
pa_status pa_prefill_chunk_window(void* out, const void* query, const void* key,
                                  const void* value, const int32_t* cu_q_lens,
                                  const void* key_cache, const void* value_cache,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t BS,
                                  int32_t MBPS, int32_t max_chunk_len, float softmax_scale,
                                  pa_dtype act_dtype, int32_t window, void* stream);

/*
 * pa_prefill_chunk_window_quant -- pa_prefill_chunk_window over a quantised
 * ring ("PagedAttention in mistral.rs", section "KV Cache Quantization", for
 * E4M3; "libmir-metal 0.2.0, src/native/trace/kv.rs", fn build, for the
 * per-token/head INT8 cache).
 *
 * cache_dtype     PA_F8E4M3: the ring holds E4M3 codes standing for
 *                 code * k_scale (K) and code * v_scale (V); key_scales and
 *                 value_scales are ignored (may be NULL).
 *                 PA_I8: the ring holds INT8 codes and key_scales /
 *                 value_scales [NB][Hkv][BS] fp32 (4-byte aligned) their
 *                 rows' scales; k_scale and v_scale are ignored.
 *                 act_dtype: the same as pa_prefill_chunk_window.
 * The ring rows are read at those values; the chunk's own rows (key, value)
 * are the activations as given (they are quantised only when written into
 * the ring after this call).  Over an E4M3 ring the kernel folds k_scale
 * and v_scale into the score and output scales and reads the chunk's rows
 * as key / k_scale and value / v_scale rounded to act_dtype and clamped to
 * +-448 (the E4M3 range): the same values up to that rounding whenever the
 * scales cover the chunk (|key| <= 448 * k_scale, |value| <= 448 *
 * v_scale), as they must for the ring the chunk is written into.  Over an
 * INT8 ring each ring row is read as its codes times its row scale rounded
 * to act_dtype (one rounding beyond the exact code * scale).  Other
 * arguments, outputs and errors as
 * pa_prefill_chunk_window; PA_ERR_UNSUPPORTED for another cache_dtype;
 * PA_ERR_INVALID for E4M3 scales that are not finite and > 0, or NULL INT8
 * scale pools.
 */
pa_status pa_prefill_chunk_window_quant(void* out, const void* query, const void* key,
                                        const void* value, const int32_t* cu_q_lens,
                                        const void* key_cache, const void* value_cache,
                                        const float* key_scales, const float* value_scales,
                                        const int32_t* block_tables, const int32_t* context_lens,
                                        int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                        int32_t BS, int32_t MBPS, int32_t max_chunk_len,
                                        float softmax_scale, pa_dtype act_dtype,
                                        pa_dtype cache_dtype, float k_scale, float v_scale,
                                        int32_t window, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_PA_H */
