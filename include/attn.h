/*
 * attn.h -- C ABI of the MI355X (gfx950) fused exact-attention library
 *           (libattn_mi355x.so).
 *
 * Operation (page "Attention Kernel", section "问题与成本"):
 *
 *     P = softmax(Q K^T * scale + M),   O = P V,   LSE_i = ln sum_j exp(s_ij)
 *
 * computed without writing the S_q x S_k score matrix anywhere: K/V tiles
 * stream through on-chip memory against a resident Q tile and the running
 * (max, normaliser, unnormalised output) state of every query row is
 * rescaled as each tile arrives (page "Attention 算子加速史", sections 1.1-1.3
 * and 2.1-2.2; page "Attention Kernel", section "Online softmax").
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library neither allocates nor frees memory and keeps no global state
 *     (the one exception: the static workspace of attn_decode_paged_noalloc).
 *     Pointers named *_host are HOST pointers read synchronously during the
 *     call.  Everything is contiguous row-major.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream) and never synchronise.  Inputs are read-only; o/lse are fully
 *     overwritten (including masked rows) and must not alias the inputs.
 *   - dtype ATTN_BF16: q/k/v/o hold bfloat16 (uint16 bits); products are
 *     accumulated in fp32; o is rounded once to bf16 (round-to-nearest-even).
 *     ATTN_F32: q/k/v/o are fp32.  lse is always fp32, natural log.
 *   - GQA: query head h reads KV head h / (A / A_kv) (contiguous groups; page
 *     "Attention Kernel", section "问题与成本", GQA paragraph).
 *   - Lengths: a sequence (S_q, S_k, a packed sequence, a chunk or a cached
 *     length) of more than 2^31 - 1025 positions is ATTN_ERR_UNSUPPORTED
 *     (the kernels count positions in int32, up to a tile past a length).
 *   - Mask: M_ij is the optional dense additive term bias[i][j] and the
 *     optional ALiBi term (see attn_mask) plus -inf when: causal and j > i + (S_k - S_q)
 *     (bottom-right alignment), q_keep[i] == 0, k_keep[j] == 0, a window,
 *     a key range or a block mask excludes (i, j).  A row with every key masked (including
 *     S_k == 0) returns O = 0 and LSE = -inf (page "Attention Kernel",
 *     section "Online softmax", fully-masked-row contract), never NaN.
 *   - scale must be finite and > 0.  Inputs must be finite.
 *   - Alignment: bf16 q/k/v/o (and the caches) must be 16-byte aligned (the
 *     kernels copy and store 16-byte groups of a row), fp32 q/k/v/o and
 *     every lse, int32 table and fp32 scale array 4-byte aligned; uint8 keep
 *     masks need none.  A misaligned pointer is ATTN_ERR_INVAL.
 *   - Errors are reported before any launch: ATTN_ERR_INVAL for bad
 *     arguments (NULL required pointer, negative size, A % A_kv != 0,
 *     scale not finite and positive, inconsistent lengths, workspace too
 *     small, misaligned pointer), ATTN_ERR_UNSUPPORTED for a valid request outside the built
 *     kernels (see each entry point), ATTN_ERR_LAUNCH when the runtime
 *     rejects a launch.  Device-side contract violations (a block-table
 *     entry outside [0, num_pages), cu_seqlens that differ from
 *     cu_seqlens_host) are the caller's responsibility.
 */
#ifndef ATTN_MI355X_H
#define ATTN_MI355X_H

#include <stddef.h>
#include <stdint.h>

/* The value attn_abi_version() returns for this header. */
#define ATTN_ABI_VERSION 8

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVAL = 1,
    ATTN_ERR_UNSUPPORTED = 2,
    ATTN_ERR_LAUNCH = 3
} attn_status;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;

/* Optional keep-masks (uint8, 1 = keep, 0 = mask to -inf); any may be NULL.
 * Layout: attn_fwd q_keep [B, S_q], k_keep [B, S_k]; attn_fwd_varlen [T].
 *
 * block_keep (bf16): block sparsity (page "Attention Kernel",
 * section "可编程 mask": the block level decides which tiles are skipped
 * whole).  uint8 [B, block_heads, ceil(S_q / 128), ceil(S_k / 128)];
 * block_keep[b][h'][i][j] = 0 masks every (row, key) pair with row in
 * [128 i, 128 i + 128) and key in [128 j, 128 j + 128) (h' = 0 when
 * block_heads == 1, else the query head); those key tiles are never loaded.
 * block_heads is 1 or A (ignored when block_keep is NULL).  Requires
 * S_k <= 262144.  attn_fwd, attn_fwd_varlen, attn_prefill_paged_masked,
 * attn_bwd and attn_bwd_varlen take it; the other paged entry points have
 * no mask argument.  attn_fwd_varlen and attn_bwd_varlen: uint8 [n_seq,
 * block_heads, nb, nb] with nb = ceil(longest sequence / 128); entry
 * [s][h'][i][j] is block (i, j) of sequence s's own rows and keys (positions
 * within the sequence); entries past a shorter sequence's blocks are never
 * read.
 *
 * bias: the general dense additive mask M of the operation
 * (page "Attention Kernel", section "可编程 mask"; the term "+ M" of section
 * "问题与成本").  fp32 [B, bias_heads, S_q, bias_ld], row (b, h', i) holding
 * M_ij for keys j < S_k (h' = 0 when bias_heads == 1, else the query head).
 * Rows are read in 16-byte groups, so entries S_k .. bias_ld - 1 of a row
 * may be read; their values are ignored.  Each entry j < S_k is finite or
 * -inf (-inf masks the pair; +inf and NaN are contract violations).  The
 * term is added to scale * q_i . k_j, so it is not multiplied by scale.
 * Range: with c = min(scale, ln 2), finite entries are supported down to
 * -FLT_MAX * c / 4 and up to +FLT_MAX * c / 4; an entry below -FLT_MAX * c
 * is a masking fill value and counts as -inf (the float32 minimum, the
 * usual fill value of additive masks, is always one: a row filled with it
 * returns O = 0 and LSE = -inf); entries between the two bounds are outside
 * the contract.  (The kernels scale scores to base 2 in fp32, where a term
 * below -FLT_MAX * c has no finite representation.)
 * Requires bias_heads in {1, A}, bias_ld >= S_k and a multiple of 4, and
 * bias 16-byte aligned; bf16 calls also need 128 * bias_ld * 4 < 2^32
 * (ATTN_ERR_UNSUPPORTED otherwise).  It combines with every other mask; key
 * tiles are skipped only through block_keep, which attn_block_keep_from_bias
 * derives from a bias.  attn_fwd, attn_fwd_varlen (bf16),
 * attn_prefill_paged_masked, attn_bwd and attn_bwd_varlen take it; in bf16
 * calls it does not combine with key_range (ATTN_ERR_UNSUPPORTED: fold the
 * ranges into the term).
 * attn_fwd_varlen and attn_bwd_varlen: fp32 [bias_heads, T, bias_ld], row
 * (h', t) holding M for token t (position i in its sequence) against the
 * keys at positions j < len of the same sequence (bias_ld >= the longest
 * sequence).
 *
 * key_range: per-row key ranges (page "Attention Kernel", section
 * "可编程 mask": document boundaries and prefix-LM are element rules; the
 * block level skips the key tiles no row of a tile keeps).  int32 pairs
 * (first, last): query row i keeps key j only when first_i <= j <= last_i
 * (both ends included; first_i > last_i keeps no key, and any int32 value is
 * accepted).  Shared by every head; combined with every other mask.
 * Packed documents: each row's range is its own document (with causal = 1
 * the diagonal cuts it); prefix-LM: (0, max(i, prefix - 1)) with causal = 0.
 * Layouts: attn_fwd, attn_fwd_fp8 and attn_bwd [B, S_q, 2] over keys
 * 0 .. S_k - 1; attn_fwd_varlen and attn_bwd_varlen [T, 2], the pair of
 * token t counting key positions within its sequence;
 * attn_prefill_paged_masked [T_q, 2], the pair of chunk token t counting
 * key positions of its sequence's cache (0 .. seq_lens[s] - 1).  Must be
 * 8-byte aligned (ATTN_ERR_INVAL otherwise).  The forward loads only the key
 * tiles between the smallest first and the largest last of a 128-row tile
 * and applies no per-element test to tiles inside every row's range; the
 * dK/dV pass of the gradient visits only the query rows whose ranges reach
 * its keys.
 *
 * alibi_slopes: ALiBi (page "Attention Kernel", section "正确性契约" names it
 * among the transforms fused into the score).  fp32 [A], one slope per query
 * head; the term -alibi_slopes[h] * |p_i - j| joins M (it is added to
 * scale * q_i . k_j, like bias), with p_i query i's bottom-right aligned
 * position (i + S_k - S_q; packed calls: within the sequence; paged chunks:
 * seq_lens[s] - q_len + i over cache positions j).  Computed in the kernels
 * (no term is read); bf16 calls form the distance in fp32, exact below 2^24
 * and rounded to fp32 (relative 2^-24) beyond.  attn_fwd, attn_fwd_varlen, attn_prefill_paged_masked,
 * attn_bwd and attn_bwd_varlen take it; in bf16 calls it combines with the
 * causal flag, windows and keep-masks but not with block masks, bias or
 * key_range (ATTN_ERR_UNSUPPORTED), nor with attn_fwd_fp8.  4-byte aligned. */
typedef struct {
    const uint8_t *q_keep;
    const uint8_t *k_keep;
    const uint8_t *block_keep;
    int block_heads;
    const float *bias;
    int bias_heads;
    int bias_ld;
    const int32_t *key_range;
    const float *alibi_slopes;
} attn_mask;

/* Optional sliding window (page "Attention Kernel", section "可编程 mask":
 * a window is an element rule, and key tiles outside every row's window are
 * skipped whole).  Query i sits at position p_i = i + (S_k - S_q) (within its
 * sequence for varlen); key j is kept when p_i - left <= j <= p_i + right.
 * -1 leaves a side unbounded; other negative values are ATTN_ERR_INVAL.  With
 * causal = 1 the right edge is min(right, 0) (right = -1 gives the causal
 * diagonal).  NULL = no window.  Any edge value is accepted: an edge wider
 * than the key range is the same as -1.  A call with a window returns
 * ATTN_ERR_UNSUPPORTED when its row plus key extent exceeds INT_MAX - 1024. */
typedef struct {
    int left;
    int right;
} attn_window;

/*
 * Batched prefill attention (page "Attention Kernel", section "问题与成本";
 * causal tile skipping and the saved log-sum-exp: section "FlashAttention 的
 * 稳定基础"; outer loop over query tiles, inner over key/value tiles with a
 * single deferred division: page "Attention 算子加速史", sections 2.1-2.2).
 *
 *   q, o : [B, A, S_q, d_h]        k, v : [B, A_kv, S_k, d_h]
 *   lse  : [B, A, S_q] fp32        mask : NULL or keep-masks as above
 *   window : NULL or a sliding window as above
 *
 * Supported: bf16 with d_h in {64, 128}; fp32 with 1 <= d_h <= 128.
 * B, A, A_kv >= 1; S_q, S_k >= 0.
 */
attn_status attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                     int B, int A, int A_kv, int S_q, int S_k, int d_h, float scale,
                     int causal, const attn_mask *mask, const attn_window *window,
                     attn_dtype dtype, void *stream);

/*
 * attn_fwd with FP8 queries and keys (page "Attention 算子加速史", section
 * 3.3: FP8 attention with block-wise adaptive scaling; the QK^T products run
 * on gfx950's FP8 matrix instructions).  q and k hold one OCP E4M3 byte per
 * element (4 exponent bits, bias 7, 3 mantissa bits, largest finite 448, no
 * infinities; 0x7F / 0xFF are NaN and must not occur), with one fp32 scale per
 * 128 consecutive tokens of each (batch, head); element value = byte value *
 * scale of its block:
 *
 *   q      : uint8 [B, A, S_q, 128]      q_scale : fp32 [B, A, ceil(S_q / 128)]
 *   k      : uint8 [B, A_kv, S_k, 128]   k_scale : fp32 [B, A_kv, ceil(S_k / 128)]
 *   v, o   : bf16 [B, A_kv, S_k, 128] / [B, A, S_q, 128];   lse : fp32 [B, A, S_q]
 *
 * Scores are formed exactly from the FP8 products (fp32 accumulation), then
 * multiplied by scale * q_scale * k_scale; the probabilities are rounded to
 * bf16 for the bf16 P V product, as in attn_fwd.  Scales must be finite and
 * > 0.  causal, keep-masks, key ranges and window as attn_fwd; block masks
 * and additive terms are ATTN_ERR_UNSUPPORTED.  Supported: d_h = 128, S_k <= 262144.
 */
attn_status attn_fwd_fp8(const uint8_t *q, const uint8_t *k, const void *v, void *o, float *lse,
                         const float *q_scale, const float *k_scale, int B, int A, int A_kv, int S_q, int S_k,
                         int d_h, float scale, int causal, const attn_mask *mask, const attn_window *window,
                         void *stream);

/*
 * Block mask of a dense additive mask (page "Attention Kernel", section
 * "可编程 mask": the block level of a mask decides which tiles are skipped
 * whole).  Writes block_keep [B, bias_heads, ceil(S_q / 128), ceil(S_k / 128)]
 * uint8 (device, caller-owned): 1 when some entry bias[b][h'][i][j] with i in
 * [128 qb, 128 qb + 128) ∩ [0, S_q) and j in [128 kb, 128 kb + 128) ∩ [0, S_k)
 * is greater than -inf, else 0.  Passed to attn_fwd with the same bias (and
 * block_heads = bias_heads) it changes no result and skips the key tiles the
 * bias masks whole.  bias: as in attn_mask.  Asynchronous on stream.
 */
attn_status attn_block_keep_from_bias(const float *bias, int B, int bias_heads, int S_q, int S_k, int bias_ld,
                                      uint8_t *block_keep, void *stream);

/*
 * Packed variable-length prefill (page "Attention Kernel", section
 * "Paged 与 ragged KV", ragged batches described by cumulative lengths).
 * Sequence s occupies tokens [cu_seqlens[s], cu_seqlens[s+1]); a query only
 * sees keys of its own sequence, and causal compares positions within it.
 *
 *   q, o : [A, T, d_h]      k, v : [A_kv, T, d_h]      lse : [A, T]
 *   cu_seqlens      : device int32 [n_seq + 1], cu[0] = 0, non-decreasing,
 *                     cu[n_seq] = T (= total_tokens); empty sequences allowed
 *   cu_seqlens_host : host copy of the same values (used for launch planning)
 *   mask            : NULL or q_keep [T], k_keep [T]; bf16 also a block mask
 *                     [n_seq, block_heads, nb, nb] and an additive term
 *                     [bias_heads, T, bias_ld] per sequence (see attn_mask)
 *   window          : NULL or a sliding window (positions within a sequence)
 *
 * Supported: as attn_fwd (block masks and terms: bf16 only).
 */
attn_status attn_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                            const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                            int n_seq, int total_tokens, int A, int A_kv, int d_h, float scale,
                            int causal, const attn_mask *mask, const attn_window *window,
                            attn_dtype dtype, void *stream);

/*
 * Single-query decode over a paged KV cache, split along the KV length and
 * merged by log-sum-exp (page "Attention Kernel", section "Paged 与 ragged
 * KV": token t of a sequence lives in physical page block_table[t / page_size]
 * at offset t % page_size; page "Attention 算子加速史", section 4.2: each
 * split emits a partial output plus its LSE and a reduction merges them with
 * the two-state rule of page "Attention Kernel", section "Online softmax").
 *
 *   q, o        : [B, A, d_h]            lse : [B, A] fp32
 *   k_cache,
 *   v_cache     : [num_pages, page_size, A_kv, d_h]
 *   block_table : device int32 [B, max_pages]; entries past
 *                 ceil(seq_lens[b] / page_size) are never read
 *   seq_lens    : device int32 [B]; seq_lens_host: host copy (split planning)
 *   workspace   : device buffer of at least
 *                 attn_decode_paged_workspace_bytes(...) bytes, 256-byte
 *                 aligned; its contents on entry are ignored
 *
 * The split boundaries depend on seq_lens and on the device's compute-unit
 * count (one resident wave of workgroups covers all tokens), never on page
 * ids: on one device the result does not depend on which physical pages the
 * block table names (bit for bit), while devices or partition modes with a
 * different CU count may round differently, within the stated tolerance.
 * Supported: bf16, d_h in {64, 128}, page_size a multiple of 16, A / A_kv <= 64
 * (MQA included).
 */
attn_status attn_decode_paged(const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *block_table, const int32_t *seq_lens,
                              const int32_t *seq_lens_host, int page_size, void *o, float *lse,
                              int B, int A, int A_kv, int d_h, int max_pages, int num_pages,
                              float scale, attn_dtype dtype, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * attn_decode_paged with a sliding window (page "Attention Kernel", section
 * "可编程 mask": a sliding window bounds how far back a query looks).  The
 * query of sequence b sits at position seq_lens[b] - 1 and sees the keys t
 * with t >= seq_lens[b] - 1 - window_left: its own and the window_left before
 * it.  window_left = -1 is attn_decode_paged (every key; bit for bit).  Only
 * the 16-token chunks from the one holding the first visible key are read
 * and split, so the work per sequence is min(len, window_left + 1) tokens
 * rounded out to chunks.  Arguments, workspace (attn_decode_paged_workspace_
 * bytes suffices), support and errors as attn_decode_paged; window_left <
 * -1 is ATTN_ERR_INVAL.
 */
attn_status attn_decode_paged_window(const void *q, const void *k_cache, const void *v_cache,
                                     const int32_t *block_table, const int32_t *seq_lens,
                                     const int32_t *seq_lens_host, int page_size, void *o,
                                     float *lse, int B, int A, int A_kv, int d_h, int max_pages,
                                     int num_pages, float scale, int window_left,
                                     attn_dtype dtype, void *workspace, size_t workspace_bytes,
                                     void *stream);

/*
 * attn_decode_paged over an FP8 KV cache (page "Attention Kernel", sections
 * "Paged 与 ragged KV" and "正确性契约": the cache dtype and its scale
 * metadata are part of the contract; page "Attention 算子加速史", section
 * 3.3: FP8 attention with block-wise scales).  The caches hold one OCP FP8 E4M3
 * byte per element (4 exponent bits, bias 7, 3 mantissa bits, largest finite
 * value 448, no infinities; 0x7F / 0xFF are NaN and must not occur), with
 * the layout [num_pages, page_size, A_kv, d_h]; element value =
 * byte value * scale[page, kv head]:
 *
 *   k_scale, v_scale : device fp32 [num_pages, A_kv], finite
 *
 * q, o, lse, block table, lengths and workspace are as in attn_decode_paged
 * (q, o bf16; same workspace size, from attn_decode_paged_workspace_bytes).
 * Supported: d_h in {64, 128}, page_size a multiple of 16, A / A_kv <= 64.
 */
attn_status attn_decode_paged_fp8(const void *q, const uint8_t *k_cache, const uint8_t *v_cache,
                                  const float *k_scale, const float *v_scale,
                                  const int32_t *block_table, const int32_t *seq_lens,
                                  const int32_t *seq_lens_host, int page_size, void *o, float *lse,
                                  int B, int A, int A_kv, int d_h, int max_pages, int num_pages,
                                  float scale, void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_decode_paged_fp8 with a sliding window (page "Attention Kernel",
 * section "可编程 mask"), defined as for attn_decode_paged_window: the query
 * of sequence b sees the keys t >= seq_lens[b] - 1 - window_left, and only
 * the 16-token chunks from the one holding the first visible key are read.
 * window_left = -1 is attn_decode_paged_fp8 (every key; bit for bit).
 * Arguments, workspace, support and errors as attn_decode_paged_fp8;
 * window_left < -1 is ATTN_ERR_INVAL.
 */
attn_status attn_decode_paged_fp8_window(const void *q, const uint8_t *k_cache, const uint8_t *v_cache,
                                         const float *k_scale, const float *v_scale,
                                         const int32_t *block_table, const int32_t *seq_lens,
                                         const int32_t *seq_lens_host, int page_size, void *o, float *lse,
                                         int B, int A, int A_kv, int d_h, int max_pages, int num_pages,
                                         float scale, int window_left, void *workspace,
                                         size_t workspace_bytes, void *stream);

/*
 * attn_decode_paged_window with ALiBi (page "Attention Kernel", section
 * "正确性契约" names ALiBi among the transforms fused into the score): key t
 * of sequence b, len = seq_lens[b] tokens, gets the term
 * -alibi_slopes[h] * (len - 1 - t) added to scale * q . k_t, the decode row's
 * part of attn_fwd's ALiBi (the query sits at position len - 1).  The
 * distance is formed in fp32: exact below 2^24, rounded to fp32 beyond.
 * alibi_slopes: device fp32 [A], 4-byte aligned, non-NULL (ATTN_ERR_INVAL
 * otherwise).  window_left as attn_decode_paged_window.  Arguments,
 * workspace, support and errors as attn_decode_paged_window.
 */
attn_status attn_decode_paged_alibi(const void *q, const void *k_cache, const void *v_cache,
                                    const int32_t *block_table, const int32_t *seq_lens,
                                    const int32_t *seq_lens_host, int page_size, void *o, float *lse,
                                    int B, int A, int A_kv, int d_h, int max_pages, int num_pages,
                                    float scale, int window_left, const float *alibi_slopes,
                                    attn_dtype dtype, void *workspace, size_t workspace_bytes,
                                    void *stream);

/*
 * attn_decode_paged_fp8_window with ALiBi, defined as for
 * attn_decode_paged_alibi (the term joins the score after the key scale).
 * Arguments, workspace, support and errors as attn_decode_paged_fp8_window;
 * alibi_slopes as attn_decode_paged_alibi.
 */
attn_status attn_decode_paged_fp8_alibi(const void *q, const uint8_t *k_cache, const uint8_t *v_cache,
                                        const float *k_scale, const float *v_scale,
                                        const int32_t *block_table, const int32_t *seq_lens,
                                        const int32_t *seq_lens_host, int page_size, void *o, float *lse,
                                        int B, int A, int A_kv, int d_h, int max_pages, int num_pages,
                                        float scale, int window_left, const float *alibi_slopes,
                                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_decode_paged without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * forbid allocation, harnesses without an allocator).  Same arguments,
 * semantics, kernels and result as attn_decode_paged (bit for bit), but the
 * split partials live in a static device array of the library, one copy per
 * device, 48 MiB (ATTN_DECODE_NOALLOC_MAX_BYTES), held from the first call on a
 * device until the process ends.  The call allocates nothing.
 *   - Returns ATTN_ERR_UNSUPPORTED when the workspace the call would need
 *     (attn_decode_paged_workspace_bytes of the same arguments) exceeds that
 *     size: e.g. A = 32, d_h = 128 allows up to B = 1000 sequences.
 *   - Every call on one device shares that device's array: calls that overlap
 *     in time on one device (several streams or host threads) race and must
 *     be serialised by the caller.  Calls on different devices do not share.
 *   - The array keeps the last call's partials; nothing in it needs to start
 *     at zero (every partial a call reads, that call wrote first).
 */
#define ATTN_DECODE_NOALLOC_MAX_BYTES ((size_t)48 << 20)
attn_status attn_decode_paged_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                      const int32_t *block_table, const int32_t *seq_lens,
                                      const int32_t *seq_lens_host, int page_size, void *o, float *lse,
                                      int B, int A, int A_kv, int d_h, int max_pages, int num_pages,
                                      float scale, attn_dtype dtype, void *stream);

/* Workspace bytes attn_decode_paged needs for these lengths (0 on bad input). */
size_t attn_decode_paged_workspace_bytes(int B, int A, int A_kv, int d_h, int page_size,
                                         const int32_t *seq_lens_host);

/*
 * Prefill of new query chunks over a paged KV cache, as one batched call
 * (page "Attention 算子加速史", section 4.2: paged KV addressed through the
 * block table inside the kernel, and one scheduling abstraction for a batch
 * that mixes prefill chunks with decode rows; page "Attention Kernel",
 * section "Paged 与 ragged KV").
 *
 *   q, o        : [A, T_q, d_h] packed chunks; lse : [A, T_q] fp32
 *   cu_seqlens_q: device int32 [n_seq + 1], chunk s = rows [cu[s], cu[s+1]);
 *                 cu_seqlens_q_host: host copy (launch planning)
 *   k_cache,
 *   v_cache     : [num_pages, page_size, A_kv, d_h], already holding every
 *                 sequence's tokens including its chunk
 *   block_table : device int32 [n_seq, max_pages]; token t of sequence s is in
 *                 page block_table[s][t / page_size] at offset t % page_size;
 *                 entries past ceil(seq_lens[s] / page_size) are never read
 *   seq_lens    : device int32 [n_seq] (KV length of each sequence, chunk
 *                 included); seq_lens_host: host copy (validation)
 *
 * Chunk s holds the last q_s = cu[s+1] - cu[s] tokens of its sequence: row i
 * of the chunk sits at position seq_lens[s] - q_s + i (the bottom-right
 * alignment of attn_fwd).  causal and window apply to these positions.  A
 * decode step is a chunk of length 1, so prefill chunks and decode rows can
 * share one call.  Requires q_s <= seq_lens[s] <= max_pages * page_size.
 * Supported: bf16, d_h in {64, 128}, page_size a power of two and a multiple
 * of 16 (d_h = 128) or 32 (d_h = 64).
 */
attn_status attn_prefill_paged(const void *q, const void *k_cache, const void *v_cache,
                               const int32_t *block_table, const int32_t *seq_lens,
                               const int32_t *seq_lens_host, const int32_t *cu_seqlens_q,
                               const int32_t *cu_seqlens_q_host, int page_size, void *o, float *lse,
                               int n_seq, int total_q, int A, int A_kv, int d_h, int max_pages,
                               int num_pages, float scale, int causal, const attn_window *window,
                               attn_dtype dtype, void *stream);

/*
 * attn_prefill_paged with a block mask and a dense additive term (page
 * "Attention Kernel", section "可编程 mask": block-level skipping, then an
 * element rule, over the paged chunks of section "Paged 与 ragged KV").  Each
 * sequence's chunk rows (index i within the chunk, at position
 * seq_lens[s] - q_len + i) face its keys at positions j < seq_lens[s]:
 *
 *   mask->block_keep : NULL or uint8 [n_seq, block_heads, nqb, nkb] with nqb =
 *                      ceil(longest chunk / 128), nkb = ceil(longest
 *                      seq_lens / 128); entry [s][h'][i][j] = 0 masks chunk
 *                      rows [128 i, 128 i + 128) against keys [128 j, 128 j +
 *                      128) of sequence s; those key tiles are never loaded
 *   mask->bias       : NULL or fp32 [bias_heads, total_q, bias_ld]; row (h', t)
 *                      holds the term of chunk token t against the keys at
 *                      positions j < seq_lens of its sequence (bias_ld >= the
 *                      longest seq_lens, a multiple of 4); values and range as
 *                      in attn_mask
 *   mask->q_keep, k_keep : must be NULL (ATTN_ERR_UNSUPPORTED otherwise)
 *
 * Everything else as attn_prefill_paged (bf16 caches only).  A NULL mask is
 * attn_prefill_paged.
 */
attn_status attn_prefill_paged_masked(const void *q, const void *k_cache, const void *v_cache,
                                      const int32_t *block_table, const int32_t *seq_lens,
                                      const int32_t *seq_lens_host, const int32_t *cu_seqlens_q,
                                      const int32_t *cu_seqlens_q_host, int page_size, void *o,
                                      float *lse, int n_seq, int total_q, int A, int A_kv, int d_h,
                                      int max_pages, int num_pages, float scale, int causal,
                                      const attn_mask *mask, const attn_window *window,
                                      attn_dtype dtype, void *stream);

/*
 * attn_prefill_paged over FP8 caches (page "Attention Kernel", sections "Paged
 * 与 ragged KV" and "正确性契约": the cache dtype and its scale metadata are
 * part of the contract; page "Attention 算子加速史", section 3.3).  The caches
 * hold one OCP E4M3 byte per element with the layout [num_pages, page_size,
 * A_kv, d_h] and the scales of attn_decode_paged_fp8 (element value = byte
 * value * scale[page, kv head]):
 *
 *   k_scale, v_scale : device fp32 [num_pages, A_kv], finite
 *
 * Every other argument, the result's definition and the support are those of
 * attn_prefill_paged (q, o bf16); the caches must be 8-byte aligned.  The
 * bytes are widened exactly to bf16; key scales multiply scores, value scales
 * the probabilities before the PV product.
 */
attn_status attn_prefill_paged_fp8(const void *q, const uint8_t *k_cache, const uint8_t *v_cache,
                                   const float *k_scale, const float *v_scale, const int32_t *block_table,
                                   const int32_t *seq_lens, const int32_t *seq_lens_host,
                                   const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_q_host, int page_size,
                                   void *o, float *lse, int n_seq, int total_q, int A, int A_kv, int d_h,
                                   int max_pages, int num_pages, float scale, int causal,
                                   const attn_window *window, void *stream);

/*
 * Backward of attn_fwd (dense batch): dQ, dK, dV of O = softmax(Q K^T *
 * scale + M) V for an incoming dO, with the probabilities recomputed tile by
 * tile from Q, K and the forward's LSE instead of being stored (page
 * "Attention 算子加速史", FAQ Q1; page "Attention Kernel", section
 * "Backward 与重计算": same scale, same mask, same GQA mapping as the
 * forward).  Per row i and key j, with D_i = sum_e dO_ie O_ie:
 *   dV_j = sum_i P_ij dO_i,    dS_ij = P_ij (dO_i . v_j - D_i),
 *   dQ_i = scale sum_j dS_ij k_j,    dK_j = scale sum_i dS_ij q_i,
 * and for GQA dK, dV of a KV head sum over the query heads that read it.
 *
 *   q, o, dout, dq : [B, A, S_q, d_h]     k, v, dk, dv : [B, A_kv, S_k, d_h]
 *   lse       : [B, A, S_q] fp32, as attn_fwd wrote it for the same q, k, v,
 *               scale, causal and mask; rows with lse = -inf take no part
 *   o         : attn_fwd's output for the same call
 *   mask      : NULL or the attn_fwd mask of the same call: keep-masks
 *               [B, S_q] / [B, S_k], a block mask (block_keep, block_heads)
 *               and a dense additive term (bias, bias_heads, bias_ld), with
 *               the layouts and rules of attn_mask; a block mask requires
 *               ceil(S_k / 128) <= 2048 and (A / A_kv) * ceil(S_q / 128) <=
 *               4096 (ATTN_ERR_UNSUPPORTED otherwise)
 *   window    : NULL or the sliding window given to attn_fwd
 *   workspace : device buffer of at least attn_bwd_workspace_bytes(B, A, S_q)
 *               bytes, 256-byte aligned (two fp32 per query row: the base-2
 *               LSE and D_i); contents on entry are ignored
 *
 * dq, dk, dv are fully overwritten (zero where no element contributes) and
 * must not alias the inputs or each other.  Every output element is written
 * by one thread with a fixed summation order: the result is deterministic.
 * All tensor pointers must be 16-byte aligned (ATTN_ERR_INVAL otherwise).
 * Supported: bf16 with d_h in {64, 128}.  B, A, A_kv >= 1; S_q, S_k >= 0.
 */
attn_status attn_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
                     const float *lse, void *dq, void *dk, void *dv, int B, int A, int A_kv, int S_q,
                     int S_k, int d_h, float scale, int causal, const attn_mask *mask,
                     const attn_window *window, attn_dtype dtype, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * Backward of attn_fwd_varlen (page "Attention Kernel", section "Backward 与
 * 重计算": packed-sequence boundaries are part of the backward's contract):
 * dQ, dK, dV of each packed sequence, every sequence its own problem as in
 * the forward (a query sees keys of its own sequence only; causal and the
 * window compare positions within it).
 *
 *   q, o, dout, dq : [A, T, d_h]      k, v, dk, dv : [A_kv, T, d_h]
 *   lse            : [A, T] fp32, attn_fwd_varlen's for the same call
 *   cu_seqlens, cu_seqlens_host, n_seq, total_tokens : as attn_fwd_varlen
 *   mask           : NULL or the forward's: keep-masks q_keep [T], k_keep
 *                    [T], a block mask [n_seq, block_heads, nb, nb] and an
 *                    additive term [bias_heads, T, bias_ld] as attn_fwd_varlen
 *                    takes them (see attn_mask)
 *   window         : NULL or the sliding window given to attn_fwd_varlen
 *   workspace      : device buffer of at least attn_bwd_workspace_bytes(1,
 *                    A, total_tokens) bytes, 256-byte aligned
 *
 * Outputs, determinism, alignment and support as attn_bwd (block masks: nb <=
 * 2048 and (A / A_kv) * nb <= 4096, else ATTN_ERR_UNSUPPORTED).
 */
attn_status attn_bwd_varlen(const void *q, const void *k, const void *v, const void *o, const void *dout,
                            const float *lse, void *dq, void *dk, void *dv, const int32_t *cu_seqlens,
                            const int32_t *cu_seqlens_host, int n_seq, int total_tokens, int A, int A_kv,
                            int d_h, float scale, int causal, const attn_mask *mask, const attn_window *window,
                            attn_dtype dtype, void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes attn_bwd needs (0 on bad input); attn_bwd_varlen needs
 * attn_bwd_workspace_bytes(1, A, total_tokens). */
size_t attn_bwd_workspace_bytes(int B, int A, int S_q);

/* Static text for a status code. */
const char *attn_status_string(attn_status s);

/* ABI version of this header (incremented on incompatible change). */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_H */
