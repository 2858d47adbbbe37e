// attn_kernels.h -- host-side launch interface between the C ABI layer and
// the kernel translation units.  Arguments are validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// Parameters of one prefill launch (dense batch or packed varlen).
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const uint8_t* q_keep;
  const uint8_t* k_keep;
  const int32_t* cu_seqlens;  // device; varlen only
  int B, A, A_kv, G;          // G = A / A_kv
  int S_q, S_k;               // dense only
  int n_seq, T;               // varlen only
  int n_qt;                   // dense: query tiles per head; varlen: max tiles of any sequence
  int total_tiles;            // varlen: sum over sequences of query tiles (per head)
  int d;
  int causal;
  float scale;                // softmax scale (> 0)
  float scale_log2;           // scale * log2(e)
  int xcd_heads;              // dense: (batch, head) pairs per XCD block; varlen/paged: heads per XCD block; 0 = plain order
  int xcd_group;              // dense: heads whose query tiles are issued together
  // sliding window around query i's position i + off (off = S_k - S_q): key
  // j is kept when i + off - win_left <= j <= i + off + win_right; -1 leaves
  // a side unbounded.  The causal flag is folded into win_right (<= 0).
  int win_left, win_right;
  // paged KV (prefill over a paged cache): k, v are the caches [num_pages,
  // page_size, A_kv, d]; sequence s's token t lives in page
  // block_table[s * max_pages + t / page_size]; seq_lens[s] = its KV length
  const int32_t* block_table;
  const int32_t* seq_lens;
  int page_shift;  // log2(page_size)
  int max_pages;
  // block sparsity (dense prefill): block_keep[b][hm][qb][kb] (hm = 0 when
  // block_heads == 1, else the head) says whether the 128 x 128 block of query
  // rows qb*128.. and keys kb*128.. is computed at all; n_kb = ceil(S_k / 128)
  const uint8_t* block_keep;
  int block_heads, n_kb;
  // dense additive mask (dense prefill): bias[((b * bias_heads + hm) * S_q +
  // i) * bias_ld + j] is added to scale * q_i . k_j (hm = 0 when bias_heads
  // == 1, else the head); inv_scale = 1 / scale
  const float* bias;
  int bias_heads, bias_ld;
  float inv_scale;
  // FP8 queries and keys (dense prefill, d = 128): q, k hold OCP E4M3 codes,
  // one fp32 scale per 128 consecutive tokens of each (batch, head):
  // q_scale [B, A, ceil(S_q / 128)], k_scale [B, A_kv, ceil(S_k / 128)]
  const float* q_scale;
  const float* k_scale;
  // E4M3 paged cache (paged prefill): k_scale, v_scale [num_pages, A_kv]
  const float* v_scale;
  // per-row key ranges: row i keeps key j only when key_range[2 i] <= j <=
  // key_range[2 i + 1]; dense [B, S_q, 2], packed [T, 2] (positions within
  // the sequence), paged [T_q, 2] (positions in the sequence's cache); or null
  const int32_t* key_range;
  // ALiBi: slope per query head [A]; the term -slope_h |p_i - j| joins the
  // score (p_i: row i's bottom-right aligned position); or null.  Uses inv_scale.
  const float* alibi_slopes;
};

// Dense prefill grid order.  Workgroups are dealt to the 8 XCDs round-robin
// by index, and each XCD has its own L2.  When B*A is a multiple of 8, XCD x
// is given the contiguous (batch, head) block [x*H, (x+1)*H), H = B*A/8
// (query heads that share a KV head stay together), and it takes its heads
// in groups of `group` (up to 8), each group's query tiles heaviest first, so
// the tiles of a head stream the same K/V at about the same time and the
// XCD's L2 serves most re-reads.  Groups of 8 keep enough heavy tiles at the
// head of each XCD's queue that the grid still ends evenly (groups of 4 fetch
// less but leave a tail of long tiles).  Otherwise: query tiles heaviest
// first across all heads.
constexpr int kXcds = 8;
inline void plan_dense_order(FwdParams& p) {
  const int bh = p.B * p.A;
  p.xcd_heads = 0;
  p.xcd_group = 0;
  if (bh % kXcds != 0) return;
  const int h = bh / kXcds;
  int g = 8;
  while (g > 1 && h % g != 0) g >>= 1;
  p.xcd_heads = h;
  p.xcd_group = g;
}

// Packed (varlen or paged) prefill grid order: heads dealt to the XCDs in
// contiguous blocks of A/8 when those blocks hold whole GQA groups, so the
// query heads of one KV head share an XCD's L2 (GQA only: measured 2% slower
// without heads to share); otherwise plain order.
inline void plan_varlen_order(FwdParams& p) {
  p.xcd_heads = 0;
  p.xcd_group = 0;
  if (p.G > 1 && p.A % kXcds == 0 && (p.A / kXcds) % p.G == 0) p.xcd_heads = p.A / kXcds;
}

// bf16 prefill (d in {64, 128}).  Returns hipSuccess or the launch error.
hipError_t launch_prefill_bf16(const FwdParams& p, bool varlen, hipStream_t stream);
// bf16 prefill of packed query chunks over a paged KV cache (d in {64, 128};
// page_size a power of two and a multiple of 2048 / d).
hipError_t launch_prefill_paged_bf16(const FwdParams& p, hipStream_t stream);
// prefill with FP8 (E4M3) queries and keys and bf16 values (d = 128, S_k <=
// kFp8MaxKeys): the QK^T products on the FP8 matrix cores
constexpr int kFp8MaxKeys = 262144;
hipError_t launch_prefill_fp8(const FwdParams& p, hipStream_t stream);
// bf16 prefill of packed query chunks over an E4M3 paged cache with
// per-(page, KV head) scales (same page-size rules as the bf16 cache)
hipError_t launch_prefill_paged_fp8(const FwdParams& p, hipStream_t stream);
// fp32 prefill (1 <= d <= 128).
hipError_t launch_prefill_f32(const FwdParams& p, bool varlen, hipStream_t stream);
// block_keep[b][h][qb][kb] = whether some bias entry of the 128 x 128 block is
// greater than -inf (n_kb <= 65535)
hipError_t launch_block_keep_from_bias(const float* bias, int B, int heads, int S_q, int S_k, int ld,
                                       uint8_t* block_keep, hipStream_t stream);
// query rows per workgroup of the bf16 prefill kernel
constexpr int kPrefillRows = 128;
constexpr int kPrefillRowsF32 = 16;

// Paged decode, split along the KV length (Stream-K over 16-token chunks).
struct DecodeParams {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* o;
  float* lse;
  float* part_o;    // workspace [n_slots, A, d] fp32: partial outputs, normalised within the partial
  float* part_lse;  // workspace [n_slots, A] fp32: base-2 LSE of each partial
  const float* k_scale;  // fp8 caches: [num_pages, A_kv] dequantisation scales (else null)
  const float* v_scale;
  int B, A, A_kv, G, d;
  int page_size, max_pages;
  // sliding window: the query (position len - 1) sees keys t >= len - 1 -
  // win_left; -1 = every key.  A sequence's chunk list covers the 16-token
  // chunks from the one holding its first visible key.
  int win_left;
  long long n_chunks;  // sum over sequences of decode_chunks(len, win_left)
  int n_wg;            // workgroups along the chunk list (set at launch)
  float scale, scale_log2;
  // ALiBi: slope per query head [A]; key t of a sequence of len tokens gets
  // -slope_h (len - 1 - t) (divided by the scale, on the raw product); or null
  const float* alibi_slopes;
  float inv_scale;
};

// upper bound on workgroups along the chunk list; sizes the workspace
constexpr int kMaxDecodeGroups = 2048;

struct DecodePlan {
  long long n_chunks;
  int n_slots;  // partial slots: workgroup + sequence < kMaxDecodeGroups + B
};
// first visible key of a sequence of len tokens, and its chunks in the list
__host__ __device__ inline int decode_first_key(int len, int win_left) {
  return (win_left < 0 || len - 1 - win_left <= 0) ? 0 : len - 1 - win_left;
}
__host__ __device__ inline int decode_chunks(int len, int win_left) {
  return len <= 0 ? 0 : (len + 15) / 16 - decode_first_key(len, win_left) / 16;
}
DecodePlan plan_decode(int B, const int32_t* seq_lens_host, int win_left = -1);
size_t decode_workspace_bytes(int A, int d, const DecodePlan& plan);
size_t decode_workspace_lse_offset(int A, int d, const DecodePlan& plan);

hipError_t launch_decode_bf16(const DecodeParams& p, hipStream_t stream);
// Size of the static split workspace of attn_decode_paged_noalloc (one copy per
// device), and its device address on the current device (looked up once per
// device; no allocation).
constexpr size_t kDecodeStaticScratchBytes = size_t(48) << 20;
hipError_t decode_static_scratch(void** ptr);
// Same, over FP8 (OCP E4M3) caches with per-(page, KV head) scales.
hipError_t launch_decode_fp8(const DecodeParams& p, hipStream_t stream);

}  // namespace attn
