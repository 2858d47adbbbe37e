// attn_bwd.h -- host/device interface of the backward-pass kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Backward pass of the dense prefill (bf16, d in {64, 128}).
struct BwdParams {
  const void* q;    // [B, A, S_q, d]
  const void* k;    // [B, A_kv, S_k, d]
  const void* v;
  const void* o;    // forward output, [B, A, S_q, d]
  const void* dout;  // incoming gradient of o
  const float* lse;  // forward LSE (natural log), [B, A, S_q]
  float* row_stats;  // workspace [B, A, S_q, 2]: (LSE * log2 e, or +inf for a row that
                     // takes no part; rowsum(dO * O)), written by the dQ pass
  void* dq;          // [B, A, S_q, d]
  void* dk;          // [B, A_kv, S_k, d]
  void* dv;
  const uint8_t* q_keep;  // [B, S_q] or null
  const uint8_t* k_keep;  // [B, S_k] or null
  int B, A, A_kv, G, S_q, S_k, d;
  int causal;
  float scale, scale_log2;
  // sliding window around query i's position i + S_k - S_q: key j is kept
  // when i + off - win_left <= j <= i + off + win_right; -1 leaves a side
  // unbounded.  The causal flag is folded into win_right (<= 0).
  int win_left, win_right;
  // XCD-blocked grid orders (0 = plain order), set by launch_bwd_bf16
  int dq_units_per_xcd, dq_group;  // units: (batch, query head)
  int kv_units_per_xcd, kv_group;  // units: (batch, KV head)
  // packed sequences (cu_seqlens != null): q, o, dout, dq are [A, T, d], k, v,
  // dk, dv [A_kv, T, d], lse [A, T], row_stats [A, T, 2]; sequence s holds
  // tokens [cu_seqlens[s], cu_seqlens[s+1]) and is its own problem (S_q = S_k
  // = its length); keep masks are [T].  B = 1.
  const int32_t* cu_seqlens;
  int n_seq, T;
  int max_tiles;    // most 128-row tiles of any sequence
  int total_tiles;  // 128-row tiles summed over the sequences
  // block mask (dense only): block_keep[b][hm][qb][kb] for 128 x 128 blocks,
  // hm = 0 when block_heads == 1, else the query head; n_qb, n_kb blocks
  const uint8_t* block_keep;
  int block_heads, n_qb, n_kb;
  // dense additive term (dense only): bias[((b * bias_heads + hm) * S_q + i) *
  // bias_ld + j] added to scale * q_i . k_j (as M / scale to the raw product)
  const float* bias;
  int bias_heads, bias_ld;
  float inv_scale;
  // per-row key ranges: row i keeps key j only when key_range[2 i] <= j <=
  // key_range[2 i + 1]; dense [B, S_q, 2], packed [T, 2] (positions within
  // the sequence); or null
  const int32_t* key_range;
  // ALiBi: slope per query head [A] (the forward's); uses inv_scale; or null
  const float* alibi_slopes;
};
// Block-mask limits of the backward: the dQ pass keeps one flag per 128-key
// block of its row block in LDS, the dK/dV pass one per (query head of the
// group, 128-row block).
constexpr int kBwdMaxKeyBlocks = 2048;
constexpr int kBwdMaxRowBlocks = 4096;
constexpr int kBwdQRows = 128;   // query rows per dQ workgroup
constexpr int kBwdKRows = 128;   // keys per dK/dV workgroup
hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream);

}  // namespace attn
