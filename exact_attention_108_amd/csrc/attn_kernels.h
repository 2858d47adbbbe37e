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
};

// bf16 prefill (d in {64, 128}).  Returns hipSuccess or the launch error.
hipError_t launch_prefill_bf16(const FwdParams& p, bool varlen, hipStream_t stream);
// fp32 prefill (1 <= d <= 128).
hipError_t launch_prefill_f32(const FwdParams& p, bool varlen, hipStream_t stream);
// query rows per workgroup of the bf16 prefill kernel
constexpr int kPrefillRows = 128;
constexpr int kPrefillRowsF32 = 16;

// Paged decode, split along the KV length.
struct DecodeParams {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* o;
  float* lse;
  float* part_o;    // workspace [B, A, n_split, d] fp32 (normalised partial outputs)
  float* part_lse;  // workspace [B, A, n_split] fp32 (natural-log LSE of each split)
  int B, A, A_kv, G, d;
  int page_size, max_pages;
  int split_tokens;  // tokens per split (multiple of the page size)
  int n_split;       // splits per sequence = ceil(max seq_len / split_tokens)
  float scale, scale_log2;
};

// Split plan shared by the workspace query and the launch.
struct DecodePlan {
  int split_tokens;
  int n_split;
};
DecodePlan plan_decode(int B, int A_kv, int page_size, const int32_t* seq_lens_host);
size_t decode_workspace_bytes(int B, int A, int d, const DecodePlan& plan);

// total_units = sum_b ceil(seq_lens[b] / split_tokens)
hipError_t launch_decode_bf16(const DecodeParams& p, int total_units, hipStream_t stream);

}  // namespace attn
