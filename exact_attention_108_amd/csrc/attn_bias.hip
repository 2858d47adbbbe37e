// attn_bias.hip -- block mask of a dense additive mask (gfx950).
//
// The general dense mask M of page "Attention Kernel", section "可编程 mask",
// has a block level that decides which key tiles are skipped whole: a
// 128 x 128 block of (query row, key) pairs whose entries are all -inf
// contributes nothing and need not be loaded.  This kernel derives that block
// level from an fp32 M so that the prefill can skip those tiles.
#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {

constexpr int kBlock = 128;    // rows and keys per block (the prefill's block-mask granularity)
constexpr int kThreads = 256;  // 32 float4 columns x 8 rows per step

// One workgroup per (batch, head, query block, key block), flattened as
// ((bh * n_qb) + qb) * n_kb + kb.  Each thread reads float4 columns of 8
// rows apart; the workgroup ORs "some entry > -inf" over the block.
__global__ __launch_bounds__(kThreads) void block_keep_kernel(const float* bias, int S_q, int S_k, int ld, int n_qb,
                                                              int n_kb, uint8_t* out) {
  const long long id = blockIdx.x;
  const int kb = (int)(id % n_kb);
  const long long r = id / n_kb;
  const int qb = (int)(r % n_qb);
  const long long bh = r / n_qb;
  const int tid = threadIdx.x;
  const int c4 = tid & 31, rr = tid >> 5;
  const int j = kb * kBlock + 4 * c4;
  bool any = false;
  if (j < S_k) {
    const float* base = bias + ((size_t)bh * S_q) * ld + j;
    for (int row = rr; row < kBlock; row += kThreads / 32) {
      const int i = qb * kBlock + row;
      if (i >= S_q) break;
      // j <= ld - 4 (ld and j are multiples of 4, j < S_k <= ld): in the row
      const f32x4 m = *(const f32x4*)(base + (size_t)i * ld);
#pragma unroll
      for (int e = 0; e < 4; ++e) any = any || (j + e < S_k && m[e] > -INFINITY);
    }
  }
  any = __syncthreads_or(any);
  if (tid == 0) out[id] = any ? 1 : 0;
}

}  // namespace

hipError_t launch_block_keep_from_bias(const float* bias, int B, int heads, int S_q, int S_k, int ld,
                                       uint8_t* block_keep, hipStream_t stream) {
  const int n_qb = (S_q + kBlock - 1) / kBlock, n_kb = (S_k + kBlock - 1) / kBlock;
  const long long n = (long long)B * heads * n_qb * n_kb;
  if (n <= 0) return hipSuccess;
  if (n > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(block_keep_kernel, dim3((unsigned)n), dim3(kThreads), 0, stream, bias, S_q, S_k, ld, n_qb, n_kb,
                     block_keep);
  return hipGetLastError();
}

}  // namespace attn
