// attn_prefill_f32.hip -- fused exact attention forward with fp32 inputs and
// fp32 arithmetic throughout (no reduced-precision step), gfx950.
//
// Same method as the bf16 kernel (page "Attention 算子加速史", sections 1.3 and
// 2.1-2.2; page "Attention Kernel", section "Online softmax"): K/V tiles of 64
// keys stream through LDS, every query row keeps a running (m, l, o) state and
// the division by l happens once at the end.  Scores and products use scalar
// fp32 FMAs on the vector ALUs, so this path is exact to fp32 rounding.
//
// A dense additive mask M (dense batches) enters each score as M / scale
// before the scaling, i.e. s * scale + M.  Per-row key ranges (page
// "Attention Kernel", section "可编程 mask") mask the keys outside each row's
// range.  ALiBi adds -slope_h |p_i - j| the same way (as -slope_h |p_i - j| /
// scale to the raw product).
//
// A workgroup owns 16 query rows; wave w owns rows 4w..4w+3.  In the score
// step lane j computes the scores of key j of the tile for the wave's 4 rows;
// in the output step lane j accumulates output dimensions j and j + 64.
#include "attn_device.h"
#include "attn_kernels.h"
#include "attn_rowblock.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 4;
constexpr int kRows = kWaves * kRowsPerWave;
constexpr int kBc = 64;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxD = 128;
static_assert(kRows == kPrefillRowsF32, "row tile");

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

template <bool kVarlen>
__global__ __launch_bounds__(kThreads) void prefill_f32_kernel(FwdParams p) {
  __shared__ float sQ[kRows][kMaxD];
  __shared__ float sK[kBc][kMaxD + 1];  // +1: lanes read different rows at one column
  __shared__ float sV[kBc][kMaxD];
  __shared__ float sP[kWaves][kRowsPerWave][kBc];
  __shared__ uint8_t sKeep[kBc];

  const int D = p.d;
  RowBlock rb;
  if constexpr (kVarlen) {
    if (!setup_varlen<kRows>(p, D * 4, rb)) return;
  } else {
    rb = setup_dense<kRows>(p, D * 4);
  }
  const float* gq = (const float*)rb.q;
  const float* gk = (const float*)rb.k;
  const float* gv = (const float*)rb.v;
  float* go = (float*)rb.o;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S_q = rb.S_q, S_k = rb.S_k, off = S_k - S_q;
  const int wl = p.win_left, wr = p.win_right;  // window edges (causal folded into wr)
  const float cs = p.scale_log2;

  for (int idx = tid; idx < kRows * D; idx += kThreads) {
    const int r = idx / D, e = idx % D;
    const int row = rb.q0 + r;
    sQ[r][e] = row < S_q ? gq[(size_t)row * D + e] : 0.f;
  }

  // keys some row of the workgroup keeps: [kbeg, kend)
  int kbeg = 0, kend = S_k;
  if (wr >= 0) kend = min(kend, rb.q0 + kRows - 1 + off + wr + 1);
  if (wl >= 0) kbeg = max(rb.q0 + off - wl, 0);
  const int j_lo = kbeg / kBc;
  const int j_hi = kend > kbeg ? (kend + kBc - 1) / kBc : j_lo;

  // dense additive mask (dense batches only): row (b, head, i) of M, added to
  // the raw product as M / scale so that the scaling by scale * log2(e)
  // applies to both
  const float* bias_rows = nullptr;
  if constexpr (!kVarlen) {
    if (p.bias) {
      const int hm = p.bias_heads == 1 ? 0 : rb.h;
      bias_rows = p.bias + (size_t)(rb.b * p.bias_heads + hm) * S_q * p.bias_ld;
    }
  }

  // ALiBi: this head's slope over the scale (0 without ALiBi)
  const float alibi_b = p.alibi_slopes ? p.alibi_slopes[rb.h] * p.inv_scale : 0.f;
  // this wave's rows keep keys [r_lo, r_hi] under their key ranges
  int r_lo[kRowsPerWave], r_hi[kRowsPerWave];
#pragma unroll
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    const int row = rb.q0 + wave * kRowsPerWave + rr;
    int2 r = make_int2(-1, S_k);
    if (rb.key_range && row < S_q) r = load_key_range(rb.key_range, row, S_k);
    r_lo[rr] = r.x;
    r_hi[rr] = r.y;
  }

  float m_run[kRowsPerWave], l_run[kRowsPerWave], acc[kRowsPerWave][2];
#pragma unroll
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    m_run[rr] = -INFINITY;
    l_run[rr] = 0.f;
    acc[rr][0] = acc[rr][1] = 0.f;
  }

  for (int j = j_lo; j < j_hi; ++j) {
    const int k0 = j * kBc;
    __syncthreads();  // previous tile fully consumed (and sQ written)
    for (int idx = tid; idx < kBc * D; idx += kThreads) {
      const int r = idx / D, e = idx % D;
      const int key = k0 + r;
      const bool in = key < S_k;
      sK[r][e] = in ? gk[(size_t)key * D + e] : 0.f;
      sV[r][e] = in ? gv[(size_t)key * D + e] : 0.f;
    }
    if (tid < kBc) {
      const int key = k0 + tid;
      sKeep[tid] = key < S_k ? (rb.k_keep ? rb.k_keep[key] : 1) : 0;
    }
    __syncthreads();

    // scores of key k0 + lane for the wave's rows
    const int key = k0 + lane;
#pragma unroll
    for (int rr = 0; rr < kRowsPerWave; ++rr) {
      const int qr = wave * kRowsPerWave + rr;
      const int row = rb.q0 + qr;
      float s = 0.f;
      for (int e = 0; e < D; ++e) s = fmaf(sQ[qr][e], sK[lane][e], s);
      if (bias_rows && key < S_k && row < S_q) s = fmaf(bias_rows[(size_t)row * p.bias_ld + key], p.inv_scale, s);
      s = fmaf(-fabsf((float)(key - (row + off))), alibi_b, s);
      const bool dead = sKeep[lane] == 0 || (wr >= 0 && key > row + off + wr) || (wl >= 0 && key < row + off - wl) ||
                        key < r_lo[rr] || key > r_hi[rr];
      s = dead ? -INFINITY : s;
      const float mx = wave_max(s);
      const float m_new = fmaxf(m_run[rr], mx * cs);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2_fast(m_run[rr] - m_use);
      m_run[rr] = m_new;
      sP[wave][rr][lane] = exp2_fast(fmaf(s, cs, -m_use));
      l_run[rr] *= alpha;
      acc[rr][0] *= alpha;
      acc[rr][1] *= alpha;
    }
    __syncthreads();  // sP visible to the whole wave
#pragma unroll
    for (int rr = 0; rr < kRowsPerWave; ++rr) {
      float ls = 0.f, a0 = 0.f, a1 = 0.f;
      for (int t = 0; t < kBc; ++t) {
        const float pt = sP[wave][rr][t];
        ls += pt;
        a0 = fmaf(pt, sV[t][lane], a0);
        if (lane + 64 < D) a1 = fmaf(pt, sV[t][lane + 64], a1);
      }
      l_run[rr] += ls;
      acc[rr][0] += a0;
      acc[rr][1] += a1;
    }
  }

#pragma unroll
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    const int row = rb.q0 + wave * kRowsPerWave + rr;
    if (row >= S_q) continue;
    bool ok = l_run[rr] > 0.f;
    if (rb.q_keep && rb.q_keep[row] == 0) ok = false;
    const float inv = ok ? 1.f / l_run[rr] : 0.f;
    if (lane < D) go[(size_t)row * D + lane] = ok ? acc[rr][0] * inv : 0.f;
    if (lane + 64 < D) go[(size_t)row * D + lane + 64] = ok ? acc[rr][1] * inv : 0.f;
    if (lane == 0) rb.lse[row] = ok ? (m_run[rr] + log2_fast(l_run[rr])) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_prefill_f32(const FwdParams& p, bool varlen, hipStream_t stream) {
  if (p.d < 1 || p.d > kMaxD) return hipErrorInvalidValue;
  const int grid = varlen ? p.total_tiles * p.A : p.n_qt * p.A * p.B;
  if (grid <= 0) return hipSuccess;
  if (varlen) {
    hipLaunchKernelGGL(prefill_f32_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL(prefill_f32_kernel<false>, dim3(grid), dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace attn
