// attn_decode_bf16.hip -- single-query decode over a paged KV cache, split
// along the KV length, merged by log-sum-exp (gfx950).
//
// Paged addressing (page "Attention Kernel", section "Paged 与 ragged KV"):
// token t of sequence b lives in physical page block_table[b][t / page_size]
// at offset t % page_size; a cache row is [page][offset][kv head][d].
//
// Split-KV (page "Attention 算子加速史", section 4.2; page "快速Transformer
// （续）", section "Stream-K", split-K with a fix-up pass): every sequence's
// keys are cut into splits of `split_tokens`; one wavefront handles one
// (sequence, split, KV head) unit for all G = A / A_kv query heads that share
// the KV head (page "Attention Kernel", GQA paragraph), and writes a partial
// output normalised within its split plus the split's log-sum-exp.  The merge
// kernel combines the partials of a (sequence, head) with the two-state rule
// of page "Attention Kernel", section "Online softmax":
//     lse = log sum_s exp(lse_s),   O = sum_s exp(lse_s - lse) O_s.
// Splits depend only on seq_lens, so the result is the same for any choice of
// physical pages.
//
// Matrix-core mapping (v_mfma_f32_16x16x32_bf16), per 32-token chunk:
//   S^T[token, head] = K_chunk . Q^T     (A = K straight from global memory:
//                                         lane holds 8 consecutive d of one
//                                         token row; B = Q^T, heads >= G are 0)
//   O^T[d, head]    += V^T . P^T         (B = P^T from the S^T registers;
//                                         A = V^T from the transposing LDS
//                                         read of the row-major V chunk)
// Decode is bound by HBM bandwidth (each KV byte feeds ~4 flops, page
// "Attention Kernel", section "Prefill 与 decode 是两种 kernel"), so the
// design goal is many 16-byte loads in flight per CU; the matrix cores only
// keep the arithmetic off the critical path.
#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {

constexpr int kChunk = 32;  // tokens per inner step (two 16-token blocks)

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

template <int D>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeParams p) {
  constexpr int NCH = D / 8;
  constexpr int KSTEPS = D / 32;  // k-steps of the 16x16x32 QK MFMA
  constexpr int MB = D / 16;      // 16-row blocks of O^T
  __shared__ __attribute__((aligned(16))) uint16_t sV[kChunk * D];

  const int lane = threadIdx.x;
  const int l16 = lane & 15, grp = lane >> 4;
  const int g = blockIdx.x % p.A_kv;
  int unit = blockIdx.x / p.A_kv;

  // ---- locate (sequence b, split s) of this unit: units are numbered
  // sequence-major, sequence b owning ceil(len_b / split_tokens) of them.
  const int C = p.split_tokens;
  int b = -1, s = 0, len = 0;
  for (int base = 0; base < p.B; base += 64) {
    const int bb = base + lane;
    const int lb = bb < p.B ? p.seq_lens[bb] : 0;
    const int ns = (lb + C - 1) / C;
    const int incl = wave_incl_scan(ns, lane);
    const int total = __shfl(incl, 63);
    if (unit < total) {
      const uint64_t m = __ballot(incl > unit);
      const int src = __ffsll((long long)m) - 1;
      b = base + src;
      s = unit - (__shfl(incl, src) - __shfl(ns, src));
      len = __shfl(lb, src);
      break;
    }
    unit -= total;
  }
  if (b < 0) return;

  const int G = p.G;
  const int t_begin = s * C;
  const int t_end = min(len, t_begin + C);

  // ---- Q^T operand: lane holds Q[head l16][32t + 8 grp .. +7]; heads >= G are 0
  const uint16_t* qb = (const uint16_t*)p.q + ((size_t)b * p.A + (size_t)g * G) * D;
  bf16x8 qf[KSTEPS];
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t) {
    qf[t] = l16 < G ? *(const bf16x8*)(qb + (size_t)l16 * D + 32 * t + 8 * grp) : bf16x8{};
  }

  const uint16_t* kc = (const uint16_t*)p.k_cache;
  const uint16_t* vc = (const uint16_t*)p.v_cache;
  const int32_t* bt = p.block_table + (size_t)b * p.max_pages;
  const size_t row_stride = (size_t)p.A_kv * D;  // elements between tokens of a page

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{};
  const float cs = p.scale_log2;

  for (int c0 = t_begin; c0 < t_end; c0 += kChunk) {
    // ---- gather: lane reads token (c0 + 16 tb + l16), d chunk (4 t + grp)
    uint4 kr[2][KSTEPS], vr[2][KSTEPS];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int tok = c0 + 16 * tb + l16;
      if (tok < t_end) {
        const int page = bt[tok / p.page_size];
        const size_t row = ((size_t)page * p.page_size + (tok % p.page_size)) * row_stride + (size_t)g * D;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
          kr[tb][t] = *(const uint4*)(kc + row + 32 * t + 8 * grp);
          vr[tb][t] = *(const uint4*)(vc + row + 32 * t + 8 * grp);
        }
      } else {
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
          kr[tb][t] = uint4{0, 0, 0, 0};
          vr[tb][t] = uint4{0, 0, 0, 0};
        }
      }
    }
    // ---- V chunk to LDS, row-major [token][d] with a 16-byte-chunk swizzle
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int row = 16 * tb + l16;
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t) {
        const int c = 4 * t + grp;
        *(uint4*)(sV + row * D + (c ^ (row & (NCH - 1))) * 8) = vr[tb][t];
      }
    }
    // ---- S^T = K . Q^T
    f32x4 sc[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      sc[tb] = f32x4{};
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t) {
        sc[tb] = mfma16(__builtin_bit_cast(bf16x8, kr[tb][t]), qf[t], sc[tb]);
      }
    }
    // lane holds tokens c0 + 16 tb + 4 grp + r of head l16
    float mx = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = c0 + 16 * tb + 4 * grp + r;
        if (tok >= t_end) sc[tb][r] = -INFINITY;
        mx = fmaxf(mx, sc[tb][r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = max_with_other_half(mx);
    const float m_new = fmaxf(m_run, mx * cs);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2_fast(m_run - m_use);
    m_run = m_new;
    bf16x8 pb;
    float rs = 0.f;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = exp2_fast(fmaf(sc[tb][r], cs, -m_use));
        rs += e;
        pb[4 * tb + r] = (__bf16)e;
      }
    }
    l_run = fmaf(l_run, alpha, rs);
    // ---- O^T += V^T . P^T ; V^T slot s of lane group grp = token
    // (s < 4 ? 4 grp + s : 16 + 4 grp + s - 4), matching pb
    const int tr_r = l16 >> 2, tr_q = l16 & 3;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      acc[mb] *= alpha;
      const int c = 2 * mb + (tr_q >> 1);
      const int r0 = 4 * grp + tr_r, r1 = r0 + 16;
      const uint16_t* a0 = sV + r0 * D + (c ^ (r0 & (NCH - 1))) * 8 + (tr_q & 1) * 4;
      const uint16_t* a1 = sV + r1 * D + (c ^ (r1 & (NCH - 1))) * 8 + (tr_q & 1) * 4;
      acc[mb] = mfma16(concat(lds_read_tr16(a0), lds_read_tr16(a1)), pb, acc[mb]);
    }
  }

  // ---- partial (normalised within the split) and its base-2 LSE
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot = sum_with_other_half(l_tot);
  const bool ok = l_tot > 0.f;
  const float inv = ok ? 1.f / l_tot : 0.f;
  if (l16 < G) {
    const int h = g * G + l16;
    const size_t slot = ((size_t)b * p.n_split + s) * p.A + h;
    float* po = p.part_o + slot * D;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      f32x4 w = acc[mb] * inv;
      *(f32x4*)(po + 16 * mb + 4 * grp) = w;
    }
    if (grp == 0) p.part_lse[slot] = ok ? m_run + log2_fast(l_tot) : -INFINITY;
  }
}

// One wavefront per (sequence, head): combine the sequence's split partials.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeParams p) {
  const int lane = threadIdx.x;
  const int bh = blockIdx.x;
  const int b = bh / p.A, h = bh % p.A;
  const int len = p.seq_lens[b];
  const int ns = (len + p.split_tokens - 1) / p.split_tokens;
  const size_t base = (size_t)b * p.n_split * p.A + h;  // slot of split 0
  float mx = -INFINITY;
  for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, p.part_lse[base + (size_t)s * p.A]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  constexpr int PER = D / 64;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float wsum = 0.f;
  if (mx != -INFINITY) {
    for (int s = 0; s < ns; ++s) {
      const size_t slot = base + (size_t)s * p.A;
      const float ls = p.part_lse[slot];
      if (ls == -INFINITY) continue;
      const float w = exp2_fast(ls - mx);
      wsum += w;
      const float* po = p.part_o + slot * D;
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] = fmaf(w, po[lane + 64 * i], acc[i]);
    }
  }
  const bool ok = wsum > 0.f;
  const float inv = ok ? 1.f / wsum : 0.f;
  uint16_t* o = (uint16_t*)p.o + ((size_t)b * p.A + h) * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    o[lane + 64 * i] = __builtin_bit_cast(uint16_t, (__bf16)(acc[i] * inv));
  }
  if (lane == 0) p.lse[(size_t)b * p.A + h] = ok ? (mx + log2_fast(wsum)) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch_decode_d(const DecodeParams& p, int total_units, hipStream_t stream) {
  if (total_units > 0) {
    hipLaunchKernelGGL(decode_split_kernel<D>, dim3(total_units * p.A_kv), dim3(64), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(decode_merge_kernel<D>, dim3(p.B * p.A), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

DecodePlan plan_decode(int B, int A_kv, int page_size, const int32_t* seq_lens_host) {
  // Split size: aim for ~32k (unit, KV head) wavefronts over the whole batch
  // (>= 100 per CU, so the last round of waves is a small tail), in whole
  // 32-token chunks and whole pages, between 64 and 4096 tokens.
  long long total = 0;
  int max_len = 0;
  for (int b = 0; b < B; ++b) {
    total += seq_lens_host[b];
    max_len = seq_lens_host[b] > max_len ? seq_lens_host[b] : max_len;
  }
  const long long target_units = 32768;
  long long c = (total * A_kv + target_units - 1) / target_units;
  const int quantum = page_size > kChunk ? page_size : kChunk;  // page_size % 16 == 0
  int lcm = quantum;
  while (lcm % kChunk != 0 || lcm % page_size != 0) lcm += quantum;
  if (c < 64) c = 64;
  if (c > 4096) c = 4096;
  c = ((c + lcm - 1) / lcm) * lcm;
  DecodePlan plan;
  plan.split_tokens = (int)c;
  plan.n_split = max_len > 0 ? (int)((max_len + c - 1) / c) : 0;
  return plan;
}

size_t decode_workspace_bytes(int B, int A, int d, const DecodePlan& plan) {
  const size_t slots = (size_t)B * (size_t)plan.n_split * (size_t)A;
  const size_t o_bytes = ((slots * (size_t)d * 4) + 255) / 256 * 256;
  const size_t l_bytes = ((slots * 4) + 255) / 256 * 256;
  return o_bytes + l_bytes;
}

hipError_t launch_decode_bf16(const DecodeParams& p, int total_units, hipStream_t stream) {
  if (p.d == 128) return launch_decode_d<128>(p, total_units, stream);
  if (p.d == 64) return launch_decode_d<64>(p, total_units, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
