// attn_prefill_bf16.hip -- fused exact attention forward, bf16 in / fp32
// accumulate, for gfx950 (MI355X).
//
// What is computed: O = softmax(Q K^T * scale + M) V and the per-row LSE
// (page "Attention Kernel", section "问题与成本"), by streaming K/V tiles
// against a resident Q tile and rescaling a running (m, l, o) state per query
// row (page "Attention 算子加速史", section 1.3; page "Attention Kernel",
// section "Online softmax").  The score tile lives only in registers.
//
// Work decomposition (page "Attention 算子加速史", section 2.1, loop order:
// outer over query tiles, inner over key/value tiles; section 2.3 read as each
// wavefront owning disjoint query rows so no wave ever merges state with
// another).  A workgroup = 4 wave64s = 128 query rows of one (batch, head);
// wave w owns rows 32w..32w+31.  Key/value tiles of 64 rows are double
// buffered in LDS and shared by the 4 waves.
//
// Per tile and wave, on the matrix cores (v_mfma_f32_32x32x16_bf16):
//   S^T[key, query] = K_tile . Q^T      -- A operand K from LDS, B operand Q
//                                          from registers.  The result puts one
//                                          query per lane (lane % 32) and 16
//                                          keys per lane, so row max / row sum
//                                          are in-lane plus one exchange with
//                                          lane ^ 32.
//   O^T[d, query] += V^T . P^T          -- B operand P^T straight from the S^T
//                                          registers (as bf16); A operand V^T
//                                          read from the row-major V tile with
//                                          the transposing LDS read.  O^T keeps
//                                          one query per lane, so the rescale
//                                          by exp(m_old - m_new) is per lane.
// The softmax runs in base 2: s * scale * log2(e) feeds v_exp_f32 directly;
// LSE is converted back to natural log at the end.  Division by the
// normaliser happens once, in the epilogue (page "Attention 算子加速史",
// section 2.2).
//
// Causal: tiles wholly above the diagonal are never loaded; a wave whose rows
// all precede a tile skips it; only tiles crossing the diagonal take the
// per-element predicate (page "Attention Kernel", section "FlashAttention 的
// 稳定基础").  Query tiles are issued heaviest first (most key tiles) so the
// tail of the grid holds the short ones (page "快速Transformer（续）",
// section "Stream-K", wave quantisation).
#include "attn_device.h"
#include "attn_kernels.h"
#include "attn_rowblock.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kRows = 32 * kWaves;  // query rows per workgroup
constexpr int kBc = 64;             // keys per tile
constexpr int kThreads = 64 * kWaves;
static_assert(kRows == kPrefillRows, "row tile");

template <int D, bool kVarlen>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_bf16_kernel(FwdParams p) {
  constexpr int NCH = D / 8;               // 16-byte chunks per row
  constexpr int KSTEPS = D / 16;           // k-steps of the QK^T MFMA
  constexpr int MB = D / 32;               // 32-row blocks of O^T
  constexpr int TILE_CH = kBc * NCH;       // chunks per K (or V) tile
  constexpr int LD_PER_T = TILE_CH / kThreads;
  static_assert(TILE_CH % kThreads == 0, "tile load split");

  // [K buf 0 | K buf 1 | V buf 0 | V buf 1]; the epilogue reuses it for staging
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * kBc * D];
  __shared__ uint8_t sKeep[2][kBc];
  auto sK = [&](int buf) { return smem + buf * (kBc * D); };
  auto sV = [&](int buf) { return smem + (2 + buf) * (kBc * D); };

  RowBlock rb;
  if constexpr (kVarlen) {
    if (!setup_varlen<kRows>(p, D * 2, rb)) return;
  } else {
    rb = setup_dense<kRows>(p, D * 2);
  }

  const uint16_t* gq = (const uint16_t*)rb.q;
  const uint16_t* gk = (const uint16_t*)rb.k;
  const uint16_t* gv = (const uint16_t*)rb.v;
  uint16_t* go = (uint16_t*)rb.o;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;                   // which half of the wave
  const int S_q = rb.S_q, S_k = rb.S_k;
  const int off = S_k - S_q;                 // causal: query i sits at position i + off
  const int qrow = rb.q0 + wave * 32 + l32;  // this lane's query row
  const bool causal = p.causal != 0;

  // ---- number of key tiles this workgroup needs
  int kend = S_k;
  if (causal) kend = min(kend, rb.q0 + kRows - 1 + off + 1);
  const int n_tiles = kend > 0 ? (kend + kBc - 1) / kBc : 0;

  // ---- resident Q operand: lane holds Q[qrow][16t + 8g .. +7] for each t
  bf16x8 qf[KSTEPS];
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t) {
    if (qrow < S_q) {
      qf[t] = *(const bf16x8*)(gq + (size_t)qrow * D + 16 * t + 8 * g);
    } else {
      qf[t] = bf16x8{};
    }
  }

  // ---- tile loader: thread handles LD_PER_T chunks of K and of V
  uint4 kr[LD_PER_T], vr[LD_PER_T];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int i = 0; i < LD_PER_T; ++i) {
      const int cid = tid + i * kThreads;
      const int row = cid / NCH, c = cid % NCH;
      const int key = j * kBc + row;
      if (key < S_k) {
        kr[i] = *(const uint4*)(gk + (size_t)key * D + c * 8);
        vr[i] = *(const uint4*)(gv + (size_t)key * D + c * 8);
      } else {
        kr[i] = uint4{0, 0, 0, 0};
        vr[i] = uint4{0, 0, 0, 0};
      }
    }
  };
  uint8_t keep_r = 1;
  auto load_keep = [&](int j) {
    if (rb.k_keep && tid < kBc) {
      const int key = j * kBc + tid;
      keep_r = key < S_k ? rb.k_keep[key] : 0;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LD_PER_T; ++i) {
      const int cid = tid + i * kThreads;
      const int row = cid / NCH, c = cid % NCH;
      const int pc = lds_chunk<D>(row, c);
      *(uint4*)(sK(buf) + row * D + pc * 8) = kr[i];
      *(uint4*)(sV(buf) + row * D + pc * 8) = vr[i];
    }
    if (rb.k_keep && tid < kBc) sKeep[buf][tid] = keep_r;
  };

  // ---- online-softmax state: m (base-2 scaled running max), l (this half's
  // partial normaliser), o (O^T accumulators: d = 32mb + 8(r/4) + 4g + r%4)
  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x16 acc_o[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc_o[mb] = f32x16{};

  const float cs = p.scale_log2;
  const int wave_q0 = rb.q0 + wave * 32;
  const bool wave_live = wave_q0 < S_q;

  // per-lane LDS byte offsets (within a tile buffer) for the K-operand reads
  // and the transposing V reads; the swizzle depends only on row % 16.
  const int kt_row = l32;  // + 32*kb
  const int j16 = lane & 15, tr_r = j16 >> 2, tr_q = j16 & 3, half16 = (lane >> 4) & 1;
  const int v_row = 4 * g + tr_r;  // + 32kb + 16h (+8 for the second read)

  if (n_tiles > 0) {
    load_tile(0);
    load_keep(0);
    store_tile(0);
  }
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    const bool has_next = j + 1 < n_tiles;
    if (has_next) {
      load_tile(j + 1);
      load_keep(j + 1);
    }
    const int k0 = j * kBc;
    // skip tiles no row of this wave can see
    const bool wave_active = wave_live && !(causal && k0 > wave_q0 + 31 + off);
    if (wave_active) {
      const uint16_t* tK = sK(buf);
      const uint16_t* tV = sV(buf);
      // ---- S^T = K . Q^T : two 32-key blocks
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const int row = 32 * kb + kt_row;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
          const bf16x8 a = *(const bf16x8*)(tK + row * D + lds_chunk<D>(row, 2 * t + g) * 8);
          s[kb] = mfma32(a, qf[t], s[kb]);
        }
      }
      // ---- mask: keys past S_k, causal diagonal, key keep-mask
      const bool need_mask = (k0 + kBc > S_k) || (causal && k0 + kBc - 1 > wave_q0 + off) ||
                             (rb.k_keep != nullptr);
      if (need_mask) {
        const int qpos = qrow + off;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kl = 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
            const int key = k0 + kl;
            bool dead = key >= S_k || (causal && key > qpos);
            if (rb.k_keep) dead = dead || sKeep[buf][kl] == 0;
            if (dead) s[kb][r] = -INFINITY;
          }
        }
      }
      // ---- online softmax (base 2)
      float mx = s[0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
      mx = max_with_other_half(mx);
      const float m_new = fmaxf(m_run, mx * cs);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2_fast(m_run - m_use);
      m_run = m_new;
      const float neg = -m_use;
      float rs = 0.f;
      bf16x8 pb[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = exp2_fast(fmaf(s[kb][r], cs, neg));
          rs += e;
          pb[kb][r >> 3][r & 7] = (__bf16)e;
        }
      }
      l_run = fmaf(l_run, alpha, rs);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc_o[mb] *= alpha;
      // ---- O^T += V^T . P^T
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int c = 4 * mb + 2 * half16 + (tr_q >> 1);
            const int r0 = 32 * kb + 16 * h + v_row;
            const int r1 = r0 + 8;
            const uint16_t* a0 = tV + r0 * D + lds_chunk<D>(r0, c) * 8 + (tr_q & 1) * 4;
            const uint16_t* a1 = tV + r1 * D + lds_chunk<D>(r1, c) * 8 + (tr_q & 1) * 4;
            const bf16x8 a = concat(lds_read_tr16(a0), lds_read_tr16(a1));
            acc_o[mb] = mfma32(a, pb[kb][h], acc_o[mb]);
          }
        }
      }
    }
    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = o / l (0 for an empty row), LSE = ln 2 * (m + log2 l)
  const float l_tot = sum_with_other_half(l_run);
  bool row_ok = qrow < S_q && l_tot > 0.f;
  if (rb.q_keep && qrow < S_q && rb.q_keep[qrow] == 0) row_ok = false;
  const float inv = row_ok ? 1.f / l_tot : 0.f;

  // stage the wave's 32 x D output through LDS for row-contiguous stores
  constexpr int PITCH = D + 8;  // elements; breaks the row-to-bank alignment
  static_assert(kWaves * 32 * PITCH <= 4 * kBc * D, "epilogue staging fits");
  uint16_t* stage = smem + wave * 32 * PITCH;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = 32 * mb + 8 * r4 + 4 * g;
      bf16x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = (__bf16)(acc_o[mb][4 * r4 + i] * inv);
      *(bf16x4*)(stage + l32 * PITCH + d0) = w;
    }
  }
  if (g == 0 && qrow < S_q) {
    rb.lse[qrow] = row_ok ? (m_run + log2_fast(l_tot)) * kLn2 : -INFINITY;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < (32 * NCH) / 64; ++i) {
    const int cid = lane + 64 * i;
    const int row = cid / NCH, c = cid % NCH;
    const int qr = wave_q0 + row;
    if (qr < S_q) {
      const uint4 val = *(const uint4*)(stage + row * PITCH + c * 8);
      *(uint4*)(go + (size_t)qr * D + c * 8) = val;
    }
  }
}

template <int D>
hipError_t launch_d(const FwdParams& p, bool varlen, hipStream_t stream) {
  int grid;
  if (varlen) {
    grid = p.total_tiles * p.A;
  } else {
    grid = p.n_qt * p.A * p.B;
  }
  if (grid <= 0) return hipSuccess;
  if (varlen) {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, true>), dim3(grid), dim3(kThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, false>), dim3(grid), dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const FwdParams& p, bool varlen, hipStream_t stream) {
  if (p.d == 128) return launch_d<128>(p, varlen, stream);
  if (p.d == 64) return launch_d<64>(p, varlen, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
