// attn_bwd_bf16.hip -- backward pass of the fused exact attention prefill,
// bf16 in / fp32 accumulate, for gfx950 (MI355X).
//
// What is computed: dQ, dK, dV of O = softmax(Q K^T * scale + M) V for an
// incoming dO.  Nothing of the forward is stored but O and the per-row LSE;
// every tile recomputes its probabilities P = exp(s * scale - LSE) from Q and
// K (page "Attention 算子加速史", FAQ Q1: recompute instead of storing the
// N x N matrix; page "Attention Kernel", section "Backward 与重计算": the
// forward's log-sum-exp decides how the backward recomputes, with the same
// scale, mask and GQA mapping).  The chain rule, per row i and key j:
//   dV_j += P_ij dO_i,   dP_ij = dO_i . v_j,   D_i = rowsum(dO_i * O_i),
//   dS_ij = P_ij (dP_ij - D_i),   dQ_i = scale sum_j dS_ij k_j,
//   dK_j += scale sum_i dS_ij q_i.
// (D_i = sum_j P_ij dP_ij because O_i = sum_j P_ij v_j.)
//
// Three launches, none of which writes the same output element twice, so the
// result is deterministic and needs no atomics (the "no race in accumulation"
// requirement of the same section):
//   1. delta: D_i = rowsum(dO_i * O_i) into the caller's workspace;
//   2. dQ: one workgroup per 128 query rows of one (batch, head), streaming the
//      K/V tiles of its KV head -- the forward's layout (one query per lane):
//        S^T = K . Q^T,  dP^T = V . dO^T  (Q and dO rows resident),
//        dQ^T += K^T . dS^T  (K^T through the transposing LDS read);
//   3. dK/dV: one workgroup per 128 keys of one (batch, KV head), four waves
//      of 32 keys each, streaming 32-row blocks of Q and dO of every query
//      head that reads this KV head (this is the GQA sum), one key per lane:
//        S = Q . K^T,  dP = dO . V^T  (K and V rows resident),
//        dV^T += dO^T . P,  dK^T += Q^T . dS  (transposing reads of Q, dO).
// The per-element predicate (causal bottom-right diagonal, keep masks, rows
// and keys past the ends) is the forward's; rows whose LSE is -inf (fully
// masked) take no part.
#include <type_traits>

#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kKeyTile = 64;  // keys per tile in the dQ kernel
constexpr int kQBlock = 32;   // query rows per block in the dK/dV kernel
static_assert(kBwdQRows == 128 && kBwdKRows == 128, "four waves of 32");

// ---------------------------------------------------------------- delta
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_delta_kernel(BwdParams p, int n_rows) {
  constexpr int LPR = D / 8;              // lanes per row, 8 elements each
  constexpr int RPW = kThreads / LPR;     // rows per workgroup
  const int row = blockIdx.x * RPW + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < n_rows) {
    const bf16x8 a = *(const bf16x8*)((const uint16_t*)p.dout + (size_t)row * D + 8 * c);
    const bf16x8 b = *(const bf16x8*)((const uint16_t*)p.o + (size_t)row * D + 8 * c);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf((float)a[i], (float)b[i], acc);
  }
#pragma unroll
  for (int o = LPR / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (row < n_rows && c == 0) p.delta[row] = acc;
}

// Copy rows [r0, r0 + NROWS) of a row-major [rows_total, D] bf16 tensor into an
// LDS tile with the forward's chunk swizzle; rows past rows_total arrive as
// zeros (range-checked buffer resource).  All kThreads threads take part.
template <int D, int NROWS>
__device__ __forceinline__ void copy_rows(const uint16_t* base, int rows_total, int r0, uint32_t lds_dst) {
  constexpr int NCH = D / 8;
  constexpr int SLOTS = NROWS * NCH;
  constexpr int PARTS = SLOTS / kThreads;
  constexpr int RPC = kThreads / NCH;  // rows per part
  static_assert(SLOTS % kThreads == 0, "tile split");
  const int tid = threadIdx.x;
  const int rowc = tid / NCH, pcc = tid % NCH;
  const int cc = lds_chunk<D>(rowc, pcc);  // RPC is a multiple of 16, so part i has the same swizzle
  const int rows = min(max(rows_total - r0, 0), NROWS);
  const i32x4 rsrc = make_buffer_rsrc(base + (size_t)r0 * D, (uint32_t)(rows * D * 2));
  const uint32_t wave_base = lds_dst + (uint32_t)__builtin_amdgcn_readfirstlane(tid >> 6) * 1024u;
#pragma unroll
  for (int i = 0; i < PARTS; ++i)
    lds_copy16_buf(rsrc, (uint32_t)((i * RPC + rowc) * D * 2 + cc * 16), wave_base + (uint32_t)(i * RPC * D * 2));
}

// ---------------------------------------------------------------- dQ
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 2))) void bwd_dq_kernel(BwdParams p,
                                                                                                    int n_qt) {
  constexpr int KSTEPS = D / 16;
  constexpr int MB = D / 32;
  constexpr int TILE_BYTES = kKeyTile * D * 2;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kKeyTile * D];  // [K tile | V tile]
  __shared__ uint8_t sKeep[kKeyTile];

  // heaviest query tiles first (most causal key tiles), then batch * head
  const int lin = blockIdx.x;
  const int bh_n = p.A * p.B;
  const int qt = n_qt - 1 - lin / bh_n;
  const int bh = lin % bh_n;
  const int h = bh % p.A, b = bh / p.A, hk = h / p.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, g = lane >> 5;
  const int S_q = p.S_q, S_k = p.S_k, off = S_k - S_q;
  const bool causal = p.causal != 0;
  const size_t q_row0 = (size_t)(b * p.A + h) * S_q;
  const size_t k_row0 = (size_t)(b * p.A_kv + hk) * S_k;
  const int q0 = qt * kBwdQRows;
  const int qrow = q0 + wave * 32 + l32;
  const bool row_in = qrow < S_q;

  // resident Q and dO rows of this lane's query; its base-2 LSE (+inf when the
  // row takes no part, so that every p of it is exactly 0) and delta
  bf16x8 qf[KSTEPS], dof[KSTEPS];
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t) {
    qf[t] = row_in ? *(const bf16x8*)((const uint16_t*)p.q + (q_row0 + qrow) * D + 16 * t + 8 * g) : bf16x8{};
    dof[t] = row_in ? *(const bf16x8*)((const uint16_t*)p.dout + (q_row0 + qrow) * D + 16 * t + 8 * g) : bf16x8{};
  }
  float lrow = INFINITY, drow = 0.f;
  if (row_in) {
    const float lse = p.lse[q_row0 + qrow];
    const bool keep = p.q_keep == nullptr || p.q_keep[(size_t)b * S_q + qrow] != 0;
    if (keep && lse != -INFINITY) lrow = lse * kLog2e;
    drow = p.delta[q_row0 + qrow];
  }

  int kend = S_k;
  if (causal) kend = min(kend, q0 + kBwdQRows - 1 + off + 1);
  const int n_tiles = kend > 0 ? (kend + kKeyTile - 1) / kKeyTile : 0;

  int koff[KSTEPS];  // row-major operand read: row l32, chunk 2t + g
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t) koff[t] = (l32 * D + lds_chunk<D>(l32, 2 * t + g) * 8) * 2;
  const int j16 = lane & 15, tr_r = j16 >> 2, tr_q = j16 & 3, half16 = (lane >> 4) & 1;
  const int v_row = 4 * g + tr_r;
  int voff[MB][2];  // transposing read of d-block mb: rows v_row + 8 rd
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int row = v_row + 8 * rd;
      const int c = 4 * mb + 2 * half16 + (tr_q >> 1);
      voff[mb][rd] = (row * D + lds_chunk<D>(row, c) * 8 + (tr_q & 1) * 4) * 2;
    }
  }
  const char* lds = (const char*)smem;
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
  const float cs = p.scale_log2;

  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x16{};

  for (int j = 0; j < n_tiles; ++j) {
    const int k0 = j * kKeyTile;
    __syncthreads();  // every wave is done with the previous tile
    copy_rows<D, kKeyTile>((const uint16_t*)p.k + k_row0 * D, S_k, k0, lds_base);
    copy_rows<D, kKeyTile>((const uint16_t*)p.v + k_row0 * D, S_k, k0, lds_base + TILE_BYTES);
    if (p.k_keep && tid < kKeyTile) {
      const int key = k0 + tid;
      sKeep[tid] = key < S_k ? p.k_keep[(size_t)b * S_k + key] : 0;
    }
    lds_copy_wait_all();
    __syncthreads();

    // S^T = K . Q^T and dP^T = V . dO^T: two 32-key blocks
    f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t) {
        const bf16x8 ka = *(const bf16x8*)(lds + kb * 32 * D * 2 + koff[t]);
        const bf16x8 va = *(const bf16x8*)(lds + TILE_BYTES + kb * 32 * D * 2 + koff[t]);
        s[kb] = mfma32(ka, qf[t], s[kb]);
        dp[kb] = mfma32(va, dof[t], dp[kb]);
      }
    }
    // element (kb, r) holds key k0 + kl, kl = 32kb + 8(r/4) + 4g + r%4
    bool valid = k0 + lane < S_k;
    if (p.k_keep) valid = valid && sKeep[lane] != 0;
    const uint64_t kvalid = __ballot(valid) >> (4 * g);
    const int lim = causal ? qrow + off - k0 - 4 * g : (1 << 30);
    bf16x8 dsb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 32 * kb + 8 * (r >> 2) + (r & 3);
        const bool live = ((kvalid >> c) & 1) && c <= lim;
        const float pr = live ? exp2_fast(fmaf(s[kb][r], cs, -lrow)) : 0.f;
        dsb[kb][r >> 3][r & 7] = (__bf16)(pr * (dp[kb][r] - drow));
      }
    }
    // dQ^T += K^T . dS^T
#pragma unroll
    for (int kh = 0; kh < 4; ++kh) {
      const int kb = kh >> 1, hh = kh & 1;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const char* base = lds + (32 * kb + 16 * hh) * D * 2;
        const bf16x8 kt = concat(lds_read_tr16(base + voff[mb][0]), lds_read_tr16(base + voff[mb][1]));
        acc[mb] = mfma32(kt, dsb[kb][hh], acc[mb]);
      }
    }
  }

  // dQ = scale * (dQ^T)^T: lane holds d = 32mb + 8(r/4) + 4g + r%4 of its row
  if (row_in) {
    uint16_t* dst = (uint16_t*)p.dq + (q_row0 + qrow) * D + 4 * g;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (__bf16)(acc[mb][4 * r4 + i] * p.scale);
        *(bf16x4*)(dst + 32 * mb + 8 * r4) = w;
      }
    }
  }
}

// ---------------------------------------------------------------- dK / dV
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dkdv_kernel(BwdParams p,
                                                                                                      int n_kt) {
  constexpr int KSTEPS = D / 16;
  constexpr int MB = D / 32;
  constexpr int BLOCK_BYTES = kQBlock * D * 2;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kQBlock * D];  // [Q block | dO block]
  __shared__ __attribute__((aligned(16))) float sL[kQBlock];  // base-2 LSE (+inf: row takes no part)
  __shared__ __attribute__((aligned(16))) float sD[kQBlock];  // delta

  // key tiles in order (the first ones see the most query rows when causal),
  // then batch * KV head
  const int lin = blockIdx.x;
  const int bk_n = p.A_kv * p.B;
  const int kt = lin / bk_n;
  const int bk = lin % bk_n;
  const int hk = bk % p.A_kv, b = bk / p.A_kv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, g = lane >> 5;
  const int S_q = p.S_q, S_k = p.S_k, off = S_k - S_q;
  const bool causal = p.causal != 0;
  const size_t k_row0 = (size_t)(b * p.A_kv + hk) * S_k;
  const int kw0 = kt * kBwdKRows + wave * 32;  // this wave's first key
  const int key = kw0 + l32;                   // this lane's key
  bool key_live = key < S_k;
  if (key_live && p.k_keep) key_live = p.k_keep[(size_t)b * S_k + key] != 0;

  bf16x8 kres[KSTEPS], vres[KSTEPS];
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t) {
    kres[t] = key < S_k ? *(const bf16x8*)((const uint16_t*)p.k + (k_row0 + key) * D + 16 * t + 8 * g) : bf16x8{};
    vres[t] = key < S_k ? *(const bf16x8*)((const uint16_t*)p.v + (k_row0 + key) * D + 16 * t + 8 * g) : bf16x8{};
  }

  int koff[KSTEPS];
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t) koff[t] = (l32 * D + lds_chunk<D>(l32, 2 * t + g) * 8) * 2;
  const int j16 = lane & 15, tr_r = j16 >> 2, tr_q = j16 & 3, half16 = (lane >> 4) & 1;
  const int v_row = 4 * g + tr_r;
  int voff[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int row = v_row + 8 * rd;
      const int c = 4 * mb + 2 * half16 + (tr_q >> 1);
      voff[mb][rd] = (row * D + lds_chunk<D>(row, c) * 8 + (tr_q & 1) * 4) * 2;
    }
  }
  const char* lds = (const char*)smem;
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
  const float cs = p.scale_log2;

  f32x16 acc_dk[MB], acc_dv[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc_dk[mb] = acc_dv[mb] = f32x16{};

  // query rows that can see a key of this workgroup: i + off >= first key
  const int k_first = kt * kBwdKRows;
  const int i_first = causal ? max(k_first - off, 0) : 0;
  const int qb_first = i_first / kQBlock;
  const int n_qb = (S_q + kQBlock - 1) / kQBlock;

  for (int gh = 0; gh < p.G; ++gh) {
    const int h = hk * p.G + gh;
    const size_t q_row0 = (size_t)(b * p.A + h) * S_q;
    for (int qb = qb_first; qb < n_qb; ++qb) {
      const int r0 = qb * kQBlock;
      __syncthreads();  // every wave is done with the previous block
      copy_rows<D, kQBlock>((const uint16_t*)p.q + q_row0 * D, S_q, r0, lds_base);
      copy_rows<D, kQBlock>((const uint16_t*)p.dout + q_row0 * D, S_q, r0, lds_base + BLOCK_BYTES);
      if (tid < kQBlock) {
        const int row = r0 + tid;
        float lv = INFINITY, dv = 0.f;
        if (row < S_q) {
          const float lse = p.lse[q_row0 + row];
          const bool keep = p.q_keep == nullptr || p.q_keep[(size_t)b * S_q + row] != 0;
          if (keep && lse != -INFINITY) lv = lse * kLog2e;
          dv = p.delta[q_row0 + row];
        }
        sL[tid] = lv;
        sD[tid] = dv;
      }
      lds_copy_wait_all();
      __syncthreads();

      // S = Q . K^T, dP = dO . V^T for this wave's 32 keys
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t) {
        const bf16x8 qa = *(const bf16x8*)(lds + koff[t]);
        const bf16x8 da = *(const bf16x8*)(lds + BLOCK_BYTES + koff[t]);
        s = mfma32(qa, kres[t], s);
        dp = mfma32(da, vres[t], dp);
      }
      // element r holds query row r0 + m, m = 8(r/4) + 4g + r%4, of this lane's key
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int m0 = 8 * r4 + 4 * g;
        const float4 lv = *(const float4*)(sL + m0);
        const float4 dv = *(const float4*)(sD + m0);
        const float lvv[4] = {lv.x, lv.y, lv.z, lv.w}, dvv[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * r4 + i;
          const int row = r0 + m0 + i;
          bool live = key_live;
          if (causal) live = live && key <= row + off;
          const float pr = live ? exp2_fast(fmaf(s[r], cs, -lvv[i])) : 0.f;
          pb[r >> 3][r & 7] = (__bf16)pr;
          dsb[r >> 3][r & 7] = (__bf16)(pr * (dp[r] - dvv[i]));
        }
      }
      // dV^T += dO^T . P and dK^T += Q^T . dS: two 16-row k-steps
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const char* qbase = lds + 16 * kk * D * 2;
          const char* dbase = lds + BLOCK_BYTES + 16 * kk * D * 2;
          const bf16x8 dt = concat(lds_read_tr16(dbase + voff[mb][0]), lds_read_tr16(dbase + voff[mb][1]));
          const bf16x8 qt_ = concat(lds_read_tr16(qbase + voff[mb][0]), lds_read_tr16(qbase + voff[mb][1]));
          acc_dv[mb] = mfma32(dt, pb[kk], acc_dv[mb]);
          acc_dk[mb] = mfma32(qt_, dsb[kk], acc_dk[mb]);
        }
      }
    }
  }

  // dK = scale * (dK^T)^T, dV = (dV^T)^T: lane holds d = 32mb + 8(r/4) + 4g + r%4
  if (key < S_k) {
    uint16_t* dkp = (uint16_t*)p.dk + (k_row0 + key) * D + 4 * g;
    uint16_t* dvp = (uint16_t*)p.dv + (k_row0 + key) * D + 4 * g;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 wk, wv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          wk[i] = (__bf16)(acc_dk[mb][4 * r4 + i] * p.scale);
          wv[i] = (__bf16)acc_dv[mb][4 * r4 + i];
        }
        *(bf16x4*)(dkp + 32 * mb + 8 * r4) = wk;
        *(bf16x4*)(dvp + 32 * mb + 8 * r4) = wv;
      }
    }
  }
}

template <int D>
hipError_t launch_bwd_d(const BwdParams& p, hipStream_t stream) {
  const int n_rows = p.B * p.A * p.S_q;
  if (n_rows > 0) {
    constexpr int RPW = kThreads / (D / 8);
    hipLaunchKernelGGL(bwd_delta_kernel<D>, dim3((n_rows + RPW - 1) / RPW), dim3(kThreads), 0, stream, p, n_rows);
    const int n_qt = (p.S_q + kBwdQRows - 1) / kBwdQRows;
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3(n_qt * p.A * p.B), dim3(kThreads), 0, stream, p, n_qt);
  }
  if (p.S_k > 0) {
    // with no query row every key gradient is zero; the kernel still writes them
    const int n_kt = (p.S_k + kBwdKRows - 1) / kBwdKRows;
    hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3(n_kt * p.A_kv * p.B), dim3(kThreads), 0, stream, p, n_kt);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream) {
  if (p.d == 128) return launch_bwd_d<128>(p, stream);
  if (p.d == 64) return launch_bwd_d<64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
