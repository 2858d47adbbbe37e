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
#include <type_traits>

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
  constexpr int LD_PER_T = TILE_CH / kThreads;  // 16-byte copies per thread per K (or V) tile
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

  // ---- tile loader: global -> LDS copies (global_load_lds_dwordx4) that do
  // not pass through registers.  One copy round of the workgroup fills RPC
  // tile rows: lane L of wave w the 16 bytes of slot w*64 + L, i.e. row
  // i*RPC + rowc, physical chunk pcc; the global address is chosen so that
  // those bytes hold the row's swizzled chunk.  Only the last tile can reach
  // past S_k; its missing rows re-read row S_k - 1 (finite, masked to weight 0).
  constexpr int RPC = kThreads / NCH;  // rows per copy round (a multiple of 16)
  constexpr int TILE_BYTES = kBc * D * 2;
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
  const int rowc = (wave * 64 + lane) / NCH, pcc = (wave * 64 + lane) % NCH;
  const int cc = lds_chunk<D>(rowc, pcc);  // the swizzle is an involution; it depends on row % 16 only
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // wave index in a scalar register
  // Copy part `part` (of LD_PER_T) of tile j into buffer buf: one K and one V
  // 16-byte copy per lane.  The parts are issued at spread-out points of the
  // previous tile's computation, so the waves of a CU do not all queue their
  // copies on the load path at the same moment.
  auto copy_part = [&](int j, int buf, int i) {
    const int key = min(j * kBc + i * RPC + rowc, S_k - 1);
    const uint16_t* src = gk + (size_t)key * D + cc * 8;
    const size_t vdiff = (size_t)(gv - gk);
    const uint32_t lk = lds_base + (uint32_t)(buf * TILE_BYTES + i * RPC * D * 2) + (uint32_t)wave_u * 1024u;
    lds_copy16(src, lk);
    lds_copy16(src + vdiff, lk + 2 * TILE_BYTES);
  };
  auto copy_keep = [&](int j, int buf) {
    if (rb.k_keep && tid < kBc) {
      const int key = j * kBc + tid;
      sKeep[buf][tid] = key < S_k ? rb.k_keep[key] : 0;
    }
  };
  auto copy_tile = [&](int j, int buf) {
#pragma unroll
    for (int i = 0; i < LD_PER_T; ++i) copy_part(j, buf, i);
    copy_keep(j, buf);
  };

  // ---- online-softmax state.  m_ref: the base-2 reference the exponentials
  // of this row are taken against (-inf until the row has seen a key); l: this
  // lane-half's partial normaliser; acc_o: O^T accumulators (d = 32mb +
  // 8(r/4) + 4g + r%4 of this lane's query).  m_ref only moves when a tile's
  // max exceeds it by more than kLazy (so p <= 2^kLazy); o and l always share
  // the same reference, so the final o / l is the exact softmax average
  // whatever reference was used (page "Attention Kernel", Online softmax:
  // the state may be rescaled by any common factor).
  constexpr float kLazy = 8.f;
  float m_ref = -INFINITY;
  float l_run = 0.f;
  f32x16 acc_o[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc_o[mb] = f32x16{};

  const float cs = p.scale_log2;
  const int wave_q0 = rb.q0 + wave * 32;
  const bool wave_live = wave_q0 < S_q;

  // ---- per-lane LDS byte offsets of the operand reads inside a tile buffer.
  // The swizzle depends on row % 16 only, so the row blocks (32 rows per kb,
  // 16 per h) and the buffer choice are compile-time immediates.
  int koff[KSTEPS];  // K operand of k-step t: row l32, chunk 2t + g
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t) koff[t] = (l32 * D + lds_chunk<D>(l32, 2 * t + g) * 8) * 2;
  const int j16 = lane & 15, tr_r = j16 >> 2, tr_q = j16 & 3, half16 = (lane >> 4) & 1;
  const int v_row = 4 * g + tr_r;
  int voff[MB][2];  // transposing V read rd of block mb: row v_row + 8 rd, chunk 4mb + 2 half16 + tr_q/2
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

  // One key tile for this wave.  BUF is the tile's LDS buffer (compile time).
  // MASKED selects the per-element predicate (keys past S_k, the causal
  // diagonal, the key keep-mask); interior tiles take the unmasked instance.
  // Operand reads run PF steps ahead of the MFMAs that consume them.
  auto tile = [&](auto masked_tag, auto buf_tag, int k0, auto&& issue_copy) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr int BUF = decltype(buf_tag)::value;
    constexpr int KB = BUF * TILE_BYTES;            // K tile of this buffer
    constexpr int VB = (2 + BUF) * TILE_BYTES;      // V tile of this buffer
    constexpr int PF = 3;
    // ---- S^T = K . Q^T : two 32-key blocks, k-steps interleaved across them
    constexpr int NQ = 2 * KSTEPS;
    f32x16 s[2] = {f32x16{}, f32x16{}};
    bf16x8 ka[NQ];
    auto kread = [&](int p) {  // step p: kb = p % 2, t = p / 2
      ka[p] = *(const bf16x8*)(lds + KB + (p % 2) * 32 * D * 2 + koff[p / 2]);
    };
#pragma unroll
    for (int p = 0; p < PF; ++p) kread(p);
    issue_copy(0);
#pragma unroll
    for (int p = 0; p < NQ; ++p) {
      if (p + PF < NQ) kread(p + PF);
      s[p % 2] = mfma32(ka[p], qf[p / 2], s[p % 2]);
      if (p == NQ / 2) issue_copy(1);
    }
    if constexpr (MASKED) {
      // bit k of kvalid: key k0 + k exists and is kept (same for every lane)
      bool valid = k0 + lane < S_k;
      if (rb.k_keep) valid = valid && sKeep[BUF][lane] != 0;
      const uint64_t kvalid = __ballot(valid) >> (4 * g);
      // element (kb, r) holds key k0 + kl, kl = 32kb + 8(r/4) + 4g + r%4;
      // causal: dead when kl > qrow + off - k0
      const int lim = causal ? qrow + off - k0 - 4 * g : (1 << 30);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = 32 * kb + 8 * (r >> 2) + (r & 3);  // kl - 4g
          const bool live = ((kvalid >> c) & 1) && c <= lim;
          s[kb][r] = live ? s[kb][r] : -INFINITY;
        }
      }
    }
    // ---- row max of the tile (raw scores), both lane halves
    float mx0 = fmaxf(s[0][0], s[0][1]), mx1 = fmaxf(s[1][0], s[1][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) {
      mx0 = fmaxf(mx0, fmaxf(s[0][r], s[0][r + 1]));
      mx1 = fmaxf(mx1, fmaxf(s[1][r], s[1][r + 1]));
    }
    const float mxs = max_with_other_half(fmaxf(mx0, mx1)) * cs;  // scale > 0
    // ---- move the reference only when some row of the wave needs it
    if (__builtin_amdgcn_ballot_w64(mxs > m_ref + kLazy) != 0) {
      const float m_new = fmaxf(m_ref, mxs);
      const float alpha = (m_ref == -INFINITY) ? 0.f : exp2_fast(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc_o[mb] *= alpha;
    }
    issue_copy(2);
    const float neg = (m_ref == -INFINITY) ? 0.f : -m_ref;
    float rs0 = 0.f, rs1 = 0.f, rs2 = 0.f, rs3 = 0.f;
    bf16x8 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const float e0 = exp2_fast(fmaf(s[kb][r + 0], cs, neg));
        const float e1 = exp2_fast(fmaf(s[kb][r + 1], cs, neg));
        const float e2 = exp2_fast(fmaf(s[kb][r + 2], cs, neg));
        const float e3 = exp2_fast(fmaf(s[kb][r + 3], cs, neg));
        rs0 += e0;
        rs1 += e1;
        rs2 += e2;
        rs3 += e3;
        pb[kb][r >> 3][(r & 7) + 0] = (__bf16)e0;
        pb[kb][r >> 3][(r & 7) + 1] = (__bf16)e1;
        pb[kb][r >> 3][(r & 7) + 2] = (__bf16)e2;
        pb[kb][r >> 3][(r & 7) + 3] = (__bf16)e3;
      }
    }
    l_run += (rs0 + rs1) + (rs2 + rs3);
    // ---- O^T += V^T . P^T ; steps (kb, h, mb) with mb innermost: MB
    // independent accumulator chains
    constexpr int NV = 4 * MB;
    bf16x8 va[NV];
    auto vread = [&](int q) {  // step q: mb = q % MB, (kb, h) = q / MB
      const int mb = q % MB, kh = q / MB, kb = kh >> 1, h = kh & 1;
      const char* base = lds + VB + (32 * kb + 16 * h) * D * 2;
      va[q] = concat(lds_read_tr16(base + voff[mb][0]), lds_read_tr16(base + voff[mb][1]));
    };
#pragma unroll
    for (int q = 0; q < PF; ++q) vread(q);
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      if (q + PF < NV) vread(q + PF);
      const int mb = q % MB, kh = q / MB;
      acc_o[mb] = mfma32(va[q], pb[kh >> 1][kh & 1], acc_o[mb]);
      if (q == NV / 2) issue_copy(3);
    }
  };

  // ---- main loop, unrolled by the two buffers: tile j sits in buffer j % 2
  auto step = [&](auto buf_tag, int j) {
    constexpr int BUF = decltype(buf_tag)::value;
    // tile j has landed in LDS for this thread's copies; after the barrier,
    // for everyone's -- and every wave is done with tile j-1, whose buffer
    // the copy of tile j+1 below overwrites
    lds_copy_wait_all();
    __syncthreads();
    // the copies of tile j+1 are issued in LD_PER_T parts spread over the
    // computation of tile j (four issue points in tile()).  After the last
    // tile they re-copy it into the idle buffer (harmless, and it keeps the
    // tile body free of branches).
    const int jn = min(j + 1, n_tiles - 1);
    if (j + 1 < n_tiles) copy_keep(j + 1, BUF ^ 1);
    auto issue = [&](int at) {
#pragma unroll
      for (int i = 0; i < LD_PER_T; ++i)
        if (i * 4 / LD_PER_T == at) copy_part(jn, BUF ^ 1, i);
    };
    const int k0 = j * kBc;
    // skip tiles no row of this wave can see
    const bool wave_active = wave_live && !(causal && k0 > wave_q0 + 31 + off);
    if (wave_active) {
      const bool need_mask = (k0 + kBc > S_k) || (causal && k0 + kBc - 1 > wave_q0 + off) ||
                             (rb.k_keep != nullptr);
      if (need_mask) {
        tile(std::integral_constant<bool, true>{}, buf_tag, k0, issue);
      } else {
        tile(std::integral_constant<bool, false>{}, buf_tag, k0, issue);
      }
    } else {
#pragma unroll
      for (int i = 0; i < LD_PER_T; ++i) copy_part(jn, BUF ^ 1, i);
    }
  };
  if (n_tiles > 0) copy_tile(0, 0);
  for (int j = 0; j < n_tiles; j += 2) {
    step(std::integral_constant<int, 0>{}, j);
    if (j + 1 < n_tiles) step(std::integral_constant<int, 1>{}, j + 1);
  }
  lds_copy_wait_all();  // the trailing copies have landed ...
  __syncthreads();      // ... and all reads of the last tile are done before the epilogue reuses LDS

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
    rb.lse[qrow] = row_ok ? (m_ref + log2_fast(l_tot)) * kLn2 : -INFINITY;
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

