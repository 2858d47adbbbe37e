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
// Two launches, neither of which writes an output element twice, so the
// result is deterministic and needs no atomics (the "no race in accumulation"
// requirement of the same section):
//   1. dQ: one workgroup per 128 query rows of one (batch, head), four waves
//      of 32 rows, streaming double-buffered 64-key K/V tiles of its KV head in
//      the forward's layout (one query per lane):
//        S^T = K . Q^T,  dP^T = V . dO^T  (Q and dO rows resident),
//        dQ^T += K^T . dS^T  (K^T through the transposing LDS read);
//      its prologue also forms D_i and the base-2 LSE of each row and stores
//      both in the workspace for the second launch;
//   2. dK/dV: one workgroup per 128 keys of one (batch, KV head), four waves
//      of 32 keys, streaming 32-row blocks of Q, dO and the row
//      statistics of every query head that reads this KV head (this is the GQA
//      sum), one key per lane:
//        S = Q . K^T,  dP = dO . V^T  (V rows in registers; K rows in
//                                      registers, or in LDS for the two-wave
//                                      form at d = 128),
//        dV^T += dO^T . P,  dK^T += Q^T . dS  (transposing reads of Q, dO).
// The per-element predicate (sliding window whose right edge is the causal
// bottom-right diagonal, keep masks, rows and keys past the ends) is the
// forward's; rows whose LSE is -inf (fully masked) take no part.
#include <climits>
#include <type_traits>

#include "attn_bwd.h"
#include "attn_device.h"

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kXcdCount = 8;
constexpr int kKeyTile = 64;  // keys per tile in the dQ kernel
constexpr int kQBlock = 32;   // query rows per block in the dK/dV kernel
static_assert(kBwdQRows == 128 && kBwdKRows == 128, "four waves of 32");

// Copy rows [r0, r0 + NROWS) of a row-major [rows_total, D] bf16 tensor into an
// LDS tile with the forward's chunk swizzle; rows past rows_total arrive as
// zeros (range-checked buffer resource).  All kThreads threads take part; each
// wave issues NROWS * D / 2048 copy instructions.
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

// Grid order.  Workgroups are dealt to the 8 XCDs round-robin by index and
// each XCD has its own L2.  With `group` > 0, XCD x owns the units (batch,
// head pairs) [x * per, (x + 1) * per) and takes them `group` at a time, each
// group's tiles heaviest first (rank 0 first), so the workgroups that stream
// the same K/V (dQ pass) or the same Q/dO (dK/dV pass) run at about the same
// time on one XCD.  Otherwise: rank-major over all units.
__device__ __forceinline__ void grid_order(int lin, int n_tiles, int n_units, int per, int group, int& rank,
                                           int& unit) {
  if (group > 0) {
    const int x = lin % kXcdCount, i = lin / kXcdCount;
    const int per_group = group * n_tiles;
    const int grp = i / per_group, r = i % per_group;
    rank = r / group;
    unit = x * per + grp * group + r % group;
  } else {
    rank = lin / n_units;
    unit = lin % n_units;
  }
}

// Packed sequences: the rank-th workgroup of one head when the sequences'
// 128-row tiles are ordered by tile index t descending, then by sequence.
// count(t) = sum_s max(0, n_s - t) workgroups have an index >= t; a binary
// search finds t, a ballot the sequence.  Returns false past the last tile.
__device__ __forceinline__ bool varlen_tile(const int32_t* cu, int n_seq, int max_tiles, int rank, int& t_out,
                                            int& seq_out) {
  const int lane = threadIdx.x & 63;
  auto ntiles = [&](int s) -> int { return (cu[s + 1] - cu[s] + kBwdQRows - 1) / kBwdQRows; };
  auto count_ge = [&](int t) -> int {
    int c = 0;
    for (int s = lane; s < n_seq; s += 64) c += max(0, ntiles(s) - t);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o);
    return c;
  };
  int lo = 0, hi = max_tiles;  // count_ge(lo) > rank >= count_ge(hi) (= 0)
  if (count_ge(0) <= rank) return false;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (count_ge(mid) > rank) lo = mid; else hi = mid;
  }
  int k = rank - count_ge(lo + 1);  // the k-th sequence (in order) with more than lo tiles
  int seq = -1;
  for (int base = 0; base < n_seq && seq < 0; base += 64) {
    const int s = base + lane;
    const bool has = s < n_seq && ntiles(s) > lo;
    const uint64_t m = __ballot(has);
    const int c = __popcll(m);
    if (k < c) {
      const uint64_t below = m & (lane == 0 ? 0ull : (~0ull >> (64 - lane)));
      const uint64_t w = __ballot(has && __popcll(below) == k);
      seq = base + __ffsll((long long)w) - 1;
    } else {
      k -= c;
    }
  }
  if (seq < 0) return false;
  t_out = __builtin_amdgcn_readfirstlane(lo);
  seq_out = __builtin_amdgcn_readfirstlane(seq);
  return true;
}

template <int N>
using Slot = std::integral_constant<int, N>;

// ---------------------------------------------------------------- dQ
// kVarlen: packed sequences (see BwdParams); kMasks: the block mask, the
// dense additive term and the per-row key ranges (each runtime-optional);
// kRange (without kMasks): per-row key ranges alone; kAlibi: ALiBi.  Two
// waves per SIMD, one for the masked form at d = 128 (at two its term loads
// spill).
template <int D, bool kMasks>
constexpr int kDqWavesPerSimd = (D == 128 && kMasks) ? 1 : 2;

template <int D, bool kVarlen, bool kMasks, bool kRange = false, bool kAlibi = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kDqWavesPerSimd<D, kMasks>, kDqWavesPerSimd<D, kMasks>))) void bwd_dq_kernel(BwdParams p,
                                                                                                    int n_qt) {
  constexpr int KSTEPS = D / 16;
  constexpr int MB = D / 32;
  constexpr int TILE_BYTES = kKeyTile * D * 2;
  constexpr int SLOT_BYTES = 2 * TILE_BYTES;  // [K tile | V tile]
  constexpr int NSLOT = 2;
  __shared__ __attribute__((aligned(16))) uint16_t smem[NSLOT * SLOT_BYTES / 2];
  // block mask: flag of each 128-key block of this row block's key range
  __shared__ uint8_t sBlk[kMasks ? kBwdMaxKeyBlocks : 1];
  // per-row key ranges: the key bounds of each wave's rows
  static_assert(!(kMasks && kRange), "the masked form takes key ranges at run time");
  static_assert(!kAlibi || (!kMasks && !kRange), "ALiBi: no other term or range");
  // key ranges: compiled in (kRange), or optional at run time (kMasks)
  constexpr bool kRng = kMasks || kRange;
  __shared__ KeyBounds sKb[kRng ? 4 : 1];
  // each row's clamped range, read back only by the wave that owns the row
  // (for the masked tiles; registers are scarce here)
  __shared__ int2 sRange[kRng ? kBwdQRows : 1];

  // heaviest query tiles first (most causal key tiles)
  int qt, h, b = 0, S_q, S_k;
  size_t q_row0, k_row0, tok0 = 0;
  if constexpr (kVarlen) {
    h = blockIdx.x % p.A;
    int seq;
    if (!varlen_tile(p.cu_seqlens, p.n_seq, p.max_tiles, blockIdx.x / p.A, qt, seq)) return;
    b = seq;  // packed masks: block flags [n_seq, heads, nb, nb]
    tok0 = p.cu_seqlens[seq];
    S_q = S_k = p.cu_seqlens[seq + 1] - (int)tok0;
    q_row0 = (size_t)h * p.T + tok0;
    k_row0 = (size_t)(h / p.G) * p.T + tok0;
  } else {
    int rank, bh;
    grid_order(blockIdx.x, n_qt, p.A * p.B, p.dq_units_per_xcd, p.dq_group, rank, bh);
    qt = n_qt - 1 - rank;
    h = bh % p.A;
    b = bh / p.A;
    S_q = p.S_q;
    S_k = p.S_k;
    q_row0 = (size_t)(b * p.A + h) * S_q;
    k_row0 = (size_t)(b * p.A_kv + h / p.G) * S_k;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, g = lane >> 5;
  const int off = S_k - S_q;
  const int wl = p.win_left, wr = p.win_right;
  const uint8_t* qkeep = p.q_keep ? p.q_keep + (kVarlen ? tok0 : (size_t)b * S_q) : nullptr;
  const int q0 = qt * kBwdQRows;
  const int qrow = q0 + wave * 32 + l32;
  const bool row_in = qrow < S_q;

  // resident Q and dO halves of this lane's query row (lanes l and l ^ 32
  // hold the two halves); D = rowsum(dO * O) in fp32
  bf16x8 qf[KSTEPS], dof[KSTEPS];
  float dsum = 0.f;
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t) {
    const size_t e = (q_row0 + qrow) * D + 16 * t + 8 * g;
    qf[t] = row_in ? *(const bf16x8*)((const uint16_t*)p.q + e) : bf16x8{};
    dof[t] = row_in ? *(const bf16x8*)((const uint16_t*)p.dout + e) : bf16x8{};
    const bf16x8 of = row_in ? *(const bf16x8*)((const uint16_t*)p.o + e) : bf16x8{};
#pragma unroll
    for (int i = 0; i < 8; ++i) dsum = fmaf((float)dof[t][i], (float)of[i], dsum);
  }
  const float drow = sum_with_other_half(dsum);
  // base-2 LSE, +inf when the row takes no part (every p of it is then 0)
  float lrow = INFINITY;
  if (row_in) {
    const float lse = p.lse[q_row0 + qrow];
    const bool keep = qkeep == nullptr || qkeep[qrow] != 0;
    if (keep && lse != -INFINITY) lrow = lse * kLog2e;
    if (g == 0) *(float2*)(p.row_stats + 2 * (q_row0 + qrow)) = make_float2(lrow, drow);
  }

  // per-row key ranges (the forward's mask): this lane's row keeps keys
  // [rng.x, rng.y] (clamped into [-1, S_k]); the bounds of the wave's and the
  // workgroup's rows narrow the tile range and pick the whole tiles
  [[maybe_unused]] KeyBounds kb_wave{0, S_k, 0, S_k}, kb_wg{0, S_k, 0, S_k};
  if constexpr (kRng) {
    int2 rng = make_int2(-1, S_k);
    if (kRange || p.key_range) {
      const int32_t* kr = p.key_range + 2 * (kVarlen ? tok0 : (size_t)b * S_q);
      rng = row_in ? load_key_range(kr, qrow, S_k) : make_int2(0, -1);
    }
    if (g == 0) sRange[wave * 32 + l32] = rng;
    if (kRange || p.key_range) {
      kb_wave = wave_key_bounds(row_in, rng.x, rng.y);
      kb_wg = workgroup_key_bounds<4>(kb_wave, sKb, wave, lane);
    }
  }

  // key tiles some row of the workgroup keeps: j_lo + [0, n_tiles)
  int kbeg = 0, kend = S_k;
  if (wr >= 0) kend = min(kend, q0 + kBwdQRows - 1 + off + wr + 1);
  if (wl >= 0) kbeg = max(q0 + off - wl, 0);
  if constexpr (kRng) {
    kbeg = max(kbeg, kb_wg.any_lo);
    kend = min(kend, kb_wg.any_hi);
  }
  const int j_lo = kbeg / kKeyTile;
  const int n_tiles = kend > kbeg ? (kend + kKeyTile - 1) / kKeyTile - j_lo : 0;
  // key ranges: tiles j_lo + [jw_lo, jw_hi) lie inside the range of every row
  // of this wave
  [[maybe_unused]] int jw_lo = 0, jw_hi = n_tiles;
  if constexpr (kRng) {
    jw_lo = (max(kb_wave.all_lo, 0) + kKeyTile - 1) / kKeyTile - j_lo;
    jw_hi = max(kb_wave.all_hi, 0) / kKeyTile - j_lo;
  }

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
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
  const float cs = p.scale_log2;
  [[maybe_unused]] float alibi_b = 0.f;  // ALiBi: this head's slope over the scale
  if constexpr (kAlibi) alibi_b = p.alibi_slopes[h] * p.inv_scale;
  const uint16_t* kbase = (const uint16_t*)p.k + k_row0 * D;
  const uint16_t* vbase = (const uint16_t*)p.v + k_row0 * D;
  const uint8_t* kkeep = p.k_keep ? p.k_keep + (kVarlen ? tok0 : (size_t)b * S_k) : nullptr;

  // Block mask: this row block's flags for the 128-key blocks of its range,
  // staged in LDS (the loop's first barrier orders them); a tile of a masked
  // block is skipped whole (its copy still runs: the pipeline stays fixed).
  // Additive term: this lane's row of M.
  [[maybe_unused]] const int kb0 = j_lo >> 1;
  [[maybe_unused]] const float* brow = nullptr;
  if constexpr (kMasks) {
    if (p.block_keep) {
      const int hm = p.block_heads == 1 ? 0 : h;
      const uint8_t* bk = p.block_keep + ((size_t)(b * p.block_heads + hm) * p.n_qb + qt) * p.n_kb;
      const int nkb = n_tiles > 0 ? ((j_lo + n_tiles - 1) >> 1) - kb0 + 1 : 0;
      for (int i = tid; i < nkb; i += kThreads) sBlk[i] = bk[kb0 + i];
    }
    if (p.bias) {
      // dense [B, heads, S_q, ld]; packed [heads, T, ld] (row t: token t of its sequence)
      const int hm = p.bias_heads == 1 ? 0 : h;
      brow = kVarlen ? p.bias + ((size_t)hm * p.T + tok0 + min(qrow, S_q - 1)) * p.bias_ld
                     : p.bias + ((size_t)(b * p.bias_heads + hm) * S_q + min(qrow, S_q - 1)) * p.bias_ld;
    }
  }
  auto tile_kept = [&](int j) -> bool {
    if constexpr (kMasks) {
      if (p.block_keep) return __builtin_amdgcn_readfirstlane((int)sBlk[((j_lo + j) >> 1) - kb0]) != 0;
    }
    return true;
  };

  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x16{};

  auto issue = [&](int j, int slot) {
    const uint32_t dst = lds_base + slot * SLOT_BYTES;
    copy_rows<D, kKeyTile>(kbase, S_k, (j_lo + j) * kKeyTile, dst);
    copy_rows<D, kKeyTile>(vbase, S_k, (j_lo + j) * kKeyTile, dst + TILE_BYTES);
  };
  // key k0 + lane is in range and kept.  The keep byte is an ordinary load,
  // so with a key mask each step also waits for the copies in flight.
  auto key_ok = [&](int j) -> bool {
    const int key = (j_lo + j) * kKeyTile + lane;
    return key < S_k && (kkeep == nullptr || kkeep[key] != 0);
  };

  // 32-key half kb of tile j in `lds`: S^T, dP^T, then P, dS and dQ^T += K^T . dS^T
  const int wave_row0 = q0 + wave * 32;
  auto tile_masked = [&](int j, bool ok) -> bool {
    if constexpr (kMasks) {
      if (p.bias) return true;
    }
    const int k0 = (j_lo + j) * kKeyTile;
    bool full = k0 + kKeyTile <= S_k && __ballot(ok) == ~0ull;
    if (wr >= 0) full = full && k0 + kKeyTile - 1 <= wave_row0 + off + wr;
    if (wl >= 0) full = full && k0 >= wave_row0 + 31 + off - wl;
    // (the key-range form takes the per-element step on every tile: with a
    // whole-tile test the compiler's allocation spills over a hundred registers)
    if constexpr (kRange) return true;
    if constexpr (kRng) full = full && j >= jw_lo && j < jw_hi;
    return !full;
  };
  auto half = [&](const char* lds, int j, bool ok, int kb, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int k0 = (j_lo + j) * kKeyTile;
    f32x16 s = f32x16{}, dp = f32x16{};
    if constexpr (kAlibi) {
      // the forward's ALiBi term as the accumulators' initial value: element
      // r is key k0 + 32 kb + 8 (r / 4) + 4 g + r % 4 of this lane's row
      const float x0 = (float)(k0 + 32 * kb + 4 * g - (qrow + off));
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = -fabsf(x0 + (float)(8 * (r >> 2) + (r & 3))) * alibi_b;
    }
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      const bf16x8 ka = *(const bf16x8*)(lds + kb * 32 * D * 2 + koff[t]);
      const bf16x8 va = *(const bf16x8*)(lds + TILE_BYTES + kb * 32 * D * 2 + koff[t]);
      s = mfma32(ka, qf[t], s);
      dp = mfma32(va, dof[t], dp);
    }
    // additive term of the 16 keys of this lane in the half: element r is key
    // k0 + 32 kb + 8 (r / 4) + 4 g + r % 4, four runs of 4 keys (keys at or
    // past S_k are not read; the predicate masks them)
    if constexpr (kMasks) {
      if (brow) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int kk = k0 + 32 * kb + 8 * q4 + 4 * g;
          const f32x4 mt = kk < S_k ? *(const f32x4*)(brow + kk) : f32x4{};
#pragma unroll
          for (int i = 0; i < 4; ++i) s[4 * q4 + i] = fmaf(mt[i], p.inv_scale, s[4 * q4 + i]);
        }
      }
    }
    const uint64_t kvalid = __ballot(ok) >> (4 * g);
    int lim = wr >= 0 ? qrow + off + wr - k0 - 4 * g : (1 << 30);
    int lo = wl >= 0 ? qrow + off - wl - k0 - 4 * g : -(1 << 30);
    if constexpr (kRng) {
      const int2 rng = sRange[wave * 32 + l32];
      lim = min(lim, rng.y - k0 - 4 * g);
      lo = max(lo, rng.x - k0 - 4 * g);
    }
    bf16x8 dsb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = fmaf(s[r], cs, -lrow);
      if constexpr (MASKED) {
        const int c = 32 * kb + 8 * (r >> 2) + (r & 3);
        x = (((kvalid >> c) & 1) && c <= lim && c >= lo) ? x : -INFINITY;
      }
      const float pr = exp2_fast(x);
      dsb[r >> 3][r & 7] = (__bf16)(pr * (dp[r] - drow));
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const char* base = lds + (32 * kb + 16 * hh) * D * 2;
        const bf16x8 kt = concat(lds_read_tr16(base + voff[mb][0]), lds_read_tr16(base + voff[mb][1]));
        acc[mb] = mfma32(kt, dsb[hh], acc[mb]);
      }
    }
  };
  auto step = [&](int j, auto slot_tag) {
    constexpr int SC = decltype(slot_tag)::value;
    lds_copy_wait_all();
    __syncthreads();  // tile j has landed; every wave is done with tile j - 1
    if (j + 1 < n_tiles) issue(j + 1, SC ^ 1);
    const char* lc = (const char*)smem + SC * SLOT_BYTES;
    if (!tile_kept(j)) return;
    const bool ok = key_ok(j);
    if (tile_masked(j, ok)) {
      half(lc, j, ok, 0, std::true_type{});
      half(lc, j, ok, 1, std::true_type{});
    } else {
      half(lc, j, ok, 0, std::false_type{});
      half(lc, j, ok, 1, std::false_type{});
    }
  };
  if (n_tiles > 0) issue(0, 0);
  int j = 0;
  for (; j + 2 <= n_tiles; j += 2) {
    step(j, Slot<0>{});
    step(j + 1, Slot<1>{});
  }
  if (j < n_tiles) step(j, Slot<0>{});

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
// Two forms.  KLDS = false: the K and V rows of a wave's keys stay in
// registers and the loop is software-pipelined over 4 LDS slots; at d = 128
// that takes about 380 registers, so one wave per SIMD (two at d = 64).
// KLDS = true (d = 128): the workgroup's 128 K rows live in LDS (32 KB, read as
// the B operand of S), V stays in registers and the Q/dO blocks are
// double-buffered, which fits 256 registers: two waves per SIMD, twice the
// resident workgroups.  The launch picks it when the grid has enough
// workgroups to fill those slots several times over.
// kRange: per-row key ranges, forms of their own (the ranges of a block are
// staged beside its statistics, every block takes the per-element step);
// the register form runs one wave per SIMD at both head dimensions (at
// d = 64 two spill), the K-in-LDS form two.
template <int D, bool KLDS, bool kRange>
constexpr int kDkdvWavesPerSimd = ((D == 64 && !kRange) || KLDS) ? 2 : 1;

template <int D, bool KLDS, bool kVarlen, bool kMasks, bool kRange = false, bool kAlibi = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kDkdvWavesPerSimd<D, KLDS, kRange>, kDkdvWavesPerSimd<D, KLDS, kRange>))) void bwd_dkdv_kernel(BwdParams p,
                                                                                                      int n_kt) {
  static_assert(!(KLDS && kMasks), "the K-in-LDS form takes no block mask or term");
  static_assert(!kAlibi || (!kMasks && !kRange), "ALiBi: no other term or range");
  constexpr int KSTEPS = D / 16;
  constexpr int MB = D / 32;
  constexpr int BLOCK_BYTES = kQBlock * D * 2;
  constexpr int STATS_BYTES = kQBlock * 8;                    // (L2, D) per row
  constexpr int RANGE_BYTES = kRange ? kQBlock * 8 : 0;       // per-row key ranges
  constexpr int SLOT_BYTES = 2 * BLOCK_BYTES + STATS_BYTES + RANGE_BYTES;  // [Q block | dO block | stats | ranges]
  constexpr int NSLOT = KLDS ? 2 : 4;
  constexpr int KTILE_BYTES = KLDS ? kBwdKRows * D * 2 : 0;  // [slots | K tile]
  // copy instructions per wave per block
  constexpr int COPIES = 2 * (kQBlock * D / 8 / kThreads) + 1 + (kRange ? 1 : 0);
  __shared__ __attribute__((aligned(16))) uint16_t smem[(NSLOT * SLOT_BYTES + KTILE_BYTES) / 2];
  // block mask: flag of each (query head of the group, 128-row block) for this key block
  __shared__ uint8_t sBlk[kMasks ? kBwdMaxRowBlocks : 1];
  // per-row key ranges: the first and last row (per wave) that keep a key of this workgroup
  __shared__ int sHull[kRange ? 8 : 1];

  // key tiles in order (the first ones see the most query rows when causal)
  int kt, hk, b = 0, S_q, S_k;
  size_t k_row0, tok0 = 0;
  if constexpr (kVarlen) {
    // packed: the sequences' key tiles counted from each sequence's end, so
    // that the tiles seeing the most query rows (the first) come first
    hk = blockIdx.x % p.A_kv;
    int from_end, seq;
    if (!varlen_tile(p.cu_seqlens, p.n_seq, p.max_tiles, blockIdx.x / p.A_kv, from_end, seq)) return;
    b = seq;  // packed masks: block flags [n_seq, heads, nb, nb]
    tok0 = p.cu_seqlens[seq];
    S_q = S_k = p.cu_seqlens[seq + 1] - (int)tok0;
    kt = (S_k + kBwdKRows - 1) / kBwdKRows - 1 - from_end;
    k_row0 = (size_t)hk * p.T + tok0;
  } else {
    int bk;
    grid_order(blockIdx.x, n_kt, p.A_kv * p.B, p.kv_units_per_xcd, p.kv_group, kt, bk);
    hk = bk % p.A_kv;
    b = bk / p.A_kv;
    S_q = p.S_q;
    S_k = p.S_k;
    k_row0 = (size_t)(b * p.A_kv + hk) * S_k;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, g = lane >> 5;
  const int off = S_k - S_q;
  const int wl = p.win_left, wr = p.win_right;
  const int key = kt * kBwdKRows + wave * 32 + l32;  // this lane's key
  bool key_live = key < S_k;
  if (key_live && p.k_keep) key_live = p.k_keep[(kVarlen ? tok0 : (size_t)b * S_k) + key] != 0;
  // first row of query head gh of the group (dense: of batch row b)
  auto q_head_row0 = [&](int gh) -> size_t {
    const int h = hk * p.G + gh;
    return kVarlen ? (size_t)h * p.T + tok0 : (size_t)(b * p.A + h) * S_q;
  };

  bf16x8 kres[KLDS ? 1 : KSTEPS], vres[KSTEPS];
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t) {
    if constexpr (!KLDS)
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
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
  const float cs = p.scale_log2;

  f32x16 acc_dk[MB], acc_dv[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc_dk[mb] = acc_dv[mb] = f32x16{};

  // query rows that can see a key of this workgroup: i + off >= first key;
  // blocks run over (query head of the group, 32-row block)
  // (row i keeps key j when i + off - wl <= j <= i + off + wr)
  const int k_first = kt * kBwdKRows, k_last = k_first + kBwdKRows - 1;
  int i_first = wr >= 0 ? max(k_first - off - wr, 0) : 0;
  int i_end = wl >= 0 ? min(k_last - off + wl + 1, S_q) : S_q;
  // Per-row key ranges (the forward's mask): only rows whose range reaches a
  // key of this workgroup take part; a scan of every row's range gives the
  // first and last of them (rows past the window's range stay out as well).
  if constexpr (kRange) {
    {
      const int32_t* kr = p.key_range + 2 * (kVarlen ? tok0 : (size_t)b * S_q);
      int lo_row = INT_MAX, hi_row = -1;
      // rows outside [i_first, i_end) are out already (window, causal
      // diagonal); four loads in flight per thread
      for (int i0 = i_first + tid; i0 < i_end; i0 += 4 * kThreads) {
        int2 r[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + u * kThreads;
          r[u] = i < i_end ? *(const int2*)(kr + 2 * (size_t)i) : make_int2(1, 0);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + u * kThreads;
          if (r[u].x <= r[u].y && r[u].x <= k_last && r[u].y >= k_first) {
            lo_row = min(lo_row, i);
            hi_row = max(hi_row, i);
          }
        }
      }
      lo_row = wave_min_i32(lo_row);
      hi_row = wave_max_i32(hi_row);
      if (lane == 0) {
        sHull[wave] = lo_row;
        sHull[4 + wave] = hi_row;
      }
      __syncthreads();
      lo_row = min(min(sHull[0], sHull[1]), min(sHull[2], sHull[3]));
      hi_row = max(max(sHull[4], sHull[5]), max(sHull[6], sHull[7]));
      i_first = max(i_first, lo_row);
      i_end = min(i_end, hi_row + 1);
    }
  }
  const int qb_first = i_first / kQBlock;
  const int qb_end = i_end > i_first ? (i_end + kQBlock - 1) / kQBlock : qb_first;
  const int nq = qb_end - qb_first;
  const int n_blocks = p.G * nq;

  // Block mask: the flags of this key block for every (query head of the
  // group, 128-row block) of the row range, staged in LDS (ordered by the
  // loop's first barrier); a 32-row block of a masked block is skipped whole
  // (its copy still runs).  Additive term: M[row][this lane's key].
  [[maybe_unused]] const int rb0 = qb_first / 4;
  [[maybe_unused]] const int nrb = nq > 0 ? (qb_end - 1) / 4 - rb0 + 1 : 0;
  if constexpr (kMasks) {
    if (p.block_keep) {
      for (int i = tid; i < p.G * nrb; i += kThreads) {
        const int gh = i / nrb, r = rb0 + i % nrb;
        const int hm = p.block_heads == 1 ? 0 : hk * p.G + gh;
        sBlk[i] = p.block_keep[((size_t)(b * p.block_heads + hm) * p.n_qb + r) * p.n_kb + kt];
      }
    }
  }
  auto block_kept = [&](int idx) -> bool {
    if constexpr (kMasks) {
      if (p.block_keep) {
        const int gh = idx / nq, qb = qb_first + idx % nq;
        return __builtin_amdgcn_readfirstlane((int)sBlk[gh * nrb + qb / 4 - rb0]) != 0;
      }
    }
    return true;
  };

  auto issue = [&](int idx, int slot) {
    const int gh = idx / nq, qb = qb_first + idx % nq;
    const size_t q_row0 = q_head_row0(gh);
    const int r0 = qb * kQBlock;
    const uint32_t dst = lds_base + slot * SLOT_BYTES;
    copy_rows<D, kQBlock>((const uint16_t*)p.q + q_row0 * D, S_q, r0, dst);
    copy_rows<D, kQBlock>((const uint16_t*)p.dout + q_row0 * D, S_q, r0, dst + BLOCK_BYTES);
    // (L2, D) of rows r0 + 8 wave .. + 7: four lanes of 16 bytes per wave
    const int rows = min(S_q - r0, kQBlock);
    const i32x4 rsrc = make_buffer_rsrc(p.row_stats + 2 * (q_row0 + r0), (uint32_t)(rows * 8));
    const uint32_t sdst = dst + 2 * BLOCK_BYTES + (uint32_t)__builtin_amdgcn_readfirstlane(wave) * 64u;
    if (lane < 4) lds_copy16_buf(rsrc, (uint32_t)(wave * 64 + lane * 16), sdst);
    if constexpr (kRange) {
      // the rows' key ranges
      const i32x4 rrng = make_buffer_rsrc(p.key_range + 2 * ((kVarlen ? tok0 : (size_t)b * S_q) + r0),
                                          (uint32_t)(rows * 8));
      if (lane < 4) lds_copy16_buf(rrng, (uint32_t)(wave * 64 + lane * 16), sdst + STATS_BYTES);
    }
  };

  // S and dP of the block in `lds` for this wave's 32 keys
  // (K tile in LDS: this wave's rows 32 wave + l32 have the swizzle of rows l32)
  const char* lds_k = (const char*)smem + NSLOT * SLOT_BYTES + wave * 32 * D * 2;
  auto scores = [&](const char* lds, int idx, f32x16& s, f32x16& dp) {
    s = f32x16{};
    dp = f32x16{};
    if constexpr (kAlibi) {
      // the forward's ALiBi term (the slope of the block's query head) as the
      // accumulators' initial value: element r is row r0 + 8 (r / 4) + 4 g +
      // r % 4 against this lane's key
      const int gh = idx / nq, r0 = (qb_first + idx % nq) * kQBlock;
      const float ab = p.alibi_slopes[hk * p.G + gh] * p.inv_scale;
      const float x0 = (float)(key - off - r0 - 4 * g);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = -fabsf(x0 - (float)(8 * (r >> 2) + (r & 3))) * ab;
    }
    (void)idx;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      const bf16x8 qa = *(const bf16x8*)(lds + koff[t]);
      const bf16x8 da = *(const bf16x8*)(lds + BLOCK_BYTES + koff[t]);
      if constexpr (KLDS) {
        s = mfma32(qa, *(const bf16x8*)(lds_k + koff[t]), s);
      } else {
        s = mfma32(qa, kres[t], s);
      }
      dp = mfma32(da, vres[t], dp);
    }
  };
  // P and dS of block idx, then dV^T += dO^T . P and dK^T += Q^T . dS.  A
  // dead row has L2 = +inf, so its p is 0 without a mask; MASKED adds the
  // per-element predicate (rows past S_q, which arrive zero-filled with L2 =
  // 0, dropped or absent keys, the window's edges).
  auto grad = [&](const char* lds, int idx, const f32x16& s_in, const f32x16& dp, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const float* st = (const float*)(lds + 2 * BLOCK_BYTES);
    const int r0 = (qb_first + idx % nq) * kQBlock;
    f32x16 s = s_in;
    if constexpr (kMasks) {
      if (p.bias) {
        // M[r0 + m][key], m = 8(r/4) + 4g + r%4: for a fixed m the 32 lanes of a
        // half-wave read 32 consecutive keys; rows past S_q and keys past S_k
        // are not read (the predicate masks them)
        const int gh = idx / nq, hm = p.bias_heads == 1 ? 0 : hk * p.G + gh;
        const float* bcol = (kVarlen ? p.bias + ((size_t)hm * p.T + tok0) * p.bias_ld
                                     : p.bias + (size_t)(b * p.bias_heads + hm) * S_q * p.bias_ld) +
                            min(key, S_k - 1);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = r0 + 8 * (r >> 2) + 4 * g + (r & 3);
          const float m = row < S_q ? bcol[(size_t)row * p.bias_ld] : 0.f;
          s[r] = fmaf(m, p.inv_scale, s[r]);
        }
      }
    }
    // element r holds query row r0 + m, m = 8(r/4) + 4g + r%4, of this lane's key
    const int m_lo = wr >= 0 ? key - off - wr - r0 - 4 * g : -(1 << 30);
    int m_hi = key_live ? S_q - r0 - 4 * g : -(1 << 30);
    if (wl >= 0) m_hi = min(m_hi, key - off + wl - r0 - 4 * g + 1);
    [[maybe_unused]] const int* rg = (const int*)(st + 2 * kQBlock);  // the rows' key ranges
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 a = *(const f32x4*)(st + 2 * (8 * r4 + 4 * g));
      const f32x4 c = *(const f32x4*)(st + 2 * (8 * r4 + 4 * g) + 4);
      const float lv[4] = {a[0], a[2], c[0], c[2]}, dv[4] = {a[1], a[3], c[1], c[3]};

#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * r4 + i;
        float x = fmaf(s[r], cs, -lv[i]);
        if constexpr (MASKED) {
          const int m = 8 * r4 + i;
          bool live = m >= m_lo && m < m_hi;
          if constexpr (kRange) {
            const int2 r = *(const int2*)(rg + 2 * m + 8 * g);
            live = live && key >= r.x && key <= r.y;
          }
          x = live ? x : -INFINITY;
        }
        const float pr = exp2_fast(x);
        pb[r >> 3][r & 7] = (__bf16)pr;
        dsb[r >> 3][r & 7] = (__bf16)(pr * (dp[r] - dv[i]));
      }
    }
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
  };
  // whether block idx needs the per-element predicate in this wave (uniform)
  const bool wave_keys_live = __ballot(key_live) == ~0ull;
  const int wave_key_first = kt * kBwdKRows + wave * 32, wave_key_last = wave_key_first + 31;
  auto block_masked = [&](int idx) -> bool {
    if constexpr (kRange) return true;
    if constexpr (kMasks) {
      if (p.bias) return true;
    }
    const int r0 = (qb_first + idx % nq) * kQBlock;
    bool full = wave_keys_live && r0 + kQBlock <= S_q;
    if (wr >= 0) full = full && wave_key_last <= r0 + off + wr;
    if (wl >= 0) full = full && wave_key_first >= r0 + kQBlock - 1 + off - wl;
    return !full;
  };

  // Software pipeline over blocks: step idx waits for block idx + 1, issues
  // the copy of block idx + 3 into the slot block idx - 1 used, and computes,
  // in one basic block so that the two interleave, S and dP of block idx + 1
  // and the gradient of block idx.  Slot of block idx: idx % 4; the two
  // register sets alternate.
  struct SD {
    f32x16 s, dp;
  };
  SD ra, rb;
  auto step = [&](int idx, auto slot_tag, SD& cur, SD& nxt) {
    constexpr int SC = decltype(slot_tag)::value;
    constexpr int SN = (SC + 1) % NSLOT, SI = (SC + 3) % NSLOT;
    if (idx + 2 < n_blocks)
      lds_copy_wait<COPIES>();  // block idx + 1 has landed; idx + 2 may still be in flight
    else
      lds_copy_wait_all();
    __syncthreads();  // and for every wave; every wave is done with block idx - 1
    if (idx + 3 < n_blocks) issue(idx + 3, SI);
    const char* lc = (const char*)smem + SC * SLOT_BYTES;
    // at the last block this reads a stale (in-bounds) slot; the result is unused
    const char* ln = (const char*)smem + SN * SLOT_BYTES;
    if constexpr (kMasks) {
      // a block the block mask drops contributes nothing: its scores are not
      // needed and its gradient is not formed
      const bool keep_cur = block_kept(idx), keep_nxt = idx + 1 < n_blocks && block_kept(idx + 1);
      if (keep_nxt) scores(ln, idx + 1, nxt.s, nxt.dp);
      if (keep_cur) grad(lc, idx, cur.s, cur.dp, std::true_type{});
      return;
    }
    if (block_masked(idx)) {
      interleave_hint();
      scores(ln, idx + 1, nxt.s, nxt.dp);
      grad(lc, idx, cur.s, cur.dp, std::true_type{});
    } else {
      interleave_hint();
      scores(ln, idx + 1, nxt.s, nxt.dp);
      grad(lc, idx, cur.s, cur.dp, std::false_type{});
    }
  };

  if constexpr (KLDS) {
    // Two slots: step idx waits for block idx (and, at the first step, the K
    // tile), issues the copy of block idx + 1 into the other slot and computes
    // block idx; the other workgroup's waves on the SIMD fill the gaps.
    auto step2 = [&](int idx, auto slot_tag) {
      constexpr int SC = decltype(slot_tag)::value;
      lds_copy_wait_all();
      __syncthreads();  // block idx has landed for every wave; all are done with block idx - 1
      if (idx + 1 < n_blocks) issue(idx + 1, SC ^ 1);
      const char* lc = (const char*)smem + SC * SLOT_BYTES;
      if (!block_kept(idx)) return;
      SD cur;
      if (block_masked(idx)) {
        interleave_hint();
        scores(lc, idx, cur.s, cur.dp);
        grad(lc, idx, cur.s, cur.dp, std::true_type{});
      } else {
        interleave_hint();
        scores(lc, idx, cur.s, cur.dp);
        grad(lc, idx, cur.s, cur.dp, std::false_type{});
      }
    };
    if (n_blocks > 0) {
      // the workgroup's K rows (rows past S_k arrive as zeros)
      copy_rows<D, kBwdKRows>((const uint16_t*)p.k + k_row0 * D, S_k, kt * kBwdKRows,
                              lds_base + NSLOT * SLOT_BYTES);
      issue(0, 0);
    }
    for (int idx = 0; idx < n_blocks; idx += 2) {
      step2(idx, Slot<0>{});
      if (idx + 1 < n_blocks) step2(idx + 1, Slot<1>{});
    }
  } else {
    if (n_blocks > 0) {
      issue(0, 0);
      if (n_blocks > 1) issue(1, 1);
      if (n_blocks > 2) issue(2, 2);
      if (n_blocks > 2)
        lds_copy_wait<2 * COPIES>();
      else if (n_blocks > 1)
        lds_copy_wait<COPIES>();
      else
        lds_copy_wait_all();
      __syncthreads();
      if (block_kept(0)) scores((const char*)smem, 0, ra.s, ra.dp);
    }
    int idx = 0;
    for (; idx + 4 <= n_blocks; idx += 4) {
      step(idx, Slot<0>{}, ra, rb);
      step(idx + 1, Slot<1>{}, rb, ra);
      step(idx + 2, Slot<2>{}, ra, rb);
      step(idx + 3, Slot<3>{}, rb, ra);
    }
    if (idx < n_blocks) step(idx, Slot<0>{}, ra, rb);
    if (idx + 1 < n_blocks) step(idx + 1, Slot<1>{}, rb, ra);
    if (idx + 2 < n_blocks) step(idx + 2, Slot<2>{}, ra, rb);
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

// Groups of 8 query heads for the dQ pass (as in the forward); groups of 2
// KV heads for the dK/dV pass, whose 16 key tiles per head already keep an
// XCD busy (measured: the order moves the time by a few percent at most).
constexpr int kDqGroupMax = 8;
constexpr int kKvGroupMax = 2;
// workgroups from which the dK/dV pass takes its two-wave form at d = 128
// (four per resident slot of that form: 256 CUs x 2)
constexpr int kKlDsMinWorkgroups = 2048;
// XCD blocking of `units` (see grid_order): a multiple of 8 units is split
// into 8 contiguous blocks taken in groups of up to `group_max`.
void plan_order(int units, int group_max, int& per, int& group) {
  per = group = 0;
  if (units % kXcdCount != 0) return;
  per = units / kXcdCount;
  int g = group_max;
  while (g > 1 && per % g != 0) g >>= 1;
  group = g;
}

template <int D, bool kVarlen, bool kMasks, bool kRange, bool kAlibi = false>
hipError_t launch_bwd_v(const BwdParams& p_in, hipStream_t stream) {
  BwdParams p = p_in;
  int n_qt, n_units_q, n_units_kv;
  if constexpr (kVarlen) {
    n_qt = p.total_tiles;  // 128-row tiles of all sequences (per head); the key tiles are the same
    n_units_q = p.A;
    n_units_kv = p.A_kv;
    p.dq_units_per_xcd = p.dq_group = p.kv_units_per_xcd = p.kv_group = 0;
  } else {
    n_qt = (p.S_q + kBwdQRows - 1) / kBwdQRows;
    n_units_q = p.A * p.B;
    n_units_kv = p.A_kv * p.B;
    plan_order(p.A * p.B, kDqGroupMax, p.dq_units_per_xcd, p.dq_group);
    plan_order(p.A_kv * p.B, kKvGroupMax, p.kv_units_per_xcd, p.kv_group);
  }
  const int n_kt = kVarlen ? p.total_tiles : (p.S_k + kBwdKRows - 1) / kBwdKRows;
  // the dQ pass writes the row statistics the dK/dV pass reads: same stream, in order
  if (n_qt > 0 && (kVarlen || p.S_q > 0)) {
    hipLaunchKernelGGL((bwd_dq_kernel<D, kVarlen, kMasks, kRange && !kMasks, kAlibi>), dim3(n_qt * n_units_q),
                       dim3(kThreads), 0, stream, p, n_qt);
  }
  if (n_kt > 0 && (kVarlen || p.S_k > 0)) {
    // with no query row every key gradient is zero; the kernel still writes them
    const int n_wg = n_kt * n_units_kv;
    // The K-in-LDS form doubles the resident workgroups but halves what one
    // of them gets of its SIMD.  Causal key tiles differ in length (the first
    // sees every query row), so with few workgroups per slot the longest one
    // sets the time and the one-wave form is faster (GQA B=1 S=8192: 512
    // workgroups); with several per slot the two-wave form wins (MHA B=4
    // S=2048: 2048 workgroups, +18%).  With a block mask or an additive term,
    // and for packed sequences, the one-wave form runs (its register budget
    // holds the term loads and the sequence bookkeeping).
    bool two_wave = false;
    if constexpr (D == 128 && !kMasks && !kVarlen) two_wave = n_wg >= kKlDsMinWorkgroups;
    if constexpr (D == 128 && !kMasks && !kVarlen) {
      if (two_wave) {
        hipLaunchKernelGGL((bwd_dkdv_kernel<128, true, kVarlen, false, kRange, kAlibi>), dim3(n_wg), dim3(kThreads),
                           0, stream, p, n_kt);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, false, kVarlen, kMasks, kRange, kAlibi>), dim3(n_wg), dim3(kThreads), 0,
                       stream, p, n_kt);
    (void)two_wave;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_d(const BwdParams& p, hipStream_t stream) {
  // (key ranges with a term, and ALiBi with any mask form but keep masks and
  // windows, are rejected before the launch)
  const bool masks = p.block_keep || p.bias, rng = p.key_range != nullptr;
  if (p.alibi_slopes) {
    if (p.cu_seqlens) return launch_bwd_v<D, true, false, false, true>(p, stream);
    return launch_bwd_v<D, false, false, false, true>(p, stream);
  }
  if (p.cu_seqlens) {
    if (masks && rng) return launch_bwd_v<D, true, true, true>(p, stream);
    if (masks) return launch_bwd_v<D, true, true, false>(p, stream);
    if (rng) return launch_bwd_v<D, true, false, true>(p, stream);
    return launch_bwd_v<D, true, false, false>(p, stream);
  }
  if (masks && rng) return launch_bwd_v<D, false, true, true>(p, stream);
  if (masks) return launch_bwd_v<D, false, true, false>(p, stream);
  if (rng) return launch_bwd_v<D, false, false, true>(p, stream);
  return launch_bwd_v<D, false, false, false>(p, stream);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream) {
  if (p.d == 128) return launch_bwd_d<128>(p, stream);
  if (p.d == 64) return launch_bwd_d<64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
