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
//
// Instantiations (template flags; page "Attention Kernel", sections "Paged 与
// ragged KV" and "可编程 mask"):
//   kVarlen  packed sequences described by cumulative lengths;
//   kPaged   packed query chunks over a paged KV cache (each 16-token part of a
//            key tile is one page, found through the block table);
//   kBlocks  the key tiles of a row block listed from a 128 x 128 block mask,
//            so masked blocks are never loaded;
//   kBias    a dense additive term M on every score (loaded a tile ahead as
//            the initial value of the score accumulators);
//   kRange   per-row key ranges (kept apart so that the other forms keep
//            their register allocation; not combined with kBias);
//   kAlibi   ALiBi, the per-head distance penalty computed in the kernel (no
//            block mask, term or key ranges beside it).
// Sliding windows, per-row key ranges, keep masks and the causal flag are
// runtime arguments of every instantiation.
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

// Key tiles one workgroup can list under a block mask (S_k up to 262144).
constexpr int kMaxListedTiles = 4096;

// Waves per SIMD: two at d = 128 (the kernel needs up to 256 VGPRs); three
// at d = 64, whose accumulators and operands fit the 168-VGPR budget that
// needs, with three workgroups' 32 KB of tiles in LDS (measured +9% on a
// causal S = 2048 batch, +16% on ragged varlen batches).  The paged,
// dense-additive-mask and key-range variants stay at two: at three they spill.
template <int D, bool kPaged, bool kBias, bool kRange, bool kAlibi>
constexpr int kWavesPerSimd = (D == 64 && !kPaged && !kBias && !kRange && !kAlibi) ? 3 : 2;

// kFp8: queries and keys are OCP E4M3 codes with one fp32 scale per 128
// tokens (FwdParams::q_scale / k_scale); S^T = K . Q^T runs on the FP8 matrix
// cores (v_mfma_scale_f32_32x32x64_f8f6f4 with unit block exponents) and is
// scaled by q_scale * k_scale in fp32; values stay bf16 (dense, d = 128).
// kCache8 (paged only): the cache holds OCP E4M3 codes with one fp32 scale
// per (page, KV head) (FwdParams::k_scale / v_scale, [num_pages, A_kv]).  The
// tile parts are loaded into registers, widened exactly to bf16 and written
// where the bf16 copy would land; a key's scale multiplies its scores, a
// value's scale its probabilities before the PV product (the normaliser sums
// the unscaled ones).
template <int D, bool kVarlen, bool kPaged = false, bool kBlocks = false, bool kBias = false, bool kFp8 = false,
          bool kCache8 = false, bool kRange = false, bool kAlibi = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<D, kPaged, kBias, kRange, kAlibi>, kWavesPerSimd<D, kPaged, kBias, kRange, kAlibi>))) void prefill_bf16_kernel(FwdParams p) {
  static_assert(!kFp8 || (D == 128 && !kVarlen && !kPaged && !kBlocks && !kBias), "fp8: dense, d = 128");
  static_assert(!kCache8 || kPaged, "E4M3 caches: paged prefill only");
  static_assert(!kRange || (!kBias && !kCache8), "key ranges: not with a dense additive term or an E4M3 cache");
  static_assert(!kAlibi || (!kBias && !kBlocks && !kRange && !kFp8 && !kCache8), "ALiBi: bf16 values, no other term");
  constexpr int NCH = D / 8;               // 16-byte chunks per row
  constexpr int KSTEPS = D / 16;           // k-steps of the QK^T MFMA
  constexpr int MB = D / 32;               // 32-row blocks of O^T
  constexpr int TILE_CH = kBc * NCH;       // chunks per K (or V) tile
  constexpr int LD_PER_T = TILE_CH / kThreads;  // 16-byte copies per thread per K (or V) tile
  static_assert(TILE_CH % kThreads == 0, "tile load split");
  // K rows in 2-byte units: an FP8 key row of D bytes is laid out, copied and
  // swizzled like a bf16 row of D / 2 elements
  constexpr int DK = kFp8 ? D / 2 : D;
  constexpr int NCHK = DK / 8;
  constexpr int LD_K = kBc * NCHK / kThreads;   // copies per thread per K tile
  constexpr int KTILE_BYTES = kBc * DK * 2;

  // [K buf 0 | K buf 1 | V buf 0 | V buf 1]; the epilogue reuses it for staging
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kBc * DK + 2 * kBc * D];
  __shared__ uint8_t sKeep[2][kBc];
  // block-sparse mode: the physical index of each listed key tile, and the
  // per-wave counts of the list-building scans
  __shared__ uint16_t sTiles[kBlocks ? kMaxListedTiles : 1];
  __shared__ int sCnt[kBlocks ? kWaves : 1];
  // fp8: the key scales of the 128-key blocks of this workgroup's key range
  __shared__ float sKs[kFp8 ? kFp8MaxKeys / 128 : 1];
  // E4M3 cache: the scales of the parts of each K and V buffer's tile
  __shared__ f32x4 sKsc[kCache8 ? 2 : 1];
  __shared__ f32x4 sVsc[kCache8 ? 2 : 1];
  // per-row key ranges: each row's clamped (first, last), read back only by
  // the wave that owns the row, and the key bounds of each wave's rows
  __shared__ int2 sRange[kRange ? kRows : 1];
  __shared__ KeyBounds sKb[kRange ? kWaves : 1];

  RowBlock rb;
  if constexpr (kPaged) {
    if (!setup_paged<kRows>(p, D * 2, rb, kCache8 ? D : 0)) return;
  } else if constexpr (kVarlen) {
    if (!setup_varlen<kRows>(p, D * 2, rb)) return;
  } else {
    rb = setup_dense<kRows>(p, D * 2, kFp8 ? D : 0);
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

  // ---- per-row key ranges (page "Attention Kernel", section "可编程 mask":
  // document boundaries and prefix-LM as per-row ranges): each row's range,
  // clamped into [-1, S_k] so that offsets stay in int32, is kept in LDS for
  // the predicate of the masked tiles (registers are scarce here), and the
  // bounds of the wave's and the workgroup's rows narrow the tile range
  const int wl = p.win_left, wr = p.win_right;
  KeyBounds kb_wave{0, S_k, 0, S_k}, kb_wg{0, S_k, 0, S_k};
  if constexpr (kRange) {
    const int2 r = qrow < S_q ? load_key_range(rb.key_range, qrow, S_k) : make_int2(0, -1);
    if (g == 0) sRange[wave * 32 + l32] = r;
    kb_wave = wave_key_bounds(qrow < S_q, r.x, r.y);
    kb_wg = workgroup_key_bounds<kWaves>(kb_wave, sKb, wave, lane);
  }

  // ---- key tiles this workgroup needs: [j_lo, j_hi), the keys some row of
  // it keeps under the window and the key ranges
  const int q_first = rb.q0, q_last = rb.q0 + kRows - 1;
  int kbeg = 0, kend = S_k;
  if (wr >= 0) kend = min(kend, q_last + off + wr + 1);
  if (wl >= 0) kbeg = max(q_first + off - wl, 0);
  if constexpr (kRange) {
    kbeg = max(kbeg, kb_wg.any_lo);
    kend = min(kend, kb_wg.any_hi);
  }
  const int j_lo = kbeg / kBc;
  const int n_range = kend > kbeg ? (kend + kBc - 1) / kBc - j_lo : 0;

  // ---- tile order.  The tiles [j_ul, j_uh) need no per-element predicate for
  // any row of the workgroup (inside S_k, inside every row's window, no key
  // mask); they run first, the masked tiles [j_lo, j_ul) and [j_uh, j_hi)
  // after them (the online softmax does not depend on the order).  Logical
  // tile t is physical tile phys(t).
  int j_ul = j_lo, j_uh = j_lo;
  if (rb.k_keep == nullptr && n_range > 0) {
    int ul = wl >= 0 ? (max(q_last + off - wl, 0) + kBc - 1) / kBc : 0;
    int uh = S_k / kBc;
    if (wr >= 0) uh = min(uh, max(q_first + off + wr + 1, 0) / kBc);
    if constexpr (kRange) {
      ul = max(ul, (max(kb_wg.all_lo, 0) + kBc - 1) / kBc);
      uh = min(uh, max(kb_wg.all_hi, 0) / kBc);
    }
    ul = max(ul, j_lo);
    uh = min(uh, j_lo + n_range);
    if (ul < uh) {
      j_ul = ul;
      j_uh = uh;
    }
  }
  int n_tiles = n_range, n_mid = j_uh - j_ul;
  const int n_left = j_ul - j_lo;
  if constexpr (kBlocks) {
    // Block sparsity (page "Attention Kernel", section "可编程 mask": the
    // block level decides which tiles are skipped whole).  List the tiles of
    // [j_lo, j_lo + n_range) whose 128-key block this row block keeps, the
    // predicate-free ones ([j_ul, j_uh)) first, each group in ascending order
    // (workgroup-wide prefix sums, so the order -- and the result -- is fixed).
    const uint8_t* brow = p.block_keep +
        (((size_t)rb.b * p.block_heads + (p.block_heads == 1 ? 0 : rb.h)) * p.n_qt + rb.qt) * p.n_kb;
    auto scan = [&](bool f, int& total) -> int {  // exclusive prefix of f over the workgroup
      const uint64_t m = __ballot(f);
      const int in_wave = __popcll(m & ((1ull << lane) - 1ull));
      if (lane == 0) sCnt[wave] = __popcll(m);
      __syncthreads();
      int before = 0;
      total = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        before += w < wave ? sCnt[w] : 0;
        total += sCnt[w];
      }
      __syncthreads();
      return before + in_wave;
    };
    auto classify = [&](int base, bool& keep, bool& free) {
      const int jj = j_lo + base + tid;
      keep = base + tid < n_range && brow[jj >> 1] != 0;
      free = keep && jj >= j_ul && jj < j_uh;
    };
    int n_free = 0;
    for (int base = 0; base < n_range; base += kThreads) {
      bool keep, free;
      classify(base, keep, free);
      int t;
      scan(free, t);
      n_free += t;
    }
    int at_free = 0, at_rest = n_free;
    for (int base = 0; base < n_range; base += kThreads) {
      bool keep, free;
      classify(base, keep, free);
      int tf, tr;
      const int pf = scan(free, tf), pr = scan(keep && !free, tr);
      if (free) sTiles[at_free + pf] = (uint16_t)(j_lo + base + tid);
      if (keep && !free) sTiles[at_rest + pr] = (uint16_t)(j_lo + base + tid);
      at_free += tf;
      at_rest += tr;
    }
    __syncthreads();
    n_tiles = __builtin_amdgcn_readfirstlane(at_rest);
    n_mid = __builtin_amdgcn_readfirstlane(n_free);
  }
  // (written with 0/1 factors: selects here became branches at the top of
  // every iteration.  Without a left edge n_left = 0 and phys(t) = j_ul + t.)
  auto phys = [=](int t) -> int {
    if constexpr (kBlocks) {
      return __builtin_amdgcn_readfirstlane((int)sTiles[t]);
    } else {
      const int u = t - n_mid;
      const int in_left = (unsigned)u < (unsigned)n_left;  // u in [0, n_left): left edge tiles
      const int past = u >= n_left;                         // right edge tiles
      const int base = j_ul + t - past * n_left;            // middle, then [j_uh, j_hi)
      return base + in_left * (j_lo + u - base);
    }
  };

  // ---- resident Q operand: lane holds Q[qrow][16t + 8g .. +7] for each t
  // (fp8: the 32 code bytes [64t + 32g, +32) of its row for each 64-wide t)
  [[maybe_unused]] bf16x8 qf[kFp8 ? 1 : KSTEPS];
  [[maybe_unused]] i32x8 qf8[kFp8 ? D / 64 : 1];
  if constexpr (kFp8) {
    const uint8_t* q8 = (const uint8_t*)rb.q;
#pragma unroll
    for (int t = 0; t < D / 64; ++t)
      qf8[t] = qrow < S_q ? *(const i32x8*)(q8 + (size_t)qrow * D + 64 * t + 32 * g) : i32x8{};
  } else {
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      if (qrow < S_q) {
        qf[t] = *(const bf16x8*)(gq + (size_t)qrow * D + 16 * t + 8 * g);
      } else {
        qf[t] = bf16x8{};
      }
    }
  }

  // ---- tile loader: buffer -> LDS copies (buffer_load_dwordx4 ... lds) that
  // do not pass through registers.  One copy round of the workgroup fills RPC
  // tile rows: lane L of wave w the 16 bytes of slot w*64 + L, i.e. row
  // i*RPC + rowc, physical chunk pcc; the source offset is chosen so that
  // those bytes hold the row's swizzled chunk.  Each tile gets its own buffer
  // resource covering exactly its rows that exist, so the rows of a ragged
  // last tile past S_k arrive as zeros (finite, and masked to weight 0)
  // without any per-lane address arithmetic in the loop.
  //
  // LDS holds [K buf 0 | K buf 1 | V buf 0 | V buf 1]; tile t's K sits in K
  // buffer t % 2 and its V in V buffer t % 2.  K runs one tile ahead of V:
  // iteration j multiplies Q by K of tile j+1 while it applies P of tile j to
  // V of tile j, and meanwhile copies K of tile j+2 and V of tile j+1 into the
  // buffers iteration j-1 finished with.
  constexpr int RPC = kThreads / NCH;  // rows per copy round (a multiple of 16)
  constexpr int TILE_BYTES = kBc * D * 2;
  constexpr int VB0 = 2 * KTILE_BYTES;  // LDS byte offset of V buffer 0
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
  const int rowc = (wave * 64 + lane) / NCH, pcc = (wave * 64 + lane) % NCH;
  const int cc = lds_chunk<D>(rowc, pcc);  // the swizzle is an involution; it depends on row % 16 only
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // wave index in a scalar register
  uint32_t coff[LD_PER_T];  // byte offset of this lane's copy of part i inside a tile
#pragma unroll
  for (int i = 0; i < LD_PER_T; ++i) coff[i] = (uint32_t)((i * RPC + rowc) * D * 2 + cc * 16);
  auto tile_rsrc = [&](const uint16_t* gsrc, int t) {
    const int k0 = phys(t) * kBc;
    const int rows = min(max(S_k - k0, 0), kBc);
    return make_buffer_rsrc(gsrc + (size_t)k0 * D, (uint32_t)(rows * D * 2));
  };
  // part i (of LD_PER_T) of one tile of K (or V) into LDS byte offset `dst`
  auto copy_part = [&](const i32x4& rsrc, uint32_t dst, int i) {
    lds_copy16_buf(rsrc, coff[i], lds_base + dst + (uint32_t)(i * RPC * D * 2) + (uint32_t)wave_u * 1024u);
  };
  // the same for K tiles in the DK geometry (fp8 keys; = the above for bf16)
  constexpr int RPCK = kThreads / NCHK;
  const int rowck = (wave * 64 + lane) / NCHK, pcck = (wave * 64 + lane) % NCHK;
  const int cck = lds_chunk<DK>(rowck, pcck);
  uint32_t coffk[LD_K];
#pragma unroll
  for (int i = 0; i < LD_K; ++i) coffk[i] = (uint32_t)((i * RPCK + rowck) * DK * 2 + cck * 16);
  auto tile_rsrc_k = [&](const uint16_t* gsrc, int t) {
    const int k0 = phys(t) * kBc;
    const int rows = min(max(S_k - k0, 0), kBc);
    return make_buffer_rsrc(gsrc + (size_t)k0 * DK, (uint32_t)(rows * DK * 2));
  };
  auto copy_part_k = [&](const i32x4& rsrc, uint32_t dst, int i) {
    lds_copy16_buf(rsrc, coffk[i], lds_base + dst + (uint32_t)(i * RPCK * DK * 2) + (uint32_t)wave_u * 1024u);
  };
  // Paged KV: part i of a tile is RPC consecutive tokens, which the page size
  // (a power of two, a multiple of RPC) keeps inside one page.  Its resource
  // starts at the part's first token row in that page (rows are A_kv * D
  // elements apart) and covers only tokens < S_k, so the block table is never
  // read past the sequence and absent rows arrive as zeros.
  [[maybe_unused]] const uint32_t kv_stride = (uint32_t)(kPaged ? p.A_kv * D * 2 : D * 2);
  [[maybe_unused]] const uint32_t poff = (uint32_t)rowc * kv_stride + (uint32_t)cc * 16;
  // Page ids.  The prologue reads them with scalar loads.  In the loop a
  // scalar load would be costly: scalar loads may return out of order, so
  // while one is in flight every wait for an LDS operand read becomes a wait
  // for all of them.  The loop therefore fetches the next iteration's pages
  // with one vector load (lane i: part i), which the wait for the tile
  // copies at the top of the next iteration covers, and reads them out of
  // the lanes there.
  [[maybe_unused]] auto page_of = [&](int t, int i) -> int {  // page of part i of tile t
    const int row0 = phys(t) * kBc + i * RPC;
    return load_uniform_i32(rb.bt, min(row0, S_k - 1) >> p.page_shift);
  };
  [[maybe_unused]] auto pages_vec = [&](int t) -> int {  // lane i < LD_PER_T: page of part i of tile t
    const int row0 = phys(t) * kBc + min(lane, LD_PER_T - 1) * RPC;
    return rb.bt[min(row0, S_k - 1) >> p.page_shift];
  };
  [[maybe_unused]] auto part_rsrc = [&](const char* gbase, int t, int i, int page) -> i32x4 {
    const int row0 = phys(t) * kBc + i * RPC;
    const int in_page = row0 & ((1 << p.page_shift) - 1);
    const int rows = min(max(S_k - row0, 0), RPC);
    return make_buffer_rsrc(gbase + ((size_t)page << p.page_shift | (size_t)in_page) * kv_stride,
                            (uint32_t)rows * kv_stride);
  };
  [[maybe_unused]] auto copy_part_paged = [&](const char* gbase, int t, uint32_t dst, int i, int page) {
    lds_copy16_buf(part_rsrc(gbase, t, i, page), poff,
                   lds_base + dst + (uint32_t)(i * RPC * D * 2) + (uint32_t)wave_u * 1024u);
  };
  // E4M3 cache: this lane's 8 code bytes of part i of tile t (the logical
  // chunk cc of its row, as the bf16 copy moves), zero past S_k; widened to
  // bf16 and stored at the slot that copy would fill
  [[maybe_unused]] const uint32_t kv_stride8 = (uint32_t)(p.A_kv * D);
  [[maybe_unused]] auto load_part8 = [&](const char* gbase8, int t, int i, int page) -> uint2 {
    const int row0 = phys(t) * kBc + i * RPC;
    const int in_page = row0 & ((1 << p.page_shift) - 1);
    const char* src = gbase8 + ((size_t)page << p.page_shift | (size_t)in_page) * kv_stride8 +
                      (size_t)rowc * kv_stride8 + (size_t)cc * 8;
    return row0 + rowc < S_k ? *(const uint2*)src : uint2{0u, 0u};
  };
  [[maybe_unused]] auto store_part8 = [&](uint2 w, uint32_t dst, int i) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const b2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.f, false);
    const b2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.f, true);
    const b2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.f, false);
    const b2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.f, true);
    *(bf16x8*)((char*)smem + dst + i * RPC * D * 2 + wave * 1024 + lane * 16) =
        bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  };
  // scale of (page, this KV head) from lane `i` (< LD_PER_T) of a page vector
  [[maybe_unused]] const int hk_c = rb.h / p.G;
  [[maybe_unused]] auto scale_of = [&](const float* tab, int page) -> float {
    return tab[(size_t)page * p.A_kv + hk_c];
  };
  // pages of the parts of the K tile the current iteration copies (the next
  // iteration copies V of that same tile), and, in lanes, of the next
  // iteration's K tile
  [[maybe_unused]] int pg_k[LD_PER_T] = {};
  [[maybe_unused]] int pg_n = 0;
  auto copy_keep = [&](int t) {
    if (rb.k_keep && tid < kBc && t < n_tiles) {
      const int key = phys(t) * kBc + tid;
      sKeep[t & 1][tid] = key < S_k ? rb.k_keep[key] : 0;
    }
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
  // FP8 keys and queries: tile t's scores scale by q_scale (this row block) *
  // k_scale (the 128-key block of tile t); the key scales of the workgroup's
  // range are staged in LDS (the prologue's barrier orders them)
  [[maybe_unused]] float cs_q = cs;
  [[maybe_unused]] const int kblk0 = j_lo >> 1;
  if constexpr (kFp8) {
    cs_q = cs * p.q_scale[(size_t)(rb.b * p.A + rb.h) * p.n_qt + rb.qt];
    const int n_kblk = (S_k + 127) / 128;
    const float* ks = p.k_scale + (size_t)(rb.b * p.A_kv + rb.h / p.G) * n_kblk;
    const int nkb = n_range > 0 ? ((j_lo + n_range - 1) >> 1) - kblk0 + 1 : 0;
    for (int i = tid; i < nkb; i += kThreads) sKs[i] = ks[kblk0 + i];
  }
  auto cs_of = [&](int t) -> float {
    if constexpr (kFp8) {
      const int bits = __builtin_amdgcn_readfirstlane(__float_as_int(sKs[(phys(t) >> 1) - kblk0]));
      return cs_q * __int_as_float(bits);
    } else {
      return cs;
    }
  };
  const int wave_q0 = rb.q0 + wave * 32;
  // keys [kbeg_w, kend_w) hold every key some row of this wave keeps; a
  // tile outside them is dead for the whole wave (only edge tiles can be:
  // the predicate-free ones lie inside every row's range)
  int kbeg_w = 0, kend_w = S_k;
  if (wr >= 0) kend_w = min(kend_w, wave_q0 + 31 + off + wr + 1);
  if (wl >= 0) kbeg_w = max(wave_q0 + off - wl, 0);
  if constexpr (kRange) {
    kbeg_w = max(kbeg_w, kb_wave.any_lo);
    kend_w = min(kend_w, kb_wave.any_hi);
  }
  kbeg_w = __builtin_amdgcn_readfirstlane(kbeg_w);
  kend_w = __builtin_amdgcn_readfirstlane(kend_w);
  auto wave_sees = [&](int t) -> bool {
    const int k0 = phys(t) * kBc;
    return k0 < kend_w && k0 + kBc > kbeg_w;
  };

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
  constexpr int PF = 3;  // operand reads run PF MFMA steps ahead of their use

  // S^T = K . Q^T for the K tile in LDS buffer KBUF: two 32-key blocks, the
  // k-steps interleaved across them.  `issue` is called at two points.
  // (with an additive term, s arrives holding M / scale of the tile's scores)
  auto qk = [&](auto kbuf_tag, f32x16 (&s)[2], auto&& issue) {
    constexpr int KB = decltype(kbuf_tag)::value * KTILE_BYTES;
    if constexpr (!kBias && !kAlibi) {  // (with a term, the accumulators start from it)
      s[0] = f32x16{};
      s[1] = f32x16{};
    }
    if constexpr (kFp8) {
      // FP8: steps p = (kb = p % 2, t = p / 2) over 64-wide k-steps; lane reads
      // row l32 of key block kb, the 32 bytes [64t + 32g, +32) = logical
      // chunks 4t + 2g and 4t + 2g + 1 of the D-byte row (DK-geometry swizzle)
      constexpr int NQ8 = 2 * (D / 64);
      i32x8 ka8[NQ8];
#pragma unroll
      for (int q = 0; q < NQ8; ++q) {
        const int kb = q % 2, t = q / 2;
        const char* row = lds + KB + kb * 32 * DK * 2 + l32 * DK * 2;
        const i32x4 lo = *(const i32x4*)(row + lds_chunk<DK>(l32, 4 * t + 2 * g) * 16);
        const i32x4 hi = *(const i32x4*)(row + lds_chunk<DK>(l32, 4 * t + 2 * g + 1) * 16);
        ka8[q] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      issue(0);
#pragma unroll
      for (int q = 0; q < NQ8; ++q) {
        s[q % 2] = mfma32_fp8(ka8[q], qf8[q / 2], s[q % 2]);
        if (q == NQ8 / 2) issue(1);
      }
      return;
    }
    constexpr int NQ = 2 * KSTEPS;
    bf16x8 ka[NQ];
    auto kread = [&](int p) {  // step p: kb = p % 2, t = p / 2
      ka[p] = *(const bf16x8*)(lds + KB + (p % 2) * 32 * D * 2 + koff[p / 2]);
    };
#pragma unroll
    for (int p = 0; p < PF; ++p) kread(p);
    issue(0);
#pragma unroll
    for (int p = 0; p < NQ; ++p) {
      if (p + PF < NQ) kread(p + PF);
      s[p % 2] = mfma32(ka[p], qf[p / 2], s[p % 2]);
      if (p == NQ / 2) issue(1);
    }
  };
  // E4M3 cache: multiply the scores of the tile in K buffer kbuf by their
  // keys' scales (element (kb, r) is key 32 kb + 8 (r / 4) + 4 g + r % 4 of the
  // tile, in part (32 kb + 8 (r / 4)) / RPC)
  auto part_of = [](int kb, int r) -> int { return (32 * kb + 8 * (r >> 2)) / RPC; };
  auto kscale = [&](f32x16 (&s)[2], int kbuf) {
    if constexpr (kCache8) {
      const f32x4 ksc = sKsc[kbuf];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] *= ksc[part_of(kb, r)];
      }
    }
  };
  // per-element predicate of tile t (keys past S_k, the window's edges -- the
  // causal diagonal is its right edge --, the row's key range, the key
  // keep-mask): dead scores become -inf
  // Dense additive mask: this lane's row of M, and the 32 terms of its keys
  // in tile t (element (kb, r) of the score tile is key k0 + 32kb + 8(r/4) +
  // 4g + r%4, so keys come in runs of 4: one 16-byte load per run).  Keys at
  // or past S_k are not read (their scores are masked below).  The term
  // enters the raw product as M / scale, so that the base-2 scaling by
  // scale * log2(e) applies to both: it is the initial value of the score
  // accumulators.  A tile's terms are loaded an iteration ahead, so that the
  // wait for the tile copies at the top of the iteration covers them.
  // The terms of this workgroup's rows come through one buffer resource that
  // starts at its first row and ends at key S_k of its last row: rows past
  // S_q read zeros, and keys past S_k (padding, or the next row's terms)
  // belong to masked tiles, whose predicate discards them.  A lane's offset
  // holds its row; the tile's first key goes in the scalar offset.
  [[maybe_unused]] __amdgpu_buffer_rsrc_t bias_rsrc;
  [[maybe_unused]] uint32_t bias_voff = 0;
  if constexpr (kBias) {
    const int hm = p.bias_heads == 1 ? 0 : rb.h;
    const int rows = min(kRows, S_q - rb.q0);
    // dense [B, heads, S_q, ld]; packed [heads, T, ld] (row t: token t of its sequence)
    const float* plane = kVarlen ? p.bias + ((size_t)hm * p.T + rb.t0 + rb.q0) * p.bias_ld
                                 : p.bias + ((size_t)(rb.b * p.bias_heads + hm) * S_q + rb.q0) * p.bias_ld;
    const uint32_t nbytes = ((uint32_t)(rows - 1) * p.bias_ld + S_k) * 4u;
    bias_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)plane, 0, (int)nbytes, 0x00020000);
    bias_voff = ((uint32_t)(qrow - rb.q0) * p.bias_ld + 4 * g) * 4u;
  }
  auto bias_load = [&](int t, f32x4 (&m)[2][4]) {
    if constexpr (kBias) {
      const int k0b = __builtin_amdgcn_readfirstlane(phys(t) * kBc * 4);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          // (the run's offset goes in the scalar operand: one offset register
          // serves all eight loads)
          m[kb][q4] = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(bias_rsrc, bias_voff, k0b + (32 * kb + 8 * q4) * 4, 0));
        }
      }
    }
  };
  // ALiBi (page "Attention Kernel", section "正确性契约": a per-head linear
  // penalty on the query-key distance, fused into the score): the term
  // -slope_h |p - j| (p = qrow + off, this lane's position) enters the raw
  // product divided by the scale, as the initial value of the accumulators;
  // key j - p is formed exactly in fp32 (one add per score), the magnitude,
  // sign and slope in one multiply
  [[maybe_unused]] float alibi_b = 0.f;
  if constexpr (kAlibi) alibi_b = p.alibi_slopes[rb.h] * p.inv_scale;
  auto term_init = [&](f32x16 (&s)[2], const f32x4 (&m)[2][4], int t) {
    if constexpr (kBias) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = m[kb][r >> 2][r & 3] * p.inv_scale;
      }
    }
    if constexpr (kAlibi) {
      const float x0 = (float)(phys(t) * kBc + 4 * g - (qrow + off));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = x0 + (float)(32 * kb + 8 * (r >> 2) + (r & 3));
          s[kb][r] = -fabsf(x) * alibi_b;
        }
      }
    }
    (void)t;
  };
  auto mask = [&](f32x16 (&s)[2], int t) {
    const int k0 = phys(t) * kBc;
    // bit k of kvalid: key k0 + k exists and is kept (same for every lane)
    bool valid = k0 + lane < S_k;
    if (rb.k_keep) valid = valid && sKeep[t & 1][lane] != 0;
    const uint64_t kvalid = __ballot(valid) >> (4 * g);
    // element (kb, r) holds key k0 + kl, kl = 32kb + 8(r/4) + 4g + r%4;
    // dead when kl > qrow + off + wr - k0 or kl < qrow + off - wl - k0, or
    // outside the row's key range
    [[maybe_unused]] int lim = wr >= 0 ? qrow + off + wr - k0 - 4 * g : (1 << 30);
    [[maybe_unused]] int lo = wl >= 0 ? qrow + off - wl - k0 - 4 * g : -(1 << 30);
    if constexpr (kRange) {
      const int2 r = sRange[wave * 32 + l32];
      lim = min(lim, r.y - k0 - 4 * g);
      lo = max(lo, r.x - k0 - 4 * g);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 32 * kb + 8 * (r >> 2) + (r & 3);  // kl - 4g
        const bool live = ((kvalid >> c) & 1) && c <= lim && c >= lo;
        s[kb][r] = live ? s[kb][r] : -INFINITY;
      }
    }
  };
  // row max of a tile in base-2 units (scale > 0), both lane halves: four
  // chains of three-input maxima
  auto rowmax = [&](const f32x16 (&s)[2], float csx) {
    float mx[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int kb = c >> 1, r0 = (c & 1) * 8;
      float m = fmaxf(s[kb][r0], fmaxf(s[kb][r0 + 1], s[kb][r0 + 2]));
      m = fmaxf(m, fmaxf(s[kb][r0 + 3], s[kb][r0 + 4]));
      m = fmaxf(m, fmaxf(s[kb][r0 + 5], s[kb][r0 + 6]));
      mx[c] = fmaxf(m, s[kb][r0 + 7]);
    }
    return max_with_other_half(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]))) * csx;
  };
  // move the reference only when some row of the wave needs it
  auto rescale = [&](float mxs) {
    if (__builtin_amdgcn_ballot_w64(mxs > m_ref + kLazy) != 0) {
      const float m_new = fmaxf(m_ref, mxs);
      const float alpha = (m_ref == -INFINITY) ? 0.f : exp2_fast(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc_o[mb] *= alpha;
    }
  };
  // P = 2^(S * scale * log2 e - m) and O^T += V^T . P^T for the V tile in
  // LDS buffer VBUF; the normaliser sums p in fp32, the product takes p
  // rounded to bf16.  PV steps (kb, h, mb) with mb innermost: MB independent
  // accumulator chains.  `issue` is called at two points.
  auto exps = [&](const f32x16 (&s)[2], bf16x8 (&pb)[2][2], float csx, int vbuf) -> float {
    const float neg = (m_ref == -INFINITY) ? 0.f : -m_ref;
    [[maybe_unused]] f32x4 vsc;
    if constexpr (kCache8) vsc = sVsc[vbuf];
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const float e0 = exp2_fast(fmaf(s[kb][r + 0], csx, neg));
        const float e1 = exp2_fast(fmaf(s[kb][r + 1], csx, neg));
        const float e2 = exp2_fast(fmaf(s[kb][r + 2], csx, neg));
        const float e3 = exp2_fast(fmaf(s[kb][r + 3], csx, neg));
        rs[0] += e0;
        rs[1] += e1;
        rs[2] += e2;
        rs[3] += e3;
        if constexpr (kCache8) {
          const float v = vsc[part_of(kb, r)];
          pb[kb][r >> 3][(r & 7) + 0] = (__bf16)(e0 * v);
          pb[kb][r >> 3][(r & 7) + 1] = (__bf16)(e1 * v);
          pb[kb][r >> 3][(r & 7) + 2] = (__bf16)(e2 * v);
          pb[kb][r >> 3][(r & 7) + 3] = (__bf16)(e3 * v);
        } else {
          pb[kb][r >> 3][(r & 7) + 0] = (__bf16)e0;
          pb[kb][r >> 3][(r & 7) + 1] = (__bf16)e1;
          pb[kb][r >> 3][(r & 7) + 2] = (__bf16)e2;
          pb[kb][r >> 3][(r & 7) + 3] = (__bf16)e3;
        }
      }
    }
    return (rs[0] + rs[1]) + (rs[2] + rs[3]);
  };
  auto softmax_pv = [&](auto vbuf_tag, const f32x16 (&s)[2], float csx, auto&& issue) {
    constexpr int VB = VB0 + decltype(vbuf_tag)::value * TILE_BYTES;
    bf16x8 pb[2][2];
    l_run += exps(s, pb, csx, decltype(vbuf_tag)::value);
    constexpr int NV = 4 * MB;
    bf16x8 va[NV];
    auto vread = [&](int q) {  // step q: mb = q % MB, (kb, h) = q / MB
      const int mb = q % MB, kh = q / MB, kb = kh >> 1, h = kh & 1;
      const char* base = lds + VB + (32 * kb + 16 * h) * D * 2;
      va[q] = concat(lds_read_tr16(base + voff[mb][0]), lds_read_tr16(base + voff[mb][1]));
    };
#pragma unroll
    for (int q = 0; q < PF; ++q) vread(q);
    issue(2);
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      if (q + PF < NV) vread(q + PF);
      const int mb = q % MB, kh = q / MB;
      acc_o[mb] = mfma32(va[q], pb[kh >> 1][kh & 1], acc_o[mb]);
      if (q == NV / 2) issue(3);
    }
  };


  // ---- prologue: K, V of tile 0 and K of tile 1 in flight; S of tile 0
  f32x16 s_cur[2];
  float mx_cur = -INFINITY;
  [[maybe_unused]] f32x4 m_nx[2][4];  // additive term: the terms of the next tile's scores
  float cs_cur = cs;  // the score scale of the tile in s_cur (fp8: per tile)
  if (n_tiles > 0) {
    if constexpr (kPaged && kCache8) {
      const int t1 = min(1, n_tiles - 1);
      pg_n = pages_vec(min(2, n_tiles - 1));
      uint2 k0r[LD_PER_T], v0r[LD_PER_T], k1r[LD_PER_T];
      f32x4 ks0, vs0, ks1;
#pragma unroll
      for (int i = 0; i < LD_PER_T; ++i) {
        const int p0 = page_of(0, i);
        pg_k[i] = page_of(t1, i);
        k0r[i] = load_part8(rb.k, 0, i, p0);
        v0r[i] = load_part8(rb.v, 0, i, p0);
        k1r[i] = load_part8(rb.k, t1, i, pg_k[i]);
        ks0[i] = scale_of(p.k_scale, p0);
        vs0[i] = scale_of(p.v_scale, p0);
        ks1[i] = scale_of(p.k_scale, pg_k[i]);
      }
#pragma unroll
      for (int i = 0; i < LD_PER_T; ++i) {
        store_part8(k0r[i], 0, i);
        store_part8(v0r[i], VB0, i);
        store_part8(k1r[i], KTILE_BYTES, i);
      }
      if (tid == 0) {
        sKsc[0] = ks0;
        sVsc[0] = vs0;
        sKsc[1] = ks1;
      }
    } else if constexpr (kPaged) {
      const int t1 = min(1, n_tiles - 1);
      pg_n = pages_vec(min(2, n_tiles - 1));
#pragma unroll
      for (int i = 0; i < LD_PER_T; ++i) {
        const int p0 = page_of(0, i);
        pg_k[i] = page_of(t1, i);
        copy_part_paged(rb.k, 0, 0, i, p0);
        copy_part_paged(rb.v, 0, VB0, i, p0);
        copy_part_paged(rb.k, t1, KTILE_BYTES, i, pg_k[i]);
      }
    } else {
      const i32x4 rk0 = tile_rsrc_k(gk, 0), rv0 = tile_rsrc(gv, 0);
      const i32x4 rk1 = tile_rsrc_k(gk, min(1, n_tiles - 1));
#pragma unroll
      for (int i = 0; i < LD_PER_T; ++i) {
        if (i < LD_K) copy_part_k(rk0, 0, i);
        copy_part(rv0, VB0, i);
        if (i < LD_K) copy_part_k(rk1, KTILE_BYTES, i);
      }
    }
    copy_keep(0);
    copy_keep(1);
    f32x4 m0[2][4];
    bias_load(0, m0);
    bias_load(min(1, n_tiles - 1), m_nx);
    lds_copy_wait_all();
    __syncthreads();
    term_init(s_cur, m0, 0);
    qk(std::integral_constant<int, 0>{}, s_cur, [](int) {});
    kscale(s_cur, 0);
    if (n_mid == 0) mask(s_cur, 0);
    cs_cur = cs_of(0);
    mx_cur = rowmax(s_cur, cs_cur);
  }

  // ---- iteration j (tile j in buffers BUF = j % 2): S of tile j+1, softmax
  // and PV of tile j.  Iterations whose next tile every row sees whole run
  // first, in pairs, through the predicate-free body; the rest (the causal
  // diagonal, a ragged tail, a key mask, the last tile, an odd leftover)
  // follow in a second loop.  Keeping the two bodies in separate loops lets
  // the accumulators stay in one register set.
  auto iteration = [&](auto buf_tag, auto masked_tag, int j) {
    constexpr int BUF = decltype(buf_tag)::value;
    constexpr bool MASKED = decltype(masked_tag)::value;
    // K of tile j+1 and V of tile j have landed for this thread's copies;
    // after the barrier, for everyone's -- and every wave is done with
    // iteration j-1, whose buffers (K of tile j, V of tile j-1) the copies
    // below overwrite
    lds_copy_wait_all();
    __syncthreads();
    // copies of K of tile j+2 (into K buffer BUF) and V of tile j+1 (into V
    // buffer BUF^1), issued in parts at four points of the iteration.  Past
    // the last tile they re-copy the last tile into an idle buffer (harmless,
    // and it keeps the body free of branches).
    const int tk = min(j + 2, n_tiles - 1), tv = min(j + 1, n_tiles - 1);
    [[maybe_unused]] i32x4 rk, rv;
    [[maybe_unused]] int pg_v[LD_PER_T];
    if constexpr (!kPaged) {
      rk = tile_rsrc_k(gk, tk);
      rv = tile_rsrc(gv, tv);
    } else {
      // V of tile tv is the K tile the previous iteration copied; the pages
      // of K tile tk were loaded during the previous iteration (the copy
      // wait above covered that load); start loading those of the next one
      // (the empty asm keeps the reads below the copy wait and the barrier)
      asm volatile("" : "+v"(pg_n));
#pragma unroll
      for (int i = 0; i < LD_PER_T; ++i) {
        pg_v[i] = pg_k[i];
        pg_k[i] = __builtin_amdgcn_readlane(pg_n, i);
      }
      pg_n = pages_vec(min(j + 3, n_tiles - 1));
    }
    if constexpr (MASKED) copy_keep(j + 2);
    // E4M3 cache: the parts of K tile tk and V tile tv, and their scales, are
    // loaded into registers now and widened into the LDS buffers at the end
    // of the iteration (the buffers iteration j-1 finished with)
    [[maybe_unused]] uint2 kr8[LD_PER_T], vr8[LD_PER_T];
    [[maybe_unused]] float ks8 = 0.f, vs8 = 0.f;
    if constexpr (kCache8) {
#pragma unroll
      for (int i = 0; i < LD_PER_T; ++i) {
        kr8[i] = load_part8(rb.k, tk, i, pg_k[i]);
        vr8[i] = load_part8(rb.v, tv, i, pg_v[i]);
      }
      // lane i < LD_PER_T: the scales of part i
      int pk = pg_k[0], pv = pg_v[0];
#pragma unroll
      for (int i = 1; i < LD_PER_T; ++i) {
        if (lane == i) {
          pk = pg_k[i];
          pv = pg_v[i];
        }
      }
      ks8 = scale_of(p.k_scale, pk);
      vs8 = scale_of(p.v_scale, pv);
    }
    auto issue = [&](int at) {
#pragma unroll
      for (int i = 0; i < LD_PER_T; ++i) {
        if constexpr (kCache8) {
          (void)at;
        } else if constexpr (kPaged) {
          if (i * 4 / LD_PER_T == at) {
            copy_part_paged(rb.k, tk, BUF * KTILE_BYTES, i, pg_k[i]);
            copy_part_paged(rb.v, tv, VB0 + (BUF ^ 1) * TILE_BYTES, i, pg_v[i]);
          }
        } else {
          if (i < LD_K && i * 4 / LD_K == at) copy_part_k(rk, BUF * KTILE_BYTES, i);
          if (i * 4 / LD_PER_T == at) copy_part(rv, VB0 + (BUF ^ 1) * TILE_BYTES, i);
        }
      }
    };
    rescale(mx_cur);
    f32x16 s_next[2];
    interleave_hint();
    if constexpr (!MASKED) {
      term_init(s_next, m_nx, j + 1);
      qk(std::integral_constant<int, BUF ^ 1>{}, s_next, issue);
      kscale(s_next, BUF ^ 1);
      bias_load(min(j + 2, n_tiles - 1), m_nx);  // in flight until the next iteration's copy wait
      softmax_pv(buf_tag, s_cur, cs_cur, issue);
      cs_cur = cs_of(j + 1);
      mx_cur = rowmax(s_next, cs_cur);
      s_cur[0] = s_next[0];
      s_cur[1] = s_next[1];
    } else {
      // a wave skips the work of a tile none of its rows can see (it still
      // takes part in the copies and barriers)
      const bool has_next = j + 1 < n_tiles && wave_sees(j + 1);
      if (has_next) {
        term_init(s_next, m_nx, j + 1);
        qk(std::integral_constant<int, BUF ^ 1>{}, s_next, issue);
        kscale(s_next, BUF ^ 1);
      } else {
        issue(0);
        issue(1);
      }
      bias_load(min(j + 2, n_tiles - 1), m_nx);  // in flight until the next iteration's copy wait
      if (wave_sees(j)) {
        softmax_pv(buf_tag, s_cur, cs_cur, issue);
      } else {
        issue(2);
        issue(3);
      }
      if (has_next) {
        mask(s_next, j + 1);
        cs_cur = cs_of(j + 1);
        mx_cur = rowmax(s_next, cs_cur);
        s_cur[0] = s_next[0];
        s_cur[1] = s_next[1];
      }
    }
    if constexpr (kCache8) {
#pragma unroll
      for (int i = 0; i < LD_PER_T; ++i) {
        store_part8(kr8[i], BUF * KTILE_BYTES, i);
        store_part8(vr8[i], VB0 + (BUF ^ 1) * TILE_BYTES, i);
      }
      if (tid < LD_PER_T) {
        ((float*)&sKsc[BUF])[tid] = ks8;
        ((float*)&sVsc[BUF ^ 1])[tid] = vs8;
      }
    }
  };
  constexpr std::integral_constant<int, 0> B0{};
  constexpr std::integral_constant<int, 1> B1{};
  constexpr std::integral_constant<bool, false> UNMASKED{};
  constexpr std::integral_constant<bool, true> MASKED_T{};
  // iteration j is predicate-free when tile j+1 < n_mid
  const int n_pair_end = max(n_mid - 1, 0) & ~1;
  int j = 0;
  for (; j < n_pair_end; j += 2) {
    iteration(B0, UNMASKED, j);
    iteration(B1, UNMASKED, j + 1);
  }
  for (; j < n_tiles; j += 2) {
    iteration(B0, MASKED_T, j);
    if (j + 1 < n_tiles) iteration(B1, MASKED_T, j + 1);
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
  static_assert(kWaves * 32 * PITCH <= 2 * kBc * DK + 2 * kBc * D, "epilogue staging fits");
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
  // Each wave reads back only the rows it staged, and the LDS executes one
  // wave's operations in order, so the reads see the writes without a
  // workgroup barrier; the fence only keeps the compiler from reordering.
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  // all reads first (they are in bounds for every row), then the stores of
  // the rows that exist, so the LDS round trips overlap
  constexpr int NST = (32 * NCH) / 64;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 val[NST];
#pragma unroll
  for (int i = 0; i < NST; ++i) {
    const int cid = lane + 64 * i;
    val[i] = *(const u32x4*)(stage + (cid / NCH) * PITCH + (cid % NCH) * 8);
  }
#pragma unroll
  for (int i = 0; i < NST; ++i) asm volatile("" : "+v"(val[i]));  // (keeps the reads out of the branches)
#pragma unroll
  for (int i = 0; i < NST; ++i) {
    const int cid = lane + 64 * i;
    const int qr = wave_q0 + cid / NCH;
    if (qr < S_q) *(u32x4*)(go + (size_t)qr * D + (cid % NCH) * 8) = val[i];
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
  if (p.alibi_slopes) {
    // (block masks, terms and key ranges with ALiBi are rejected before the launch)
    if (varlen) {
      hipLaunchKernelGGL((prefill_bf16_kernel<D, true, false, false, false, false, false, false, true>), dim3(grid),
                         dim3(kThreads), 0, stream, p);
    } else {
      hipLaunchKernelGGL((prefill_bf16_kernel<D, false, false, false, false, false, false, false, true>), dim3(grid),
                         dim3(kThreads), 0, stream, p);
    }
    return hipGetLastError();
  }
  if (p.key_range) {
    // (a dense additive term with key ranges is rejected before the launch)
    if (varlen && p.block_keep) {
      hipLaunchKernelGGL((prefill_bf16_kernel<D, true, false, true, false, false, false, true>), dim3(grid),
                         dim3(kThreads), 0, stream, p);
    } else if (varlen) {
      hipLaunchKernelGGL((prefill_bf16_kernel<D, true, false, false, false, false, false, true>), dim3(grid),
                         dim3(kThreads), 0, stream, p);
    } else if (p.block_keep) {
      hipLaunchKernelGGL((prefill_bf16_kernel<D, false, false, true, false, false, false, true>), dim3(grid),
                         dim3(kThreads), 0, stream, p);
    } else {
      hipLaunchKernelGGL((prefill_bf16_kernel<D, false, false, false, false, false, false, true>), dim3(grid),
                         dim3(kThreads), 0, stream, p);
    }
    return hipGetLastError();
  }
  if (!varlen && p.bias && p.block_keep) {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, false, false, true, true>), dim3(grid), dim3(kThreads), 0, stream, p);
  } else if (!varlen && p.bias) {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, false, false, false, true>), dim3(grid), dim3(kThreads), 0, stream, p);
  } else if (!varlen && p.block_keep) {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, false, false, true>), dim3(grid), dim3(kThreads), 0, stream, p);
  } else if (varlen && p.bias && p.block_keep) {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, true, false, true, true>), dim3(grid), dim3(kThreads), 0, stream, p);
  } else if (varlen && p.bias) {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, true, false, false, true>), dim3(grid), dim3(kThreads), 0, stream, p);
  } else if (varlen && p.block_keep) {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, true, false, true>), dim3(grid), dim3(kThreads), 0, stream, p);
  } else if (varlen) {
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

hipError_t launch_prefill_fp8(const FwdParams& p, hipStream_t stream) {
  const int grid = p.n_qt * p.A * p.B;
  if (grid <= 0) return hipSuccess;
  if (p.d != 128) return hipErrorInvalidValue;
  if (p.key_range) {
    hipLaunchKernelGGL((prefill_bf16_kernel<128, false, false, false, false, true, false, true>), dim3(grid),
                       dim3(kThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL((prefill_bf16_kernel<128, false, false, false, false, true>), dim3(grid), dim3(kThreads), 0,
                       stream, p);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_paged_d(const FwdParams& p, int grid, hipStream_t stream) {
  if (p.alibi_slopes) {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, true, true, false, false, false, false, false, true>), dim3(grid),
                       dim3(kThreads), 0, stream, p);
  } else if (p.key_range && p.block_keep) {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, true, true, true, false, false, false, true>), dim3(grid),
                       dim3(kThreads), 0, stream, p);
  } else if (p.key_range) {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, true, true, false, false, false, false, true>), dim3(grid),
                       dim3(kThreads), 0, stream, p);
  } else if (p.bias && p.block_keep) {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, true, true, true, true>), dim3(grid), dim3(kThreads), 0, stream, p);
  } else if (p.bias) {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, true, true, false, true>), dim3(grid), dim3(kThreads), 0, stream, p);
  } else if (p.block_keep) {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, true, true, true>), dim3(grid), dim3(kThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, true, true>), dim3(grid), dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_paged_bf16(const FwdParams& p, hipStream_t stream) {
  const int grid = p.total_tiles * p.A;
  if (grid <= 0) return hipSuccess;
  if (p.d == 128) return launch_paged_d<128>(p, grid, stream);
  if (p.d == 64) return launch_paged_d<64>(p, grid, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_paged_fp8(const FwdParams& p, hipStream_t stream) {
  const int grid = p.total_tiles * p.A;
  if (grid <= 0) return hipSuccess;
  if (p.d == 128) {
    hipLaunchKernelGGL((prefill_bf16_kernel<128, true, true, false, false, false, true>), dim3(grid), dim3(kThreads),
                       0, stream, p);
  } else if (p.d == 64) {
    hipLaunchKernelGGL((prefill_bf16_kernel<64, true, true, false, false, false, true>), dim3(grid), dim3(kThreads),
                       0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace attn

