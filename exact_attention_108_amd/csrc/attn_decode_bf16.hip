// attn_decode_bf16.hip -- single-query decode over a paged KV cache, split
// along the KV length, merged by log-sum-exp (gfx950).
//
// Paged addressing (page "Attention Kernel", section "Paged 与 ragged KV"):
// token t of sequence b lives in physical page block_table[b][t / page_size]
// at offset t % page_size; a cache row is [page][offset][kv head][d].
//
// Split-KV (page "Attention 算子加速史", section 4.2; page "快速Transformer
// （续）", section "Stream-K"): the KV length is divided among workgroups and
// each emits a partial output normalised within its range plus the range's
// log-sum-exp; a second kernel merges the partials of a (sequence, head) with
// the two-state rule of page "Attention Kernel", section "Online softmax":
//     lse = log sum_s exp(lse_s),   O = sum_s exp(lse_s - lse) O_s.
// The ranges depend only on seq_lens (and the device's CU count), so the
// result is the same for any choice of physical pages.  The G = A / A_kv query
// heads that share a KV head (page "Attention Kernel", GQA paragraph) are
// processed together, so each KV byte is read once.
//
// Decode is bound by HBM bandwidth (each KV byte feeds ~4 flops, page
// "Attention Kernel", section "Prefill 与 decode 是两种 kernel").  The design
// goal is long, contiguous, row-sized reads with many in flight per CU; the
// matrix cores only keep the arithmetic off the critical path.
#include <mutex>

#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {

constexpr int kChunk = 16;       // tokens per inner step (one MFMA M block)
constexpr int kDecodeBufsOneWave = 3;  // LDS buffers per wave in 1-wave workgroups (bf16)
constexpr int kWavesPerGroup = 4;  // waves per workgroup, each with its own KV heads

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// LDS swizzle of the 16-byte chunks of a token row (row = token % 16): keeps
// both the K-operand reads (16 tokens, one chunk) and the transposing V reads
// (4 tokens x two adjacent chunks per 16 lanes) free of bank conflicts.
__device__ __forceinline__ int tok_swz(int tok) { return ((tok & 7) << 1) | ((tok >> 3) & 1); }

// Work split (Stream-K, page "快速Transformer（续）", section Stream-K): the
// sequences' 16-token chunks are concatenated into one list of n_chunks and
// workgroup i of n_wg takes chunks [i*n_chunks/n_wg, (i+1)*n_chunks/n_wg), so
// every workgroup streams the same amount of KV whatever the length mix.  A
// range may cover the tail of one sequence, whole sequences and the head of
// another; the workgroup emits one partial per (workgroup i, sequence b) it
// touches, in slot i + b (the touched pairs form a staircase in (i, b), so
// i + b is unique), and the merge kernel combines a sequence's partials.
//
// Wave w of the workgroup owns KV heads 4*HPW*blockIdx.y + HPW*w + [0, HPW).
// A 16-token chunk of the wave's heads is copied global -> LDS with
// global_load_lds (rows of HPW*d contiguous elements, so each load
// instruction reads whole rows; bf16 caches use two buffers per wave, the
// next chunk's copies in flight while this one is computed), then
//   S^T[token, n] = sum_hh K_hh . Q^T_hh     (16x16x32 MFMA; column n = query
//                                             head n of the wave; block
//                                             diagonal: columns of other KV
//                                             heads see a zero B operand)
//   O^T[d, n]    += sum_hh V_hh^T . P^T_hh   (16x16x16 MFMA, same masking)
//
// FP8 caches (kFp8): element e of the cache is one OCP E4M3 byte, and the
// value is byte(e) * scale[page, kv head] (page "Attention Kernel", section
// "Paged 与 ragged KV": cache dtype and scale metadata are part of the
// contract).  Each lane loads the 8 bytes of its slot, widens them exactly to
// bf16 (every E4M3 value is a bf16 value) and stores them where the bf16
// path's copy would have put them, so the MFMA code is shared.  The scales
// stay in fp32: a key's scale multiplies its scores, a value's scale its
// probabilities before the PV product (the normaliser sums the unscaled ones).
//
// Query heads per KV head (G) beyond the 16 columns of one MFMA: NCG column
// groups of 16 (G <= 16 NCG), each with its own operand, state and products;
// the K and V operands read from LDS serve every group (MQA: G up to 64).
// WPG waves per workgroup: 4, or 1 when the workgroup would have fewer KV
// heads than waves (A_kv < 4 HPW), so that no wave of a resident workgroup
// sits idle.
template <int D, int HPW, bool kFp8, int NCG, int WPG>
__global__ __launch_bounds__(64 * WPG) void decode_split_kernel(DecodeParams p) {
  constexpr int RC = HPW * D / 8;            // 16-byte chunks per token row
  constexpr int TOK_PER_LD = 64 / RC;        // tokens per load instruction
  constexpr int N_LD = kChunk / TOK_PER_LD;  // load instructions per chunk (K or V)
  constexpr int KSTEPS = D / 32;             // QK k-steps per head
  constexpr int MB = D / 16;                 // 16-row blocks of O^T
  // bf16: NBUF LDS buffers per wave, the copies of the next NBUF - 1 chunks
  // in flight while one is computed -- two in 4-wave workgroups (two of
  // them fit a CU), three in 1-wave workgroups (few KV heads: measured +22%
  // at A_kv = 2, +2% at A_kv = 1 over two; four cost more waves per CU than
  // the deeper prefetch gains); FP8: one, the next chunk's bytes wait in
  // registers
  constexpr int NBUF = kFp8 ? 1 : (WPG == 1 ? kDecodeBufsOneWave : 2);
  constexpr int BUF_BYTES = 2 * kChunk * RC * 16;  // bytes: K then V
  constexpr int WAVE_LDS = NBUF * BUF_BYTES;
  static_assert(64 % RC == 0 && kChunk % TOK_PER_LD == 0, "row split");
  __shared__ __attribute__((aligned(16))) char smem[WPG * WAVE_LDS];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
  const int G = p.G;
  const int kv0 = (blockIdx.y * WPG + wave) * HPW;  // first KV head of this wave
  if (kv0 >= p.A_kv) return;  // no barrier below: waves are independent
  const int nh = min(HPW, p.A_kv - kv0);  // KV heads of this wave
  char* const sK0 = smem + wave * WAVE_LDS;
  char* sK = sK0;
  char* sV = sK + kChunk * RC * 16;

  // ---- this workgroup's chunk range
  const long long NC = p.n_chunks;
  const int wg = blockIdx.x;
  const long long c_lo = (long long)wg * NC / p.n_wg;
  const long long c_hi = (long long)(wg + 1) * NC / p.n_wg;
  if (c_lo >= c_hi) return;

  // ---- sequence holding chunk c_lo: prefix sums of ceil(len / 16), 64 at a time
  int b = -1, len = 0;
  long long cex = 0;  // chunks of all sequences before b
  {
    long long base_chunks = 0;
    for (int base = 0; base < p.B; base += 64) {
      const int bb = base + lane;
      const int lb = bb < p.B ? p.seq_lens[bb] : 0;
      const int nc = decode_chunks(lb, p.win_left);
      const long long incl = base_chunks + wave_incl_scan(nc, lane);
      const long long total = __shfl(incl, 63);
      if (c_lo < total) {
        const uint64_t m = __ballot(incl > c_lo);
        const int src = __ffsll((long long)m) - 1;
        b = base + src;
        len = __shfl(lb, src);
        cex = __shfl(incl, src) - __shfl(nc, src);
        break;
      }
      base_chunks = total;
    }
  }
  if (b < 0) return;  // unreachable when n_chunks matches seq_lens

  const int ps = p.page_size;
  const uint16_t* kc = (const uint16_t*)p.k_cache;
  const uint16_t* vc = (const uint16_t*)p.v_cache;
  const size_t tok_stride = (size_t)p.A_kv * D;  // elements between tokens of a page
  // this lane's slot in a load instruction: token row (ld_tok), head, physical chunk
  const int ld_tok = lane / RC, ld_pc = lane % RC;
  const int ld_hh = min(ld_pc / (D / 8), nh - 1);
  const int ld_c = ld_pc % (D / 8);
  // column l16 of group cg is query head kv0 * G + 16 cg + l16
  int hh_col[NCG];  // which of the wave's KV heads the column belongs to
  bool col_live[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    hh_col[cg] = (16 * cg + l16) / G;
    col_live[cg] = 16 * cg + l16 < nh * G;
  }
  const float cs = p.scale_log2;
  const int tr_r = l16 >> 2, tr_q = l16 & 3;
  // ALiBi (page "Attention Kernel", section "正确性契约"): each column's slope
  // over the scale; key t of a sequence of len tokens is len - 1 - t before
  // the query, and its raw product gets -slope (len - 1 - t) / scale
  const bool alibi = p.alibi_slopes != nullptr;
  float ab[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg)
    ab[cg] = alibi && col_live[cg] ? p.alibi_slopes[kv0 * G + 16 * cg + l16] * p.inv_scale : 0.f;

  int k = (int)(c_lo - cex);     // chunk index within sequence b's list
  long long remaining = c_hi - c_lo;
  while (true) {
    // the list of sequence b starts at the chunk of its first visible key
    const int t_first = decode_first_key(len, p.win_left);
    const int ck0 = t_first / kChunk;
    const int nch = decode_chunks(len, p.win_left);
    const int k_end = (int)min((long long)nch, k + remaining);
    const int t_begin = (ck0 + k) * kChunk, t_end = min(len, (ck0 + k_end) * kChunk);

    // ---- Q^T operand: column n = query head kv0*G + n (n < nh*G), 8 d per lane
    const uint16_t* qb = (const uint16_t*)p.q + ((size_t)b * p.A + (size_t)kv0 * G) * D;
    bf16x8 qf[NCG][KSTEPS];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t) {
        qf[cg][t] = col_live[cg] ? *(const bf16x8*)(qb + (size_t)(16 * cg + l16) * D + 32 * t + 8 * grp)
                                 : bf16x8{};
      }
    }
    const int32_t* bt = p.block_table + (size_t)b * p.max_pages;
    const int last_page = (t_end - 1) / ps;
    int pbase = t_begin / ps;  // lane i holds block-table entry pbase + i
    int page_of_lane = pbase + lane <= last_page ? bt[pbase + lane] : 0;

    float m_run[NCG], l_run[NCG];
    f32x4 acc[NCG][MB];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      m_run[cg] = -INFINITY;
      l_run[cg] = 0.f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[cg][mb] = f32x4{};
    }

    // first token row of chunk c in the cache (for this wave's first KV head).
    // A 16-token chunk lies inside one page (page_size is a multiple of 16);
    // chunks are looked up in increasing order, each at most one page past
    // the previous, so the 64-entry block-table window only moves forward.
    auto chunk_row0 = [&](int c, int& page) -> size_t {
      int pidx = c / ps - pbase;
      if (pidx >= 64) {
        pbase += 64;
        pidx -= 64;
        page_of_lane = pbase + lane <= last_page ? bt[pbase + lane] : 0;
      }
      page = __builtin_amdgcn_readlane(page_of_lane, pidx);
      return ((size_t)page * ps + (c % ps)) * tok_stride + (size_t)kv0 * D;
    };
    // global offset of lane slot (ld_tok, ld_pc) of load instruction i: token
    // row i*TOK_PER_LD + ld_tok (rows past the end re-read the last valid row:
    // finite, weight 0), logical chunk ld_c ^ swz of head ld_hh
    auto slot_elem = [&](size_t row0, int n_valid, int i) -> size_t {
      const int tl = i * TOK_PER_LD + ld_tok;
      const int tr = min(tl, n_valid - 1);
      const int c = ld_c ^ (tok_swz(tl) & (D / 8 - 1));
      return row0 + (size_t)tr * tok_stride + (size_t)ld_hh * D + c * 8;
    };
    // FP8: the 8 E4M3 bytes of each lane slot of a chunk, and its scales, are
    // loaded one chunk ahead into registers (the loads of chunk c + 16 are in
    // flight while chunk c is computed)
    [[maybe_unused]] uint2 kr[N_LD], vr[N_LD];
    [[maybe_unused]] float ksc_n = 1.f, vsc_n = 1.f;
    [[maybe_unused]] auto fp8_load = [&](int c) {
      int page;
      const size_t row0 = chunk_row0(c, page);
      const int nv = min(kChunk, t_end - c);
      const uint8_t* kc8 = (const uint8_t*)p.k_cache;
      const uint8_t* vc8 = (const uint8_t*)p.v_cache;
#pragma unroll
      for (int i = 0; i < N_LD; ++i) {
        const size_t e = slot_elem(row0, nv, i);
        kr[i] = *(const uint2*)(kc8 + e);
        vr[i] = *(const uint2*)(vc8 + e);
      }
      const size_t srow = (size_t)page * p.A_kv + kv0 + min(hh_col[0], nh - 1);
      ksc_n = p.k_scale[srow];
      vsc_n = p.v_scale[srow];
    };
    // bf16 with two LDS buffers: chunk c's copies into buffer `buf`
    [[maybe_unused]] auto bf16_issue = [&](int c, int buf) {
      int page;
      const size_t row0 = chunk_row0(c, page);
      const int nv = min(kChunk, t_end - c);
      char* dK = sK0 + buf * BUF_BYTES;
      char* dV = dK + kChunk * RC * 16;
#pragma unroll
      for (int i = 0; i < N_LD; ++i) {
        const size_t e = slot_elem(row0, nv, i);
        __builtin_amdgcn_global_load_lds((const void*)(kc + e), (__attribute__((address_space(3))) void*)(dK + i * 1024),
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(vc + e), (__attribute__((address_space(3))) void*)(dV + i * 1024),
                                         16, 0, 0);
      }
    };
    if constexpr (kFp8) {
      if (t_begin < t_end) fp8_load(t_begin);
    } else {
#pragma unroll
      for (int i = 0; i < NBUF - 1; ++i)
        if (t_begin + i * kChunk < t_end) bf16_issue(t_begin + i * kChunk, i);
    }

    for (int c0 = t_begin; c0 < t_end; c0 += kChunk) {
      const int n_valid = min(kChunk, t_end - c0);
      [[maybe_unused]] float ksc = 1.f, vsc = 1.f;
      if constexpr (kFp8) {
        // widen to bf16 (exact) into the LDS slots the bf16 copy would fill
        auto widen = [](uint2 w) {
          typedef __bf16 b2 __attribute__((ext_vector_type(2)));
          const b2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.f, false);
          const b2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.f, true);
          const b2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.f, false);
          const b2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.f, true);
          return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
        };
#pragma unroll
        for (int i = 0; i < N_LD; ++i) {
          *(bf16x8*)(sK + i * 1024 + lane * 16) = widen(kr[i]);
          *(bf16x8*)(sV + i * 1024 + lane * 16) = widen(vr[i]);
        }
        ksc = ksc_n;
        vsc = vsc_n;
        if (c0 + kChunk < t_end) fp8_load(c0 + kChunk);
      } else {
        // the copies of chunk c0 + (NBUF - 1) 16 go into the buffer the
        // previous step computed before this chunk is waited for; vmcnt
        // counts in issue order, so leaving the copies of the chunks issued
        // after this one outstanding (2 N_LD per chunk) means this chunk's
        // have landed.  The wait is explicit (the compiler does not place
        // its own before every read of LDS written this way) and the empty
        // asm keeps the LDS reads below from moving above it.
        const int step = (c0 - t_begin) / kChunk;
        const int buf = step % NBUF;
        sK = sK0 + buf * BUF_BYTES;
        sV = sK + kChunk * RC * 16;
        const int c_new = c0 + (NBUF - 1) * kChunk;
        if (c_new < t_end) bf16_issue(c_new, (step + NBUF - 1) % NBUF);
        // chunks after this one already issued: min(NBUF - 1, those left)
        const int after = min(NBUF - 1, (t_end - c0 - 1) / kChunk);
        static_assert(2 * N_LD * (NBUF - 1) < 64, "vmcnt field");
        if (after >= 3) {
          lds_copy_wait<2 * N_LD * 3>();
        } else if (after == 2) {
          lds_copy_wait<2 * N_LD * 2>();
        } else if (after == 1) {
          lds_copy_wait<2 * N_LD>();
        } else {
          lds_copy_wait<0>();
        }
        asm volatile("" ::: "memory");
      }
      // ---- S^T = sum_hh K_hh . Q^T_hh (block diagonal over the wave's heads)
      f32x4 sc[NCG];
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) sc[cg] = f32x4{};
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
          const int c = 4 * t + grp;  // logical chunk of lane's 8 d
          const char* ka = sK + (l16 * RC + hh * (D / 8) + (c ^ (tok_swz(l16) & (D / 8 - 1)))) * 16;
          const bf16x8 a = *(const bf16x8*)ka;
#pragma unroll
          for (int cg = 0; cg < NCG; ++cg) {
            const bf16x8 bq = (col_live[cg] && hh_col[cg] == hh) ? qf[cg][t] : bf16x8{};
            sc[cg] = mfma16(a, bq, sc[cg]);
          }
        }
      }
      // lane holds tokens c0 + 4 grp + r of column l16 of each group
      bf16x4 pb[NCG];
      const float dist0 = (float)(len - 1 - c0 - 4 * grp);  // distance of token c0 + 4 grp to the query
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (kFp8) sc[cg][r] *= ksc;
          if (alibi) sc[cg][r] = fmaf((float)r - dist0, ab[cg], sc[cg][r]);
          if (4 * grp + r >= n_valid || c0 + 4 * grp + r < t_first) sc[cg][r] = -INFINITY;
          mx = fmaxf(mx, sc[cg][r]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = max_with_other_half(mx);
        const float m_new = fmaxf(m_run[cg], mx * cs);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2_fast(m_run[cg] - m_use);
        m_run[cg] = m_new;
        float rs = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = exp2_fast(fmaf(sc[cg][r], cs, -m_use));
          rs += e;
          if constexpr (kFp8)
            pb[cg][r] = (__bf16)(e * vsc);
          else
            pb[cg][r] = (__bf16)e;
        }
        l_run[cg] = fmaf(l_run[cg], alpha, rs);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[cg][mb] *= alpha;
      }
      // ---- O^T += sum_hh V_hh^T . P^T_hh ; V^T slot s of lane group grp = token 4 grp + s
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        const int row = 4 * grp + tr_r;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int c = 2 * mb + (tr_q >> 1);
          const char* va =
              sV + (row * RC + hh * (D / 8) + (c ^ (tok_swz(row) & (D / 8 - 1)))) * 16 + (tr_q & 1) * 8;
          const bf16x4 vt = __builtin_bit_cast(bf16x4, lds_read_tr16(va));
#pragma unroll
          for (int cg = 0; cg < NCG; ++cg) {
            const bf16x4 bp = (col_live[cg] && hh_col[cg] == hh) ? pb[cg] : bf16x4{};
            acc[cg][mb] = mfma16_k16(vt, bp, acc[cg][mb]);
          }
        }
      }
      // the next chunk's copies overwrite this chunk's LDS rows: all reads above
      // must have returned first
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      asm volatile("" ::: "memory");
    }

    // ---- partial of (workgroup, sequence b): normalised O and base-2 LSE per column
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      float l_tot = l_run[cg] + __shfl_xor(l_run[cg], 16);
      l_tot = sum_with_other_half(l_tot);
      const bool ok = l_tot > 0.f;
      const float inv = ok ? 1.f / l_tot : 0.f;
      if (col_live[cg]) {
        const int h = kv0 * G + 16 * cg + l16;
        const size_t slot = (size_t)(wg + b) * p.A + h;
        float* po = p.part_o + slot * D;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) *(f32x4*)(po + 16 * mb + 4 * grp) = acc[cg][mb] * inv;
        if (grp == 0) p.part_lse[slot] = ok ? m_run[cg] + log2_fast(l_tot) : -INFINITY;
      }
    }

    remaining -= k_end - k;
    if (remaining <= 0) break;
    do {  // next sequence with at least one chunk (exists while chunks remain)
      if (++b >= p.B) return;  // device lengths disagree with the host copy
      len = p.seq_lens[b];
    } while (len <= 0);
    k = 0;
  }
}

// One wavefront per (sequence, head): combine the sequence's partials.  The
// workgroups that touched sequence b are the owners of its first and last
// chunk and everything between; their partials sit in slots wg + b.  Lanes
// turn the partial LSEs into weights 2^(lse - max); the output loop then
// broadcasts one weight at a time (v_readlane) and keeps several independent
// partial-row loads in flight.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeParams p) {
  constexpr int PER = D / 64;  // output elements per lane (contiguous)
  typedef float fvec __attribute__((ext_vector_type(PER)));
  const int lane = threadIdx.x;
  const int bh = blockIdx.x;
  const int b = bh / p.A, h = bh % p.A;
  const int len = p.seq_lens[b];
  uint16_t* o = (uint16_t*)p.o + ((size_t)b * p.A + h) * D + lane * PER;
  fvec acc = {};
  float wsum = 0.f, mx = -INFINITY;
  if (len > 0) {
    // chunks before sequence b
    long long cex = 0;
    for (int base = 0; base < b; base += 64) {
      const int bb = base + lane;
      const int lb = bb < b ? p.seq_lens[bb] : 0;
      long long nc = decode_chunks(lb, p.win_left);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) nc += __shfl_xor(nc, off);
      cex += nc;
    }
    const long long nch = decode_chunks(len, p.win_left);
    const long long NC = p.n_chunks, P = p.n_wg;
    // owner of chunk c: the largest i with floor(i * NC / P) <= c
    const int first = (int)(((cex + 1) * P - 1) / NC);
    const int last = (int)(((cex + nch) * P - 1) / NC);
    const int np = last - first + 1;
    const size_t slot0 = (size_t)(first + b) * p.A + h;
    for (int j = lane; j < np; j += 64) mx = fmaxf(mx, p.part_lse[slot0 + (size_t)j * p.A]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if (mx != -INFINITY) {
      for (int j0 = 0; j0 < np; j0 += 64) {
        const int j = j0 + lane;
        const float ls = j < np ? p.part_lse[slot0 + (size_t)j * p.A] : -INFINITY;
        const float w = ls == -INFINITY ? 0.f : exp2_fast(ls - mx);
        wsum += w;
        const int cnt = min(64, np - j0);
        const float* po = p.part_o + (slot0 + (size_t)j0 * p.A) * D + lane * PER;
        const size_t step = (size_t)p.A * D;
        auto wl = [&](int jj) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), jj)); };
        int jj = 0;
        for (; jj + 4 <= cnt; jj += 4) {  // four independent row loads in flight
          const fvec r0 = *(const fvec*)(po + (jj + 0) * step);
          const fvec r1 = *(const fvec*)(po + (jj + 1) * step);
          const fvec r2 = *(const fvec*)(po + (jj + 2) * step);
          const fvec r3 = *(const fvec*)(po + (jj + 3) * step);
          acc += wl(jj) * r0;
          acc += wl(jj + 1) * r1;
          acc += wl(jj + 2) * r2;
          acc += wl(jj + 3) * r3;
        }
        for (; jj < cnt; ++jj) acc += wl(jj) * *(const fvec*)(po + jj * step);
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) wsum += __shfl_xor(wsum, off);
  const bool ok = wsum > 0.f;
  const float inv = ok ? 1.f / wsum : 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = __builtin_bit_cast(uint16_t, (__bf16)(acc[i] * inv));
  if (lane == 0) p.lse[(size_t)b * p.A + h] = ok ? (mx + log2_fast(wsum)) * kLn2 : -INFINITY;
}

template <int D, int HPW, bool kFp8, int NCG, int WPG>
int resident_groups(int cus) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_split_kernel<D, HPW, kFp8, NCG, WPG>, 64 * WPG,
                                                   0) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  // 1-wave workgroups: whole waves per SIMD (LDS allows 6 per CU at three
  // buffers, which would leave two SIMDs with two waves and two with one;
  // 4 per CU measured 1-2% faster at A_kv = 1, 2 and 13-31% on short batches)
  if (WPG == 1 && per_cu >= 4) per_cu = per_cu / 4 * 4;
  return cus * per_cu;
}

// Split kernel for this (head dim, heads per wave, column groups, waves per
// workgroup) choice: one resident wave of workgroups covers the chunk list
// once; then the merge.
template <int D, int HPW, bool kFp8, int NCG, int WPG>
hipError_t launch_split(DecodeParams p, int cus, hipStream_t stream) {
  const int heads_per_group = HPW * WPG;
  const int groups = (p.A_kv + heads_per_group - 1) / heads_per_group;
  long long want = resident_groups<D, HPW, kFp8, NCG, WPG>(cus) / groups;
  if (want < 1) want = 1;
  if (want > kMaxDecodeGroups) want = kMaxDecodeGroups;
  if (want > p.n_chunks) want = p.n_chunks;
  p.n_wg = (int)want;
  hipLaunchKernelGGL((decode_split_kernel<D, HPW, kFp8, NCG, WPG>), dim3(p.n_wg, groups), dim3(64 * WPG), 0, stream,
                     p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel<D>, dim3(p.B * p.A), dim3(64), 0, stream, p);
  return hipGetLastError();
}

template <int D, int HPW, bool kFp8, int NCG>
hipError_t launch_wpg(const DecodeParams& p, int cus, hipStream_t stream) {
  if (p.A_kv < kWavesPerGroup * HPW) return launch_split<D, HPW, kFp8, NCG, 1>(p, cus, stream);
  return launch_split<D, HPW, kFp8, NCG, kWavesPerGroup>(p, cus, stream);
}

template <int D, int HPW, bool kFp8>
hipError_t launch_ncg(const DecodeParams& p, int cus, hipStream_t stream) {
  const int cols = HPW * p.G;  // query-head columns of one wave
  if (cols <= 16) return launch_wpg<D, HPW, kFp8, 1>(p, cus, stream);
  if constexpr (HPW == 1) {
    if (cols <= 32) return launch_wpg<D, 1, kFp8, 2>(p, cus, stream);
    if (cols <= 64) return launch_wpg<D, 1, kFp8, 4>(p, cus, stream);
  }
  return hipErrorInvalidValue;
}

template <int D, bool kFp8>
hipError_t launch_decode_d(DecodeParams p, hipStream_t stream) {
  if (p.n_chunks <= 0) {
    // no token at all: the merge alone writes O = 0 and LSE = -inf
    p.n_wg = 1;
    hipLaunchKernelGGL(decode_merge_kernel<D>, dim3(p.B * p.A), dim3(64), 0, stream, p);
    return hipGetLastError();
  }
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                               hipSuccess || cus < 1)
    cus = 1;
  // FP8: two KV heads per wave when 2G <= 16 MFMA columns (longer rows per
  // load); bf16: one, so that two LDS buffers per wave still leave room for
  // two workgroups per CU (measured +1.7% over one buffer at two heads)
  if constexpr (kFp8) {
    if (p.G <= 8) return launch_ncg<D, 2, kFp8>(p, cus, stream);
  }
  return launch_ncg<D, 1, kFp8>(p, cus, stream);
}

// Static split workspace for callers that cannot allocate (attn_decode_paged_noalloc).
// Each device the library runs on holds its own copy of this array from the
// first call on that device until the process ends.  In host code the name
// `scratch` is only a stand-in for the symbol: the device address of each
// device's copy comes from hipGetSymbolAddress, taken once per device with
// that device current, and only that address is handed to kernels.
__device__ __align__(256) unsigned char scratch[kDecodeStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t decode_static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

DecodePlan plan_decode(int B, const int32_t* seq_lens_host, int win_left) {
  static_assert(kChunk == 16, "decode_chunks counts 16-token chunks");
  DecodePlan plan;
  long long nc = 0;
  for (int b = 0; b < B; ++b) nc += decode_chunks(seq_lens_host[b], win_left);
  plan.n_chunks = nc;
  plan.n_slots = kMaxDecodeGroups + B;  // slot wg + b < n_wg + B
  return plan;
}

size_t decode_workspace_bytes(int A, int d, const DecodePlan& plan) {
  if (plan.n_chunks == 0) return 0;
  const size_t slots = (size_t)plan.n_slots * (size_t)A;
  const size_t o_bytes = ((slots * (size_t)d * 4) + 255) / 256 * 256;
  const size_t l_bytes = ((slots * 4) + 255) / 256 * 256;
  return o_bytes + l_bytes;
}

size_t decode_workspace_lse_offset(int A, int d, const DecodePlan& plan) {
  const size_t slots = (size_t)plan.n_slots * (size_t)A;
  return ((slots * (size_t)d * 4) + 255) / 256 * 256;
}

hipError_t launch_decode_bf16(const DecodeParams& p, hipStream_t stream) {
  if (p.d == 128) return launch_decode_d<128, false>(p, stream);
  if (p.d == 64) return launch_decode_d<64, false>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_fp8(const DecodeParams& p, hipStream_t stream) {
  if (p.d == 128) return launch_decode_d<128, true>(p, stream);
  if (p.d == 64) return launch_decode_d<64, true>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
