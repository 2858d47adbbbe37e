// attn_rowblock.h -- which query rows (and which K/V) a prefill workgroup owns.
#pragma once
#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {

struct RowBlock {
  const char* q;   // row 0 of this (sequence, head); rows are d elements apart
  const char* k;   // key 0 of the KV head (paged: the head's offset in a cache row)
  const char* v;
  const int32_t* bt;  // paged: this sequence's block-table row
  char* o;
  float* lse;
  const uint8_t* q_keep;  // or null
  const uint8_t* k_keep;  // or null
  const int32_t* key_range;  // this sequence's row 0 of the per-row key ranges, or null
  int S_q, S_k;
  int q0;                 // first query row of this workgroup
  int b, h, qt;           // batch (packed: sequence), head and query tile of this workgroup
  int t0;                 // packed: the sequence's first token (dense: 0)
};

// Dense batch: query tile index descending (heaviest causal tiles first),
// then batch*head.
template <int kRows>
__device__ __forceinline__ RowBlock setup_dense(const FwdParams& p, int row_bytes, int qk_row_bytes = 0) {
  // qk_row_bytes: row size of q and k when it differs from that of v and o
  // (FP8 queries and keys beside bf16 values); 0 = row_bytes
  if (qk_row_bytes == 0) qk_row_bytes = row_bytes;
  const int lin = blockIdx.x;
  const int bh_n = p.A * p.B;
  int qt, bh;
  if (p.xcd_heads > 0) {
    // XCD-blocked order (see plan_dense_order)
    const int x = lin % kXcds, i = lin / kXcds;
    const int per_group = p.xcd_group * p.n_qt;
    const int grp = i / per_group, r = i % per_group;
    qt = p.n_qt - 1 - r / p.xcd_group;
    bh = x * p.xcd_heads + grp * p.xcd_group + r % p.xcd_group;
  } else {
    qt = p.n_qt - 1 - lin / bh_n;
    bh = lin % bh_n;
  }
  const int h = bh % p.A, b = bh / p.A;
  const int hk = h / p.G;
  RowBlock r;
  const size_t qoff = (size_t)(b * p.A + h) * p.S_q;
  const size_t koff = (size_t)(b * p.A_kv + hk) * p.S_k;
  r.q = (const char*)p.q + qoff * qk_row_bytes;
  r.o = (char*)p.o + qoff * row_bytes;
  r.lse = p.lse + qoff;
  r.k = (const char*)p.k + koff * qk_row_bytes;
  r.v = (const char*)p.v + koff * row_bytes;
  r.q_keep = p.q_keep ? p.q_keep + (size_t)b * p.S_q : nullptr;
  r.k_keep = p.k_keep ? p.k_keep + (size_t)b * p.S_k : nullptr;
  r.key_range = p.key_range ? p.key_range + 2 * (size_t)b * p.S_q : nullptr;
  r.S_q = p.S_q;
  r.S_k = p.S_k;
  r.q0 = qt * kRows;
  r.b = b;
  r.h = h;
  r.qt = qt;
  r.t0 = 0;
  return r;
}

// Wave-wide sum of an int.
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Packed varlen: workgroups ordered by query-tile index descending across all
// sequences (tile t of any sequence sees about t+1 key tiles when causal),
// then sequence, then head.  C(t) = A * sum_s max(0, n_s - t) counts the
// workgroups whose tile index is >= t; a binary search finds this workgroup's
// tile index, a ballot finds its sequence.  With xcd_heads > 0 the heads are
// dealt to the XCDs in contiguous blocks of xcd_heads (whole GQA groups), so
// the query heads that read one KV head run on one XCD, next to each other,
// and share its L2.
template <int kRows>
__device__ __forceinline__ bool setup_varlen(const FwdParams& p, int row_bytes, RowBlock& r, int* seq_out = nullptr,
                                             int* head_out = nullptr) {
  const int lin = blockIdx.x;
  const int lane = threadIdx.x & 63;
  auto ntiles = [&](int s) -> int {
    int len = p.cu_seqlens[s + 1] - p.cu_seqlens[s];
    return (len + kRows - 1) / kRows;
  };
  auto count_ge = [&](int t) -> int {  // workgroups (per head) with tile index >= t
    int c = 0;
    for (int s = lane; s < p.n_seq; s += 64) c += max(0, ntiles(s) - t);
    return wave_sum(c);
  };
  int per_head, h;  // rank among tiles (heaviest first), head
  if (p.xcd_heads > 0) {
    const int x = lin % kXcds, i = lin / kXcds;
    per_head = i / p.xcd_heads;
    h = x * p.xcd_heads + i % p.xcd_heads;
  } else {
    per_head = lin / p.A;
    h = lin % p.A;
  }
  // largest t with count_ge(t) > per_head
  int lo = 0, hi = p.n_qt;  // count_ge(lo) > per_head, count_ge(hi) == 0
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (count_ge(mid) > per_head) lo = mid; else hi = mid;
  }
  const int t = lo;
  int k = per_head - count_ge(t + 1);  // k-th sequence (in order) with n_s > t
  int seq = -1;
  for (int base = 0; base < p.n_seq && seq < 0; base += 64) {
    int s = base + lane;
    bool has = s < p.n_seq && ntiles(s) > t;
    uint64_t m = __ballot(has);
    int c = __popcll(m);
    if (k < c) {
      uint64_t below = m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane)));
      bool mine = has && __popcll(below) == k;
      uint64_t w = __ballot(mine);
      seq = base + __ffsll((long long)w) - 1;
    } else {
      k -= c;
    }
  }
  if (seq < 0) return false;
  // t and seq are wave-uniform by construction; say so, so that everything
  // derived from them lives in scalar registers
  const int t_u = __builtin_amdgcn_readfirstlane(t);
  seq = __builtin_amdgcn_readfirstlane(seq);
  const int start = p.cu_seqlens[seq];
  const int len = p.cu_seqlens[seq + 1] - start;
  const int hk = h / p.G;
  r.q = (const char*)p.q + ((size_t)h * p.T + start) * row_bytes;
  r.o = (char*)p.o + ((size_t)h * p.T + start) * row_bytes;
  r.lse = p.lse + (size_t)h * p.T + start;
  r.k = (const char*)p.k + ((size_t)hk * p.T + start) * row_bytes;
  r.v = (const char*)p.v + ((size_t)hk * p.T + start) * row_bytes;
  r.q_keep = p.q_keep ? p.q_keep + start : nullptr;
  r.k_keep = p.k_keep ? p.k_keep + start : nullptr;
  r.key_range = p.key_range ? p.key_range + 2 * (size_t)start : nullptr;
  r.S_q = len;
  r.S_k = len;
  r.q0 = t_u * kRows;
  r.b = seq;
  r.h = h;
  r.qt = t_u;
  r.t0 = start;
  if (seq_out) *seq_out = seq;
  if (head_out) *head_out = h;
  return true;
}

// Packed query chunks over a paged KV cache: the query side is the varlen
// one (cu_seqlens over the chunks); sequence s's keys are its seq_lens[s]
// cached tokens, the chunk being the last of them (bottom-right alignment).
template <int kRows>
__device__ __forceinline__ bool setup_paged(const FwdParams& p, int row_bytes, RowBlock& r, int kv_row_bytes = 0) {
  // kv_row_bytes: bytes of one KV head's row in the cache when they differ
  // from the queries' (an E4M3 cache beside bf16 queries); 0 = row_bytes
  if (kv_row_bytes == 0) kv_row_bytes = row_bytes;
  int seq = 0, h = 0;
  if (!setup_varlen<kRows>(p, row_bytes, r, &seq, &h)) return false;
  const int hk = h / p.G;
  r.k = (const char*)p.k + (size_t)hk * kv_row_bytes;
  r.v = (const char*)p.v + (size_t)hk * kv_row_bytes;
  r.bt = p.block_table + (size_t)seq * p.max_pages;
  r.S_k = p.seq_lens[seq];
  r.q_keep = nullptr;
  r.k_keep = nullptr;
  return true;
}

}  // namespace attn
