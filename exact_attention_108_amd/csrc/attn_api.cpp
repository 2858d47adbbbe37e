// attn_api.cpp -- the extern "C" boundary of libattn_mi355x.so: argument
// validation, launch planning and kernel dispatch.  Semantics of every entry
// point are documented in include/attn.h.
#include "../../include/attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>

#include "attn_bwd.h"
#include "attn_kernels.h"
#include "attn_window.h"

#define ATTN_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kAbiVersion = ATTN_ABI_VERSION;

bool valid_scale(float s) { return std::isfinite(s) && s > 0.f; }

attn_status launch_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH; }

bool valid_window(const attn_window* w) { return w == nullptr || (w->left >= -1 && w->right >= -1); }

void window_edges(const attn_window* w, int causal, long long key_extent, long long row_extent, int& left,
                  int& right) {
  attn::window_edges(w != nullptr, w ? w->left : -1, w ? w->right : -1, causal, key_extent, row_extent, left, right);
}

bool window_arith_fits(const attn_window* w, long long rows, long long keys) {
  return attn::window_arith_fits(w != nullptr, rows, keys);
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// per-row key ranges are read as int32 pairs (8-byte loads), ALiBi slopes as floats
bool key_range_aligned(const attn_mask* m) {
  return m == nullptr || (aligned(m->key_range, 8) && aligned(m->alibi_slopes, 4));
}
// the bf16 kernels' ALiBi forms take keep masks and windows beside it, no
// other mask form
bool alibi_alone(const attn_mask* m) {
  return m == nullptr || m->alibi_slopes == nullptr || (!m->block_keep && !m->bias && !m->key_range);
}

// Longest sequence (rows or keys) any call takes: the kernels count positions
// in int32 and round up to a tile or chunk past a length.
constexpr int kMaxLen = INT_MAX - 1024;

// tensor alignment the kernels' vector loads and stores need: 16 bytes for
// bf16 rows (16-byte copies into LDS and stores), 4 for fp32 elements
uintptr_t data_align(attn_dtype dtype) { return dtype == ATTN_BF16 ? 16 : 4; }

attn::FwdParams base_params(const void* q, const void* k, const void* v, void* o, float* lse,
                            int A, int A_kv, int d_h, float scale, int causal, const attn_mask* mask,
                            const attn_window* window, long long key_extent, long long row_extent) {
  attn::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.q_keep = mask ? mask->q_keep : nullptr;
  p.k_keep = mask ? mask->k_keep : nullptr;
  p.key_range = mask ? mask->key_range : nullptr;
  p.alibi_slopes = mask ? mask->alibi_slopes : nullptr;
  p.A = A;
  p.A_kv = A_kv;
  p.G = A / A_kv;
  p.d = d_h;
  p.causal = causal ? 1 : 0;
  p.scale = scale;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);
  p.inv_scale = (float)(1.0 / (double)scale);
  window_edges(window, causal, key_extent, row_extent, p.win_left, p.win_right);
  return p;
}

// a dense additive mask the kernels can read: [B, heads, S_q, ld] fp32 with
// ld >= S_k a multiple of 4 and 16-byte rows (the kernels load 4 keys at once)
bool valid_bias(const float* bias, int heads, int A, int S_q, int S_k, int ld) {
  if (heads != 1 && heads != A) return false;
  if (ld < S_k || ld < 1 || ld % 4 != 0) return false;
  if (((uintptr_t)bias & 15u) != 0) return false;
  (void)S_q;
  return true;
}
// the bf16 kernels read a workgroup's 128 rows of terms through one buffer
// resource, whose byte range is 32 bits
bool bias_rows_fit(int ld) { return (long long)attn::kPrefillRows * ld * 4 < (1LL << 32); }

// dtype / head-dim combinations the kernels are built for
attn_status check_prefill_support(attn_dtype dtype, int d_h) {
  if (dtype == ATTN_BF16) return (d_h == 64 || d_h == 128) ? ATTN_OK : ATTN_ERR_UNSUPPORTED;
  if (dtype == ATTN_F32) return (d_h >= 1 && d_h <= 128) ? ATTN_OK : ATTN_ERR_UNSUPPORTED;
  return ATTN_ERR_INVAL;
}

}  // namespace

ATTN_EXPORT attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int B, int A, int A_kv, int S_q, int S_k, int d_h, float scale,
                                 int causal, const attn_mask* mask, const attn_window* window,
                                 attn_dtype dtype, void* stream) {
  if (B < 1 || A < 1 || A_kv < 1 || S_q < 0 || S_k < 0 || d_h < 1 || A % A_kv != 0) return ATTN_ERR_INVAL;
  if (!valid_scale(scale) || !valid_window(window)) return ATTN_ERR_INVAL;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVAL;
  if (S_q > 0 && (!q || !o || !lse)) return ATTN_ERR_INVAL;
  if (S_k > 0 && (!k || !v)) return ATTN_ERR_INVAL;
  for (const void* t : {q, k, v, (const void*)o})
    if (!aligned(t, data_align(dtype))) return ATTN_ERR_INVAL;
  if (!aligned(lse, 4) || !key_range_aligned(mask)) return ATTN_ERR_INVAL;
  attn_status sup = check_prefill_support(dtype, d_h);
  if (sup != ATTN_OK) return sup;
  if (!window_arith_fits(window, S_q, S_k)) return ATTN_ERR_UNSUPPORTED;
  const bool blocks = mask && mask->block_keep;
  if (blocks) {
    if (mask->block_heads != 1 && mask->block_heads != A) return ATTN_ERR_INVAL;
    if (dtype != ATTN_BF16 || S_k > 262144) return ATTN_ERR_UNSUPPORTED;
  }
  const bool bias = mask && mask->bias;
  if (bias && !valid_bias(mask->bias, mask->bias_heads, A, S_q, S_k, mask->bias_ld)) return ATTN_ERR_INVAL;
  if (bias && dtype == ATTN_BF16 && !bias_rows_fit(mask->bias_ld)) return ATTN_ERR_UNSUPPORTED;
  if (bias && mask->key_range && dtype == ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (dtype == ATTN_BF16 && !alibi_alone(mask)) return ATTN_ERR_UNSUPPORTED;
  // the kernels count rows and key positions in int32, up to a tile past a length
  if (S_q > kMaxLen || S_k > kMaxLen) return ATTN_ERR_UNSUPPORTED;
  if (S_q == 0) return ATTN_OK;
  const int rows = dtype == ATTN_BF16 ? attn::kPrefillRows : attn::kPrefillRowsF32;
  const long long n_qt = (S_q + rows - 1) / rows;
  if (n_qt * (long long)A * (long long)B > INT_MAX) return ATTN_ERR_UNSUPPORTED;
  // element offsets inside the kernels are size_t; per-(b,h) row counts are int
  if ((long long)B * A * (long long)S_q > INT_MAX || (long long)B * A_kv * (long long)S_k > INT_MAX)
    return ATTN_ERR_UNSUPPORTED;
  attn::FwdParams p = base_params(q, k, v, o, lse, A, A_kv, d_h, scale, causal, mask, window, S_k, S_q);
  p.B = B;
  p.S_q = S_q;
  p.S_k = S_k;
  p.n_qt = (int)n_qt;
  if (blocks) {
    p.block_keep = mask->block_keep;
    p.block_heads = mask->block_heads;
    p.n_kb = (S_k + 127) / 128;
  }
  if (bias) {
    p.bias = mask->bias;
    p.bias_heads = mask->bias_heads;
    p.bias_ld = mask->bias_ld;
    p.inv_scale = (float)(1.0 / (double)scale);
  }
  attn::plan_dense_order(p);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = dtype == ATTN_BF16 ? attn::launch_prefill_bf16(p, false, st) : attn::launch_prefill_f32(p, false, st);
  return launch_status(e);
}

ATTN_EXPORT attn_status attn_fwd_fp8(const uint8_t* q, const uint8_t* k, const void* v, void* o, float* lse,
                                     const float* q_scale, const float* k_scale, int B, int A, int A_kv, int S_q,
                                     int S_k, int d_h, float scale, int causal, const attn_mask* mask,
                                     const attn_window* window, void* stream) {
  if (B < 1 || A < 1 || A_kv < 1 || S_q < 0 || S_k < 0 || d_h < 1 || A % A_kv != 0) return ATTN_ERR_INVAL;
  if (!valid_scale(scale) || !valid_window(window)) return ATTN_ERR_INVAL;
  if (S_q > 0 && (!q || !o || !lse || !q_scale)) return ATTN_ERR_INVAL;
  if (S_k > 0 && (!k || !v || !k_scale)) return ATTN_ERR_INVAL;
  for (const void* t : {(const void*)q, (const void*)k, v, (const void*)o})
    if (!aligned(t, 16)) return ATTN_ERR_INVAL;
  for (const void* t : {(const void*)lse, (const void*)q_scale, (const void*)k_scale})
    if (!aligned(t, 4)) return ATTN_ERR_INVAL;
  if (!key_range_aligned(mask)) return ATTN_ERR_INVAL;
  if (d_h != 128) return ATTN_ERR_UNSUPPORTED;
  if (mask && (mask->block_keep || mask->bias || mask->alibi_slopes)) return ATTN_ERR_UNSUPPORTED;
  if (S_k > attn::kFp8MaxKeys) return ATTN_ERR_UNSUPPORTED;
  if (!window_arith_fits(window, S_q, S_k)) return ATTN_ERR_UNSUPPORTED;
  if (S_q > kMaxLen || S_k > kMaxLen) return ATTN_ERR_UNSUPPORTED;
  if (S_q == 0) return ATTN_OK;
  const long long n_qt = (S_q + attn::kPrefillRows - 1) / attn::kPrefillRows;
  if (n_qt * (long long)A * (long long)B > INT_MAX) return ATTN_ERR_UNSUPPORTED;
  if ((long long)B * A * (long long)S_q > INT_MAX || (long long)B * A_kv * (long long)S_k > INT_MAX)
    return ATTN_ERR_UNSUPPORTED;
  attn::FwdParams p = base_params(q, k, v, o, lse, A, A_kv, d_h, scale, causal, mask, window, S_k, S_q);
  p.B = B;
  p.S_q = S_q;
  p.S_k = S_k;
  p.n_qt = (int)n_qt;
  p.q_scale = q_scale;
  p.k_scale = k_scale;
  attn::plan_dense_order(p);
  return launch_status(attn::launch_prefill_fp8(p, (hipStream_t)stream));
}

ATTN_EXPORT attn_status attn_block_keep_from_bias(const float* bias, int B, int bias_heads, int S_q, int S_k,
                                                  int bias_ld, uint8_t* block_keep, void* stream) {
  if (B < 1 || S_q < 0 || S_k < 0 || bias_heads < 1) return ATTN_ERR_INVAL;
  if (!bias || !block_keep || !valid_bias(bias, bias_heads, bias_heads, S_q, S_k, bias_ld)) return ATTN_ERR_INVAL;
  if (S_q == 0 || S_k == 0) return ATTN_OK;  // the block mask is empty
  if (S_q > kMaxLen || S_k > kMaxLen) return ATTN_ERR_UNSUPPORTED;
  const long long n_qb = (S_q + 127) / 128, n_kb = (S_k + 127) / 128;
  if ((long long)B * bias_heads * n_qb > INT_MAX || n_kb > 65535) return ATTN_ERR_UNSUPPORTED;
  return launch_status(attn::launch_block_keep_from_bias(bias, B, bias_heads, S_q, S_k, bias_ld, block_keep,
                                                         (hipStream_t)stream));
}

ATTN_EXPORT attn_status attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                                        const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                        int n_seq, int total_tokens, int A, int A_kv, int d_h, float scale,
                                        int causal, const attn_mask* mask, const attn_window* window,
                                        attn_dtype dtype, void* stream) {
  if (n_seq < 0 || total_tokens < 0 || A < 1 || A_kv < 1 || d_h < 1 || A % A_kv != 0) return ATTN_ERR_INVAL;
  if (!valid_scale(scale) || !valid_window(window)) return ATTN_ERR_INVAL;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVAL;
  if (!cu_seqlens || !cu_seqlens_host) return ATTN_ERR_INVAL;
  if (cu_seqlens_host[0] != 0 || cu_seqlens_host[n_seq] != total_tokens) return ATTN_ERR_INVAL;
  for (int s = 0; s < n_seq; ++s)
    if (cu_seqlens_host[s + 1] < cu_seqlens_host[s]) return ATTN_ERR_INVAL;
  if (total_tokens > 0 && (!q || !k || !v || !o || !lse)) return ATTN_ERR_INVAL;
  for (const void* t : {q, k, v, (const void*)o})
    if (!aligned(t, data_align(dtype))) return ATTN_ERR_INVAL;
  if (!aligned(lse, 4) || !aligned(cu_seqlens, 4) || !key_range_aligned(mask)) return ATTN_ERR_INVAL;
  attn_status sup = check_prefill_support(dtype, d_h);
  if (sup != ATTN_OK) return sup;
  int max_len = 0;
  for (int s = 0; s < n_seq; ++s) max_len = std::max(max_len, cu_seqlens_host[s + 1] - cu_seqlens_host[s]);
  // block masks [n_seq, block_heads, nb, nb] (nb = ceil(max_len / 128)) and
  // terms [bias_heads, T, bias_ld] (row t: keys at positions of t's sequence)
  const bool blocks = mask && mask->block_keep;
  const bool bias = mask && mask->bias;
  if (blocks && mask->block_heads != 1 && mask->block_heads != A) return ATTN_ERR_INVAL;
  if (bias && !valid_bias(mask->bias, mask->bias_heads, A, max_len, max_len, mask->bias_ld)) return ATTN_ERR_INVAL;
  if ((blocks || bias) && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (blocks && max_len > 262144) return ATTN_ERR_UNSUPPORTED;
  if (bias && !bias_rows_fit(mask->bias_ld)) return ATTN_ERR_UNSUPPORTED;
  if (bias && mask->key_range) return ATTN_ERR_UNSUPPORTED;
  if (dtype == ATTN_BF16 && !alibi_alone(mask)) return ATTN_ERR_UNSUPPORTED;
  if (max_len > kMaxLen) return ATTN_ERR_UNSUPPORTED;
  if (total_tokens == 0) return ATTN_OK;
  if ((long long)A * total_tokens > INT_MAX) return ATTN_ERR_UNSUPPORTED;
  const int rows = dtype == ATTN_BF16 ? attn::kPrefillRows : attn::kPrefillRowsF32;
  long long total_tiles = 0;
  int max_tiles = 0;
  for (int s = 0; s < n_seq; ++s) {
    const int len = cu_seqlens_host[s + 1] - cu_seqlens_host[s];
    const int nt = (len + rows - 1) / rows;
    total_tiles += nt;
    if (nt > max_tiles) max_tiles = nt;
  }
  if (total_tiles * A > INT_MAX) return ATTN_ERR_UNSUPPORTED;
  if (!window_arith_fits(window, max_len, max_len)) return ATTN_ERR_UNSUPPORTED;
  attn::FwdParams p = base_params(q, k, v, o, lse, A, A_kv, d_h, scale, causal, mask, window, max_len, max_len);
  p.cu_seqlens = cu_seqlens;
  p.n_seq = n_seq;
  p.T = total_tokens;
  p.B = 1;
  p.n_qt = max_tiles;
  p.total_tiles = (int)total_tiles;
  if (blocks) {
    p.block_keep = mask->block_keep;
    p.block_heads = mask->block_heads;
    p.n_kb = max_tiles;  // bf16 row tiles are 128 rows: nb = max_tiles
  }
  if (bias) {
    p.bias = mask->bias;
    p.bias_heads = mask->bias_heads;
    p.bias_ld = mask->bias_ld;
    p.inv_scale = (float)(1.0 / (double)scale);
  }
  if (dtype == ATTN_BF16) attn::plan_varlen_order(p);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = dtype == ATTN_BF16 ? attn::launch_prefill_bf16(p, true, st) : attn::launch_prefill_f32(p, true, st);
  return launch_status(e);
}

namespace {

attn_status check_decode(int B, int A, int A_kv, int d_h, int page_size, const int32_t* seq_lens_host,
                         int max_pages, bool check_pages) {
  if (B < 1 || A < 1 || A_kv < 1 || d_h < 1 || A % A_kv != 0 || page_size < 1) return ATTN_ERR_INVAL;
  if (!seq_lens_host) return ATTN_ERR_INVAL;
  for (int b = 0; b < B; ++b) {
    if (seq_lens_host[b] < 0) return ATTN_ERR_INVAL;
    if (check_pages && (long long)seq_lens_host[b] > (long long)max_pages * page_size) return ATTN_ERR_INVAL;
    // the split kernels count positions in int32, up to a few chunks past a length
    if (seq_lens_host[b] > kMaxLen) return ATTN_ERR_UNSUPPORTED;
  }
  if (d_h != 64 && d_h != 128) return ATTN_ERR_UNSUPPORTED;
  if (page_size % 16 != 0) return ATTN_ERR_UNSUPPORTED;
  if (A / A_kv > 64) return ATTN_ERR_UNSUPPORTED;  // query-head column groups of the split kernel
  return ATTN_OK;
}

}  // namespace

ATTN_EXPORT size_t attn_decode_paged_workspace_bytes(int B, int A, int A_kv, int d_h, int page_size,
                                                     const int32_t* seq_lens_host) {
  if (check_decode(B, A, A_kv, d_h, page_size, seq_lens_host, 0, false) != ATTN_OK) return 0;
  const attn::DecodePlan plan = attn::plan_decode(B, seq_lens_host);
  return attn::decode_workspace_bytes(A, d_h, plan);
}

namespace {

// validation shared by attn_decode_paged and attn_decode_paged_noalloc; on
// ATTN_OK `need` holds the split workspace's size
attn_status check_decode_call(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                              const int32_t* seq_lens, const int32_t* seq_lens_host, int page_size, void* o,
                              float* lse, int B, int A, int A_kv, int d_h, int max_pages, int num_pages,
                              float scale, attn_dtype dtype, size_t& need) {
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVAL;
  if (max_pages < 0 || num_pages < 0) return ATTN_ERR_INVAL;
  attn_status st = check_decode(B, A, A_kv, d_h, page_size, seq_lens_host, max_pages, true);
  if (st != ATTN_OK) return st;
  if (!valid_scale(scale)) return ATTN_ERR_INVAL;
  if (!q || !o || !lse || !seq_lens) return ATTN_ERR_INVAL;
  long long total_tokens = 0;
  for (int b = 0; b < B; ++b) total_tokens += seq_lens_host[b];
  if (total_tokens > 0 && (!k_cache || !v_cache || !block_table || num_pages < 1)) return ATTN_ERR_INVAL;
  for (const void* t : {q, k_cache, v_cache, (const void*)o})
    if (!aligned(t, 16)) return ATTN_ERR_INVAL;
  if (!aligned(lse, 4) || !aligned(seq_lens, 4) || !aligned(block_table, 4)) return ATTN_ERR_INVAL;
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if ((long long)B * A > INT_MAX) return ATTN_ERR_UNSUPPORTED;
  need = attn::decode_workspace_bytes(A, d_h, attn::plan_decode(B, seq_lens_host));
  return ATTN_OK;
}

attn_status launch_decode_call(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* seq_lens_host, int page_size, void* o,
                               float* lse, int B, int A, int A_kv, int d_h, int max_pages, float scale,
                               int window_left, void* workspace, void* stream,
                               const float* alibi_slopes = nullptr) {
  const attn::DecodePlan plan = attn::plan_decode(B, seq_lens_host, window_left);
  attn::DecodeParams p{};
  p.win_left = window_left;
  p.alibi_slopes = alibi_slopes;
  p.inv_scale = (float)(1.0 / (double)scale);
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.o = o;
  p.lse = lse;
  p.part_o = (float*)workspace;
  p.part_lse = (float*)((char*)workspace + attn::decode_workspace_lse_offset(A, d_h, plan));
  p.B = B;
  p.A = A;
  p.A_kv = A_kv;
  p.G = A / A_kv;
  p.d = d_h;
  p.page_size = page_size;
  p.max_pages = max_pages;
  p.n_chunks = plan.n_chunks;
  p.scale = scale;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);
  return launch_status(attn::launch_decode_bf16(p, (hipStream_t)stream));
}

}  // namespace

ATTN_EXPORT attn_status attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                                          const int32_t* block_table, const int32_t* seq_lens,
                                          const int32_t* seq_lens_host, int page_size, void* o, float* lse,
                                          int B, int A, int A_kv, int d_h, int max_pages, int num_pages,
                                          float scale, attn_dtype dtype, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  size_t need = 0;
  attn_status st = check_decode_call(q, k_cache, v_cache, block_table, seq_lens, seq_lens_host, page_size, o, lse,
                                     B, A, A_kv, d_h, max_pages, num_pages, scale, dtype, need);
  if (st != ATTN_OK) return st;
  if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255) != 0))
    return ATTN_ERR_INVAL;
  return launch_decode_call(q, k_cache, v_cache, block_table, seq_lens, seq_lens_host, page_size, o, lse, B, A,
                            A_kv, d_h, max_pages, scale, -1, workspace, stream);
}

ATTN_EXPORT attn_status attn_decode_paged_window(const void* q, const void* k_cache, const void* v_cache,
                                                 const int32_t* block_table, const int32_t* seq_lens,
                                                 const int32_t* seq_lens_host, int page_size, void* o, float* lse,
                                                 int B, int A, int A_kv, int d_h, int max_pages, int num_pages,
                                                 float scale, int window_left, attn_dtype dtype, void* workspace,
                                                 size_t workspace_bytes, void* stream) {
  if (window_left < -1) return ATTN_ERR_INVAL;
  size_t need = 0;
  attn_status st = check_decode_call(q, k_cache, v_cache, block_table, seq_lens, seq_lens_host, page_size, o, lse,
                                     B, A, A_kv, d_h, max_pages, num_pages, scale, dtype, need);
  if (st != ATTN_OK) return st;
  if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255) != 0))
    return ATTN_ERR_INVAL;
  return launch_decode_call(q, k_cache, v_cache, block_table, seq_lens, seq_lens_host, page_size, o, lse, B, A,
                            A_kv, d_h, max_pages, scale, window_left, workspace, stream);
}

ATTN_EXPORT attn_status attn_decode_paged_alibi(const void* q, const void* k_cache, const void* v_cache,
                                                const int32_t* block_table, const int32_t* seq_lens,
                                                const int32_t* seq_lens_host, int page_size, void* o, float* lse,
                                                int B, int A, int A_kv, int d_h, int max_pages, int num_pages,
                                                float scale, int window_left, const float* alibi_slopes,
                                                attn_dtype dtype, void* workspace, size_t workspace_bytes,
                                                void* stream) {
  if (window_left < -1 || !alibi_slopes || !aligned(alibi_slopes, 4)) return ATTN_ERR_INVAL;
  size_t need = 0;
  attn_status st = check_decode_call(q, k_cache, v_cache, block_table, seq_lens, seq_lens_host, page_size, o, lse,
                                     B, A, A_kv, d_h, max_pages, num_pages, scale, dtype, need);
  if (st != ATTN_OK) return st;
  if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255) != 0))
    return ATTN_ERR_INVAL;
  return launch_decode_call(q, k_cache, v_cache, block_table, seq_lens, seq_lens_host, page_size, o, lse, B, A,
                            A_kv, d_h, max_pages, scale, window_left, workspace, stream, alibi_slopes);
}

ATTN_EXPORT attn_status attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                                  const int32_t* block_table, const int32_t* seq_lens,
                                                  const int32_t* seq_lens_host, int page_size, void* o, float* lse,
                                                  int B, int A, int A_kv, int d_h, int max_pages, int num_pages,
                                                  float scale, attn_dtype dtype, void* stream) {
  size_t need = 0;
  attn_status st = check_decode_call(q, k_cache, v_cache, block_table, seq_lens, seq_lens_host, page_size, o, lse,
                                     B, A, A_kv, d_h, max_pages, num_pages, scale, dtype, need);
  if (st != ATTN_OK) return st;
  if (need > attn::kDecodeStaticScratchBytes) return ATTN_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (need > 0 && attn::decode_static_scratch(&ws) != hipSuccess) return ATTN_ERR_LAUNCH;
  return launch_decode_call(q, k_cache, v_cache, block_table, seq_lens, seq_lens_host, page_size, o, lse, B, A,
                            A_kv, d_h, max_pages, scale, -1, ws, stream);
}

namespace {

// attn_prefill_paged and its E4M3-cache form: validation, planning, launch
attn_status prefill_paged_call(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                               const float* v_scale, bool fp8, const int32_t* block_table, const int32_t* seq_lens,
                               const int32_t* seq_lens_host, const int32_t* cu_seqlens_q,
                               const int32_t* cu_seqlens_q_host, int page_size, void* o, float* lse, int n_seq,
                               int total_q, int A, int A_kv, int d_h, int max_pages, int num_pages, float scale,
                               int causal, const attn_window* window, attn_dtype dtype, void* stream,
                               const attn_mask* mask = nullptr) {
  if (n_seq < 0 || total_q < 0 || A < 1 || A_kv < 1 || d_h < 1 || A % A_kv != 0) return ATTN_ERR_INVAL;
  if (page_size < 1 || max_pages < 0 || num_pages < 0) return ATTN_ERR_INVAL;
  if (!valid_scale(scale) || !valid_window(window)) return ATTN_ERR_INVAL;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVAL;
  if (!cu_seqlens_q || !cu_seqlens_q_host || !seq_lens || (n_seq > 0 && !seq_lens_host)) return ATTN_ERR_INVAL;
  if (cu_seqlens_q_host[0] != 0 || cu_seqlens_q_host[n_seq] != total_q) return ATTN_ERR_INVAL;
  long long total_kv = 0;
  for (int s = 0; s < n_seq; ++s) {
    const int q_len = cu_seqlens_q_host[s + 1] - cu_seqlens_q_host[s];
    if (q_len < 0 || seq_lens_host[s] < q_len) return ATTN_ERR_INVAL;
    if ((long long)seq_lens_host[s] > (long long)max_pages * page_size) return ATTN_ERR_INVAL;
    total_kv += seq_lens_host[s];
  }
  if (total_q > 0 && (!q || !o || !lse)) return ATTN_ERR_INVAL;
  if (total_kv > 0 && (!k_cache || !v_cache || !block_table || num_pages < 1)) return ATTN_ERR_INVAL;
  if (fp8 && total_kv > 0 && (!k_scale || !v_scale)) return ATTN_ERR_INVAL;
  for (const void* t : {q, (const void*)o})
    if (!aligned(t, 16)) return ATTN_ERR_INVAL;
  for (const void* t : {k_cache, v_cache})
    if (!aligned(t, fp8 ? 8 : 16)) return ATTN_ERR_INVAL;
  for (const void* t : {(const void*)lse, (const void*)seq_lens, (const void*)block_table, (const void*)cu_seqlens_q,
                        (const void*)k_scale, (const void*)v_scale})
    if (!aligned(t, 4)) return ATTN_ERR_INVAL;
  if (!key_range_aligned(mask)) return ATTN_ERR_INVAL;
  if (dtype != ATTN_BF16 || (d_h != 64 && d_h != 128)) return ATTN_ERR_UNSUPPORTED;
  // masks: block flags [n_seq, block_heads, nqb, nkb] over (chunk row, key
  // position) and terms [bias_heads, total_q, bias_ld] (row: chunk token;
  // columns: key positions of its sequence); no keep-masks here
  const bool blocks = mask && mask->block_keep;
  const bool bias = mask && mask->bias;
  int max_q = 0, max_kv_len = 0;
  for (int s = 0; s < n_seq; ++s) {
    max_q = std::max(max_q, cu_seqlens_q_host[s + 1] - cu_seqlens_q_host[s]);
    max_kv_len = std::max(max_kv_len, seq_lens_host[s]);
  }
  if (mask && (mask->q_keep || mask->k_keep)) return ATTN_ERR_UNSUPPORTED;
  if (blocks && mask->block_heads != 1 && mask->block_heads != A) return ATTN_ERR_INVAL;
  if (bias && !valid_bias(mask->bias, mask->bias_heads, A, max_q, max_kv_len, mask->bias_ld)) return ATTN_ERR_INVAL;
  if ((blocks || bias) && fp8) return ATTN_ERR_UNSUPPORTED;
  if (max_q > kMaxLen || max_kv_len > kMaxLen) return ATTN_ERR_UNSUPPORTED;
  if (blocks && max_kv_len > 262144) return ATTN_ERR_UNSUPPORTED;
  if (bias && !bias_rows_fit(mask->bias_ld)) return ATTN_ERR_UNSUPPORTED;
  if (bias && mask->key_range) return ATTN_ERR_UNSUPPORTED;
  if (!alibi_alone(mask)) return ATTN_ERR_UNSUPPORTED;
  if (fp8 && mask && mask->alibi_slopes) return ATTN_ERR_UNSUPPORTED;
  const int rows_per_part = 2048 / d_h;  // tokens one copy round of a workgroup moves
  if ((page_size & (page_size - 1)) != 0 || page_size % rows_per_part != 0) return ATTN_ERR_UNSUPPORTED;
  if (total_q == 0) return ATTN_OK;
  if ((long long)A * total_q > INT_MAX) return ATTN_ERR_UNSUPPORTED;
  // the cache's byte offsets must fit the kernels' 32-bit buffer ranges per page row
  if ((long long)page_size * A_kv * d_h * 2 > INT_MAX) return ATTN_ERR_UNSUPPORTED;
  long long total_tiles = 0;
  int max_tiles = 0;
  for (int s = 0; s < n_seq; ++s) {
    const int len = cu_seqlens_q_host[s + 1] - cu_seqlens_q_host[s];
    const int nt = (len + attn::kPrefillRows - 1) / attn::kPrefillRows;
    total_tiles += nt;
    if (nt > max_tiles) max_tiles = nt;
  }
  if (total_tiles * A > INT_MAX) return ATTN_ERR_UNSUPPORTED;
  int max_kv = 0;
  for (int s = 0; s < n_seq; ++s) max_kv = std::max(max_kv, seq_lens_host[s]);
  if (!window_arith_fits(window, max_kv, max_kv)) return ATTN_ERR_UNSUPPORTED;
  attn::FwdParams p = base_params(q, k_cache, v_cache, o, lse, A, A_kv, d_h, scale, causal, nullptr, window, max_kv,
                                  max_kv);
  p.cu_seqlens = cu_seqlens_q;
  p.n_seq = n_seq;
  p.T = total_q;
  p.B = 1;
  p.n_qt = max_tiles;
  p.total_tiles = (int)total_tiles;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.max_pages = max_pages;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.key_range = mask ? mask->key_range : nullptr;
  p.alibi_slopes = mask ? mask->alibi_slopes : nullptr;
  if (blocks) {
    p.block_keep = mask->block_keep;
    p.block_heads = mask->block_heads;
    p.n_kb = (max_kv_len + 127) / 128;
  }
  if (bias) {
    p.bias = mask->bias;
    p.bias_heads = mask->bias_heads;
    p.bias_ld = mask->bias_ld;
    p.inv_scale = (float)(1.0 / (double)scale);
  }
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  p.page_shift = shift;
  attn::plan_varlen_order(p);
  hipStream_t st = (hipStream_t)stream;
  return launch_status(fp8 ? attn::launch_prefill_paged_fp8(p, st) : attn::launch_prefill_paged_bf16(p, st));
}

}  // namespace

ATTN_EXPORT attn_status attn_prefill_paged(const void* q, const void* k_cache, const void* v_cache,
                                           const int32_t* block_table, const int32_t* seq_lens,
                                           const int32_t* seq_lens_host, const int32_t* cu_seqlens_q,
                                           const int32_t* cu_seqlens_q_host, int page_size, void* o, float* lse,
                                           int n_seq, int total_q, int A, int A_kv, int d_h, int max_pages,
                                           int num_pages, float scale, int causal, const attn_window* window,
                                           attn_dtype dtype, void* stream) {
  return prefill_paged_call(q, k_cache, v_cache, nullptr, nullptr, false, block_table, seq_lens, seq_lens_host,
                            cu_seqlens_q, cu_seqlens_q_host, page_size, o, lse, n_seq, total_q, A, A_kv, d_h,
                            max_pages, num_pages, scale, causal, window, dtype, stream);
}

ATTN_EXPORT attn_status attn_prefill_paged_masked(const void* q, const void* k_cache, const void* v_cache,
                                                  const int32_t* block_table, const int32_t* seq_lens,
                                                  const int32_t* seq_lens_host, const int32_t* cu_seqlens_q,
                                                  const int32_t* cu_seqlens_q_host, int page_size, void* o,
                                                  float* lse, int n_seq, int total_q, int A, int A_kv, int d_h,
                                                  int max_pages, int num_pages, float scale, int causal,
                                                  const attn_mask* mask, const attn_window* window,
                                                  attn_dtype dtype, void* stream) {
  return prefill_paged_call(q, k_cache, v_cache, nullptr, nullptr, false, block_table, seq_lens, seq_lens_host,
                            cu_seqlens_q, cu_seqlens_q_host, page_size, o, lse, n_seq, total_q, A, A_kv, d_h,
                            max_pages, num_pages, scale, causal, window, dtype, stream, mask);
}

ATTN_EXPORT attn_status attn_prefill_paged_fp8(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                                               const float* k_scale, const float* v_scale,
                                               const int32_t* block_table, const int32_t* seq_lens,
                                               const int32_t* seq_lens_host, const int32_t* cu_seqlens_q,
                                               const int32_t* cu_seqlens_q_host, int page_size, void* o, float* lse,
                                               int n_seq, int total_q, int A, int A_kv, int d_h, int max_pages,
                                               int num_pages, float scale, int causal, const attn_window* window,
                                               void* stream) {
  return prefill_paged_call(q, k_cache, v_cache, k_scale, v_scale, true, block_table, seq_lens, seq_lens_host,
                            cu_seqlens_q, cu_seqlens_q_host, page_size, o, lse, n_seq, total_q, A, A_kv, d_h,
                            max_pages, num_pages, scale, causal, window, ATTN_BF16, stream);
}

namespace {

size_t bwd_workspace_bytes(int B, int A, int S_q) {
  const size_t n = (size_t)B * (size_t)A * (size_t)S_q * 2 * sizeof(float);
  return (n + 255) & ~(size_t)255;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

ATTN_EXPORT size_t attn_bwd_workspace_bytes(int B, int A, int S_q) {
  if (B < 1 || A < 1 || S_q < 0) return 0;
  return bwd_workspace_bytes(B, A, S_q);
}

namespace {

// fields of a backward launch shared by the dense and packed entry points
attn::BwdParams bwd_params(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, void* dq, void* dk, void* dv, int A, int A_kv, int d_h, float scale,
                           int causal, const attn_mask* mask, void* workspace) {
  attn::BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.row_stats = (float*)workspace;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.q_keep = mask ? mask->q_keep : nullptr;
  p.k_keep = mask ? mask->k_keep : nullptr;
  p.key_range = mask ? mask->key_range : nullptr;
  p.alibi_slopes = mask ? mask->alibi_slopes : nullptr;
  p.A = A;
  p.A_kv = A_kv;
  p.G = A / A_kv;
  p.d = d_h;
  p.causal = causal ? 1 : 0;
  p.scale = scale;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);
  p.inv_scale = (float)(1.0 / (double)scale);
  return p;
}

}  // namespace

ATTN_EXPORT attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                 const float* lse, void* dq, void* dk, void* dv, int B, int A, int A_kv, int S_q,
                                 int S_k, int d_h, float scale, int causal, const attn_mask* mask,
                                 const attn_window* window, attn_dtype dtype, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (B < 1 || A < 1 || A_kv < 1 || S_q < 0 || S_k < 0 || d_h < 1 || A % A_kv != 0) return ATTN_ERR_INVAL;
  if (!valid_scale(scale) || !valid_window(window)) return ATTN_ERR_INVAL;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVAL;
  if (S_q > 0 && (!q || !o || !dout || !lse || !dq)) return ATTN_ERR_INVAL;
  if (S_k > 0 && (!k || !v || !dk || !dv)) return ATTN_ERR_INVAL;
  for (const void* t : {q, k, v, o, dout, (const void*)lse, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!aligned16(t)) return ATTN_ERR_INVAL;
  if (!key_range_aligned(mask)) return ATTN_ERR_INVAL;
  if (dtype != ATTN_BF16 || (d_h != 64 && d_h != 128)) return ATTN_ERR_UNSUPPORTED;
  const bool blocks = mask && mask->block_keep;
  const bool bias = mask && mask->bias;
  if (blocks && mask->block_heads != 1 && mask->block_heads != A) return ATTN_ERR_INVAL;
  if (bias && !valid_bias(mask->bias, mask->bias_heads, A, S_q, S_k, mask->bias_ld)) return ATTN_ERR_INVAL;
  if (bias && mask->key_range) return ATTN_ERR_UNSUPPORTED;  // as the forward
  if (!alibi_alone(mask)) return ATTN_ERR_UNSUPPORTED;
  if (S_q > kMaxLen || S_k > kMaxLen) return ATTN_ERR_UNSUPPORTED;
  const long long n_qb = (S_q + 127) / 128, n_kb = (S_k + 127) / 128;
  if (blocks && (n_kb > attn::kBwdMaxKeyBlocks || (long long)(A / A_kv) * n_qb > attn::kBwdMaxRowBlocks))
    return ATTN_ERR_UNSUPPORTED;
  if ((long long)B * A * (long long)S_q > INT_MAX || (long long)B * A_kv * (long long)S_k > INT_MAX)
    return ATTN_ERR_UNSUPPORTED;
  if (!window_arith_fits(window, S_q, S_k)) return ATTN_ERR_UNSUPPORTED;
  const long long n_qt = (S_q + attn::kBwdQRows - 1) / attn::kBwdQRows;
  const long long n_kt = (S_k + attn::kBwdKRows - 1) / attn::kBwdKRows;
  if (n_qt * A * B > INT_MAX || n_kt * A_kv * B > INT_MAX) return ATTN_ERR_UNSUPPORTED;
  const size_t need = S_q > 0 ? bwd_workspace_bytes(B, A, S_q) : 0;
  if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255) != 0))
    return ATTN_ERR_INVAL;
  attn::BwdParams p = bwd_params(q, k, v, o, dout, lse, dq, dk, dv, A, A_kv, d_h, scale, causal, mask, workspace);
  p.B = B;
  p.S_q = S_q;
  p.S_k = S_k;
  if (blocks) {
    p.block_keep = mask->block_keep;
    p.block_heads = mask->block_heads;
    p.n_qb = (int)n_qb;
    p.n_kb = (int)n_kb;
  }
  if (bias) {
    p.bias = mask->bias;
    p.bias_heads = mask->bias_heads;
    p.bias_ld = mask->bias_ld;
    p.inv_scale = (float)(1.0 / (double)scale);
  }
  window_edges(window, causal, S_k, S_q, p.win_left, p.win_right);
  return launch_status(attn::launch_bwd_bf16(p, (hipStream_t)stream));
}

ATTN_EXPORT attn_status attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                        const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int n_seq,
                                        int total_tokens, int A, int A_kv, int d_h, float scale, int causal,
                                        const attn_mask* mask, const attn_window* window, attn_dtype dtype,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  if (n_seq < 0 || total_tokens < 0 || A < 1 || A_kv < 1 || d_h < 1 || A % A_kv != 0) return ATTN_ERR_INVAL;
  if (!valid_scale(scale) || !valid_window(window)) return ATTN_ERR_INVAL;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVAL;
  if (!cu_seqlens || !cu_seqlens_host) return ATTN_ERR_INVAL;
  if (cu_seqlens_host[0] != 0 || cu_seqlens_host[n_seq] != total_tokens) return ATTN_ERR_INVAL;
  for (int s = 0; s < n_seq; ++s)
    if (cu_seqlens_host[s + 1] < cu_seqlens_host[s]) return ATTN_ERR_INVAL;
  if (total_tokens > 0 && (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv)) return ATTN_ERR_INVAL;
  for (const void* t : {q, k, v, o, dout, (const void*)lse, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!aligned16(t)) return ATTN_ERR_INVAL;
  if (!aligned(cu_seqlens, 4) || !key_range_aligned(mask)) return ATTN_ERR_INVAL;
  if (dtype != ATTN_BF16 || (d_h != 64 && d_h != 128)) return ATTN_ERR_UNSUPPORTED;
  long long total_tiles = 0;
  int max_tiles = 0, max_len = 0;
  for (int s = 0; s < n_seq; ++s) {
    const int len = cu_seqlens_host[s + 1] - cu_seqlens_host[s];
    const int nt = (len + attn::kBwdQRows - 1) / attn::kBwdQRows;
    total_tiles += nt;
    max_tiles = std::max(max_tiles, nt);
    max_len = std::max(max_len, len);
  }
  // the forward's packed masks: block flags [n_seq, block_heads, nb, nb]
  // (nb = max_tiles: 128-row tiles), terms [bias_heads, T, bias_ld]
  const bool blocks = mask && mask->block_keep;
  const bool bias = mask && mask->bias;
  if (blocks && mask->block_heads != 1 && mask->block_heads != A) return ATTN_ERR_INVAL;
  if (bias && !valid_bias(mask->bias, mask->bias_heads, A, max_len, max_len, mask->bias_ld)) return ATTN_ERR_INVAL;
  if (bias && mask->key_range) return ATTN_ERR_UNSUPPORTED;  // as the forward
  if (!alibi_alone(mask)) return ATTN_ERR_UNSUPPORTED;
  if (blocks && (max_tiles > attn::kBwdMaxKeyBlocks || (long long)(A / A_kv) * max_tiles > attn::kBwdMaxRowBlocks))
    return ATTN_ERR_UNSUPPORTED;
  if (total_tokens == 0) return ATTN_OK;
  if (max_len > kMaxLen || (long long)A * total_tokens > INT_MAX) return ATTN_ERR_UNSUPPORTED;
  if (total_tiles * A > INT_MAX) return ATTN_ERR_UNSUPPORTED;
  if (!window_arith_fits(window, max_len, max_len)) return ATTN_ERR_UNSUPPORTED;
  const size_t need = bwd_workspace_bytes(1, A, total_tokens);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255) != 0) return ATTN_ERR_INVAL;
  attn::BwdParams p = bwd_params(q, k, v, o, dout, lse, dq, dk, dv, A, A_kv, d_h, scale, causal, mask, workspace);
  p.B = 1;
  p.cu_seqlens = cu_seqlens;
  p.n_seq = n_seq;
  p.T = total_tokens;
  p.max_tiles = max_tiles;
  p.total_tiles = (int)total_tiles;
  if (blocks) {
    p.block_keep = mask->block_keep;
    p.block_heads = mask->block_heads;
    p.n_qb = p.n_kb = max_tiles;
  }
  if (bias) {
    p.bias = mask->bias;
    p.bias_heads = mask->bias_heads;
    p.bias_ld = mask->bias_ld;
    p.inv_scale = (float)(1.0 / (double)scale);
  }
  window_edges(window, causal, max_len, max_len, p.win_left, p.win_right);
  return launch_status(attn::launch_bwd_bf16(p, (hipStream_t)stream));
}

namespace {

attn_status decode_fp8_call(const void* q, const uint8_t* k_cache, const uint8_t* v_cache, const float* k_scale,
                            const float* v_scale, const int32_t* block_table, const int32_t* seq_lens,
                            const int32_t* seq_lens_host, int page_size, void* o, float* lse, int B, int A,
                            int A_kv, int d_h, int max_pages, int num_pages, float scale, int window_left,
                            void* workspace, size_t workspace_bytes, void* stream,
                            const float* alibi_slopes = nullptr) {
  if (max_pages < 0 || num_pages < 0) return ATTN_ERR_INVAL;
  attn_status st = check_decode(B, A, A_kv, d_h, page_size, seq_lens_host, max_pages, true);
  if (st != ATTN_OK) return st;
  if (!valid_scale(scale)) return ATTN_ERR_INVAL;
  if (!q || !o || !lse || !seq_lens) return ATTN_ERR_INVAL;
  long long total_tokens = 0;
  for (int b = 0; b < B; ++b) total_tokens += seq_lens_host[b];
  if (total_tokens > 0 && (!k_cache || !v_cache || !k_scale || !v_scale || !block_table || num_pages < 1))
    return ATTN_ERR_INVAL;
  if (!aligned(k_cache, 8) || !aligned(v_cache, 8) || !aligned(q, 16) || !aligned(o, 16)) return ATTN_ERR_INVAL;
  for (const void* t : {(const void*)lse, (const void*)seq_lens, (const void*)block_table, (const void*)k_scale,
                        (const void*)v_scale})
    if (!aligned(t, 4)) return ATTN_ERR_INVAL;
  const attn::DecodePlan plan = attn::plan_decode(B, seq_lens_host, window_left);
  const size_t need = attn::decode_workspace_bytes(A, d_h, plan);
  if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255) != 0))
    return ATTN_ERR_INVAL;
  if ((long long)B * A > INT_MAX) return ATTN_ERR_UNSUPPORTED;
  attn::DecodeParams p{};
  p.win_left = window_left;
  p.alibi_slopes = alibi_slopes;
  p.inv_scale = (float)(1.0 / (double)scale);
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.o = o;
  p.lse = lse;
  p.part_o = (float*)workspace;
  p.part_lse = (float*)((char*)workspace + attn::decode_workspace_lse_offset(A, d_h, plan));
  p.B = B;
  p.A = A;
  p.A_kv = A_kv;
  p.G = A / A_kv;
  p.d = d_h;
  p.page_size = page_size;
  p.max_pages = max_pages;
  p.n_chunks = plan.n_chunks;
  p.scale = scale;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);
  return launch_status(attn::launch_decode_fp8(p, (hipStream_t)stream));
}

}  // namespace

ATTN_EXPORT attn_status attn_decode_paged_fp8(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                                              const float* k_scale, const float* v_scale,
                                              const int32_t* block_table, const int32_t* seq_lens,
                                              const int32_t* seq_lens_host, int page_size, void* o, float* lse,
                                              int B, int A, int A_kv, int d_h, int max_pages, int num_pages,
                                              float scale, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_fp8_call(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, seq_lens_host, page_size, o,
                         lse, B, A, A_kv, d_h, max_pages, num_pages, scale, -1, workspace, workspace_bytes, stream);
}

ATTN_EXPORT attn_status attn_decode_paged_fp8_window(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                                                     const float* k_scale, const float* v_scale,
                                                     const int32_t* block_table, const int32_t* seq_lens,
                                                     const int32_t* seq_lens_host, int page_size, void* o,
                                                     float* lse, int B, int A, int A_kv, int d_h, int max_pages,
                                                     int num_pages, float scale, int window_left, void* workspace,
                                                     size_t workspace_bytes, void* stream) {
  if (window_left < -1) return ATTN_ERR_INVAL;
  return decode_fp8_call(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, seq_lens_host, page_size, o,
                         lse, B, A, A_kv, d_h, max_pages, num_pages, scale, window_left, workspace,
                         workspace_bytes, stream);
}

ATTN_EXPORT attn_status attn_decode_paged_fp8_alibi(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                                                    const float* k_scale, const float* v_scale,
                                                    const int32_t* block_table, const int32_t* seq_lens,
                                                    const int32_t* seq_lens_host, int page_size, void* o,
                                                    float* lse, int B, int A, int A_kv, int d_h, int max_pages,
                                                    int num_pages, float scale, int window_left,
                                                    const float* alibi_slopes, void* workspace,
                                                    size_t workspace_bytes, void* stream) {
  if (window_left < -1 || !alibi_slopes || !aligned(alibi_slopes, 4)) return ATTN_ERR_INVAL;
  return decode_fp8_call(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, seq_lens_host, page_size, o,
                         lse, B, A, A_kv, d_h, max_pages, num_pages, scale, window_left, workspace,
                         workspace_bytes, stream, alibi_slopes);
}

ATTN_EXPORT const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVAL: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

ATTN_EXPORT int attn_abi_version(void) { return kAbiVersion; }
