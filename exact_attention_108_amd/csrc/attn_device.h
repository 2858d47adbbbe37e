// attn_device.h -- device-side types and helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) (v_log_f32).
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Value held by lane l ^ 32, combined with this lane's: v_permlane32_swap
// exchanges the upper half of the first operand with the lower half of the
// second, so with both operands = x the pair is {x[l], x[l ^ 32]} in every lane.
__device__ __forceinline__ float max_with_other_half(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float sum_with_other_half(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 32x32x64 over OCP E4M3 (format 0) operands: lane l holds row (A) / column
// (B) l % 32, 32 bytes of the K dimension.  The instruction's block-exponent
// operands are 127 (2^0) for both sides, so the product is unscaled.
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x16 mfma32_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 16x16x16 (K = 16): lane l holds A[l % 16][4 (l / 16) + s], B[4 (l / 16) + s][l % 16]
__device__ __forceinline__ f32x4 mfma16_k16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b), c,
                                                   0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element (i & 3) of the 4-element chunk addressed by lane
// 4*r + (i >> 2), for r = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// 16-byte global -> LDS copy (global_load_lds_dwordx4): lane L's 16 bytes land
// at LDS byte lds_wave_base + 16 * L.  The copy is issued from inline assembly
// so the compiler does not add its own (whole-queue) wait before later LDS
// reads; the caller orders it with lds_copy_wait_all() and a barrier.  M0
// carries the wave-uniform LDS base; no other code in these kernels uses M0.
__device__ __forceinline__ void lds_copy16(const void* gptr, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds_wave_base), "v"(gptr)
               : "memory");
}
// Buffer resource (V#) for raw byte-addressed loads from `base`: stride 0, so
// a lane's access is in range iff its byte offset < num_bytes; out-of-range
// lanes touch no memory and read zeros.  Every field is wave-uniform (SGPRs).
__device__ __forceinline__ i32x4 make_buffer_rsrc(const void* base, uint32_t num_bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane((int)num_bytes);
  r[3] = 0x00020000;  // 32-bit data format, no swizzle (gfx9 family)
  return r;
}
// 16-byte buffer -> LDS copy (buffer_load_dwordx4 ... lds): lane L's 16 bytes
// at byte `voff` of the resource land at LDS byte lds_wave_base + 16 * L; a
// lane whose offset is out of the resource's range writes 16 zero bytes.
// Ordered like lds_copy16 (explicit waits, M0 holds the LDS base).
__device__ __forceinline__ void lds_copy16_buf(i32x4 rsrc, uint32_t voff, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_wave_base), "v"(voff), "s"(rsrc)
               : "memory");
}
// Wait until at most N vector-memory loads of this wave are outstanding
// (loads complete in issue order, so every older LDS copy has landed).
template <int N>
__device__ __forceinline__ void lds_copy_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x0F70);  // vmcnt(N)
  asm volatile("" ::: "memory");
}
// Wait until every vector-memory load of this wave (including the LDS copies)
// has completed.
__device__ __forceinline__ void lds_copy_wait_all() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  asm volatile("" ::: "memory");
}

// Scheduling hint for a basic block that mixes MFMA chains with the LDS reads
// and vector-ALU work feeding them: LLVM's interleaving strategy 0 for
// MFMA-heavy code spreads the reads and ALU work between the matrix
// instructions (measured: 1-2% on the prefill loop, 6-11% on the backward
// passes, bit-identical results).
__device__ __forceinline__ void interleave_hint() { __builtin_amdgcn_iglp_opt(0); }

// Wave-uniform load of one int32 (base[idx], both uniform): the address is
// made scalar and read through the constant address space, so the load is an
// s_load_dword, counted by lgkmcnt.  A vector load would be counted by vmcnt,
// and waiting for it would also wait for every asynchronous LDS copy in flight.
__device__ __forceinline__ int load_uniform_i32(const int32_t* base, int idx) {
  const uint64_t a = (uint64_t)(uintptr_t)(base + idx);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
  return *(const_i32_ptr)(((uint64_t)hi << 32) | lo);
}

// Per-row key ranges (the mask rule first <= j <= last).  A row's pair is
// clamped to [-1, n_keys]: the same keys of 0 .. n_keys - 1 stay kept, and
// position arithmetic on the ends stays far from int32 overflow.
__device__ __forceinline__ int2 load_key_range(const int32_t* kr, int row, int n_keys) {
  const int2 r = *(const int2*)(kr + 2 * (size_t)row);
  return make_int2(min(max(r.x, -1), n_keys), min(max(r.y, -1), n_keys));
}
__device__ __forceinline__ int wave_min_i32(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = min(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_max_i32(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = max(x, __shfl_xor(x, o));
  return x;
}
// Key bounds of a group of rows under key ranges: [any_lo, any_hi) holds
// every key some row keeps (empty when none keeps a key), [all_lo, all_hi)
// the keys every row keeps (empty when some row keeps none).
struct KeyBounds {
  int any_lo, any_hi, all_lo, all_hi;
};
constexpr int kNoKey = 1 << 30;
// the bounds of this wave's rows: `row` says whether the lane holds a row that
// exists, (lo, hi) its clamped range; the result is wave-uniform
__device__ __forceinline__ KeyBounds wave_key_bounds(bool row, int lo, int hi) {
  const bool some = row && lo <= hi;
  KeyBounds b;
  b.any_lo = __builtin_amdgcn_readfirstlane(wave_min_i32(some ? lo : kNoKey));
  b.any_hi = __builtin_amdgcn_readfirstlane(wave_max_i32(some ? hi + 1 : -kNoKey));
  b.all_lo = __builtin_amdgcn_readfirstlane(wave_max_i32(row ? lo : -kNoKey));
  b.all_hi = __builtin_amdgcn_readfirstlane(wave_min_i32(row ? hi + 1 : kNoKey));
  return b;
}
// combine the bounds of a workgroup's waves through `slots` (one per wave,
// in LDS); every thread of the workgroup must call it (it holds a barrier)
template <int kWaves>
__device__ __forceinline__ KeyBounds workgroup_key_bounds(const KeyBounds& w, KeyBounds* slots, int wave, int lane) {
  if (lane == 0) slots[wave] = w;
  __syncthreads();
  KeyBounds b = slots[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) {
    const KeyBounds o = slots[i];
    b.any_lo = min(b.any_lo, o.any_lo);
    b.any_hi = max(b.any_hi, o.any_hi);
    b.all_lo = max(b.all_lo, o.all_lo);
    b.all_hi = min(b.all_hi, o.all_hi);
  }
  return b;
}

__device__ __forceinline__ bf16x8 concat(i16x4 a, i16x4 b) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// LDS row swizzle over 16-byte chunks (chunk c of row `row` lives at chunk
// c ^ sigma(row)).  sigma is chosen so that (a) 16 consecutive rows read at one
// logical chunk hit 16 distinct bank groups, and (b) 4 consecutive rows (row %
// 4 == 0 at the first) x 4 consecutive chunks (first % 4 == 0) also do -- the
// two access shapes of the K-operand reads and the transposing V reads.
template <int D>
__device__ __forceinline__ int lds_chunk(int row, int c) {
  if constexpr (D == 128) {
    return c ^ (((row & 3) << 2) | ((row >> 2) & 3));
  } else {
    static_assert(D == 64, "head dim 64 or 128");
    return c ^ ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
  }
}

}  // namespace attn
