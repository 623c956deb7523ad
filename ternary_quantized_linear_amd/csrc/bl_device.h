// bl_device.h -- device helpers shared by the gfx950 kernels of libbitlinear.
//
// Wave64 reductions use DPP row operations (quad_perm, row_shr, row_bcast) and
// readlane; no LDS round trip. The 2-bit unpack and the activation transpose below
// fix the k-order that every product kernel uses inside a 16-code group (see
// unpack_u2 and transpose16).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

constexpr int kWave = 64;

// ---------------------------------------------------------------- DPP reductions
// dpp_ctrl encodings (GFX9): quad_perm = 0x00..0xFF, row_shr:n = 0x110 + n,
// row_bcast:15 = 0x142, row_bcast:31 = 0x143.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, true);
}

// Sum of v over each group of L consecutive lanes (L = 16, 32 or 64); the group total
// lands in the group's last lane (lane % L == L-1). Other lanes hold partial sums.
template <int L>
__device__ __forceinline__ int group_sum_to_last(int v) {
  v += dpp_i32<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_i32<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_i32<0x114>(v);  // row_shr:4
  v += dpp_i32<0x118>(v);  // row_shr:8   -> row total in lane 15 of each row
  if constexpr (L >= 32) v += dpp_i32<0x142, 0xA>(v);  // row_bcast:15 -> lanes 31, 63
  if constexpr (L >= 64) v += dpp_i32<0x143, 0xC>(v);  // row_bcast:31 -> lane 63
  return v;
}

// The same moves for a double (both halves with one control) and a float. A lane whose
// source is outside its row, or whose row is masked off, receives +0.0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_f64(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const unsigned lo = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)b, CTRL, ROW_MASK, 0xF, true);
  const unsigned hi =
      (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)(b >> 32), CTRL, ROW_MASK, 0xF, true);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(dpp_i32<CTRL, ROW_MASK>(__float_as_int(v)));
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)b, lane);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b >> 32), lane);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

__device__ __forceinline__ float readlane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Maximum of non-negative v over each group of L lanes, into the group's last lane
// (the +0.0 of lanes without a source never exceeds a non-negative value).
template <int L>
__device__ __forceinline__ float group_max_to_last(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  if constexpr (L >= 8) v = fmaxf(v, dpp_f32<0x114>(v));
  if constexpr (L >= 16) v = fmaxf(v, dpp_f32<0x118>(v));
  if constexpr (L >= 32) v = fmaxf(v, dpp_f32<0x142, 0xA>(v));
  if constexpr (L >= 64) v = fmaxf(v, dpp_f32<0x143, 0xC>(v));
  return v;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
  return __builtin_amdgcn_readlane(group_sum_to_last<64>(v), 63);
}

__device__ __forceinline__ unsigned wave_max_u32(unsigned v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    unsigned o = (unsigned)__shfl_xor((int)v, m, kWave);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// ---------------------------------------------------------------- double-double
// Error-free transformations (Knuth's two-sum, Dekker's fast-two-sum). The library is
// compiled with -ffp-contract=off, so no product or sum below is fused or reordered.
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

__device__ __forceinline__ void dd_add(double& hi, double& lo, double bhi, double blo) {
  double s, e;
  two_sum(hi, bhi, s, e);
  e += lo + blo;
  hi = s + e;               // fast-two-sum renormalization (|s| >= |e|)
  lo = e - (hi - s);
}

// Double-double sum over each group of L lanes into the group's last lane, in the same
// DPP pattern as group_sum_to_last (a fixed order: every call combines the same pairs).
template <int L>
__device__ __forceinline__ void group_dd_sum_to_last(double& hi, double& lo) {
#define BL_DD_STEP(...)                                              \
  {                                                                  \
    const double th = dpp_f64<__VA_ARGS__>(hi), tl = dpp_f64<__VA_ARGS__>(lo); \
    dd_add(hi, lo, th, tl);                                          \
  }
  BL_DD_STEP(0xB1)
  BL_DD_STEP(0x4E)
  if constexpr (L >= 8) BL_DD_STEP(0x114)
  if constexpr (L >= 16) BL_DD_STEP(0x118)
  if constexpr (L >= 32) BL_DD_STEP(0x142, 0xA)
  if constexpr (L >= 64) BL_DD_STEP(0x143, 0xC)
#undef BL_DD_STEP
}

// ---------------------------------------------------------------- 2-bit codes
// A packed dword holds 16 codes: byte b carries codes 4b+0..4b+3 in bit pairs
// [1:0], [3:2], [5:4], [7:6] as u = q + 1 in {0, 1, 2}. unpack_u2 returns four dwords:
// dword p, byte b = u of code 4b + p. So the 16 codes leave in "p-major" order.
__device__ __forceinline__ void unpack_u2(uint32_t w, uint32_t u[4]) {
  u[0] = w & 0x03030303u;
  u[1] = (w >> 2) & 0x03030303u;
  u[2] = (w >> 4) & 0x03030303u;
  u[3] = (w >> 6) & 0x03030303u;
}

// Signed codes q = u - 1 in {-1, 0, 1} for the same order: v_perm_b32 with the u value
// of each byte as a selector into the byte table {0xFF, 0x00, 0x01}.
__device__ __forceinline__ void unpack_q2(uint32_t w, uint32_t q[4]) {
  constexpr uint32_t kTable = 0x000100FFu;  // byte0 = -1, byte1 = 0, byte2 = +1
  uint32_t u[4];
  unpack_u2(w, u);
#pragma unroll
  for (int p = 0; p < 4; ++p) q[p] = __builtin_amdgcn_perm(0u, kTable, u[p]);
}

// 4x4 byte transpose of 16 activation bytes x[0..15] held as 4 dwords (a[b] holds
// x[4b..4b+3]): out dword p, byte b = x[4b + p] -- the same p-major order as
// unpack_u2, so a dot product over a dword pair multiplies matching codes.
__device__ __forceinline__ void transpose16(const uint32_t a[4], uint32_t o[4]) {
  uint32_t lo01 = __builtin_amdgcn_perm(a[1], a[0], 0x05010400u);  // a0.0 a1.0 a0.1 a1.1
  uint32_t hi01 = __builtin_amdgcn_perm(a[1], a[0], 0x07030602u);  // a0.2 a1.2 a0.3 a1.3
  uint32_t lo23 = __builtin_amdgcn_perm(a[3], a[2], 0x05010400u);
  uint32_t hi23 = __builtin_amdgcn_perm(a[3], a[2], 0x07030602u);
  o[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);  // a0.0 a1.0 a2.0 a3.0
  o[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);  // a0.1 a1.1 a2.1 a3.1
  o[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
  o[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
}

// 128-bit load marked non-temporal (streamed once; keeps it from displacing reused
// data in the caches).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// fp32 -> bf16 bits, round to nearest, ties to even (the carry out of the dropped
// 16 bits, biased by the kept part's last bit); NaN stays NaN (quiet).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// Sum of the four signed bytes of a dword.
__device__ __forceinline__ int byte_sum(uint32_t a) { return sdot4(a, 0x01010101u, 0); }

}  // namespace bl
