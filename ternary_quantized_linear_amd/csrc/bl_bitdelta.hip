// bl_bitdelta.hip -- BitDelta inference: one base weight matrix shared by B fine-tuned
// models, each model a 1-bit delta (sign bits and one scale), one token per model.
//
// [BitDelta] "BitDelta: Your Fine-Tune May Only Be Worth One Bit": Eq. (1) the delta of
// a fine-tune is alpha * Sign(delta); Eq. (2) Sign(W) = +1 for W > 0, -1 otherwise;
// Eq. (4) alpha = mean |delta|; Eq. (6) the fine-tuned product is the base product plus
// the 1-bit delta product: y_i = W_base x_i + alpha_i Sign(delta_i) x_i. Figure 4 times
// this for B = 8 models at N = M = 8192 (one base matrix and B deltas read per token
// batch, instead of B full matrices).
//
// Layout: W_base bf16 [N, M] row-major; the models' sign bits interleaved per 16-code
// group in 8 slots: row n, group j, model i at bytes ((n * M/16 + j) * 8 + i) * 2 (bit
// c = code 16j + c, set for +1; slots >= B unused), so that one aligned 16-byte load
// brings a lane every model's bits for its 16 codes; X fp32 [B, M]; Y fp32 [B, N].
//
// Kernel: a workgroup of 8 waves takes rows n = w, w + nwg, ...; wave s owns codes
// [1024 s, 1024 s + 1024) of every row (M <= 8192), 16 per lane, and keeps those 16
// activations of every token in registers (with their sums). Per row and lane: the
// 16 bf16 base weights against all B tokens (fp32 FMAs), and for model i the sum of its
// activations where the sign bit is set, P_i, so that sign . x = 2 P_i - sum x
// (bit -> all-ones mask by a one-bit signed extract, AND, add). The lane's B values
// b_i + alpha_i (2 P_i - sum x_i) are summed across the wave with DPP; each wave leaves
// its B row partials in its own LDS slot [row][wave][model]; after the sweep, one
// barrier, and each thread sums the slots of one (row, model) in wave order and stores
// it. Every sum is taken in a fixed order, so Y is the same bit for bit from call to
// call. Weights and bits are buffer loads in a
// ring three rows deep (rows past N read as zeros without a memory access).
#include "bl_device.h"
#include "bl_internal.h"
#include "bl_plan.h"

namespace bl {

constexpr int kBdWaves = 8;
constexpr int kBdThreads = kBdWaves * kWave;
constexpr int kBdLaneCodes = 16;
constexpr int kBdWaveCodes = kBdLaneCodes * kWave;  // 1024
constexpr int kBdMaxB = 8;
constexpr int kBdDepth = 3;

struct BdArgs {
  const uint16_t* base;
  const uint8_t* D;
  const float* alpha;
  const float* X;
  float* Y;
  int N, M, B, S, R, nwg;
};

// LDS per workgroup: the row partials [R][S][kBdMaxB] (bl_plan.h).
using plan::bd_lds_bytes;
constexpr size_t kBdLdsMax = plan::kBdLdsMax;
static_assert(plan::kBdMaxB == kBdMaxB && plan::kBdWaves == kBdWaves, "plan constants");

typedef __amdgpu_buffer_rsrc_t BdRsrc;
constexpr uint32_t kBdOob = 0x80000000u;

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float bd_dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, true));
}

// Sum over the 64 lanes into lane 63 (same DPP pattern as the integer reductions).
__device__ __forceinline__ float wave_sum_to_last(float v) {
  v += bd_dpp<0xB1>(v);
  v += bd_dpp<0x4E>(v);
  v += bd_dpp<0x114>(v);
  v += bd_dpp<0x118>(v);
  v += bd_dpp<0x142, 0xA>(v);
  v += bd_dpp<0x143, 0xC>(v);
  return v;
}

// One wave's share of the rows: codes [1024 wave, 1024 wave + 1024) of every row of the
// workgroup; its B partial row sums go to LDS slot [row][wave][model].
__device__ __forceinline__ void bd_sweep(const BdArgs& a, float* sums, int wave) {
  const int lane = threadIdx.x & (kWave - 1);
  const int k0 = wave * kBdWaveCodes + kBdLaneCodes * lane;
  const bool on = k0 < a.M;
  const int B = a.B;

  float x[kBdMaxB][kBdLaneCodes];
  float xs[kBdMaxB];
  float al[kBdMaxB];
#pragma unroll
  for (int i = 0; i < kBdMaxB; ++i) {
    const bool ok = on && i < B;
    xs[i] = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 f = ok ? reinterpret_cast<const float4*>(a.X + (int64_t)i * a.M + k0)[q]
                          : make_float4(0.f, 0.f, 0.f, 0.f);
      x[i][4 * q] = f.x;
      x[i][4 * q + 1] = f.y;
      x[i][4 * q + 2] = f.z;
      x[i][4 * q + 3] = f.w;
    }
#pragma unroll
    for (int c = 0; c < kBdLaneCodes; ++c) xs[i] += x[i][c];
    al[i] = i < B ? a.alpha[i] : 0.0f;
  }

  const BdRsrc br = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.base), 0,
                                                      (int)((uint32_t)a.N * (uint32_t)a.M * 2u),
                                                      0x00020000);
  const BdRsrc dr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.D), 0,
                                                      (int)((uint32_t)a.N * (uint32_t)a.M),
                                                      0x00020000);
  const int wgl = blockIdx.x;
  uint4 wb[kBdDepth][2], wd[kBdDepth];
  int fr = 0;
  auto load_row = [&](int d) {
    const int n = wgl + fr * a.nwg;
    const bool ok = on && n < a.N;
    const uint32_t bo = ok ? ((uint32_t)n * (uint32_t)a.M + (uint32_t)k0) * 2u : kBdOob;
    const uint32_t dof = ok ? ((uint32_t)n * (uint32_t)(a.M / 16) + (uint32_t)(k0 / 16)) * 16u
                            : kBdOob;
    typedef int v4i __attribute__((ext_vector_type(4)));
    const v4i b0 = __builtin_amdgcn_raw_buffer_load_b128(br, bo, 0, 2);
    const v4i b1 = __builtin_amdgcn_raw_buffer_load_b128(br, bo + 16, 0, 2);
    const v4i dd = __builtin_amdgcn_raw_buffer_load_b128(dr, dof, 0, 2);
    wb[d][0] = make_uint4(b0[0], b0[1], b0[2], b0[3]);
    wb[d][1] = make_uint4(b1[0], b1[1], b1[2], b1[3]);
    wd[d] = make_uint4(dd[0], dd[1], dd[2], dd[3]);
    ++fr;
  };
#pragma unroll
  for (int d = 0; d < kBdDepth; ++d) load_row(d);

  int cr = 0;
  auto step = [&](int d, bool prefetch) {
    float w[kBdLaneCodes];
    const uint32_t bw[8] = {wb[d][0].x, wb[d][0].y, wb[d][0].z, wb[d][0].w,
                            wb[d][1].x, wb[d][1].y, wb[d][1].z, wb[d][1].w};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      w[2 * c] = __uint_as_float(bw[c] << 16);
      w[2 * c + 1] = __uint_as_float(bw[c] & 0xFFFF0000u);
    }
    const uint32_t dw[4] = {wd[d].x, wd[d].y, wd[d].z, wd[d].w};
    float v[kBdMaxB];
#pragma unroll
    for (int i = 0; i < kBdMaxB; ++i) {
      float b = 0.0f, p = 0.0f;
#pragma unroll
      for (int c = 0; c < kBdLaneCodes; ++c) b = __fmaf_rn(w[c], x[i][c], b);
      const uint32_t bits = (dw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
#pragma unroll
      for (int c = 0; c < kBdLaneCodes; ++c) {
        const int m = __builtin_amdgcn_sbfe((int)bits, c, 1);  // 0 or -1
        p += __int_as_float(__float_as_int(x[i][c]) & m);
      }
      v[i] = b + al[i] * (2.0f * p - xs[i]);
    }
    if (prefetch) load_row(d);
#pragma unroll
    for (int i = 0; i < kBdMaxB; ++i) v[i] = wave_sum_to_last(v[i]);
    if (lane == kWave - 1) {
      float* row = sums + (cr * a.S + wave) * kBdMaxB;
#pragma unroll
      for (int i = 0; i < kBdMaxB; ++i) row[i] = v[i];
    }
    ++cr;
  };
  int n = 0;
  while (a.R - n >= kBdDepth) {
#pragma unroll
    for (int d = 0; d < kBdDepth; ++d) step(d, true);
    n += kBdDepth;
  }
#pragma unroll
  for (int d = 0; d < kBdDepth - 1; ++d)
    if (n + d < a.R) step(d, false);
}

__global__ __launch_bounds__(kBdThreads) void bitdelta_kernel(BdArgs a) {
  extern __shared__ float bd_lds[];
  float* sums = bd_lds;  // [R][S][kBdMaxB]: each wave's partial of each row and model
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave < a.S) bd_sweep(a, sums, wave);  // waves past the codes only wait below
  // every partial is in LDS: thread (row, model) sums the S slots in wave order
  __syncthreads();
  for (int idx = threadIdx.x; idx < a.R * a.B; idx += kBdThreads) {
    const int cr = idx / a.B, i = idx - cr * a.B;
    const int n = blockIdx.x + cr * a.nwg;
    if (n >= a.N) continue;
    const float* row = sums + cr * a.S * kBdMaxB + i;
    float y = row[0];
    for (int s = 1; s < a.S; ++s) y += row[s * kBdMaxB];
    a.Y[(int64_t)i * a.N + n] = y;
  }
}

}  // namespace bl

using namespace bl;

bool bl_bitdelta_supports(int64_t N, int64_t M, int B) {
  return N >= 1 && M >= 16 && M % 16 == 0 && M <= kBdWaves * kBdWaveCodes && B >= 1 &&
         B <= kBdMaxB && N * M * 2 < (int64_t(1) << 31);
}

hipError_t bl_launch_bitdelta(const uint16_t* base, const uint8_t* D, const float* alpha,
                              const float* X, float* Y, int64_t N, int64_t M, int B,
                              hipStream_t stream) {
  static int cap_slot = 0;
  const int cap = bl_resident_wgs((const void*)bitdelta_kernel, kBdThreads, 4096, 1, &cap_slot);
  BdArgs a{};
  a.base = base;
  a.D = D;
  a.alpha = alpha;
  a.X = X;
  a.Y = Y;
  a.N = (int)N;
  a.M = (int)M;
  a.B = B;
  a.S = (int)((M + kBdWaveCodes - 1) / kBdWaveCodes);
  a.nwg = plan::bd_plan(N, a.S, cap, &a.R);
  const size_t lds = bd_lds_bytes(a.R, a.S);
  if (lds > kBdLdsMax) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bitdelta_kernel, dim3((unsigned)a.nwg), dim3(kBdThreads), lds, stream, a);
  return hipGetLastError();
}
