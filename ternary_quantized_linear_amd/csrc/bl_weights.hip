// bl_weights.hip -- absmean ternary weight quantization and 2-bit packing on gfx950.
//
// [HF-1.58] "Fine-tuning LLMs to 1.58 bits" (Hugging Face post summary), "How
// quantization works", weights: one scale per tensor, the reciprocal of the mean
// absolute value; weights are scaled, rounded and clamped to [-1, 1]. [b1.58] "The Era
// of 1-bit LLMs" review, "Proposed method": absmean quantization. [HF-1.58] "Key
// findings": four ternary codes per int8.
//
// Three launches, no host synchronization:
//   1. wq_abssum: every workgroup sums |w| over a grid-stride share of W EXACTLY, as an
//      integer in units of 2^-149 (the fp32 denormal step): |w| = m * 2^sh with a 24-bit
//      m. A wave loads 1024 values, finds its largest sh, and adds m << (sh - base) into
//      64-bit lane accumulators for the values within 36 binades of that maximum
//      (sixteen values below 2^60 cannot overflow 2^64). The wave total is added, as
//      32-bit digits, into a long accumulator in LDS (one uint64 per digit, carries
//      deferred); values further below go into the same accumulator one by one. The
//      workgroup's digits go to the workspace. This is Kulisch's long-accumulator
//      idea with a floating window in front of it.
//   2. wq_finalize: one workgroup adds the workgroups' digits, propagates carries, and rounds
//      the exact integer once to fp64 (round to nearest, ties to even): S. Then
//      gamma = S / (N*K) in fp64 and beta = fp32(gamma).
//   3. wq_pack: codes q = clamp(rint(w * fp32(1/beta)), -1, 1) (one fp32 product, rint
//      rounds half to even), u = q + 1 packed four per byte, code k = 4j+i in bits
//      [2i+1:2i] of byte j. beta < FLT_MIN gives all codes 0.
// The sum is exact, so gamma and the codes do not depend on the grid, the launch
// order or the hardware scheduling.
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {

constexpr int kSumThreads = 256;
constexpr int kSumWaves = kSumThreads / kWave;
constexpr int kSumMaxBlocks = 1024;
constexpr int kDigits = 12;  // 32-bit digits: 384 bits >= 2^277 * 2^40 magnitudes
constexpr int kWindow = 36;  // binades covered by the 64-bit lane accumulators

// Adds v (< 2^40) at bit position pos of the long accumulator.
__device__ __forceinline__ void lacc_add(unsigned long long* dig, unsigned long long v,
                                         int pos) {
  int d = pos >> 5, o = pos & 31;
  unsigned long long lo = v << o;
  unsigned long long hi = o ? (v >> (64 - o)) : 0ull;
  unsigned long long d0 = lo & 0xFFFFFFFFull, d1 = lo >> 32;
  if (d0) atomicAdd(&dig[d], d0);
  if (d1) atomicAdd(&dig[d + 1], d1);
  if (hi) atomicAdd(&dig[d + 2], hi);
}

__device__ __forceinline__ void split_abs(float x, unsigned& m, int& sh) {
  unsigned b = __float_as_uint(x) & 0x7FFFFFFFu;
  unsigned e = b >> 23;
  if (e == 0xFFu) e = 0xFEu;  // Inf/NaN: result unspecified, but keep indices in range
  m = (b & 0x7FFFFFu) | (e ? 0x800000u : 0u);
  sh = e ? (int)e - 1 : 0;
}

__global__ __launch_bounds__(kSumThreads) void wq_abssum(const float4* __restrict__ W4,
                                                         int64_t n4,
                                                         unsigned long long* __restrict__ ws) {
  __shared__ unsigned long long dig[kDigits];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  if (tid < kDigits) dig[tid] = 0ull;
  __syncthreads();

  const int64_t nchunks = (n4 + 255) / 256;  // a chunk = 256 float4 = 1024 values
  const int64_t wave_id = (int64_t)blockIdx.x * kSumWaves + wave;
  const int64_t nwaves = (int64_t)gridDim.x * kSumWaves;
  for (int64_t c = wave_id; c < nchunks; c += nwaves) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int64_t i = c * 256 + j * 64 + lane;
      float4 f = i < n4 ? W4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      v[4 * j + 0] = f.x; v[4 * j + 1] = f.y; v[4 * j + 2] = f.z; v[4 * j + 3] = f.w;
    }
    unsigned m[16];
    int sh[16];
    int top = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      split_abs(v[j], m[j], sh[j]);
      top = (m[j] && sh[j] > top) ? sh[j] : top;
    }
    top = (int)wave_max_u32((unsigned)top);
    const int base = top > kWindow ? top - kWindow : 0;
    unsigned long long acc = 0ull;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (m[j] == 0u) continue;
      if (sh[j] >= base) acc += (unsigned long long)m[j] << (sh[j] - base);
      else lacc_add(dig, m[j], sh[j]);  // more than 36 binades below the wave's top
    }
    unsigned long long slo = wave_sum_u64(acc & 0xFFFFFFFFull);
    unsigned long long shi = wave_sum_u64(acc >> 32);
    if (lane == 0) {
      lacc_add(dig, slo, base);
      lacc_add(dig, shi, base + 32);
    }
  }
  __syncthreads();
  if (tid < kDigits) ws[(int64_t)blockIdx.x * kDigits + tid] = dig[tid];
}

__global__ __launch_bounds__(kSumThreads) void wq_finalize(const unsigned long long* __restrict__ ws,
                                                           int nblocks, int64_t count,
                                                           float* __restrict__ w_scale,
                                                           double* __restrict__ w_gamma) {
  __shared__ unsigned long long part[kDigits][kSumWaves];
  __shared__ unsigned long long col[kDigits];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  // digit columns summed over the workgroups' records: every thread a share of the
  // records (independent loads), then the waves, then the four wave partials
  unsigned long long s[kDigits];
#pragma unroll
  for (int d = 0; d < kDigits; ++d) s[d] = 0ull;
  for (int b = tid; b < nblocks; b += kSumThreads)
#pragma unroll
    for (int d = 0; d < kDigits; ++d) s[d] += ws[(int64_t)b * kDigits + d];
#pragma unroll
  for (int d = 0; d < kDigits; ++d) {
    const unsigned long long v = wave_sum_u64(s[d]);
    if (lane == 0) part[d][wave] = v;
  }
  __syncthreads();
  if (tid < kDigits) {
    unsigned long long c = 0ull;
#pragma unroll
    for (int w = 0; w < kSumWaves; ++w) c += part[tid][w];
    col[tid] = c;
  }
  __syncthreads();
  if (tid != 0) return;
  // carry propagation into plain 32-bit digits
  constexpr int kBig = kDigits + 3;
  unsigned big[kBig];
  unsigned long long carry = 0ull;
  for (int d = 0; d < kBig; ++d) {
    unsigned long long t = (d < kDigits ? col[d] : 0ull) + carry;
    big[d] = (unsigned)(t & 0xFFFFFFFFull);
    carry = t >> 32;
  }
  int top = -1;  // index of the most significant set bit
  for (int d = kBig - 1; d >= 0 && top < 0; --d)
    if (big[d]) top = 32 * d + 31 - __clz((int)big[d]);
  double S = 0.0;
  if (top >= 0) {
    auto bit = [&](int p) -> unsigned { return p < 0 ? 0u : (big[p >> 5] >> (p & 31)) & 1u; };
    unsigned long long mant = 0ull;
    int lsb = top - 52;  // position of the last kept bit
    for (int p = top; p >= lsb; --p) mant = (mant << 1) | bit(p);
    if (lsb > 0) {
      unsigned rbit = bit(lsb - 1);
      bool sticky = false;
      for (int p = lsb - 2; p >= 0 && !sticky; --p) sticky = bit(p) != 0u;
      if (rbit && (sticky || (mant & 1ull))) {
        ++mant;
        if (mant == (1ull << 53)) { mant >>= 1; ++lsb; }
      }
    }
    // value = mant * 2^lsb in units of 2^-149 (lsb < 0 only when top < 52: mant is then
    // the exact integer shifted left, and lsb compensates)
    S = ldexp((double)mant, lsb - 149);
  }
  double gamma = S / (double)count;
  w_scale[0] = (float)gamma;
  if (w_gamma) w_gamma[0] = gamma;
}

__global__ __launch_bounds__(256) void wq_pack(const float4* __restrict__ W4, int64_t n4,
                                               const float* __restrict__ w_scale,
                                               uint8_t* __restrict__ P) {
  const float beta = w_scale[0];
  const bool zero = !(beta >= 1.17549435e-38f);  // beta < FLT_MIN: every code is 0
  const float s = 1.0f / beta;                     // IEEE division (correctly rounded)
  const int64_t stride = (int64_t)gridDim.x * 1024;
  for (int64_t b = (int64_t)blockIdx.x * 1024 + threadIdx.x; b < n4; b += stride) {
    float4 f[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int64_t i = b + 256 * j;
      f[j] = i < n4 ? W4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int64_t i = b + 256 * j;
      if (i >= n4) break;
      float w[4] = {f[j].x, f[j].y, f[j].z, f[j].w};
      unsigned byte = 0u;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float t = w[c] * s;
        float r = fminf(fmaxf(rintf(t), -1.0f), 1.0f);
        int u = zero ? 1 : (int)r + 1;
        byte |= (unsigned)u << (2 * c);
      }
      P[i] = (uint8_t)byte;
    }
  }
}

}  // namespace bl

using namespace bl;

size_t bl_weight_workspace_bytes_impl(int64_t N, int64_t K) {
  (void)N;
  (void)K;
  return (size_t)kSumMaxBlocks * kDigits * sizeof(unsigned long long);
}

hipError_t bl_launch_quantize_weights(const float* W, int64_t N, int64_t K, uint8_t* P,
                                      float* w_scale, double* w_gamma, void* ws,
                                      hipStream_t stream) {
  const int64_t n = N * K;
  const int64_t n4 = n / 4;  // K % 4 == 0, so n % 4 == 0
  const int64_t nchunks = (n4 + 255) / 256;
  int64_t blocks = (nchunks + kSumWaves - 1) / kSumWaves;
  if (blocks > kSumMaxBlocks) blocks = kSumMaxBlocks;
  if (blocks < 1) blocks = 1;
  auto* dig = static_cast<unsigned long long*>(ws);
  hipLaunchKernelGGL(wq_abssum, dim3((unsigned)blocks), dim3(kSumThreads), 0, stream,
                     reinterpret_cast<const float4*>(W), n4, dig);
  hipLaunchKernelGGL(wq_finalize, dim3(1), dim3(kSumThreads), 0, stream, dig, (int)blocks, n,
                     w_scale, w_gamma);
  int64_t pblocks = (n4 + 1023) / 1024;
  if (pblocks > 4096) pblocks = 4096;
  if (pblocks < 1) pblocks = 1;
  hipLaunchKernelGGL(wq_pack, dim3((unsigned)pblocks), dim3(256), 0, stream,
                     reinterpret_cast<const float4*>(W), n4, w_scale, P);
  return hipGetLastError();
}
