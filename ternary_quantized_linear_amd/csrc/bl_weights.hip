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
//
// The 1-bit sign variant ([bitnet.cpp] "1. Weight binarization", the original BitNet:
// W_f = Sign(W - alpha) with alpha the mean of W, Sign(x) = +1 for x > 0 and -1
// otherwise; [BitDelta] Eq. (2) states the same rule, Eq. (4) gives mean |W| as the
// scale of a sign code) runs the same three steps: wq_abssum<true> also sums the
// magnitudes of the negative weights into a second long accumulator, wq_finalize<true>
// forms the exact signed sum (all - 2 * negatives) and rounds it once to fp64:
// alpha = sum / (N*K) in fp64, beta = fp32(mean |W|) as above. wq_pack1 sets bit i of
// byte j (code k = 8j+i) when fp64(w) > alpha, an exact comparison.
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

// SIGNED: a second accumulator (neg) collects |w| of the negative weights.
// DIFF: the values summed are fp32(w - base), base given as bf16 bits (BitDelta deltas).
template <bool SIGNED, bool DIFF = false>
__global__ __launch_bounds__(kSumThreads) void wq_abssum(const float4* __restrict__ W4,
                                                         int64_t n4,
                                                         unsigned long long* __restrict__ ws,
                                                         const uint2* __restrict__ base4) {
  constexpr int ND = SIGNED ? 2 * kDigits : kDigits;
  __shared__ unsigned long long dig[ND];
  unsigned long long* neg = dig + kDigits;  // used only when SIGNED
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  if (tid < ND) dig[tid] = 0ull;
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
      if constexpr (DIFF) {
        const uint2 b = i < n4 ? base4[i] : make_uint2(0u, 0u);
        f.x = f.x - __uint_as_float(b.x << 16);
        f.y = f.y - __uint_as_float(b.x & 0xFFFF0000u);
        f.z = f.z - __uint_as_float(b.y << 16);
        f.w = f.w - __uint_as_float(b.y & 0xFFFF0000u);
      }
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
    unsigned long long acc = 0ull, accn = 0ull;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (m[j] == 0u) continue;
      const bool isneg = SIGNED && v[j] < 0.0f;
      if (sh[j] >= base) {
        const unsigned long long t = (unsigned long long)m[j] << (sh[j] - base);
        acc += t;
        if (isneg) accn += t;
      } else {  // more than 36 binades below the wave's top
        lacc_add(dig, m[j], sh[j]);
        if (isneg) lacc_add(neg, m[j], sh[j]);
      }
    }
    unsigned long long slo = wave_sum_u64(acc & 0xFFFFFFFFull);
    unsigned long long shi = wave_sum_u64(acc >> 32);
    if (lane == 0) {
      lacc_add(dig, slo, base);
      lacc_add(dig, shi, base + 32);
    }
    if constexpr (SIGNED) {
      unsigned long long nlo = wave_sum_u64(accn & 0xFFFFFFFFull);
      unsigned long long nhi = wave_sum_u64(accn >> 32);
      if (lane == 0) {
        lacc_add(neg, nlo, base);
        lacc_add(neg, nhi, base + 32);
      }
    }
  }
  __syncthreads();
  if (tid < ND) ws[(int64_t)blockIdx.x * ND + tid] = dig[tid];
}

constexpr int kBig = kDigits + 3;  // carried 32-bit digits

// Column sums (uint64 per digit, carries deferred) -> plain 32-bit digits.
__device__ void carry_digits(const unsigned long long* col, unsigned* big) {
  unsigned long long carry = 0ull;
  for (int d = 0; d < kBig; ++d) {
    unsigned long long t = (d < kDigits ? col[d] : 0ull) + carry;
    big[d] = (unsigned)(t & 0xFFFFFFFFull);
    carry = t >> 32;
  }
}

// The integer in big (units of 2^-149) rounded once to fp64, ties to even.
__device__ double round_digits(const unsigned* big) {
  int top = -1;  // index of the most significant set bit
  for (int d = kBig - 1; d >= 0 && top < 0; --d)
    if (big[d]) top = 32 * d + 31 - __clz((int)big[d]);
  if (top < 0) return 0.0;
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
  return ldexp((double)mant, lsb - 149);
}

// Sums the workgroups' digit records (ND digits each): every thread a share of the
// records (independent loads), then the waves, then the four wave partials. Then
// thread 0 rounds: gamma = S / count (and, SIGNED, alpha = signed sum / count, stored
// at ws_alpha for the packing kernel and at w_alpha when given).
template <bool SIGNED>
__global__ __launch_bounds__(kSumThreads) void wq_finalize(const unsigned long long* __restrict__ ws,
                                                           int nblocks, int64_t count,
                                                           float* __restrict__ w_scale,
                                                           double* __restrict__ w_gamma,
                                                           double* __restrict__ ws_alpha,
                                                           double* __restrict__ w_alpha) {
  constexpr int ND = SIGNED ? 2 * kDigits : kDigits;
  __shared__ unsigned long long part[ND][kSumWaves];
  __shared__ unsigned long long col[ND];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  unsigned long long s[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) s[d] = 0ull;
  for (int b = tid; b < nblocks; b += kSumThreads)
#pragma unroll
    for (int d = 0; d < ND; ++d) s[d] += ws[(int64_t)b * ND + d];
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    const unsigned long long v = wave_sum_u64(s[d]);
    if (lane == 0) part[d][wave] = v;
  }
  __syncthreads();
  if (tid < ND) {
    unsigned long long c = 0ull;
#pragma unroll
    for (int w = 0; w < kSumWaves; ++w) c += part[tid][w];
    col[tid] = c;
  }
  __syncthreads();
  if (tid != 0) return;
  unsigned big[kBig];
  carry_digits(col, big);
  const double gamma = round_digits(big) / (double)count;
  w_scale[0] = (float)gamma;
  if (w_gamma) w_gamma[0] = gamma;
  if constexpr (SIGNED) {
    // signed sum = all - 2 * negatives, as sign and magnitude
    unsigned nb[kBig], two[kBig];
    carry_digits(col + kDigits, nb);
    unsigned c = 0u;
    for (int d = 0; d < kBig; ++d) {
      two[d] = (nb[d] << 1) | c;
      c = nb[d] >> 31;
    }
    int cmp = 0;
    for (int d = kBig - 1; d >= 0 && cmp == 0; --d)
      cmp = big[d] > two[d] ? 1 : (big[d] < two[d] ? -1 : 0);
    const unsigned* hi = cmp >= 0 ? big : two;
    const unsigned* lo = cmp >= 0 ? two : big;
    unsigned mag[kBig];
    long long borrow = 0;
    for (int d = 0; d < kBig; ++d) {
      long long t = (long long)hi[d] - (long long)lo[d] - borrow;
      borrow = t < 0 ? 1 : 0;
      mag[d] = (unsigned)(t + (borrow << 32));
    }
    const double m = round_digits(mag);
    const double alpha = (cmp >= 0 ? m : -m) / (double)count;
    ws_alpha[0] = alpha;
    if (w_alpha) w_alpha[0] = alpha;
  }
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

// Eight sign codes per byte: bit i of byte j is code 8j+i, set when fp64(w) > alpha.
// Thread b writes packed dword b (32 codes = 8 float4).
__global__ __launch_bounds__(256) void wq_pack1(const float4* __restrict__ W4, int64_t ndw,
                                                const double* __restrict__ alpha_p,
                                                uint32_t* __restrict__ P) {
  const double alpha = alpha_p[0];
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < ndw; b += stride) {
    float4 f[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = W4[8 * b + j];
    uint32_t word = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float w[4] = {f[j].x, f[j].y, f[j].z, f[j].w};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        word |= ((double)w[c] > alpha ? 1u : 0u) << (4 * j + c);
    }
    P[b] = word;
  }
}

// Bytes of the last partial dword (n % 32 codes), one thread each.
__global__ void wq_pack1_tail(const float* __restrict__ W, int64_t n,
                              const double* __restrict__ alpha_p, uint8_t* __restrict__ P) {
  const double alpha = alpha_p[0];
  const int64_t first = (n / 32) * 4;  // first byte not written by wq_pack1
  const int64_t byte = first + threadIdx.x;
  if (byte >= n / 8) return;
  unsigned v = 0u;
  for (int i = 0; i < 8; ++i) v |= ((double)W[8 * byte + i] > alpha ? 1u : 0u) << i;
  P[byte] = (uint8_t)v;
}

// BitDelta signs ([BitDelta] Eq. (2): +1 where delta > 0, else -1) of one model into the
// batched layout: row n, 16-code group j, model slot `model` of 8: 2 bytes at
// ((n * (M/16) + j) * 8 + model) * 2, bit i of the pair = code 16j + i.
__global__ __launch_bounds__(256) void bd_pack(const float4* __restrict__ fine4,
                                               const uint2* __restrict__ base4, int64_t groups,
                                               int model, uint16_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < groups; g += stride) {
    uint32_t bits = 0u;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 f = fine4[4 * g + q];
      const uint2 b = base4[4 * g + q];
      const float d[4] = {f.x - __uint_as_float(b.x << 16), f.y - __uint_as_float(b.x & 0xFFFF0000u),
                          f.z - __uint_as_float(b.y << 16), f.w - __uint_as_float(b.y & 0xFFFF0000u)};
#pragma unroll
      for (int c = 0; c < 4; ++c) bits |= (d[c] > 0.0f ? 1u : 0u) << (4 * q + c);
    }
    out[g * 8 + model] = (uint16_t)bits;
  }
}

}  // namespace bl

using namespace bl;

// Digit records of both accumulators (the sign variant needs two), then alpha.
size_t bl_weight_workspace_bytes_impl(int64_t N, int64_t K) {
  (void)N;
  (void)K;
  return (size_t)kSumMaxBlocks * 2 * kDigits * sizeof(unsigned long long) + 256;
}

namespace {
int64_t sum_blocks(int64_t n4) {
  const int64_t nchunks = (n4 + 255) / 256;
  int64_t blocks = (nchunks + kSumWaves - 1) / kSumWaves;
  if (blocks > kSumMaxBlocks) blocks = kSumMaxBlocks;
  if (blocks < 1) blocks = 1;
  return blocks;
}
double* alpha_slot(void* ws) {
  return reinterpret_cast<double*>(static_cast<char*>(ws) +
                                   (size_t)kSumMaxBlocks * 2 * kDigits * sizeof(unsigned long long));
}
}  // namespace

hipError_t bl_launch_quantize_weights(const float* W, int64_t N, int64_t K, uint8_t* P,
                                      float* w_scale, double* w_gamma, void* ws,
                                      hipStream_t stream) {
  const int64_t n = N * K;
  const int64_t n4 = n / 4;  // K % 4 == 0, so n % 4 == 0
  const int64_t blocks = sum_blocks(n4);
  auto* dig = static_cast<unsigned long long*>(ws);
  hipLaunchKernelGGL((wq_abssum<false, false>), dim3((unsigned)blocks), dim3(kSumThreads), 0,
                     stream, reinterpret_cast<const float4*>(W), n4, dig, (const uint2*)nullptr);
  hipLaunchKernelGGL(wq_finalize<false>, dim3(1), dim3(kSumThreads), 0, stream, dig, (int)blocks,
                     n, w_scale, w_gamma, (double*)nullptr, (double*)nullptr);
  int64_t pblocks = (n4 + 1023) / 1024;
  if (pblocks > 4096) pblocks = 4096;
  if (pblocks < 1) pblocks = 1;
  hipLaunchKernelGGL(wq_pack, dim3((unsigned)pblocks), dim3(256), 0, stream,
                     reinterpret_cast<const float4*>(W), n4, w_scale, P);
  return hipGetLastError();
}

hipError_t bl_launch_quantize_weights_sign(const float* W, int64_t N, int64_t K, uint8_t* P,
                                           float* w_scale, double* w_alpha, void* ws,
                                           hipStream_t stream) {
  const int64_t n = N * K;
  const int64_t n4 = n / 4;  // K % 8 == 0
  const int64_t blocks = sum_blocks(n4);
  auto* dig = static_cast<unsigned long long*>(ws);
  hipLaunchKernelGGL((wq_abssum<true, false>), dim3((unsigned)blocks), dim3(kSumThreads), 0,
                     stream, reinterpret_cast<const float4*>(W), n4, dig, (const uint2*)nullptr);
  hipLaunchKernelGGL(wq_finalize<true>, dim3(1), dim3(kSumThreads), 0, stream, dig, (int)blocks,
                     n, w_scale, (double*)nullptr, alpha_slot(ws), w_alpha);
  const int64_t ndw = n / 32;  // packed dwords; K % 8 == 0 but n may not be a multiple of 32
  int64_t pblocks = (ndw + 255) / 256;
  if (pblocks > 4096) pblocks = 4096;
  if (pblocks < 1) pblocks = 1;
  if (ndw > 0)
    hipLaunchKernelGGL(wq_pack1, dim3((unsigned)pblocks), dim3(256), 0, stream,
                       reinterpret_cast<const float4*>(W), ndw, alpha_slot(ws),
                       reinterpret_cast<uint32_t*>(P));
  if (n % 32) {
    // the last few bytes (n % 32 = 8, 16 or 24 codes): one thread per byte
    hipLaunchKernelGGL(wq_pack1_tail, dim3(1), dim3(64), 0, stream, W, n, alpha_slot(ws), P);
  }
  return hipGetLastError();
}

hipError_t bl_launch_bitdelta_compress(const float* W_fine, const uint16_t* W_base, int64_t N,
                                       int64_t M, int model, uint8_t* D, float* alpha, void* ws,
                                       hipStream_t stream) {
  const int64_t n = N * M;
  const int64_t n4 = n / 4;  // M % 16 == 0
  const int64_t blocks = sum_blocks(n4);
  auto* dig = static_cast<unsigned long long*>(ws);
  hipLaunchKernelGGL((wq_abssum<false, true>), dim3((unsigned)blocks), dim3(kSumThreads), 0, stream,
                     reinterpret_cast<const float4*>(W_fine), n4, dig,
                     reinterpret_cast<const uint2*>(W_base));
  hipLaunchKernelGGL(wq_finalize<false>, dim3(1), dim3(kSumThreads), 0, stream, dig, (int)blocks,
                     n, alpha, (double*)nullptr, (double*)nullptr, (double*)nullptr);
  const int64_t groups = n / 16;
  int64_t pblocks = (groups + 255) / 256;
  if (pblocks > 4096) pblocks = 4096;
  hipLaunchKernelGGL(bd_pack, dim3((unsigned)pblocks), dim3(256), 0, stream,
                     reinterpret_cast<const float4*>(W_fine), reinterpret_cast<const uint2*>(W_base),
                     groups, model, reinterpret_cast<uint16_t*>(D));
  return hipGetLastError();
}
