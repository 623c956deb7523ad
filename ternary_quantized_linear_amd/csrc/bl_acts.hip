// bl_acts.hip -- fused RMSNorm + per-token absmax int8 activation quantization.
//
// [b1.58] "The Era of 1-bit LLMs" review, "Proposed method": RMSNorm (LLaMA-style
// blocks). [HF-1.58] "Fine-tuning LLMs to 1.58 bits", "How quantization works",
// activations: a normalization before the quantizer, then absmax per token into
// [-128, 127]. [bitnet.cpp] "Microsoft's inference framework brings 1-bit LLMs to local
// devices", "2. Activation quantization": the scale comes from ||x||_inf and a small
// epsilon keeps it finite.
//
// One workgroup per token row (grid.y = entry of a grouped call). Per row:
//   ss  = sum x^2: each square exact in fp64, accumulated in double-double per lane,
//         across lanes and waves with double-double adds, rounded once to fp64
//   r   = 1 / sqrt(ss / K + eps)                   (fp64, IEEE division and sqrt)
//   y_k = fp32((x_k * r) * g_k)                    (fp64 products; no g without gain)
//   s_t = 127 / max(max|y|, 1e-5)                  (fp32 IEEE division)
//   q_k = clamp(rint(y_k * s_t), -128, 127)        (one fp32 product, half to even)
// With the row in registers (VPT float4 per lane) X is read from HBM once; rows too
// long for registers take the streaming variant, which reads X three times.
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {

struct ActEntry {
  const float* X;
  const float* gain;
  int8_t* Xq;
  float* s;
  uint16_t* xfq;  // training side: bf16 of y + lam * (Xq / s - y), or null
  double* rinv;   // training side: r per token, or null
  int K;
};

struct ActArgs {
  ActEntry e[BL_GROUP_CAP];
  int T;
  float eps;
  int no_norm;
  float lam;
};

__device__ __forceinline__ int code_of(float v, float s) {
  return (int)fminf(fmaxf(rintf(v * s), -128.0f), 127.0f);
}

// Training side ([HF-1.58] "Dynamic warm-up quantization", "How quantization works"):
// y + lam * (q / s - y) with q / s one fp32 division and every step one fp32 rounding
// (no contraction), then bf16. q / s is read from a table of the 256 quotients of the
// row: each entry is that IEEE division, done once per row instead of once per element.
__device__ __forceinline__ uint32_t fq_tab(float y, float s, float lam, const float* quot) {
  const float d = quot[code_of(y, s) + 128] - y;
  const float t = lam * d;
  return bf16_bits(y + t);
}

__device__ __forceinline__ uint2 fq4_tab(float4 y, float s, float lam, const float* quot) {
  const uint32_t a = fq_tab(y.x, s, lam, quot), b = fq_tab(y.y, s, lam, quot);
  const uint32_t c = fq_tab(y.z, s, lam, quot), d = fq_tab(y.w, s, lam, quot);
  return make_uint2(a | (b << 16), c | (d << 16));
}

// quot[i] = fp32(i - 128) / s for the 256 codes, by the workgroup's threads; the caller
// synchronizes before the table is read.
template <int NT>
__device__ __forceinline__ void fill_quot(float* quot, float s) {
  for (int i = threadIdx.x; i < 256; i += NT) quot[i] = (float)(i - 128) / s;
}

// Block-wide double-double sum. Each wave reduces its lanes with DPP into lane 63; after
// one barrier every wave reduces the per-wave partials itself (DPP over the first NW
// lanes, zeros beyond), in the same order, so all waves hold the same bits without a
// second barrier. The second level takes only the steps that NW lanes need (2 for 4
// waves, 3 for 8): the steps it leaves out would add zero pairs, which changes nothing.
template <int NT>
__device__ __forceinline__ void block_dd_sum(double& hi, double& lo, double* sh_hi,
                                             double* sh_lo) {
  constexpr int NW = NT / kWave;
  constexpr int NL = NW < 4 ? 4 : NW;  // lanes of the second level
  static_assert(NW <= 16, "partials are combined within one DPP row");
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  group_dd_sum_to_last<kWave>(hi, lo);
  if (lane == kWave - 1) { sh_hi[wave] = hi; sh_lo[wave] = lo; }
  __syncthreads();
  hi = lane < NW ? sh_hi[lane] : 0.0;
  lo = lane < NW ? sh_lo[lane] : 0.0;
  group_dd_sum_to_last<NL>(hi, lo);
  const double h = readlane_f64(hi, NL - 1), l = readlane_f64(lo, NL - 1);
  hi = h;
  lo = l;
}

// The double-double sum and the maximum of non-negative values together: both wave
// reductions (independent chains), one LDS round and one barrier, then both second levels.
template <int NT>
__device__ __forceinline__ void block_dd_sum_max(double& hi, double& lo, float& mx, double* sh_hi,
                                                 double* sh_lo, float* sh_m) {
  constexpr int NW = NT / kWave;
  constexpr int NL = NW < 4 ? 4 : NW;
  static_assert(NW <= 16, "partials are combined within one DPP row");
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  group_dd_sum_to_last<kWave>(hi, lo);
  mx = group_max_to_last<kWave>(mx);
  if (lane == kWave - 1) {
    sh_hi[wave] = hi;
    sh_lo[wave] = lo;
    sh_m[wave] = mx;
  }
  __syncthreads();
  hi = lane < NW ? sh_hi[lane] : 0.0;
  lo = lane < NW ? sh_lo[lane] : 0.0;
  float m = lane < NW ? sh_m[lane] : 0.0f;
  group_dd_sum_to_last<NL>(hi, lo);
  m = group_max_to_last<NL>(m);
  const double h = readlane_f64(hi, NL - 1), l = readlane_f64(lo, NL - 1);
  hi = h;
  lo = l;
  mx = readlane_f32(m, NL - 1);
}

// Block-wide maximum of non-negative values, same structure.
template <int NT>
__device__ __forceinline__ float block_max(float v, float* sh) {
  constexpr int NW = NT / kWave;
  constexpr int NL = NW < 4 ? 4 : NW;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  v = group_max_to_last<kWave>(v);
  if (lane == kWave - 1) sh[wave] = v;
  __syncthreads();
  float m = lane < NW ? sh[lane] : 0.0f;
  m = group_max_to_last<NL>(m);
  return readlane_f32(m, NL - 1);
}

// Squares of fp32 values are exact in fp64. Four independent cascaded sums (one per
// float4 component) keep four dependency chains in flight; they meet at the end.
// Every term and every running sum is non-negative, so the larger of the two addends
// is also the larger in magnitude and Dekker's fast two-sum on (max, min) gives the
// exact rounding error: the same sum and error as Knuth's two-sum, in 5 operations
// instead of 6.
struct SumSq4 {
  double h[4] = {0.0, 0.0, 0.0, 0.0}, l[4] = {0.0, 0.0, 0.0, 0.0};
  __device__ __forceinline__ void add(float4 f) {
    const double d[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const double b = d[c] * d[c];
      const double big = fmax(h[c], b), small = fmin(h[c], b);
      const double s = big + small;
      l[c] += small - (s - big);
      h[c] = s;
    }
  }
  // one renormalized double-double pair
  __device__ __forceinline__ void total(double& hi, double& lo) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const double s = h[c] + l[c];
      l[c] = l[c] - (s - h[c]);
      h[c] = s;
    }
    dd_add(h[0], l[0], h[1], l[1]);
    dd_add(h[2], l[2], h[3], l[3]);
    dd_add(h[0], l[0], h[2], l[2]);
    hi = h[0];
    lo = l[0];
  }
};

__device__ __forceinline__ float norm_one(float x, double r, float g, bool has_gain) {
  double v = (double)x * r;
  if (has_gain) v = v * (double)g;
  return (float)v;
}

__device__ __forceinline__ float4 norm4(float4 x, double r, float4 g, bool has_gain) {
  return make_float4(norm_one(x.x, r, g.x, has_gain), norm_one(x.y, r, g.y, has_gain),
                     norm_one(x.z, r, g.z, has_gain), norm_one(x.w, r, g.w, has_gain));
}

// Four codes clamp(round(y * s), -128, 127) as bytes. The clamp comes first (its bounds
// are integers, so the order does not change the result); adding 1.5 * 2^23 then rounds
// to the nearest integer, ties to even, and leaves its two's-complement byte in the low
// byte of the sum's bits (the spacing of floats in [2^23, 2^24) is 1).
__device__ __forceinline__ uint32_t quant4(float4 y, float s) {
  auto q = [&](float v) -> uint32_t {
    return __float_as_uint(__builtin_amdgcn_fmed3f(v * s, -128.0f, 127.0f) + 12582912.0f);
  };
  const uint32_t lo = __builtin_amdgcn_perm(q(y.y), q(y.x), 0x0C0C0400u);  // x, y, 0, 0
  const uint32_t hi = __builtin_amdgcn_perm(q(y.w), q(y.z), 0x04000C0Cu);  // 0, 0, z, w
  return lo | hi;
}

// Row held in registers: lane i owns float4 i, i+NT, ..., i+(VPT-1)NT of the row. GAIN:
// the instance for calls with a gain (it holds the gain's float4 as well).
template <int NT, int VPT, bool FQ, bool GAIN>
__global__ __launch_bounds__(NT) void act_quant_reg(ActArgs a) {
  __shared__ double sh_hi[NT / kWave], sh_lo[NT / kWave];
  __shared__ float sh_m[NT / kWave];
  const ActEntry& e = a.e[blockIdx.y];
  const int t = blockIdx.x;
  const int K4 = e.K >> 2;
  const float4* x4 = reinterpret_cast<const float4*>(e.X + (int64_t)t * e.K);
  const bool has_gain = GAIN && e.gain != nullptr && !a.no_norm;
  const float4* g4 = reinterpret_cast<const float4*>(e.gain);
  // the row is loaded once, up front; the gain (shared by every row, so cache-resident)
  // only where the norm needs it, which keeps it out of the registers that hold the row
  float4 v[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    int i = threadIdx.x + j * NT;
    v[j] = i < K4 ? x4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (!a.no_norm && !has_gain && !FQ) {
    // Without a gain, y = fp32(fp64(x) * r) is two roundings of a product that grows with
    // |x|, each rounding monotone and odd, so max|y| = fp32(fp64(max|x|) * r) exactly: the
    // maximum rides with the sum of squares through one block reduction (one barrier
    // instead of two), and y is formed where it is quantized.
    SumSq4 acc;
    float mx = 0.0f;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      acc.add(v[j]);
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
    }
    double hi, lo;
    acc.total(hi, lo);
    block_dd_sum_max<NT>(hi, lo, mx, sh_hi, sh_lo, sh_m);
    const double r = 1.0 / sqrt(hi / (double)e.K + (double)a.eps);
    const float s = 127.0f / fmaxf((float)((double)mx * r), 1e-5f);
    uint32_t* q4 = reinterpret_cast<uint32_t*>(e.Xq + (int64_t)t * e.K);
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      int i = threadIdx.x + j * NT;
      if (i < K4) q4[i] = quant4(norm4(v[j], r, make_float4(1.f, 1.f, 1.f, 1.f), false), s);
    }
    if (threadIdx.x == 0) e.s[t] = s;
    return;
  }
  if (!a.no_norm) {
    SumSq4 acc;
#pragma unroll
    for (int j = 0; j < VPT; ++j) acc.add(v[j]);
    // With a gain and room in the registers, the gain's float4 are all asked for here, so
    // that they arrive during the block reduction (loaded where the norm uses them, each
    // load is waited for before the next is issued: seven round trips for a row of 14336)
    constexpr bool kPre = GAIN && VPT <= 8;
    float4 gv[kPre ? VPT : 1];
    if (kPre && has_gain) {
#pragma unroll
      for (int j = 0; j < (kPre ? VPT : 0); ++j) gv[j] = g4[min((int)threadIdx.x + j * NT, K4 - 1)];
    }
    double hi, lo;
    acc.total(hi, lo);
    block_dd_sum<NT>(hi, lo, sh_hi, sh_lo);
    const double ss = hi;  // hi + lo is already rounded into hi by dd_add
    const double r = 1.0 / sqrt(ss / (double)e.K + (double)a.eps);
    if (has_gain) {
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        int i = threadIdx.x + j * NT;
        if constexpr (kPre) v[j] = norm4(v[j], r, gv[j], true);  // lanes past K4 store nothing
        else v[j] = norm4(v[j], r, i < K4 ? g4[i] : make_float4(1.f, 1.f, 1.f, 1.f), true);
      }
    } else {
#pragma unroll
      for (int j = 0; j < VPT; ++j) v[j] = norm4(v[j], r, make_float4(1.f, 1.f, 1.f, 1.f), false);
    }
    if (FQ && e.rinv && threadIdx.x == 0) e.rinv[t] = r;
  } else if (FQ && e.rinv && threadIdx.x == 0) {
    e.rinv[t] = 1.0;
  }
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < VPT; ++j)
    m = fmaxf(m, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
  m = block_max<NT>(m, sh_m);
  const float s = 127.0f / fmaxf(m, 1e-5f);
  uint32_t* q4 = reinterpret_cast<uint32_t*>(e.Xq + (int64_t)t * e.K);
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    int i = threadIdx.x + j * NT;
    if (i < K4) q4[i] = quant4(v[j], s);
  }
  if constexpr (FQ) {
    if (e.xfq) {
      __shared__ float quot[256];
      fill_quot<NT>(quot, s);
      __syncthreads();
      uint2* f2 = reinterpret_cast<uint2*>(e.xfq + (int64_t)t * e.K);
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        int i = threadIdx.x + j * NT;
        if (i < K4) f2[i] = fq4_tab(v[j], s, a.lam, quot);
      }
    }
  }
  if (threadIdx.x == 0) e.s[t] = s;
}

// Rows longer than the register budget: three passes over X (L2-resident by then).
template <int NT, bool FQ>
__global__ __launch_bounds__(NT) void act_quant_stream(ActArgs a) {
  __shared__ double sh_hi[NT / kWave], sh_lo[NT / kWave];
  __shared__ float sh_m[NT / kWave];
  const ActEntry& e = a.e[blockIdx.y];
  const int t = blockIdx.x;
  const int K4 = e.K >> 2;
  const float4* x4 = reinterpret_cast<const float4*>(e.X + (int64_t)t * e.K);
  const bool has_gain = e.gain != nullptr && !a.no_norm;
  const float4* g4 = reinterpret_cast<const float4*>(e.gain);
  double r = 1.0;
  if (!a.no_norm) {
    SumSq4 acc;
    for (int i = threadIdx.x; i < K4; i += NT) acc.add(x4[i]);
    double hi, lo;
    acc.total(hi, lo);
    block_dd_sum<NT>(hi, lo, sh_hi, sh_lo);
    r = 1.0 / sqrt(hi / (double)e.K + (double)a.eps);
  }
  if (FQ && e.rinv && threadIdx.x == 0) e.rinv[t] = r;
  auto load_y = [&](int i) -> float4 {
    const float4 f = x4[i];
    if (a.no_norm) return f;
    return norm4(f, r, has_gain ? g4[i] : make_float4(1.f, 1.f, 1.f, 1.f), has_gain);
  };
  float m = 0.0f;
  for (int i = threadIdx.x; i < K4; i += NT) {
    float4 y = load_y(i);
    m = fmaxf(m, fmaxf(fmaxf(fabsf(y.x), fabsf(y.y)), fmaxf(fabsf(y.z), fabsf(y.w))));
  }
  m = block_max<NT>(m, sh_m);
  const float s = 127.0f / fmaxf(m, 1e-5f);
  uint32_t* q4 = reinterpret_cast<uint32_t*>(e.Xq + (int64_t)t * e.K);
  __shared__ float quot[FQ ? 256 : 1];
  if constexpr (FQ) {
    if (e.xfq) {
      fill_quot<NT>(quot, s);
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < K4; i += NT) {
    const float4 y = load_y(i);
    q4[i] = quant4(y, s);
    if constexpr (FQ) {
      if (e.xfq) reinterpret_cast<uint2*>(e.xfq + (int64_t)t * e.K)[i] = fq4_tab(y, s, a.lam, quot);
    }
  }
  if (threadIdx.x == 0) e.s[t] = s;
}

}  // namespace bl

using namespace bl;

namespace {

template <bool FQ, bool G>
hipError_t launch_acts_g(const ActArgs& a, int maxK, int64_t T, int count, hipStream_t stream) {
  dim3 grid((unsigned)T, (unsigned)count);
  const int f4 = (maxK + 3) / 4;  // float4 per row
  if (T <= 64) {
    // Few rows: latency-bound, each row on one CU, whose four SIMDs do all of its fp64
    // arithmetic. The fewest waves that hold the row: every wave repeats the block
    // reductions, so 512 lanes beat 1024 (4-input decode call 4.6 us against 5.3 us,
    // same bits), and 256 lanes suit rows of up to 4096 (2.8 us against 3.1). Rows of
    // 14336 (the MLP down projection's input) take an instance that fits them exactly
    // (7 float4 per lane; with 8 the last eighth of the unrolled work is on zeros):
    // the 4-input decode call 4.91 -> 4.66 us together with the shorter second
    // reduction level and the fast two-sum.
    if (f4 <= 256) hipLaunchKernelGGL((act_quant_reg<256, 1, FQ, G>), grid, dim3(256), 0, stream, a);
    else if (f4 <= 512) hipLaunchKernelGGL((act_quant_reg<256, 2, FQ, G>), grid, dim3(256), 0, stream, a);
    else if (f4 <= 1024) hipLaunchKernelGGL((act_quant_reg<256, 4, FQ, G>), grid, dim3(256), 0, stream, a);
    else if (f4 <= 2048) hipLaunchKernelGGL((act_quant_reg<512, 4, FQ, G>), grid, dim3(512), 0, stream, a);
    else if (f4 <= 3584) hipLaunchKernelGGL((act_quant_reg<512, 7, FQ, G>), grid, dim3(512), 0, stream, a);
    else if (f4 <= 4096) hipLaunchKernelGGL((act_quant_reg<512, 8, FQ, G>), grid, dim3(512), 0, stream, a);
    else if (f4 <= 8192) hipLaunchKernelGGL((act_quant_reg<512, 16, FQ, G>), grid, dim3(512), 0, stream, a);
    else hipLaunchKernelGGL((act_quant_stream<1024, FQ>), grid, dim3(1024), 0, stream, a);
    return hipGetLastError();
  }
  // many rows: throughput-bound; the smallest register footprint that holds the row
  if (f4 <= 256) hipLaunchKernelGGL((act_quant_reg<256, 1, FQ, G>), grid, dim3(256), 0, stream, a);
  else if (f4 <= 512) hipLaunchKernelGGL((act_quant_reg<256, 2, FQ, G>), grid, dim3(256), 0, stream, a);
  else if (f4 <= 1024) hipLaunchKernelGGL((act_quant_reg<256, 4, FQ, G>), grid, dim3(256), 0, stream, a);
  else if (f4 <= 2048) hipLaunchKernelGGL((act_quant_reg<256, 8, FQ, G>), grid, dim3(256), 0, stream, a);
  else if (f4 <= 4096) hipLaunchKernelGGL((act_quant_reg<512, 8, FQ, G>), grid, dim3(512), 0, stream, a);
  else if (f4 <= 8192) hipLaunchKernelGGL((act_quant_reg<512, 16, FQ, G>), grid, dim3(512), 0, stream, a);
  else hipLaunchKernelGGL((act_quant_stream<1024, FQ>), grid, dim3(1024), 0, stream, a);
  return hipGetLastError();
}

// the gain instances when an entry has a gain and the norm is on
template <bool FQ>
hipError_t launch_acts(const ActArgs& a, int maxK, int64_t T, int count, hipStream_t stream) {
  bool gain = false;
  for (int i = 0; i < count; ++i) gain = gain || (a.e[i].gain != nullptr && !a.no_norm);
  return gain ? launch_acts_g<FQ, true>(a, maxK, T, count, stream)
              : launch_acts_g<FQ, false>(a, maxK, T, count, stream);
}

}  // namespace

hipError_t bl_launch_quantize_acts(const bl_act_desc* d, int count, int64_t T, float eps,
                                   uint32_t flags, hipStream_t stream) {
  ActArgs a{};
  int maxK = 0;
  for (int i = 0; i < count; ++i) {
    a.e[i] = ActEntry{d[i].X, d[i].gain, d[i].Xq, d[i].x_scale, nullptr, nullptr, (int)d[i].K};
    if ((int)d[i].K > maxK) maxK = (int)d[i].K;
  }
  a.T = (int)T;
  a.eps = eps;
  a.no_norm = (flags & BL_NO_NORM) ? 1 : 0;
  a.lam = 0.0f;
  return launch_acts<false>(a, maxK, T, count, stream);
}

hipError_t bl_launch_fake_quant_acts(const float* X, const float* gain, int64_t T, int64_t K,
                                     float eps, uint32_t flags, float lam, int8_t* Xq, float* xs,
                                     uint16_t* xfq, double* rinv, hipStream_t stream) {
  ActArgs a{};
  a.e[0] = ActEntry{X, gain, Xq, xs, xfq, rinv, (int)K};
  a.T = (int)T;
  a.eps = eps;
  a.no_norm = (flags & BL_NO_NORM) ? 1 : 0;
  a.lam = lam;
  return launch_acts<true>(a, (int)K, T, 1, stream);
}
