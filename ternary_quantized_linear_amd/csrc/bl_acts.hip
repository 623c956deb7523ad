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
  int K;
};

struct ActArgs {
  ActEntry e[BL_GROUP_CAP];
  int T;
  float eps;
  int no_norm;
};

// Block-wide double-double sum. Each wave reduces its lanes with shuffles; after one
// barrier every wave reduces the per-wave partials itself, in the same order, so all
// waves hold the same bits without a second barrier.
template <int NT>
__device__ __forceinline__ void block_dd_sum(double& hi, double& lo, double* sh_hi,
                                             double* sh_lo) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    double oh = __shfl_xor(hi, m, kWave), ol = __shfl_xor(lo, m, kWave);
    dd_add(hi, lo, oh, ol);
  }
  if (lane == 0) { sh_hi[wave] = hi; sh_lo[wave] = lo; }
  __syncthreads();
  hi = lane < NW ? sh_hi[lane] : 0.0;
  lo = lane < NW ? sh_lo[lane] : 0.0;
#pragma unroll
  for (int m = NW / 2; m >= 1; m >>= 1) {
    double oh = __shfl_xor(hi, m, kWave), ol = __shfl_xor(lo, m, kWave);
    dd_add(hi, lo, oh, ol);
  }
  hi = __shfl(hi, 0, kWave);
  lo = __shfl(lo, 0, kWave);
}

template <int NT>
__device__ __forceinline__ float block_max(float v, float* sh) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  v = wave_max_f32(v);
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  float m = lane < NW ? sh[lane] : 0.0f;
#pragma unroll
  for (int k = NW / 2; k >= 1; k >>= 1) m = fmaxf(m, __shfl_xor(m, k, kWave));
  return __shfl(m, 0, kWave);
}

__device__ __forceinline__ float norm_one(float x, double r, const float* gain, int k) {
  double v = (double)x * r;
  if (gain) v = v * (double)gain[k];
  return (float)v;
}

__device__ __forceinline__ uint32_t quant4(float4 y, float s) {
  auto q = [&](float v) -> uint32_t {
    float t = fminf(fmaxf(rintf(v * s), -128.0f), 127.0f);
    return (uint32_t)((int)t & 0xFF);
  };
  return q(y.x) | (q(y.y) << 8) | (q(y.z) << 16) | (q(y.w) << 24);
}

// Row held in registers: lane i owns float4 i, i+NT, ..., i+(VPT-1)NT of the row.
template <int NT, int VPT>
__global__ __launch_bounds__(NT) void act_quant_reg(ActArgs a) {
  __shared__ double sh_hi[NT / kWave], sh_lo[NT / kWave];
  __shared__ float sh_m[NT / kWave];
  const ActEntry& e = a.e[blockIdx.y];
  const int t = blockIdx.x;
  const int K4 = e.K >> 2;
  const float4* x4 = reinterpret_cast<const float4*>(e.X + (int64_t)t * e.K);
  float4 v[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    int i = threadIdx.x + j * NT;
    v[j] = i < K4 ? x4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (!a.no_norm) {
    double hi = 0.0, lo = 0.0;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      double d0 = v[j].x, d1 = v[j].y, d2 = v[j].z, d3 = v[j].w;
      dd_add1(hi, lo, d0 * d0);
      dd_add1(hi, lo, d1 * d1);
      dd_add1(hi, lo, d2 * d2);
      dd_add1(hi, lo, d3 * d3);
    }
    // renormalize the lane pair before the cross-lane adds
    double s = hi + lo;
    lo = lo - (s - hi);
    hi = s;
    block_dd_sum<NT>(hi, lo, sh_hi, sh_lo);
    const double ss = hi;  // hi + lo is already rounded into hi by dd_add
    const double r = 1.0 / sqrt(ss / (double)e.K + (double)a.eps);
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      int i = threadIdx.x + j * NT;
      int k = 4 * i;
      if (i < K4) {
        v[j].x = norm_one(v[j].x, r, e.gain, k);
        v[j].y = norm_one(v[j].y, r, e.gain, k + 1);
        v[j].z = norm_one(v[j].z, r, e.gain, k + 2);
        v[j].w = norm_one(v[j].w, r, e.gain, k + 3);
      }
    }
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
  if (threadIdx.x == 0) e.s[t] = s;
}

// Rows longer than the register budget: three passes over X (L2-resident by then).
template <int NT>
__global__ __launch_bounds__(NT) void act_quant_stream(ActArgs a) {
  __shared__ double sh_hi[NT / kWave], sh_lo[NT / kWave];
  __shared__ float sh_m[NT / kWave];
  const ActEntry& e = a.e[blockIdx.y];
  const int t = blockIdx.x;
  const int K4 = e.K >> 2;
  const float4* x4 = reinterpret_cast<const float4*>(e.X + (int64_t)t * e.K);
  double r = 1.0;
  if (!a.no_norm) {
    double hi = 0.0, lo = 0.0;
    for (int i = threadIdx.x; i < K4; i += NT) {
      float4 f = x4[i];
      double d0 = f.x, d1 = f.y, d2 = f.z, d3 = f.w;
      dd_add1(hi, lo, d0 * d0);
      dd_add1(hi, lo, d1 * d1);
      dd_add1(hi, lo, d2 * d2);
      dd_add1(hi, lo, d3 * d3);
    }
    double s = hi + lo;
    lo = lo - (s - hi);
    hi = s;
    block_dd_sum<NT>(hi, lo, sh_hi, sh_lo);
    r = 1.0 / sqrt(hi / (double)e.K + (double)a.eps);
  }
  auto load_y = [&](int i) -> float4 {
    float4 f = x4[i];
    if (a.no_norm) return f;
    int k = 4 * i;
    return make_float4(norm_one(f.x, r, e.gain, k), norm_one(f.y, r, e.gain, k + 1),
                       norm_one(f.z, r, e.gain, k + 2), norm_one(f.w, r, e.gain, k + 3));
  };
  float m = 0.0f;
  for (int i = threadIdx.x; i < K4; i += NT) {
    float4 y = load_y(i);
    m = fmaxf(m, fmaxf(fmaxf(fabsf(y.x), fabsf(y.y)), fmaxf(fabsf(y.z), fabsf(y.w))));
  }
  m = block_max<NT>(m, sh_m);
  const float s = 127.0f / fmaxf(m, 1e-5f);
  uint32_t* q4 = reinterpret_cast<uint32_t*>(e.Xq + (int64_t)t * e.K);
  for (int i = threadIdx.x; i < K4; i += NT) q4[i] = quant4(load_y(i), s);
  if (threadIdx.x == 0) e.s[t] = s;
}

}  // namespace bl

using namespace bl;

hipError_t bl_launch_quantize_acts(const bl_act_desc* d, int count, int64_t T, float eps,
                                   uint32_t flags, hipStream_t stream) {
  ActArgs a{};
  int maxK = 0;
  for (int i = 0; i < count; ++i) {
    a.e[i] = ActEntry{d[i].X, d[i].gain, d[i].Xq, d[i].x_scale, (int)d[i].K};
    if ((int)d[i].K > maxK) maxK = (int)d[i].K;
  }
  a.T = (int)T;
  a.eps = eps;
  a.no_norm = (flags & BL_NO_NORM) ? 1 : 0;
  dim3 grid((unsigned)T, (unsigned)count);
  const int f4 = (maxK + 3) / 4;  // float4 per row
  if (T <= 64) {
    // few rows: latency-bound, so spread each row over 1024 lanes
    if (f4 <= 1024) hipLaunchKernelGGL((act_quant_reg<1024, 1>), grid, dim3(1024), 0, stream, a);
    else if (f4 <= 2048) hipLaunchKernelGGL((act_quant_reg<1024, 2>), grid, dim3(1024), 0, stream, a);
    else if (f4 <= 4096) hipLaunchKernelGGL((act_quant_reg<1024, 4>), grid, dim3(1024), 0, stream, a);
    else if (f4 <= 8192) hipLaunchKernelGGL((act_quant_reg<1024, 8>), grid, dim3(1024), 0, stream, a);
    else hipLaunchKernelGGL((act_quant_stream<1024>), grid, dim3(1024), 0, stream, a);
    return hipGetLastError();
  }
  // many rows: throughput-bound; the smallest register footprint that holds the row
  if (f4 <= 256) hipLaunchKernelGGL((act_quant_reg<256, 1>), grid, dim3(256), 0, stream, a);
  else if (f4 <= 512) hipLaunchKernelGGL((act_quant_reg<256, 2>), grid, dim3(256), 0, stream, a);
  else if (f4 <= 1024) hipLaunchKernelGGL((act_quant_reg<256, 4>), grid, dim3(256), 0, stream, a);
  else if (f4 <= 2048) hipLaunchKernelGGL((act_quant_reg<256, 8>), grid, dim3(256), 0, stream, a);
  else if (f4 <= 4096) hipLaunchKernelGGL((act_quant_reg<256, 16>), grid, dim3(256), 0, stream, a);
  else if (f4 <= 8192) hipLaunchKernelGGL((act_quant_reg<512, 16>), grid, dim3(512), 0, stream, a);
  else hipLaunchKernelGGL((act_quant_stream<1024>), grid, dim3(1024), 0, stream, a);
  return hipGetLastError();
}
