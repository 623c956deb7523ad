// bl_train.hip -- the training side of BitLinear: fake quantization of the weights with
// the warm-up lambda, and the backward of the RMSNorm in front of the activation
// quantizer (the quantizers themselves pass gradients through unchanged).
//
// [HF-1.58] "Fine-tuning LLMs to 1.58 bits": "Training with the straight-through
// estimator (STE)": round() has no useful gradient; its gradient is taken as 1, so the
// gradient with respect to a quantizer's input is the gradient with respect to its
// output. "Dynamic warm-up quantization": lambda = min(step / total_steps, 1) scales
// the difference between the quantized and the original values, x + lambda (Q(x) - x).
// "How quantization works": quantized weights are rescaled back, beta * q.
//
// fq_weights_kernel: W_lam = bf16(w + lam * (beta * q - w)), q the ternary code of the
// forward quantizer (one fp32 product by fp32(1/beta), rint, clamp), every step one
// fp32 rounding (no contraction). HBM-bound: 4 bytes in, 2 out per weight.
// rmsnorm_bwd_kernel: one workgroup per token: c = sum_k g_k dy_k x_k in fp64, then
// dx_k = r g_k dy_k - x_k r^3 c / K in fp64, rounded once. dgain_kernel: one thread per
// feature, dg_k = sum_t r_t dy_tk x_tk in fp64.
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {

__global__ __launch_bounds__(256) void fq_weights_kernel(const float4* __restrict__ W4, int64_t n4,
                                                          const float* __restrict__ w_scale,
                                                          float lam, uint2* __restrict__ out) {
  const float beta = w_scale[0];
  const bool zero = !(beta >= 1.17549435e-38f);  // beta < FLT_MIN: every code is 0
  const float s = 1.0f / beta;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    const float4 f = W4[i];
    const float w[4] = {f.x, f.y, f.z, f.w};
    uint32_t h[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float q = zero ? 0.0f : fminf(fmaxf(rintf(w[c] * s), -1.0f), 1.0f);
      const float wq = q * beta;  // exact: q in {-1, 0, 1}
      const float d = wq - w[c];
      const float t = lam * d;
      h[c] = bf16_bits(w[c] + t);
    }
    out[i] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  }
}

constexpr int kBwdThreads = 256;

__global__ __launch_bounds__(kBwdThreads) void rmsnorm_bwd_kernel(
    const float* __restrict__ X, const float* __restrict__ gain, const double* __restrict__ rinv,
    const float* __restrict__ dY, int K, float* __restrict__ dX) {
  __shared__ double part[kBwdThreads / kWave];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const float* x = X + (int64_t)t * K;
  const float* dy = dY + (int64_t)t * K;
  double c = 0.0;
  for (int k = threadIdx.x; k < K; k += kBwdThreads) {
    const double g = gain ? (double)gain[k] : 1.0;
    c += g * (double)dy[k] * (double)x[k];
  }
  for (int m = 32; m >= 1; m >>= 1) c += __shfl_xor(c, m, kWave);
  if (lane == 0) part[wave] = c;
  __syncthreads();
  c = 0.0;
#pragma unroll
  for (int w = 0; w < kBwdThreads / kWave; ++w) c += part[w];
  const double r = rinv[t];
  const double b = r * r * r * c / (double)K;
  float* dx = dX + (int64_t)t * K;
  for (int k = threadIdx.x; k < K; k += kBwdThreads) {
    const double g = gain ? (double)gain[k] : 1.0;
    dx[k] = (float)(r * g * (double)dy[k] - (double)x[k] * b);
  }
}

__global__ __launch_bounds__(256) void dgain_kernel(const float* __restrict__ X,
                                                     const double* __restrict__ rinv,
                                                     const float* __restrict__ dY, int T, int K,
                                                     float* __restrict__ dgain) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  double acc = 0.0;
  for (int t = 0; t < T; ++t)
    acc += rinv[t] * (double)dY[(int64_t)t * K + k] * (double)X[(int64_t)t * K + k];
  dgain[k] = (float)acc;
}

}  // namespace bl

using namespace bl;

hipError_t bl_launch_fake_quant_weights(const float* W, int64_t N, int64_t K, const float* w_scale,
                                        float lam, uint16_t* out, hipStream_t stream) {
  const int64_t n4 = N * K / 4;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(fq_weights_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const float4*>(W), n4, w_scale, lam,
                     reinterpret_cast<uint2*>(out));
  return hipGetLastError();
}

hipError_t bl_launch_rmsnorm_backward(const float* X, const float* gain, const double* rinv,
                                      const float* dY, int64_t T, int64_t K, float* dX,
                                      float* dgain, hipStream_t stream) {
  hipLaunchKernelGGL(rmsnorm_bwd_kernel, dim3((unsigned)T), dim3(kBwdThreads), 0, stream, X, gain,
                     rinv, dY, (int)K, dX);
  if (dgain)
    hipLaunchKernelGGL(dgain_kernel, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, stream, X,
                       rinv, dY, (int)T, (int)K, dgain);
  return hipGetLastError();
}
