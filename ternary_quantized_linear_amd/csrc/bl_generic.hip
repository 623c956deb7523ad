// bl_generic.hip -- the ternary x int8 product for any K % 4 == 0 and any T: one
// thread per output, codes decoded byte by byte. It serves shapes the tiled kernels
// do not (K not a multiple of 64/128/256, unaligned tails) and is a second, simpler
// GPU path that the tiled kernels are compared with.
//
// [HF-1.58] "Computation paradigm": acc = sum over k of x_k * q_k with q in {-1,0,1};
// [bitnet.cpp] "3. BitLinear operation": Y = acc * beta / s_t.
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {

__global__ __launch_bounds__(256) void generic_kernel(bl_proj_internal p, int T) {
  const int o = (int)blockIdx.x * 256 + (int)threadIdx.x;
  const int t = (int)blockIdx.y;
  if (o >= p.N || t >= T) return;
  const uint8_t* w = p.W + (int64_t)o * (p.K >> 2);
  const int8_t* x = p.Xq + (int64_t)t * p.K;
  int acc = 0;
  for (int j = 0; j < (p.K >> 2); ++j) {
    const unsigned b = w[j];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = (int)((b >> (2 * i)) & 3u) - 1;
      acc += (int)x[4 * j + i] * q;
    }
  }
  const float f = p.w_scale[o / p.rpg] / p.x_scale[t];
  p.Y[(int64_t)t * p.N + o] = (float)acc * f;
  if (p.acc) p.acc[(int64_t)t * p.N + o] = acc;
}

// 1-bit sign codes ([bitnet.cpp] "1. Weight binarization"): bit i of byte j is code
// 8j+i, +1 when set, -1 otherwise; K % 8 == 0.
__global__ __launch_bounds__(256) void generic_sign_kernel(bl_proj_internal p, int T) {
  const int o = (int)blockIdx.x * 256 + (int)threadIdx.x;
  const int t = (int)blockIdx.y;
  if (o >= p.N || t >= T) return;
  const uint8_t* w = p.W + (int64_t)o * (p.K >> 3);
  const int8_t* x = p.Xq + (int64_t)t * p.K;
  int acc = 0;
  for (int j = 0; j < (p.K >> 3); ++j) {
    const unsigned b = w[j];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = ((b >> i) & 1u) ? 1 : -1;
      acc += (int)x[8 * j + i] * c;
    }
  }
  const float f = p.w_scale[0] / p.x_scale[t];
  p.Y[(int64_t)t * p.N + o] = (float)acc * f;
  if (p.acc) p.acc[(int64_t)t * p.N + o] = acc;
}

}  // namespace bl

hipError_t bl_launch_generic_sign(const bl_proj_internal* p, int T, hipStream_t stream) {
  dim3 grid((unsigned)((p->N + 255) / 256), (unsigned)T);
  hipLaunchKernelGGL(bl::generic_sign_kernel, grid, dim3(256), 0, stream, *p, T);
  return hipGetLastError();
}

hipError_t bl_launch_generic(const bl_proj_internal* p, int T, hipStream_t stream) {
  dim3 grid((unsigned)((p->N + 255) / 256), (unsigned)T);
  hipLaunchKernelGGL(bl::generic_kernel, grid, dim3(256), 0, stream, *p, T);
  return hipGetLastError();
}
