// bl_roof.hip -- the two rooflines the BitLinear products are measured against, as
// kernels timed on the part itself: an HBM read stream and an int8 MFMA stream.
//
// [HF-1.58] "Fine-tuning LLMs to 1.58 bits", "Tiled matrix multiplication": the product
// is limited by memory bandwidth and redundant accesses, so the decode kernels are
// judged by the bytes per second a plain read of the same buffers reaches; the
// prefill GEMM ("a real dense contraction") by the int8 matrix-core rate.
//
// roof_read_kernel: reads up to 8 buffers (the projections of a layer, or one
// allocation) once, 16 bytes per lane and load, as 1 KiB blocks per wave over the
// concatenated block index, in one of four static schedules (the caller times each and
// takes the fastest as the roof), with nothing stored but one word per wave (so the
// loads are not removed).
//
// roof_mfma_kernel: each wave issues v_mfma_i32_32x32x32_i8 on eight independent
// accumulators (no operand traffic: the operands stay in registers), and records its
// start and end in two clocks, s_memtime (the shader clock) and s_memrealtime (a fixed
// 100 MHz counter), so the host can report the shader clock under matrix load.
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {

constexpr int kRoofThreads = 256;
constexpr int kRoofBufs = 8;

struct RoofReadArgs {
  const uint4* buf[kRoofBufs];
  int64_t first[kRoofBufs + 1];  // first 1 KiB block of each buffer; first[count] = total
  int64_t n16[kRoofBufs];        // 16-byte pieces of each buffer
  int count;
  uint32_t* sink;
};

typedef const RoofReadArgs __attribute__((address_space(4)))* RoofArgsPtr;

// Buffer of concatenated block b (uniform per wave) and the load of lane `lane` of it.
__device__ __forceinline__ void roof_block(RoofArgsPtr a, int count, int64_t b, int lane,
                                           uint32_t& x) {
  int i = 0;
#pragma unroll
  for (int j = 1; j < kRoofBufs; ++j) i += (j < count && b >= a->first[j]) ? 1 : 0;
  i = __builtin_amdgcn_readfirstlane(i);
  const int64_t piece = (b - a->first[i]) * kWave + lane;
  if (piece < a->n16[i]) {
    const uint4 v = load_stream(a->buf[i] + piece);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
}

// Schedules (all read every byte once):
//   0: block b goes to wave b mod W (grid-stride), one block in flight per wave;
//   1: the same with D = 2 blocks in flight;
//   2: wave w reads the contiguous blocks [w * per, (w + 1) * per), 2 in flight;
//   3: (one buffer) as 0 without the per-block buffer lookup and lane guard.
template <int SCHED>
__global__ __launch_bounds__(kRoofThreads) void roof_read_kernel(RoofReadArgs) {
  // the arguments are indexed in place in the kernel-argument segment (a copy of the
  // struct indexed by a computed buffer number would live in scratch memory)
  const RoofArgsPtr a = (RoofArgsPtr)__builtin_amdgcn_kernarg_segment_ptr();
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t nw = (int64_t)gridDim.x * (kRoofThreads / kWave);
  const int64_t w = (int64_t)blockIdx.x * (kRoofThreads / kWave) + (threadIdx.x >> 6);
  const int count = a->count;
  const int64_t total = a->first[count];
  uint32_t x = 0;
  if constexpr (SCHED == 0) {
    for (int64_t b = w; b < total; b += nw) roof_block(a, count, b, lane, x);
  } else if constexpr (SCHED == 3) {
    // one buffer: whole blocks grid-stride with no per-block lookup or lane guard, the
    // partial last block (if any) by the wave that would take it
    const uint4* buf = a->buf[0];
    const int64_t n16 = a->n16[0], full = n16 / kWave;
    for (int64_t b = w; b < full; b += nw) {
      const uint4 v = load_stream(buf + b * kWave + lane);
      x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (full * kWave < n16 && w == full % nw && full * kWave + lane < n16) {
      const uint4 v = load_stream(buf + full * kWave + lane);
      x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  } else if constexpr (SCHED == 1) {
    int64_t b = w;
    for (; b + nw < total; b += 2 * nw) {
      uint32_t x0 = 0, x1 = 0;
      roof_block(a, count, b, lane, x0);
      roof_block(a, count, b + nw, lane, x1);
      x ^= x0 ^ x1;
    }
    if (b < total) roof_block(a, count, b, lane, x);
  } else {
    const int64_t per = (total + nw - 1) / nw;
    int64_t b = w * per;
    const int64_t e = min(total, b + per);
    for (; b + 1 < e; b += 2) {
      uint32_t x0 = 0, x1 = 0;
      roof_block(a, count, b, lane, x0);
      roof_block(a, count, b + 1, lane, x1);
      x ^= x0 ^ x1;
    }
    if (b < e) roof_block(a, count, b, lane, x);
  }
  // one word per wave: the xor of what it read
  x = (uint32_t)__builtin_amdgcn_readfirstlane((int)x) ^ (uint32_t)lane;
  if (lane == 0) a->sink[w] = x;
}

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(kRoofThreads) void roof_mfma_kernel(int iters, int32_t* sink,
                                                                 uint64_t* clocks) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t w = (int64_t)blockIdx.x * (kRoofThreads / kWave) + (threadIdx.x >> 6);
  const v4i a = v4i{lane, lane + 1, lane + 2, lane + 3};
  const v4i b = v4i{3 * lane, lane ^ 5, lane + 7, lane * 11};
  v16i acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = j + r;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[j], 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  sink[w * kWave + lane] = s;
  if (lane == 0) {
    clocks[4 * w] = t0;
    clocks[4 * w + 1] = t1;
    clocks[4 * w + 2] = r0;
    clocks[4 * w + 3] = r1;
  }
}

}  // namespace bl

using namespace bl;

size_t bl_roof_read_sink_words(int64_t total_bytes) {
  (void)total_bytes;
  return (size_t)4096 * (kRoofThreads / kWave);
}

hipError_t bl_launch_roof_read(const void* const* bufs, const int64_t* bytes, int count,
                               int schedule, uint32_t* sink, hipStream_t stream) {
  RoofReadArgs a{};
  int64_t blocks = 0;
  for (int i = 0; i < count; ++i) {
    a.buf[i] = static_cast<const uint4*>(bufs[i]);
    a.first[i] = blocks;
    a.n16[i] = bytes[i] / 16;
    blocks += (a.n16[i] + kWave - 1) / kWave;
  }
  a.first[count] = blocks;
  a.count = count;
  a.sink = sink;
  // 4096 workgroups of 4 waves with one block in flight per wave, or 1024 with two
  switch (schedule) {
    case 0: hipLaunchKernelGGL(roof_read_kernel<0>, dim3(4096), dim3(kRoofThreads), 0, stream, a); break;
    case 1: hipLaunchKernelGGL(roof_read_kernel<1>, dim3(1024), dim3(kRoofThreads), 0, stream, a); break;
    case 3:
      if (count == 1) {
        hipLaunchKernelGGL(roof_read_kernel<3>, dim3(4096), dim3(kRoofThreads), 0, stream, a);
        break;
      }
      hipLaunchKernelGGL(roof_read_kernel<0>, dim3(4096), dim3(kRoofThreads), 0, stream, a);
      break;
    default: hipLaunchKernelGGL(roof_read_kernel<2>, dim3(1024), dim3(kRoofThreads), 0, stream, a); break;
  }
  return hipGetLastError();
}

hipError_t bl_launch_roof_mfma(int iters, int wgs, int32_t* sink, uint64_t* clocks,
                               hipStream_t stream) {
  hipLaunchKernelGGL(roof_mfma_kernel, dim3((unsigned)wgs), dim3(kRoofThreads), 0, stream, iters,
                     sink, clocks);
  return hipGetLastError();
}
