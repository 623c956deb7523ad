// bl_gemv.hip -- decode GEMV for T <= 2 tokens: packed ternary weights x int8
// activations with int8 dot4 (v_dot4c_i32_i8), int32 accumulation, fused rescale.
//
// [HF-1.58] "Fine-tuning LLMs to 1.58 bits", "Computation paradigm": the ternary
// product needs only integer additions; "Inference optimization and custom kernels":
// the 2-bit weights are unpacked on the fly inside the product; "Tiled matrix
// multiplication": memory bandwidth is the bottleneck. [bitnet.cpp] "3. BitLinear
// operation": the integer product is rescaled by the weight scale and the activation
// dequantization factor.
//
// Design (gfx950, wave64):
//   - A workgroup (4 waves) owns a block of rows of one projection. It first stages the
//     T activation rows into LDS, each 16-byte group 4x4 byte-transposed so that a
//     dword of activations lines up with a dword of unpacked codes (transpose16 /
//     unpack_u2), and sums each token's int8 values (sum_x).
//   - A row of K codes is K/4 bytes = C chunks of 16 bytes (64 codes). L lanes cover a
//     row (L = 64, 32 or 16, the largest that divides C), each lane streaming I = C/L
//     chunks with 128-bit loads; 64/L rows are in flight per wave instruction.
//   - Codes are used as u = q + 1 in {0, 1, 2} (no sign fix-up in the loop); the
//     product is corrected once per row: acc = sum x*u - sum_x.
//   - The L partial sums are reduced with DPP; Y = fp32(acc) * fp32(beta / s_t).
// Several projections (for example the seven of a decoder layer, which read four
// different inputs) go in one launch: the grid is the concatenation of their row
// blocks.
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / kWave;

struct GemvProj {
  const int8_t* Xq;
  const float* xs;
  const uint4* W;
  const float* ws;
  float* Y;
  int32_t* acc;
  int N, K;
  int blk0;     // first block index of this projection in the grid
  int rows_pb;  // rows per block
  int cfg;      // row-mapping variant (see gemv_kernel)
};

struct GemvArgs {
  GemvProj p[BL_GROUP_CAP];
  int count;
};

template <class E, int CAP>
__device__ __forceinline__ E pick(const E (&arr)[CAP], int idx) {
  E r = arr[0];
#pragma unroll
  for (int i = 1; i < CAP; ++i)
    if (i == idx) r = arr[i];
  return r;
}

// LDS layout of the staged activations: token t starts at byte t * (K + 16); inside a
// token the 16-byte group 4c + d (chunk c, sub-group d) sits at slot d * C + c, so that
// lanes reading consecutive chunks hit consecutive 16-byte slots.
__device__ __forceinline__ int xslot(int t, int c, int d, int C, int tstride16) {
  return t * tstride16 + d * C + c;
}

template <int TT>
__device__ __forceinline__ void stage_acts(const GemvProj& P, uint4* xl, int* sums) {
  const int K = P.K, G = K >> 4, C = K >> 6, ts16 = G + 1;
  int part[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) part[t] = 0;
  for (int g = threadIdx.x; g < TT * G; g += kGemvThreads) {
    const int t = g / G, gi = g - t * G;
    const uint4 v = reinterpret_cast<const uint4*>(P.Xq + (int64_t)t * K)[gi];
    const uint32_t a[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
    transpose16(a, o);
    xl[xslot(t, gi >> 2, gi & 3, C, ts16)] = make_uint4(o[0], o[1], o[2], o[3]);
    const int s = byte_sum(v.x) + byte_sum(v.y) + byte_sum(v.z) + byte_sum(v.w);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
      if (tt == t) part[tt] += s;
  }
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const int w = wave_sum_i32(part[t]);
    if ((threadIdx.x & (kWave - 1)) == 0) atomicAdd(&sums[t], w);
  }
}

template <int TT>
__device__ __forceinline__ void dot_chunk(const uint4 w, const uint4* xl, int c, int C,
                                          int ts16, int (&acc)[TT]) {
  const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t u[4];
    unpack_u2(words[d], u);
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const uint4 x = xl[xslot(t, c, d, C, ts16)];
      int a = acc[t];
      a = sdot4(u[0], x.x, a);
      a = sdot4(u[1], x.y, a);
      a = sdot4(u[2], x.z, a);
      a = sdot4(u[3], x.w, a);
      acc[t] = a;
    }
  }
}

template <int TT, int L>
__device__ __forceinline__ void finish_row(const GemvProj& P, int row, bool valid,
                                           const int (&acc)[TT], const int* sums,
                                           const float* fac) {
  const int j = threadIdx.x & (L - 1);
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const int tot = group_sum_to_last<L>(acc[t]);
    if (valid && j == L - 1) {
      const int a = tot - sums[t];
      P.Y[(int64_t)t * P.N + row] = (float)a * fac[t];
      if (P.acc) P.acc[(int64_t)t * P.N + row] = a;
    }
  }
}

// Fixed mapping: C == L * I chunks per row, R row groups per wave iteration.
template <int TT, int L, int I, int R>
__device__ __forceinline__ void rows_fixed(const GemvProj& P, int row0, int row1,
                                           const uint4* xl, const int* sums, const float* fac) {
  constexpr int RW = kWave / L;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int sub = lane / L, j = lane & (L - 1);
  const int C = P.K >> 6, ts16 = (P.K >> 4) + 1;
  for (int rg = row0 + wave * RW * R; rg < row1; rg += kGemvWaves * RW * R) {
    uint4 w[R][I];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min(rg + r * RW + sub, row1 - 1);
      const uint4* wr = P.W + (int64_t)row * C;
#pragma unroll
      for (int i = 0; i < I; ++i) w[r][i] = load_stream(wr + j + L * i);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int acc[TT];
#pragma unroll
      for (int t = 0; t < TT; ++t) acc[t] = 0;
#pragma unroll
      for (int i = 0; i < I; ++i) dot_chunk<TT>(w[r][i], xl, j + L * i, C, ts16, acc);
      const int row = rg + r * RW + sub;
      finish_row<TT, L>(P, row, row < row1, acc, sums, fac);
    }
  }
}

// Any K % 64 == 0: 64 lanes per row, ceil(C/64) masked iterations.
template <int TT>
__device__ __forceinline__ void rows_any(const GemvProj& P, int row0, int row1,
                                         const uint4* xl, const int* sums, const float* fac) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int C = P.K >> 6, ts16 = (P.K >> 4) + 1;
  for (int row = row0 + wave; row < row1; row += kGemvWaves) {
    int acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = 0;
    for (int c = lane; c < C; c += kWave) {
      const uint4 w = load_stream(P.W + (int64_t)row * C + c);
      dot_chunk<TT>(w, xl, c, C, ts16, acc);
    }
    finish_row<TT, 64>(P, row, true, acc, sums, fac);
  }
}

template <int TT>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(GemvArgs a) {
  extern __shared__ uint4 smem[];
  __shared__ int sums[TT];
  __shared__ float fac[TT];
  int pi = 0;
#pragma unroll
  for (int i = 1; i < BL_GROUP_CAP; ++i)
    if (i < a.count && (int)blockIdx.x >= a.p[i].blk0) pi = i;
  const GemvProj P = pick(a.p, pi);
  if (threadIdx.x < TT) {
    sums[threadIdx.x] = 0;
    fac[threadIdx.x] = P.ws[0] / P.xs[threadIdx.x];
  }
  __syncthreads();
  stage_acts<TT>(P, smem, sums);
  __syncthreads();
  const int row0 = ((int)blockIdx.x - P.blk0) * P.rows_pb;
  const int row1 = min(row0 + P.rows_pb, P.N);
  switch (P.cfg) {
    case 0: rows_fixed<TT, 64, 1, 4>(P, row0, row1, smem, sums, fac); break;  // C = 64
    case 1: rows_fixed<TT, 64, 2, 2>(P, row0, row1, smem, sums, fac); break;  // C = 128
    case 2: rows_fixed<TT, 32, 7, 1>(P, row0, row1, smem, sums, fac); break;  // C = 224
    case 3: rows_fixed<TT, 64, 7, 1>(P, row0, row1, smem, sums, fac); break;  // C = 448
    case 4: rows_fixed<TT, 16, 1, 4>(P, row0, row1, smem, sums, fac); break;  // C = 16
    case 5: rows_fixed<TT, 32, 1, 4>(P, row0, row1, smem, sums, fac); break;  // C = 32
    default: rows_any<TT>(P, row0, row1, smem, sums, fac); break;
  }
}

int gemv_cfg(int K) {
  switch (K >> 6) {
    case 64: return 0;
    case 128: return 1;
    case 224: return 2;
    case 448: return 3;
    case 16: return 4;
    case 32: return 5;
    default: return 6;
  }
}

// Rows per workgroup: about 64 KiB of packed weights, a multiple of 16 rows.
int gemv_rows_per_block(int K) {
  int r = (64 * 1024) / (K / 4);
  r = (r / 16) * 16;
  return r < 16 ? 16 : (r > 256 ? 256 : r);
}

constexpr int kGemvMaxLds = 96 * 1024;

// The dynamic-LDS limit is raised once per instance (the first launch on the device),
// so no attribute call happens inside a stream capture after that.
template <int TT>
hipError_t launch_gemv_t(dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                         const GemvArgs& a) {
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)gemv_kernel<TT>, hipFuncAttributeMaxDynamicSharedMemorySize, kGemvMaxLds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(gemv_kernel<TT>, grid, block, lds, stream, a);
  return hipGetLastError();
}

}  // namespace bl

using namespace bl;

bool bl_gemv_supports(int T, int K) {
  if (T < 1 || T > 2 || K % 64) return false;
  return (size_t)T * (K + 16) <= (size_t)kGemvMaxLds;
}

hipError_t bl_launch_gemv(const bl_proj_internal* p, int count, int T, hipStream_t stream) {
  GemvArgs a{};
  int blocks = 0, maxK = 0;
  for (int i = 0; i < count; ++i) {
    GemvProj& g = a.p[i];
    g.Xq = p[i].Xq;
    g.xs = p[i].x_scale;
    g.W = reinterpret_cast<const uint4*>(p[i].W);
    g.ws = p[i].w_scale;
    g.Y = p[i].Y;
    g.acc = p[i].acc;
    g.N = p[i].N;
    g.K = p[i].K;
    g.cfg = gemv_cfg(p[i].K);
    g.rows_pb = gemv_rows_per_block(p[i].K);
    g.blk0 = blocks;
    blocks += (p[i].N + g.rows_pb - 1) / g.rows_pb;
    if (p[i].K > maxK) maxK = p[i].K;
  }
  a.count = count;
  const size_t lds = (size_t)T * (maxK + 16);
  dim3 grid((unsigned)blocks), block(kGemvThreads);
  return T == 1 ? launch_gemv_t<1>(grid, block, lds, stream, a)
                : launch_gemv_t<2>(grid, block, lds, stream, a);
}
