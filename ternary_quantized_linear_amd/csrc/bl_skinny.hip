// bl_skinny.hip -- ternary x int8 product for 1 < T <= 64 tokens on int8 MFMA
// (v_mfma_i32_16x16x64_i8), int32 accumulation, fused rescale.
//
// [HF-1.58] "Fine-tuning LLMs to 1.58 bits", "Inference optimization and custom
// kernels": weights stay packed in memory and are unpacked inside the product;
// "Computation paradigm": integer arithmetic only. [bitnet.cpp] "3. BitLinear
// operation": rescale by the weight and activation scales.
//
// Below ~80 tokens the product is still bound by the packed-weight stream (2 ops per
// weight per token against 1/4 byte per weight), so each weight is read from HBM once
// and unpacked in registers, never staged:
//   - A workgroup (4 waves) owns 64*RB rows of one projection; each wave owns 16*RB
//     rows and all T tokens (TB blocks of 16).
//   - The K dimension is walked in chunks of KC codes. For each chunk the workgroup
//     stages the T activation rows into LDS (16-byte groups 4x4 byte-transposed to the
//     unpack order, token stride padded by 16 bytes against bank conflicts) and keeps
//     each token's sum of int8 values.
//   - Per 256 codes a lane loads 16 bytes of its row (lane % 16 = row, lane / 16 = which
//     64 codes), i.e. one 128-bit load feeds four MFMAs; the dword of 16 codes becomes
//     the A operand as u = q + 1 (unpack_u2); the B operand is the matching 16 bytes of
//     a token from LDS. The MFMA output is corrected once: acc = D - sum_x.
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kSkThreads = 256;
constexpr int kSkWaves = kSkThreads / kWave;
constexpr int kSkRB = 2;                 // 16-row blocks per wave
constexpr int kSkRows = kSkWaves * 16 * kSkRB;
constexpr size_t kSkLdsBudget = 72 * 1024;

struct SkProj {
  const int8_t* Xq;
  const float* xs;
  const uint8_t* W;
  const float* ws;
  float* Y;
  int32_t* acc;
  int N, K;
  int blk0;
  int KC;  // codes per staged chunk (multiple of 256, divides K)
};

struct SkArgs {
  SkProj p[BL_GROUP_CAP];
  int count;
  int T;
};

template <class E, int CAP>
__device__ __forceinline__ E pick_sk(const E (&arr)[CAP], int idx) {
  E r = arr[0];
#pragma unroll
  for (int i = 1; i < CAP; ++i)
    if (i == idx) r = arr[i];
  return r;
}

template <int TB>
__global__ __launch_bounds__(kSkThreads) void skinny_kernel(SkArgs a) {
  extern __shared__ uint4 xl[];
  __shared__ int sums[64];
  __shared__ float fac[64];
  int pi = 0;
#pragma unroll
  for (int i = 1; i < BL_GROUP_CAP; ++i)
    if (i < a.count && (int)blockIdx.x >= a.p[i].blk0) pi = i;
  const SkProj P = pick_sk(a.p, pi);
  const int T = a.T;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  if (tid < 64) {
    sums[tid] = 0;
    fac[tid] = tid < T ? P.ws[0] / P.xs[tid] : 0.0f;
  }
  const int rowbase = ((int)blockIdx.x - P.blk0) * kSkRows + wave * 16 * kSkRB;
  const int Kb = P.K >> 2;
  const int KC = P.KC, C = KC >> 6, G = KC >> 4, ts16 = G + 1;
  const uint8_t* wrow[kSkRB];
#pragma unroll
  for (int rb = 0; rb < kSkRB; ++rb)
    wrow[rb] = P.W + (int64_t)min(rowbase + rb * 16 + li, P.N - 1) * Kb + 16 * lg;

  v4i acc[kSkRB][TB];
#pragma unroll
  for (int rb = 0; rb < kSkRB; ++rb)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[rb][tb] = v4i{0, 0, 0, 0};

  for (int kc = 0; kc < P.K; kc += KC) {
    __syncthreads();  // LDS of the previous chunk fully read
    for (int t = wave; t < T; t += kSkWaves) {
      const uint4* src = reinterpret_cast<const uint4*>(P.Xq + (int64_t)t * P.K + kc);
      int part = 0;
      for (int gi = lane; gi < G; gi += kWave) {
        const uint4 v = src[gi];
        const uint32_t in[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[4];
        transpose16(in, o);
        xl[t * ts16 + (gi & 3) * C + (gi >> 2)] = make_uint4(o[0], o[1], o[2], o[3]);
        part += byte_sum(v.x) + byte_sum(v.y) + byte_sum(v.z) + byte_sum(v.w);
      }
      part = wave_sum_i32(part);
      if (lane == 0) sums[t] += part;
    }
    __syncthreads();
    const int nsteps = KC >> 8;
    const int kb0 = kc >> 2;
    for (int s = 0; s < nsteps; ++s) {
      uint4 wv[kSkRB];
#pragma unroll
      for (int rb = 0; rb < kSkRB; ++rb)
        wv[rb] = *reinterpret_cast<const uint4*>(wrow[rb] + kb0 + 64 * s);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        v4i xf[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
          const int tok = 16 * tb + li;
          if (tok < T) {
            const uint4 x = xl[tok * ts16 + m * C + 4 * s + lg];
            xf[tb] = v4i{(int)x.x, (int)x.y, (int)x.z, (int)x.w};
          } else {
            xf[tb] = v4i{0, 0, 0, 0};
          }
        }
#pragma unroll
        for (int rb = 0; rb < kSkRB; ++rb) {
          const uint32_t word = m == 0 ? wv[rb].x : m == 1 ? wv[rb].y : m == 2 ? wv[rb].z : wv[rb].w;
          uint32_t u[4];
          unpack_u2(word, u);
          const v4i ua = v4i{(int)u[0], (int)u[1], (int)u[2], (int)u[3]};
#pragma unroll
          for (int tb = 0; tb < TB; ++tb)
            acc[rb][tb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ua, xf[tb], acc[rb][tb], 0, 0, 0);
        }
      }
    }
  }
  // D[row][token]: lane holds rows 4*lg + r (r = 0..3) of the block, token li.
#pragma unroll
  for (int rb = 0; rb < kSkRB; ++rb)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int tok = 16 * tb + li;
      if (tok >= T) continue;
      const int sx = sums[tok];
      const float f = fac[tok];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rowbase + rb * 16 + 4 * lg + r;
        if (row < P.N) {
          const int v = acc[rb][tb][r] - sx;
          P.Y[(int64_t)tok * P.N + row] = (float)v * f;
          if (P.acc) P.acc[(int64_t)tok * P.N + row] = v;
        }
      }
    }
}

int skinny_chunk(int T, int K) {
  const int units = K / 256;
  int best = 1;
  for (int d = 1; d <= units; ++d)
    if (units % d == 0 && (size_t)T * (256 * d + 16) <= kSkLdsBudget) best = d;
  return 256 * best;
}

// The dynamic-LDS limit is raised once per instance (first launch), never inside a
// stream capture after that.
template <int TB>
hipError_t launch_skinny_t(dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                           const SkArgs& a) {
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)skinny_kernel<TB>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSkLdsBudget);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(skinny_kernel<TB>, grid, block, lds, stream, a);
  return hipGetLastError();
}

}  // namespace bl

using namespace bl;

bool bl_skinny_supports(int T, int K) { return T >= 1 && T <= 64 && K % 256 == 0; }

hipError_t bl_launch_skinny(const bl_proj_internal* p, int count, int T, hipStream_t stream) {
  SkArgs a{};
  int blocks = 0;
  size_t lds = 0;
  for (int i = 0; i < count; ++i) {
    SkProj& s = a.p[i];
    s.Xq = p[i].Xq;
    s.xs = p[i].x_scale;
    s.W = p[i].W;
    s.ws = p[i].w_scale;
    s.Y = p[i].Y;
    s.acc = p[i].acc;
    s.N = p[i].N;
    s.K = p[i].K;
    s.KC = skinny_chunk(T, p[i].K);
    s.blk0 = blocks;
    blocks += (p[i].N + kSkRows - 1) / kSkRows;
    size_t need = (size_t)T * (s.KC + 16);
    if (need > lds) lds = need;
  }
  a.count = count;
  a.T = T;
  dim3 grid((unsigned)blocks), block(kSkThreads);
  switch ((T + 15) / 16) {
    case 1: return launch_skinny_t<1>(grid, block, lds, stream, a);
    case 2: return launch_skinny_t<2>(grid, block, lds, stream, a);
    case 3: return launch_skinny_t<3>(grid, block, lds, stream, a);
    default: return launch_skinny_t<4>(grid, block, lds, stream, a);
  }
}
