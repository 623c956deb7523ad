// bl_skinny.hip -- ternary x int8 product for 1 < T <= 64 tokens on int8 MFMA
// (v_mfma_i32_16x16x64_i8), int32 accumulation, fused rescale.
//
// [HF-1.58] "Fine-tuning LLMs to 1.58 bits", "Inference optimization and custom
// kernels": weights stay packed in memory and are unpacked inside the product;
// "Computation paradigm": integer arithmetic only. [bitnet.cpp] "3. BitLinear
// operation": rescale by the weight and activation scales.
//
// Below ~80 tokens the product is bound by the packed-weight stream (2 ops per weight per
// token against 1/4 byte per weight), so the kernel is built like the decode GEMV: every
// weight byte is read from HBM once, straight into registers, by waves that each keep a
// ring of loads in flight, with no barrier in the main loop.
//   - A row group is 16*RB weight rows (RB MFMA row blocks). A row group's K is cut into
//     S = 1, 2 or 4 contiguous segments of 256-code chunks, one per wave of the
//     workgroup; the S partial tiles meet in LDS (atomic adds and an arrival count; the
//     last wave writes the tile).
//   - Per chunk a lane loads 16 bytes of row (lane % 16) of each row block, codes
//     64*(lane/16) .. +63: one 128-bit load feeds four MFMAs, whose A operands are the
//     u = q + 1 codes of one dword each (unpack_u2, p-major order). The B operands are
//     the matching 16 activation bytes of token (lane % 16) + 16*tb, loaded from global
//     memory (L2) with the weights and 4x4 byte-transposed to the same order; tokens past
//     T reuse the last token's bytes and their output columns are dropped.
//   - sum x*u - sum x = sum x*q: the sum of the activations comes from one more MFMA per
//     B operand with an all-ones A, so the VALU only unpacks and transposes.
//   - Workgroups are partitioned among the projections of a grouped call in proportion
//     to their bytes; the grid is one round of resident workgroups.
// Output tile: MFMA lane l, register r holds row 4*(l/16) + r of the block, token l % 16.
#include "bl_device.h"
#include "bl_internal.h"

#include <climits>

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kSkThreads = 256;
constexpr int kSkWaves = kSkThreads / kWave;  // 4
constexpr int kSkDepth = 2;                    // chunks in flight per wave
constexpr int kSkRB = 2;                       // MFMA row blocks per row group
constexpr size_t kSkLdsMax = 64 * 1024;

struct SkProj {
  const int8_t* Xq;
  const float* xs;
  const uint8_t* W;
  const float* ws;
  float* Y;
  int32_t* acc;
  int N, K, C4;   // C4 = 256-code chunks per row
  int wg0, nwg;   // this projection's workgroups
  int S, CW;      // K segments per row group, chunks per segment
  int tile;       // LDS words of one combine tile (S > 1)
};

struct SkArgs {
  int wg0[BL_GROUP_CAP];  // first workgroup of each projection (INT_MAX when unused)
  SkProj p[BL_GROUP_CAP];
  int count;
  int T;
  int lds_words;  // combine words per workgroup (0: no segmented row groups)
};

typedef const SkArgs __attribute__((address_space(4)))* SkArgsPtr;

__device__ __forceinline__ SkProj load_sk(SkArgsPtr a, int i) {
  SkProj P;
  P.Xq = a->p[i].Xq;
  P.xs = a->p[i].xs;
  P.W = a->p[i].W;
  P.ws = a->p[i].ws;
  P.Y = a->p[i].Y;
  P.acc = a->p[i].acc;
  P.N = a->p[i].N;
  P.K = a->p[i].K;
  P.C4 = a->p[i].C4;
  P.wg0 = a->p[i].wg0;
  P.nwg = a->p[i].nwg;
  P.S = a->p[i].S;
  P.CW = a->p[i].CW;
  P.tile = a->p[i].tile;
  return P;
}

__device__ __forceinline__ v4i as_v4i(const uint4& v) {
  return v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
}

__device__ __forceinline__ v4i transpose_v4i(const uint4& v) {
  const uint32_t in[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
  transpose16(in, o);
  return v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int d) {
  return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

// One projection's partition: row groups g = wgl * (4/S) + wave / S + it * stride, wave
// wave % S taking K segment wave % S of each.
template <int TB, int S>
__device__ __forceinline__ void sk_sweep(const SkProj& P, int T, int wgl, int wave, int* lds) {
  constexpr int RB = kSkRB;
  constexpr int GPW = kSkWaves / S;  // row groups per workgroup step
  constexpr int D = kSkDepth;
  const int lane = threadIdx.x & (kWave - 1), li = lane & 15, lg = lane >> 4;
  const int nrg = (P.N + 16 * RB - 1) / (16 * RB);
  const int stride = P.nwg * GPW;
  const int grp = wave / S;
  const int g0 = wgl * GPW + grp;
  if (g0 >= nrg) return;  // the S waves of a row group leave together
  const int niter = (nrg - 1 - g0) / stride + 1;
  const int c0 = (wave % S) * P.CW;
  const int nck = min(P.C4, c0 + P.CW) - c0;
  const int Kb = P.K >> 2;
  const int total = niter * nck;

  // per-lane constant parts of the addresses
  uint32_t xoff[TB];
  float fac[TB];
  typedef const float __attribute__((address_space(4)))* ConstF;
  const float beta = *(ConstF)P.ws;
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int t = min(16 * tb + li, T - 1);
    xoff[tb] = (uint32_t)t * (uint32_t)P.K + 64u * (uint32_t)lg;
    fac[tb] = beta / P.xs[t];
  }
  const uint8_t* dummy = reinterpret_cast<const uint8_t*>(P.Xq);  // 64 L2-resident bytes
  const uint32_t doff = 16u * (uint32_t)(lane & 3);

  uint4 w[D][RB];
  uint4 b[D][TB][4];
  auto load = [&](int it, int m, int d) {
    const bool real = it < niter;
    const int row0 = (g0 + it * stride) * 16 * RB;
    const int chunk = c0 + min(m, nck - 1);
    const uint8_t* wbase = real ? P.W + (int64_t)row0 * Kb : dummy;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const uint32_t roff =
          (uint32_t)(min(row0 + rb * 16 + li, P.N - 1) - row0) * (uint32_t)Kb + 64u * chunk + 16u * lg;
      w[d][rb] = load_stream(reinterpret_cast<const uint4*>(wbase + (real ? roff : doff)));
    }
    const uint8_t* xbase = reinterpret_cast<const uint8_t*>(P.Xq) + 256 * chunk;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        b[d][tb][q] = *reinterpret_cast<const uint4*>(xbase + xoff[tb] + 16 * q);
  };

  v4i acc[RB][TB], cs[TB];
  auto clear = [&]() {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      cs[tb] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[rb][tb] = v4i{0, 0, 0, 0};
    }
  };
  clear();

  // row group finished by this wave: combine the S segments, rescale, store
  auto finish = [&](int it) {
    const int row0 = (g0 + it * stride) * 16 * RB;
    v4i res[RB][TB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) res[rb][tb] = acc[rb][tb] - cs[tb];
    bool last = true;
    if constexpr (S > 1) {
      int* tile = lds + (it * GPW + grp) * P.tile;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            atomicAdd(&tile[((rb * TB + tb) * 4 + r) * kWave + lane], res[rb][tb][r]);
      int arrived = 0;
      if (lane == 0) arrived = atomicAdd(&tile[RB * TB * 4 * kWave], 1);
      last = __builtin_amdgcn_readfirstlane(arrived) == S - 1;
      if (last) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              res[rb][tb][r] = atomicAdd(&tile[((rb * TB + tb) * 4 + r) * kWave + lane], 0);
      }
    }
    if (last) {
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const int tok = 16 * tb + li;
        if (tok < T) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = row0 + rb * 16 + 4 * lg + r;
              if (row < P.N) {
                const int v = res[rb][tb][r];
                P.Y[(int64_t)tok * P.N + row] = (float)v * fac[tb];
                if (P.acc) P.acc[(int64_t)tok * P.N + row] = v;
              }
            }
        }
      }
    }
    clear();
  };

  int itp = 0, mp = 0;  // next chunk to load
  auto advance = [&](int& it, int& m) {
    if (++m == nck) {
      m = 0;
      ++it;
    }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) {
    load(itp, mp, d);
    advance(itp, mp);
  }
  int itc = 0, mc = 0;  // next chunk to consume
  const v4i ones = v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101};
  auto step = [&](int d, bool prefetch) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v4i bt[TB];
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        bt[tb] = transpose_v4i(b[d][tb][q]);
        cs[tb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ones, bt[tb], cs[tb], 0, 0, 0);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        uint32_t u[4];
        unpack_u2(word_of(w[d][rb], q), u);
        const v4i ua = v4i{(int)u[0], (int)u[1], (int)u[2], (int)u[3]};
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
          acc[rb][tb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ua, bt[tb], acc[rb][tb], 0, 0, 0);
      }
    }
    if (prefetch) {
      load(itp, mp, d);
      advance(itp, mp);
    }
    if (mc == nck - 1) finish(itc);
    advance(itc, mc);
  };
  // whole rounds of D chunks in a loop with one exit, then the rest straight-line
  int left = total;
  while (left >= D) {
#pragma unroll
    for (int d = 0; d < D; ++d) step(d, true);
    left -= D;
  }
#pragma unroll
  for (int d = 0; d < D - 1; ++d)
    if (d < left) step(d, false);
}

template <int TB>
__global__ __launch_bounds__(kSkThreads) void skinny_kernel(SkArgs) {
  extern __shared__ int sk_lds[];
  const SkArgsPtr a = (SkArgsPtr)__builtin_amdgcn_kernarg_segment_ptr();
  const int wg = (int)blockIdx.x;
  int pi = 0;
#pragma unroll
  for (int i = 1; i < BL_GROUP_CAP; ++i) pi += wg >= a->wg0[i] ? 1 : 0;
  const SkProj P = load_sk(a, pi);
  const int T = a->T;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wgl = wg - P.wg0;
  if (P.S > 1) {  // combine tiles start at zero
    for (int i = threadIdx.x; i < a->lds_words; i += kSkThreads) sk_lds[i] = 0;
    __syncthreads();
  }
  switch (P.S) {
    case 1: sk_sweep<TB, 1>(P, T, wgl, wave, sk_lds); break;
    case 2: sk_sweep<TB, 2>(P, T, wgl, wave, sk_lds); break;
    default: sk_sweep<TB, 4>(P, T, wgl, wave, sk_lds); break;
  }
}

template <int TB>
int sk_resident(size_t lds) {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
  }
  int per = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, skinny_kernel<TB>, kSkThreads, lds) !=
          hipSuccess ||
      per < 1)
    per = 1;
  return cus * per;
}

// The dynamic-LDS limit is raised once per instance (first launch), never inside a
// stream capture after that.
template <int TB>
hipError_t launch_skinny_t(const bl_proj_internal* p, int count, int T, hipStream_t stream) {
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)skinny_kernel<TB>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSkLdsMax);
  if (attr != hipSuccess) return attr;
  SkArgs a{};
  int64_t total = 0;
  for (int i = 0; i < count; ++i) total += (int64_t)p[i].N * (p[i].K / 4);
  // S: enough chunks per segment (at least 8) to keep the ring busy
  int S[BL_GROUP_CAP];
  for (int i = 0; i < count; ++i) {
    const int c4 = p[i].K / 256;
    S[i] = c4 >= 32 ? 4 : c4 >= 16 ? 2 : 1;
  }
  const int tile = kSkRB * TB * 4 * kWave + 4;  // partial sums + arrival count (padded)
  int cap = 0;
  int wgs = 0, words = 0;
  for (int pass = 0; pass < 2; ++pass) {
    // first pass: partition with the occupancy at the LDS the partition needs
    cap = sk_resident<TB>(sizeof(int) * (size_t)words);
    wgs = 0;
    words = 0;
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
      s.C4 = p[i].K / 256;
      s.S = S[i];
      s.CW = (s.C4 + s.S - 1) / s.S;
      s.tile = tile;
      const int64_t bytes = (int64_t)p[i].N * (p[i].K / 4);
      const int nrg = (p[i].N + 16 * kSkRB - 1) / (16 * kSkRB);
      const int gpw = kSkWaves / s.S;
      int64_t n = (bytes * (int64_t)(cap - count) + total - 1) / total;
      n = n < 1 ? 1 : n;
      const int64_t most = (nrg + gpw - 1) / gpw;
      n = n > most ? most : n;
      s.nwg = (int)n;
      s.wg0 = wgs;
      a.wg0[i] = wgs;
      wgs += s.nwg;
      if (s.S > 1) {
        const int64_t iters = (nrg + n * gpw - 1) / (n * gpw);
        const int64_t need = iters * gpw * tile;
        if (need > words) words = (int)need;
      }
    }
  }
  if (sizeof(int) * (size_t)words > kSkLdsMax) return hipErrorInvalidValue;
  for (int i = count; i < BL_GROUP_CAP; ++i) a.wg0[i] = INT_MAX;
  a.count = count;
  a.T = T;
  a.lds_words = words;
  hipLaunchKernelGGL(skinny_kernel<TB>, dim3((unsigned)wgs), dim3(kSkThreads),
                     sizeof(int) * (size_t)words, stream, a);
  return hipGetLastError();
}

}  // namespace bl

using namespace bl;

bool bl_skinny_supports(int T, int K) { return T >= 1 && T <= 64 && K % 256 == 0; }

hipError_t bl_launch_skinny(const bl_proj_internal* p, int count, int T, hipStream_t stream) {
  switch ((T + 15) / 16) {
    case 1: return launch_skinny_t<1>(p, count, T, stream);
    case 2: return launch_skinny_t<2>(p, count, T, stream);
    case 3: return launch_skinny_t<3>(p, count, T, stream);
    default: return launch_skinny_t<4>(p, count, T, stream);
  }
}
