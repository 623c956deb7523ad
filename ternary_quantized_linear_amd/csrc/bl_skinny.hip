// bl_skinny.hip -- ternary x int8 product for a few tokens (up to 32 per pass) on int8 MFMA
// (v_mfma_i32_16x16x64_i8), int32 accumulation, fused rescale.
//
// [HF-1.58] "Fine-tuning LLMs to 1.58 bits", "Inference optimization and custom
// kernels": weights stay packed in memory and are unpacked inside the product;
// "Computation paradigm": integer arithmetic only. [bitnet.cpp] "3. BitLinear
// operation": rescale by the weight and activation scales.
//
// With few tokens the product is bound by the packed-weight stream (2 ops per weight per
// token against 1/4 byte per weight): every weight byte is read from HBM once, straight
// into registers, by waves that keep a ring of loads in flight.
//   - A workgroup has 8 waves: S teams (S = 1, 2 or 4) of G = 8/S waves. Team s owns
//     the s-th of S contiguous K segments; its G waves own G row blocks of 16 rows. A
//     step is 512 codes: per row block a lane loads 32 bytes (row lane % 16, bytes
//     32*(lane/16) of the step's 128) with two 128-bit loads, so every instruction pair
//     reads whole 128-byte lines, and feeds eight MFMAs.
//   - The activations of a step (16*TB tokens x 512 codes per team) are loaded once per
//     workgroup, coalesced, by all 512 threads, each step's ahead of its weights (so
//     that waiting for them never waits for those weights),
//     4x4 byte-transposed to the unpack order and written to one of two LDS stages, laid
//     out so that each MFMA's B operand is one conflict-free 1 KB read. One barrier per
//     step hands a stage from writers to readers; the weight loads in flight are not
//     waited for there.
//   - MFMA j of a step takes codes 64j + 16*ks for lane k-slot ks: each token's four
//     lanes read 64 contiguous staged bytes. The A operand of MFMA j at lane (row, ks) is
//     the packed dword at byte 16j + 4ks of the row's 128 bytes, which lane (row, j / 2)
//     loaded as its register 4*(j % 2) + ks: two 4x4 transposes across the four lane
//     rows (v_permlane32_swap, v_permlane16_swap) bring them over, and unpack_u2 gives
//     u = q + 1 in p-major order.
//   - sum x*u - sum x = sum x*q: the activation sum comes from one more MFMA per B
//     operand with an all-ones A operand.
//   - The S teams' partial tiles meet in LDS at the end of each row-block iteration;
//     team 0 rescales and stores Y = fp32(acc) * fp32(beta / s_t).
//   - Workgroups are partitioned among the projections of a grouped call in proportion
//     to their bytes; the grid is one round of resident workgroups.
// MFMA output: lane l, register r holds row 4*(l/16) + r of the block, token l % 16.
#include "bl_device.h"
#include "bl_internal.h"

#include <climits>

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kSkWaves = 8;
constexpr int kSkThreads = kSkWaves * kWave;  // 512
constexpr int kSkDepth = 2;                    // steps in flight (weights and activations)
constexpr int kSkKS = 512;                     // codes per step
constexpr int kSkNM = kSkKS / 64;              // MFMAs per step per token block
constexpr int kSkStepBytes = kSkKS / 4;        // packed bytes per row per step
constexpr size_t kSkLdsMax = 80 * 1024;  // two workgroups per CU

struct SkProj {
  const int8_t* Xq;
  const float* xs;
  const uint8_t* W;
  const float* ws;
  float* Y;
  int32_t* acc;
  int N, K;
  int steps;    // ceil(K / 512)
  int wg0, nwg;
  int S, CW;    // teams (K segments) and steps per segment
};

struct SkArgs {
  int wg0[BL_GROUP_CAP];  // first workgroup of each projection (INT_MAX when unused)
  SkProj p[BL_GROUP_CAP];
  int count;
  int T;
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
  P.steps = a->p[i].steps;
  P.wg0 = a->p[i].wg0;
  P.nwg = a->p[i].nwg;
  P.S = a->p[i].S;
  P.CW = a->p[i].CW;
  return P;
}

// 4x4 transpose of dwords across the four 16-lane rows: on return, register q of lane
// (row s) holds what register s of lane (row q) held.
__device__ __forceinline__ void transpose_rows(uint32_t (&r)[4]) {
  auto a = __builtin_amdgcn_permlane32_swap(r[0], r[2], false, false);
  auto b = __builtin_amdgcn_permlane32_swap(r[1], r[3], false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  r[0] = c[0];
  r[1] = c[1];
  r[2] = d[0];
  r[3] = d[1];
}

// LDS bytes of one stage and of a whole workgroup, per team count S and token blocks TB.
__host__ __device__ constexpr int sk_stage_bytes(int S, int TB) { return S * kSkNM * TB * 1024; }
__host__ __device__ constexpr int sk_lds_bytes(int S, int TB) {
  return 2 * sk_stage_bytes(S, TB) + kSkWaves * TB * 1024;
}

template <int TB, int S>
__device__ __forceinline__ void sk_sweep(const SkProj& P, int T, int wgl, int wave, uint8_t* lds) {
  constexpr int G = kSkWaves / S;
  constexpr int D = kSkDepth;
  constexpr int PIECES = S * 16 * TB * (kSkKS / 16);  // 16-byte activation pieces per step
  constexpr int PPT = (PIECES + kSkThreads - 1) / kSkThreads;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), li = lane & 15, lg = lane >> 4;
  const int seg = wave / G, mem = wave % G;
  const int nrb = (P.N + 15) / 16;
  // every wave of the workgroup runs the same number of steps (one barrier per step)
  const int niter = (nrb - wgl * G + P.nwg * G - 1) / (P.nwg * G);
  const int CW = P.CW;
  const int total = niter * CW;
  const int Kb = P.K >> 2;
  uint8_t* stage0 = lds;
  uint8_t* stage1 = lds + sk_stage_bytes(S, TB);
  int* comb = reinterpret_cast<int*>(lds + 2 * sk_stage_bytes(S, TB));

  // activation pieces this thread stages: piece q = tid + p * 512 -> team, token, offset
  int pt_tok[PPT], pt_seg[PPT], pt_off[PPT], pt_lds[PPT];
  bool pt_on[PPT];
#pragma unroll
  for (int p = 0; p < PPT; ++p) {
    const int q = tid + p * kSkThreads;
    pt_on[p] = q < PIECES;
    const int qq = pt_on[p] ? q : 0;
    const int o16 = qq % (kSkKS / 16);
    const int t = (qq / (kSkKS / 16)) % (16 * TB);
    const int s = qq / ((kSkKS / 16) * 16 * TB);
    pt_tok[p] = min(t, T - 1);  // tokens past T: any valid row (their columns are dropped)
    pt_seg[p] = s;
    pt_off[p] = 16 * o16;
    const int j = o16 >> 2, ks = o16 & 3;
    pt_lds[p] = ((((s * kSkNM + j) * TB + (t >> 4)) * kWave) + ks * 16 + (t & 15)) * 16;
  }
  const uint8_t* dummy = reinterpret_cast<const uint8_t*>(P.Xq);

  uint4 w[D][2];
  uint4 xr[D][PPT];
  // weights of step n (iteration n / CW, segment step n % CW) into ring slot d: this
  // wave's row block, its team's segment; lanes past the row end read a dummy block
  auto load_w = [&](int n, int d) {
    const int it = n / CW, m = n - it * CW;
    const int rb = (wgl + it * P.nwg) * G + mem;
    const int st = seg * CW + m;
    const bool real = n < total && st * kSkKS + 128 * lg < P.K;
    const int row = min(rb * 16 + li, P.N - 1);
    const uint8_t* wp =
        real ? P.W + (int64_t)row * Kb + st * kSkStepBytes + 32 * lg : dummy + 32 * (lane & 3);
    w[d][0] = *reinterpret_cast<const uint4*>(wp);
    w[d][1] = *reinterpret_cast<const uint4*>(wp + 16);
  };
  // activations of step n into slot d: pieces of every team's step (past the row end,
  // any valid bytes: they are replaced by zeros when staged)
  auto load_x = [&](int n, int d) {
    const int m = n - (n / CW) * CW;
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
      if (!pt_on[p]) continue;  // wave-uniform: pieces come in whole waves
      const int code = min((pt_seg[p] * CW + m) * kSkKS + pt_off[p], P.K - 16);
      xr[d][p] = *reinterpret_cast<const uint4*>(P.Xq + (int64_t)pt_tok[p] * P.K + code);
    }
  };
  // staged activations of step n (from slot d), transposed; zero past the row end
  auto stage = [&](int n, int d, uint8_t* dst) {
    const int m = n - (n / CW) * CW;
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
      if (!pt_on[p]) continue;
      uint4 v = xr[d][p];
      if ((pt_seg[p] * CW + m) * kSkKS + pt_off[p] >= P.K) v = make_uint4(0u, 0u, 0u, 0u);
      const uint32_t in[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[4];
      transpose16(in, o);
      *reinterpret_cast<uint4*>(dst + pt_lds[p]) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  };

  v4i acc[TB], cs[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    acc[tb] = v4i{0, 0, 0, 0};
    cs[tb] = v4i{0, 0, 0, 0};
  }
  typedef const float __attribute__((address_space(4)))* ConstF;
  const float beta = *(ConstF)P.ws;
  float fac[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) fac[tb] = beta / P.xs[min(16 * tb + li, T - 1)];

  // end of a row-block iteration: teams meet in LDS, team 0 stores
  auto finish = [&](int it) {
    if constexpr (S > 1) {
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          comb[(((seg * G + mem) * TB + tb) * 4 + r) * kWave + lane] = acc[tb][r] - cs[tb][r];
      __syncthreads();
    }
    if (seg == 0) {
      const int row0 = ((wgl + it * P.nwg) * G + mem) * 16;
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        v4i v = acc[tb] - cs[tb];
#pragma unroll
        for (int s2 = 1; s2 < S; ++s2)
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] += comb[(((s2 * G + mem) * TB + tb) * 4 + r) * kWave + lane];
        const int tok = 16 * tb + li;
        if (tok < T) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = row0 + 4 * lg + r;
            if (row < P.N) {
              P.Y[(int64_t)tok * P.N + row] = (float)v[r] * fac[tb];
              if (P.acc) P.acc[(int64_t)tok * P.N + row] = v[r];
            }
          }
        }
      }
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      acc[tb] = v4i{0, 0, 0, 0};
      cs[tb] = v4i{0, 0, 0, 0};
    }
  };

  const v4i ones = v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101};
  // prologue: steps 0 and 1 in flight, each step's activations ahead of its weights
  // (waiting for the activations of a step never waits for its weights); step 0 staged
#pragma unroll
  for (int d = 0; d < D; ++d) {
    load_x(d, d);
    load_w(d, d);
  }
  stage(0, 0, stage0);
  __syncthreads();

  // step n consumes ring slot and stage n % 2, issues step n + 2 into that slot and
  // stages step n + 1 from the other one
  auto step = [&](int n, int d, bool prefetch) {
    uint8_t* cur = d ? stage1 : stage0;
    uint8_t* nxt = d ? stage0 : stage1;
    // A operands: MFMA j's dword ks sits in lane row j / 2, register 4 * (j % 2) + ks
    uint32_t a0[4] = {w[d][0].x, w[d][0].y, w[d][0].z, w[d][0].w};
    uint32_t a1[4] = {w[d][1].x, w[d][1].y, w[d][1].z, w[d][1].w};
    transpose_rows(a0);
    transpose_rows(a1);
#pragma unroll
    for (int j = 0; j < kSkNM; ++j) {
      uint32_t u[4];
      unpack_u2((j & 1) ? a1[j >> 1] : a0[j >> 1], u);
      const v4i ua = v4i{(int)u[0], (int)u[1], (int)u[2], (int)u[3]};
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const uint4 bx = *reinterpret_cast<const uint4*>(
            cur + (((seg * kSkNM + j) * TB + tb) * kWave + lane) * 16);
        const v4i bv = v4i{(int)bx.x, (int)bx.y, (int)bx.z, (int)bx.w};
        acc[tb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ua, bv, acc[tb], 0, 0, 0);
        cs[tb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ones, bv, cs[tb], 0, 0, 0);
      }
    }
    if (prefetch) {
      load_x(n + D, d);
      load_w(n + D, d);
    }
    if (n + 1 < total) stage(n + 1, d ^ 1, nxt);
    const int it = n / CW;
    if (n - it * CW == CW - 1) finish(it);
    __syncthreads();
  };
  // whole rounds of D steps, then the rest: every wave of the workgroup runs the same
  // steps, so every barrier is reached by all of them
  int n = 0;
  while (total - n >= D) {
#pragma unroll
    for (int d = 0; d < D; ++d) step(n + d, d, true);
    n += D;
  }
#pragma unroll
  for (int d = 0; d < D - 1; ++d)
    if (n + d < total) step(n + d, d, false);
}

template <int TB>
__global__ __launch_bounds__(kSkThreads) void skinny_kernel(SkArgs) {
  extern __shared__ uint4 sk_lds[];
  const SkArgsPtr a = (SkArgsPtr)__builtin_amdgcn_kernarg_segment_ptr();
  const int wg = (int)blockIdx.x;
  int pi = 0;
#pragma unroll
  for (int i = 1; i < BL_GROUP_CAP; ++i) pi += wg >= a->wg0[i] ? 1 : 0;
  const SkProj P = load_sk(a, pi);
  const int T = a->T;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wgl = wg - P.wg0;
  uint8_t* lds = reinterpret_cast<uint8_t*>(sk_lds);
  switch (P.S) {
    case 1: sk_sweep<TB, 1>(P, T, wgl, wave, lds); break;
    case 2: sk_sweep<TB, 2>(P, T, wgl, wave, lds); break;
    default:
      if constexpr (TB == 1) sk_sweep<TB, 4>(P, T, wgl, wave, lds);
      break;
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

// Teams per row block: segments of at least 4 steps, more teams while the row blocks
// alone would leave the device short of waves.
int sk_teams(int steps, int nrb, int TB) {
  const int smax = TB == 1 ? 4 : 2;  // keeps the stages and the combine area within 80 KB
  int S = 1;
  while (S < smax && steps / (2 * S) >= 4 && nrb * S < 4096) S *= 2;
  return S;
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
    s.steps = (p[i].K + kSkKS - 1) / kSkKS;
    s.S = sk_teams(s.steps, (s.N + 15) / 16, TB);
    s.CW = (s.steps + s.S - 1) / s.S;
    const size_t need = (size_t)sk_lds_bytes(s.S, TB);
    lds = need > lds ? need : lds;
    total += (int64_t)p[i].N * (p[i].K / 4);
  }
  if (lds > kSkLdsMax) return hipErrorInvalidValue;
  const int cap = sk_resident<TB>(lds);
  int wgs = 0;
  for (int i = 0; i < count; ++i) {
    SkProj& s = a.p[i];
    const int G = kSkWaves / s.S;
    const int nrb = (s.N + 15) / 16;
    const int64_t bytes = (int64_t)p[i].N * (p[i].K / 4);
    int64_t n = (bytes * (int64_t)(cap - count) + total - 1) / total;
    n = n < 1 ? 1 : n;
    const int64_t most = (nrb + G - 1) / G;  // no workgroup without a row block
    n = n > most ? most : n;
    s.nwg = (int)n;
    s.wg0 = wgs;
    a.wg0[i] = wgs;
    wgs += s.nwg;
  }
  for (int i = count; i < BL_GROUP_CAP; ++i) a.wg0[i] = INT_MAX;
  a.count = count;
  a.T = T;
  hipLaunchKernelGGL(skinny_kernel<TB>, dim3((unsigned)wgs), dim3(kSkThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace bl

using namespace bl;

bool bl_skinny_supports(int T, int K) { return T >= 1 && T <= 128 && K % 256 == 0; }

// Up to 32 tokens in one launch; more run as passes over slices of 32 tokens (each pass
// streams the weights again: the choice of the caller when the GEMM's tiles would
// leave most of the device idle).
hipError_t bl_launch_skinny(const bl_proj_internal* p, int count, int T, hipStream_t stream) {
  for (int t0 = 0; t0 < T; t0 += 32) {
    const int tn = T - t0 < 32 ? T - t0 : 32;
    bl_proj_internal q[BL_GROUP_CAP];
    for (int i = 0; i < count; ++i) {
      q[i] = p[i];
      q[i].Xq += (int64_t)t0 * p[i].K;
      q[i].x_scale += t0;
      q[i].Y += (int64_t)t0 * p[i].N;
      if (q[i].acc) q[i].acc += (int64_t)t0 * p[i].N;
    }
    const hipError_t e = tn <= 16 ? launch_skinny_t<1>(q, count, tn, stream)
                                  : launch_skinny_t<2>(q, count, tn, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
