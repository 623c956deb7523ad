// bl_gemv.hip -- decode GEMV for one token: packed ternary weights x int8 activations
// with int8 dot4 (v_dot4c_i32_i8), int32 accumulation, fused rescale.
//
// [HF-1.58] "Fine-tuning LLMs to 1.58 bits", "Computation paradigm": the ternary
// product needs only integer additions; "Inference optimization and custom kernels":
// the 2-bit weights are unpacked on the fly inside the product; "Tiled matrix
// multiplication": memory bandwidth is the bottleneck. [bitnet.cpp] "3. BitLinear
// operation": the integer product is rescaled by the weight scale and the activation
// dequantization factor.
//
// For one token the product streams 1/4 byte per weight, so the design is about HBM:
//   - A row of K codes is K/4 bytes = C chunks of 16 bytes (64 codes, one 128-bit load
//     per lane). A row of up to 64 chunks is one wave's (L = 16 or 32 lanes per row when
//     it has at most 16 or 32 chunks, so one wave instruction covers 64/L rows). A longer
//     row is cut into S = 2 or 4 contiguous segments, read at the same time by S waves of
//     one workgroup, each wave always taking the same segment: every wave keeps the
//     activations of its own chunks in registers for the whole run. The S partial sums
//     meet in one 64-bit LDS word (partial sum in the low bits, arrival count from bit
//     40); the wave whose add completes the count writes the row.
//   - Activations are 4x4 byte-transposed (transpose16) so that dword p of a chunk holds
//     the codes in bit pair p of the four packed bytes. Lanes past the row end or past
//     their segment hold zero activations, so whatever weights they read add nothing.
//   - Workgroups are partitioned among the projections of the launch (for example the
//     seven of a decoder layer) in proportion to their bytes; inside a partition the rows
//     are swept grid-stride, so each partition reads one compact window of its matrix at
//     a time. The grid is part of one round of resident workgroups. Each wave keeps D row groups
//     of weights in flight in a ring of registers; a prefetch past the wave's last row
//     reads a small L2-resident block instead, so no load sits under a branch and each
//     step waits for exactly the oldest buffer.
//   - The wave index is made explicitly uniform (readfirstlane): the whole schedule stays
//     in scalar registers and the row bases are scalar.
//   - Unpacking is 5 ALU ops per packed dword: bit pairs 0, 1, 2 are masked in place
//     (values u, 4u, 16u with u = q + 1 in {0, 1, 2}) and pair 3 shifted down; pairs 0
//     and 3 share one dot4 accumulator, pairs 1 and 2 have one each; the sum is
//     a03 + a1/4 + a2/16 (exact shifts of exact multiples) started at minus the lane's
//     own activation sum: sum x*q exactly.
//   - Lane sums are reduced with DPP; Y = fp32(acc) * fp32(beta / s).
//
// The same kernel serves the 1-bit sign variant ([bitnet.cpp] "1. Weight
// binarization": codes +-1, eight per byte, bit i of byte j = code 8j+i set for +1).
// A 16-byte chunk then holds 128 codes; the lane keeps its 128 activations as eight
// "bit planes" per packed dword (plane i, byte b = activation of code 8b+i). Planes 0..6
// are masked in place (values 2^i * bit, all below 128) into their own dot4
// accumulator, plane 7 is shifted down and shares plane 0's; sum_i a_i / 2^i is the
// sum of the activations whose code is +1, P, and sum c*x = 2P - sum x.
#include "bl_device.h"
#include "bl_internal.h"
#include "bl_plan.h"

#include <climits>
#include <cstddef>

namespace bl {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / kWave;  // 4
// Row groups in flight per wave, 2-bit form: two in the instance for rows of up to 256
// chunks (with five eighths of a round of workgroups), three in the instance that
// also takes longer rows (with half a round; the 70B down projection, 448 chunks per
// row, measured 5% faster so). The 1-bit rows carry half the bytes: four in flight.
constexpr int kGemvDepth = 2;
constexpr int kGemvDepthBig = 3;
#ifndef BL_GEMV_SIGN_DEPTH
#define BL_GEMV_SIGN_DEPTH 4
#endif
constexpr int kGemvSignDepth = BL_GEMV_SIGN_DEPTH;  // the 1-bit rows carry half the bytes
constexpr int kGemvMaxC = plan::kGemvMaxC;         // K <= 32768

struct GemvProj {
  const int8_t* Xq;
  const float* xs;
  const uint4* W;
  const float* ws;
  float* Y;
  int32_t* acc;
  int N, C;
  int wg0, nwg;  // this projection's workgroups
  int cfg;       // mapping (see gemv_kernel)
  int CW;        // chunks per wave segment
  int rpg;       // rows per weight scale group
};

struct GemvArgs {
  GemvProj p[BL_GROUP_CAP];
  int count;
};

typedef const GemvArgs __attribute__((address_space(4)))* ArgsPtr;

// The kernel's argument list: the partition starts and the combine-word count come first,
// as scalars, so that they can be preloaded into SGPRs at wave launch (the build asks
// for 8 preloaded dwords): a wave then finds its projection without a round trip to the
// argument memory, and the projection's fields are its first load.
struct GemvKernArgs {
  int wg0[BL_GROUP_CAP - 1];  // first workgroup of projections 1..7 (INT_MAX when unused)
  int slots;                  // 64-bit combine words per workgroup (0: no segmented rows)
  GemvArgs g;
};
constexpr int kGemvArgsOffset = 32;
static_assert(offsetof(GemvKernArgs, g) == kGemvArgsOffset, "argument layout");

// Field-by-field copy out of the constant (kernel-argument) address space.
__device__ __forceinline__ GemvProj load_proj(ArgsPtr a, int i) {
  GemvProj P;
  P.Xq = a->p[i].Xq;
  P.xs = a->p[i].xs;
  P.W = a->p[i].W;
  P.ws = a->p[i].ws;
  P.Y = a->p[i].Y;
  P.acc = a->p[i].acc;
  P.N = a->p[i].N;
  P.C = a->p[i].C;
  P.wg0 = a->p[i].wg0;
  P.nwg = a->p[i].nwg;
  P.cfg = a->p[i].cfg;
  P.CW = a->p[i].CW;
  P.rpg = a->p[i].rpg;
  return P;
}

// Accumulators by factor: pairs 0 and 3 carry 1, pair 1 carries 4, pair 2 carries 16.
struct Acc4 {
  int a0, a1, a2;  // pairs 0 and 3 (factor 1) share a0
};

__device__ __forceinline__ void dot_word(uint32_t w, const uint4& x, Acc4& s) {
  s.a0 = sdot4(w & 0x03030303u, x.x, s.a0);
  s.a1 = sdot4(w & 0x0C0C0C0Cu, x.y, s.a1);
  s.a2 = sdot4(w & 0x30303030u, x.z, s.a2);
  s.a0 = sdot4((w >> 6) & 0x03030303u, x.w, s.a0);
}

__device__ __forceinline__ void dot_chunk(const uint4 w, const uint4 (&x)[4], Acc4& s) {
  dot_word(w.x, x[0], s);
  dot_word(w.y, x[1], s);
  dot_word(w.z, x[2], s);
  dot_word(w.w, x[3], s);
}

__device__ __forceinline__ int acc_total(const Acc4& s) {
  return s.a0 + (s.a1 >> 2) + (s.a2 >> 4);
}

// 1-bit: accumulator i carries plane i times 2^i (plane 7 rides on accumulator 0).
struct Acc8 {
  int a[7];
};

__device__ __forceinline__ void dot_word1(uint32_t w, const uint32_t (&x)[8], Acc8& s) {
  s.a[0] = sdot4(w & 0x01010101u, x[0], s.a[0]);
  s.a[1] = sdot4(w & 0x02020202u, x[1], s.a[1]);
  s.a[2] = sdot4(w & 0x04040404u, x[2], s.a[2]);
  s.a[3] = sdot4(w & 0x08080808u, x[3], s.a[3]);
  s.a[4] = sdot4(w & 0x10101010u, x[4], s.a[4]);
  s.a[5] = sdot4(w & 0x20202020u, x[5], s.a[5]);
  s.a[6] = sdot4(w & 0x40404040u, x[6], s.a[6]);
  s.a[0] = sdot4((w >> 7) & 0x01010101u, x[7], s.a[0]);
}

// sum over the lane's codes of c * x, from the plane sums and the lane's activation sum
__device__ __forceinline__ int acc1_total(const Acc8& s, int xsum) {
  const int pos = s.a[0] + (s.a[1] >> 1) + (s.a[2] >> 2) + (s.a[3] >> 3) + (s.a[4] >> 4) +
                  (s.a[5] >> 5) + (s.a[6] >> 6);
  return 2 * pos - xsum;
}

// The 128 activations of 1-bit chunk c (eight 16-byte loads).
__device__ __forceinline__ void load_raw1(const int8_t* x, int c, uint4 (&v)[8]) {
  const uint4* src = reinterpret_cast<const uint4*>(x + 128 * c);
#pragma unroll
  for (int d = 0; d < 8; ++d) v[d] = src[d];
}

// Those activations as 4 x 8 bit planes, and their sum.
__device__ __forceinline__ void planes1(const uint4 (&v)[8], uint32_t (&o)[4][8], int& xsum) {
  uint32_t raw[32];
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    raw[4 * d] = v[d].x;
    raw[4 * d + 1] = v[d].y;
    raw[4 * d + 2] = v[d].z;
    raw[4 * d + 3] = v[d].w;
    xsum += byte_sum(v[d].x) + byte_sum(v[d].y) + byte_sum(v[d].z) + byte_sum(v[d].w);
  }
  // packed dword j covers codes 32j..32j+31; plane i byte b = x[32j + 8b + i], which is
  // byte i % 4 of raw dword 8j + 2b + i / 4
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int h = i >> 2, q = i & 3;
      const uint32_t sel = 0x0C0C0000u | (uint32_t)(4 + q) << 8 | (uint32_t)q;  // lo: b0, b1
      const uint32_t lo = __builtin_amdgcn_perm(raw[8 * j + 2 + h], raw[8 * j + h], sel);
      const uint32_t hi = __builtin_amdgcn_perm(raw[8 * j + 6 + h], raw[8 * j + 4 + h], sel);
      o[j][i] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
}

// 1-bit planes in LDS, one 128-byte record per chunk: 16-byte piece q of chunk c at
// 16 (q ^ (c % 8)), so that the lanes of one read (consecutive chunks, the same piece)
// spread over all banks; the chunk sums follow the records.
__device__ __forceinline__ void store_planes1(uint8_t* lds, int c, const uint32_t (&o)[4][8]) {
  const uint32_t* f = &o[0][0];
#pragma unroll
  for (int q = 0; q < 8; ++q)
    *reinterpret_cast<uint4*>(lds + 128 * c + 16 * (q ^ (c & 7))) =
        make_uint4(f[4 * q], f[4 * q + 1], f[4 * q + 2], f[4 * q + 3]);
}

__device__ __forceinline__ void read_planes1(const uint8_t* lds, int c, bool on,
                                             uint32_t (&o)[4][8]) {
  uint32_t* f = &o[0][0];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint4 v = *reinterpret_cast<const uint4*>(lds + 128 * c + 16 * (q ^ (c & 7)));
    if (!on) v = make_uint4(0u, 0u, 0u, 0u);
    f[4 * q] = v.x;
    f[4 * q + 1] = v.y;
    f[4 * q + 2] = v.z;
    f[4 * q + 3] = v.w;
  }
}

// 2-bit: the workgroup's transposed activations in LDS, one 64-byte record per chunk with
// piece q of chunk c at 16 (q ^ ((c / 2) % 4)): two records share a 128-byte bank row,
// so eight consecutive chunks read the same piece from eight distinct bank groups.
__device__ __forceinline__ void load_raw0(const int8_t* x, int c, uint4 (&v)[4]) {
  const uint4* src = reinterpret_cast<const uint4*>(x + 64 * c);
#pragma unroll
  for (int d = 0; d < 4; ++d) v[d] = src[d];
}

__device__ __forceinline__ void store_chunk0(uint8_t* lds, int c, const uint4 (&v)[4], int& xsum) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t in[4] = {v[d].x, v[d].y, v[d].z, v[d].w};
    uint32_t t[4];
    transpose16(in, t);
    *reinterpret_cast<uint4*>(lds + 64 * c + 16 * (d ^ ((c >> 1) & 3))) = make_uint4(t[0], t[1], t[2], t[3]);
    xsum += byte_sum(v[d].x) + byte_sum(v[d].y) + byte_sum(v[d].z) + byte_sum(v[d].w);
  }
}

__device__ __forceinline__ void read_chunk0(const uint8_t* lds, int c, bool on, uint4 (&o)[4]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint4 v = *reinterpret_cast<const uint4*>(lds + 64 * c + 16 * (d ^ ((c >> 1) & 3)));
    if (!on) v = make_uint4(0u, 0u, 0u, 0u);
    o[d] = v;
  }
}

// Activations of chunk c (64 codes): 4 x 16 bytes, transposed, and their sum; zeros when
// the lane has no chunk.
__device__ __forceinline__ void load_act_chunk(const int8_t* x, int c, bool on, uint4 (&o)[4],
                                               int& xsum) {
  const uint4* src = reinterpret_cast<const uint4*>(x + 64 * c);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint4 v = src[d];
    if (!on) v = make_uint4(0u, 0u, 0u, 0u);
    const uint32_t in[4] = {v.x, v.y, v.z, v.w};
    uint32_t t[4];
    transpose16(in, t);
    o[d] = make_uint4(t[0], t[1], t[2], t[3]);
    xsum += byte_sum(v.x) + byte_sum(v.y) + byte_sum(v.z) + byte_sum(v.w);
  }
}

// One projection's partition. L lanes per row, I chunks per lane, S waves per row
// (S > 1 needs L = 64). Wave `wave` of partition workgroup `wgl` takes segment wave % S
// of row groups wgl * (4/S) + wave / S + k * stride, k = 0, 1, ...
// Builds this thread's chunks' records (the first from araw, loaded earlier): bit planes
// (1-bit) or transposed bytes (2-bit), with their sums, in LDS; then waits for the whole
// workgroup's.
template <int FMT, int NR>
__device__ __forceinline__ void publish_acts(const GemvProj& P, uint8_t* plds, int* psum,
                                             const uint4 (&araw)[NR], unsigned long long* slots,
                                             int nslots) {
  // segmented rows: the combine words start at zero; cleared here, before the one barrier
  // that also publishes the activations (the weight ring is already in flight)
  for (int i = threadIdx.x; i < nslots; i += kGemvThreads) slots[i] = 0ull;
  for (int c = threadIdx.x; c < P.C; c += kGemvThreads) {
    uint4 v[NR];
    if (c == (int)threadIdx.x) {
#pragma unroll
      for (int d = 0; d < NR; ++d) v[d] = araw[d];
    } else {
      if constexpr (FMT == 1) load_raw1(P.Xq, c, v);
      else load_raw0(P.Xq, c, v);
    }
    int xs = 0;
    if constexpr (FMT == 1) {
      uint32_t o[4][8];
      planes1(v, o, xs);
      store_planes1(plds, c, o);
    } else {
      store_chunk0(plds, c, v, xs);
    }
    psum[c] = xs;
  }
  __syncthreads();
}

template <int L, int I, int S, int FMT, int MAXI>
__device__ __forceinline__ void sweep(const GemvProj& P, int wgl, int wave,
                                      unsigned long long* slots, int plane_base, int nslots) {
  constexpr int RW = kWave / L;        // rows per row group
  constexpr int GPW = kGemvWaves / S;  // row groups per workgroup step
  const int lane = threadIdx.x & (kWave - 1);
  const int sub = lane / L, jl = lane & (L - 1);
  const int C = P.C;
  const int cw = S > 1 ? P.CW : C;  // chunks of this wave's segment
  const int cbase = (wave % S) * cw;
  const int ngroups = (P.N + RW - 1) / RW;
  const int stride = P.nwg * GPW;
  const int g0 = wgl * GPW + wave / S;
  // The workgroup prepares the row's activations once, in LDS after the combine words
  // (thread t takes chunk t, t + 256, ...): 1-bit bit planes, 2-bit transposed bytes;
  // the first chunk's activations are asked for before the weight ring, and every wave,
  // with rows or not, passes the barrier that publishes them.
  constexpr int NR = FMT == 1 ? 8 : 4;  // 16-byte pieces per chunk record
  uint8_t* const plds = reinterpret_cast<uint8_t*>(slots) + plane_base;
  int* const psum = reinterpret_cast<int*>(plds + 16 * NR * C);
  uint4 araw[NR];
  if ((int)threadIdx.x < C) {
    if constexpr (FMT == 1) load_raw1(P.Xq, threadIdx.x, araw);
    else load_raw0(P.Xq, threadIdx.x, araw);
  }
  if (g0 >= ngroups) {
    publish_acts<FMT, NR>(P, plds, psum, araw, slots, nslots);
    return;
  }
  const int glast = g0 + ((ngroups - 1 - g0) / stride) * stride;

  // lane chunk i is cbase + jl + L*i when that is inside the segment and the row; a
  // lane without a chunk reads its segment's first one (same cache line as lane 0)
  int ci[I];
  bool on[I];
#pragma unroll
  for (int i = 0; i < I; ++i) {
    const int c = jl + L * i;
    on[i] = c < cw && cbase + c < C;
    ci[i] = on[i] ? cbase + c : cbase;
  }
  const uint4* dummy = reinterpret_cast<const uint4*>(P.Xq);  // 64 bytes, L2-resident
  // the row group's base is wave-uniform (scalar); each lane adds a 32-bit offset
  // (a scalar base plus a 32-bit unsigned byte offset per lane: one VGPR per address)
  uint32_t boff[I];
#pragma unroll
  for (int i = 0; i < I; ++i) boff[i] = 16u * (uint32_t)ci[i];
  const uint32_t doff = 16u * (uint32_t)(lane & 3);
  // The prefetch walks the row groups with a scalar pointer advanced by a fixed step;
  // only the last group of a ragged projection (RW > 1) needs the row clamp.
  const int64_t gstep = (int64_t)stride * RW * C * 16;
  const char* wnext = reinterpret_cast<const char*>(P.W) + (int64_t)g0 * RW * C * 16;
  int gnext = g0;
  auto load_w = [&](uint4 (&w)[I]) {
    const bool real = gnext <= glast;
    const char* base = real ? wnext : reinterpret_cast<const char*>(dummy);
    uint32_t roff = 0u;
    if constexpr (RW > 1) {
      const int row0 = gnext * RW;
      roff = 16u * (uint32_t)((min(row0 + sub, P.N - 1) - row0) * C);
    }
#pragma unroll
    for (int i = 0; i < I; ++i)
      w[i] = load_stream(reinterpret_cast<const uint4*>(base + (real ? roff + boff[i] : doff)));
    wnext += gstep;
    gnext += stride;
  };
  // The weight ring goes out before the activations: vector loads complete in issue
  // order, so this way the first row waits for one memory latency, not two in a row.
  // The two scales come through the scalar cache, off the vector counter.
  constexpr int D = FMT == 0 ? (MAXI >= 2 ? kGemvDepthBig : kGemvDepth) : kGemvSignDepth;
  uint4 w[D][I];
#pragma unroll
  for (int d = 0; d < D; ++d) load_w(w[d]);
  // activations: 2-bit chunks as 4 transposed uint4, 1-bit chunks as 4 x 8 bit planes
  uint4 x[FMT == 0 ? I : 1][4];
  uint32_t x1[FMT == 1 ? I : 1][4][8];
  int xsum = 0;
  publish_acts<FMT, NR>(P, plds, psum, araw, slots, nslots);
#pragma unroll
  for (int i = 0; i < I; ++i) {
    if constexpr (FMT == 0) read_chunk0(plds, ci[i], on[i], x[i]);
    else read_planes1(plds, ci[i], on[i], x1[i]);
    xsum += on[i] ? psum[ci[i]] : 0;
  }
  typedef const float __attribute__((address_space(4)))* ConstF;
  const float xsc = *(ConstF)P.xs;
  const float f = *(ConstF)P.ws / xsc;  // one weight scale (rpg >= N)
  const bool scale_groups = P.rpg < P.N;
  // with weight scale groups, each lane's scale for the rows of the first flush is
  // loaded now, while the weights stream (a load at the flush would add a round trip);
  // it is first used, and so first waited for, at the flush
  auto lane_scale = [&](int gbase) {
    const int row = min((gbase + (lane / RW) * stride) * RW + lane % RW, P.N - 1);
    return P.ws[row / P.rpg];
  };
  const float ws0 = scale_groups ? lane_scale(g0) : 0.0f;
  int g = g0, k = 0;
  // Row totals wait in a register (lane j holds slot j) and leave in one store per 64
  // slots: no store sits between the ring's loads, so each wait counts loads only.
  int res = 0;
  unsigned long long keep = 0;  // bit j: slot j holds a row to write
  int nb = 0, gb = g0;          // slots filled; row group of slot 0
  auto flush = [&]() {
    const int row = (gb + (lane / RW) * stride) * RW + lane % RW;
    if (lane < nb && ((keep >> lane) & 1ull) && row < P.N) {
      P.Y[row] = (float)res * (!scale_groups ? f : (gb == g0 ? ws0 : lane_scale(gb)) / xsc);
      if (P.acc) P.acc[row] = res;
    }
    nb = 0;
    keep = 0;
    gb = g;
  };
  // one row group: consume buffer d, refill it D groups ahead (prefetch), keep the total
  auto step = [&](int d, bool prefetch) {
    int lane_tot;
    if constexpr (FMT == 0) {
      Acc4 s{-xsum, 0, 0};
#pragma unroll
      for (int i = 0; i < I; ++i) dot_chunk(w[d][i], x[i], s);
      lane_tot = acc_total(s);
    } else {
      Acc8 s{{0, 0, 0, 0, 0, 0, 0}};
#pragma unroll
      for (int i = 0; i < I; ++i) {
        dot_word1(w[d][i].x, x1[i][0], s);
        dot_word1(w[d][i].y, x1[i][1], s);
        dot_word1(w[d][i].z, x1[i][2], s);
        dot_word1(w[d][i].w, x1[i][3], s);
      }
      lane_tot = acc1_total(s, xsum);
    }
    if (prefetch) load_w(w[d]);
    int tot = group_sum_to_last<L>(lane_tot);
    if constexpr (S > 1) {
      // the S segment sums of this row meet in one LDS word; the wave that completes
      // the count holds the row total
      int done = 0;
      if (lane == kWave - 1) {
        const unsigned long long mine = (1ull << 40) + (unsigned long long)(long long)tot;
        const unsigned long long now = atomicAdd(&slots[k * GPW + wave / S], mine) + mine;
        const unsigned long long n = (now + (1ull << 39)) >> 40;
        done = n == (unsigned long long)S;
        tot = (int)(long long)(now - (n << 40));
      }
      const int t = __builtin_amdgcn_readlane(tot, kWave - 1);
      res = lane == nb ? t : res;
      keep |= (unsigned long long)(__builtin_amdgcn_readlane(done, kWave - 1) & 1) << nb;
      nb += 1;
    } else {
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        const int t = __builtin_amdgcn_readlane(tot, r * L + L - 1);
        res = lane == nb + r ? t : res;
      }
      keep |= ((1ull << RW) - 1) << nb;
      nb += RW;
    }
    g += stride;
    ++k;
    if (nb == kWave) flush();
  };
  // Whole rounds of D groups in a loop with a single exit, then the remaining groups
  // (already in flight) straight-line: no exit in the middle of the ring, so the wait
  // before each group is for its own buffer only.
  int left = (glast - g0) / stride + 1;
  while (left >= D) {
#pragma unroll
    for (int d = 0; d < D; ++d) step(d, true);
    left -= D;
  }
#pragma unroll
  for (int d = 0; d < D - 1; ++d)
    if (d < left) step(d, false);
  flush();
}

// MAXI = 2 adds the mapping for rows of more than 256 chunks (two chunks per lane);
// the MAXI = 1 instance leaves it out so that its register budget stays small.
template <int MAXI, int FMT>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(int w1, int w2, int w3, int w4,
                                                            int w5, int w6, int w7, int nslots,
                                                            GemvArgs) {
  extern __shared__ unsigned long long slots[];
  const ArgsPtr a = (ArgsPtr)((const char __attribute__((address_space(4)))*)
                                  __builtin_amdgcn_kernarg_segment_ptr() + kGemvArgsOffset);
  const int wg = (int)blockIdx.x;
  // the starts ascend, unused ones are INT_MAX: the projection is the count of starts <= wg
  const int pi = (wg >= w1) + (wg >= w2) + (wg >= w3) + (wg >= w4) + (wg >= w5) + (wg >= w6) +
                 (wg >= w7);
  const GemvProj P = load_proj(a, pi);
  // the wave index is uniform per wave: readfirstlane keeps the row schedule, the
  // branches and the row bases in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wgl = wg - P.wg0;
  const int ns = P.cfg >= 3 ? nslots : 0;  // combine words to clear (segmented rows)
  const int pb = (8 * nslots + 15) & ~15;  // 1-bit planes after the combine words
  switch (P.cfg) {
    case 0: sweep<16, 1, 1, FMT, MAXI>(P, wgl, wave, slots, pb, ns); break;  // C <= 16
    case 1: sweep<32, 1, 1, FMT, MAXI>(P, wgl, wave, slots, pb, ns); break;  // C <= 32
    case 2: sweep<64, 1, 1, FMT, MAXI>(P, wgl, wave, slots, pb, ns); break;  // C <= 64
    case 3: sweep<64, 1, 2, FMT, MAXI>(P, wgl, wave, slots, pb, ns); break;  // C <= 128
    case 4: sweep<64, 1, 4, FMT, MAXI>(P, wgl, wave, slots, pb, ns); break;  // C <= 256
    default:
      if constexpr (MAXI >= 2) sweep<64, 2, 4, FMT, MAXI>(P, wgl, wave, slots, pb, ns);  // C <= 512
      break;
  }
}

// Workgroups of one instance the device keeps resident at once (queried once per
// instance; the combine words never take enough LDS to change it).
template <int FMT>
int gemv_resident(bool big, size_t lds) {
  static int cached[2] = {0, 0};
  const void* f = big ? (const void*)gemv_kernel<2, FMT> : (const void*)gemv_kernel<1, FMT>;
  return bl_resident_wgs(f, kGemvThreads, lds, 2, &cached[big ? 1 : 0]);
}

}  // namespace bl

using namespace bl;

bool bl_gemv_supports(int T, int K) { return T == 1 && K % 64 == 0 && K / 64 <= kGemvMaxC; }
bool bl_gemv_sign_supports(int T, int K) {
  return T == 1 && K % 128 == 0 && K / 128 <= kGemvMaxC;
}

namespace {
// The partition (bl_plan.h, gemv_plan): a round of part of the resident workgroups,
// shared by the projections in proportion to their bytes (segmented rows weighted
// 1.25x, the costliest first in dispatch order). Measured on the 8B decode layer in one
// allocation (q|k|v, o, gate|up, down): three quarters of a round with two row groups in
// flight per wave beat half a round with three by 4-5% (11.2 against 11.7 us, same box,
// alternating runs; the 70B gate projection 2% faster), and five eighths beat three
// quarters by 1.4% (11.35 against 11.51 us; 70B gate 12.3-12.45 against 12.6, down the
// same; a full round and half a round, or three in flight at three quarters, measured
// slower on the layer); launches with rows of more than 256 chunks keep half a round
// with three in flight (70B down: 5% faster than the other); the 1-bit form keeps half
// a round with four in flight (5% faster than a full round). A partition dispatched
// later gets its first rows later, so in the 2-bit form each partition's cost is raised
// by the fraction of the total dispatched before it (1.5-3% on the 8B layer; the 1-bit
// form measured 5% slower with it).
template <int FMT>
hipError_t launch_gemv_fmt(const bl_proj_internal* p, int count, hipStream_t stream) {
  constexpr int kCodes = FMT == 0 ? 64 : 128;  // codes per 16-byte chunk
  int64_t N[BL_GROUP_CAP], K[BL_GROUP_CAP];
  bool big = false;
  for (int i = 0; i < count; ++i) {
    N[i] = p[i].N;
    K[i] = p[i].K;
    big = big || plan::gemv_cfg((int)(p[i].K / kCodes)).cfg == 5;
  }
  // the prepared activations of the longest row (a record and a sum per chunk) in LDS,
  // which bounds the workgroups a CU keeps resident
  int maxC = 0;
  for (int i = 0; i < count; ++i) maxC = max(maxC, (int)(p[i].K / kCodes));
  const size_t plane_bytes = (size_t)(FMT == 1 ? 128 + 4 : 64 + 4) * maxC;
  int resident = gemv_resident<FMT>(big, 4096);
  {
    static const hipError_t attr1 = hipFuncSetAttribute(
        (const void*)gemv_kernel<1, FMT>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    static const hipError_t attr2 = hipFuncSetAttribute(
        (const void*)gemv_kernel<2, FMT>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr1 != hipSuccess) return attr1;
    if (attr2 != hipSuccess) return attr2;
  }
  // fraction of a round of resident workgroups (numerator, denominator)
  const int rnum = FMT == 0 && !big ? 5 : 1, rden = FMT == 0 && !big ? 8 : 2;
  plan::GemvPlan pl = plan::gemv_plan(N, K, count, kCodes, resident, FMT == 0, rnum, rden);
  {  // fewer workgroups when the activation records' LDS keeps fewer resident
    const size_t need = ((sizeof(unsigned long long) * pl.slots + 15) & ~(size_t)15) + plane_bytes;
    const int cap = bl_device_cus() * max(1, (int)((size_t)160 * 1024 / need));
    if (cap < resident)
      pl = plan::gemv_plan(N, K, count, kCodes, cap, FMT == 0, rnum, rden);
  }
  GemvKernArgs ka{};
  GemvArgs& a = ka.g;
  for (int o = 0; o < count; ++o) {
    const plan::GemvEntry& e = pl.e[o];
    const bl_proj_internal& q = p[e.src];
    GemvProj& g = a.p[o];
    g.Xq = q.Xq;
    g.xs = q.x_scale;
    g.W = reinterpret_cast<const uint4*>(q.W);
    g.ws = q.w_scale;
    g.Y = q.Y;
    g.acc = q.acc;
    g.N = e.N;
    g.C = e.C;
    g.cfg = e.c.cfg;
    g.CW = e.CW;
    g.rpg = q.rpg;
    g.nwg = e.nwg;
    g.wg0 = e.wg0;
    if (o > 0) ka.wg0[o - 1] = e.wg0;
  }
  for (int i = max(count, 1); i < BL_GROUP_CAP; ++i) ka.wg0[i - 1] = INT_MAX;
  a.count = count;
  ka.slots = pl.slots;
  const size_t lds = ((sizeof(unsigned long long) * (size_t)pl.slots + 15) & ~(size_t)15) + plane_bytes;
  const int* w = ka.wg0;
  if (pl.big)
    hipLaunchKernelGGL((gemv_kernel<2, FMT>), dim3((unsigned)pl.wgs), dim3(kGemvThreads), lds, stream,
                       w[0], w[1], w[2], w[3], w[4], w[5], w[6], ka.slots, a);
  else
    hipLaunchKernelGGL((gemv_kernel<1, FMT>), dim3((unsigned)pl.wgs), dim3(kGemvThreads), lds, stream,
                       w[0], w[1], w[2], w[3], w[4], w[5], w[6], ka.slots, a);
  return hipGetLastError();
}
}  // namespace

hipError_t bl_launch_gemv(const bl_proj_internal* p, int count, int T, hipStream_t stream) {
  (void)T;
  return launch_gemv_fmt<0>(p, count, stream);
}

hipError_t bl_launch_gemv_sign(const bl_proj_internal* p, int count, hipStream_t stream) {
  return launch_gemv_fmt<1>(p, count, stream);
}
