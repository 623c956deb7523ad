// bl_skinny.hip -- ternary x int8 product for a few tokens (up to 64 per pass) on int8 MFMA
// (v_mfma_i32_16x16x64_i8), int32 accumulation, fused rescale.
//
// [HF-1.58] "Fine-tuning LLMs to 1.58 bits", "Inference optimization and custom
// kernels": weights stay packed in memory and are unpacked inside the product;
// "Computation paradigm": integer arithmetic only. [bitnet.cpp] "3. BitLinear
// operation": rescale by the weight and activation scales.
//
// With few tokens the product is bound by the packed-weight stream (2 ops per weight per
// token against 1/4 byte per weight). The activations are the only reused operand and
// they are small (T x K bytes), so each wave keeps its share of them in registers and
// streams weight rows past them, like the decode GEMV:
//   - K is cut into segments of 256*MPW codes (MPW = 1, 2, 4 or 7). A workgroup has 8
//     waves: teams of S waves, wave s of a team owning segment s (with more segments
//     than S, the team makes several passes, reloading its activations per pass).
//   - Per wave and segment, the MFMA B operands (16 tokens x 64 codes each: lane (token
//     t, k-slot g) holds 16 activation bytes) live in registers for the whole sweep.
//     They are 4x4 byte-transposed to the order in which a packed dword unpacks, and
//     the code -> k-slot assignment is chosen so that the 16 packed bytes of row
//     lane % 16 at bytes 64m + 16g of the segment are directly the A operand of four
//     MFMAs.
//   - Those 16 rows x 64 bytes are not what a wave loads: every load instruction reads
//     contiguous 16-byte pieces (the wave's segment of row 0, then of row 1, ...), and
//     the wave moves them through its own LDS area (rows padded by 16 bytes) into the
//     MFMA layout. Loading the 16-row layout directly (16 pieces of 64 bytes, one per
//     row, per instruction) measured 8-9% slower at 8-32 tokens.
//   - A team sweeps its row blocks (16 rows each); per row block every wave loads 16
//     rows x 64*MPW bytes with MPW 128-bit buffer loads per lane, kept in a ring D row
//     blocks deep (non-temporal; rows past N and codes past K fall outside the buffer
//     range, so they read as zeros without a memory access or a branch), unpacks
//     u = q + 1 and issues 4*MPW MFMAs per token block, starting from -sum(x) of its
//     segment (sum x*u - sum x = sum x*q; the sum is one MFMA per B operand with an
//     all-ones A, once per pass).
//   - The S partial 16x16 tiles of a row block meet in LDS by ds_add (integer, so the
//     order of arrival does not matter), followed by one arrival count per wave; the
//     wave whose arrival completes the count reads the tile back and stores
//     Y = fp32(acc) * fp32(beta / s_t). One barrier per launch (after the tiles are
//     zeroed): every row block has its own tile for the whole launch (more workgroups
//     when they would not fit).
//   - Workgroups are partitioned among the projections of a grouped call so that each
//     workgroup's packed-weight bytes plus a quarter of its activation bytes are about
//     equal, in one round of resident workgroups.
// MFMA output: lane l, register r holds row 4*(l/16) + r of the block, token l % 16.
#include "bl_device.h"
#include "bl_internal.h"
#include "bl_plan.h"

#include <climits>
#include <cstddef>

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));

// LDS: the partial tiles of a workgroup's row blocks (up to kSkTileKB KiB), then the
// per-wave weight regroup areas (16 rows of 64 * MPW + 16 bytes, sized for MPW = 7);
// all of a CU's LDS is one workgroup's (bl_plan.h)
constexpr int kSkWaves = plan::kSkWaves;
constexpr int kSkThreads = kSkWaves * kWave;  // 512
constexpr size_t kSkLdsMax = plan::kSkLdsMax;
constexpr int kSkLdsCU = plan::kSkLdsCU;
constexpr size_t kSkRegroup = plan::kSkRegroup;

struct SkProj {
  const int8_t* Xq;
  const float* xs;
  const uint8_t* W;
  const float* ws;
  float* Y;
  int32_t* acc;
  int N, K;
  int nrb;       // row blocks of 16
  int mpw;       // a segment is 256 * mpw codes: mpw 128-bit loads per lane and row block
  int nseg;      // segments covering K
  int S, teams;  // waves per team, teams per workgroup
  int npass;     // passes of a team over the segments
  int R;         // row blocks per team
  int rpg;       // rows per weight scale group
  int T;         // tokens of this entry (entries may be token slices of one product)
  int wg0, nwg;
};

struct SkArgs {
  int wg0[plan::kSkEntries];  // first workgroup of each entry (INT_MAX when unused)
  SkProj p[plan::kSkEntries];
  int count;
  int wbase;  // byte offset of the per-wave weight regroup areas in dynamic LDS
};

typedef const SkArgs __attribute__((address_space(4)))* SkArgsPtr;

// The kernel's argument list: the starts of entries 1..7 and the regroup offset come
// first, as scalars, so that they can be preloaded into SGPRs at wave launch (the build
// asks for 8 preloaded dwords): a wave of a launch with up to 8 entries finds its entry
// without a round trip to the argument memory, and the entry's fields are its first
// load. Launches with more entries read the remaining starts from SkArgs.
struct SkKernArgs {
  int wg0[7];  // first workgroup of entries 1..7 (INT_MAX when unused)
  int wbase;
  SkArgs s;
};
constexpr int kSkArgsOffset = 32;
static_assert(offsetof(SkKernArgs, s) == kSkArgsOffset, "argument layout");

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
  P.nrb = a->p[i].nrb;
  P.mpw = a->p[i].mpw;
  P.nseg = a->p[i].nseg;
  P.S = a->p[i].S;
  P.teams = a->p[i].teams;
  P.npass = a->p[i].npass;
  P.R = a->p[i].R;
  P.rpg = a->p[i].rpg;
  P.T = a->p[i].T;
  P.wg0 = a->p[i].wg0;
  P.nwg = a->p[i].nwg;
  return P;
}

// Position of (token, row) in a 16 x 16 tile of ints: rows of one token are contiguous,
// XOR-swizzled so that the 64 lanes of one ds_add (4 rows x 16 tokens) hit distinct
// banks, both as 64 banks and as two halves of 32.
__device__ __forceinline__ int sk_pos(int tok, int row) {
  const int h = ((tok >> 2) & 3) | (((tok >> 1) & 1) << 3);
  return tok * 16 + (row ^ h);
}

typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kOob = 0x80000000u;  // a buffer offset past every range: reads 0, drops writes
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

// Zeroes the partial tiles and arrival counts of a workgroup (every thread takes a share).
__device__ __forceinline__ void sk_clear(int* lds, int words) {
  for (int i = threadIdx.x; i < words; i += kSkThreads) lds[i] = 0;
}

template <int TB, int MPW, int D>
__device__ __forceinline__ void sk_sweep(const SkProj& P, int T, int wgl, int wave, int* tiles,
                                         int* counts, float* facs, uint8_t* wlds, int nclear) {
  constexpr int RS = 64 * MPW + 16;  // LDS bytes per row of the wave's regroup area
  constexpr int PPR = 4 * MPW;       // 16-byte pieces per row segment
  const int lane = threadIdx.x & (kWave - 1), li = lane & 15, lg = lane >> 4;
  const int S = P.S, teams = P.teams;
  const int team = wave / S;
  const int seg = wave - team * S;
  const int R = P.R, npass = P.npass;
  const int nsteps = npass * R;
  const int target = S * npass;  // arrivals that complete a row block
  const int TT = P.nwg * teams;  // teams over the projection
  const int tg = wgl * teams + team;
  const int Kb = P.K >> 2;
  const v4i ones = v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101};
  const Rsrc xr = make_rsrc(P.Xq, (uint32_t)T * (uint32_t)P.K);
  const Rsrc yr = make_rsrc(P.Y, (uint32_t)T * (uint32_t)P.N * 4u);
  const Rsrc ar = make_rsrc(P.acc, P.acc ? (uint32_t)T * (uint32_t)P.N * 4u : 0u);

  // B operands of this wave's segment in pass p (padding tokens and codes past K read
  // as zeros through the buffer range), then minus their per-token sums
  uint4 braw[MPW][4][TB];
  v4i B[MPW][4][TB];
  v4i ncs[TB];
  auto issue_B = [&](int p) {
    const int sg = p * S + seg;
#pragma unroll
    for (int m = 0; m < MPW; ++m)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const int tok = 16 * tb + li;
        const int code = (sg * MPW + m) * 256 + 64 * lg;
        const bool ok = sg < P.nseg && tok < T && code < P.K;
        const uint32_t off = ok ? (uint32_t)tok * (uint32_t)P.K + (uint32_t)code : kOob;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const v4i v = __builtin_amdgcn_raw_buffer_load_b128(xr, off + 16 * i, 0, 0);
          braw[m][i][tb] = make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
        }
      }
  };
  auto finish_B = [&]() {
#pragma unroll
    for (int m = 0; m < MPW; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
          const uint4 v = braw[m][i][tb];
          const uint32_t in[4] = {v.x, v.y, v.z, v.w};
          uint32_t o[4];
          transpose16(in, o);
          B[m][i][tb] = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
        }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      v4i c = v4i{0, 0, 0, 0};
#pragma unroll
      for (int m = 0; m < MPW; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_i32_16x16x64_i8(ones, B[m][i][tb], c, 0, 0, 0);
      ncs[tb] = v4i{0, 0, 0, 0} - c;
    }
  };

  // weight ring: row block rb as a buffer of its (up to) 16 rows, empty past the matrix;
  // the prefetch position (pass, row-block ordinal) advances per load
  // Load m of a row block: piece f = 64m + lane of the wave's 16 x PPR pieces (row f / PPR,
  // piece f % PPR of the row's segment), so each instruction reads contiguous bytes.
  uint4 w[D][MPW];
  uint8_t* const wl = wlds + wave * 16 * RS;
  int fn = 0, fr = 0, fp = 0;
  auto load_w = [&](int d) {
    const int rb = tg + fr * TT;
    const int sg = fp * S + seg;
    const bool valid = fn < nsteps && rb < P.nrb && sg < P.nseg;
    const int rows = valid ? min(16, P.N - rb * 16) : 0;
    const Rsrc wr = make_rsrc(P.W + (valid ? (int64_t)rb * 16 * Kb : 0), (uint32_t)(rows * Kb));
#pragma unroll
    for (int m = 0; m < MPW; ++m) {
      const int f = m * kWave + lane;
      const int r = f / PPR, c = f - (f / PPR) * PPR;
      const int byte = sg * MPW * 64 + 16 * c;
      const uint32_t off = byte < Kb ? (uint32_t)(r * Kb + byte) : kOob;
      const v4i v = __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 2);  // non-temporal
      w[d][m] = make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
    }
    ++fn;
    if (++fr == R) {
      fr = 0;
      ++fp;
    }
  };

  // Set-up: the partial tiles zeroed and the rescale factors fac[t] = beta / s_t stored in
  // LDS, then the workgroup's one barrier, which must come before the first tile add.
  // With one token block the factors' operands, the activations (L2-resident) and the
  // weight ring are asked for first and the set-up runs while they are in flight; the
  // barrier then sits in the first step, so no wave waits for another's loads before
  // its first MFMAs (the 8B layer at 16 tokens 0.2-0.4 us faster). With more token
  // blocks each wave asks for up to 40 KB at once, and the barrier goes first (tying
  // the waves together at their first step measured 2-3% slower at 48-64 tokens). The
  // activation registers are rearranged while the weights are still in flight.
  typedef const float __attribute__((address_space(4)))* ConstF;
  const bool fl = threadIdx.x < 16 * TB;
  bool synced = TB > 1;
  if constexpr (TB > 1) {
    sk_clear(tiles, nclear);
    if (fl) facs[threadIdx.x] = *(ConstF)P.ws / P.xs[min((int)threadIdx.x, T - 1)];
    __syncthreads();
  }
  float fx = 1.0f;
  if constexpr (TB == 1) {
    if (fl) fx = P.xs[min((int)threadIdx.x, T - 1)];
    __builtin_amdgcn_sched_barrier(0);  // that load first, then the activations and ring
  }
  issue_B(0);
#pragma unroll
  for (int d = 0; d < D; ++d) load_w(d);
  if constexpr (TB == 1) {
    __builtin_amdgcn_sched_barrier(0);
    sk_clear(tiles, nclear);
    if (fl) facs[threadIdx.x] = *(ConstF)P.ws / fx;
  }
  finish_B();

  // the loaded pieces of ring slot d into the wave's LDS rows, then back in the MFMA
  // layout (row li, bytes 64m + 16lg); the wavefront fences keep the reads after every
  // lane's writes
  uint4 wa[MPW];
  auto regroup = [&](int d) {
#pragma unroll
    for (int m = 0; m < MPW; ++m) {
      const int f = m * kWave + lane;
      const int r = f / PPR, c = f - (f / PPR) * PPR;
      *reinterpret_cast<uint4*>(wl + r * RS + 16 * c) = w[d][m];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int m = 0; m < MPW; ++m)
      wa[m] = *reinterpret_cast<const uint4*>(wl + li * RS + 64 * m + 16 * lg);
  };
  if constexpr (TB == 1) regroup(0);
  const bool vec_store = (P.N & 3) == 0;
  int cr = 0, cp = 0;
  auto step = [&](int d, bool prefetch) {
    v4i acc[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[tb] = ncs[tb];
    // up to 16 tokens the slot was regrouped at the end of the previous step
    if constexpr (TB > 1) regroup(d);
    const bool more = cp * R + cr + 1 < nsteps;
#pragma unroll
    for (int m = 0; m < MPW; ++m) {
      const uint32_t wd[4] = {wa[m].x, wa[m].y, wa[m].z, wa[m].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t u[4];
        unpack_u2(wd[i], u);
        const v4i ua = v4i{(int)u[0], (int)u[1], (int)u[2], (int)u[3]};
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
          acc[tb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ua, B[m][i][tb], acc[tb], 0, 0, 0);
      }
    }
    if (prefetch) load_w(d);
    // one token block: the next slot's regroup runs here, under this step's MFMAs (1-2%
    // faster at 8-16 tokens; with two token blocks it measured slower)
    if constexpr (TB == 1) {
      if (more) regroup((d + 1) % D);
    }
    if (!synced) {  // one token block: the first step of every wave (see the set-up)
      __syncthreads();
      synced = true;
    }
    // partial tile into LDS, then one arrival; the wave that completes the count owns
    // the sum (every earlier arrival's adds were performed before its count)
    const int slot = team * R + cr;
    int* tile = tiles + slot * TB * 256;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        __hip_atomic_fetch_add(tile + tb * 256 + sk_pos(li, 4 * lg + r), acc[tb][r],
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    int old = 0;
    if (lane == 0)
      old = __hip_atomic_fetch_add(counts + slot, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old == target - 1) {
      const int rb = tg + cr * TT;
      const int row = rb * 16 + 4 * lg;
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const int t = 16 * tb + li;
        int v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          v[r] = __hip_atomic_load(tile + tb * 256 + sk_pos(li, 4 * lg + r), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
        float f = facs[t];
        const bool tin = t < T;
        float fr[4] = {f, f, f, f};
        if (P.rpg < P.N) {  // weight scale groups: the scale of each row's group
#pragma unroll
          for (int r = 0; r < 4; ++r) fr[r] = P.ws[min(row + r, P.N - 1) / P.rpg] / P.xs[min(t, T - 1)];
        }
        if (vec_store) {
          const uint32_t off = tin && row < P.N ? ((uint32_t)t * (uint32_t)P.N + (uint32_t)row) * 4u : kOob;
          const v4i y = v4i{__float_as_int((float)v[0] * fr[0]), __float_as_int((float)v[1] * fr[1]),
                            __float_as_int((float)v[2] * fr[2]), __float_as_int((float)v[3] * fr[3])};
          __builtin_amdgcn_raw_buffer_store_b128(y, yr, off, 0, 0);
          if (P.acc) __builtin_amdgcn_raw_buffer_store_b128(v4i{v[0], v[1], v[2], v[3]}, ar, off, 0, 0);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t off =
                tin && row + r < P.N ? ((uint32_t)t * (uint32_t)P.N + (uint32_t)(row + r)) * 4u : kOob;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_int((float)v[r] * fr[r]), yr, off, 0, 0);
            if (P.acc) __builtin_amdgcn_raw_buffer_store_b32(v[r], ar, off, 0, 0);
          }
        }
      }
    }
    if (++cr == R) {
      cr = 0;
      ++cp;
      if (npass > 1 && cp < npass) {
        issue_B(cp);
        finish_B();
      }
    }
  };
  // whole rounds of D steps, then the rest (single exit, static ring slots)
  int n = 0;
  while (nsteps - n >= D) {
#pragma unroll
    for (int d = 0; d < D; ++d) step(d, true);
    n += D;
  }
#pragma unroll
  for (int d = 0; d < D - 1; ++d)
    if (n + d < nsteps) step(d, false);
}

template <int TB>
__global__ __launch_bounds__(kSkThreads) void skinny_kernel(int w1, int w2, int w3, int w4, int w5,
                                                             int w6, int w7, int wbase, SkArgs) {
  extern __shared__ int sk_lds[];
  const SkArgsPtr a = (SkArgsPtr)((const char __attribute__((address_space(4)))*)
                                      __builtin_amdgcn_kernarg_segment_ptr() + kSkArgsOffset);
  const int wg = (int)blockIdx.x;
  // the starts ascend, unused ones are INT_MAX: the entry is the count of starts <= wg
  int pi = (wg >= w1) + (wg >= w2) + (wg >= w3) + (wg >= w4) + (wg >= w5) + (wg >= w6) + (wg >= w7);
  if (pi == 7) {
#pragma unroll
    for (int i = 8; i < plan::kSkEntries; ++i) pi += wg >= a->wg0[i] ? 1 : 0;
  }
  const SkProj P = load_sk(a, pi);
  const int T = P.T;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wgl = wg - P.wg0;
  const int nslot = P.teams * P.R;
  const int nclear = nslot * (TB * 256 + 1);
  int* tiles = sk_lds;
  int* counts = sk_lds + nslot * TB * 256;
  float* facs = reinterpret_cast<float*>(counts + nslot);
  // Every wave passes exactly one barrier: in its sweep (in the set-up, or in the first
  // step with one token block: a working wave has at least one step), or here (leftover
  // waves without a segment, and segment lengths no plan gives).
  uint8_t* const wlds = reinterpret_cast<uint8_t*>(sk_lds) + wbase;
  bool swept = false;
  if (wave < P.S * P.teams) {
    swept = true;
    switch (P.mpw) {
      case 1: sk_sweep<TB, 1, 4>(P, T, wgl, wave, tiles, counts, facs, wlds, nclear); break;
      case 2: sk_sweep<TB, 2, 4>(P, T, wgl, wave, tiles, counts, facs, wlds, nclear); break;
      case 4:
        if constexpr (TB <= 2) sk_sweep<TB, 4, 3>(P, T, wgl, wave, tiles, counts, facs, wlds, nclear);
        else swept = false;
        break;
      default:
        if constexpr (TB == 1) sk_sweep<TB, 7, 2>(P, T, wgl, wave, tiles, counts, facs, wlds, nclear);
        else swept = false;
        break;
    }
  }
  if (!swept) {
    sk_clear(sk_lds, nclear);
    __syncthreads();
  }
}

// (always asked with the same LDS size, so one cached value per instance)
template <int TB>
int sk_resident(size_t lds) {
  static int cached = 0;
  return bl_resident_wgs((const void*)skinny_kernel<TB>, kSkThreads, lds, 1, &cached);
}

// The dynamic-LDS limit is raised once per instance (first launch), never inside a
// stream capture after that.
template <int TB>
hipError_t launch_skinny_t(const bl_proj_internal* p, int count, const int* T, hipStream_t stream) {
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)skinny_kernel<TB>, hipFuncAttributeMaxDynamicSharedMemorySize, kSkLdsCU);
  if (attr != hipSuccess) return attr;
  // one workgroup per CU: its registers and, with the regroup areas, its LDS bound it
  const int cap = sk_resident<TB>(kSkLdsMax + 16 + kSkRegroup);
  int64_t N[plan::kSkEntries], K[plan::kSkEntries];
  for (int i = 0; i < count; ++i) {
    N[i] = p[i].N;
    K[i] = p[i].K;
  }
  const plan::SkPlan pl = plan::skinny_plan(N, K, count, TB, cap, T);
  if (!pl.fits) return hipErrorInvalidValue;
  SkArgs a{};
  for (int i = 0; i < count; ++i) {
    const plan::SkEntry& e = pl.e[i];
    SkProj& s = a.p[i];
    s.Xq = p[i].Xq;
    s.xs = p[i].x_scale;
    s.W = p[i].W;
    s.ws = p[i].w_scale;
    s.Y = p[i].Y;
    s.acc = p[i].acc;
    s.N = e.N;
    s.K = e.K;
    s.nrb = e.nrb;
    s.rpg = p[i].rpg;
    s.T = T[i];
    s.mpw = e.mpw;
    s.nseg = e.nseg;
    s.S = e.S;
    s.teams = e.teams;
    s.npass = e.npass;
    s.R = e.R;
    s.nwg = e.nwg;
    s.wg0 = e.wg0;
    a.wg0[i] = e.wg0;
  }
  for (int i = count; i < plan::kSkEntries; ++i) a.wg0[i] = INT_MAX;
  a.count = count;
  a.wbase = pl.wbase;
  const int wgs = pl.wgs;
  const size_t lds = pl.lds;
  const int* w = a.wg0;
  hipLaunchKernelGGL(skinny_kernel<TB>, dim3((unsigned)wgs), dim3(kSkThreads), lds, stream, w[1], w[2],
                     w[3], w[4], w[5], w[6], w[7], a.wbase, a);
  return hipGetLastError();
}

}  // namespace bl

using namespace bl;

// Output offsets of one pass (64 tokens) are 32-bit buffer offsets.
bool bl_skinny_supports(int T, int64_t N, int K) {
  return T >= 1 && T <= 128 && K % 256 == 0 && N * 64 * 4 < (int64_t(1) << 31);
}

// Token blocks per slice for a pass of tn tokens over a projection of N x K: the slices
// of one pass are entries of one grouped launch that read the same weights, so a slice
// beyond the first mostly re-reads them from the caches while each slice keeps its
// activations in one pass over K (wide slices reload theirs per pass when 256 * MPW
// codes per wave do not cover K). Measured on one box (us per product, graph replays,
// rotating weight copies, bit-identical outputs), one slice / halves of 32 / slices of 16:
//   N x K, packed bytes       24 tokens          32 tokens          48 tokens          64 tokens
//   28672 x 8192, 58.7 MB     20.9 / - / 22.9    22.4 / - / 22.6    30.8 / 30.6 / 38.4 33.7 / 29.8 / 35.1
//   28672 x 4096, 29.4 MB     15.5 / - / 14.6    16.9 / - / 14.7    20.4 / 20.9 / 21.3 21.1 / 21.2 / 21.6
//   4096 x 14336, 14.7 MB     15.9 / - / 13.5    18.6 / - / 13.6    27.3 / 21.9 / 16.5 32.6 / 21.1 / 16.9
//   6144 x 4096, 12.6 MB      10.2 / - / 8.4     11.5 / - / 8.6     11.4 / 12.9 / 10.0 12.8 / 13.1 / 10.3
// So: slices of 16 for long rows (K >= 14336) and small matrices (up to 16 MB, or up to
// 32 MB for at most 32 tokens); halves of 32 for larger matrices beyond 32 tokens;
// otherwise one slice.
static int sk_slice_tb(int tn, int64_t N, int64_t K) {
  const int64_t bytes = N * (K / 4);
  const int one = tn <= 16 ? 1 : tn <= 32 ? 2 : 4;
  if (tn <= 16) return 1;
  if (K >= 14336 || bytes <= ((int64_t)16 << 20)) return 1;
  if (tn <= 32) return bytes <= ((int64_t)32 << 20) ? 1 : 2;
  return bytes > ((int64_t)32 << 20) ? 2 : one;
}

// Up to 64 tokens in one launch, more as passes of 64 (each pass streams the weights
// again: the caller's choice when the GEMM's tiles would leave most of the device idle).
// A pass of tn tokens runs as slices of 16 * TB tokens, each slice an entry of one
// grouped launch of the TB kernel (the last slice ragged); the largest projection of a
// grouped call picks TB.
hipError_t bl_launch_skinny(const bl_proj_internal* p, int count, int T, hipStream_t stream) {
  for (int t0 = 0; t0 < T; t0 += 64) {
    const int tn = T - t0 < 64 ? T - t0 : 64;
    int big = 0;
    for (int i = 1; i < count; ++i)
      if ((int64_t)p[i].N * p[i].K > (int64_t)p[big].N * p[big].K) big = i;
    const int whole = tn <= 16 ? 1 : tn <= 32 ? 2 : 4;  // one slice
    int TB = sk_slice_tb(tn, p[big].N, p[big].K);
    const int per = 16 * TB, slices = (tn + per - 1) / per, last = tn - (slices - 1) * per;
    // a short last slice costs nearly a full pass over the weights (the 8B layer's seven
    // projections at 17 / 20 / 24 tokens: 26.0 / 25.4 / 24.3 us in slices of 16 against
    // 21.2 / 22.1 / 23.3 in one, 24.8 against 26.5 at 32): slices need a last one of at
    // least 8 tokens, and in a grouped call (whose many partitions do not keep the
    // slices' workgroups on the same XCDs) every slice full
    if (slices * count > plan::kSkEntries || last < 8 || (count > 1 && last < per)) TB = whole;
    const int ns = (tn + 16 * TB - 1) / (16 * TB);
    bl_proj_internal q[plan::kSkEntries];
    int Ts[plan::kSkEntries];
    int n = 0;
    for (int i = 0; i < count; ++i)
      for (int j = 0; j < ns; ++j) {
        const int a = t0 + j * 16 * TB, tj = min(16 * TB, t0 + tn - a);
        q[n] = p[i];
        q[n].Xq += (int64_t)a * p[i].K;
        q[n].x_scale += a;
        q[n].Y += (int64_t)a * p[i].N;
        if (q[n].acc) q[n].acc += (int64_t)a * p[i].N;
        Ts[n++] = tj;
      }
    const hipError_t e = TB == 1   ? launch_skinny_t<1>(q, n, Ts, stream)
                         : TB == 2 ? launch_skinny_t<2>(q, n, Ts, stream)
                                   : launch_skinny_t<4>(q, n, Ts, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
