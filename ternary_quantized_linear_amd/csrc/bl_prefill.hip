// bl_prefill.hip -- ternary x int8 GEMM for long token counts (prefill) on int8 MFMA
// (v_mfma_i32_32x32x32_i8), int32 accumulation, fused rescale.
//
// [HF-1.58] "Fine-tuning LLMs to 1.58 bits", "Tiled matrix multiplication": the
// matrices are split into tiles held in fast on-chip memory to cut global-memory
// traffic; "Inference optimization and custom kernels": 2-bit weights unpacked on
// the fly. [bitnet.cpp] "3. BitLinear operation": rescale of the integer product.
//
// Y[T, N] = Xq[T, K] * q[N, K]^T in tiles of BM tokens x BN weight rows, 4 waves per
// workgroup, k-tiles of 128 codes. Two kernels:
//
// prefill_big_kernel (problems that give every CU at least one 128 x 256 tile): waves
// side by side along the rows (each 128 tokens x 64 rows), weights kept packed in LDS
// and unpacked by each wave in registers as u = q + 1 in {0, 1, 2}, with the token sums
// sum_k x subtracted in the epilogue; two LDS stages (one barrier per k-tile) and two
// register sets, so that the global loads of k-tile kt + 2 and the staging of kt + 1
// both run under the MFMAs of k-tile kt. Described in full above the kernel.
//
// prefill_kernel (smaller problems; 2 x 2 waves, one LDS stage, two workgroups per CU):
//   - weights: BN x 32 packed bytes, unpacked ONCE per workgroup to signed int8
//     (unpack_q2, v_perm_b32 table) and written to LDS in the activations' swizzled
//     layout, so every wave reads both operands with plain 128-bit LDS reads;
//   - the next k-tile is loaded from global memory into registers while the MFMAs of
//     the current one run, then written over it between two barriers.
//
// Both: activations are staged as whole 128-byte row segments (8 lanes per row:
// scattered 64-byte pieces cost the cache path about three times as much), each 16-byte
// group 4x4 byte-transposed to the unpack order, groups XOR-swizzled by row
// (conflict-free 128-bit reads and writes). Workgroups are numbered XCD-major: the tiles
// one XCD (one L2) runs are consecutive token tiles of the same weight tiles.
// Epilogue: Y = fp32(acc) * fp32(beta / s_t), the sixteen factors of a lane read from LDS
// before its stores.
#include "bl_device.h"
#include "bl_internal.h"
#include "bl_plan.h"

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kPfThreads = 256;
constexpr int kPfKT = 128;  // codes per k-tile = bytes per staged row

typedef __amdgpu_buffer_rsrc_t PfRsrc;

// A raw buffer resource over [base, base + bytes): reads past the range return zeros.
__device__ __forceinline__ PfRsrc pf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// LDS position of 16-byte group g (0..7) of staged row t: rows are 128 bytes and the
// group index is XORed with bits 1..3 of the row, so that 16 lanes reading one group
// of 16 consecutive rows, or writing the eight groups of 2 consecutive rows, hit 16
// distinct 4-bank slots.
__device__ __forceinline__ int pf_pos(int t, int g) {
  return t * kPfKT + 16 * (g ^ ((t >> 1) & 7));
}

struct PfArgs {
  const int8_t* Xq;
  const float* xs;
  const uint8_t* W;
  const float* ws;
  float* Y;
  int32_t* acc;
  int T, N, K;
  int tiles_m, tiles_n;
  int per_xcd;  // logical tiles per XCD
  int rpg;      // rows per weight scale group
  // split K (large-tile kernel only): workgroup slice p of P covers k-tiles
  // [p * ktn, min((p + 1) * ktn, K / 128)) and, with P > 1, writes its exact partial
  // products to part[p][t][n] (int32) instead of the epilogue
  int P, ktn;
  int32_t* part;
};

// Epilogue of one 32 x 32 accumulator block (v_mfma_i32_32x32x32_i8 D layout): the lane
// holds output row n and tokens tb + 8q + e (q, e = 0..3) in c[4q + e]. fac[] holds
// fp32(beta / s_t) of the tile's tokens for the scale group of the tile's first row, and
// sub[] the amounts to subtract from the integer sums (or null). The sixteen factors and
// sums are read before any store (four 128-bit LDS reads each); a tile that lies inside
// T, N and one scale group stores without per-element checks.
__device__ __forceinline__ void pf_store_block(const PfArgs& a, const v16i& c, int m0, int n0,
                                               int tb, int n, const float* fac, const int* sub,
                                               bool full) {
  float f[16];
  int d[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = *reinterpret_cast<const float4*>(fac + tb + 8 * q);
    f[4 * q] = v.x; f[4 * q + 1] = v.y; f[4 * q + 2] = v.z; f[4 * q + 3] = v.w;
    if (sub) {
      const int4 w = *reinterpret_cast<const int4*>(sub + tb + 8 * q);
      d[4 * q] = w.x; d[4 * q + 1] = w.y; d[4 * q + 2] = w.z; d[4 * q + 3] = w.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) d[4 * q + e] = 0;
    }
  }
  float* yp = a.Y + (int64_t)(m0 + tb) * a.N + n;
  int32_t* ap = a.acc ? a.acc + (int64_t)(m0 + tb) * a.N + n : nullptr;
  if (full) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int dt = 8 * (r >> 2) + (r & 3);
      const int v = c[r] - d[r];
      yp[(int64_t)dt * a.N] = (float)v * f[r];
      if (ap) ap[(int64_t)dt * a.N] = v;
    }
    return;
  }
  if (n >= a.N) return;
  // rows of another scale group than the tile's first row divide their own scale
  const bool own = n / a.rpg == n0 / a.rpg;
  const float wsn = own ? 0.0f : a.ws[n / a.rpg];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int dt = 8 * (r >> 2) + (r & 3);
    const int t = m0 + tb + dt;
    if (t < a.T) {
      const int v = c[r] - d[r];
      yp[(int64_t)dt * a.N] = (float)v * (own ? f[r] : wsn / a.xs[t]);
      if (ap) ap[(int64_t)dt * a.N] = v;
    }
  }
}

template <int BM, int BN>
__global__ __launch_bounds__(kPfThreads, 2) void prefill_kernel(PfArgs a) {
  constexpr int WM = BM / 2, WN = BN / 2, MI = WM / 32, NI = WN / 32;
  constexpr int XQ = BM * (kPfKT / 16) / kPfThreads;       // 16-byte activation pieces per thread
  constexpr int WQ = BN * (kPfKT / 4 / 16) / kPfThreads;   // 16-byte packed weight pieces per thread
  static_assert(XQ >= 1 && WQ >= 1, "tile does not fit the thread count");
  __shared__ __attribute__((aligned(16))) uint8_t xs_l[BM * kPfKT];
  __shared__ __attribute__((aligned(16))) uint8_t ws_l[BN * kPfKT];
  __shared__ __attribute__((aligned(16))) float fac[BM];

  // XCD-major numbering: workgroup b runs on XCD b % 8
  const int bid = (int)blockIdx.x;
  const int tile = plan::xcd_tile(bid, a.per_xcd);
  if (tile >= a.tiles_m * a.tiles_n) return;
  const int tm = tile % a.tiles_m, tn = tile / a.tiles_m;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = tm * BM, n0 = tn * BN;
  const int Kb = a.K >> 2;
  const int nk = a.K / kPfKT;
  const float beta = a.ws[n0 / a.rpg];
  for (int i = tid; i < BM; i += kPfThreads) {
    const int t = m0 + i;
    fac[i] = t < a.T ? beta / a.xs[t] : 0.0f;
  }

  // Global sources (rows clamped into range; clamped rows are never stored). Eight
  // consecutive lanes read the 128 bytes of one activation row (a wave instruction: 8
  // whole rows of the k-tile); two lanes the 32 packed bytes of one weight row.
  const int8_t* xsrc[XQ];
  int xdst[XQ];
#pragma unroll
  for (int r = 0; r < XQ; ++r) {
    const int q = tid + kPfThreads * r, t = q >> 3, g = q & 7;
    xsrc[r] = a.Xq + (int64_t)min(m0 + t, a.T - 1) * a.K + 16 * g;
    xdst[r] = pf_pos(t, g);
  }
  const uint8_t* wsrc[WQ];
  int wrow[WQ], wh[WQ];
#pragma unroll
  for (int r = 0; r < WQ; ++r) {
    const int q = tid + kPfThreads * r;
    wrow[r] = q >> 1;
    wh[r] = q & 1;
    wsrc[r] = a.W + (int64_t)min(n0 + wrow[r], a.N - 1) * Kb + 16 * wh[r];
  }
  // the next k-tile waits in registers while the MFMAs of the current one run; past the
  // last k-tile the loads repeat it (in range, never stored), so no load is under a branch
  uint4 xr[XQ], wr[WQ];
  auto load_tile = [&](int kt) {
    kt = min(kt, nk - 1);
#pragma unroll
    for (int r = 0; r < XQ; ++r) xr[r] = *reinterpret_cast<const uint4*>(xsrc[r] + kt * kPfKT);
#pragma unroll
    for (int r = 0; r < WQ; ++r) wr[r] = *reinterpret_cast<const uint4*>(wsrc[r] + kt * (kPfKT / 4));
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int r = 0; r < XQ; ++r) {
      const uint32_t in[4] = {xr[r].x, xr[r].y, xr[r].z, xr[r].w};
      uint32_t o[4];
      transpose16(in, o);
      *reinterpret_cast<uint4*>(&xs_l[xdst[r]]) = make_uint4(o[0], o[1], o[2], o[3]);
    }
#pragma unroll
    for (int r = 0; r < WQ; ++r) {
      const uint32_t pw[4] = {wr[r].x, wr[r].y, wr[r].z, wr[r].w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t q[4];
        unpack_q2(pw[d], q);
        *reinterpret_cast<uint4*>(&ws_l[pf_pos(wrow[r], 4 * wh[r] + d)]) =
            make_uint4(q[0], q[1], q[2], q[3]);
      }
    }
  };

  v16i acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  const int li = lane & 31, lg = lane >> 5;
  load_tile(0);
  store_tile();
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    load_tile(kt + 1);
#pragma unroll
    for (int s = 0; s < kPfKT / 32; ++s) {
      v4i af[MI], bf[NI];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const uint4 x = *reinterpret_cast<const uint4*>(&xs_l[pf_pos(wm * WM + i * 32 + li, 2 * s + lg)]);
        af[i] = v4i{(int)x.x, (int)x.y, (int)x.z, (int)x.w};
      }
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const uint4 w = *reinterpret_cast<const uint4*>(&ws_l[pf_pos(wn * WN + j * 32 + li, 2 * s + lg)]);
        bf[j] = v4i{(int)w.x, (int)w.y, (int)w.z, (int)w.w};
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();  // every wave is done reading the tile
    store_tile();     // past the last tile: written, never read
    __syncthreads();
  }

  // D[token][row]: lane holds row li of the 32 x 32 block, tokens 8*(r/4) + 4*lg + r%4.
  const bool full = m0 + BM <= a.T && n0 + BN <= a.N && n0 / a.rpg == (n0 + BN - 1) / a.rpg;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      pf_store_block(a, acc[i][j], m0, n0, wm * WM + i * 32 + 4 * lg, n0 + wn * WN + j * 32 + li,
                     fac, nullptr, full);
      __builtin_amdgcn_sched_barrier(0);
    }
}

// Large tiles for large problems: 4 waves in a WY x WX grid (WY along tokens), each
// computing (32 MI) x (32 NI); BM = 32 MI WY, BN = 32 NI WX. One k-tile is 128 codes.
//   - The weights stay packed in LDS (32 bytes per row and k-tile, a quarter of the
//     unpacked bytes) and each wave unpacks the fragments it multiplies in registers.
//     With WY = 1 no two waves unpack the same rows.
//   - The MFMAs take the unsigned codes u = q + 1 in {0, 1, 2} (four masks and three
//     shifts per packed dword, no sign conversion), so the integer product is
//     sum_k x u = acc + sum_k x; the per-token sums sum_k x come from the activation
//     bytes as they are staged (one v_dot4 per dword) and are subtracted in the
//     epilogue. All of it is exact integer arithmetic.
//   - Two LDS stages and a ring of RD register sets: during the MFMAs of k-tile kt,
//     k-tile kt + 1 is staged from its register set into the other LDS stage and the
//     set is refilled at once with k-tile kt + 1 + RD, in three parts spread over the
//     MFMA steps; one barrier per k-tile. A load so has RD k-tiles to arrive (a second
//     set that is loaded while the first is staged would give it one): the big tiles
//     take RD = 2 at two workgroups per CU and 3 at one, the few-token tiles, with one
//     workgroup per CU and little work per k-tile, a deeper ring.
//   - Split K (a.P > 1): workgroup tile and slice come from one index (the tiles of a
//     slice adjacent, so an XCD's workgroups share activation k-tiles); the slice's
//     exact partial (token sums already subtracted) goes to plane p of a.part, and
//     splitk_reduce_kernel sums the planes and rescales.
//
// Order of the codes: the 128 codes of a k-tile are the eight packed dwords d0..d7 of a
// row (dword d = codes 16d..16d+15). MFMA step s (s = 0..3) takes dword 4 lg + s in lane
// half lg (the sum over k does not depend on which codes a step takes, as long as both
// operands take the same ones), so the packed row is staged in LDS as it is in memory
// and lane half lg reads its four steps in one 128-bit read; the activations of step s
// in half lg are 16-byte group 4 lg + s of the staged token row.
template <int MI, int NI, int WY, int OCC, int RD>
__global__ __launch_bounds__(kPfThreads, OCC) void prefill_big_kernel(PfArgs a) {
  constexpr int WX = 4 / WY;
  constexpr int WM = 32 * MI, WN = 32 * NI, BM = WM * WY, BN = WN * WX;
  constexpr int XQ = BM * (kPfKT / 16) / kPfThreads;  // 16-byte activation pieces per thread
  constexpr int WQ = BN * 2 / kPfThreads;             // 16-byte packed halves per thread
  constexpr int XB = BM * kPfKT, WB = BN * (kPfKT / 4), SB = XB + WB;
  static_assert(WY * WX == 4 && XQ >= 1 && WQ >= 1, "tile does not fit the thread count");
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * SB];
  __shared__ __attribute__((aligned(16))) float fac[BM];
  __shared__ __attribute__((aligned(16))) int xsum[BM];

  const int bid = (int)blockIdx.x;
  const int tile = plan::xcd_tile(bid, a.per_xcd);
  const int mn = a.tiles_m * a.tiles_n;
  if (tile >= mn * a.P) return;
  const int sl = tile / mn, tmn = tile - sl * mn;  // K slice; tiles of one slice adjacent
  const int tm = tmn % a.tiles_m, tn = tmn / a.tiles_m;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int wm = wave / WX, wn = wave % WX;
  const int m0 = tm * BM, n0 = tn * BN;
  const int Kb = a.K >> 2;
  const int kb = sl * a.ktn;                      // first k-tile of the slice
  const int nk = min(a.ktn, a.K / kPfKT - kb);    // k-tiles of the slice (>= 1)
  const float beta = a.ws[n0 / a.rpg];
  for (int i = tid; i < BM; i += kPfThreads) {
    const int t = m0 + i;
    fac[i] = t < a.T ? beta / a.xs[t] : 0.0f;
  }

  // Staging. Activation piece r of a thread: row tid/8 + 32r, 16-byte group tid%8 (eight
  // lanes read one 128-byte row segment); its LDS slot is pf_pos, whose swizzle term
  // depends on the row only through (tid/8 / 2) % 8, the same for every r. Packed
  // weight half r: row tid/2 + 128r, half tid%2 (dwords 4h..4h+3). Both are buffer loads
  // through a resource that covers the tile's rows: one 32-bit offset per thread plus a
  // uniform term per piece and k-tile (64-bit pointers per piece cost the registers
  // that the MFMA fragments need), and rows past T or N read zeros without a memory
  // access (they are never stored).
  const int xt = tid >> 3, xg = tid & 7;
  const PfRsrc xrs = pf_rsrc(a.Xq + (int64_t)m0 * a.K, (uint32_t)min(BM, a.T - m0) * (uint32_t)a.K);
  const uint32_t xvo = (uint32_t)xt * (uint32_t)a.K + 16u * (uint32_t)xg;  // + 32 r K + 128 kt
  const int xdst = pf_pos(xt, xg);  // + 32 r rows = + 4096 r bytes
  const int wt = tid >> 1, wh = tid & 1;
  const PfRsrc wrs = pf_rsrc(a.W + (int64_t)n0 * Kb, (uint32_t)min(BN, a.N - n0) * (uint32_t)Kb);
  const uint32_t wvo = (uint32_t)wt * (uint32_t)Kb + 16u * (uint32_t)wh;   // + 128 r Kb + 32 kt
  const int wdst = XB + wt * 32 + 16 * wh;  // + 128 r rows = + 4096 r bytes

  // The register ring: k-tile j lives in set j % RD from its load until it is staged.
  // Items 0..XQ-1 are activation pieces, XQ..XQ+WQ-1 packed weight halves; they are
  // staged and reloaded in three parts spread over the MFMA steps.
  constexpr int NITEM = XQ + WQ;
  static_assert(RD >= 2, "ring depth");
  struct Regs { uint4 v[NITEM]; };
  Regs ring[RD];
  int rs[XQ];  // this thread's part of the token sums sum_k x
#pragma unroll
  for (int r = 0; r < XQ; ++r) rs[r] = 0;
  auto load_part = [&](Regs& R, int kt, int part) {
    kt = kb + min(kt, nk - 1);  // past the slice's last k-tile: reload it (never read back)
#pragma unroll
    for (int q = 0; q < NITEM; ++q) {
      if (q * 3 / NITEM != part) continue;
      const uint32_t off = q < XQ ? xvo + (uint32_t)(32 * q) * (uint32_t)a.K + (uint32_t)kt * kPfKT
                                  : wvo + (uint32_t)(128 * (q - XQ)) * (uint32_t)Kb + (uint32_t)kt * (kPfKT / 4);
      const v4i v = __builtin_amdgcn_raw_buffer_load_b128(q < XQ ? xrs : wrs, off, 0, 0);
      R.v[q] = make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
    }
  };
  auto store_part = [&](const Regs& R, uint8_t* st, bool count, int part) {
#pragma unroll
    for (int q = 0; q < NITEM; ++q) {
      if (q * 3 / NITEM != part) continue;
      if (q < XQ) {
        const uint32_t in[4] = {R.v[q].x, R.v[q].y, R.v[q].z, R.v[q].w};
        if (count) {
#pragma unroll
          for (int d = 0; d < 4; ++d)
            rs[q] = __builtin_amdgcn_sdot4((int)in[d], 0x01010101, rs[q], false);
        }
        uint32_t o[4];
        transpose16(in, o);
        *reinterpret_cast<uint4*>(st + xdst + 4096 * q) = make_uint4(o[0], o[1], o[2], o[3]);
      } else {
        // the packed half as loaded: no register moves between the load and the store
        *reinterpret_cast<uint4*>(st + wdst + 4096 * (q - XQ)) = R.v[q];
      }
    }
  };

  v16i acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  // Reads. Activation fragment i at step s: row wm WM + 32 i + li, group 4 lg + s; the
  // swizzle term ((row / 2) % 8) reduces to (li / 2) % 8, so the four per-step offsets
  // are per-lane constants and i adds 4096 i.
  const int li = lane & 31, lg = lane >> 5;
  const int sw = (li >> 1) & 7;
  int xo[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) xo[s] = (wm * WM + li) * kPfKT + 16 * ((4 * lg + s) ^ sw);
  const int wo = XB + (wn * WN + li) * 32 + 16 * lg;  // + 1024 j

  // One MFMA step s reads MI activation fragments and unpacks NI weight dwords. The
  // fragments of step s + 1 are read and unpacked while the MFMAs of step s run (two
  // fragment sets; the scheduling barriers keep the compiler from hoisting every read of
  // the k-tile, which would need more registers than the wave has).
  auto read_step = [&](const uint8_t* st, const uint4 (&pk)[NI], int s, v4i (&af)[MI],
                       v4i (&bf)[NI]) {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const uint4 x = *reinterpret_cast<const uint4*>(st + xo[s] + 4096 * i);
      af[i] = v4i{(int)x.x, (int)x.y, (int)x.z, (int)x.w};
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const uint32_t w = s == 0 ? pk[j].x : s == 1 ? pk[j].y : s == 2 ? pk[j].z : pk[j].w;
      uint32_t u[4];
      unpack_u2(w, u);
      bf[j] = v4i{(int)u[0], (int)u[1], (int)u[2], (int)u[3]};
    }
  };
  auto mfma_step = [&](const v4i (&af)[MI], const v4i (&bf)[NI]) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
  };
  // One k-tile kt from LDS stage kt % 2: step-0 reads, then four MFMA steps; under
  // them, k-tile kt + 1 is staged from register set S into the other LDS stage and S is
  // reloaded with k-tile kt + 1 + RD, part by part.
  auto compute = [&](int kt, Regs& S) {
    const uint8_t* st = lds + SB * (kt & 1);
    uint8_t* nx = lds + SB * ((kt + 1) & 1);
    const bool count = kt + 1 < nk;  // past the last k-tile: staged, never read or counted
    uint4 pk[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) pk[j] = *reinterpret_cast<const uint4*>(st + wo + 1024 * j);
    v4i a0[MI], b0[NI], a1[MI], b1[NI];
    read_step(st, pk, 0, a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    // in each step: the next step's fragment reads go out before this step's MFMAs
    read_step(st, pk, 1, a1, b1);
    mfma_step(a0, b0);
    store_part(S, nx, count, 0);
    load_part(S, kt + 1 + RD, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, MI, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, MI * NI, 0);
    __builtin_amdgcn_sched_barrier(0);
    read_step(st, pk, 2, a0, b0);
    mfma_step(a1, b1);
    store_part(S, nx, count, 1);
    load_part(S, kt + 1 + RD, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, MI, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, MI * NI, 0);
    __builtin_amdgcn_sched_barrier(0);
    read_step(st, pk, 3, a1, b1);
    mfma_step(a0, b0);
    store_part(S, nx, count, 2);
    load_part(S, kt + 1 + RD, 2);
    __builtin_amdgcn_sched_group_barrier(0x100, MI, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, MI * NI, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(a1, b1);
  };

  // k-tiles 0..RD - 1 into the ring in order, k-tile 0 staged, its set refilled with
  // k-tile RD (loads complete in issue order, so each staging waits for its own tile)
#pragma unroll
  for (int j = 0; j < RD; ++j)
#pragma unroll
    for (int part = 0; part < 3; ++part) load_part(ring[j], j, part);
#pragma unroll
  for (int part = 0; part < 3; ++part) store_part(ring[0], lds, true, part);
#pragma unroll
  for (int part = 0; part < 3; ++part) load_part(ring[0], RD, part);
  __syncthreads();
  // unrolled by a multiple of RD and 2, so that k-tile kt's set (kt + 1) % RD is static
  constexpr int U = RD % 2 ? 2 * RD : RD;
  int kt = 0;
  for (; kt + U <= nk; kt += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      compute(kt + u, ring[(u + 1) % RD]);
      __syncthreads();
    }
  }
#pragma unroll
  for (int u = 0; u < U - 1; ++u) {
    if (kt + u < nk) {
      compute(kt + u, ring[(u + 1) % RD]);
      __syncthreads();
    }
  }
  // token sums: the eight lanes of a row segment hold its eight 16-byte groups
#pragma unroll
  for (int r = 0; r < XQ; ++r) {
    int v = rs[r];
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    if (xg == 0) xsum[xt + 32 * r] = v;
  }
  __syncthreads();

  if (a.P > 1) {
    // one K slice of several: the exact partial sum_k x q of the slice, rescaled later
    int32_t* pp = a.part + (int64_t)sl * a.T * a.N;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int n = n0 + wn * WN + j * 32 + li;
        const int tb = wm * WM + i * 32 + 4 * lg;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int dt = 8 * (r >> 2) + (r & 3);
          const int t = m0 + tb + dt;
          if (t < a.T && n < a.N) pp[(int64_t)t * a.N + n] = acc[i][j][r] - xsum[tb + dt];
        }
      }
    return;
  }
  const bool full = m0 + BM <= a.T && n0 + BN <= a.N && n0 / a.rpg == (n0 + BN - 1) / a.rpg;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      pf_store_block(a, acc[i][j], m0, n0, wm * WM + i * 32 + 4 * lg, n0 + wn * WN + j * 32 + li,
                     fac, xsum, full);
      __builtin_amdgcn_sched_barrier(0);
    }
}

// Sum of the P slice partials of a split-K product and the rescale (the same arithmetic
// as every other epilogue): acc = sum_p part[p][t][n], Y = fp32(acc) * fp32(beta_g / s_t).
// One thread per four consecutive outputs of a token row (grid.y = token), read and
// written as 16-byte vectors when N % 4 == 0 (every base pointer is 16-byte aligned).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(PfArgs a) {
  const int t = blockIdx.y;
  const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (n >= a.N) return;
  const float xs = a.xs[t];
  const int64_t plane = (int64_t)a.T * a.N;
  const int64_t o = (int64_t)t * a.N + n;
  if ((a.N & 3) == 0) {
    int4 v = make_int4(0, 0, 0, 0);
    for (int q = 0; q < a.P; ++q) {
      const int4 w = *reinterpret_cast<const int4*>(a.part + q * plane + o);
      v.x += w.x;
      v.y += w.y;
      v.z += w.z;
      v.w += w.w;
    }
    const float4 y = make_float4((float)v.x * (a.ws[n / a.rpg] / xs),
                                 (float)v.y * (a.ws[(n + 1) / a.rpg] / xs),
                                 (float)v.z * (a.ws[(n + 2) / a.rpg] / xs),
                                 (float)v.w * (a.ws[(n + 3) / a.rpg] / xs));
    *reinterpret_cast<float4*>(a.Y + o) = y;
    if (a.acc) *reinterpret_cast<int4*>(a.acc + o) = v;
    return;
  }
  for (int e = 0; e < 4 && n + e < a.N; ++e) {
    int v = 0;
    for (int q = 0; q < a.P; ++q) v += a.part[q * plane + o + e];
    a.Y[o + e] = (float)v * (a.ws[(n + e) / a.rpg] / xs);
    if (a.acc) a.acc[o + e] = v;
  }
}

inline int pf_cus() { return bl_device_cus(); }

// Register ring of the few-token (split-K) tiles: one workgroup per CU streams 8 KB of
// packed weights per k-tile in a fraction of a microsecond, so a load needs several
// k-tiles to arrive under load (70B down at 8-128 tokens: four sets 1-2% faster than
// six, eight 2-4% slower). At two workgroups per CU deeper rings measured slower (70B
// gate 3-6% with three or four sets), and the large tiles would spill.
#ifndef BL_PF_RING_SMALL
#define BL_PF_RING_SMALL 4
#endif
constexpr int kPfRingSmall = BL_PF_RING_SMALL;
#ifndef BL_PF_RING_TWO
#define BL_PF_RING_TWO 2
#endif
constexpr int kPfRingTwo = BL_PF_RING_TWO;  // few-token tiles at two workgroups per CU

template <int MI, int NI, int WY, int OCC, int RD>
hipError_t launch_prefill_big(const bl_proj_internal* p, int T, int P, int32_t* part,
                              hipStream_t stream) {
  constexpr int BM = 32 * MI * WY, BN = 32 * NI * (4 / WY);
  PfArgs a{};
  a.Xq = p->Xq;
  a.xs = p->x_scale;
  a.W = p->W;
  a.ws = p->w_scale;
  a.Y = p->Y;
  a.acc = p->acc;
  a.T = T;
  a.N = p->N;
  a.K = p->K;
  a.rpg = p->rpg;
  a.tiles_m = (T + BM - 1) / BM;
  a.tiles_n = (p->N + BN - 1) / BN;
  const plan::SplitK sk = plan::splitk_shape(p->K, P);  // no empty slice
  a.ktn = sk.ktn;
  a.P = sk.P;
  a.part = a.P > 1 ? part : nullptr;
  a.per_xcd = plan::xcd_per((int64_t)a.tiles_m * a.tiles_n * a.P);
  hipLaunchKernelGGL((prefill_big_kernel<MI, NI, WY, OCC, RD>), dim3((unsigned)(8 * a.per_xcd)),
                     dim3(kPfThreads), 0, stream, a);
  if (a.P > 1)
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((a.N + 1023) / 1024), (unsigned)T),
                       dim3(256), 0, stream, a);
  return hipGetLastError();
}

// Split-K plan (bl_plan.h) on this device's compute units.
inline int splitk_slices(int T, int N, int K) { return plan::splitk_slices(T, N, K, pf_cus()); }

template <int BM, int BN>
hipError_t launch_prefill_t(const bl_proj_internal* p, int T, hipStream_t stream) {
  PfArgs a{};
  a.Xq = p->Xq;
  a.xs = p->x_scale;
  a.W = p->W;
  a.ws = p->w_scale;
  a.Y = p->Y;
  a.acc = p->acc;
  a.T = T;
  a.N = p->N;
  a.K = p->K;
  a.rpg = p->rpg;
  a.tiles_m = (T + BM - 1) / BM;
  a.tiles_n = (p->N + BN - 1) / BN;
  a.per_xcd = plan::xcd_per((int64_t)a.tiles_m * a.tiles_n);
  hipLaunchKernelGGL((prefill_kernel<BM, BN>), dim3((unsigned)(8 * a.per_xcd)), dim3(kPfThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace bl

using namespace bl;

bool bl_prefill_supports(int T, int K) { return T >= 1 && K % 128 == 0; }

bool bl_prefill_splits(int T, int N, int K) {
  const int P = splitk_slices(T, N, K);
  return P > 1 && (int64_t)((N + 255) / 256) * P * 4 >= (int64_t)pf_cus() * 3;
}

size_t bl_prefill_scratch_bytes(int T, int N, int K) {
  return plan::splitk_scratch_bytes(T, N, K, pf_cus());
}

// Up to 128 tokens: 32*MI x 256 tiles (1 x 4 waves of 32*MI x 64), with K cut into
// slices when the tiles alone would leave CUs idle; the slices' exact int32 partials go
// to the caller's scratch (bl_prefill_scratch_bytes) and a second kernel sums and
// rescales them. Without that scratch, the single-stage tiles below.
// Beyond 128 tokens: 128 x 256 tiles when they give every CU at least one; two
// workgroups per CU when there are more tiles than CUs, so that one workgroup's epilogue
// (the fp32 stores) runs under the other's MFMAs, one otherwise (then the accumulators
// sit in AGPRs and nothing spills). Smaller problems take the single-stage tiles.
hipError_t bl_launch_prefill(const bl_proj_internal* p, int T, int32_t* scratch,
                             size_t scratch_bytes, hipStream_t stream) {
  const int cus = pf_cus();
  if (T <= 128) {
    const int P = splitk_slices(T, p->N, p->K);
    const bool have = P == 1 || (scratch && scratch_bytes >= bl_prefill_scratch_bytes(T, p->N, p->K));
    const int MI = (T + 31) / 32;
    const int64_t tiles = (int64_t)((p->N + 255) / 256) * P;
    if (have && tiles * 4 >= (int64_t)cus * 3) {
      if (tiles <= cus) {  // one workgroup per CU: the deep register ring
        if (MI == 1) return launch_prefill_big<1, 2, 1, 1, kPfRingSmall>(p, T, P, scratch, stream);
        if (MI == 2) return launch_prefill_big<2, 2, 1, 1, kPfRingSmall>(p, T, P, scratch, stream);
        if (MI == 3) return launch_prefill_big<3, 2, 1, 1, kPfRingSmall>(p, T, P, scratch, stream);
        return launch_prefill_big<4, 2, 1, 1, kPfRingSmall>(p, T, P, scratch, stream);
      }
      // more workgroups than CUs: two per CU, each with the two-set ring
      if (MI == 1) return launch_prefill_big<1, 2, 1, 2, kPfRingTwo>(p, T, P, scratch, stream);
      if (MI == 2) return launch_prefill_big<2, 2, 1, 2, kPfRingTwo>(p, T, P, scratch, stream);
      if (MI == 3) return launch_prefill_big<3, 2, 1, 2, kPfRingTwo>(p, T, P, scratch, stream);
      return launch_prefill_big<4, 2, 1, 2, kPfRingTwo>(p, T, P, scratch, stream);
    }
  }
  const int64_t tiles = (int64_t)((T + 127) / 128) * ((p->N + 255) / 256);
  // (one per CU: a third register set in the ring, which the AGPRs leave room for; the
  // 2048 x 4096 x 14336 product 127.2 / 127.5 -> 123.7 / 124.3 us in alternating runs,
  // four sets 125.1 / 126.1)
  if (T >= 128 && tiles >= cus)
    return tiles > cus ? launch_prefill_big<4, 2, 1, 2, 2>(p, T, 1, nullptr, stream)
                       : launch_prefill_big<4, 2, 1, 1, 3>(p, T, 1, nullptr, stream);
  const int64_t big = (int64_t)((T + 255) / 256) * ((p->N + 127) / 128);
  if (T >= 256 && big >= 512) return launch_prefill_t<256, 128>(p, T, stream);
  return launch_prefill_t<128, 128>(p, T, stream);
}
