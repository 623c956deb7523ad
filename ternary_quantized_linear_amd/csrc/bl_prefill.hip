// bl_prefill.hip -- ternary x int8 GEMM for long token counts (prefill) on int8 MFMA
// (v_mfma_i32_32x32x32_i8), int32 accumulation, fused rescale.
//
// [HF-1.58] "Fine-tuning LLMs to 1.58 bits", "Tiled matrix multiplication": the
// matrices are split into tiles held in fast on-chip memory to cut global-memory
// traffic; "Inference optimization and custom kernels": 2-bit weights unpacked on
// the fly. [bitnet.cpp] "3. BitLinear operation": rescale of the integer product.
//
// Y[T, N] = Xq[T, K] * q[N, K]^T. A workgroup (4 waves, 2 x 2) computes a BM x BN tile
// (BM tokens x BN weight rows); each wave a (BM/2) x (BN/2) sub-tile of 32 x 32 MFMA
// blocks. Per k-tile of 128 codes:
//   - activations: BM x 128 bytes into LDS, read from global memory as whole 128-byte
//     row segments (8 lanes per row: scattered 64-byte pieces cost the cache path about
//     three times as much), 16-byte groups 4x4 byte-transposed to the unpack order,
//     groups XOR-swizzled by row (conflict-free 128-bit reads and writes);
//   - weights: BN x 32 packed bytes, unpacked ONCE per workgroup to signed
//     int8 (unpack_q2, v_perm_b32 table) and written to LDS in the same swizzled layout,
//     so every wave reads both operands with plain 128-bit LDS reads and spends no ALU
//     on them;
//   - the next k-tile is loaded from global memory into registers while the MFMAs of
//     the current one run, then written over it between two barriers (one LDS buffer
//     per workgroup, so that two workgroups fit a CU and one stages while the other
//     computes).
// Workgroups are numbered XCD-major: the tiles one XCD (one L2) runs are consecutive
// token tiles of the same weight tiles.
// Epilogue: Y = fp32(acc) * fp32(beta / s_t).
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kPfThreads = 256;
constexpr int kPfKT = 128;  // codes per k-tile = bytes per staged row

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
};

template <int BM, int BN>
__global__ __launch_bounds__(kPfThreads, 2) void prefill_kernel(PfArgs a) {
  constexpr int WM = BM / 2, WN = BN / 2, MI = WM / 32, NI = WN / 32;
  constexpr int XQ = BM * (kPfKT / 16) / kPfThreads;       // 16-byte activation pieces per thread
  constexpr int WQ = BN * (kPfKT / 4 / 16) / kPfThreads;   // 16-byte packed weight pieces per thread
  static_assert(XQ >= 1 && WQ >= 1, "tile does not fit the thread count");
  __shared__ __attribute__((aligned(16))) uint8_t xs_l[BM * kPfKT];
  __shared__ __attribute__((aligned(16))) uint8_t ws_l[BN * kPfKT];
  __shared__ float fac[BM];

  // XCD-major numbering: workgroup b runs on XCD b % 8
  const int bid = (int)blockIdx.x;
  const int tile = (bid & 7) * a.per_xcd + (bid >> 3);
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
  // One block at a time, addresses advanced per token, so that the epilogue does not
  // hold every store address at once.
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int n = n0 + wn * WN + j * 32 + li;
      const int tb = wm * WM + i * 32 + 4 * lg;
      float* yp = a.Y + (int64_t)(m0 + tb) * a.N + n;
      int32_t* ap = a.acc ? a.acc + (int64_t)(m0 + tb) * a.N + n : nullptr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int dt = 8 * (r >> 2) + (r & 3);
        const int t = m0 + tb + dt;
        if (t < a.T && n < a.N) {
          const int v = acc[i][j][r];
          // fac holds beta of the tile's first row's group; rows of another group (scale
          // groups smaller than the tile or straddling it) divide their own scale
          const float f = n / a.rpg == n0 / a.rpg ? fac[tb + dt] : a.ws[n / a.rpg] / a.xs[t];
          yp[(int64_t)dt * a.N] = (float)v * f;
          if (ap) ap[(int64_t)dt * a.N] = v;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
}

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
  const int tiles = a.tiles_m * a.tiles_n;
  a.per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL((prefill_kernel<BM, BN>), dim3((unsigned)(8 * a.per_xcd)), dim3(kPfThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace bl

using namespace bl;

bool bl_prefill_supports(int T, int K) { return T >= 1 && K % 128 == 0; }

// 256-token tiles (a 128 x 64 sub-tile per wave: each weight fragment feeds four MFMAs)
// while they still give the device two rounds of workgroups; 128 x 128 otherwise.
hipError_t bl_launch_prefill(const bl_proj_internal* p, int T, hipStream_t stream) {
  const int64_t big = (int64_t)((T + 255) / 256) * ((p->N + 127) / 128);
  if (T >= 256 && big >= 512) return launch_prefill_t<256, 128>(p, T, stream);
  return launch_prefill_t<128, 128>(p, T, stream);
}
