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
//   - activations: BM x 128 bytes into LDS, 16-byte groups 4x4 byte-transposed to the
//     unpack order, rows padded to 144 bytes (conflict-free 128-bit reads);
//   - weights: BN x 32 packed bytes into LDS (rows padded to 36 bytes) -- a quarter of
//     the bytes an int8 tile would take; each wave unpacks its B fragments in
//     registers to signed int8 (unpack_q2, v_perm_b32 table lookup);
//   - the next k-tile is loaded from global memory into registers while the MFMAs of
//     the current one run, then written to the other LDS buffer (one barrier per tile).
// Epilogue: Y = fp32(acc) * fp32(beta / s_t), stored as 128-byte row segments.
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kPfThreads = 256;
constexpr int kPfKT = 128;            // codes per k-tile
constexpr int kPfXStride = kPfKT + 16;  // bytes per staged activation row
constexpr int kPfWStride = kPfKT / 4 + 4;  // bytes per staged packed weight row

struct PfArgs {
  const int8_t* Xq;
  const float* xs;
  const uint8_t* W;
  const float* ws;
  float* Y;
  int32_t* acc;
  int T, N, K;
  int tiles_m, tiles_n;
};

template <int BM, int BN>
__global__ __launch_bounds__(kPfThreads) void prefill_kernel(PfArgs a) {
  constexpr int WM = BM / 2, WN = BN / 2, MI = WM / 32, NI = WN / 32;
  constexpr int XQ = BM * kPfKT / 16 / kPfThreads;       // uint4 of activations per thread
  constexpr int WQ = BN * (kPfKT / 4) / 16 / kPfThreads;  // uint4 of weights per thread
  static_assert(XQ >= 1 && WQ >= 1, "tile too small for the thread count");
  __shared__ __attribute__((aligned(16))) uint8_t xs_l[2][BM * kPfXStride];
  __shared__ __attribute__((aligned(16))) uint8_t ws_l[2][BN * kPfWStride];
  __shared__ float fac[BM];

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tm = (int)blockIdx.x % a.tiles_m, tn = (int)blockIdx.x / a.tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int Kb = a.K >> 2;
  const float beta = a.ws[0];
  for (int i = tid; i < BM; i += kPfThreads) {
    const int t = m0 + i;
    fac[i] = t < a.T ? beta / a.xs[t] : 0.0f;
  }

  // global source addresses (rows clamped into range; clamped rows are never stored)
  const int8_t* xsrc[XQ];
  int xdst[XQ];
#pragma unroll
  for (int r = 0; r < XQ; ++r) {
    const int q = tid + kPfThreads * r, t = q >> 3, g = q & 7;
    xsrc[r] = a.Xq + (int64_t)min(m0 + t, a.T - 1) * a.K + 16 * g;
    xdst[r] = t * kPfXStride + 16 * g;
  }
  const uint8_t* wsrc[WQ];
  int wdst[WQ];
#pragma unroll
  for (int r = 0; r < WQ; ++r) {
    const int q = tid + kPfThreads * r, j = q >> 1, h = q & 1;
    wsrc[r] = a.W + (int64_t)min(n0 + j, a.N - 1) * Kb + 16 * h;
    wdst[r] = j * kPfWStride + 16 * h;
  }
  uint4 xr[XQ], wr[WQ];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int r = 0; r < XQ; ++r) xr[r] = *reinterpret_cast<const uint4*>(xsrc[r] + kt * kPfKT);
#pragma unroll
    for (int r = 0; r < WQ; ++r) wr[r] = *reinterpret_cast<const uint4*>(wsrc[r] + kt * (kPfKT / 4));
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int r = 0; r < XQ; ++r) {
      const uint32_t in[4] = {xr[r].x, xr[r].y, xr[r].z, xr[r].w};
      uint32_t o[4];
      transpose16(in, o);
      *reinterpret_cast<uint4*>(&xs_l[buf][xdst[r]]) = make_uint4(o[0], o[1], o[2], o[3]);
    }
#pragma unroll
    for (int r = 0; r < WQ; ++r) {
      uint32_t* d = reinterpret_cast<uint32_t*>(&ws_l[buf][wdst[r]]);
      d[0] = wr[r].x;
      d[1] = wr[r].y;
      d[2] = wr[r].z;
      d[3] = wr[r].w;
    }
  };

  v16i acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  const int nk = a.K / kPfKT;
  const int li = lane & 31, lg = lane >> 5;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tile(kt + 1);
    const uint8_t* xb = xs_l[buf];
    const uint8_t* wb = ws_l[buf];
#pragma unroll
    for (int s = 0; s < kPfKT / 32; ++s) {
      v4i af[MI], bf[NI];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int t = wm * WM + i * 32 + li;
        const uint4 x = *reinterpret_cast<const uint4*>(xb + t * kPfXStride + 16 * (2 * s + lg));
        af[i] = v4i{(int)x.x, (int)x.y, (int)x.z, (int)x.w};
      }
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int n = wn * WN + j * 32 + li;
        const uint32_t w = *reinterpret_cast<const uint32_t*>(wb + n * kPfWStride + 4 * (2 * s + lg));
        uint32_t q[4];
        unpack_q2(w, q);
        bf[j] = v4i{(int)q[0], (int)q[1], (int)q[2], (int)q[3]};
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tile(buf ^ 1);
    __syncthreads();
  }

  // D[token][row]: lane holds row li of the 32 x 32 block, tokens 8*(r/4) + 4*lg + r%4.
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int n = n0 + wn * WN + j * 32 + li;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tl = wm * WM + i * 32 + 8 * (r >> 2) + 4 * lg + (r & 3);
        const int t = m0 + tl;
        if (t < a.T && n < a.N) {
          const int v = acc[i][j][r];
          a.Y[(int64_t)t * a.N + n] = (float)v * fac[tl];
          if (a.acc) a.acc[(int64_t)t * a.N + n] = v;
        }
      }
    }
}

}  // namespace bl

using namespace bl;

bool bl_prefill_supports(int T, int K) { return T >= 1 && K % kPfKT == 0; }

hipError_t bl_launch_prefill(const bl_proj_internal* p, int T, hipStream_t stream) {
  constexpr int BM = 128, BN = 128;
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
  a.tiles_m = (T + BM - 1) / BM;
  a.tiles_n = (p->N + BN - 1) / BN;
  dim3 grid((unsigned)(a.tiles_m * a.tiles_n)), block(kPfThreads);
  hipLaunchKernelGGL((prefill_kernel<BM, BN>), grid, block, 0, stream, a);
  return hipGetLastError();
}
