// bl_capi.hip -- the C ABI of libbitlinear.so (declared in include/bitlinear.h):
// host-side argument validation, kernel dispatch, status reporting. No C++ exception
// crosses the ABI; nothing here allocates device memory or synchronizes the stream
// (the scratch of split-K products is the caller's workspace, or for the
// allocation-free grouped forward a static device array of this file).
#include <math.h>
#include <string.h>

#include <mutex>

#include "bl_internal.h"

int bl_device_cus() {
  static int cached = 0;
  int v = __atomic_load_n(&cached, __ATOMIC_RELAXED);
  if (v > 0) return v;
  int dev = 0, n = 0;
  v = hipGetDevice(&dev) == hipSuccess &&
              hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
              n > 0
          ? n
          : 256;
  __atomic_store_n(&cached, v, __ATOMIC_RELAXED);
  return v;
}

int bl_resident_wgs(const void* kernel, int threads, size_t lds, int fallback, int* slot) {
  int v = __atomic_load_n(slot, __ATOMIC_RELAXED);
  if (v > 0) return v;
  int per = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, lds) != hipSuccess ||
      per < 1)
    per = fallback;
  v = bl_device_cus() * per;
  __atomic_store_n(slot, v, __ATOMIC_RELAXED);
  return v;
}

namespace {

thread_local char g_last_error[256] = "";

bl_status hip_status(hipError_t e) {
  if (e == hipSuccess) return BL_OK;
  const char* s = hipGetErrorString(e);
  strncpy(g_last_error, s ? s : "unknown HIP error", sizeof(g_last_error) - 1);
  g_last_error[sizeof(g_last_error) - 1] = '\0';
  return BL_ERR_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned_n(const void* p, uintptr_t n) { return ((uintptr_t)p & (n - 1)) == 0; }

constexpr int64_t kMaxRows = 0x7FFFFFFF;  // N, T fit an int
constexpr int64_t kMaxTokens = 65535;
constexpr int64_t kMaxWeights = int64_t(1) << 31;  // exact-sum digit capacity

bl_status check_acts(const float* X, const float* gain, int64_t T, int64_t K, int8_t* Xq,
                     float* xs) {
  if (!X || !Xq || !xs) return BL_ERR_NULL;
  if (T <= 0 || K <= 0 || K % 4 || T > kMaxTokens) return BL_ERR_DIM;
  if (K > BL_MAX_K) return BL_ERR_K_TOO_LARGE;
  if (!aligned16(X) || !aligned16(Xq) || !aligned_n(xs, 4) || (gain && !aligned16(gain)))
    return BL_ERR_ALIGN;
  return BL_OK;
}

bl_status check_proj(const int8_t* Xq, const float* xs, int64_t T, int64_t K,
                     const uint8_t* W, const float* ws, int64_t N, float* Y, int32_t* acc) {
  if (!Xq || !xs || !W || !ws || !Y) return BL_ERR_NULL;
  if (T <= 0 || N <= 0 || K <= 0 || K % 4 || T > kMaxTokens || N > kMaxRows) return BL_ERR_DIM;
  if (K > BL_MAX_K) return BL_ERR_K_TOO_LARGE;
  if (!aligned16(Xq) || !aligned16(W) || !aligned16(Y) || (acc && !aligned16(acc)) ||
      !aligned_n(xs, 4) || !aligned_n(ws, 4))
    return BL_ERR_ALIGN;
  return BL_OK;
}

bl_kernel choose(int64_t T, int64_t N, int64_t K, size_t ws_bytes = 0) {
  // one token: dot4 GEMV. Up to 128 tokens the streaming MFMA kernel (passes of 64),
  // except where the LDS-tiled GEMM measures faster: from 96 tokens on, beyond 64 (a
  // second streaming pass) when it can cut K into slices that fill the device (which
  // takes a workspace for the partials), beyond 16 (two token blocks) when it can and
  // K >= 16384 (the streaming kernel reloads its activations many times over long
  // rows), or when its 128 x 128 tiles alone give every CU two workgroups. Beyond 128
  // tokens the tiled GEMM. Measured on the 70B shapes: gate (K = 8192) at 32 / 48 / 64 /
  // 80 tokens 21 / 30 / 33 / 49 us streaming against 27 / 34 / 37 / 44 us split; down
  // (K = 28672, 512-code segments) at 12 / 14 / 16 / 17 / 32 tokens 20.8 / 20.8 / 22.3 /
  // 26.9 / 37 us streaming against 23.6 / 23.4 / 23.6 / 24.0 / 25.1 us split.
  if (bl_gemv_supports((int)T, (int)K)) return BL_KERNEL_GEMV;
  const bool tiled = bl_prefill_supports((int)T, (int)K);
  if (bl_skinny_supports((int)T, N, (int)K)) {
    const int64_t tiles = ((T + 127) / 128) * ((N + 127) / 128);
    const bool split = tiled && bl_prefill_splits((int)T, (int)N, (int)K) &&
                       ws_bytes >= bl_prefill_scratch_bytes((int)T, (int)N, (int)K);
    const bool prefer_tiled = tiled && (T >= 96 || (T > 64 && split) ||
                                        (T > 16 && K >= 16384 && split) ||
                                        (T > 32 && tiles >= 512));
    if (!prefer_tiled) return BL_KERNEL_SKINNY;
  }
  if (tiled) return BL_KERNEL_PREFILL;
  return BL_KERNEL_GENERIC;
}

bool supports(bl_kernel k, int64_t T, int64_t N, int64_t K) {
  switch (k) {
    case BL_KERNEL_GEMV: return bl_gemv_supports((int)T, (int)K);
    case BL_KERNEL_SKINNY: return bl_skinny_supports((int)T, N, (int)K);
    case BL_KERNEL_PREFILL: return bl_prefill_supports((int)T, (int)K);
    case BL_KERNEL_GENERIC: return true;
    default: return false;
  }
}

bl_proj_internal to_internal(const int8_t* Xq, const float* xs, int64_t K, const uint8_t* W,
                             const float* ws, int64_t N, float* Y, int32_t* acc) {
  return bl_proj_internal{Xq, xs, W, ws, Y, acc, (int)N, (int)K, (int)N};
}

// ws: the caller's workspace (or null); the projections of a grouped call run one after
// another on s, so each may use all of it
hipError_t run(bl_kernel k, const bl_proj_internal* p, int count, int T, hipStream_t s,
               void* ws = nullptr, size_t ws_bytes = 0) {
  switch (k) {
    case BL_KERNEL_GEMV: return bl_launch_gemv(p, count, T, s);
    case BL_KERNEL_SKINNY: return bl_launch_skinny(p, count, T, s);
    case BL_KERNEL_PREFILL:
      for (int i = 0; i < count; ++i) {
        hipError_t e = bl_launch_prefill(p + i, T, static_cast<int32_t*>(ws), ws ? ws_bytes : 0, s);
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    default:
      for (int i = 0; i < count; ++i) {
        hipError_t e = bl_launch_generic(p + i, T, s);
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
  }
}

}  // namespace

extern "C" {

size_t bitlinear_weight_workspace_bytes(int64_t N, int64_t K) {
  return bl_weight_workspace_bytes_impl(N, K);
}

bl_status bitlinear_quantize_weights(const float* W, int64_t N, int64_t K, uint8_t* W_packed,
                                     float* w_scale, double* w_gamma, void* workspace,
                                     size_t workspace_bytes, bl_stream_t stream) {
  if (!W || !W_packed || !w_scale) return BL_ERR_NULL;
  if (N <= 0 || K <= 0 || K % 4 || N > kMaxRows || N * K > kMaxWeights) return BL_ERR_DIM;
  if (!workspace || workspace_bytes < bitlinear_weight_workspace_bytes(N, K))
    return BL_ERR_WORKSPACE;
  if (!aligned16(W) || !aligned16(workspace) || !aligned_n(w_scale, 4) ||
      (w_gamma && !aligned_n(w_gamma, 8)))
    return BL_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(bl_launch_quantize_weights(W, N, K, W_packed, w_scale, w_gamma, workspace,
                                               (hipStream_t)stream));
}

bl_status bitlinear_quantize_acts(const float* X, const float* gain, int64_t T, int64_t K,
                                  float eps, uint32_t flags, int8_t* Xq, float* x_scale,
                                  bl_stream_t stream) {
  bl_act_desc d{X, gain, Xq, x_scale, K};
  return bitlinear_quantize_acts_grouped(&d, 1, T, eps, flags, stream);
}

bl_status bitlinear_quantize_acts_grouped(const bl_act_desc* descs, int count, int64_t T,
                                          float eps, uint32_t flags, bl_stream_t stream) {
  if (!descs) return BL_ERR_NULL;
  if (count < 1 || count > BL_MAX_GROUP) return BL_ERR_ARG;
  if ((flags & ~BL_NO_NORM) != 0u) return BL_ERR_ARG;
  if (!(eps >= 0.0f) || !isfinite(eps)) return BL_ERR_ARG;
  for (int i = 0; i < count; ++i) {
    bl_status s = check_acts(descs[i].X, descs[i].gain, T, descs[i].K, descs[i].Xq,
                             descs[i].x_scale);
    if (s != BL_OK) return s;
  }
  (void)hipGetLastError();
  return hip_status(bl_launch_quantize_acts(descs, count, T, eps, flags, (hipStream_t)stream));
}

bl_kernel bitlinear_forward_choice(int64_t T, int64_t N, int64_t K) { return choose(T, N, K); }

bl_kernel bitlinear_forward_choice_ws(int64_t T, int64_t N, int64_t K, size_t workspace_bytes) {
  return choose(T, N, K, workspace_bytes);
}

size_t bitlinear_forward_workspace_bytes(int64_t T, int64_t N, int64_t K) {
  if (T <= 0 || N <= 0 || K <= 0 || K % 4 || T > kMaxTokens || N > kMaxRows || K > BL_MAX_K)
    return 0;
  return bl_prefill_scratch_bytes((int)T, (int)N, (int)K);
}

bl_status bitlinear_forward_ws(const int8_t* Xq, const float* x_scale, int64_t T, int64_t K,
                               const uint8_t* W_packed, const float* w_scale, int64_t N,
                               float* Y, int32_t* acc, bl_kernel kernel, void* workspace,
                               size_t workspace_bytes, bl_stream_t stream) {
  bl_status s = check_proj(Xq, x_scale, T, K, W_packed, w_scale, N, Y, acc);
  if (s != BL_OK) return s;
  if (workspace && !aligned16(workspace)) return BL_ERR_ALIGN;
  const size_t ws = workspace ? workspace_bytes : 0;
  if (kernel == BL_KERNEL_AUTO) kernel = choose(T, N, K, ws);
  if (!supports(kernel, T, N, K)) return BL_ERR_ARG;
  bl_proj_internal p = to_internal(Xq, x_scale, K, W_packed, w_scale, N, Y, acc);
  (void)hipGetLastError();
  return hip_status(run(kernel, &p, 1, (int)T, (hipStream_t)stream, workspace, ws));
}

bl_status bitlinear_forward_ex(const int8_t* Xq, const float* x_scale, int64_t T, int64_t K,
                               const uint8_t* W_packed, const float* w_scale, int64_t N,
                               float* Y, int32_t* acc, bl_kernel kernel, bl_stream_t stream) {
  return bitlinear_forward_ws(Xq, x_scale, T, K, W_packed, w_scale, N, Y, acc, kernel, nullptr,
                              0, stream);
}

bl_status bitlinear_forward(const int8_t* Xq, const float* x_scale, int64_t T, int64_t K,
                            const uint8_t* W_packed, const float* w_scale, int64_t N, float* Y,
                            int32_t* acc, bl_stream_t stream) {
  return bitlinear_forward_ex(Xq, x_scale, T, K, W_packed, w_scale, N, Y, acc, BL_KERNEL_AUTO,
                              stream);
}

bl_status bitlinear_forward_grouped(const bl_proj_desc* descs, int count, int64_t T,
                                    bl_stream_t stream) {
  return bitlinear_forward_grouped_ws(descs, count, T, nullptr, 0, stream);
}

bl_status bitlinear_forward_grouped_ws(const bl_proj_desc* descs, int count, int64_t T,
                                       void* workspace, size_t workspace_bytes,
                                       bl_stream_t stream) {
  if (!descs) return BL_ERR_NULL;
  if (count < 1 || count > BL_MAX_GROUP) return BL_ERR_ARG;
  if (workspace && !aligned16(workspace)) return BL_ERR_ALIGN;
  const size_t ws = workspace ? workspace_bytes : 0;
  bl_proj_internal p[BL_MAX_GROUP];
  for (int i = 0; i < count; ++i) {
    const bl_proj_desc& d = descs[i];
    bl_status s = check_proj(d.Xq, d.x_scale, T, d.K, d.W_packed, d.w_scale, d.N, d.Y, d.acc);
    if (s != BL_OK) return s;
    p[i] = to_internal(d.Xq, d.x_scale, d.K, d.W_packed, d.w_scale, d.N, d.Y, d.acc);
  }
  (void)hipGetLastError();
  // one launch per kernel kind: entries sharing the kernel choice go together
  bl_proj_internal batch[BL_MAX_GROUP];
  const bl_kernel kinds[4] = {BL_KERNEL_GEMV, BL_KERNEL_SKINNY, BL_KERNEL_PREFILL,
                              BL_KERNEL_GENERIC};
  for (bl_kernel k : kinds) {
    int n = 0;
    for (int i = 0; i < count; ++i)
      if (choose(T, descs[i].N, descs[i].K, ws) == k) batch[n++] = p[i];
    if (n == 0) continue;
    bl_status s = hip_status(run(k, batch, n, (int)T, (hipStream_t)stream, workspace, ws));
    if (s != BL_OK) return s;
  }
  return BL_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- allocation-free forward
// The split-K workspace of bitlinear_forward_grouped_noalloc: a file-scope device array,
// one copy per GPU, present from the module's load until the process ends. Host code
// never passes `scratch` itself (in host code it names a host-side stand-in, not the
// device array): the address comes from hipGetSymbolAddress, once per device, and only
// that address reaches the kernels.
static __device__ __align__(256) uint8_t scratch[BL_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the current device, looked up on the first call there.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

bl_status bitlinear_forward_grouped_noalloc(const bl_proj_desc* descs, int count, int64_t T,
                                            bl_stream_t stream) {
  if (!descs) return BL_ERR_NULL;
  if (count < 1 || count > BL_MAX_GROUP) return BL_ERR_ARG;
  for (int i = 0; i < count; ++i) {
    const bl_proj_desc& d = descs[i];
    bl_status s = check_proj(d.Xq, d.x_scale, T, d.K, d.W_packed, d.w_scale, d.N, d.Y, d.acc);
    if (s != BL_OK) return s;
    if (bitlinear_forward_workspace_bytes(T, d.N, d.K) > BL_NOALLOC_SCRATCH_BYTES)
      return BL_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  (void)hipGetLastError();
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) {
    const bl_status s = hip_status(e);
    strncat(g_last_error, " (bitlinear_forward_grouped_noalloc: scratch address lookup)",
            sizeof(g_last_error) - strlen(g_last_error) - 1);
    return s;
  }
  return bitlinear_forward_grouped_ws(descs, count, T, ws, BL_NOALLOC_SCRATCH_BYTES, stream);
}

bl_status bitlinear_quantize_weights_scale_groups(const float* W, int64_t N, int64_t K, int64_t G,
                                                  uint8_t* W_packed, float* w_scale,
                                                  double* w_gamma, void* workspace,
                                                  size_t workspace_bytes, bl_stream_t stream) {
  if (!W || !W_packed || !w_scale) return BL_ERR_NULL;
  if (N <= 0 || K <= 0 || K % 4 || N > kMaxRows || N * K > kMaxWeights) return BL_ERR_DIM;
  if (G < 1 || N % G) return BL_ERR_ARG;
  if (!workspace || workspace_bytes < bitlinear_weight_workspace_bytes(N, K))
    return BL_ERR_WORKSPACE;
  if (!aligned16(W) || !aligned16(workspace) || !aligned_n(w_scale, 4) ||
      (w_gamma && !aligned_n(w_gamma, 8)))
    return BL_ERR_ALIGN;
  (void)hipGetLastError();
  const int64_t rows = N / G;
  // one block of rows after the other on the stream (the workspace is reused)
  for (int64_t g = 0; g < G; ++g) {
    bl_status s = hip_status(bl_launch_quantize_weights(
        W + g * rows * K, rows, K, W_packed + g * rows * (K / 4), w_scale + g,
        w_gamma ? w_gamma + g : nullptr, workspace, (hipStream_t)stream));
    if (s != BL_OK) return s;
  }
  return BL_OK;
}

bl_status bitlinear_forward_grouped_scale_groups(const bl_proj_desc* descs, const int64_t* groups,
                                                 int count, int64_t T, bl_stream_t stream) {
  if (!descs || !groups) return BL_ERR_NULL;
  if (count < 1 || count > BL_MAX_GROUP) return BL_ERR_ARG;
  bl_proj_internal p[BL_MAX_GROUP];
  for (int i = 0; i < count; ++i) {
    const bl_proj_desc& d = descs[i];
    bl_status s = check_proj(d.Xq, d.x_scale, T, d.K, d.W_packed, d.w_scale, d.N, d.Y, d.acc);
    if (s != BL_OK) return s;
    if (groups[i] < 1 || d.N % groups[i]) return BL_ERR_ARG;
    p[i] = to_internal(d.Xq, d.x_scale, d.K, d.W_packed, d.w_scale, d.N, d.Y, d.acc);
    p[i].rpg = (int)(d.N / groups[i]);
  }
  (void)hipGetLastError();
  bl_proj_internal batch[BL_MAX_GROUP];
  const bl_kernel kinds[4] = {BL_KERNEL_GEMV, BL_KERNEL_SKINNY, BL_KERNEL_PREFILL,
                              BL_KERNEL_GENERIC};
  for (bl_kernel k : kinds) {
    int n = 0;
    for (int i = 0; i < count; ++i)
      if (choose(T, descs[i].N, descs[i].K) == k) batch[n++] = p[i];
    if (n == 0) continue;
    bl_status s = hip_status(run(k, batch, n, (int)T, (hipStream_t)stream));
    if (s != BL_OK) return s;
  }
  return BL_OK;
}

bl_status bitlinear_forward_scale_groups(const int8_t* Xq, const float* x_scale, int64_t T,
                                         int64_t K, const uint8_t* W_packed, const float* w_scale,
                                         int64_t N, int64_t G, float* Y, int32_t* acc,
                                         bl_kernel kernel, bl_stream_t stream) {
  bl_status s = check_proj(Xq, x_scale, T, K, W_packed, w_scale, N, Y, acc);
  if (s != BL_OK) return s;
  if (G < 1 || N % G) return BL_ERR_ARG;
  if (kernel == BL_KERNEL_AUTO) kernel = choose(T, N, K);
  if (!supports(kernel, T, N, K)) return BL_ERR_ARG;
  bl_proj_internal p = to_internal(Xq, x_scale, K, W_packed, w_scale, N, Y, acc);
  p.rpg = (int)(N / G);
  (void)hipGetLastError();
  return hip_status(run(kernel, &p, 1, (int)T, (hipStream_t)stream));
}

bl_status bitlinear_quantize_weights_sign(const float* W, int64_t N, int64_t K, uint8_t* W_bits,
                                          float* w_scale, double* w_alpha, void* workspace,
                                          size_t workspace_bytes, bl_stream_t stream) {
  if (!W || !W_bits || !w_scale) return BL_ERR_NULL;
  if (N <= 0 || K <= 0 || K % 8 || N > kMaxRows || N * K > kMaxWeights) return BL_ERR_DIM;
  if (!workspace || workspace_bytes < bitlinear_weight_workspace_bytes(N, K))
    return BL_ERR_WORKSPACE;
  if (!aligned16(W) || !aligned16(W_bits) || !aligned16(workspace) || !aligned_n(w_scale, 4) ||
      (w_alpha && !aligned_n(w_alpha, 8)))
    return BL_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(bl_launch_quantize_weights_sign(W, N, K, W_bits, w_scale, w_alpha, workspace,
                                                    (hipStream_t)stream));
}

bl_status bitlinear_forward_sign_grouped(const bl_proj_desc* descs, int count, int64_t T,
                                         bl_stream_t stream) {
  if (!descs) return BL_ERR_NULL;
  if (count < 1 || count > BL_MAX_GROUP) return BL_ERR_ARG;
  bl_proj_internal gemv[BL_MAX_GROUP];
  int ng = 0;
  for (int i = 0; i < count; ++i) {
    const bl_proj_desc& d = descs[i];
    bl_status s = check_proj(d.Xq, d.x_scale, T, d.K, d.W_packed, d.w_scale, d.N, d.Y, d.acc);
    if (s != BL_OK) return s;
    if (d.K % 8) return BL_ERR_DIM;
  }
  (void)hipGetLastError();
  for (int i = 0; i < count; ++i) {
    const bl_proj_desc& d = descs[i];
    const bl_proj_internal p = to_internal(d.Xq, d.x_scale, d.K, d.W_packed, d.w_scale, d.N, d.Y,
                                           d.acc);
    if (bl_gemv_sign_supports((int)T, (int)d.K)) {
      gemv[ng++] = p;
    } else {
      bl_status s = hip_status(bl_launch_generic_sign(&p, (int)T, (hipStream_t)stream));
      if (s != BL_OK) return s;
    }
  }
  if (ng > 0) return hip_status(bl_launch_gemv_sign(gemv, ng, (hipStream_t)stream));
  return BL_OK;
}

bl_status bitlinear_forward_sign(const int8_t* Xq, const float* x_scale, int64_t T, int64_t K,
                                 const uint8_t* W_bits, const float* w_scale, int64_t N,
                                 float* Y, int32_t* acc, bl_stream_t stream) {
  const bl_proj_desc d{Xq, x_scale, W_bits, w_scale, Y, acc, N, K};
  return bitlinear_forward_sign_grouped(&d, 1, T, stream);
}

float bitlinear_warmup_lambda(int64_t step, int64_t total) {
  if (total <= 0 || step >= total) return 1.0f;
  if (step <= 0) return 0.0f;
  return (float)((double)step / (double)total);
}

bl_status bitlinear_fake_quant_weights(const float* W, int64_t N, int64_t K, const float* w_scale,
                                       float lambda, uint16_t* W_out, bl_stream_t stream) {
  if (!W || !w_scale || !W_out) return BL_ERR_NULL;
  if (N <= 0 || K <= 0 || K % 4 || N > kMaxRows || N * K > kMaxWeights) return BL_ERR_DIM;
  if (!(lambda >= 0.0f && lambda <= 1.0f)) return BL_ERR_ARG;
  if (!aligned16(W) || !aligned16(W_out) || !aligned_n(w_scale, 4)) return BL_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(bl_launch_fake_quant_weights(W, N, K, w_scale, lambda, W_out,
                                                 (hipStream_t)stream));
}

bl_status bitlinear_fake_quant_acts(const float* X, const float* gain, int64_t T, int64_t K,
                                    float eps, uint32_t flags, float lambda, int8_t* Xq,
                                    float* x_scale, uint16_t* X_out, double* x_rinv,
                                    bl_stream_t stream) {
  bl_status s = check_acts(X, gain, T, K, Xq, x_scale);
  if (s != BL_OK) return s;
  if (!X_out) return BL_ERR_NULL;
  if ((flags & ~BL_NO_NORM) != 0u) return BL_ERR_ARG;
  if (!(eps >= 0.0f) || !isfinite(eps)) return BL_ERR_ARG;
  if (!(lambda >= 0.0f && lambda <= 1.0f)) return BL_ERR_ARG;
  if (!aligned16(X_out) || (x_rinv && !aligned_n(x_rinv, 8))) return BL_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(bl_launch_fake_quant_acts(X, gain, T, K, eps, flags, lambda, Xq, x_scale, X_out,
                                              x_rinv, (hipStream_t)stream));
}

bl_status bitlinear_rmsnorm_backward(const float* X, const float* gain, const double* x_rinv,
                                     const float* dY, int64_t T, int64_t K, float* dX,
                                     float* dgain, bl_stream_t stream) {
  if (!X || !x_rinv || !dY || !dX) return BL_ERR_NULL;
  if (T <= 0 || K <= 0 || T > kMaxTokens || K > kMaxRows) return BL_ERR_DIM;
  if (!aligned_n(X, 4) || !aligned_n(dY, 4) || !aligned_n(dX, 4) || !aligned_n(x_rinv, 8) ||
      (gain && !aligned_n(gain, 4)) || (dgain && !aligned_n(dgain, 4)))
    return BL_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(bl_launch_rmsnorm_backward(X, gain, x_rinv, dY, T, K, dX, dgain,
                                               (hipStream_t)stream));
}

bl_status bitlinear_bitdelta_compress(const float* W_fine, const uint16_t* W_base, int64_t N,
                                      int64_t M, int B, int model, uint8_t* D, float* alpha,
                                      void* workspace, size_t workspace_bytes,
                                      bl_stream_t stream) {
  if (!W_fine || !W_base || !D || !alpha) return BL_ERR_NULL;
  if (!bl_bitdelta_supports(N, M, B)) return BL_ERR_DIM;
  if (model < 0 || model >= B) return BL_ERR_ARG;
  if (!workspace || workspace_bytes < bitlinear_weight_workspace_bytes(N, M))
    return BL_ERR_WORKSPACE;
  if (!aligned16(W_fine) || !aligned16(W_base) || !aligned16(D) || !aligned16(workspace) ||
      !aligned_n(alpha, 4))
    return BL_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(bl_launch_bitdelta_compress(W_fine, W_base, N, M, model, D, alpha + model,
                                                workspace, (hipStream_t)stream));
}

bl_status bitlinear_bitdelta_forward(const uint16_t* W_base, const uint8_t* D, const float* alpha,
                                     const float* X, int64_t N, int64_t M, int B, float* Y,
                                     bl_stream_t stream) {
  if (!W_base || !D || !alpha || !X || !Y) return BL_ERR_NULL;
  if (!bl_bitdelta_supports(N, M, B)) return BL_ERR_DIM;
  if (!aligned16(W_base) || !aligned16(X) || !aligned16(D) || !aligned_n(alpha, 4) ||
      !aligned_n(Y, 4))
    return BL_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(bl_launch_bitdelta(W_base, D, alpha, X, Y, N, M, B, (hipStream_t)stream));
}

bl_status bitlinear_roof_read(const void* const* bufs, const int64_t* bytes, int count,
                              int schedule, uint32_t* sink, bl_stream_t stream) {
  if (!bufs || !bytes || !sink) return BL_ERR_NULL;
  if (count < 1 || count > BL_MAX_GROUP || schedule < 0 || schedule > 3) return BL_ERR_ARG;
  for (int i = 0; i < count; ++i) {
    if (!bufs[i]) return BL_ERR_NULL;
    if (bytes[i] <= 0 || bytes[i] % 16) return BL_ERR_DIM;
    if (!aligned16(bufs[i])) return BL_ERR_ALIGN;
  }
  if (!aligned_n(sink, 4)) return BL_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(bl_launch_roof_read(bufs, bytes, count, schedule, sink, (hipStream_t)stream));
}

bl_status bitlinear_roof_mfma_i8(int iters, int workgroups, int32_t* sink, uint64_t* clocks,
                                 bl_stream_t stream) {
  if (!sink || !clocks) return BL_ERR_NULL;
  if (iters < 1 || workgroups < 1 || workgroups > (1 << 20)) return BL_ERR_DIM;
  if (!aligned_n(sink, 4) || !aligned_n(clocks, 8)) return BL_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(bl_launch_roof_mfma(iters, workgroups, sink, clocks, (hipStream_t)stream));
}

const char* bitlinear_status_str(bl_status s) {
  switch (s) {
    case BL_OK: return "ok";
    case BL_ERR_NULL: return "a required pointer is NULL";
    case BL_ERR_DIM: return "invalid dimensions (T, N, K must be positive, K a multiple of 4)";
    case BL_ERR_K_TOO_LARGE: return "K exceeds BL_MAX_K";
    case BL_ERR_WORKSPACE: return "workspace missing or too small";
    case BL_ERR_ALIGN: return "pointer not aligned as required";
    case BL_ERR_HIP: return "HIP error";
    case BL_ERR_ARG: return "invalid argument";
  }
  return "unknown status";
}

const char* bitlinear_last_hip_error(void) { return g_last_error; }

int bitlinear_abi_version(void) { return BL_ABI_VERSION; }

}  // extern "C"
