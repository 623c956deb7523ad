// bl_internal.h -- host-side launch functions shared between the kernel sources and
// the C ABI (bl_capi.hip). Validation happens in the C ABI before any of these runs.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bitlinear.h"

#define BL_GROUP_CAP BL_MAX_GROUP

// One projection as the product kernels see it (host-validated, K % 4 == 0).
struct bl_proj_internal {
  const int8_t* Xq;
  const float* x_scale;
  const uint8_t* W;
  const float* w_scale;
  float* Y;
  int32_t* acc;
  int N;
  int K;
  int rpg;  // rows per weight scale group: row o uses w_scale[o / rpg] (rpg = N: one scale)
};

// Compute units of the current device, queried once per process and cached (the
// library targets one part, so every device it runs on has the same count). Safe to
// call from several threads: a race only repeats the query and stores the same value.
int bl_device_cus();
// Resident workgroups of `kernel` with `threads` threads and `lds` dynamic LDS bytes
// (the occupancy query times bl_device_cus(); `fallback` per CU if the query fails),
// cached in `slot`; the same thread-safety as bl_device_cus.
int bl_resident_wgs(const void* kernel, int threads, size_t lds, int fallback, int* slot);

size_t bl_weight_workspace_bytes_impl(int64_t N, int64_t K);
hipError_t bl_launch_quantize_weights(const float* W, int64_t N, int64_t K, uint8_t* P,
                                      float* w_scale, double* w_gamma, void* ws,
                                      hipStream_t stream);
hipError_t bl_launch_quantize_acts(const bl_act_desc* d, int count, int64_t T, float eps,
                                   uint32_t flags, hipStream_t stream);

// Product kernels: each takes 1..BL_GROUP_CAP projections sharing T.
bool bl_gemv_supports(int T, int K);
hipError_t bl_launch_gemv(const bl_proj_internal* p, int count, int T, hipStream_t stream);
bool bl_skinny_supports(int T, int64_t N, int K);
hipError_t bl_launch_skinny(const bl_proj_internal* p, int count, int T, hipStream_t stream);
bool bl_prefill_supports(int T, int K);
// scratch: int32 partial products of a split-K launch, at least
// bl_prefill_scratch_bytes(T, N, K) bytes, or null (then no split)
size_t bl_prefill_scratch_bytes(int T, int N, int K);
// true when a product of T <= 128 tokens would run split-K (slices fill the device)
bool bl_prefill_splits(int T, int N, int K);
hipError_t bl_launch_prefill(const bl_proj_internal* p, int T, int32_t* scratch,
                             size_t scratch_bytes, hipStream_t stream);
hipError_t bl_launch_generic(const bl_proj_internal* p, int T, hipStream_t stream);

// BitDelta: base bf16 [N, M] plus B interleaved 1-bit deltas, one token per model.
hipError_t bl_launch_bitdelta_compress(const float* W_fine, const uint16_t* W_base, int64_t N,
                                       int64_t M, int model, uint8_t* D, float* alpha, void* ws,
                                       hipStream_t stream);
bool bl_bitdelta_supports(int64_t N, int64_t M, int B);
hipError_t bl_launch_bitdelta(const uint16_t* base, const uint8_t* D, const float* alpha,
                              const float* X, float* Y, int64_t N, int64_t M, int B,
                              hipStream_t stream);

// The training side: fake quantization with the warm-up lambda, RMSNorm backward.
hipError_t bl_launch_fake_quant_weights(const float* W, int64_t N, int64_t K, const float* w_scale,
                                        float lam, uint16_t* out, hipStream_t stream);
hipError_t bl_launch_fake_quant_acts(const float* X, const float* gain, int64_t T, int64_t K,
                                     float eps, uint32_t flags, float lam, int8_t* Xq, float* xs,
                                     uint16_t* xfq, double* rinv, hipStream_t stream);
hipError_t bl_launch_rmsnorm_backward(const float* X, const float* gain, const double* rinv,
                                      const float* dY, int64_t T, int64_t K, float* dX,
                                      float* dgain, hipStream_t stream);

// The 1-bit sign variant: weights 8 codes per byte (N rows of K/8 bytes).
hipError_t bl_launch_quantize_weights_sign(const float* W, int64_t N, int64_t K, uint8_t* P,
                                           float* w_scale, double* w_alpha, void* ws,
                                           hipStream_t stream);
bool bl_gemv_sign_supports(int T, int K);
hipError_t bl_launch_gemv_sign(const bl_proj_internal* p, int count, hipStream_t stream);
hipError_t bl_launch_generic_sign(const bl_proj_internal* p, int T, hipStream_t stream);

// Measurement: the HBM read stream and the int8 MFMA stream (bl_roof.hip).
size_t bl_roof_read_sink_words(int64_t total_bytes);
hipError_t bl_launch_roof_read(const void* const* bufs, const int64_t* bytes, int count,
                               int schedule, uint32_t* sink, hipStream_t stream);
hipError_t bl_launch_roof_mfma(int iters, int wgs, int32_t* sink, uint64_t* clocks,
                               hipStream_t stream);
