// Internal launch interface between the C ABI (abi.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "check.h"

namespace orthrus {

// Launch a kernel whose only parameter is an argument struct; returns the
// launch status directly (hipLaunchKernel reports configuration errors itself,
// so no sticky error of an unrelated earlier call is picked up).
template <typename A>
hipError_t launch_kernel(void (*kernel)(A), dim3 grid, dim3 block, hipStream_t stream, A args) {
  void* ptrs[] = {static_cast<void*>(&args)};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0, stream);
}

hipError_t launch_attention(const AttnPlan& plan, const orthrus_kv& kv, const void* q,
                            const void* k_blk, const void* v_blk, void* out, float scale,
                            bool verify, void* ws, hipStream_t stream);

// Device address of the static attention scratch on the current device
// (kStaticScratchBytes bytes), looked up once per device.
hipError_t static_attn_scratch(void** ptr);

// Device address of the current device's error word (ORTHRUS_DEVERR_* bits),
// looked up once per device; and the call that copies (and clears) it.
hipError_t device_error_word(unsigned int** ptr);
hipError_t launch_device_errors(uint32_t* out, int clear, hipStream_t stream);

hipError_t launch_argmax(const ArgmaxPlan& plan, const float* logits, int32_t* out, void* ws,
                         hipStream_t stream);

hipError_t launch_accept(const ArgmaxPlan& plan, const float* logits_a, const int32_t* draft,
                         int B, int K, int32_t* a, int32_t* n_acc, int32_t* n_emit,
                         int32_t* next_anchor, void* ws, hipStream_t stream);

// Row maxima of per-chunk argmax keys [rows][nchunks] (keys.h).
hipError_t launch_argmax_keys(const unsigned long long* keys, int rows, int nchunks, int32_t* out,
                              hipStream_t stream);

// Acceptance from per-chunk keys of the AR view's rows [B*K][nchunks].
hipError_t launch_accept_keys(const unsigned long long* keys, int nchunks, const int32_t* draft, int B,
                              int K, int32_t* a, int32_t* n_acc, int32_t* n_emit, int32_t* next_anchor,
                              hipStream_t stream);

// LM head + per-workgroup argmax keys [rows][plan.nwg] into ws (optionally
// also the fp32 logits [rows][vocab]).
hipError_t launch_lmhead(const LmHeadPlan& plan, const void* hidden, const void* weight, float* logits,
                         void* ws, hipStream_t stream);

hipError_t launch_commit(const orthrus_kv& kv, int layers, int64_t pool_layer_stride,
                         const void* k_blk, const void* v_blk, int64_t blk_layer_stride,
                         const int32_t* n_emit, int B, int K, int32_t* seq_lens_out,
                         hipStream_t stream);

// Temperature sampling (statistics + one draw per row) and the
// speculative-sampling consensus (statistics, acceptance, residual draw).
hipError_t launch_sample(const SamplePlan& plan, const float* logits, float temperature, const float* u,
                         int32_t* out, void* ws, hipStream_t stream);
hipError_t launch_accept_sampled(const SamplePlan& plan, const float* logits_d, const float* logits_a,
                                 const int32_t* draft, int B, int K, float temperature, const float* u_acc,
                                 const float* u_res, int32_t* tokens, int32_t* n_acc, int32_t* n_emit,
                                 int32_t* next_anchor, void* ws, hipStream_t stream);

// bf16 [rows][Hkv][D] -> e4m3 codes with per-head scales, K and V in one launch.
hipError_t launch_quantize_kv(const void* k, const void* v, const float* k_scale, const float* v_scale,
                              int rows, int Hkv, int D, void* k_out, void* v_out, hipStream_t stream);

}  // namespace orthrus
