// Host-side launchers of the MoE layer kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

size_t route_ws_bytes(int T, int H, int E, bool bf16, bool prob);
hipError_t launch_route(const void* x, const void* wg, const float* bias, int T, int H, int E,
                        int k, bool bf16, int32_t* topk_idx, float* topk_w, float* prob_mean,
                        void* ws, hipStream_t s);

int dispatch_blocks(int T, int k);
size_t dispatch_ws_bytes(int T, int E, int k);
hipError_t launch_dispatch(const int32_t* topk_idx, const void* x, int T, int H, int E, int k,
                           int cap, bool bf16, int32_t* counts, int32_t* offsets, int32_t* perm,
                           int32_t* inv, void* xs, void* ws, hipStream_t s);

size_t noalloc_scratch_bytes();
hipError_t launch_dispatch_noalloc(const int32_t* topk_idx, const void* x, int T, int H, int E,
                                   int k, bool bf16, int32_t* counts, int32_t* offsets,
                                   int32_t* perm, int32_t* inv, void* xs, hipStream_t s);

size_t ffn_ws_bytes(int rows, int T, int E, int H, int F, int Fs, bool bf16);
hipError_t launch_expert_ffn(const void* xs, const int32_t* gather, int gk,
                             const int32_t* offsets, int rows, int E, int H, int F, const void* w1,
                             const void* w2, const void* x, const void* ws1, const void* ws2,
                             int T, int Fs, bool bf16, void* ys, void* ysh, void* ws,
                             hipStream_t s, void* const* events = nullptr);

hipError_t launch_combine(const void* ys, const int32_t* inv, const float* topk_w,
                          const void* ysh, int T, int H, int k, bool bf16, void* out,
                          hipStream_t s);

hipError_t launch_load_stats(const int32_t* counts, int T, int E, int k, double cf,
                             void* stats, int32_t* overflow, int32_t* straggler_ids,
                             hipStream_t s);

hipError_t launch_bias_update(const int32_t* counts, int E, float gamma, float* bias,
                              float* load_frac, hipStream_t s);

}  // namespace moe
