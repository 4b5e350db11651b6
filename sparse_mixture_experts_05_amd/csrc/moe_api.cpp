// C ABI of the MoE layer library: argument validation (always before any HIP
// call, so a rejected call enqueues nothing), workspace sizing, launches on
// the caller's stream. The semantics of each entry point are documented in
// include/moe.h.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <cmath>

#include "kernels.hpp"

namespace {

constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 8;

bool dtype_ok(int dt) { return dt == MOE_F32 || dt == MOE_BF16; }

// Shared shape checks of (T, H, E, k). Returns MOE_OK or an error status.
int check_tokens(int T, int H, int E, int k) {
  if (T < 1 || H < 1 || E < 1 || k < 1) return MOE_ERR_INVALID_ARG;
  if (E > kMaxExperts || k > kMaxTopK || k > E) return MOE_ERR_UNSUPPORTED;
  if (H % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if ((long long)T * k >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Rows and weights are read and written with 16-byte vector accesses.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, non-positive size or bad dtype)";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape (needs 1<=E<=256, 1<=k<=min(E,8), H%64==0, F%64==0, T*k<2^31)";
    case MOE_ERR_WORKSPACE: return "workspace missing or smaller than the size query returned";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_SCRATCH: return "request exceeds the fixed 1 MiB scratch of moe_dispatch_noalloc (needs E * ceil(T / 256) * 4 <= 1 MiB; use moe_dispatch with a workspace)";
    default: return "unknown status";
  }
}

size_t moe_route_workspace_bytes(int T, int H, int E, int k, int dtype) {
  if (!dtype_ok(dtype) || check_tokens(T, H, E, k) != MOE_OK) return 0;
  return moe::route_ws_bytes(T, H, E, dtype == MOE_BF16, true);
}

int moe_route(const void* x, const void* wg, const float* bias, int T, int H, int E, int k,
              int dtype, int32_t* topk_idx, float* topk_w, float* prob_mean, void* ws,
              size_t ws_bytes, void* stream) {
  if (!x || !wg || !topk_idx || !topk_w || !dtype_ok(dtype)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(wg) || (ws && !aligned16(ws))) return MOE_ERR_INVALID_ARG;
  const int st = check_tokens(T, H, E, k);
  if (st != MOE_OK) return st;
  const size_t need = moe::route_ws_bytes(T, H, E, dtype == MOE_BF16, prob_mean != nullptr);
  if (need > 0 && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  return from_hip(moe::launch_route(x, wg, bias, T, H, E, k, dtype == MOE_BF16, topk_idx, topk_w,
                                    prob_mean, ws, as_stream(stream)));
}

size_t moe_dispatch_workspace_bytes(int T, int E, int k) {
  if (check_tokens(T, 64, E, k) != MOE_OK) return 0;
  return moe::dispatch_ws_bytes(T, E, k);
}

int moe_dispatch(const int32_t* topk_idx, const void* x, int T, int H, int E, int k, int dtype,
                 int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv, void* xs,
                 void* ws, size_t ws_bytes, void* stream) {
  if (!topk_idx || !counts || !offsets || !perm || !inv || !dtype_ok(dtype))
    return MOE_ERR_INVALID_ARG;
  if (xs && (!x || !aligned16(x) || !aligned16(xs))) return MOE_ERR_INVALID_ARG;
  const int st = check_tokens(T, H, E, k);
  if (st != MOE_OK) return st;
  if (!ws || ws_bytes < moe::dispatch_ws_bytes(T, E, k)) return MOE_ERR_WORKSPACE;
  return from_hip(moe::launch_dispatch(topk_idx, x, T, H, E, k, -1, dtype == MOE_BF16, counts,
                                       offsets, perm, inv, xs, ws, as_stream(stream)));
}

int moe_dispatch_noalloc(const int32_t* topk_idx, const void* x, int T, int H, int E, int k,
                         int dtype, int32_t* counts, int32_t* offsets, int32_t* perm,
                         int32_t* inv, void* xs, void* stream) {
  if (!topk_idx || !counts || !offsets || !perm || !inv || !dtype_ok(dtype))
    return MOE_ERR_INVALID_ARG;
  if (xs && (!x || !aligned16(x) || !aligned16(xs))) return MOE_ERR_INVALID_ARG;
  const int st = check_tokens(T, H, E, k);
  if (st != MOE_OK) return st;
  if (moe::dispatch_ws_bytes(T, E, k) > moe::noalloc_scratch_bytes()) return MOE_ERR_SCRATCH;
  return from_hip(moe::launch_dispatch_noalloc(topk_idx, x, T, H, E, k, dtype == MOE_BF16, counts,
                                               offsets, perm, inv, xs, as_stream(stream)));
}

int64_t moe_capacity(int T, int k, int E, double capacity_factor) {
  if (T < 1 || k < 1 || E < 1) return -1;
  if (!(capacity_factor > 0.0) || !std::isfinite(capacity_factor)) return -1;
  // the same double operations as the statistics kernel: (T*k)/E first, then *cf
  const double cap = ((double)((long long)T * k) / (double)E) * capacity_factor;
  if (cap >= 2147483647.0) return 2147483647;
  return (int64_t)cap;
}

int moe_dispatch_capped(const int32_t* topk_idx, const void* x, int T, int H, int E, int k,
                        int capacity, int dtype, int32_t* counts, int32_t* offsets, int32_t* perm,
                        int32_t* inv, void* xs, void* ws, size_t ws_bytes, void* stream) {
  if (!topk_idx || !counts || !offsets || !perm || !inv || !dtype_ok(dtype) || capacity < 0)
    return MOE_ERR_INVALID_ARG;
  if (xs && (!x || !aligned16(x) || !aligned16(xs))) return MOE_ERR_INVALID_ARG;
  const int st = check_tokens(T, H, E, k);
  if (st != MOE_OK) return st;
  if (!ws || ws_bytes < moe::dispatch_ws_bytes(T, E, k)) return MOE_ERR_WORKSPACE;
  return from_hip(moe::launch_dispatch(topk_idx, x, T, H, E, k, capacity, dtype == MOE_BF16,
                                       counts, offsets, perm, inv, xs, ws, as_stream(stream)));
}

static int check_ffn(int rows, int T, int H, int E, int F, int Fs, int dtype) {
  if (rows < 1 || T < 1 || H < 1 || E < 1 || F < 1 || Fs < 0 || !dtype_ok(dtype))
    return MOE_ERR_INVALID_ARG;
  if (E > kMaxExperts || H % 64 != 0 || F % 64 != 0 || Fs % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if ((long long)rows > (long long)T * kMaxTopK) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t moe_expert_ffn_workspace_bytes(int rows, int T, int H, int E, int F, int Fs, int dtype) {
  if (check_ffn(rows, T, H, E, F, Fs, dtype) != MOE_OK) return 0;
  return moe::ffn_ws_bytes(rows, T, E, H, F, Fs, dtype == MOE_BF16);
}

int moe_expert_ffn(const void* xs, const int32_t* offsets, int rows, int E, int H, int F,
                   const void* w1, const void* w2, const void* x, const void* ws1,
                   const void* ws2, int T, int Fs, int dtype, void* ys, void* ysh, void* ws,
                   size_t ws_bytes, void* stream) {
  if (!xs || !offsets || !w1 || !w2 || !ys) return MOE_ERR_INVALID_ARG;
  if (!aligned16(xs) || !aligned16(w1) || !aligned16(w2) || !aligned16(ys)) return MOE_ERR_INVALID_ARG;
  const int st = check_ffn(rows, T, H, E, F, Fs, dtype);
  if (st != MOE_OK) return st;
  if (Fs > 0 && (!x || !ws1 || !ws2 || !ysh)) return MOE_ERR_INVALID_ARG;
  if (Fs > 0 && (!aligned16(x) || !aligned16(ws1) || !aligned16(ws2) || !aligned16(ysh)))
    return MOE_ERR_INVALID_ARG;
  if (ws && !aligned16(ws)) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < moe::ffn_ws_bytes(rows, T, E, H, F, Fs, dtype == MOE_BF16))
    return MOE_ERR_WORKSPACE;
  return from_hip(moe::launch_expert_ffn(xs, nullptr, 0, offsets, rows, E, H, F, w1, w2, x, ws1,
                                         ws2, T, Fs, dtype == MOE_BF16, ys,
                                         Fs > 0 ? ysh : nullptr, ws, as_stream(stream)));
}

int moe_expert_ffn_gather(const void* x, const int32_t* perm, int k, const int32_t* offsets,
                          int rows, int E, int H, int F, const void* w1, const void* w2,
                          const void* ws1, const void* ws2, int T, int Fs, int dtype, void* ys,
                          void* ysh, void* ws, size_t ws_bytes, void* stream) {
  return moe_expert_ffn_gather_timed(x, perm, k, offsets, rows, E, H, F, w1, w2, ws1, ws2, T, Fs,
                                     dtype, ys, ysh, ws, ws_bytes, stream, nullptr);
}

int moe_expert_ffn_gather_timed(const void* x, const int32_t* perm, int k, const int32_t* offsets,
                                int rows, int E, int H, int F, const void* w1, const void* w2,
                                const void* ws1, const void* ws2, int T, int Fs, int dtype,
                                void* ys, void* ysh, void* ws, size_t ws_bytes, void* stream,
                                void* const* events) {
  if (!x || !perm || !offsets || !w1 || !w2 || !ys) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w1) || !aligned16(w2) || !aligned16(ys)) return MOE_ERR_INVALID_ARG;
  if (k < 1) return MOE_ERR_INVALID_ARG;
  if (k > kMaxTopK || (long long)T * k >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  const int st = check_ffn(rows, T, H, E, F, Fs, dtype);
  if (st != MOE_OK) return st;
  if ((long long)rows > (long long)T * k) return MOE_ERR_UNSUPPORTED;
  if (Fs > 0 && (!ws1 || !ws2 || !ysh)) return MOE_ERR_INVALID_ARG;
  if (Fs > 0 && (!aligned16(ws1) || !aligned16(ws2) || !aligned16(ysh))) return MOE_ERR_INVALID_ARG;
  if (ws && !aligned16(ws)) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < moe::ffn_ws_bytes(rows, T, E, H, F, Fs, dtype == MOE_BF16))
    return MOE_ERR_WORKSPACE;
  return from_hip(moe::launch_expert_ffn(x, perm, k, offsets, rows, E, H, F, w1, w2, x, ws1, ws2,
                                         T, Fs, dtype == MOE_BF16, ys, Fs > 0 ? ysh : nullptr, ws,
                                         as_stream(stream), events));
}

int moe_combine(const void* ys, const int32_t* inv, const float* topk_w, const void* ysh, int T,
                int H, int k, int dtype, void* out, void* stream) {
  if (!ys || !inv || !topk_w || !out || !dtype_ok(dtype)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(ys) || !aligned16(out) || (ysh && !aligned16(ysh))) return MOE_ERR_INVALID_ARG;
  const int st = check_tokens(T, H, kMaxTopK, k);
  if (st != MOE_OK) return st;
  return from_hip(moe::launch_combine(ys, inv, topk_w, ysh, T, H, k, dtype == MOE_BF16, out,
                                      as_stream(stream)));
}

int moe_load_stats(const int32_t* counts, int T, int E, int k, double capacity_factor,
                   moe_load_stats_t* stats, int32_t* overflow, int32_t* straggler_ids,
                   void* stream) {
  if (!counts || !stats || !straggler_ids) return MOE_ERR_INVALID_ARG;
  if (!(capacity_factor > 0.0) || !std::isfinite(capacity_factor)) return MOE_ERR_INVALID_ARG;
  const int st = check_tokens(T, 64, E, k);
  if (st != MOE_OK) return st;
  return from_hip(moe::launch_load_stats(counts, T, E, k, capacity_factor, stats, overflow,
                                         straggler_ids, as_stream(stream)));
}

int moe_bias_update(const int32_t* counts, int E, float gamma, float* bias, float* load_frac,
                    void* stream) {
  if (!counts || !bias || E < 1 || !std::isfinite(gamma) || gamma < 0.0f)
    return MOE_ERR_INVALID_ARG;
  if (E > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  return from_hip(moe::launch_bias_update(counts, E, gamma, bias, load_frac, as_stream(stream)));
}

}  // extern "C"
