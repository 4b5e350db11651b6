/*
 * moe.h - C ABI of the single-GPU fine-grained Mixture-of-Experts FFN layer
 * forward for AMD Instinct MI355X (gfx950).
 *
 * The layer has five steps, one entry point each:
 *   moe_route      gate scores, softmax, top-k, renormalised weights
 *   moe_dispatch   expert histogram, offsets, stable permutation, row gather
 *                  (moe_dispatch_capped: the same with each expert's capacity enforced)
 *   moe_expert_ffn grouped Linear -> erf-GeLU -> Linear over ragged segments
 *                  (plus the optional always-on shared expert; moe_expert_ffn_gather:
 *                  the same reading the token rows through perm, no xs copy)
 *   moe_combine    weighted sum of each token's k expert rows (+ shared row)
 *   moe_load_stats capacity, overflow / drops, skew, Gini, stragglers
 * and, after the layer, the routing-bias feedback of the next step:
 *   moe_bias_update dynamic bias B from the expert counts, load fractions f_i
 *   (the mean router probabilities P_i are an optional output of moe_route)
 *
 * Sources of the method (three web pages; cited by title and section):
 *   [K3]   "hncyxsy.com Kimi K3 fine-grained MoE" article: router listing
 *          (FineGrainedMoERouter), the dispatch / local expert FFN / combine
 *          flow, the shared expert, the FFN cost equation.
 *   [DIAG] "Kimi K3 专家路由不均衡诊断" (bjdmk.com.cn): section 3 diagnostics
 *          module (MoERouteDiagnostics) and section 4.2 (biased score).
 *   [BLOG] "lpqz.cn MoE engineering blog": section 3.1 (expert = two Linear
 *          layers with GeLU; dispatcher with one shared buffer).
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE memory owned by the caller, row-major and
 *     contiguous, 16-byte aligned. The library never allocates, frees or keeps
 *     a pointer past the call. Scratch memory comes from a caller-provided
 *     workspace whose size the *_workspace_bytes queries return.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Every
 *     call only enqueues work on it and returns; there is no host
 *     synchronisation, so device-resident results (e.g. offsets) feed the next
 *     call directly. Calls keep no global state and are re-entrant.
 *   - Return value: MOE_OK (0) or a negative moe_status. Arguments are
 *     validated on the host before any HIP call; on error nothing is
 *     enqueued. A failed launch returns MOE_ERR_HIP. A row or weight tensor
 *     (x, wg, xs, w1, w2, ws1, ws2, ys, ysh, out) or workspace whose address
 *     is not a multiple of 16 returns MOE_ERR_INVALID_ARG.
 *   - dtype: MOE_F32 (fp32 activations, weights, arithmetic) or MOE_BF16
 *     (bf16 activations and weights, fp32 accumulation, bf16 results rounded
 *     to nearest even).
 *   - Supported shapes: 1 <= E <= 256, 1 <= k <= min(E, 8), H % 64 == 0,
 *     F % 64 == 0, Fs % 64 == 0 (or Fs == 0), T >= 1, T*k < 2^31.
 *     Anything else returns MOE_ERR_UNSUPPORTED (or MOE_ERR_INVALID_ARG for
 *     null pointers / non-positive sizes).
 *   - Weights use the [out, in] layout of a Linear layer: Wg [E,H],
 *     W1 [E,F,H], W2 [E,H,F], Ws1 [Fs,H], Ws2 [H,Fs]. No Linear has a bias.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null or misaligned pointer, non-positive size, bad enum */
  MOE_ERR_UNSUPPORTED = -2, /* shape outside the supported range */
  MOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than the query */
  MOE_ERR_HIP = -4,         /* a HIP launch failed */
  MOE_ERR_SCRATCH = -5      /* beyond the fixed scratch of moe_dispatch_noalloc */
} moe_status;

/* Load diagnostics of one step ([DIAG] section 3). Written to device memory. */
typedef struct {
  int64_t num_tokens;      /* T */
  int64_t assignments;     /* T*k */
  int64_t capacity;        /* int((T*k / E) * cf), evaluated in double */
  int64_t max_load;        /* max_e counts[e] */
  int64_t min_load;        /* min_e counts[e] */
  int64_t dropped;         /* sum_e max(0, counts[e] - capacity); counted only */
  int64_t num_stragglers;  /* #{e : counts[e] > capacity} */
  int64_t gini_num;        /* 2*sum_i i*c_(i) - (E+1)*sum c  (c sorted ascending, i = 1..E) */
  int64_t gini_den;        /* E * sum c (1 when sum c == 0) */
  double load_skew_ratio;  /* (double)max / ((double)min + 1e-5) */
  double gini;             /* (double)gini_num / (double)gini_den, one division; 0 if sum c == 0 */
  double drop_rate;        /* (double)dropped / (double)(T*k) */
} moe_load_stats_t;

/*
 * moe_route - top-k softmax gating ([K3] router listing; [DIAG] section 4.2).
 *   s[t,e]  = sum_h x[t,h] * wg[e,h] + bias[e]          (fp32 accumulation)
 *   topk_idx[t,0..k-1] = the k largest s[t,:], descending; equal scores take
 *                        the lower expert id first
 *   topk_w[t,j] = exp(s[t,idx_j] - m) / sum_j' exp(s[t,idx_j'] - m), m = max_e s[t,e]
 *               (the softmax over all E experts renormalised over the k chosen
 *                ones; the full-E denominator cancels)
 *   prob_mean[e] = (1/T) sum_t p[t,e], p[t,e] = exp(s[t,e] - m) / sum_e' exp(s[t,e'] - m)
 *               (the P_i of [DIAG] section 4.1: mean router probability of the
 *                biased softmax over all E experts; fp32 sums per workgroup in
 *                token order, summed over workgroups in double in a fixed
 *                order, so repeated calls give the same bits)
 * x        [T,H] dtype          device, read
 * wg       [E,H] dtype          device, read
 * bias     [E]   fp32 or NULL   device, read (NULL = no routing bias)
 * topk_idx [T,k] int32          device, written
 * topk_w   [T,k] fp32           device, written
 * prob_mean [E]  fp32 or NULL   device, written (NULL = not computed)
 * ws / ws_bytes: device workspace of at least moe_route_workspace_bytes(T,H,E,k,dtype)
 *          (NULL / 0 allowed when prob_mean is NULL and the query's score part is 0)
 */
int moe_route(const void* x, const void* wg, const float* bias, int T, int H, int E, int k,
              int dtype, int32_t* topk_idx, float* topk_w, float* prob_mean, void* ws,
              size_t ws_bytes, void* stream);

/* Workspace bytes moe_route needs for (T, H, E, k, dtype) with prob_mean
 * requested: partial score tiles when few tokens (T < 2048, bf16) take the
 * two-launch path, plus one row of E partial probability sums per workgroup.
 * Without prob_mean only the score part is needed, which is 0 for T >= 2048
 * or fp32. Returns 0 on unsupported sizes. */
size_t moe_route_workspace_bytes(int T, int H, int E, int k, int dtype);

/* Workspace bytes moe_dispatch needs for (T, E, k); 0 on unsupported sizes. */
size_t moe_dispatch_workspace_bytes(int T, int E, int k);

/*
 * moe_dispatch - group the T*k (token, slot) assignments by expert
 * ([BLOG] section 3.1 dispatcher; histogram as in [DIAG] section 3).
 *   counts[e]   = #{(t,j) : topk_idx[t,j] == e}
 *   offsets[0]  = 0, offsets[e+1] = offsets[e] + counts[e]
 *   perm[p]     = t*k + j for buffer row p, in expert-major, token-ascending
 *                 order (a stable sort of the row-major assignments by expert)
 *   inv[t*k+j]  = p, the inverse of perm
 *   xs[p,:]     = x[perm[p] / k, :] (exact copy)
 * topk_idx [T,k] int32 in [0,E)  device, read (ids of one token are distinct)
 * x        [T,H] dtype           device, read
 * counts [E], offsets [E+1], perm [T*k], inv [T*k] int32; xs [T*k,H] dtype: device, written
 * xs may be NULL: then no rows are copied (x is not read and may be NULL too),
 * for moe_expert_ffn_gather, which reads x through perm itself.
 * ws / ws_bytes: device workspace of at least moe_dispatch_workspace_bytes(T,E,k)
 */
int moe_dispatch(const int32_t* topk_idx, const void* x, int T, int H, int E, int k, int dtype,
                 int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv, void* xs,
                 void* ws, size_t ws_bytes, void* stream);

/*
 * moe_dispatch_noalloc - moe_dispatch for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same kernels and results, bit for bit, with the
 * histogram table in a fixed 1 MiB device array of the library instead of a
 * caller workspace. The library itself never allocates in this call.
 * Limit: the table needs E * ceil(T / 256) * 4 bytes (64-token blocks for
 * 256 < T <= 4096 with k >= 4), which must fit 1 MiB: every T <= 2^26 / E
 * (T <= 262144 at E = 256). A larger request returns MOE_ERR_SCRATCH and
 * enqueues nothing.
 * Each GPU holds one copy of the array until the process ends, and every call
 * on that GPU shares it: two calls that may run at the same time on one GPU
 * (on different streams, or from different host threads) race and give wrong
 * results; calls ordered on one stream do not. Nothing in the array needs
 * clearing between calls (the histogram launch writes every entry the rank
 * launch reads). Arguments, outputs and other errors as moe_dispatch.
 */
int moe_dispatch_noalloc(const int32_t* topk_idx, const void* x, int T, int H, int E, int k,
                         int dtype, int32_t* counts, int32_t* offsets, int32_t* perm,
                         int32_t* inv, void* xs, void* stream);

/*
 * moe_capacity - the per-expert capacity of [DIAG] section 3 (its
 * diagnostics listing: the mean assignments per expert times the capacity
 * factor, truncated to an integer):
 *   capacity = int(((double)(T*k) / (double)E) * capacity_factor)
 * evaluated in double in that order, the value moe_load_stats reports in
 * moe_load_stats_t.capacity and the one to pass to moe_dispatch_capped.
 * Host-only: reads no device memory and enqueues nothing.
 * Returns -1 if T < 1, k < 1, E < 1 or capacity_factor is not a finite
 * value > 0; a capacity above INT32_MAX is returned as INT32_MAX (every
 * assignment is then kept, since T*k < 2^31).
 */
int64_t moe_capacity(int T, int k, int E, double capacity_factor);

/*
 * moe_dispatch_capped - moe_dispatch with each expert's capacity enforced
 * ([DIAG] section 3 counts the assignments past an expert's capacity
 * int(T*k/E*cf); section 5 describes dropping them). Every expert keeps its
 * first `capacity` assignments in token order (the order of moe_dispatch);
 * the others are dropped: they get no buffer row and inv = -1.
 *   counts[e]  = raw count, as in moe_dispatch (before dropping)
 *   offsets[0] = 0, offsets[e+1] = offsets[e] + min(counts[e], capacity)
 *   perm[p], xs[p] for p < offsets[E]: the kept rows, as in moe_dispatch
 *                  (entries p >= offsets[E] are not written)
 *   inv[t*k+j]  = the buffer row of a kept assignment, -1 for a dropped one
 * moe_expert_ffn then runs on the kept rows (pass rows = T*k: an upper bound)
 * and moe_combine skips the dropped assignments without renormalising the
 * kept weights. capacity >= 0 (0 drops every assignment); the layer's value
 * is moe_capacity(T, k, E, capacity_factor). Other arguments, the workspace
 * and errors as moe_dispatch.
 */
int moe_dispatch_capped(const int32_t* topk_idx, const void* x, int T, int H, int E, int k,
                        int capacity, int dtype, int32_t* counts, int32_t* offsets, int32_t* perm,
                        int32_t* inv, void* xs, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes moe_expert_ffn needs; 0 on unsupported sizes. */
size_t moe_expert_ffn_workspace_bytes(int rows, int T, int H, int E, int F, int Fs, int dtype);

/*
 * moe_expert_ffn - grouped expert FFN over the expert-contiguous buffer
 * ([BLOG] section 3.1: each expert is Linear -> GeLU -> Linear; [K3]: one
 * always-on shared expert; FLOPs 4*rows*H*F + 4*T*H*Fs as in [K3]'s
 * compute-time equation).
 *   for each expert e and row p in [offsets[e], offsets[e+1]):
 *     h      = GeLU(xs[p,:] . W1[e]^T)      GeLU(a) = 0.5*a*(1 + erf(a/sqrt(2)))
 *     ys[p,:] = h . W2[e]^T
 *   shared expert (when Fs > 0): ysh[t,:] = GeLU(x[t,:] . Ws1^T) . Ws2^T
 * xs [rows,H], offsets [E+1] (device, from moe_dispatch or moe_dispatch_capped;
 *   offsets[E] <= rows: rows is an upper bound that sizes the launch and the
 *   workspace, and ys rows past offsets[E] are not written)
 * w1 [E,F,H], w2 [E,H,F]; x [T,H], ws1 [Fs,H], ws2 [H,Fs] (NULL / Fs = 0: no shared expert)
 * ys [rows,H], ysh [T,H] (NULL when Fs = 0): device, written.
 * In bf16 mode h is rounded to bf16 before the second Linear (fp32 accumulation
 * in both); ys and ysh are rounded to bf16; erf is evaluated with Abramowitz &
 * Stegun formula 7.1.26 (|error| <= 1.5e-7, far below the bf16 step of h). fp32
 * mode uses the device library's erff.
 * ws / ws_bytes: device workspace of at least moe_expert_ffn_workspace_bytes(...)
 */
int moe_expert_ffn(const void* xs, const int32_t* offsets, int rows, int E, int H, int F,
                   const void* w1, const void* w2, const void* x, const void* ws1,
                   const void* ws2, int T, int Fs, int dtype, void* ys, void* ysh, void* ws,
                   size_t ws_bytes, void* stream);

/*
 * moe_expert_ffn_gather - moe_expert_ffn with the dispatch gather fused into
 * the first Linear: buffer row p of the routed experts is read from the token
 * rows directly, xs[p,:] = x[perm[p] / k, :] ([BLOG] section 3.1 groups token
 * indices by expert; the copy into a shared buffer is not materialised).
 * Results are bit-identical to moe_dispatch (with xs) followed by moe_expert_ffn.
 * x [T,H] dtype, perm [rows] int32 (device, from moe_dispatch or
 *   moe_dispatch_capped, which may run with xs = NULL), 1 <= k <= 8 the
 *   experts per token of that dispatch; a perm entry outside [0, T*k) is
 *   clamped into it (never read out of bounds).
 * All other arguments, the workspace (moe_expert_ffn_workspace_bytes) and the
 * errors as moe_expert_ffn; x is required (it is the routed input as well as
 * the shared expert's).
 */
int moe_expert_ffn_gather(const void* x, const int32_t* perm, int k, const int32_t* offsets,
                          int rows, int E, int H, int F, const void* w1, const void* w2,
                          const void* ws1, const void* ws2, int T, int Fs, int dtype, void* ys,
                          void* ysh, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_expert_ffn_gather_timed - moe_expert_ffn_gather that also records
 * caller-created HIP events on `stream`, for timing the grouped GEMM kernel
 * itself (the FFN's dominant kernel) with events on the stream it runs on:
 * events[0] / events[1] right before / after the up projection's GEMM launch,
 * events[2] / events[3] the same for the down projection. The planning launch
 * and any split-K reduce launch fall outside the pairs. events: host array of
 * 4 hipEvent_t (as void*), owned by the caller; NULL, or a NULL entry, records
 * nothing there. Results, arguments and errors as moe_expert_ffn_gather; a
 * failed event record returns MOE_ERR_HIP.
 */
int moe_expert_ffn_gather_timed(const void* x, const int32_t* perm, int k, const int32_t* offsets,
                                int rows, int E, int H, int F, const void* w1, const void* w2,
                                const void* ws1, const void* ws2, int T, int Fs, int dtype,
                                void* ys, void* ysh, void* ws, size_t ws_bytes, void* stream,
                                void* const* events);

/*
 * moe_combine - weighted combine back to token order ([K3] combine phase;
 * [BLOG] section 3.1 "scatter back to the original positions").
 *   out[t,:] = sum_{j=0..k-1} topk_w[t,j] * ys[inv[t*k+j],:]  (+ ysh[t,:])
 * summed in fp32, j ascending, shared row last; one write per token (no atomics).
 * An assignment with inv < 0 (dropped by moe_dispatch_capped) adds nothing;
 * the other weights are used as they are.
 * ys [T*k,H] dtype, inv [T*k] int32, topk_w [T,k] fp32, ysh [T,H] dtype or NULL: device, read
 * out [T,H] dtype: device, written
 */
int moe_combine(const void* ys, const int32_t* inv, const float* topk_w, const void* ysh, int T,
                int H, int k, int dtype, void* out, void* stream);

/*
 * moe_load_stats - per-step load diagnostics ([DIAG] section 3) from the
 * expert counts that moe_dispatch produced (the routing actually taken).
 * counts        [E] int32            device, read (sum must be T*k)
 * stats         moe_load_stats_t     device, written
 * overflow      [E] int32 or NULL    device, written: max(0, counts[e] - capacity)
 * straggler_ids [E] int32            device, written: ids with counts[e] > capacity,
 *                                    ascending, then -1 up to E entries
 * capacity_factor > 0.
 */
int moe_load_stats(const int32_t* counts, int T, int E, int k, double capacity_factor,
                   moe_load_stats_t* stats, int32_t* overflow, int32_t* straggler_ids,
                   void* stream);

/*
 * moe_bias_update - one step of the dynamic routing bias ([DIAG] section 4.2:
 * lower the bias of an overloaded expert by a small step, raise that of an
 * idle one) and the load fractions of [DIAG] section 4.1.
 *   mean = sum_e counts[e] / E (compared exactly: counts[e]*E vs sum)
 *   bias[e] <- bias[e] - gamma  if counts[e] > mean   (fp32 arithmetic)
 *              bias[e] + gamma  if counts[e] < mean
 *              bias[e]          otherwise
 *   load_frac[e] = counts[e] / sum_e' counts[e'] (double division, rounded
 *                  to fp32; 0 when the sum is 0)
 * counts    [E] int32 >= 0  device, read (one step's counts from moe_dispatch,
 *                           or counts summed by the caller over a window)
 * bias      [E] fp32        device, read and written in place
 * load_frac [E] fp32 or NULL device, written
 * gamma: finite, >= 0. 1 <= E <= 256.
 * The bias feeds the next moe_route; calls on one stream keep that order.
 */
int moe_bias_update(const int32_t* counts, int E, float gamma, float* bias, float* load_frac,
                    void* stream);

/* Static, human-readable text for a status code. */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
