/*
 * moe.h -- C ABI of libmoe.so: the forward pass of one Mixture-of-Experts
 * layer on one AMD Instinct MI355X (gfx950), in five calls.
 *
 * Sources for what each call computes:
 *   [Routing page] "MoE混合专家模型路由机制原理与稀疏激活实现" (yunthe.com):
 *     section "MoE混合专家模型架构与门控路由原理" -- gate equation
 *       G(x) = softmax(TopK(x . W_g)) and output y = sum_i G(x)_i E_i(x);
 *     section "Top-K门控路由的PyTorch实现" -- TopKRouter (bias-free linear
 *       gate, softmax, top-k, renormalise), Expert (w2(silu(w1 x)) with
 *       biases), MoELayer (slot-by-slot gate-weighted accumulation) and
 *       load_balancing_loss (E * sum f * P);
 *     section "Expert Choice路由策略与容量因子调优" -- capacity
 *       = tokens / experts * factor; rejected tokens pass on the residual.
 *   [Trilemma page] "MoE三难困境破解：按需加载+路由解耦+显存精控"
 *     (0539edu.com), sections 3.2-3.3 -- the router returns (weights,
 *     indices); the executor counts tokens per expert and runs one grouped
 *     FFN per expert group.
 *   [Guide page] "MoE 架构完整指南：路由、负载均衡、EP、训练稳定性、Serving"
 *     (walkerchi.com), section 5.2 -- a per-expert router bias on the logits.
 *
 * Conventions shared by every call:
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise.
 *     Tensors are dense, row-major, and 16-byte aligned.
 *   - The caller owns every buffer, workspace included. The library never
 *     allocates, frees or synchronises, and holds no state between calls.
 *   - Each call enqueues its kernels on `stream` (a hipStream_t; NULL means
 *     the null stream) and returns at once with a status code. Arguments are
 *     validated on the host before anything is launched; on a non-zero status
 *     nothing was enqueued, except for MOE_ERR_LAUNCH.
 *   - dtype is MOE_F32 or MOE_BF16 and applies to x, the weights, the expert
 *     biases and residual; out is fp32 or, for bf16 layers, optionally bf16.
 *     The expert outputs y_perm are fp32 (fp32 layers) or block fixed point
 *     (bf16 layers; see moe_expert_output_bytes). Logits, gates, probability
 *     sums, f, P and the loss are always fp32; indices and offsets are int32.
 *   - Inputs must be finite: NaN or Inf in x or the weights is outside the
 *     contract.
 *   - Results are deterministic: every sum has a fixed order and no kernel
 *     uses floating-point atomics.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *moe_stream_t; /* a hipStream_t */

enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID = 1,     /* bad pointer, size or flag */
    MOE_ERR_UNSUPPORTED = 2, /* shape or dtype this build has no kernel for */
    MOE_ERR_LAUNCH = 3,      /* the HIP runtime rejected a launch */
    MOE_ERR_WORKSPACE = 4    /* ws_bytes smaller than moe_workspace_size() */
};

enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 };

enum moe_op {
    MOE_OP_ROUTER = 0,
    MOE_OP_PERMUTE = 1,
    MOE_OP_FFN = 2,
    MOE_OP_FFN_BWD = 3,   /* moe_grouped_ffn_backward */
    MOE_OP_ROUTER_BWD = 4 /* moe_router_weight_backward */
};

/* Static text for a status code (host memory, never freed). */
const char *moe_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int moe_version(void);

/*
 * Host-side check of the permutation arrays   [Routing page, counting sort
 * of the MoELayer dispatch; capacity section for the drops]. All pointers
 * are HOST pointers; any of the three arrays may be NULL:
 *   offsets [E+1]: offsets[0] = 0, non-decreasing, R = offsets[E] <= T*k;
 *   sorted_token [R] (needs offsets): every entry in [0, T);
 *   dest_row [T*k]: every entry -1 or in [0, R) (R = T*k without offsets);
 *   with all three: each row 0..R-1 is the row of exactly one slot i
 *   (dest_row[i] = r) and sorted_token[r] = i / k, the slot's token.
 * The token-choice layout has k slots per token; the Expert Choice layout
 * has E (k = E). Returns MOE_OK or MOE_ERR_INVALID; reads nothing else,
 * writes nothing. A library built with MOE_HOST_BOUNDS_CHECK runs these
 * checks on the device arrays (copied to the host after synchronising the
 * stream) at the top of moe_grouped_ffn, moe_grouped_ffn_train,
 * moe_grouped_ffn_cached, moe_combine, moe_combine_backward,
 * moe_grouped_ffn_backward and moe_gather_backward, and returns
 * MOE_ERR_INVALID instead of launching on bad arrays.
 */
int moe_check_permutation(const int32_t *offsets, int E, const int32_t *sorted_token,
                          const int32_t *dest_row, int T, int k);

/* 1 in a library built with MOE_HOST_BOUNDS_CHECK (the debug build), else 0. */
int moe_debug_checks(void);

/*
 * Bytes of `rows` rows of y_perm, the expert outputs of moe_grouped_ffn that
 * moe_combine and moe_combine_backward read. MOE_F32: rows * d * 4 (fp32).
 * MOE_BF16: rows * MOE_YQ_ROW_BYTES(d), a block fixed point: each row holds d
 * int16 mantissas (2d bytes), then one int8 exponent per block of 8
 * consecutive features (d/8 bytes, padded to a multiple of 16). Feature c of
 * a row is mantissa[c] * 2^(exponent[c/8] - 14); a block whose largest
 * magnitude m has 2^e <= m < 2^(e+1) is stored with exponent e (-127 for a
 * block below the fp32 normal range), so each value is within 2^-15 m of
 * the fp32 accumulation (2^-14 m where a mantissa clamps at +-32767). 0 for
 * a bad dtype, rows < 0, d < 1, or d % 8 != 0 with MOE_BF16.
 */
#define MOE_YQ_ROW_BYTES(d) (2 * (size_t)(d) + ((((size_t)(d) / 8) + 15) & ~(size_t)15))
size_t moe_expert_output_bytes(int dtype, int rows, int d);

/*
 * Workspace bytes that call `op` needs for these sizes (dtype-independent
 * upper bound; d, h unused by some ops). Returns 0 for a bad op or size,
 * E > 512 included.
 */
size_t moe_workspace_size(int op, int T, int d, int h, int E, int k);

/*
 * Router: logits, softmax, top-k selection and gates   [Routing page, gate
 * equation and TopKRouter; Guide page 5.2 for gate_bias].
 *   logits[t,e] = sum_i x[t,i] * w_gate[e,i] (+ gate_bias[e]), fp32 accumulate
 *   topk_idx[t,j]: the k experts with the largest logits, in descending
 *                  order; equal logits go to the lower expert index (+0 and -0
 *                  compare equal)
 *   p[t,e]       = softmax over all E logits of token t
 *   topk_gate[t,j] = renorm ? p[t,idx_j] / sum_j' p[t,idx_j'] : p[t,idx_j]
 *   prob_sum[e]  = sum_t p[t,e]   (feeds f of the aux loss)
 * x [T][d] dtype; w_gate [E][d] dtype; gate_bias [E] fp32 or NULL;
 * logits_out [T][E] fp32 or NULL; topk_idx [T][k] int32; topk_gate [T][k]
 * fp32; prob_sum [E] fp32 or NULL. 1 <= k <= E <= 512, k <= 16, T >= 0.
 * With topk_idx, topk_gate and prob_sum all NULL only the logits are
 * computed (logits_out is then required; Expert Choice routes from them);
 * they are the same bits as in a full call.
 * Workspace: moe_workspace_size(MOE_OP_ROUTER, ...).
 */
int moe_router_topk(const void *x, int dtype, int T, int d, const void *w_gate,
                    const float *gate_bias, int E, int k, int renorm, float *logits_out,
                    int32_t *topk_idx, float *topk_gate, float *prob_sum, void *ws,
                    size_t ws_bytes, moe_stream_t stream);

/*
 * Permute: per-expert counting sort with capacity   [Trilemma page 3.3
 * (count tokens per expert, group them); Routing page capacity section].
 * The T*k assignments are taken in flat order f = t*k + j.
 *   counts[e]  = #{f : topk_idx[f] == e}   (before any drop)
 *   kept[e]    = capacity < 0 ? counts[e] : min(counts[e], capacity)
 *   offsets[e] = sum_{e'<e} kept[e'],  offsets[E] = R (rows kept)
 *   dest_row[f] = offsets[e] + rank of f among expert e's assignments in
 *                 ascending f, if that rank < kept[e]; otherwise -1 (dropped)
 *   sorted_token[dest_row[f]] = f / k   (entries R..T*k-1 are not written)
 * counts [E], offsets [E+1], dest_row [T*k], sorted_token [T*k]: int32.
 * Indices outside [0, E) are outside the contract. E <= 512.
 * Workspace: moe_workspace_size(MOE_OP_PERMUTE, ...).
 */
int moe_permute(const int32_t *topk_idx, int T, int k, int E, int capacity, int32_t *counts,
                int32_t *offsets, int32_t *dest_row, int32_t *sorted_token, void *ws,
                size_t ws_bytes, moe_stream_t stream);

/*
 * moe_permute without a workspace, for callers that cannot allocate (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): same arguments and outputs as moe_permute. Its per-chunk
 * histograms live in a static device array of the library (4 MiB on each GPU
 * it runs on, held until the process ends), so T*k may be at most
 * MOE_PERMUTE_NOALLOC_MAX_ASSIGN (status MOE_ERR_UNSUPPORTED beyond). Every
 * call on one GPU uses that GPU's one array: calls that overlap on one GPU
 * (two streams, or two host threads) race and must be ordered by the caller.
 * The first call on a device looks up the array's address there (no
 * allocation); nothing in the array needs clearing between calls.
 */
#define MOE_PERMUTE_NOALLOC_MAX_ASSIGN (1L << 20)
int moe_permute_noalloc(const int32_t *topk_idx, int T, int k, int E, int capacity,
                        int32_t *counts, int32_t *offsets, int32_t *dest_row,
                        int32_t *sorted_token, moe_stream_t stream);

/*
 * Grouped expert FFN over the permuted rows   [Routing page, Expert;
 * Trilemma page 3.3, one grouped FFN per expert]:
 *   for each expert e and row r in [offsets[e], offsets[e+1]):
 *     H[r]      = SiLU(W1[e] . x[sorted_token[r]] + b1[e]),  SiLU(z) = z/(1+e^-z)
 *     y_perm[r] = W2[e] . H[r] + b2[e]
 * x [T][d]; w1 [E][h][d]; b1 [E][h] or NULL; w2 [E][d][h]; b2 [E][d] or
 * NULL; y_perm: T*k rows of moe_expert_output_bytes(dtype, 1, d) bytes (rows
 * 0..R-1 written, R = offsets[E] read on the device). fp32 accumulation;
 * with MOE_BF16, H is rounded to bf16 (the second product's operand) and
 * y_perm holds the accumulation in block fixed point (within 2^-15 of the
 * largest of every 8 consecutive features; see moe_expert_output_bytes),
 * far finer than a bf16 rounding of each value. offsets and sorted_token come from moe_permute with the same T, k, E,
 * or from moe_expert_choice with k = ceil(E * min(C, T) / T) (any k with
 * R <= T*k). The kernel choice depends only on T*k (no device-to-host read).
 * bf16 needs d and h to be multiples of 64. Workspace holds H:
 * moe_workspace_size(MOE_OP_FFN, ...).
 */
int moe_grouped_ffn(const void *x, int dtype, int T, int d, int h, int E, int k,
                    const int32_t *offsets, const int32_t *sorted_token, const void *w1,
                    const void *b1, const void *w2, const void *b2, void *y_perm, void *ws,
                    size_t ws_bytes, moe_stream_t stream);

/*
 * Combine: gate-weighted sum of each token's expert outputs   [Routing page,
 * output equation and MoELayer accumulation; capacity section for the
 * residual pass-through of dropped tokens]:
 *   out[t] = (residual ? residual[t] : 0)
 *            + sum_{j=0..k-1, dest_row[t,j] >= 0} topk_gate[t,j] * y_perm[dest_row[t,j]]
 * summed in fp32 in ascending j, then stored as out_dtype. A token with every
 * slot dropped gets residual[t] (or 0). y_perm: T*k rows as moe_grouped_ffn
 * writes them (fp32, or block fixed point for MOE_BF16, decoded exactly);
 * residual [T][d] (or NULL) is `dtype`; dest_row [T][k]; topk_gate [T][k] fp32; out [T][d]
 * is `out_dtype`: MOE_F32 (always allowed; keeps the fp32 sum unrounded) or
 * MOE_BF16 (only with dtype MOE_BF16). 1 <= k <= 512: with the slots of
 * moe_expert_choice (k = E) a token sums its choosing experts in ascending
 * expert order.
 */
int moe_combine(const void *y_perm, int dtype, const int32_t *dest_row, const float *topk_gate,
                int T, int k, int d, const void *residual, void *out, int out_dtype,
                moe_stream_t stream);

/*
 * Expert Choice routing   [Routing page, "Expert Choice路由策略与容量因子调优":
 * experts choose tokens, each expert takes the same number of them,
 * capacity = tokens / E * capacity_factor, tokens no expert takes keep only
 * the residual]:
 *   scores[e][t] = softmax over e' of logits[t][e']   (fp32, written)
 *   expert e takes the Cc = min(C, T) tokens with the largest scores[e][t]
 *   (ties: lower t), in ascending token order as rows [e*Cc, (e+1)*Cc):
 *     offsets[e] = e*Cc,  sorted_token[e*Cc + i] = i-th chosen token,
 *     dest_row[t][e] = its row or -1,  gate[t][e] = scores[e][t] or 0.
 * logits [T][E] fp32 (e.g. moe_router_topk's logits_out); scores [E][T]
 * fp32; offsets [E+1]; sorted_token [E*Cc]; dest_row [T][E] int32; gate
 * [T][E] fp32. The outputs feed moe_grouped_ffn (k = ceil(E*Cc/T)) and
 * moe_combine (k = E). C >= 0 is the caller's capacity (the page's
 * tokens/E*factor, rounded by the caller). Status 1 for negative sizes or
 * missing buffers, 2 for E > 512 or T*E >= 2^31. No workspace.
 */
int moe_expert_choice(const float *logits, int T, int E, int C, float *scores, int32_t *offsets,
                      int32_t *sorted_token, int32_t *dest_row, float *gate,
                      moe_stream_t stream);

/*
 * Host-resident experts streamed on demand   [Trilemma page 3.1: an expert
 * container holding metadata and an LRU of loaded experts, an expert loaded
 * when routing selects it; 3.2: routing returns indices, the executor loads
 * the active experts, then runs the grouped FFN; Guide page 5.3: hot experts
 * resident, cold ones fetched into an LRU cache]. The experts' weights live
 * in host memory (pinned by the caller, so copies are asynchronous); S
 * device slots hold the loaded ones.
 *
 * moe_cache_state_bytes(E, S): size of the caller-owned host state block
 *   (0 for E < 1, S < 1 or E > 512). moe_cache_init(state, E, S): all slots
 *   empty.
 * moe_cache_step(state, counts, ntensors, host_base, dev_base,
 *                bytes_per_expert, slot_of_dev, phase_of_dev, n_loaded,
 *                compute_stream, copy_stream):
 *   counts [E] (host, e.g. moe_permute's counts read back): experts with
 *   count > 0 are needed. A needed expert already in a slot is a hit (phase
 *   0); a needed one that is not takes the least recently used slot this
 *   step does not need (phase 1) and, for each of the ntensors tensors, its
 *   bytes_per_expert[i] bytes at host_base[i] + e*bytes are copied to
 *   dev_base[i] + slot*bytes on copy_stream. phase -1: not needed. The slot
 *   table [E] and the phases [E] are then copied to slot_of_dev /
 *   phase_of_dev (device, may be NULL) on compute_stream; *n_loaded (may be
 *   NULL) gets the number of experts copied. Status 2 if one step needs more
 *   experts than slots. The state must not change while an earlier step's
 *   table copy is pending (a synchronising read of the next counts on the
 *   compute stream guarantees it).
 * moe_cache_slot_of(state, slot_of, phase_of): host copies of the tables.
 */
size_t moe_cache_state_bytes(int E, int S);
int moe_cache_init(void *state, int E, int S);
int moe_cache_step(void *state, const int32_t *counts, int ntensors, const void *const *host_base,
                   void *const *dev_base, const size_t *bytes_per_expert, int32_t *slot_of_dev,
                   int32_t *phase_of_dev, int *n_loaded, moe_stream_t compute_stream,
                   moe_stream_t copy_stream);
int moe_cache_slot_of(const void *state, int32_t *slot_of, int32_t *phase_of);

/*
 * Grouped expert FFN over cached experts   [as moe_grouped_ffn; Trilemma
 * page 3.2 for running the loaded experts]: the same computation, with
 * expert e's weights at slot slot_of[e] of w1 [S][h][d], b1 [S][h], w2
 * [S][d][h], b2 [S][d], and only the experts with phase_of[e] == phase
 * computed (run phase 0 while the misses are copied, then phase 1 after
 * the copy stream's work). bf16 only, decode-size batches (T*k <= 4*E and
 * <= 1024, the weight-streaming path): status 2 otherwise. Same workspace
 * as moe_grouped_ffn; y_perm as there.
 */
int moe_grouped_ffn_cached(const void *x, int dtype, int T, int d, int h, int E, int k,
                           const int32_t *offsets, const int32_t *sorted_token,
                           const int32_t *slot_of, const int32_t *phase_of, int phase,
                           const void *w1, const void *b1, const void *w2, const void *b2,
                           void *y_perm, void *ws, size_t ws_bytes, moe_stream_t stream);

/*
 * Load-balancing auxiliary loss   [Routing page, load_balancing_loss]:
 *   f[e] = prob_sum[e] / T,  P[e] = counts[e] / T,  loss = E * sum_e f[e]*P[e]
 * counts are before capacity drops, so sum_e P[e] = k. prob_sum [E] fp32,
 * counts [E] int32; f [E], P [E], loss [1] fp32 (any may be NULL except
 * loss). T >= 1, E <= 512.
 */
int moe_aux_loss(const float *prob_sum, const int32_t *counts, int T, int E, float *f, float *P,
                 float *loss, moe_stream_t stream);

/* ===================================================================== *
 * Backward pass of the layer: gradients of                               *
 *   L = sum_t <dout[t], out[t]> + daux * aux_loss                        *
 * through the forward above [Routing page: gate equation, output         *
 * equation, Expert, MoELayer, load_balancing_loss; Sparse-inference page *
 * 2.3: the router is trained jointly and its kept logits pass the        *
 * softmax so gradients reach them]. Top-k selection, counts and capacity *
 * drops carry no gradient; the gradient reaches the gate values, the     *
 * router probabilities of the aux loss and every product. Call order:    *
 * (forward with moe_grouped_ffn_train), moe_combine_backward ->          *
 * moe_router_backward -> moe_grouped_ffn_backward ->                      *
 * moe_gather_backward and moe_router_weight_backward. Same               *
 * conventions as the forward: device pointers, caller-owned buffers,     *
 * asynchronous on `stream`, status codes as above.                        *
 * ===================================================================== */

/*
 * Combine backward: for every kept slot (t, j) (r = dest_row[t*k+j] >= 0)
 *   dy_perm[r] = topk_gate[t,j] * dout[t]          (dtype, [T*k][d] rows)
 *   dgate[t,j] = sum_i dout[t,i] * y_perm[r,i]     (fp32, fixed-order sum)
 * and dgate = 0 for dropped slots. y_perm: the forward's expert outputs, T*k
 * rows as moe_grouped_ffn writes them (MOE_BF16 needs d % 8 == 0); dout
 * [T][d] is `dtype`.
 * k <= 512 (Expert Choice layouts included).
 */
int moe_combine_backward(const void *y_perm, int dtype, const int32_t *dest_row,
                         const float *topk_gate, int T, int k, int d, const void *dout,
                         void *dy_perm, float *dgate, moe_stream_t stream);

/*
 * Router backward to the logits (fp32 [T][E]):
 *   renorm = 1: dlogits[t, S_j] += g_j (dgate_j - sum_i g_i dgate_i)
 *   renorm = 0: dp[t, S_j] += dgate_j
 *   aux (daux != 0): dp[t, e] += daux * E * counts[e] / T^2
 *   dlogits[t] += p (dp - <p, dp>),  p = softmax(logits[t]) recomputed.
 * logits, topk_idx, topk_gate: the forward router's outputs; counts: the
 * permute's pre-drop counts (read only when daux != 0). E <= 512.
 * Expert Choice (moe_expert_choice's gate [T][E] as topk_gate, k = E,
 * renorm = 0, daux = 0): topk_idx = NULL means slot j is expert j, and the
 * gate of a chosen pair is its probability, so the same rule applies.
 */
int moe_router_backward(const float *logits, const int32_t *topk_idx, const float *topk_gate,
                        const float *dgate, const int32_t *counts, int T, int E, int k,
                        int renorm, float daux, float *dlogits, moe_stream_t stream);

/*
 * Grouped expert FFN forward for training   [as moe_grouped_ffn]: the same
 * computation and outputs, and also keeps, for every kept row r, the
 * pre-activation z_perm[r] = W1[e] x[sorted_token[r]] + b1[e] and the hidden
 * row h_perm[r] = SiLU(z) (both [T*k][h] in the layer dtype, rows [0, R)
 * written) for moe_grouped_ffn_backward. h_perm holds exactly the hidden
 * rows the second product reads, so y_perm equals moe_grouped_ffn's bit for
 * bit. Same workspace as moe_grouped_ffn.
 */
int moe_grouped_ffn_train(const void *x, int dtype, int T, int d, int h, int E, int k,
                          const int32_t *offsets, const int32_t *sorted_token, const void *w1,
                          const void *b1, const void *w2, const void *b2, void *y_perm,
                          void *z_perm, void *h_perm, void *ws, size_t ws_bytes,
                          moe_stream_t stream);

/*
 * Grouped expert FFN backward over the permutation of the forward
 * (offsets, sorted_token from moe_permute), for each expert e and its rows:
 *   Z = W1[e] x[sorted_token] + b1[e]          (z_perm and H = h_perm from
 *                                              moe_grouped_ffn_train, or,
 *                                              both NULL, recomputed)
 *   dZ = (dy_perm W2[e]) * SiLU'(Z)
 *   dx_perm = dZ W1[e]                         ([T*k][d], rows [0, R))
 *   dw1[e] = dZ^T X_e,  db1[e] = sum of dZ rows        (dw1 [E][h][d])
 *   dw2[e] = dy_perm^T H,  db2[e] = sum of dy rows       (dw2 [E][d][h])
 * Weight and bias gradients are overwritten (zero for experts without
 * rows); db1 / db2 may be NULL (no bias). Gradients have the layer dtype;
 * products accumulate in fp32. bf16: d and h multiples of 256 (status 2
 * otherwise). Workspace: moe_workspace_size(MOE_OP_FFN_BWD, ...), which
 * holds the work lists, Z and dZ, split-K partials and the gathered input
 * rows; every operand is read in place (K-major ones through LDS
 * transpose loads).
 */
int moe_grouped_ffn_backward(const void *x, int dtype, int T, int d, int h, int E, int k,
                             const int32_t *offsets, const int32_t *sorted_token, const void *w1,
                             const void *b1, const void *w2, const void *dy_perm,
                             const void *z_perm, const void *h_perm, void *dx_perm, void *dw1,
                             void *db1, void *dw2, void *db2, void *ws, size_t ws_bytes,
                             moe_stream_t stream);

/*
 * Input gradient:
 *   dx[t] = sum_e dlogits[t,e] w_gate[e]        (if dlogits)
 *         + dout_residual[t]                    (if not NULL: residual layers)
 *         + sum_j dx_perm[dest_row[t*k+j]]      (kept slots, j ascending)
 * summed in fp32 in that order, stored in dtype. k, E <= 512. The router
 * term: bf16 layers with d % 128 == 0 compute it on the matrix cores from
 * dlogits split into two bf16 parts (hi = bf16(v), lo = bf16(v - hi), 16
 * significant bits) with fp32 accumulation; otherwise fp32 FMA, e
 * ascending.
 */
int moe_gather_backward(const void *dx_perm, int dtype, const int32_t *dest_row, int T, int k,
                        int d, const void *dout_residual, const float *dlogits,
                        const void *w_gate, int E, void *dx, moe_stream_t stream);

/*
 * Router weight gradients:
 *   dw_gate[e][i] = sum_t dlogits[t,e] x[t,i]   (dtype [E][d])
 *   dgate_bias[e] = sum_t dlogits[t,e]          (fp32 [E], may be NULL)
 * Sums run over fixed token ranges (their number depends only on T, d, E)
 * in a fixed order. bf16 layers with d % 128 == 0 form dw_gate on the
 * matrix cores with dlogits split into two bf16 parts as in
 * moe_gather_backward; otherwise fp32 FMA. Workspace:
 * moe_workspace_size(MOE_OP_ROUTER_BWD, ...).
 */
int moe_router_weight_backward(const void *x, int dtype, int T, int d, int E,
                               const float *dlogits, void *dw_gate, float *dgate_bias, void *ws,
                               size_t ws_bytes, moe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
