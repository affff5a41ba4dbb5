/*
 * moe.h -- C ABI of the MI355X (gfx950) mixture-of-experts layer library.
 *
 * The library computes one MoE layer, forward and backward, on one GPU:
 *
 *     y_t = s(x_t) + sum_{j<k} g[t,j] * FFN_{idx[t,j]}(x_t)
 *     FFN_e(z) = (silu(z W_g[e]^T) * (z W_u[e]^T)) W_d[e]^T        (SwiGLU, no bias)
 *
 * where a router picks k of E experts per token from fp32 logits x W_r^T,
 * the picked experts' outputs are weighted by the gates and summed, and the
 * optional shared experts s(.) run on every token, ungated.
 *
 * Sources of the definition (the web pages this library follows):
 *  - The Ultimate MoE Training Handbook (Hugging Face), section 1
 *    "Introduction" (the three new concerns of a MoE layer: router, load
 *    balancing, token exchange) and section 2.5 "First training of MoE"
 *    (router picks 8 of 64 experts; tokens are sent to the selected experts
 *    and the outputs returned; experts are SwiGLU without bias; router logits
 *    in fp32; grouped GEMM for the local experts).
 *  - Apex-3 code page, "What's inside", row "Fine-grained MoE" (sigmoid
 *    router, per-expert bias that balances load and only steers selection,
 *    experts as grouped GEMMs).
 *  - KempnerForge README, "Features / Architecture" (softmax top-k and
 *    DeepSeek-V3 sigmoid routers, shared experts, fine-grained experts).
 *  - "Train Large Model from Scratch" README, "Configuration / Model
 *    Configuration" (num_experts, num_experts_per_tok, moe_intermediate_size).
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers to row-major, contiguous data,
 *    16-byte aligned (else MOE_ERR_ALIGN).  The caller owns every buffer;
 *    the compute calls allocate no memory, free nothing and keep no state
 *    between calls.  Workspaces are caller-provided, sized by the query
 *    functions.  The one stateful part is the per-stage timing aid
 *    (moe_stage_timing below): while enabled it creates HIP events and keeps
 *    process-wide records of them.
 *  - bf16 means IEEE bfloat16 bit patterns (uint16 storage).
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *    default stream).  No call synchronises or copies device->host: counts
 *    and offsets stay on the device.
 *  - Arguments are validated on the host before anything is launched; an
 *    invalid call returns a non-zero status and launches nothing.  Launch
 *    failures return MOE_ERR_HIP.  Nothing aborts or throws across the ABI.
 *  - Results are bitwise deterministic for fixed inputs (no float atomics).
 *  - Every output element is written (empty experts get zero weight grads).
 *  - Apart from the timing aid, the library is stateless; concurrent calls on
 *    different streams with disjoint outputs are safe.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 4

/* ---------------------------------------------------------------- status */
enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = 1,      /* bad shape, null required pointer, bad enum   */
  MOE_ERR_ALIGN = 2,        /* a pointer is not 16-byte aligned              */
  MOE_ERR_UNSUPPORTED = 3,  /* valid request this build does not implement   */
  MOE_ERR_WORKSPACE = 4,    /* workspace smaller than the query's answer     */
  MOE_ERR_HIP = 5           /* the HIP runtime reported an error             */
};

/* element type of activations, expert weights and their gradients */
enum { MOE_F32 = 0, MOE_BF16 = 1 };

/* router score function (KempnerForge README, "Features / Architecture") */
enum {
  MOE_SOFTMAX = 0,  /* p = softmax(l) over experts; selection by l; gate = p
                       (or p / sum of picked p when renorm != 0)            */
  MOE_SIGMOID = 1   /* s = sigmoid(l); selection by fp32(s + bias); gate =
                       s / sum of picked s (bias never enters the gate)     */
};

/* Layer description.  Limits: 1 <= E <= 256, 1 <= k <= min(E, 16);
 * d_model, d_ff and d_ff_shared multiples of 64; T >= 0 (T = 0 is a no-op). */
typedef struct moe_desc {
  int64_t num_tokens;   /* T                                              */
  int64_t d_model;      /* d                                              */
  int64_t num_experts;  /* E (routed experts)                             */
  int64_t top_k;        /* k (experts per token)                          */
  int64_t d_ff;         /* f, hidden width of one routed expert           */
  int64_t num_shared;   /* number of shared experts (0 = none)            */
  int64_t d_ff_shared;  /* hidden width of one shared expert              */
  int32_t score;        /* MOE_SOFTMAX or MOE_SIGMOID                     */
  int32_t renorm;       /* softmax only: renormalise picked probabilities */
  int32_t dtype;        /* MOE_F32 or MOE_BF16                            */
  int32_t reserved;     /* must be 0                                      */
} moe_desc_t;

/* Parameters.  F = num_shared * d_ff_shared: the shared experts are stored
 * concatenated along their hidden width, which is the same function as their
 * sum.  Router weight and bias are always fp32 (Handbook 2.5: fp32 router). */
typedef struct moe_weights {
  const float *w_router;  /* [E, d] fp32                                      */
  const float *bias;      /* [E] fp32, sigmoid selection only; NULL = zero    */
  const void *w_gateup;   /* [E, 2f, d]: rows 0..f-1 gate W_g, f..2f-1 up W_u */
  const void *w_down;     /* [E, d, f]                                        */
  const void *s_gateup;   /* [2F, d] (gate rows, then up rows); NULL if F = 0 */
  const void *s_down;     /* [d, F]; NULL if F = 0                            */
} moe_weights_t;

/* Forward intermediates kept for the backward pass (A = T*k rows).
 * Caller-allocated; moe_forward fills them, moe_backward reads them. */
typedef struct moe_saved {
  float *logits;     /* [T, E] fp32 router logits                             */
  int32_t *idx;      /* [T, k] picked experts, slot j = j-th best             */
  float *gate;       /* [T, k] fp32 gates                                     */
  int32_t *counts;   /* [E] rows per expert                                   */
  int32_t *offsets;  /* [E+1] exclusive prefix of counts                      */
  int32_t *pos;      /* [A] permuted row of assignment a = t*k + j            */
  int32_t *src;      /* [A] assignment held by permuted row p (inverse of pos) */
  int32_t *tok;      /* [A] token of permuted row p (src[p] / k)              */
  void *x_perm;      /* [A, d] token rows in expert-contiguous order, or NULL:
                        then the routed gate/up products (forward and weight
                        gradient) read the rows of x through tok, and no
                        permuted copy is written (bf16 layers with d a multiple
                        of 256, d_ff of 128 and T*d <= 2^31; else
                        MOE_ERR_UNSUPPORTED)                                  */
  void *preact;      /* [A, 2f] gate|up pre-activations; may be NULL in an
                        inference-only forward (then backward is invalid)     */
  void *h;           /* [A, f] silu(G) * U                                    */
  void *y_perm;      /* [A, d] expert outputs, permuted order                 */
  void *s_preact;    /* [T, 2F] shared pre-activations, or NULL if F = 0      */
  void *s_h;         /* [T, F] shared hidden, or NULL if F = 0                */
} moe_saved_t;

/* Gradients written by moe_backward (overwritten, not accumulated). */
typedef struct moe_grads {
  float *d_w_router;  /* [E, d] fp32                      */
  void *d_w_gateup;   /* [E, 2f, d]                       */
  void *d_w_down;     /* [E, d, f]                        */
  void *d_s_gateup;   /* [2F, d], NULL if F = 0           */
  void *d_s_down;     /* [d, F], NULL if F = 0            */
} moe_grads_t;

/* Router training terms added by moe_backward (each 0 = off).  With q[t,e]
 * the router's distribution over the E experts (softmax probabilities, or the
 * sigmoid scores normalised to sum 1):
 *   aux     = aux_coeff * E * sum_e f_e P_e,  f_e = counts_e / (T k),
 *             P_e = mean over tokens of q[t,e]          (Handbook 2.5, the
 *             auxiliary balance loss with coefficient 1e-3)
 *   seq_aux = seq_aux_coeff * mean over sequences s of sum_e f^s_e P^s_e,
 *             f^s_e = E/(k S) * #(tokens of s picking e), P^s_e = mean over
 *             s of q[t,e]                                (Apex-3 "Run it
 *             yourself", seq_aux_alpha; KempnerForge "MoE roadmap")
 *   z       = z_coeff * mean over tokens of logsumexp(l_t)^2 (KempnerForge
 *             "Features": router z-loss)
 * The load shares f carry no gradient; the gradients reach the logits
 * through q (and the softmax for z).  seq_len must divide T (0: the whole
 * batch is one sequence); coefficients must be finite and >= 0. */
typedef struct {
  float aux_coeff;
  float seq_aux_coeff;
  float z_coeff;
  int32_t seq_len;
} moe_router_terms_t;

/* grouped GEMM layouts and epilogues (see moe_grouped_gemm) */
enum { MOE_GEMM_NT = 0, MOE_GEMM_NN = 1, MOE_GEMM_TN = 2 };
enum { MOE_EPI_NONE = 0, MOE_EPI_SWIGLU = 1, MOE_EPI_DSWIGLU = 2 };

/* workspace kinds for moe_workspace_bytes */
enum {
  MOE_WS_PERMUTE = 0,
  MOE_WS_FORWARD = 1,
  MOE_WS_BACKWARD = 2,
  MOE_WS_FORWARD_FP8 = 3,        /* moe_forward_fp8                         */
  MOE_WS_BACKWARD_FP8 = 4,       /* moe_backward_fp8, bf16 weight gradients */
  MOE_WS_BACKWARD_FP8_WGRAD = 5  /* moe_backward_fp8 with fp8 weight gradients */
};

/* ---------------------------------------------------------------- queries */

/* Human-readable name of a status code (static string, never NULL). */
const char *moe_status_str(int status);

/* MOE_ABI_VERSION of the built library. */
int moe_abi_version(void);

/* Number of int32 elements of the per-block expert histogram that moe_route
 * writes and moe_permute reads: E * ceil(T / MOE_ROUTE_BLOCK).  0 if desc is
 * invalid. */
size_t moe_route_hist_elems(const moe_desc_t *desc);

/* Bytes of device workspace the named call needs (0 if desc is invalid). */
size_t moe_workspace_bytes(const moe_desc_t *desc, int which);

/* The saved buffers of moe_forward (moe_saved_t) in one caller allocation.
 * flags: MOE_SAVED_TRAINING keeps the pre-activations the backward needs
 * (preact, s_preact); MOE_SAVED_PERMUTED_COPY keeps x_perm (else the
 * gate/up products gather the token rows through tok).
 *   moe_saved_bytes: bytes of that allocation (0 if desc or flags are invalid)
 *   moe_saved_carve: fills *saved with 256-byte aligned fields inside base
 *     (fields the flags leave out are NULL); base 256-byte aligned, bytes >=
 *     moe_saved_bytes(desc, flags); no device access. */
enum { MOE_SAVED_TRAINING = 1, MOE_SAVED_PERMUTED_COPY = 2 };
size_t moe_saved_bytes(const moe_desc_t *desc, int flags);
int moe_saved_carve(const moe_desc_t *desc, int flags, void *base, size_t bytes, moe_saved_t *saved);

/* Bytes of device workspace moe_grouped_gemm needs for this problem. */
size_t moe_grouped_gemm_workspace_bytes(int layout, int dtype, int64_t G, int64_t M_total,
                                        int64_t N, int64_t K);

/* ---------------------------------------------------------------- calls */

/* Router: scores, top-k selection and gates from fp32 logits.
 * (Apex-3 "Fine-grained MoE"; KempnerForge "Features / Architecture".)
 *   logits     [T, E] fp32 (in)
 *   bias       [E] fp32 or NULL (sigmoid only; ignored for softmax)
 *   idx        [T, k] int32 (out): experts by key descending, ties to the
 *              lower expert index.  Softmax key: the logit.  Sigmoid key:
 *              fp32(s + bias) with s = sigmoid(l) evaluated in fp64 and
 *              rounded once to fp32.
 *   gate       [T, k] fp32 (out)
 *   block_hist [moe_route_hist_elems] int32 (out): per block of
 *              MOE_ROUTE_BLOCK tokens, how many of its assignments went to
 *              each expert (layout [E][blocks]); consumed by moe_permute. */
int moe_route(const moe_desc_t *desc, const float *logits, const float *bias, int32_t *idx,
              float *gate, int32_t *block_hist, void *stream);

/* Token permutation into expert-contiguous order ("tokens must be sent to the
 * selected experts", Handbook 2.5): histogram (from moe_route), prefix scan
 * over experts and blocks, stable scatter.
 *   x       [T, d] (in, desc dtype);  idx [T, k], block_hist (in)
 *   counts  [E], offsets [E+1] (out): offsets[E] = T*k
 *   pos     [T*k] (out): row of assignment a = t*k + j; rows of one expert
 *           are ordered by increasing a (stable)
 *   src     [T*k] (out): src[pos[a]] = a
 *   tok     [T*k] (out) or NULL: tok[p] = src[p] / k, the token of row p
 *   x_perm  [T*k, d] (out): x_perm[pos[t*k+j]] = x[t]; or NULL (no copy)
 *   ws      >= moe_workspace_bytes(desc, MOE_WS_PERMUTE) bytes of scratch */
int moe_permute(const moe_desc_t *desc, const void *x, const int32_t *idx,
                const int32_t *block_hist, int32_t *counts, int32_t *offsets, int32_t *pos,
                int32_t *src, int32_t *tok, void *x_perm, void *ws, size_t ws_bytes,
                void *stream);

/* Grouped GEMM over G groups of rows ("experts run as grouped GEMMs", Apex-3
 * "Fine-grained MoE"; Handbook 2.5 grouped GEMM for the local experts).
 * group_offsets: device int32 [G+1], non-decreasing, offsets[0] = 0,
 * offsets[G] = M_total; group g owns rows [offsets[g], offsets[g+1]).  With
 * G = 1 it may be NULL: one group of all M_total rows.
 * Accumulation is fp32; C is rounded once to `dtype`.
 *   MOE_GEMM_NT (forward):  C[m,n] = sum_k A[m,k] B[g,n,k]
 *        A [M_total,K], B [G,N,K], C [M_total,N]
 *        MOE_EPI_SWIGLU: N = 2F, B rows 0..F-1 are gate, F..2F-1 up;
 *        C [M_total,F] = silu(gate) * up; aux [M_total,2F] receives the
 *        pre-activations gate|up (aux may be NULL).
 *   MOE_GEMM_NN (data gradient): C[m,k] = sum_n A[m,n] B[g,n,k]
 *        A [M_total,N], B [G,N,K], C [M_total,K]
 *        MOE_EPI_DSWIGLU: the product is dH [M_total,K]; aux [M_total,2K]
 *        holds the forward pre-activations G|U; C [M_total,2K] receives
 *        dG = dH*U*silu'(G) | dU = dH*silu(G).
 *   MOE_GEMM_TN (weight gradient): C[g,n,k] = sum_{m in g} A[m,n] B[m,k]
 *        A [M_total,N], B [M_total,K], C [G,N,K]; empty groups give zeros.
 * N and K multiples of 64.  ws >= moe_grouped_gemm_workspace_bytes(...). */
int moe_grouped_gemm(int layout, int epilogue, int dtype, int64_t G, int64_t M_total, int64_t N,
                     int64_t K, const int32_t *group_offsets, const void *A, const void *B, void *C,
                     void *aux, void *ws, size_t ws_bytes, void *stream);

/* The grouped GEMM of moe_grouped_gemm with the routed rows gathered from
 * the un-permuted token matrix (gather-on-load: the permuted copy of the
 * tokens is never materialised).  bf16 only, no workspace.
 *   MOE_GEMM_NT (MOE_EPI_NONE or MOE_EPI_SWIGLU): A is the token matrix
 *        [src_rows, K]; routed row m reads A[rows[m]].
 *   MOE_GEMM_TN (MOE_EPI_NONE): B is the token matrix [src_rows, K];
 *        routed row m of the reduction reads B[rows[m]].
 *   rows [M_total] int32 (device), each in [0, src_rows) (not checked on the
 *        device: the caller's contract; moe_permute's tok satisfies it).
 * Shapes as for moe_grouped_gemm, and: NT SwiGLU needs N/2 a multiple of 128;
 * TN needs K a multiple of 256; src_rows * K * 2 <= 2^32; 1 <= G <= 256.
 * Otherwise MOE_ERR_UNSUPPORTED. */
int moe_grouped_gemm_gather(int layout, int epilogue, int64_t G, int64_t M_total, int64_t N,
                            int64_t K, const int32_t *group_offsets, const void *A, const void *B,
                            void *C, void *aux, const int32_t *rows, int64_t src_rows,
                            void *stream);

/* Weighted combine / unpermute ("the experts' output must be returned",
 * Handbook 2.5):  y[t] = sum_{j<k} gate[t,j] * y_perm[pos[t*k+j]] (+ shared_y[t])
 * accumulated in fp32 in slot order, shared last, rounded once.
 *   y_perm [T*k, d], gate [T, k] fp32, pos [T*k], shared_y [T, d] or NULL,
 *   y [T, d] (out; may alias shared_y). */
int moe_combine(const moe_desc_t *desc, const void *y_perm, const float *gate,
                const int32_t *pos, const void *shared_y, void *y, void *stream);

/* Whole forward pass: router GEMM (fp32) -> route -> permute -> gate/up
 * grouped GEMM with SwiGLU -> down grouped GEMM -> shared experts -> combine.
 * This is the layer as the Handbook lays it out: section 1 "Introduction"
 * (a router picks experts per token, the load is balanced, tokens travel to
 * their experts) and section 2.5 "First training of MoE" (the selected
 * experts' outputs come back and are summed by gate weight; fp32 router;
 * grouped GEMM over the local experts); shared experts as in KempnerForge
 * "Features / Architecture", added ungated on every token.
 *   x [T, d] (in), y [T, d] (out), saved (out, all buffers caller-allocated)
 *   ws >= moe_workspace_bytes(desc, MOE_WS_FORWARD) */
int moe_forward(const moe_desc_t *desc, const moe_weights_t *w, const void *x, void *y,
                const moe_saved_t *saved, void *ws, size_t ws_bytes, void *stream);

/* moe_forward for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments and results as moe_forward (bit for
 * bit: the same kernels) without ws; its scratch (the routing histogram and
 * its scan) lives in a device array of
 * MOE_STATIC_SCRATCH_BYTES inside the library, one copy per GPU, held until
 * the process ends.  Allocates nothing and calls no allocating routine.
 *   MOE_ERR_WORKSPACE when the layer needs more scratch than that
 *   (moe_workspace_bytes(desc, MOE_WS_FORWARD) > MOE_STATIC_SCRATCH_BYTES,
 *   which is about E * ceil(T / 32) > 2^20 with E experts and T tokens).
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (different streams, or different host threads) race and must
 * not be issued; calls in one stream are ordered and safe.  The stream must
 * belong to the current device. */
#define MOE_STATIC_SCRATCH_BYTES (8u << 20)
int moe_forward_no_workspace(const moe_desc_t *desc, const moe_weights_t *w, const void *x, void *y,
                             const moe_saved_t *saved, void *stream);

/* Whole backward pass for upstream gradient dy [T, d]: combine backward
 * (gate gradient), router backward (through the gates only; the bias gets no
 * gradient), down and gate/up data and weight gradients, shared experts,
 * unpermute-sum of the input gradient.  It is the exact gradient of
 * moe_forward (the Handbook's section 2.5 layer, trained end to end there);
 * that the bias only steers selection and takes no gradient follows the
 * Apex-3 code page, "What's inside", row "Fine-grained MoE".
 *   x [T, d] (the forward input), saved (from moe_forward), dy [T, d] (in),
 *   dx [T, d] (out), grads (out)
 *   terms   NULL, or router training terms whose gradients are added to the
 *           router gradient (and so to d_w_router and dx)
 *   losses  NULL, or device float[3] receiving the aux, seq_aux and z values
 *           (requires terms)
 *   ws >= moe_workspace_bytes(desc, MOE_WS_BACKWARD) */
int moe_backward(const moe_desc_t *desc, const moe_weights_t *w, const void *x,
                 const moe_saved_t *saved, const void *dy, void *dx, const moe_grads_t *grads,
                 const moe_router_terms_t *terms, float *losses, void *ws, size_t ws_bytes,
                 void *stream);

/* Proportional load-balancing update of the sigmoid router's selection bias
 * after a step (Apex-3 code page: the per-expert bias balances the load
 * without a loss term; router_bias_update=proportional with router_bias_rate
 * 1e-3 in training and 0.01 in the benchmark):
 *   bias[e] += rate * (T k / E - counts[e]) / (T k / E)
 * evaluated in fp64 and rounded once to fp32.
 *   counts [E] int32 (device, from moe_forward), bias [E] fp32 (device, in/out)
 * MOE_ERR_INVALID for a non-finite rate or null pointers (T > 0). */
int moe_bias_update(const moe_desc_t *desc, const int32_t *counts, float rate, float *bias,
                    void *stream);

/* ---------------------------------------------------------------- fp8 experts */

/* fp8 formats (KempnerForge README, "Features": FP8 in E4M3 and E5M2): OCP
 * e4m3 (4 exponent bits, bias 7, largest finite 448, no infinities) and OCP
 * e5m2 (5 exponent bits, bias 15, largest finite 57344).  Row-wise scales are
 * amax / 448 resp. amax / 57344. */
enum { MOE_E4M3 = 0, MOE_E5M2 = 1 };

/* Row-wise fp8 quantisation (Apex-3 code page: FP8 through torchao,
 * --precision fp8_rowwise).  For each row r of x [rows, cols] (dtype bf16 or
 * fp32): s_r = amax_r / vmax in fp32 (1 for an all-zero row; vmax = 448 for
 * MOE_E4M3, 57344 for MOE_E5M2), and q[r, c] = fmt(x[r, c] / s_r), the
 * quotient in fp32, clamped to +-vmax and rounded to nearest even onto the
 * format's grid.
 *   q [rows, cols] uint8 codes (out), scale [rows] fp32 (out)
 * cols a multiple of 64; pointers 16-byte aligned. */
int moe_quantize_fp8(int64_t rows, int64_t cols, int dtype, int format, const void *x, uint8_t *q,
                     float *scale, void *stream);

/* Row-wise fp8 quantisation along the first axis of each matrix, stored
 * transposed (the weight of a data-gradient product, e.g. dX = dGU . W_gu
 * with W_gu[e] [2f, d], quantised along its reduction dimension 2f and laid
 * out [d, 2f] so that moe_grouped_gemm_fp8 runs the product in its forward
 * layout; Apex-3 code page, "What's inside": fp8 row-wise GEMMs):
 *   x [G, rows, cols] (MOE_F32 or MOE_BF16, in)
 *   scale [G, cols] fp32 (out): s[g, c] = max_r |x[g, r, c]| / 448 (1 for an
 *         all-zero column)
 *   q [G, cols, rows] uint8 e4m3 codes (out): q[g, c, r] = e4m3(x[g, r, c] / s[g, c])
 *         with the quotient an fp32 division clamped to +-448, round to
 *         nearest even
 * rows and cols multiples of 64 (rows <= 2^24, cols <= 2^22), 0 <= G <= 65535;
 * pointers 16-byte aligned.  Deterministic. */
int moe_quantize_fp8_transposed(int64_t G, int64_t rows, int64_t cols, int dtype, const void *x,
                                uint8_t *q, float *scale, void *stream);

/* Tensor-wise fp8 quantisation (the Apex-3 code page's "tensorwise" fp8
 * recipe): one scale s = amax / 448 over every element of x [rows, cols]
 * (fp32; 1 for an all-zero tensor), q[r, c] = e4m3(x[r, c] / s) as in
 * moe_quantize_fp8.  s is written to every entry of scale [rows], so that
 * moe_grouped_gemm_fp8 takes either scaling.
 *   ws >= moe_quantize_fp8_tensorwise_workspace_bytes(rows) bytes of device
 *   scratch (the row maxima and the scale)
 * cols a multiple of 64; pointers 16-byte aligned.  Deterministic. */
size_t moe_quantize_fp8_tensorwise_workspace_bytes(int64_t rows);
int moe_quantize_fp8_tensorwise(int64_t rows, int64_t cols, int dtype, const void *x, uint8_t *q,
                                float *scale, void *ws, size_t ws_bytes, void *stream);

/* fp8 grouped GEMM, forward (NT) layout, with row scales:
 *   C[m, n] = a_scale[m] * b_scale[g, n] * sum_k A[m, k] B[g, n, k]
 * with A's codes in a_format (MOE_E4M3, or MOE_E5M2 for the gradient operand
 * of a data gradient: MOE_EPI_NONE or MOE_EPI_DSWIGLU only, else
 * MOE_ERR_UNSUPPORTED) and B's in e4m3
 * for the rows m of group g (group_offsets as in moe_grouped_gemm, NULL for
 * one group), fp32
 * accumulation of the exact e4m3 products, rounded once to bf16.
 *   A [M_total, K], B [G, N, K] uint8 e4m3 codes; a_scale [M_total],
 *   b_scale [G, N] fp32; C [M_total, N] bf16 (MOE_EPI_NONE) or, with
 *   MOE_EPI_SWIGLU, C [M_total, N/2] = silu(gate) * up of the scaled
 *   products and aux [M_total, N] bf16 the scaled pre-activations (or NULL);
 *   with MOE_EPI_DSWIGLU the data gradient through SwiGLU: the scaled product
 *   is dH [M_total, N], aux [M_total, 2N] bf16 (in, required) holds the
 *   forward pre-activations G | U, and C [M_total, 2N] receives
 *   dG = dH U silu'(G) | dU = dH silu(G) (the down projection's data
 *   gradient with B the down weight from moe_quantize_fp8_transposed).
 * K a multiple of 64, N a multiple of 64 (SwiGLU: N/2 a multiple of 128),
 * 1 <= G <= 256; pointers 16-byte aligned. */
int moe_grouped_gemm_fp8(int epilogue, int a_format, int64_t G, int64_t M_total, int64_t N, int64_t K,
                         const int32_t *group_offsets, const uint8_t *A, const float *a_scale,
                         const uint8_t *B, const float *b_scale, void *C, void *aux, void *stream);

/* moe_grouped_gemm_fp8 (MOE_EPI_NONE or MOE_EPI_SWIGLU, e4m3 A) with the rows
 * of A gathered: routed row m reads the codes A[rows[m]] [src_rows, K] and the
 * scale a_scale[rows[m]] (a_scale [src_rows]), so that token rows quantised
 * once per token feed all k of their assignments.  rows [M_total] int32
 * (device), each in [0, src_rows) (not checked on the device: moe_permute's
 * tok satisfies it).  src_rows * K <= 2^32, else MOE_ERR_UNSUPPORTED. */
int moe_grouped_gemm_fp8_gather(int epilogue, int64_t G, int64_t M_total, int64_t N, int64_t K,
                                const int32_t *group_offsets, const uint8_t *A, const float *a_scale,
                                const uint8_t *B, const float *b_scale, void *C, void *aux,
                                const int32_t *rows, int64_t src_rows, void *stream);

/* fp8 weight-gradient operands: each column of x [M, C] (dtype bf16 or fp32)
 * quantised to e4m3 over the rows of each of G groups (group g owns rows
 * [offsets[g], offsets[g+1]); offsets NULL for one group of all M rows; with
 * rows, group row m reads x[rows[m]], rows[m] in [0, src_rows)):
 * scale[g, c] = max |x[., c]| over the group's rows / 448 (1 for none or all
 * zero), codes stored transposed and padded: with P'_g the group's row count
 * rounded up to 64 and P_g the sum of the earlier groups' P' (written to
 * pad_offsets [G+1]), code (m, c) of group g sits at q[C * P_g + c * P'_g + m],
 * zero for m past the group's rows.  This is row-wise quantisation along the
 * reduction dimension of a weight gradient, whose reduction runs over one
 * expert's tokens (Apex-3 code page, "Run it yourself": fp8_rowwise).
 *   q: moe_quantize_fp8_colwise_bytes(G, M, C) bytes (an upper bound), scale
 *   [G, C] fp32.  C a multiple of 64, 1 <= G <= 256. */
size_t moe_quantize_fp8_colwise_bytes(int64_t G, int64_t M, int64_t C);
int moe_quantize_fp8_colwise(int64_t G, int64_t M, int64_t C, int dtype, const int32_t *offsets,
                             const int32_t *rows, int64_t src_rows, const void *x, int32_t *pad_offsets,
                             uint8_t *q, float *scale, void *stream);

/* fp8 weight gradient over the blocks of moe_quantize_fp8_colwise:
 *   C[g, n, k] = a_scale[g, n] * b_scale[g, k] * sum_m A_g[n, m] B_g[k, m]
 * with A the codes of an [M, N] operand and B of an [M, K] operand quantised
 * with the same group offsets (pad_offsets from either call), fp32
 * accumulation of the exact e4m3 products, one rounding to bf16;
 * C [G, N, K] bf16 (groups without rows get zeros).  N, K multiples of 64. */
int moe_grouped_gemm_fp8_wgrad(int64_t G, int64_t N, int64_t K, const int32_t *pad_offsets, const uint8_t *A,
                               const float *a_scale, const uint8_t *B, const float *b_scale, void *C,
                               void *stream);

/* ---------------------------------------------------------------- fp8 layer */

/* e4m3 copies of the expert weights for the fp8 layer calls (Apex-3 code
 * page, "Run it yourself": the fp8_rowwise precision of the whole model;
 * KempnerForge README, "MoE roadmap": FP8 mixed precision).  Each copy is
 * quantised row-wise along the reduction dimension of the product it feeds
 * (codes as in moe_quantize_fp8), F = num_shared * d_ff_shared:
 *   forward layout (moe_forward_fp8), along d resp. f:
 *     gateup_q [E, 2f, d], gateup_s [E, 2f];  down_q [E, d, f], down_s [E, d]
 *     s_gateup_q [2F, d], s_gateup_s [2F];    s_down_q [d, F], s_down_s [d]
 *   data-gradient layout (moe_backward_fp8), along 2f resp. d, stored
 *   transposed as moe_quantize_fp8_transposed writes them:
 *     gateup_tq [E, d, 2f], gateup_ts [E, d]; down_tq [E, f, d], down_ts [E, f]
 *     s_gateup_tq [d, 2F], s_gateup_ts [d];   s_down_tq [F, d], s_down_ts [F]
 * Shared fields are NULL when F = 0.  Caller-owned device buffers. */
typedef struct moe_fp8_weights {
  uint8_t *gateup_q;    float *gateup_s;
  uint8_t *down_q;      float *down_s;
  uint8_t *gateup_tq;   float *gateup_ts;
  uint8_t *down_tq;     float *down_ts;
  uint8_t *s_gateup_q;  float *s_gateup_s;
  uint8_t *s_down_q;    float *s_down_s;
  uint8_t *s_gateup_tq; float *s_gateup_ts;
  uint8_t *s_down_tq;   float *s_down_ts;
} moe_fp8_weights_t;

/* which layouts moe_fp8_weights_quantize writes (a bit mask) */
enum { MOE_FP8_FORWARD_LAYOUT = 1, MOE_FP8_BACKWARD_LAYOUT = 2 };

/* Writes the e4m3 copies of the expert weights in w (bf16 layer) into the
 * buffers of w8: the forward layout (parts & MOE_FP8_FORWARD_LAYOUT), the
 * data-gradient layout (parts & MOE_FP8_BACKWARD_LAYOUT), or both.  Run once
 * per weight update; the fp8 layer calls read these copies and never the
 * bf16 weights' values for their expert products.  Deterministic.
 * MOE_ERR_UNSUPPORTED for layers moe_forward_fp8 does not take. */
int moe_fp8_weights_quantize(const moe_desc_t *desc, const moe_weights_t *w,
                             const moe_fp8_weights_t *w8, int parts, void *stream);

/* moe_forward with the expert products in e4m3 (the fp8_rowwise recipe named
 * above): the token rows x are quantised row-wise once per token and the
 * routed gate/up product gathers them through saved->tok (one scale per
 * token); H = silu(G) * U is stored in bf16 (saved->h) and that bf16 copy is
 * quantised row-wise for the down product; the shared experts likewise.  The
 * router (fp32), routing, permutation and combine are those of moe_forward,
 * and the saved buffers are the same (saved->preact holds the scaled fp8
 * pre-activations rounded to bf16).  Products accumulate the exact e4m3
 * products in fp32 and are rounded once to bf16.
 *   w    the layer's weights: the router (w_router, bias) is read; the expert
 *        fields may be NULL
 *   w8   forward-layout copies (moe_fp8_weights_quantize)
 *   ws  >= moe_workspace_bytes(desc, MOE_WS_FORWARD_FP8)
 * bf16 layers with d_ff and num_shared * d_ff_shared multiples of 128 and
 * T * d <= 2^32; else MOE_ERR_UNSUPPORTED.  saved->x_perm, when given, is
 * filled as in moe_forward (for a backward that reads it). */
int moe_forward_fp8(const moe_desc_t *desc, const moe_weights_t *w, const moe_fp8_weights_t *w8,
                    const void *x, void *y, const moe_saved_t *saved, void *ws, size_t ws_bytes,
                    void *stream);

/* moe_backward with the expert products in fp8: the gate-weighted
 * upstream rows dY~ (bf16) are quantised row-wise for dH = dY~ W_d (with the
 * SwiGLU derivative fused), dG | dU (bf16) row-wise for dX~ = (dG | dU) W_gu,
 * against the e4m3 data-gradient copies of w8; the shared experts likewise
 * (dy itself for their down product).  grad_format: MOE_E4M3, or MOE_E5M2
 * for these gradient operands (the weights stay e4m3).  With k <= 8 the
 * combine backward writes dY~'s and dy's codes as it forms the rows.
 * wgrad_fp8 = 1: the weight gradients are e4m3 products too, of dY~ and H
 * (down), dG | dU and the token rows (gate/up) quantised along each expert's
 * rows (moe_quantize_fp8_colwise, moe_grouped_gemm_fp8_wgrad); 0: bf16.  Weight gradients stay bf16 products of the
 * bf16 activations with fp32 accumulation (the row-wise recipe with
 * high-precision weight gradients); the router backward is that of
 * moe_backward.  Arguments as moe_backward, plus
 *   w8   data-gradient-layout copies (moe_fp8_weights_quantize)
 *   ws  >= moe_workspace_bytes(desc, MOE_WS_BACKWARD_FP8), or
 *          MOE_WS_BACKWARD_FP8_WGRAD with wgrad_fp8
 * w's bf16 expert weights are required (checked as moe_backward does).
 * Same layer limits as moe_forward_fp8. */
int moe_backward_fp8(const moe_desc_t *desc, const moe_weights_t *w, const moe_fp8_weights_t *w8,
                     int grad_format, int wgrad_fp8, const void *x, const moe_saved_t *saved, const void *dy,
                     void *dx,
                     const moe_grads_t *grads, const moe_router_terms_t *terms, float *losses,
                     void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------- timing */

/* Stages of moe_forward / moe_backward, for the per-stage timing below. */
enum {
  MOE_STAGE_ROUTER = 0,            /* fp32 router logits */
  MOE_STAGE_ROUTE,                 /* scores, top-k, gates, block histogram */
  MOE_STAGE_PERMUTE,               /* scan + stable scatter of the rows */
  MOE_STAGE_GATE_UP,               /* routed gate/up GEMM + SwiGLU */
  MOE_STAGE_DOWN,                  /* routed down GEMM */
  MOE_STAGE_SHARED_GATE_UP,
  MOE_STAGE_SHARED_DOWN,
  MOE_STAGE_COMBINE,
  MOE_STAGE_COMBINE_BWD,           /* + router backward to dlogits */
  MOE_STAGE_DOWN_DGRAD,            /* + SwiGLU derivative */
  MOE_STAGE_DOWN_WGRAD,
  MOE_STAGE_GATE_UP_WGRAD,
  MOE_STAGE_GATE_UP_DGRAD,
  MOE_STAGE_SHARED_DOWN_DGRAD,
  MOE_STAGE_SHARED_DOWN_WGRAD,
  MOE_STAGE_SHARED_GATE_UP_WGRAD,
  MOE_STAGE_SHARED_GATE_UP_DGRAD,
  MOE_STAGE_ROUTER_WGRAD,
  MOE_STAGE_UNPERMUTE_SUM,
  MOE_STAGE_ROUTER_TERMS,          /* balance losses and z-loss (when requested) */
  MOE_STAGE_FP8_QUANTIZE,          /* fp8 layer calls: activation quantisation */
  MOE_NUM_STAGES
};

/* Per-stage timing, a measurement aid.  While enabled, moe_forward and
 * moe_backward record a pair of HIP events around each stage's launches on
 * the caller's stream (at most 65536 pairs are kept; later stages go
 * untimed).  Process-wide state guarded by a lock; do not enable it while
 * the stream is being captured into a graph.  moe_stage_timing(1) clears
 * what was recorded; moe_stage_timing(0) stops recording. */
int moe_stage_timing(int enable);

/* As moe_stage_timing, for the stages whose bit (1 << stage) is set in mask
 * only (0 stops recording): fewer event pairs in a timed region. */
int moe_stage_timing_mask(uint32_t mask);

/* Waits for every recorded stage, adds its elapsed milliseconds to
 * ms[stage] and 1 to launches[stage] (both arrays of MOE_NUM_STAGES, written
 * in full), and clears the records.  MOE_ERR_HIP if an event query fails. */
int moe_stage_times(double *ms, int64_t *launches);

/* The matrix cores' sustained rate, a measurement aid (the compute
 * counterpart of timing a device-to-device copy as the practical HBM
 * ceiling): 2 workgroups per compute unit, 8 waves each, every wave running
 * `iters` rounds of 8 independent MFMAs of one kind on register operands
 * with finite pseudo-random data, no memory traffic.  *flop_per_launch
 * (host) receives the launch's flops (2 per multiply-add); the caller times
 * the launch on `stream`.  out: device float[1], receives a checksum.
 * MOE_ERR_INVALID for an unknown kind or iters outside [1, 2^30]. */
enum {
  MOE_MFMA_BF16_32X32X16 = 0,  /* the bf16 products' instruction           */
  MOE_MFMA_BF16_16X16X32 = 1,
  MOE_MFMA_E4M3_32X32X64 = 2,  /* the fp8 products' instruction            */
  MOE_MFMA_E4M3_16X16X128 = 3
};
int moe_mfma_ceiling(int kind, int64_t iters, float *out, double *flop_per_launch, void *stream);

/* The memory counterpart: copies `bytes` (a multiple of 16, at most 2^40)
 * from src to dst, one 16-byte vector per thread with nontemporal loads and
 * stores, the access pattern the streaming kernels of the layer use; the
 * caller times it on `stream` as the practical HBM ceiling (read + write
 * bytes over the time).  Measured on one MI355X: 6.2-6.5 TB/s for 1 GiB,
 * against 5.0 TB/s for a device-to-device hipMemcpy.  MOE_ERR_INVALID for a
 * size that is not a multiple of 16 or for null pointers with bytes > 0,
 * MOE_ERR_ALIGN for pointers not 16-byte aligned. */
int moe_hbm_ceiling(const void *src, void *dst, int64_t bytes, void *stream);

/* tokens per histogram block of moe_route / moe_permute */
#define MOE_ROUTE_BLOCK 32

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
