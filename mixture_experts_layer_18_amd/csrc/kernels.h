// Private declarations shared by the kernel sources and the ABI layer.
#pragma once

#include "../../include/moe.h"
#include "common.h"

namespace moe {

// ---- route / permute
hipError_t launch_route(const float* logits, const float* bias, int T, int E, int k, int score,
                        int renorm, int32_t* idx, float* gate, int32_t* hist, hipStream_t st);
hipError_t launch_permute(const void* x, int dtype, const int32_t* idx, const int32_t* hist, int T,
                          int d, int E, int k, int32_t* base, int32_t* counts, int32_t* offsets,
                          int32_t* pos, int32_t* src, int32_t* tok, void* x_perm, hipStream_t st);

// ---- measurement aid: the matrix cores' sustained rate (ceiling.hip)
int mfma_rate_grid();
hipError_t launch_mfma_rate(int kind, int64_t iters, float* out, hipStream_t st);

// ---- grouped GEMM
// Element types of the operands: A, B and C each f32 or bf16 (MOE_F32 / MOE_BF16).
struct GemmProblem {
  int layout, epilogue;
  int ta, tb, tc;        // element type of A, B, C (and aux = tc)
  int64_t G, M_total, N, K;
  const int32_t* offsets;  // device [G+1]
  const void* A;
  const void* B;
  void* C;
  void* aux;
  // optional row map of the operand indexed by the routed rows (NT: A, TN:
  // B): routed row r reads row rows[r] of that operand (persistent kernel)
  const int32_t* rows = nullptr;
};
size_t gemm_workspace_bytes(const GemmProblem& p);
hipError_t launch_grouped_gemm(const GemmProblem& p, void* ws, size_t ws_bytes, hipStream_t st);
hipError_t launch_gemm_mfma(const GemmProblem& p, void* ws, size_t ws_bytes,
                            hipStream_t st);  // bf16 operands only
// persistent 256 x 256 kernel (gemm_big.hip) for the products it supports
bool gemm_big_supported(const GemmProblem& p);
size_t gemm_big_workspace_bytes(const GemmProblem& p);  // fp32 row-slice partials (one-group TN)
hipError_t launch_gemm_big(const GemmProblem& p, void* ws, size_t ws_bytes, hipStream_t st);
// a routed weight gradient and a one-group one (the shared experts) in one launch
bool gemm_big_pair_supported(const GemmProblem& routed, const GemmProblem& one);
hipError_t launch_gemm_big_pair(const GemmProblem& routed, const GemmProblem& one, hipStream_t st);
hipError_t launch_iota(int32_t* p, int64_t n, hipStream_t st);  // p[i] = i
hipError_t launch_stream_copy(const void* src, void* dst, int64_t n16, hipStream_t st);  // n16 16-byte vectors
// fp8 (e4m3) forward products with row scales, persistent kernel
hipError_t launch_gemm_fp8(int epilogue, int64_t G, int64_t M_total, int64_t N, int64_t K,
                           const int32_t* offsets, const uint8_t* A, const float* a_scale,
                           const uint8_t* B, const float* b_scale, void* C, void* aux,
                           const int32_t* rows, hipStream_t st, int a_fmt = FP8_E4M3);
// column-wise over each group's rows, stored transposed and padded to
// 64-row multiples (the operands of an fp8 weight gradient); writes the
// padded group offsets pad_off [G+1] first
hipError_t launch_quantize_fp8_colwise(const void* x, int dtype, const int32_t* rows, const int32_t* offsets,
                                       int G, int64_t M, int64_t C, int32_t* pad_off, uint8_t* q, float* scale,
                                       hipStream_t st);
// fp8 weight gradient C[g] [N, K] = a_scale[g, n] b_scale[g, k] sum_m A'[n, m] B'[k, m]
// over the padded, transposed group blocks of launch_quantize_fp8_colwise
hipError_t launch_gemm_fp8_wgrad(int64_t G, int64_t N, int64_t K, const int32_t* pad_off, const uint8_t* A,
                                 const float* a_scale, const uint8_t* B, const float* b_scale, void* C,
                                 hipStream_t st);
hipError_t launch_quantize_fp8_transposed(const void* x, int dtype, int64_t G, int64_t R, int64_t C,
                                          uint8_t* q, float* scale, hipStream_t st);
// row-wise quantisation; fmt FP8_E4M3 or FP8_E5M2
hipError_t launch_quantize_fp8(const void* x, int dtype, int64_t R, int C, uint8_t* q, float* scale,
                               hipStream_t st, int fmt = FP8_E4M3);
size_t quantize_fp8_tensorwise_ws_bytes(int64_t R);
hipError_t launch_quantize_fp8_tensorwise(const void* x, int dtype, int64_t R, int C, uint8_t* q,
                                          float* scale, float* ws, hipStream_t st);
int gemm_mfma_tn_splits(const GemmProblem& p);
size_t gemm_mfma_workspace_bytes(const GemmProblem& p);
// out[i] = sum over p < nsplit of part[p * n + i], in order, rounded once to dtype
hipError_t launch_split_reduce(const float* part, int nsplit, int64_t n, void* out, int dtype,
                               hipStream_t st);

hipError_t launch_split_reduce_f32(const float* part, int nsplit, int64_t n, float* out,
                                  hipStream_t st);

// ---- fp32 router products (matrix cores)
hipError_t launch_router_logits(const void* x, int dtype, const float* w, int T, int d, int E,
                                float* logits, hipStream_t st);
// the forward's router logits with the routing of moe_route fused in (bf16 x,
// d a multiple of 128, E <= 64): logits, idx, gate and the block histogram
bool router_route_fused(int dtype, int d, int E);
hipError_t launch_router_route(const void* x, const float* w, int T, int d, int E, float* logits,
                               const float* bias, int k, int score, int renorm, int32_t* idx, float* gate,
                               int32_t* hist, hipStream_t st);
int router_wgrad_splits(int T, int d, int E);
// dw[E, d] = dl[T, E]^T x[T, d]; `part` holds router_wgrad_splits(..) * E * d floats
hipError_t launch_router_wgrad(const float* dl, const void* x, int dtype, int T, int d, int E,
                               float* part, float* dw, hipStream_t st);

// ---- router training terms
size_t router_terms_ws_bytes(int64_t T, int64_t E);
// dlogits += gradients of the enabled terms; losses (nullable): aux, seq_aux, z
hipError_t launch_router_terms(const float* logits, const int32_t* idx, const int32_t* counts,
                               int T, int E, int k, int score, float aux_coeff,
                               float seq_aux_coeff, float z_coeff, int seq_len, float* dlogits,
                               float* losses, void* ws, hipStream_t st);
hipError_t launch_bias_update(const int32_t* counts, int T, int E, int k, float rate, float* bias,
                              hipStream_t st);

// ---- combine and backward helpers
hipError_t launch_combine(int dtype, const void* y_perm, const float* gate, const int32_t* pos,
                          const void* shared_y, void* y, int T, int d, int k, hipStream_t st);
hipError_t launch_combine_bwd(int dtype, const void* dy, const void* y_perm, const float* gate,
                              const int32_t* pos, const int32_t* idx, const float* logits,
                              int score, int renorm, int T, int d, int E, int k, void* dy_perm,
                              float* dlogits, hipStream_t st);
// combine backward that also writes the row-wise e4m3 copies of dy_perm and
// dy (bf16 layers, 1 <= k <= 8)
hipError_t launch_combine_bwd_fp8(const void* dy, const void* y_perm, const float* gate, const int32_t* pos,
                                  const int32_t* idx, const float* logits, int score, int renorm, int T, int d,
                                  int E, int k, void* dy_perm, float* dlogits, uint8_t* q_perm, float* s_perm,
                                  uint8_t* q_dy, float* s_dy, hipStream_t st, int fmt = FP8_E4M3);
hipError_t launch_unpermute_sum(int dtype, const void* dx_perm, const int32_t* pos,
                                const void* dx_shared, const float* dlogits, const int32_t* idx,
                                const float* w_router, int dense_router, int T, int d, int E,
                                int k, void* dx, hipStream_t st);
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t st);

}  // namespace moe
