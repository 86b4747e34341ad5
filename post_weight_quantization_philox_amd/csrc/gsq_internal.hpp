// Launchers shared between the kernel files and the C ABI (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gsq.h"
#include "gsq_device.hpp"

namespace gsq {

struct LayerDesc {
    int grid;
    bool w_bf16;
    uint64_t rows, cols, mk;  // mk = rows * cols
    uint32_t sid;
    Key key;
};

// Per-launch temperature constants: y = l*a - b*t (Gumbel) or l*a + b*n2
// (logistic), with a = log2(e)/tau, b = eta/tau.
struct TauK {
    float a, b, invtau;
};

hipError_t launch_init_rtn(const LayerDesc& d, const void* W, float* scales, uint8_t* codes,
                           float* logits, float init_logit, hipStream_t st);
hipError_t launch_relax_fwd(const LayerDesc& d, const float* logits, const float* scales,
                            const uint8_t* codes, const void* W, uint32_t step, TauK tk,
                            uint16_t* dW, float* w_soft_dbg, hipStream_t st);
// Backward + Lion; with dW != nullptr also the next step's forward (no
// debug outputs in that mode).
hipError_t launch_relax_bwd_lion(const LayerDesc& d, const float* G, float* logits, float* mom,
                                 float* scales, float* scale_mom, const uint8_t* codes,
                                 uint32_t step, TauK tk, LionK lk_logit, LionK lk_scale,
                                 float* grad_logits_dbg, float* grad_scales_dbg, const void* W,
                                 uint32_t next_step, TauK tk_next, uint16_t* dW, hipStream_t st);
hipError_t launch_harden_pack(const LayerDesc& d, const float* logits, const float* scales,
                              const uint8_t* codes, uint8_t* codes_out, uint32_t* packed,
                              uint16_t* scales_f16, hipStream_t st);
hipError_t launch_noise_dump(const LayerDesc& d, uint32_t step, uint64_t first, uint64_t count,
                             uint32_t* out, hipStream_t st);

// Reconstruction GEMMs.
size_t recon_partials(int32_t n_experts, const int64_t* tok_offsets, int64_t rows_per_expert);
hipError_t launch_recon(int32_t n_experts, const int64_t* tok_offsets, int64_t rows_per_expert,
                        int64_t cols, const uint16_t* X, const uint16_t* XT, const uint16_t* dW,
                        float* partials, uint16_t* RT, float* G, double* loss, hipStream_t st);
// The first product alone (R^T and the loss partials, in the same launches
// and partial order as launch_recon); *n_partials receives the count.
hipError_t launch_recon_gemm1(int32_t n_experts, const int64_t* tok_offsets, int64_t rows_per_expert,
                              int64_t cols, const uint16_t* X, const uint16_t* dW, float* partials,
                              uint16_t* RT, size_t* n_partials, hipStream_t st);
// The second product fused with backward + Lion (and the next forward when
// dW_next is given): G = 2 R^T X is formed tile by tile on the matrix cores
// and consumed in registers, never stored. The first launch also sums
// n_partials loss partials into *loss (fused.hip).
hipError_t launch_recon_relax(const LayerDesc& d, int32_t n_experts, const int64_t* tok_offsets,
                              int64_t rows_per_expert, const uint16_t* XT, const uint16_t* RT,
                              const float* partials, size_t n_partials, double* loss,
                              float* logits, float* mom, float* scales, float* scale_mom,
                              const uint8_t* codes, uint32_t step, TauK tk, LionK lkl, LionK lks,
                              const void* W, uint32_t next_step, TauK tk_next, uint16_t* dW_next,
                              hipStream_t st);
// One dense layer's objective with a fixed offset on the residual:
// R^T = dW X^T + E0T (bf16 [rows][tokens]), loss = sum R^2, G = 2 R^T X.
hipError_t launch_recon_offset(int64_t rows, int64_t cols, int64_t tokens, const uint16_t* X,
                               const uint16_t* XT, const uint16_t* dW, const uint16_t* E0T,
                               float* partials, uint16_t* RT, float* G, double* loss,
                               hipStream_t st);
size_t gram_partials(int64_t rows, int64_t cols);
hipError_t launch_gram(int64_t tokens, int64_t cols, const uint16_t* XT, uint16_t* H,
                       hipStream_t st);
hipError_t launch_recon_gram(int64_t rows, int64_t cols, const uint16_t* H, const uint16_t* dW,
                             float* partials, float* G, double* loss, hipStream_t st);
// H = X^T X in fp32 (GPTQ's Hessian), [cols][cols].
hipError_t launch_gram_f32(int64_t tokens, int64_t cols, const uint16_t* XT, float* H32,
                           hipStream_t st);

// GPTQ warm start (gptq.hip): scratch carved from one caller-provided buffer.
struct GptqWorkspace {
    float* H32;           // [cols][cols] X^T X
    double* A;            // [cols][cols]: reversed Cholesky factor (lower), V (upper)
    double* P;            // [cols][rows] feedback of the finished groups, column-major
    double* Dg;           // [128][rows] the current group's rounding errors, column-major
    double* lambda;       // damping added to the diagonal
    const float* scales;  // [rows][cols/128] group scales (the caller's output)
};
size_t gptq_workspace_bytes(int64_t rows, int64_t cols);
GptqWorkspace gptq_carve(void* base, int64_t rows, int64_t cols);
hipError_t launch_gptq_factor(int64_t cols, float damp, const GptqWorkspace& ws, int32_t* info,
                              hipStream_t st);
hipError_t launch_gptq_columns(const LayerDesc& d, const void* W, const GptqWorkspace& ws,
                               uint8_t* codes, float* logits, float init_logit, hipStream_t st);

// Plain NT product C = A B^T in bf16 (fp32 accumulation), for the block forward.
hipError_t launch_matmul_nt_bf16(int64_t I, int64_t J, int64_t Rd, const uint16_t* A, int64_t lda,
                                 const uint16_t* B, int64_t ldb, uint16_t* C, int64_t ldc,
                                 hipStream_t st);
// Block forward pieces (block.hip).
hipError_t launch_rmsnorm(int64_t rows, int64_t cols, const uint16_t* x, const float* gamma,
                          float eps, uint16_t* y, hipStream_t st);
hipError_t launch_softmax_causal(int64_t n, const uint16_t* S, float scale, uint16_t* P,
                                 hipStream_t st);
hipError_t launch_silu_mul(int64_t n, const uint16_t* gate, const uint16_t* up, uint16_t* act,
                           hipStream_t st);
hipError_t launch_add(int64_t n, const uint16_t* a, const uint16_t* b, uint16_t* out,
                      hipStream_t st);
hipError_t launch_sub(int64_t n, const uint16_t* a, const uint16_t* b, uint16_t* out,
                      hipStream_t st);
hipError_t launch_dequant(const LayerDesc& d, const uint8_t* codes, const uint16_t* s16,
                          uint16_t* W, hipStream_t st);

hipError_t launch_transpose_tokens(int32_t n_experts, const int64_t* tok_offsets, int64_t cols,
                                   const uint16_t* X, uint16_t* XT, hipStream_t st);

}  // namespace gsq
