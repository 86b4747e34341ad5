// C ABI of the GSQ library: argument checks, then launches on the caller's
// stream. Every check runs before anything touches the device, so a rejected
// call has no side effect.
#include <cmath>
#include <cstdint>
#include <mutex>

#include "gsq_internal.hpp"

// Loss partials of gsq_recon_loss_grad_noalloc: a static device array
// (each device holds its own copy until the process ends). Host code never
// passes the array's name to a kernel: that name is a host-side stand-in, so
// the device address is looked up once per device and kept.
constexpr size_t kScratchFloats = size_t(1) << 16;   // 256 KiB
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {

using gsq::LayerDesc;

constexpr int64_t kMaxCoords = int64_t(1) << 40;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int num_logits(int grid) {
    switch (grid) {
        case GSQ_GRID_INT2: return 4;
        case GSQ_GRID_TERNARY: return 2;
        case GSQ_GRID_INT3_LOCAL: return 5;
        case GSQ_GRID_INT3: return 8;
        default: return 0;
    }
}

gsq_status check_layer(const gsq_layer* L, LayerDesc* d) {
    if (L == nullptr) return GSQ_ERR_NULL;
    if (num_logits(L->grid) == 0) return GSQ_ERR_GRID;
    if (L->group != 128) return GSQ_ERR_SHAPE;
    if (L->rows <= 0 || L->cols <= 0 || (L->cols % 128) != 0) return GSQ_ERR_SHAPE;
    if (L->rows > kMaxCoords / L->cols) return GSQ_ERR_SHAPE;
    if (L->w_dtype != GSQ_DTYPE_F32 && L->w_dtype != GSQ_DTYPE_BF16) return GSQ_ERR_PARAM;
    d->grid = L->grid;
    d->w_bf16 = L->w_dtype == GSQ_DTYPE_BF16;
    d->rows = static_cast<uint64_t>(L->rows);
    d->cols = static_cast<uint64_t>(L->cols);
    d->mk = d->rows * d->cols;
    d->sid = L->stream;
    d->key.k0 = static_cast<uint32_t>(L->seed);
    d->key.k1 = static_cast<uint32_t>(L->seed >> 32);
    return GSQ_OK;
}

// A required device tensor: present and 16-byte aligned.
gsq_status need(const void* p) {
    if (p == nullptr) return GSQ_ERR_NULL;
    return aligned16(p) ? GSQ_OK : GSQ_ERR_ALIGN;
}

// An optional device tensor: NULL, or 16-byte aligned.
gsq_status maybe(const void* p) { return (p == nullptr || aligned16(p)) ? GSQ_OK : GSQ_ERR_ALIGN; }

gsq_status check_tau(float tau, float noise_scale, gsq::TauK* tk) {
    if (!std::isfinite(tau) || !(tau > 0.0f)) return GSQ_ERR_PARAM;
    if (!std::isfinite(noise_scale) || noise_scale < 0.0f || noise_scale > 1.0f) return GSQ_ERR_PARAM;
    const double inv = 1.0 / static_cast<double>(tau);
    if (!std::isfinite(inv * 1.4426950408889634)) return GSQ_ERR_PARAM;
    tk->a = static_cast<float>(1.4426950408889634 * inv);
    tk->b = static_cast<float>(static_cast<double>(noise_scale) * inv);
    tk->invtau = static_cast<float>(inv);
    return GSQ_OK;
}

gsq_status lion_consts(float lr, const gsq_lion* l, gsq::LionK* k) {
    if (!std::isfinite(lr) || lr < 0.0f) return GSQ_ERR_PARAM;
    if (!(l->beta1 >= 0.0f && l->beta1 < 1.0f) || !(l->beta2 >= 0.0f && l->beta2 < 1.0f))
        return GSQ_ERR_PARAM;
    if (!std::isfinite(l->weight_decay) || l->weight_decay < 0.0f) return GSQ_ERR_PARAM;
    k->lr = lr;
    k->b1 = l->beta1;
    k->omb1 = 1.0f - l->beta1;
    k->b2 = l->beta2;
    k->omb2 = 1.0f - l->beta2;
    k->nlrwd = -(lr * l->weight_decay);
    return GSQ_OK;
}

#define GSQ_TRY(expr)                         \
    do {                                      \
        const gsq_status s_ = (expr);         \
        if (s_ != GSQ_OK) return s_;          \
    } while (0)

inline gsq_status hip_status(hipError_t e) { return e == hipSuccess ? GSQ_OK : GSQ_ERR_HIP; }

gsq_status check_offsets(int32_t n_experts, const int64_t* offs, int64_t rows_per_expert,
                         int64_t cols) {
    if (n_experts < 1) return GSQ_ERR_SHAPE;
    if (offs == nullptr) return GSQ_ERR_NULL;
    if (rows_per_expert <= 0 || rows_per_expert > INT32_MAX) return GSQ_ERR_SHAPE;
    if (cols <= 0 || (cols % 128) != 0 || cols > INT32_MAX) return GSQ_ERR_SHAPE;
    if (offs[0] != 0) return GSQ_ERR_SHAPE;
    for (int e = 0; e < n_experts; ++e) {
        const int64_t ne = offs[e + 1] - offs[e];
        if (ne < 0 || (offs[e + 1] % 64) != 0 || ne > INT32_MAX) return GSQ_ERR_SHAPE;
    }
    if (offs[n_experts] > kMaxCoords / cols) return GSQ_ERR_SHAPE;
    if (static_cast<int64_t>(n_experts) * rows_per_expert > kMaxCoords / cols) return GSQ_ERR_SHAPE;
    return GSQ_OK;
}

// The GEMM addresses each bf16 operand with 32-bit byte offsets below 2^31
// (plus the contraction length), so an operand must stay under about 2 GiB.
inline bool gemm_operand_fits(int64_t rows, int64_t ld, int64_t contraction) {
    return rows * ld * 2 <= int64_t(0x7FFFFF00) - 2 * contraction;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_dev[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call there, with that device current).
gsq_status scratch_on_current_device(float** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GSQ_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return GSQ_ERR_HIP;
        g_scratch_dev[dev] = static_cast<float*>(p);
    }
    *out = g_scratch_dev[dev];
    return GSQ_OK;
}

}  // namespace

extern "C" {

int gsq_abi_version(void) { return GSQ_ABI_VERSION; }

const char* gsq_status_str(int status) {
    switch (status) {
        case GSQ_OK: return "GSQ_OK";
        case GSQ_ERR_NULL: return "GSQ_ERR_NULL";
        case GSQ_ERR_SHAPE: return "GSQ_ERR_SHAPE";
        case GSQ_ERR_ALIGN: return "GSQ_ERR_ALIGN";
        case GSQ_ERR_GRID: return "GSQ_ERR_GRID";
        case GSQ_ERR_PARAM: return "GSQ_ERR_PARAM";
        case GSQ_ERR_HIP: return "GSQ_ERR_HIP";
        case GSQ_ERR_SCRATCH: return "GSQ_ERR_SCRATCH";
        default: return "GSQ_ERR_UNKNOWN";
    }
}

int gsq_num_logits(int grid) { return num_logits(grid); }

gsq_status gsq_init_rtn(const gsq_layer* layer, const void* W, float* scales, uint8_t* codes,
                        float* logits, float init_logit, void* stream) {
    LayerDesc d;
    GSQ_TRY(check_layer(layer, &d));
    GSQ_TRY(need(W));
    GSQ_TRY(need(scales));
    GSQ_TRY(need(codes));
    GSQ_TRY(need(logits));
    if (!std::isfinite(init_logit)) return GSQ_ERR_PARAM;
    return hip_status(gsq::launch_init_rtn(d, W, scales, codes, logits, init_logit,
                                           static_cast<hipStream_t>(stream)));
}

size_t gsq_gptq_workspace_bytes(int64_t rows, int64_t cols) {
    if (rows <= 0 || rows > INT32_MAX || cols <= 0 || (cols % 128) != 0 || cols > INT32_MAX) return 0;
    if (rows > kMaxCoords / cols || cols > kMaxCoords / cols) return 0;
    return gsq::gptq_workspace_bytes(rows, cols);
}

gsq_status gsq_init_gptq(const gsq_layer* layer, const void* W, int64_t tokens, const uint16_t* XT,
                         float damp, float init_logit, void* workspace, size_t workspace_bytes,
                         float* scales, uint8_t* codes, float* logits, int32_t* info,
                         void* stream) {
    LayerDesc d;
    GSQ_TRY(check_layer(layer, &d));
    GSQ_TRY(need(W));
    GSQ_TRY(need(XT));
    GSQ_TRY(need(workspace));
    GSQ_TRY(need(scales));
    GSQ_TRY(need(codes));
    GSQ_TRY(need(logits));
    if (info == nullptr) return GSQ_ERR_NULL;
    if (tokens <= 0 || (tokens % 64) != 0 || tokens > INT32_MAX) return GSQ_ERR_SHAPE;
    if (tokens > kMaxCoords / d.cols) return GSQ_ERR_SHAPE;
    if (!gemm_operand_fits(d.cols, tokens, tokens)) return GSQ_ERR_SHAPE;
    if (!(damp >= 0.0f) || !std::isfinite(damp) || !std::isfinite(init_logit)) return GSQ_ERR_PARAM;
    if (workspace_bytes < gsq_gptq_workspace_bytes(d.rows, d.cols)) return GSQ_ERR_SHAPE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    gsq::GptqWorkspace ws = gsq::gptq_carve(workspace, d.rows, d.cols);
    ws.scales = scales;
    hipError_t err = gsq::launch_init_rtn(d, W, scales, codes, logits, init_logit, st);
    if (err == hipSuccess) err = gsq::launch_gram_f32(tokens, d.cols, XT, ws.H32, st);
    if (err == hipSuccess) err = gsq::launch_gptq_factor(d.cols, damp, ws, info, st);
    if (err == hipSuccess) err = gsq::launch_gptq_columns(d, W, ws, codes, logits, init_logit, st);
    return hip_status(err);
}

gsq_status gsq_matmul_nt_bf16(int64_t I, int64_t J, int64_t Rd, const uint16_t* A, int64_t lda,
                              const uint16_t* B, int64_t ldb, uint16_t* C, int64_t ldc,
                              void* stream) {
    if (I <= 0 || J <= 0 || I > INT32_MAX || J > INT32_MAX) return GSQ_ERR_SHAPE;
    if (Rd <= 0 || Rd > INT32_MAX || (Rd % 64) != 0) return GSQ_ERR_SHAPE;
    if (lda < Rd || ldb < Rd || ldc < J) return GSQ_ERR_SHAPE;
    if ((lda % 8) != 0 || (ldb % 8) != 0 || (ldc % 8) != 0 || (J % 8) != 0) return GSQ_ERR_ALIGN;
    if (!gemm_operand_fits(I, lda, Rd) || !gemm_operand_fits(J, ldb, Rd)) return GSQ_ERR_SHAPE;
    GSQ_TRY(need(A));
    GSQ_TRY(need(B));
    GSQ_TRY(need(C));
    return hip_status(gsq::launch_matmul_nt_bf16(I, J, Rd, A, lda, B, ldb, C, ldc,
                                                 static_cast<hipStream_t>(stream)));
}

gsq_status gsq_rmsnorm_bf16(int64_t rows, int64_t cols, const uint16_t* x, const float* gamma,
                            float eps, uint16_t* y, void* stream) {
    if (rows <= 0 || rows > INT32_MAX || cols <= 0 || cols > kMaxCoords / rows) return GSQ_ERR_SHAPE;
    if (!(eps > 0.0f) || !std::isfinite(eps)) return GSQ_ERR_PARAM;
    GSQ_TRY(need(x));
    GSQ_TRY(need(gamma));
    GSQ_TRY(need(y));
    return hip_status(gsq::launch_rmsnorm(rows, cols, x, gamma, eps, y,
                                          static_cast<hipStream_t>(stream)));
}

gsq_status gsq_softmax_causal_bf16(int64_t n, const uint16_t* S, float scale, uint16_t* P,
                                   void* stream) {
    if (n <= 0 || n > INT32_MAX || n > kMaxCoords / n) return GSQ_ERR_SHAPE;
    if (!std::isfinite(scale)) return GSQ_ERR_PARAM;
    GSQ_TRY(need(S));
    GSQ_TRY(need(P));
    return hip_status(gsq::launch_softmax_causal(n, S, scale, P, static_cast<hipStream_t>(stream)));
}

gsq_status gsq_silu_mul_bf16(int64_t n, const uint16_t* gate, const uint16_t* up, uint16_t* act,
                             void* stream) {
    if (n < 0 || n > kMaxCoords) return GSQ_ERR_SHAPE;
    if (n == 0) return GSQ_OK;
    GSQ_TRY(need(gate));
    GSQ_TRY(need(up));
    GSQ_TRY(need(act));
    return hip_status(gsq::launch_silu_mul(n, gate, up, act, static_cast<hipStream_t>(stream)));
}

gsq_status gsq_add_bf16(int64_t n, const uint16_t* a, const uint16_t* b, uint16_t* out,
                        void* stream) {
    if (n < 0 || n > kMaxCoords) return GSQ_ERR_SHAPE;
    if (n == 0) return GSQ_OK;
    GSQ_TRY(need(a));
    GSQ_TRY(need(b));
    GSQ_TRY(need(out));
    return hip_status(gsq::launch_add(n, a, b, out, static_cast<hipStream_t>(stream)));
}

gsq_status gsq_sub_bf16(int64_t n, const uint16_t* a, const uint16_t* b, uint16_t* out,
                        void* stream) {
    if (n < 0 || n > kMaxCoords) return GSQ_ERR_SHAPE;
    if (n == 0) return GSQ_OK;
    GSQ_TRY(need(a));
    GSQ_TRY(need(b));
    GSQ_TRY(need(out));
    return hip_status(gsq::launch_sub(n, a, b, out, static_cast<hipStream_t>(stream)));
}

gsq_status gsq_dequant_bf16(const gsq_layer* layer, const uint8_t* codes,
                            const uint16_t* scales_f16, uint16_t* W, void* stream) {
    LayerDesc d;
    GSQ_TRY(check_layer(layer, &d));
    GSQ_TRY(need(codes));
    GSQ_TRY(need(scales_f16));
    GSQ_TRY(need(W));
    return hip_status(gsq::launch_dequant(d, codes, scales_f16, W, static_cast<hipStream_t>(stream)));
}

gsq_status gsq_relax_fwd(const gsq_layer* layer, const float* logits, const float* scales,
                         const uint8_t* init_codes, const void* W, uint32_t step, float tau,
                         float noise_scale, uint16_t* dW_bf16, float* w_soft_dbg, void* stream) {
    LayerDesc d;
    GSQ_TRY(check_layer(layer, &d));
    GSQ_TRY(need(logits));
    GSQ_TRY(need(scales));
    GSQ_TRY(need(W));
    GSQ_TRY(need(dW_bf16));
    GSQ_TRY(maybe(w_soft_dbg));
    if (d.grid == GSQ_GRID_INT3_LOCAL) {
        if (init_codes == nullptr) return GSQ_ERR_GRID;
        GSQ_TRY(need(init_codes));
    }
    gsq::TauK tk;
    GSQ_TRY(check_tau(tau, noise_scale, &tk));
    return hip_status(gsq::launch_relax_fwd(d, logits, scales, init_codes, W, step, tk, dW_bf16,
                                            w_soft_dbg, static_cast<hipStream_t>(stream)));
}

size_t gsq_recon_workspace_bytes(int32_t n_experts, const int64_t* tok_offsets,
                                 int64_t rows_per_expert, int64_t cols) {
    if (check_offsets(n_experts, tok_offsets, rows_per_expert, cols) != GSQ_OK) return 0;
    const size_t n = gsq::recon_partials(n_experts, tok_offsets, rows_per_expert);
    return ((n * sizeof(float) + 255) / 256) * 256 + 256;
}

gsq_status gsq_recon_loss_grad(int32_t n_experts, const int64_t* tok_offsets,
                               int64_t rows_per_expert, int64_t cols, const uint16_t* X,
                               const uint16_t* XT, const uint16_t* dW_bf16, void* workspace,
                               size_t workspace_bytes, uint16_t* RT, float* G, double* loss,
                               void* stream) {
    GSQ_TRY(check_offsets(n_experts, tok_offsets, rows_per_expert, cols));
    const bool any_tokens = tok_offsets[n_experts] > 0;
    if (any_tokens) {
        GSQ_TRY(need(X));
        GSQ_TRY(need(XT));
        GSQ_TRY(need(RT));
    }
    GSQ_TRY(need(dW_bf16));
    GSQ_TRY(need(workspace));
    GSQ_TRY(need(G));
    GSQ_TRY(need(loss));
    if (workspace_bytes < gsq_recon_workspace_bytes(n_experts, tok_offsets, rows_per_expert, cols))
        return GSQ_ERR_SHAPE;
    return hip_status(gsq::launch_recon(n_experts, tok_offsets, rows_per_expert, cols, X, XT,
                                        dW_bf16, static_cast<float*>(workspace), RT, G, loss,
                                        static_cast<hipStream_t>(stream)));
}

gsq_status gsq_recon_loss_grad_noalloc(int32_t n_experts, const int64_t* tok_offsets,
                                       int64_t rows_per_expert, int64_t cols, const uint16_t* X,
                                       const uint16_t* XT, const uint16_t* dW_bf16, uint16_t* RT,
                                       float* G, double* loss, void* stream) {
    GSQ_TRY(check_offsets(n_experts, tok_offsets, rows_per_expert, cols));
    const bool any_tokens = tok_offsets[n_experts] > 0;
    if (any_tokens) {
        GSQ_TRY(need(X));
        GSQ_TRY(need(XT));
        GSQ_TRY(need(RT));
    }
    GSQ_TRY(need(dW_bf16));
    GSQ_TRY(need(G));
    GSQ_TRY(need(loss));
    if (gsq::recon_partials(n_experts, tok_offsets, rows_per_expert) > kScratchFloats)
        return GSQ_ERR_SCRATCH;
    float* partials = nullptr;
    GSQ_TRY(scratch_on_current_device(&partials));
    // Every partial is written by the first product before the second reads
    // it, so nothing in the array needs clearing.
    return hip_status(gsq::launch_recon(n_experts, tok_offsets, rows_per_expert, cols, X, XT,
                                        dW_bf16, partials, RT, G, loss,
                                        static_cast<hipStream_t>(stream)));
}

gsq_status gsq_recon_residual(int32_t n_experts, const int64_t* tok_offsets,
                              int64_t rows_per_expert, int64_t cols, const uint16_t* X,
                              const uint16_t* dW_bf16, void* workspace, size_t workspace_bytes,
                              uint16_t* RT, void* stream) {
    GSQ_TRY(check_offsets(n_experts, tok_offsets, rows_per_expert, cols));
    if (tok_offsets[n_experts] > 0) {
        GSQ_TRY(need(X));
        GSQ_TRY(need(RT));
    }
    GSQ_TRY(need(dW_bf16));
    GSQ_TRY(need(workspace));
    if (workspace_bytes < gsq_recon_workspace_bytes(n_experts, tok_offsets, rows_per_expert, cols))
        return GSQ_ERR_SHAPE;
    size_t n_partials = 0;
    return hip_status(gsq::launch_recon_gemm1(n_experts, tok_offsets, rows_per_expert, cols, X,
                                              dW_bf16, static_cast<float*>(workspace), RT,
                                              &n_partials, static_cast<hipStream_t>(stream)));
}

gsq_status gsq_recon_bwd_lion_fwd(const gsq_layer* layer, int32_t n_experts,
                                  const int64_t* tok_offsets, const uint16_t* XT,
                                  const uint16_t* RT, const void* workspace,
                                  size_t workspace_bytes, double* loss, float* logits, float* mom,
                                  float* scales, float* scale_mom, const uint8_t* init_codes,
                                  const void* W, uint32_t step, float tau, float noise_scale,
                                  const gsq_lion* lion, int32_t with_next, uint32_t next_step,
                                  float next_tau, uint16_t* dW_bf16, void* stream) {
    LayerDesc d;
    GSQ_TRY(check_layer(layer, &d));
    if (n_experts < 1 || layer->rows % n_experts != 0) return GSQ_ERR_SHAPE;
    const int64_t rpe = layer->rows / n_experts;
    GSQ_TRY(check_offsets(n_experts, tok_offsets, rpe, layer->cols));
    if (tok_offsets[n_experts] > INT32_MAX) return GSQ_ERR_SHAPE;
    if (tok_offsets[n_experts] > 0) {
        GSQ_TRY(need(XT));
        GSQ_TRY(need(RT));
    }
    GSQ_TRY(need(workspace));
    GSQ_TRY(need(loss));
    GSQ_TRY(need(logits));
    GSQ_TRY(need(mom));
    GSQ_TRY(need(scales));
    GSQ_TRY(need(scale_mom));
    if (with_next != 0 && with_next != 1) return GSQ_ERR_PARAM;
    if (with_next) {
        GSQ_TRY(need(W));
        GSQ_TRY(need(dW_bf16));
    }
    if (d.grid == GSQ_GRID_INT3_LOCAL) {
        if (init_codes == nullptr) return GSQ_ERR_GRID;
        GSQ_TRY(need(init_codes));
    }
    if (lion == nullptr) return GSQ_ERR_NULL;
    if (workspace_bytes < gsq_recon_workspace_bytes(n_experts, tok_offsets, rpe, layer->cols))
        return GSQ_ERR_SHAPE;
    gsq::TauK tk, tk_next = {};
    GSQ_TRY(check_tau(tau, noise_scale, &tk));
    if (with_next) GSQ_TRY(check_tau(next_tau, noise_scale, &tk_next));
    gsq::LionK lkl, lks;
    GSQ_TRY(lion_consts(lion->lr_logit, lion, &lkl));
    GSQ_TRY(lion_consts(lion->lr_scale, lion, &lks));
    const size_t n_partials = gsq::recon_partials(n_experts, tok_offsets, rpe);
    return hip_status(gsq::launch_recon_relax(
        d, n_experts, tok_offsets, rpe, XT, RT, static_cast<const float*>(workspace), n_partials,
        loss, logits, mom, scales, scale_mom, init_codes, step, tk, lkl, lks, W, next_step,
        tk_next, with_next ? dW_bf16 : nullptr, static_cast<hipStream_t>(stream)));
}

gsq_status gsq_recon_loss_grad_offset(int64_t rows, int64_t cols, int64_t tokens,
                                     const uint16_t* X, const uint16_t* XT,
                                     const uint16_t* dW_bf16, const uint16_t* E0T,
                                     void* workspace, size_t workspace_bytes, uint16_t* RT,
                                     float* G, double* loss, void* stream) {
    if (tokens <= 0) return GSQ_ERR_SHAPE;
    const int64_t offs[2] = {0, tokens};
    GSQ_TRY(check_offsets(1, offs, rows, cols));
    GSQ_TRY(need(X));
    GSQ_TRY(need(XT));
    GSQ_TRY(need(dW_bf16));
    GSQ_TRY(need(E0T));
    GSQ_TRY(need(workspace));
    GSQ_TRY(need(RT));
    GSQ_TRY(need(G));
    GSQ_TRY(need(loss));
    if (workspace_bytes < gsq_recon_workspace_bytes(1, offs, rows, cols)) return GSQ_ERR_SHAPE;
    return hip_status(gsq::launch_recon_offset(rows, cols, tokens, X, XT, dW_bf16, E0T,
                                               static_cast<float*>(workspace), RT, G, loss,
                                               static_cast<hipStream_t>(stream)));
}

gsq_status gsq_transpose_tokens(int32_t n_experts, const int64_t* tok_offsets, int64_t cols,
                                const uint16_t* X, uint16_t* XT, void* stream) {
    GSQ_TRY(check_offsets(n_experts, tok_offsets, 1, cols));
    if (tok_offsets[n_experts] == 0) return GSQ_OK;
    GSQ_TRY(need(X));
    GSQ_TRY(need(XT));
    return hip_status(gsq::launch_transpose_tokens(n_experts, tok_offsets, cols, X, XT,
                                                   static_cast<hipStream_t>(stream)));
}

gsq_status gsq_gram(int64_t tokens, int64_t cols, const uint16_t* XT, uint16_t* H, void* stream) {
    if (tokens <= 0 || (tokens % 64) != 0 || tokens > INT32_MAX) return GSQ_ERR_SHAPE;
    if (cols <= 0 || (cols % 128) != 0 || cols > INT32_MAX) return GSQ_ERR_SHAPE;
    if (tokens > kMaxCoords / cols || cols > kMaxCoords / cols) return GSQ_ERR_SHAPE;
    if (!gemm_operand_fits(cols, tokens, tokens)) return GSQ_ERR_SHAPE;
    GSQ_TRY(need(XT));
    GSQ_TRY(need(H));
    return hip_status(gsq::launch_gram(tokens, cols, XT, H, static_cast<hipStream_t>(stream)));
}

size_t gsq_recon_gram_workspace_bytes(int64_t rows, int64_t cols) {
    if (rows <= 0 || rows > INT32_MAX || cols <= 0 || (cols % 128) != 0 || cols > INT32_MAX)
        return 0;
    const size_t n = gsq::gram_partials(rows, cols);
    return ((n * sizeof(float) + 255) / 256) * 256 + 256;
}

gsq_status gsq_recon_gram(int64_t rows, int64_t cols, const uint16_t* H, const uint16_t* dW_bf16,
                          void* workspace, size_t workspace_bytes, float* G, double* loss,
                          void* stream) {
    if (rows <= 0 || rows > INT32_MAX) return GSQ_ERR_SHAPE;
    if (cols <= 0 || (cols % 128) != 0 || cols > INT32_MAX) return GSQ_ERR_SHAPE;
    if (rows > kMaxCoords / cols || cols > kMaxCoords / cols) return GSQ_ERR_SHAPE;
    if (!gemm_operand_fits(rows, cols, cols) || !gemm_operand_fits(cols, cols, cols))
        return GSQ_ERR_SHAPE;
    GSQ_TRY(need(H));
    GSQ_TRY(need(dW_bf16));
    GSQ_TRY(need(workspace));
    GSQ_TRY(need(G));
    GSQ_TRY(need(loss));
    if (workspace_bytes < gsq_recon_gram_workspace_bytes(rows, cols)) return GSQ_ERR_SHAPE;
    return hip_status(gsq::launch_recon_gram(rows, cols, H, dW_bf16,
                                             static_cast<float*>(workspace), G, loss,
                                             static_cast<hipStream_t>(stream)));
}

gsq_status gsq_relax_bwd_lion(const gsq_layer* layer, const float* G, float* logits, float* mom,
                              float* scales, float* scale_mom, const uint8_t* init_codes,
                              uint32_t step, float tau, float noise_scale, const gsq_lion* lion,
                              float* grad_logits_dbg, float* grad_scales_dbg, void* stream) {
    LayerDesc d;
    GSQ_TRY(check_layer(layer, &d));
    GSQ_TRY(need(G));
    GSQ_TRY(need(logits));
    GSQ_TRY(need(mom));
    GSQ_TRY(need(scales));
    GSQ_TRY(need(scale_mom));
    GSQ_TRY(maybe(grad_logits_dbg));
    GSQ_TRY(maybe(grad_scales_dbg));
    if ((grad_logits_dbg == nullptr) != (grad_scales_dbg == nullptr)) return GSQ_ERR_NULL;
    if (d.grid == GSQ_GRID_INT3_LOCAL) {
        if (init_codes == nullptr) return GSQ_ERR_GRID;
        GSQ_TRY(need(init_codes));
    }
    if (lion == nullptr) return GSQ_ERR_NULL;
    gsq::TauK tk;
    GSQ_TRY(check_tau(tau, noise_scale, &tk));
    gsq::LionK lkl, lks;
    GSQ_TRY(lion_consts(lion->lr_logit, lion, &lkl));
    GSQ_TRY(lion_consts(lion->lr_scale, lion, &lks));
    return hip_status(gsq::launch_relax_bwd_lion(d, G, logits, mom, scales, scale_mom, init_codes,
                                                 step, tk, lkl, lks, grad_logits_dbg,
                                                 grad_scales_dbg, nullptr, 0, tk, nullptr,
                                                 static_cast<hipStream_t>(stream)));
}

gsq_status gsq_relax_bwd_lion_fwd(const gsq_layer* layer, const float* G, float* logits,
                                  float* mom, float* scales, float* scale_mom,
                                  const uint8_t* init_codes, const void* W, uint32_t step,
                                  float tau, float noise_scale, const gsq_lion* lion,
                                  uint32_t next_step, float next_tau, uint16_t* dW_bf16,
                                  void* stream) {
    LayerDesc d;
    GSQ_TRY(check_layer(layer, &d));
    GSQ_TRY(need(G));
    GSQ_TRY(need(logits));
    GSQ_TRY(need(mom));
    GSQ_TRY(need(scales));
    GSQ_TRY(need(scale_mom));
    GSQ_TRY(need(W));
    GSQ_TRY(need(dW_bf16));
    if (d.grid == GSQ_GRID_INT3_LOCAL) {
        if (init_codes == nullptr) return GSQ_ERR_GRID;
        GSQ_TRY(need(init_codes));
    }
    if (lion == nullptr) return GSQ_ERR_NULL;
    gsq::TauK tk, tk_next;
    GSQ_TRY(check_tau(tau, noise_scale, &tk));
    GSQ_TRY(check_tau(next_tau, noise_scale, &tk_next));
    gsq::LionK lkl, lks;
    GSQ_TRY(lion_consts(lion->lr_logit, lion, &lkl));
    GSQ_TRY(lion_consts(lion->lr_scale, lion, &lks));
    return hip_status(gsq::launch_relax_bwd_lion(d, G, logits, mom, scales, scale_mom, init_codes,
                                                 step, tk, lkl, lks, nullptr, nullptr, W,
                                                 next_step, tk_next, dW_bf16,
                                                 static_cast<hipStream_t>(stream)));
}

gsq_status gsq_harden_pack(const gsq_layer* layer, const float* logits, const float* scales,
                           const uint8_t* init_codes, uint8_t* codes, uint32_t* packed,
                           uint16_t* scales_f16, void* stream) {
    LayerDesc d;
    GSQ_TRY(check_layer(layer, &d));
    GSQ_TRY(need(logits));
    GSQ_TRY(maybe(codes));
    GSQ_TRY(maybe(packed));
    GSQ_TRY(maybe(scales_f16));
    if (scales_f16 != nullptr) GSQ_TRY(need(scales));
    if (d.grid == GSQ_GRID_INT3_LOCAL) {
        if (init_codes == nullptr) return GSQ_ERR_GRID;
        GSQ_TRY(need(init_codes));
    }
    if (codes == nullptr && packed == nullptr && scales_f16 == nullptr) return GSQ_OK;
    return hip_status(gsq::launch_harden_pack(d, logits, scales, init_codes, codes, packed,
                                              scales_f16, static_cast<hipStream_t>(stream)));
}

gsq_status gsq_noise_dump(const gsq_layer* layer, uint32_t step, int64_t first, int64_t count,
                          uint32_t* out, void* stream) {
    LayerDesc d;
    GSQ_TRY(check_layer(layer, &d));
    if (first < 0 || count < 0) return GSQ_ERR_SHAPE;
    if (count == 0) return GSQ_OK;
    if (out == nullptr) return GSQ_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(out) & 3u) != 0) return GSQ_ERR_ALIGN;
    return hip_status(gsq::launch_noise_dump(d, step, static_cast<uint64_t>(first),
                                             static_cast<uint64_t>(count), out,
                                             static_cast<hipStream_t>(stream)));
}

}  // extern "C"
