// GPTQ warm start on the GPU (Frantar, Ashkboos, Hoefler, Alistarh, "GPTQ:
// Accurate Post-Training Quantization for Generative Pre-trained
// Transformers", 2022), the initialisation the pages start GSQ from
// (agihunt.info optimizer paragraph; atlas.scime.ai Approach).
//
// GPTQ rounds the columns of W in order and feeds every rounding error into
// the later columns through the upper Cholesky factor of H^-1. The same
// recursion can be written on a factor of H itself, with no inverse: if
// H = R R^T with R upper triangular, column j is rounded from
//     t_j = w_j + sum_{i<j} (w_i - q_i) R_ij / R_jj
// (Babai's nearest-plane recursion; equal to GPTQ's column loop in exact
// arithmetic). R is the lower Cholesky factor of H with its index order
// reversed: R = J chol(J H J) J, J the reversal. Everything here is fp64
// except the rounding decision, which is taken in fp32 exactly like the
// round-to-nearest warm start (x = fp32(t) / s).
//
// Steps: H = X^T X (fp32, matrix cores, gemm.hip); lambda = damp * mean
// diag(H) (a zero diagonal entry counts as 1); A = J (H + lambda I) J in fp64
// (lower triangle); blocked right-looking Cholesky of A in place (64-column
// panels: the diagonal block in LDS by one wave, a triangular solve for the
// rows below, a symmetric rank-64 update of the trailing lower triangle); then
// V_ij = R_ij / R_jj for i < j, written into the unused upper triangle of A;
// then for every 128-column group: eight lanes per row run the group's 128
// columns sequentially (the group's block of V, the rows' w, w + P and
// errors in LDS),
// from targets that already hold the feedback of every earlier group; then
// the group's errors D = W - Q are fed forward into all later columns at once
// (P[:, later] += D V[group, later], an fp64 tiled product over the group's
// 128 columns that covers the whole GPU). Group scales are the absmax scales of the
// original weights (GPTQ's static groups), i.e. the round-to-nearest scales.
#include <math.h>

#include <algorithm>

#include "gsq_internal.hpp"

namespace gsq {

namespace {

constexpr int kPanel = 64;     // Cholesky panel width
constexpr int kBlock = 128;    // GPTQ column block = scale group

template <int GRID> struct GT;
template <> struct GT<GSQ_GRID_INT2> { static constexpr int L = 4, QMAX = 3, BITS = 2; };
template <> struct GT<GSQ_GRID_TERNARY> { static constexpr int L = 2, QMAX = 1, BITS = 2; };
template <> struct GT<GSQ_GRID_INT3_LOCAL> { static constexpr int L = 5, QMAX = 7, BITS = 3; };
template <> struct GT<GSQ_GRID_INT3> { static constexpr int L = 8, QMAX = 7, BITS = 3; };

__global__ void zero_info_kernel(int32_t* info) { *info = 0; }

// lambda = damp * mean(diag H), a zero diagonal entry counted as 1. One
// workgroup; fixed-order sums, so the value is deterministic.
__global__ __launch_bounds__(256) void damping_kernel(const float* __restrict__ H32, int64_t K,
                                                      float damp, double* __restrict__ lambda) {
    __shared__ double red[256];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < K; i += 256) {
        const double d = static_cast<double>(H32[i * K + i]);
        s += (d == 0.0) ? 1.0 : d;
    }
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if (static_cast<int>(threadIdx.x) < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) *lambda = static_cast<double>(damp) * (red[0] / static_cast<double>(K));
}

// A[i][j] = H[K-1-i][K-1-j] (+ lambda on the diagonal, zero diagonals set to
// 1 first) for j <= i. 2-D grid of 16x16 threads.
__global__ __launch_bounds__(256) void reverse_damp_kernel(const float* __restrict__ H32, int64_t K,
                                                           const double* __restrict__ lambda,
                                                           double* __restrict__ A) {
    const int64_t j = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x & 15);
    const int64_t i = static_cast<int64_t>(blockIdx.y) * 16 + (threadIdx.x >> 4);
    if (i >= K || j >= K || j > i) return;
    double v = static_cast<double>(H32[(K - 1 - i) * K + (K - 1 - j)]);
    if (i == j) v = ((v == 0.0) ? 1.0 : v) + *lambda;
    A[i * K + j] = v;
}

// Cholesky of the kPanel x kPanel diagonal block at (p, p), in LDS, by one
// wave (kPanel = 64 lanes, lane i owns row i), column by column: column k is
// its entries minus the products with the finished columns, then scaled by
// the pivot's square root. A pivot that is not positive records its 1-based
// column in *info (first failure only) and is replaced by 1 so the rest
// stays finite.
__global__ __launch_bounds__(kPanel) void potrf_diag_kernel(double* __restrict__ A, int64_t K,
                                                            int64_t p, int32_t* __restrict__ info) {
    static_assert(kPanel == 64, "one lane per row of the diagonal block");
    __shared__ double t[kPanel][kPanel + 1];
    const int i = threadIdx.x;
    for (int j = 0; j < kPanel; ++j) t[i][j] = (j <= i) ? A[(p + i) * K + p + j] : 0.0;
    __syncthreads();
    for (int k = 0; k < kPanel; ++k) {
        double v = 0.0;
        if (i >= k) {
            v = t[i][k];
            for (int m = 0; m < k; ++m) v = fma(-t[i][m], t[k][m], v);
        }
        if (i == k) {
            if (!(v > 0.0)) {
                if (*info == 0) *info = static_cast<int32_t>(p + k + 1);
                v = 1.0;
            }
            t[k][k] = sqrt(v);
        }
        __syncthreads();
        if (i > k) t[i][k] = v / t[k][k];
        __syncthreads();
    }
    for (int j = 0; j <= i; ++j) A[(p + i) * K + p + j] = t[i][j];
}

// Rows below the panel: x L11^T = a, one thread per row.
__global__ __launch_bounds__(256) void trsm_kernel(double* __restrict__ A, int64_t K, int64_t p) {
    __shared__ double L[kPanel][kPanel + 1];
    for (int e = threadIdx.x; e < kPanel * kPanel; e += 256) {
        const int i = e / kPanel, j = e % kPanel;
        L[i][j] = (j <= i) ? A[(p + i) * K + p + j] : 0.0;
    }
    __syncthreads();
    const int64_t i = p + kPanel + static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= K) return;
    double x[kPanel];
#pragma unroll
    for (int k = 0; k < kPanel; ++k) x[k] = A[i * K + p + k];
#pragma unroll
    for (int k = 0; k < kPanel; ++k) {
        double v = x[k];
#pragma unroll
        for (int m = 0; m < k; ++m) v -= x[m] * L[k][m];
        x[k] = v / L[k][k];
    }
#pragma unroll
    for (int k = 0; k < kPanel; ++k) A[i * K + p + k] = x[k];
}

// Trailing update A22 -= L21 L21^T on the lower triangle: 128x128 tiles
// enumerated over the lower triangle of tiles, 8x8 outputs per thread (two
// fp64 FMAs per LDS value read), the panel's kPanel columns in chunks of 16
// staged through LDS (transposed: k-major).
constexpr int kSyrk = 128;
__global__ __launch_bounds__(256) void syrk_kernel(double* __restrict__ A, int64_t K, int64_t p) {
    __shared__ double Pi[16][kSyrk + 2];
    __shared__ double Pj[16][kSyrk + 2];
    const int64_t q = p + kPanel;
    const int64_t x = blockIdx.x;
    int64_t bi = static_cast<int64_t>((sqrt(8.0 * static_cast<double>(x) + 1.0) - 1.0) * 0.5);
    while (bi * (bi + 1) / 2 > x) --bi;
    while ((bi + 1) * (bi + 2) / 2 <= x) ++bi;
    const int64_t bj = x - bi * (bi + 1) / 2;
    const int64_t r0 = q + bi * kSyrk, c0 = q + bj * kSyrk;
    const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
    // The tile's current values are loaded first, so their latency overlaps
    // the panel products that are subtracted from them.
    double acc[8][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int64_t row = r0 + ty + 16 * u;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            const int64_t col = c0 + tx + 16 * v;
            acc[u][v] = (row < K && col <= row) ? A[row * K + col] : 0.0;
        }
    }
    // Chunks of 16 panel columns staged through LDS, the next chunk loaded
    // into registers while this one is multiplied (one wave per SIMD: forcing
    // two spills and is slower here).
    constexpr int kPer = 16 * kSyrk / 256;
    double ni[kPer], nj[kPer];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int t = 0; t < kPer; ++t) {
            const int e = threadIdx.x + 256 * t;
            const int r = e >> 4, k = e & 15;
            ni[t] = (r0 + r < K) ? A[(r0 + r) * K + p + k0 + k] : 0.0;
            nj[t] = (c0 + r < K) ? A[(c0 + r) * K + p + k0 + k] : 0.0;
        }
    };
    fetch(0);
    for (int k0 = 0; k0 < kPanel; k0 += 16) {
#pragma unroll
        for (int t = 0; t < kPer; ++t) {
            const int e = threadIdx.x + 256 * t;
            Pi[e & 15][e >> 4] = ni[t];
            Pj[e & 15][e >> 4] = nj[t];
        }
        __syncthreads();
        if (k0 + 16 < kPanel) fetch(k0 + 16);
#pragma unroll 4
        for (int k = 0; k < 16; ++k) {
            double a[8], b[8];
            // rows ty + 16u, columns tx + 16v: consecutive lanes hold
            // consecutive columns, which are contiguous in A
#pragma unroll
            for (int u = 0; u < 8; ++u) { a[u] = -Pi[k][ty + 16 * u]; b[u] = Pj[k][tx + 16 * u]; }
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int v = 0; v < 8; ++v) acc[u][v] = fma(a[u], b[v], acc[u][v]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int64_t row = r0 + ty + 16 * u;
        if (row >= K) continue;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            const int64_t col = c0 + tx + 16 * v;
            if (col <= row) A[row * K + col] = acc[u][v];
        }
    }
}

// V_ij = R_ij / R_jj (i < j) into the upper triangle of A, where
// R_ij = L[K-1-i][K-1-j] (strictly lower part of A) and R_jj its diagonal.
__global__ __launch_bounds__(256) void make_v_kernel(double* __restrict__ A, int64_t K) {
    const int64_t j = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x & 15);
    const int64_t i = static_cast<int64_t>(blockIdx.y) * 16 + (threadIdx.x >> 4);
    if (i >= K || j >= K || i >= j) return;
    const int64_t ri = K - 1 - i, rj = K - 1 - j;
    A[i * K + j] = A[ri * K + rj] / A[rj * K + rj];
}

// Feed group [j0, j0 + kBlock)'s errors into every later column:
// P[c][r] (+)= sum_{k < kBlock} Dg[k][r] V[j0 + k][c] for c >= j0 + kBlock,
// r < M (P and Dg column-major over r). The first group writes P, later ones
// add to it. 128x128 output tiles, 8x8 per thread (two fp64 FMAs per LDS
// value read), the contraction in chunks of 16 staged through LDS.
constexpr int kUpd = 128;
__global__ __launch_bounds__(256, 2) void gptq_update_kernel(const double* __restrict__ Dg,
                                                          const double* __restrict__ A, int64_t K,
                                                          int64_t M, int64_t j0, int accumulate,
                                                          double* __restrict__ P) {
    __shared__ double sD[16][kUpd + 2];
    __shared__ double sV[16][kUpd + 2];
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kUpd;
    const int64_t c0 = j0 + kBlock + static_cast<int64_t>(blockIdx.y) * kUpd;
    const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
    // Later groups add to the feedback so far, loaded first so that its
    // latency overlaps the products.
    double acc[8][8];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const int64_t c = c0 + ty + 16 * v;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t r = r0 + tx + 16 * u;
            acc[u][v] = (accumulate && c < K && r < M) ? P[c * M + r] : 0.0;
        }
    }
    // Each chunk of 16 contraction steps is staged through LDS; the next
    // chunk's values are loaded into registers while this one is multiplied,
    // so the global latency hides behind the FMAs. Two waves per SIMD (the
    // launch bound) pay off here against a few spilled registers: 612 -> 457
    // us on a 4096-row, 14336-column layer's first group, bit-identical.
    constexpr int kPer = 16 * kUpd / 256;   // staged values per thread per operand
    double nd[kPer], nv[kPer];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int t = 0; t < kPer; ++t) {
            const int e = threadIdx.x + 256 * t;
            const int k = e / kUpd, c = e % kUpd;
            nd[t] = (r0 + c < M) ? Dg[static_cast<int64_t>(k0 + k) * M + r0 + c] : 0.0;
            nv[t] = (c0 + c < K) ? A[(j0 + k0 + k) * K + c0 + c] : 0.0;
        }
    };
    fetch(0);
    for (int k0 = 0; k0 < kBlock; k0 += 16) {
#pragma unroll
        for (int t = 0; t < kPer; ++t) {
            const int e = threadIdx.x + 256 * t;
            sD[e / kUpd][e % kUpd] = nd[t];
            sV[e / kUpd][e % kUpd] = nv[t];
        }
        __syncthreads();
        if (k0 + 16 < kBlock) fetch(k0 + 16);
#pragma unroll 4
        for (int k = 0; k < 16; ++k) {
            double a[8], b[8];
            // rows tx + 16u and columns ty + 16v: consecutive lanes hold
            // consecutive rows, which are contiguous in P
#pragma unroll
            for (int u = 0; u < 8; ++u) { a[u] = sD[k][tx + 16 * u]; b[u] = sV[k][ty + 16 * u]; }
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int v = 0; v < 8; ++v) acc[u][v] = fma(a[u], b[v], acc[u][v]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const int64_t c = c0 + ty + 16 * v;
        if (c >= K) continue;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t r = r0 + tx + 16 * u;
            if (r >= M) continue;
            P[c * M + r] = acc[u][v];
        }
    }
}

// Level value of a code in scale units (ternary codes are t + 1).
template <int GRID>
__device__ __forceinline__ double level_of(int code) {
    if constexpr (GRID == GSQ_GRID_TERNARY) return static_cast<double>(code - 1);
    else return static_cast<double>(2 * code - ((1 << GT<GRID>::BITS) - 1));
}

// Nearest code of target t with scale s, decided in fp32 like the
// round-to-nearest warm start: x = fp32(t) / s, u = (x + q_max) / 2, rint.
template <int GRID>
__device__ __forceinline__ int nearest_code(double t, float s) {
    constexpr float qmax = static_cast<float>(GT<GRID>::QMAX);
    const float x = (s > 0.0f) ? __fdiv_rn(static_cast<float>(t), s) : 0.0f;
    if constexpr (GRID == GSQ_GRID_TERNARY) {
        return static_cast<int>(fminf(fmaxf(rintf(x), -1.0f), 1.0f)) + 1;
    } else {
        constexpr float cmax = static_cast<float>((1 << GT<GRID>::BITS) - 1);
        const float u = __fmul_rn(__fadd_rn(x, qmax), 0.5f);
        return static_cast<int>(fminf(fmaxf(rintf(u), 0.0f), cmax));
    }
}

// One 128-column group. kSplit lanes per row round the row's columns in
// order from t_j = w_j + P_j + sum_{i<j in group} d_i V_ij, P_j the feedback
// of the earlier groups, and write the errors d to Dg. Lane s of a row sums
// the terms with i = s mod kSplit; a butterfly over the row's lanes adds the
// partial sums (each step adds the same two values in every lane, so all
// lanes hold the same t and take the same decision). A workgroup stages the
// group's strictly upper block of V (packed, 8128 doubles) in LDS once and
// then walks blocks of kRows rows, each with its w and w + P staged in LDS
// by coalesced loads; lane j mod kSplit keeps d_j, the only lane reading it.
constexpr int kSplit = 8;
constexpr int kGroupThreads = 256;
constexpr int kRows = kGroupThreads / kSplit;
template <int GRID, bool WBF16>
__global__ __launch_bounds__(kGroupThreads) void gptq_block_kernel(
    const void* __restrict__ W, int64_t M, int64_t K, int64_t j0, const double* __restrict__ A,
    const double* __restrict__ P, int has_p, const float* __restrict__ scales,
    double* __restrict__ Dg, uint8_t* __restrict__ codes) {
    // Padded by a row: the unrolled product loop may read past column j's
    // entries (the values are masked, the addresses stay inside).
    __shared__ double Vp[kBlock * (kBlock - 1) / 2 + kBlock];
    __shared__ double dl[kBlock][kRows];
    __shared__ double base[kBlock][kRows];   // w + P
    __shared__ float wv[kBlock][kRows];      // w (bf16 or fp32 values)
    __shared__ uint8_t cb[kRows][kBlock];    // the rows' codes
    const int tid = threadIdx.x;
    // Row i of the block is contiguous in A: threads read along it.
    for (int i = 0; i < kBlock - 1; ++i)
        for (int j = i + 1 + tid; j < kBlock; j += kGroupThreads)
            Vp[j * (j - 1) / 2 + i] = A[(j0 + i) * K + j0 + j];
    const int sub = tid % kSplit;
    const int rl = tid / kSplit;
    const int64_t nrb = (M + kRows - 1) / kRows;
    for (int64_t rb = blockIdx.x; rb < nrb; rb += gridDim.x) {
        const int64_t rbase = rb * kRows;
        // w along each row (contiguous in W), then P along each column
        // (contiguous over rows).
        for (int e = tid; e < kBlock * kRows; e += kGroupThreads) {
            const int rr = e / kBlock, j = e % kBlock;
            const int64_t r = rbase + rr;
            float w = 0.0f;
            if (r < M) {
                if constexpr (WBF16) w = bf16_lo(static_cast<const uint16_t*>(W)[r * K + j0 + j]);
                else w = static_cast<const float*>(W)[r * K + j0 + j];
            }
            wv[j][rr] = w;
        }
        __syncthreads();
        for (int e = tid; e < kBlock * kRows; e += kGroupThreads) {
            const int j = e / kRows, rr = e % kRows;
            const int64_t r = rbase + rr;
            double b = static_cast<double>(wv[j][rr]);
            if (has_p && r < M) b += P[(j0 + j) * M + r];
            base[j][rr] = b;
        }
        __syncthreads();
        const int64_t r = rbase + rl;
        if (r < M) {
            const float s = scales[r * (K / kBlock) + j0 / kBlock];
#pragma unroll 1
            for (int j = 0; j < kBlock; ++j) {
                const double* vj = Vp + j * (j - 1) / 2;
                // Fixed trip count (terms past j masked) so the LDS reads
                // are issued ahead of the two product chains.
                double p0 = 0.0, p1 = 0.0;
#pragma unroll
                for (int m = 0; m < kBlock / kSplit; m += 2) {
                    const int i0 = sub + m * kSplit, i1 = i0 + kSplit;
                    if (i0 < j) p0 = fma(dl[i0][rl], vj[i0], p0);
                    if (i1 < j) p1 = fma(dl[i1][rl], vj[i1], p1);
                }
                double part = p0 + p1;
#pragma unroll
                for (int m = 1; m < kSplit; m <<= 1) part += __shfl_xor(part, m, kSplit);
                const double t = base[j][rl] + part;
                const int code = nearest_code<GRID>(t, s);
                const double d = static_cast<double>(wv[j][rl]) - static_cast<double>(s) * level_of<GRID>(code);
                if (sub == (j % kSplit)) dl[j][rl] = d;
                if (sub == 0) {
                    Dg[static_cast<int64_t>(j) * M + r] = d;
                    cb[rl][j] = static_cast<uint8_t>(code);
                }
            }
        }
        __syncthreads();
        // The rows' codes, 16 bytes per thread.
        for (int e = tid; e < kRows * kBlock / 16; e += kGroupThreads) {
            const int rr = e / (kBlock / 16), q = e % (kBlock / 16);
            if (rbase + rr < M)
                reinterpret_cast<uint4*>(codes + (rbase + rr) * K + j0)[q] =
                    reinterpret_cast<const uint4*>(&cb[rr][0])[q];
        }
        __syncthreads();
    }
}

// Initial logits of the GPTQ codes (as the round-to-nearest warm start sets
// them): +init_logit on the code's level, 0 elsewhere; local shift: offset 0
// (index 2); ternary: mask +-init_logit by t != 0, sign by the sign of w.
template <int GRID, bool WBF16>
__global__ __launch_bounds__(256) void codes_to_logits_kernel(const uint8_t* __restrict__ codes,
                                                              const void* __restrict__ W, uint64_t mk,
                                                              float init_logit,
                                                              float* __restrict__ logits) {
    constexpr int L = GT<GRID>::L;
    const uint64_t i = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= mk) return;
    const int c = codes[i];
    if constexpr (GRID == GSQ_GRID_TERNARY) {
        float w;
        if constexpr (WBF16) w = bf16_lo(static_cast<const uint16_t*>(W)[i]);
        else w = static_cast<const float*>(W)[i];
        logits[i] = (c != 1) ? init_logit : -init_logit;
        logits[mk + i] = (w >= 0.0f) ? init_logit : -init_logit;
    } else if constexpr (GRID == GSQ_GRID_INT3_LOCAL) {
#pragma unroll
        for (int k = 0; k < L; ++k) logits[k * mk + i] = (k == 2) ? init_logit : 0.0f;
    } else {
#pragma unroll
        for (int k = 0; k < L; ++k) logits[k * mk + i] = (k == c) ? init_logit : 0.0f;
    }
}

inline unsigned cdivu(int64_t a, int64_t b) { return static_cast<unsigned>((a + b - 1) / b); }

template <int GRID, bool WBF16>
hipError_t gptq_columns(const LayerDesc& d, const void* W, const GptqWorkspace& ws, uint8_t* codes,
                        float* logits, float init_logit, hipStream_t st) {
    const int64_t M = d.rows, K = d.cols;
    for (int64_t j0 = 0; j0 < K; j0 += kBlock) {
        const unsigned nb = static_cast<unsigned>(std::min<int64_t>(256, (M + kRows - 1) / kRows));
        hipLaunchKernelGGL((gptq_block_kernel<GRID, WBF16>), dim3(nb), dim3(kGroupThreads), 0, st, W,
                           M, K, j0, ws.A, ws.P, j0 > 0 ? 1 : 0, ws.scales, ws.Dg, codes);
        const int64_t later = K - j0 - kBlock;
        if (later > 0) {
            hipLaunchKernelGGL(gptq_update_kernel, dim3(cdivu(M, kUpd), cdivu(later, kUpd)), dim3(256),
                               0, st, ws.Dg, ws.A, K, M, j0, j0 > 0 ? 1 : 0, ws.P);
        }
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL((codes_to_logits_kernel<GRID, WBF16>), dim3(cdivu(d.mk, 256)), dim3(256), 0,
                       st, codes, W, d.mk, init_logit, logits);
    return hipGetLastError();
}

}  // namespace

size_t gptq_workspace_bytes(int64_t rows, int64_t cols) {
    auto al = [](size_t b) { return (b + 255) / 256 * 256; };
    const size_t K = static_cast<size_t>(cols), M = static_cast<size_t>(rows);
    return al(K * K * sizeof(float)) + al(K * K * sizeof(double)) + al(M * K * sizeof(double)) +
           al(M * kBlock * sizeof(double)) + al(sizeof(double));
}

GptqWorkspace gptq_carve(void* base, int64_t rows, int64_t cols) {
    auto al = [](size_t b) { return (b + 255) / 256 * 256; };
    const size_t K = static_cast<size_t>(cols), M = static_cast<size_t>(rows);
    char* p = static_cast<char*>(base);
    GptqWorkspace ws{};
    ws.H32 = reinterpret_cast<float*>(p);  p += al(K * K * sizeof(float));
    ws.A = reinterpret_cast<double*>(p);   p += al(K * K * sizeof(double));
    ws.P = reinterpret_cast<double*>(p);   p += al(M * K * sizeof(double));
    ws.Dg = reinterpret_cast<double*>(p);  p += al(M * kBlock * sizeof(double));
    ws.lambda = reinterpret_cast<double*>(p);
    return ws;
}

hipError_t launch_gptq_factor(int64_t cols, float damp, const GptqWorkspace& ws, int32_t* info,
                              hipStream_t st) {
    const int64_t K = cols;
    hipLaunchKernelGGL(zero_info_kernel, dim3(1), dim3(1), 0, st, info);
    hipLaunchKernelGGL(damping_kernel, dim3(1), dim3(256), 0, st, ws.H32, K, damp, ws.lambda);
    hipLaunchKernelGGL(reverse_damp_kernel, dim3(cdivu(K, 16), cdivu(K, 16)), dim3(256), 0, st,
                       ws.H32, K, ws.lambda, ws.A);
    for (int64_t p = 0; p < K; p += kPanel) {
        hipLaunchKernelGGL(potrf_diag_kernel, dim3(1), dim3(kPanel), 0, st, ws.A, K, p, info);
        const int64_t rest = K - p - kPanel;
        if (rest > 0) {
            hipLaunchKernelGGL(trsm_kernel, dim3(cdivu(rest, 256)), dim3(256), 0, st, ws.A, K, p);
            const int64_t T = (rest + kSyrk - 1) / kSyrk;
            hipLaunchKernelGGL(syrk_kernel, dim3(static_cast<unsigned>(T * (T + 1) / 2)), dim3(256), 0,
                               st, ws.A, K, p);
        }
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(make_v_kernel, dim3(cdivu(K, 16), cdivu(K, 16)), dim3(256), 0, st, ws.A, K);
    return hipGetLastError();
}

hipError_t launch_gptq_columns(const LayerDesc& d, const void* W, const GptqWorkspace& ws,
                               uint8_t* codes, float* logits, float init_logit, hipStream_t st) {
#define GSQ_GPTQ(G)                                                                         \
    return d.w_bf16 ? gptq_columns<G, true>(d, W, ws, codes, logits, init_logit, st)        \
                    : gptq_columns<G, false>(d, W, ws, codes, logits, init_logit, st);
    switch (d.grid) {
        case GSQ_GRID_INT2: GSQ_GPTQ(GSQ_GRID_INT2)
        case GSQ_GRID_TERNARY: GSQ_GPTQ(GSQ_GRID_TERNARY)
        case GSQ_GRID_INT3_LOCAL: GSQ_GPTQ(GSQ_GRID_INT3_LOCAL)
        default: GSQ_GPTQ(GSQ_GRID_INT3)
    }
#undef GSQ_GPTQ
}

}  // namespace gsq
