// Elementwise and group-reduction kernels of the GSQ step (gfx950).
//
// One thread owns N consecutive coordinates of the flattened layer
// (i0 = N * global thread id); the per-coordinate arithmetic and the thread
// mapping are described in relax_device.hpp.
#include <type_traits>

#include "relax_device.hpp"

namespace gsq {

namespace {

using namespace relax;

constexpr int kThreads = 256;

// Coordinates per thread in the backward + Lion kernel: one on the 2-bit and
// full 3-bit grids (a scale group then spans two waves; 4-byte accesses and
// twice the waves stream faster: 11.70 -> 10.81 ms on the 64-expert 2-bit
// batch, 5.57 -> 5.32 ms on 28672x8192 full 3-bit), the relax default
// otherwise (ternary would draw a whole Philox block per coordinate for its
// two words: 0.376 -> 0.450 ms on 4096x14336; local shift's five words per
// coordinate do not split into blocks per lane).
template <int GRID> struct BwdN {
    static constexpr int N = (GRID == GSQ_GRID_INT2 || GRID == GSQ_GRID_INT3) ? 1 : GridT<GRID>::N;
};

// ---------------------------------------------------------------------------
// Forward: dW = s*w_hat - W, bf16.
// ---------------------------------------------------------------------------
template <int GRID, bool WBF16, bool DBG, bool O32>
__global__ __launch_bounds__(kThreads) void relax_fwd_kernel(
    const float* __restrict__ logits, const float* __restrict__ scales,
    const uint8_t* __restrict__ codes, const void* __restrict__ W, uint64_t mk, uint32_t step,
    uint32_t sid, Key key, TauK tk, uint16_t* __restrict__ dW, float* __restrict__ w_soft_dbg) {
    constexpr int L = GridT<GRID>::L;
    constexpr int N = GridT<GRID>::N;
    const uint64_t i0 = (static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x) * N;
    if (i0 >= mk) return;
    const Idx<O32> ix{i0};
    float l[L][N];
#pragma unroll
    for (int k = 0; k < L; ++k) loadv<N>(ix.at(logits, mk, k), l[k]);
    float w[N];
    load_w<N>(W, WBF16, ix, w);
    const float s = scales[i0 >> 7];
    uint32_t cw = 0;
    if constexpr (GRID == GSQ_GRID_INT3_LOCAL) cw = load_codes<N>(codes, ix);
    float out[N];
    fwd_coords<GRID>(l, s, cw, i0, step, sid, key, tk, out);
    if constexpr (DBG) storev<N>(ix.at(w_soft_dbg), out);
    store_dw<N>(dW, ix, out, w);
}

// ---------------------------------------------------------------------------
// Backward + Lion, in place. G = dLoss/dW_soft. With FWD_NEXT the kernel then
// runs the relaxed forward of the next step on the updated logits and scale
// (still in registers): this equals a separate forward call, but the logits
// are read from HBM once per step instead of twice.
// ---------------------------------------------------------------------------
template <int GRID, bool DBG, bool FWD_NEXT, bool WBF16, bool O32>
__global__ __launch_bounds__(kThreads) void relax_bwd_lion_kernel(
    const float* __restrict__ G, float* __restrict__ logits, float* __restrict__ mom,
    float* __restrict__ scales, float* __restrict__ scale_mom, const uint8_t* __restrict__ codes,
    uint64_t mk, uint32_t step, uint32_t sid, Key key, TauK tk, LionK lkl, LionK lks,
    float* __restrict__ gl_dbg, float* __restrict__ gs_dbg, const void* __restrict__ W,
    uint32_t next_step, TauK tk_next, uint16_t* __restrict__ dW) {
    constexpr int L = GridT<GRID>::L;
    constexpr int N = BwdN<GRID>::N;
    constexpr int P = 128 / N;   // lanes per scale group
    uint64_t i0 = (static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x) * N;
    // Whole scale groups (P threads) are either in range or not. A group
    // spanning two waves meets its partner at a workgroup barrier, so an
    // out-of-range group works on the group before it and stores nothing.
    bool live = true;
    if constexpr (P > 64) {
        live = i0 < mk;
        if (!live) i0 -= 128;
    } else if (i0 >= mk) {
        return;
    }
    const Idx<O32> ix{i0};
    float g[N];
    loadv<N>(ix.at(G), g);
    float l[L][N], m[L][N];
#pragma unroll
    for (int k = 0; k < L; ++k) {
        loadv<N>(ix.at(logits, mk, k), l[k]);
        loadv<N>(ix.at(mom, mk, k), m[k]);
    }
    const uint64_t grp = i0 >> 7;
    const float s = scales[grp];
    uint32_t cw = 0;
    if constexpr (GRID == GSQ_GRID_INT3_LOCAL) cw = load_codes<N>(codes, ix);
    float what = 0.0f;
    // An out-of-range group recomputes its neighbour while that neighbour's
    // threads may already be storing: it writes no debug gradients either.
    float gsum = bwd_lion_coords<GRID, DBG, O32, N>(g, l, m, s, cw, i0, step, sid, key, tk, lkl,
                                                    live ? gl_dbg : nullptr, ix, mk, &what);
    if (live) {
#pragma unroll
        for (int k = 0; k < L; ++k) {
            storev<N>(ix.at(logits, mk, k), l[k]);
            storev<N>(ix.at(mom, mk, k), m[k]);
        }
    }
    // Group sum, taken from the group's first lane so that every lane applies
    // the same Lion update to the shared scale.
    if constexpr (P <= 64) {
        gsum = __shfl(group_sum<P>(gsum), group_lane0<P>(), 64);
    } else {
        // The same additions, in the same order, as with two coordinates per
        // lane (the fused product's layout): lanes 2i and 2i+1 first form
        // fma(g_{2i+1}, w_hat_{2i+1}, g_{2i} w_hat_{2i}), the pair's term;
        // then the butterfly over the 64 pair terms, whose first stage (pairs
        // 32 apart) joins the group's two waves through LDS and whose other
        // stages are lane shuffles 32, 16, 8, 4 and 2 apart.
        const int lane = threadIdx.x & 63;
        const float t_even = __shfl(gsum, lane & ~1, 64);
        const float g_odd = __shfl(g[0], lane | 1, 64);
        const float w_odd = __shfl(what, lane | 1, 64);
        float v = __builtin_fmaf(g_odd, w_odd, t_even);
        __shared__ float xs[kThreads];
        xs[threadIdx.x] = v;
        __syncthreads();
        v += xs[threadIdx.x ^ 64];
#pragma unroll
        for (int mm = 32; mm >= 2; mm >>= 1) v += __shfl_xor(v, mm, 64);
        gsum = __shfl(v, 0, 64);
    }
    float sn = s, smn = scale_mom[grp];
    lion_update(sn, smn, gsum, lks);
    if (live && (threadIdx.x & (P - 1)) == 0) {
        scales[grp] = sn;
        scale_mom[grp] = smn;
        if constexpr (DBG) gs_dbg[grp] = gsum;
    }
    if constexpr (FWD_NEXT) {
        // W is only needed here; its load overlaps the next-step noise.
        float w[N];
        load_w<N>(W, WBF16, ix, w);
        float out[N];
        fwd_coords<GRID, N>(l, sn, cw, i0, next_step, sid, key, tk_next, out);
        if (live) store_dw<N>(dW, ix, out, w);
    }
}

// ---------------------------------------------------------------------------
// Warm start by round-to-nearest.
// ---------------------------------------------------------------------------
template <int GRID, bool WBF16>
__global__ __launch_bounds__(kThreads) void init_rtn_kernel(const void* __restrict__ W, uint64_t mk,
                                                            float init_logit, float* __restrict__ scales,
                                                            uint8_t* __restrict__ codes,
                                                            float* __restrict__ logits) {
    constexpr int L = GridT<GRID>::L;
    constexpr float qmax = static_cast<float>(GridT<GRID>::QMAX);
    const uint64_t i0 = (static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x) * 4;
    if (i0 >= mk) return;
    float w[4];
    load_w4(W, WBF16, Idx<false>{i0}, w);
    float amax = fmaxf(fmaxf(fabsf(w[0]), fabsf(w[1])), fmaxf(fabsf(w[2]), fabsf(w[3])));
    amax = group_max<32>(amax);
    const float s = __fdiv_rn(amax, qmax);
    uint32_t cw = 0;
    float lg[L][4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float x = (s > 0.0f) ? __fdiv_rn(w[c], s) : 0.0f;
        int code;
        if constexpr (GRID == GSQ_GRID_TERNARY) {
            const float t = fminf(fmaxf(rintf(x), -1.0f), 1.0f);
            code = static_cast<int>(t) + 1;
            lg[0][c] = (code != 1) ? init_logit : -init_logit;
            lg[1][c] = (w[c] >= 0.0f) ? init_logit : -init_logit;
        } else {
            constexpr float cmax = static_cast<float>((1 << GridT<GRID>::BITS) - 1);
            const float u = __fmul_rn(__fadd_rn(x, qmax), 0.5f);
            code = static_cast<int>(fminf(fmaxf(rintf(u), 0.0f), cmax));
            if constexpr (GRID == GSQ_GRID_INT2 || GRID == GSQ_GRID_INT3) {
#pragma unroll
                for (int k = 0; k < L; ++k) lg[k][c] = (k == code) ? init_logit : 0.0f;
            } else {
#pragma unroll
                for (int k = 0; k < 5; ++k) lg[k][c] = (k == 2) ? init_logit : 0.0f;
            }
        }
        cw |= static_cast<uint32_t>(code) << (8 * c);
    }
#pragma unroll
    for (int k = 0; k < L; ++k) store4(logits + k * mk + i0, lg[k]);
    *reinterpret_cast<uint32_t*>(codes + i0) = cw;
    if ((threadIdx.x & 31) == 0) scales[i0 >> 7] = s;
}

// ---------------------------------------------------------------------------
// Harden + pack: one thread per 32 consecutive coordinates (a whole number of
// 32-bit words for 2 and 3 bits per code).
// ---------------------------------------------------------------------------
template <int GRID>
__global__ __launch_bounds__(kThreads) void harden_pack_kernel(
    const float* __restrict__ logits, const float* __restrict__ scales,
    const uint8_t* __restrict__ codes0, uint64_t mk, uint8_t* __restrict__ codes_out,
    uint32_t* __restrict__ packed, uint16_t* __restrict__ scales_f16) {
    constexpr int L = GridT<GRID>::L;
    constexpr int B = GridT<GRID>::BITS;
    const uint64_t t = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (scales_f16 != nullptr && t < (mk >> 7)) scales_f16[t] = f32_to_f16_bits(scales[t]);
    const uint64_t i0 = t * 32;
    if (i0 >= mk) return;
    uint32_t words[B];
#pragma unroll
    for (int j = 0; j < B; ++j) words[j] = 0;
    uint32_t cbytes[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        float l[L][4];
#pragma unroll
        for (int k = 0; k < L; ++k) load4(logits + k * mk + i0 + 4 * q, l[k]);
        uint32_t c0w = 0;
        if constexpr (GRID == GSQ_GRID_INT3_LOCAL)
            c0w = *reinterpret_cast<const uint32_t*>(codes0 + i0 + 4 * q);
        uint32_t cb = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            uint32_t code;
            if constexpr (GRID == GSQ_GRID_TERNARY) {
                code = (l[0][c] >= 0.0f) ? ((l[1][c] >= 0.0f) ? 2u : 0u) : 1u;
            } else {
                int best = 0;
                float bv = l[0][c];
#pragma unroll
                for (int k = 1; k < L; ++k)
                    if (l[k][c] > bv) { bv = l[k][c]; best = k; }
                if constexpr (GRID == GSQ_GRID_INT2 || GRID == GSQ_GRID_INT3) {
                    code = static_cast<uint32_t>(best);
                } else {
                    int cc = static_cast<int>((c0w >> (8 * c)) & 0xFF) + best - 2;
                    code = static_cast<uint32_t>(cc < 0 ? 0 : (cc > 7 ? 7 : cc));
                }
            }
            cb |= code << (8 * c);
            const int j = 4 * q + c;           // code index within the 32
            const int bit = B * j;
            words[bit >> 5] |= code << (bit & 31);
            if ((bit & 31) + B > 32) words[(bit >> 5) + 1] |= code >> (32 - (bit & 31));
        }
        cbytes[q] = cb;
    }
    if (codes_out != nullptr) {
        uint4* dst = reinterpret_cast<uint4*>(codes_out + i0);
        dst[0] = make_uint4(cbytes[0], cbytes[1], cbytes[2], cbytes[3]);
        dst[1] = make_uint4(cbytes[4], cbytes[5], cbytes[6], cbytes[7]);
    }
    if (packed != nullptr) {
#pragma unroll
        for (int j = 0; j < B; ++j) packed[t * B + j] = words[j];
    }
}

__global__ __launch_bounds__(kThreads) void noise_dump_kernel(uint64_t first, uint64_t count,
                                                              uint32_t step, uint32_t sid, Key key,
                                                              uint32_t* __restrict__ out) {
    const uint64_t j = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (j >= count) return;
    const uint64_t e = first + j;
    uint32_t w[4];
    philox_block(e >> 2, step, sid, key, w);
    const uint32_t q = static_cast<uint32_t>(e & 3);
    out[j] = q == 0 ? w[0] : (q == 1 ? w[1] : (q == 2 ? w[2] : w[3]));
}

inline unsigned blocks_for(uint64_t threads) {
    return static_cast<unsigned>((threads + kThreads - 1) / kThreads);
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
#define GSQ_LAUNCH(kern, nblk, st, ...)                                          \
    do {                                                                         \
        hipLaunchKernelGGL((kern), dim3(nblk), dim3(kThreads), 0, (st), __VA_ARGS__); \
    } while (0)

hipError_t launch_init_rtn(const LayerDesc& d, const void* W, float* scales, uint8_t* codes,
                           float* logits, float init_logit, hipStream_t st) {
    const unsigned nb = blocks_for(d.mk / 4);
#define GSQ_INIT(G)                                                                          \
    if (d.w_bf16) GSQ_LAUNCH((init_rtn_kernel<G, true>), nb, st, W, d.mk, init_logit, scales, codes, logits); \
    else GSQ_LAUNCH((init_rtn_kernel<G, false>), nb, st, W, d.mk, init_logit, scales, codes, logits);
    switch (d.grid) {
        case GSQ_GRID_INT2: GSQ_INIT(GSQ_GRID_INT2); break;
        case GSQ_GRID_INT3: GSQ_INIT(GSQ_GRID_INT3); break;
        case GSQ_GRID_TERNARY: GSQ_INIT(GSQ_GRID_TERNARY); break;
        default: GSQ_INIT(GSQ_GRID_INT3_LOCAL); break;
    }
#undef GSQ_INIT
    return hipGetLastError();
}

// Offsets fit 32 bits when every byte offset into an fp32 [rows][cols]
// plane does.
inline bool off32(const LayerDesc& d) { return d.mk * 4 <= 0xFFFFFFF0ull; }

// Threads of the relax kernels: one per N coordinates.
inline uint64_t bwd_threads(const LayerDesc& d) {
    switch (d.grid) {
        case GSQ_GRID_INT2: return d.mk / BwdN<GSQ_GRID_INT2>::N;
        case GSQ_GRID_INT3: return d.mk / BwdN<GSQ_GRID_INT3>::N;
        case GSQ_GRID_TERNARY: return d.mk / BwdN<GSQ_GRID_TERNARY>::N;
        default: return d.mk / BwdN<GSQ_GRID_INT3_LOCAL>::N;
    }
}

inline uint64_t relax_threads(const LayerDesc& d) {
    switch (d.grid) {
        case GSQ_GRID_INT2: return d.mk / GridT<GSQ_GRID_INT2>::N;
        case GSQ_GRID_INT3: return d.mk / GridT<GSQ_GRID_INT3>::N;
        case GSQ_GRID_TERNARY: return d.mk / GridT<GSQ_GRID_TERNARY>::N;
        default: return d.mk / GridT<GSQ_GRID_INT3_LOCAL>::N;
    }
}

hipError_t launch_relax_fwd(const LayerDesc& d, const float* logits, const float* scales,
                            const uint8_t* codes, const void* W, uint32_t step, TauK tk,
                            uint16_t* dW, float* w_soft_dbg, hipStream_t st) {
    const unsigned nb = blocks_for(relax_threads(d));
    const bool o32 = off32(d);
#define GSQ_FWD(G, WB, DB, O) \
    GSQ_LAUNCH((relax_fwd_kernel<G, WB, DB, O>), nb, st, logits, scales, codes, W, d.mk, step, d.sid, d.key, tk, dW, w_soft_dbg)
#define GSQ_FWD_O(G, WB, DB) if (o32) GSQ_FWD(G, WB, DB, true); else GSQ_FWD(G, WB, DB, false);
#define GSQ_FWD_G(G)                                       \
    if (d.w_bf16) {                                        \
        if (w_soft_dbg) { GSQ_FWD_O(G, true, true); } else { GSQ_FWD_O(G, true, false); }   \
    } else {                                               \
        if (w_soft_dbg) { GSQ_FWD_O(G, false, true); } else { GSQ_FWD_O(G, false, false); } \
    }
    switch (d.grid) {
        case GSQ_GRID_INT2: GSQ_FWD_G(GSQ_GRID_INT2); break;
        case GSQ_GRID_INT3: GSQ_FWD_G(GSQ_GRID_INT3); break;
        case GSQ_GRID_TERNARY: GSQ_FWD_G(GSQ_GRID_TERNARY); break;
        default: GSQ_FWD_G(GSQ_GRID_INT3_LOCAL); break;
    }
#undef GSQ_FWD_G
#undef GSQ_FWD_O
#undef GSQ_FWD
    return hipGetLastError();
}

hipError_t launch_relax_bwd_lion(const LayerDesc& d, const float* G, float* logits, float* mom,
                                 float* scales, float* scale_mom, const uint8_t* codes,
                                 uint32_t step, TauK tk, LionK lkl, LionK lks,
                                 float* gl_dbg, float* gs_dbg, const void* W, uint32_t next_step,
                                 TauK tk_next, uint16_t* dW, hipStream_t st) {
    const unsigned nb = blocks_for(bwd_threads(d));
    const bool dbg = gl_dbg != nullptr || gs_dbg != nullptr;
    const bool fwd = dW != nullptr;
    const bool o32 = off32(d);
#define GSQ_BWD(G_, DB, FW, WB, O) \
    GSQ_LAUNCH((relax_bwd_lion_kernel<G_, DB, FW, WB, O>), nb, st, G, logits, mom, scales, scale_mom, codes, d.mk, step, d.sid, d.key, tk, lkl, lks, gl_dbg, gs_dbg, W, next_step, tk_next, dW)
#define GSQ_BWD_O(G_, DB, FW, WB) if (o32) GSQ_BWD(G_, DB, FW, WB, true); else GSQ_BWD(G_, DB, FW, WB, false);
#define GSQ_BWD_G(G_)                                                            \
    if (!fwd) { if (dbg) { GSQ_BWD_O(G_, true, false, true); } else { GSQ_BWD_O(G_, false, false, true); } } \
    else if (d.w_bf16) { GSQ_BWD_O(G_, false, true, true); }                     \
    else { GSQ_BWD_O(G_, false, true, false); }
    switch (d.grid) {
        case GSQ_GRID_INT2: GSQ_BWD_G(GSQ_GRID_INT2); break;
        case GSQ_GRID_INT3: GSQ_BWD_G(GSQ_GRID_INT3); break;
        case GSQ_GRID_TERNARY: GSQ_BWD_G(GSQ_GRID_TERNARY); break;
        default: GSQ_BWD_G(GSQ_GRID_INT3_LOCAL); break;
    }
#undef GSQ_BWD_G
#undef GSQ_BWD_O
#undef GSQ_BWD
    return hipGetLastError();
}

hipError_t launch_harden_pack(const LayerDesc& d, const float* logits, const float* scales,
                              const uint8_t* codes, uint8_t* codes_out, uint32_t* packed,
                              uint16_t* scales_f16, hipStream_t st) {
    const unsigned nb = blocks_for(d.mk / 32);
    switch (d.grid) {
        case GSQ_GRID_INT2:
            GSQ_LAUNCH((harden_pack_kernel<GSQ_GRID_INT2>), nb, st, logits, scales, codes, d.mk, codes_out, packed, scales_f16);
            break;
        case GSQ_GRID_INT3:
            GSQ_LAUNCH((harden_pack_kernel<GSQ_GRID_INT3>), nb, st, logits, scales, codes, d.mk, codes_out, packed, scales_f16);
            break;
        case GSQ_GRID_TERNARY:
            GSQ_LAUNCH((harden_pack_kernel<GSQ_GRID_TERNARY>), nb, st, logits, scales, codes, d.mk, codes_out, packed, scales_f16);
            break;
        default:
            GSQ_LAUNCH((harden_pack_kernel<GSQ_GRID_INT3_LOCAL>), nb, st, logits, scales, codes, d.mk, codes_out, packed, scales_f16);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_noise_dump(const LayerDesc& d, uint32_t step, uint64_t first, uint64_t count,
                             uint32_t* out, hipStream_t st) {
    if (count == 0) return hipSuccess;
    GSQ_LAUNCH(noise_dump_kernel, blocks_for(count), st, first, count, step, d.sid, d.key, out);
    return hipGetLastError();
}

}  // namespace gsq
