// Elementwise and group-reduction kernels of the GSQ step (gfx950).
//
// Thread mapping shared by the forward and backward kernels: one thread owns
// N consecutive coordinates i0..i0+N-1 of the flattened layer (i0 = N * global
// thread id), so every planar logit / momentum plane is read and written as
// one N*4-byte vector per thread. 128/N threads cover one scale group of 128
// coordinates and reduce it with lane shuffles. N is 2 for every grid:
// 8-byte vectors per plane stream faster than 16-byte ones on this access
// mix, and a thread holds half the registers, so more waves are in flight.
// With 5 logits (local shift) two coordinates are 10 noise words, which start
// at word 0 or 2 of a Philox block (NoiseStreamU); the other grids' words are
// whole blocks (NoiseStream).
#include <type_traits>

#include "gsq_internal.hpp"

namespace gsq {

namespace {

constexpr int kThreads = 256;

template <int GRID> struct GridT;
// L logits per coordinate, q_max, code bits, and N coordinates per thread in
// the relax kernels.
template <> struct GridT<GSQ_GRID_INT2> { static constexpr int L = 4; static constexpr int QMAX = 3; static constexpr int BITS = 2; static constexpr int N = 2; };
template <> struct GridT<GSQ_GRID_TERNARY> { static constexpr int L = 2; static constexpr int QMAX = 1; static constexpr int BITS = 2; static constexpr int N = 2; };
template <> struct GridT<GSQ_GRID_INT3_LOCAL> { static constexpr int L = 5; static constexpr int QMAX = 7; static constexpr int BITS = 3; static constexpr int N = 2; };
template <> struct GridT<GSQ_GRID_INT3> { static constexpr int L = 8; static constexpr int QMAX = 7; static constexpr int BITS = 3; static constexpr int N = 2; };

// Element i of a tensor whose planes start at wave-uniform bases. With O32
// the byte offset of i fits 32 bits (checked by the launcher: rows*cols*4 <
// 2^32), so every access is a uniform 64-bit base plus one 32-bit per-thread
// offset (the global saddr form): one offset register serves every plane.
template <bool O32>
struct Idx {
    uint64_t i;
    template <typename T>
    __device__ __forceinline__ T* at(T* base, uint64_t plane_elems = 0, int plane = 0) const {
        T* b = base + plane_elems * plane;
        if constexpr (O32) {
            const uint32_t off = static_cast<uint32_t>(i) * static_cast<uint32_t>(sizeof(T));
            using C = typename std::conditional<std::is_const<T>::value, const char, char>::type;
            return reinterpret_cast<T*>(reinterpret_cast<C*>(b) + off);
        } else {
            return b + i;
        }
    }
};

template <bool O32>
__device__ __forceinline__ void load_w4(const void* W, bool bf16, Idx<O32> ix, float w[4]) {
    if (bf16) {
        const uint2 v = *reinterpret_cast<const uint2*>(ix.at(static_cast<const uint16_t*>(W)));
        w[0] = bf16_lo(v.x); w[1] = bf16_hi(v.x); w[2] = bf16_lo(v.y); w[3] = bf16_hi(v.y);
    } else {
        const float4 v = *reinterpret_cast<const float4*>(ix.at(static_cast<const float*>(W)));
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    }
}

// Streaming accesses. Every logit, momentum, G, W and dW element is touched
// once per launch, so the relax kernels load and store them nontemporally
// (no reuse to keep in the caches); on the fused pass's mix of nine read and
// eight write streams this is worth about an eighth of the HBM time.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <typename T>
__device__ __forceinline__ T ld_nt(const T* p) { return __builtin_nontemporal_load(p); }
template <typename T>
__device__ __forceinline__ void st_nt(T v, T* p) { __builtin_nontemporal_store(v, p); }

// N = 2 or 4 consecutive values as one vector access.
template <int N>
__device__ __forceinline__ void loadv(const float* p, float (&v)[N]) {
    if constexpr (N == 4) {
        const f32x4_t x = ld_nt(reinterpret_cast<const f32x4_t*>(p));
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else {
        static_assert(N == 2, "2 or 4 coordinates per thread");
        const f32x2_t x = ld_nt(reinterpret_cast<const f32x2_t*>(p));
        v[0] = x.x; v[1] = x.y;
    }
}

template <int N>
__device__ __forceinline__ void storev(float* p, const float (&v)[N]) {
    if constexpr (N == 4) {
        st_nt(f32x4_t{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4_t*>(p));
    } else {
        st_nt(f32x2_t{v[0], v[1]}, reinterpret_cast<f32x2_t*>(p));
    }
}

template <int N, bool O32>
__device__ __forceinline__ void load_w(const void* W, bool bf16, Idx<O32> ix, float (&w)[N]) {
    if (bf16) {
        const uint16_t* p = ix.at(static_cast<const uint16_t*>(W));
        if constexpr (N == 4) {
            const u32x2_t v = ld_nt(reinterpret_cast<const u32x2_t*>(p));
            w[0] = bf16_lo(v.x); w[1] = bf16_hi(v.x); w[2] = bf16_lo(v.y); w[3] = bf16_hi(v.y);
        } else {
            const uint32_t v = ld_nt(reinterpret_cast<const uint32_t*>(p));
            w[0] = bf16_lo(v); w[1] = bf16_hi(v);
        }
    } else {
        loadv<N>(ix.at(static_cast<const float*>(W)), w);
    }
}

// The N warm-start codes (one byte each) as one little-endian word.
template <int N, bool O32>
__device__ __forceinline__ uint32_t load_codes(const uint8_t* codes, Idx<O32> ix) {
    if constexpr (N == 4) return ld_nt(reinterpret_cast<const uint32_t*>(ix.at(codes)));
    else return ld_nt(reinterpret_cast<const uint16_t*>(ix.at(codes)));
}

// dW = out - w for the N coordinates, rounded to bf16 and stored as one vector.
template <int N, bool O32>
__device__ __forceinline__ void store_dw(uint16_t* dW, Idx<O32> ix, const float (&out)[N],
                                         const float (&w)[N]) {
    if constexpr (N == 4) {
        const u32x2_t o = {pack_bf16x2(out[0] - w[0], out[1] - w[1]),
                           pack_bf16x2(out[2] - w[2], out[3] - w[3])};
        st_nt(o, reinterpret_cast<u32x2_t*>(ix.at(dW)));
    } else {
        st_nt(pack_bf16x2(out[0] - w[0], out[1] - w[1]), reinterpret_cast<uint32_t*>(ix.at(dW)));
    }
}

__device__ __forceinline__ void load4(const float* p, float v[4]) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
}

__device__ __forceinline__ void store4(float* p, const float v[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

template <int C> using Ci = std::integral_constant<int, C>;

// Calls f(Ci<0>{}) .. f(Ci<N-1>{}) in order (N = 2 or 4).
template <int N, typename F>
__device__ __forceinline__ void forN(F&& f) {
    f(Ci<0>{}); f(Ci<1>{});
    if constexpr (N == 4) { f(Ci<2>{}); f(Ci<3>{}); }
}

// Candidate value (scale units) of local-shift logit k around code c0:
// 2*clamp(c0 + k - 2, 0, 7) - 7.
__device__ __forceinline__ float local_value(int c0, int k) {
    int c = c0 + k - 2;
    c = c < 0 ? 0 : (c > 7 ? 7 : c);
    return static_cast<float>(2 * c - 7);
}

// Relaxed state of one coordinate, shared by the forward and the backward.
template <int GRID>
struct Relaxed {
    static constexpr int L = GridT<GRID>::L;
    float e[L];   // unnormalised softmax weights 2^(y_k - y_max) (2-bit, local shift)
    float inv;    // 1 / sum_k e_k, so p_k = e_k * inv
    float v[L];   // candidate values in scale units
    float what;   // soft weight in scale units
    // ternary pieces: a = P(mask on), abar = 1 - a, sg = 2b - 1, bb = b(1-b)
    float a, abar, sg, bb;
};

template <int GRID>
__device__ __forceinline__ void relax_coord(const float (&l)[GridT<GRID>::L], const uint32_t* nz,
                                            int c0, TauK tk, Relaxed<GRID>& r) {
    constexpr int L = GridT<GRID>::L;
    if constexpr (GRID == GSQ_GRID_TERNARY) {
        // y = z*log2(e) with z = (l + eta*n)/tau; sigmoid(z) = 1/(1 + 2^-y).
        const float ym = __builtin_fmaf(l[0], tk.a, tk.b * logistic_b2(nz[0]));
        const float ys = __builtin_fmaf(l[1], tk.a, tk.b * logistic_b2(nz[1]));
        const float em = hw_exp2(-ym);
        const float es = hw_exp2(-ys);
        r.a = hw_rcp(1.0f + em);
        const float b = hw_rcp(1.0f + es);
        // 1 - a without cancellation: e/(1+e) when e <= 1, 1 - a otherwise
        // (this also keeps e = inf finite).
        r.abar = (em > 1.0f) ? (1.0f - r.a) : em * r.a;
        const float bbar = (es > 1.0f) ? (1.0f - b) : es * b;
        r.sg = 2.0f * b - 1.0f;
        r.bb = b * bbar;
        r.what = r.a * r.sg;
    } else {
        float y[L];
        float ymax = -INFINITY;
#pragma unroll
        for (int k = 0; k < L; ++k) {
            y[k] = __builtin_fmaf(l[k], tk.a, -tk.b * gumbel_t(nz[k]));
            ymax = fmaxf(ymax, y[k]);
        }
        float sum = 0.0f, num = 0.0f;
#pragma unroll
        for (int k = 0; k < L; ++k) {
            // Level value 2c - (2^b - 1) of the candidate code c.
            r.v[k] = (GRID == GSQ_GRID_INT2)   ? static_cast<float>(2 * k - 3)
                     : (GRID == GSQ_GRID_INT3) ? static_cast<float>(2 * k - 7)
                                               : local_value(c0, k);
            r.e[k] = hw_exp2(y[k] - ymax);
            sum += r.e[k];
            num = __builtin_fmaf(r.e[k], r.v[k], num);
        }
        r.inv = hw_rcp(sum);
        r.what = num * r.inv;
    }
}

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
    NoiseFor<L, N> ns(i0, step, sid, key);
    float out[N];
    forN<N>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        uint32_t nz[L];
        ns.template words<c>(nz);
        float lc[L];
#pragma unroll
        for (int k = 0; k < L; ++k) lc[k] = l[k][c];
        Relaxed<GRID> r;
        relax_coord<GRID>(lc, nz, static_cast<int>((cw >> (8 * c)) & 0xFF), tk, r);
        out[c] = s * r.what;
    });
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
    constexpr int N = GridT<GRID>::N;
    constexpr int P = 128 / N;   // lanes per scale group
    const uint64_t i0 = (static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x) * N;
    // Whole scale groups (P threads) are either in range or not, so the
    // shuffles below never read a lane that returned here.
    if (i0 >= mk) return;
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
    float gsum = 0.0f;
    {
        NoiseFor<L, N> ns(i0, step, sid, key);
        const float gs_tau = s * tk.invtau;
        // Each coordinate's gradient goes straight into its Lion update, so
        // no gradient array stays live (fewer registers, more waves in flight).
        forN<N>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            uint32_t nz[L];
            ns.template words<c>(nz);
            float lc[L];
#pragma unroll
            for (int k = 0; k < L; ++k) lc[k] = l[k][c];
            Relaxed<GRID> r;
            relax_coord<GRID>(lc, nz, static_cast<int>((cw >> (8 * c)) & 0xFF), tk, r);
            const float gsc = g[c] * gs_tau;
            float glc[L];
            if constexpr (GRID == GSQ_GRID_TERNARY) {
                glc[0] = gsc * (r.a * r.abar) * r.sg;
                glc[1] = gsc * (2.0f * r.a) * r.bb;
            } else {
                // p_k = e_k / sum: the normalisation rides on the common factor.
                const float gn = gsc * r.inv;
#pragma unroll
                for (int k = 0; k < L; ++k) glc[k] = gn * r.e[k] * (r.v[k] - r.what);
            }
            gsum = __builtin_fmaf(g[c], r.what, gsum);
#pragma unroll
            for (int k = 0; k < L; ++k) {
                if constexpr (DBG) ix.at(gl_dbg, mk, k)[c] = glc[k];
                lion_update(l[k][c], m[k][c], glc[k], lkl);
            }
        });
#pragma unroll
        for (int k = 0; k < L; ++k) {
            storev<N>(ix.at(logits, mk, k), l[k]);
            storev<N>(ix.at(mom, mk, k), m[k]);
        }
    }
    // Group sum, taken from the group's first lane so that every lane applies
    // the same Lion update to the shared scale.
    gsum = __shfl(group_sum<P>(gsum), group_lane0<P>(), 64);
    float sn = s, smn = scale_mom[grp];
    lion_update(sn, smn, gsum, lks);
    if ((threadIdx.x & (P - 1)) == 0) {
        scales[grp] = sn;
        scale_mom[grp] = smn;
        if constexpr (DBG) gs_dbg[grp] = gsum;
    }
    if constexpr (FWD_NEXT) {
        // W is only needed here; its load overlaps the next-step noise.
        float w[N];
        load_w<N>(W, WBF16, ix, w);
        NoiseFor<L, N> ns(i0, next_step, sid, key);
        float out[N];
        forN<N>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            uint32_t nz[L];
            ns.template words<c>(nz);
            float lc[L];
#pragma unroll
            for (int k = 0; k < L; ++k) lc[k] = l[k][c];
            Relaxed<GRID> r;
            relax_coord<GRID>(lc, nz, static_cast<int>((cw >> (8 * c)) & 0xFF), tk_next, r);
            out[c] = sn * r.what;
        });
        store_dw<N>(dW, ix, out, w);
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
    const unsigned nb = blocks_for(relax_threads(d));
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
