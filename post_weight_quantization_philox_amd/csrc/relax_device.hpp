// Per-coordinate device code of the relaxed forward, backward and Lion
// (gfx950), shared by the stand-alone relax kernels (relax.hip) and the fused
// product + backward kernel (fused.hip), so both run the same arithmetic and
// give bit-identical results.
//
// Thread mapping: one thread owns N consecutive coordinates i0..i0+N-1 of the
// flattened layer (i0 a multiple of N), so every planar logit / momentum
// plane is read and written as one N*4-byte vector per thread. 128/N threads
// cover one scale group of 128 coordinates. GridT<>::N is 2 for every grid
// (8-byte vectors per plane stream faster than 16-byte ones on this access
// mix, and a thread holds half the registers of N = 4); the backward + Lion
// kernel instantiates the 2-bit and full 3-bit grids with N = 1 instead
// (relax.hip). With 5 logits (local shift) two coordinates are 10 noise
// words, which start at word 0 or 2 of a Philox block (NoiseStreamU); the
// other grids' words are whole blocks (NoiseStream).
#pragma once

#include <type_traits>

#include "gsq_internal.hpp"

namespace gsq {
namespace relax {

// No implicit contraction of a product into a following sum in this code: a
// separately rounded product and sum (v_k - w_hat with w_hat = num / sum, or
// s * w_hat - w) would otherwise be fused in some kernels and not in others,
// depending on how each instantiation is scheduled. Written-out fmaf calls
// are kept. Every kernel that runs these functions, in either layout, then
// gets the same bits.
#pragma clang fp contract(off)

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

// N = 1, 2 or 4 consecutive values as one access.
template <int N>
__device__ __forceinline__ void loadv(const float* p, float (&v)[N]) {
    if constexpr (N == 1) {
        v[0] = ld_nt(p);
    } else if constexpr (N == 4) {
        const f32x4_t x = ld_nt(reinterpret_cast<const f32x4_t*>(p));
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else {
        static_assert(N == 2, "1, 2 or 4 coordinates per thread");
        const f32x2_t x = ld_nt(reinterpret_cast<const f32x2_t*>(p));
        v[0] = x.x; v[1] = x.y;
    }
}

template <int N>
__device__ __forceinline__ void storev(float* p, const float (&v)[N]) {
    if constexpr (N == 1) {
        st_nt(v[0], p);
    } else if constexpr (N == 4) {
        st_nt(f32x4_t{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4_t*>(p));
    } else {
        st_nt(f32x2_t{v[0], v[1]}, reinterpret_cast<f32x2_t*>(p));
    }
}

template <int N, bool O32>
__device__ __forceinline__ void load_w(const void* W, bool bf16, Idx<O32> ix, float (&w)[N]) {
    if (bf16) {
        const uint16_t* p = ix.at(static_cast<const uint16_t*>(W));
        if constexpr (N == 1) {
            w[0] = bf16_lo(static_cast<uint32_t>(ld_nt(p)));
        } else if constexpr (N == 4) {
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
    if constexpr (N == 1) return ld_nt(ix.at(codes));
    else if constexpr (N == 4) return ld_nt(reinterpret_cast<const uint32_t*>(ix.at(codes)));
    else return ld_nt(reinterpret_cast<const uint16_t*>(ix.at(codes)));
}

// dW = out - w for the N coordinates, rounded to bf16 and stored as one vector.
template <int N, bool O32>
__device__ __forceinline__ void store_dw(uint16_t* dW, Idx<O32> ix, const float (&out)[N],
                                         const float (&w)[N]) {
    if constexpr (N == 1) {
        st_nt(static_cast<uint16_t>(pack_bf16x2(out[0] - w[0], 0.0f) & 0xFFFFu), ix.at(dW));
    } else if constexpr (N == 4) {
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

// Calls f(Ci<0>{}) .. f(Ci<N-1>{}) in order (N = 1, 2 or 4).
template <int N, typename F>
__device__ __forceinline__ void forN(F&& f) {
    f(Ci<0>{});
    if constexpr (N >= 2) f(Ci<1>{});
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
// One thread's share of a step, split so that a caller can issue the loads of
// a later group before the arithmetic of this one.
// ---------------------------------------------------------------------------

// Backward + Lion of the thread's N coordinates (logits l and momenta m in
// place): dL/dl from G (g), the old scale s and the step's regenerated noise,
// then one Lion update per logit. Each coordinate's gradient goes straight
// into its Lion update, so no gradient array stays live. Returns the
// thread's part of the scale gradient, sum_c g_c * w_hat_c (fma in
// coordinate order from 0); *what_last receives the last coordinate's w_hat.
template <int GRID, bool DBG, bool O32, int N = GridT<GRID>::N>
__device__ __forceinline__ float bwd_lion_coords(const float (&g)[N],
                                                 float (&l)[GridT<GRID>::L][N],
                                                 float (&m)[GridT<GRID>::L][N],
                                                 float s, uint32_t cw, uint64_t i0, uint32_t step,
                                                 uint32_t sid, Key key, TauK tk, LionK lkl,
                                                 float* __restrict__ gl_dbg, Idx<O32> ix,
                                                 uint64_t mk, float* what_last = nullptr) {
    constexpr int L = GridT<GRID>::L;
    float gsum = 0.0f;
    NoiseFor<L, N> ns(i0, step, sid, key);
    const float gs_tau = s * tk.invtau;
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
        if (what_last != nullptr) *what_last = r.what;
#pragma unroll
        for (int k = 0; k < L; ++k) {
            if constexpr (DBG) {
                if (gl_dbg != nullptr) ix.at(gl_dbg, mk, k)[c] = glc[k];
            }
            lion_update(l[k][c], m[k][c], glc[k], lkl);
        }
    });
    return gsum;
}

// Relaxed forward of the thread's N coordinates from logits l and scale s:
// out_c = s * w_hat_c.
template <int GRID, int N = GridT<GRID>::N>
__device__ __forceinline__ void fwd_coords(const float (&l)[GridT<GRID>::L][N],
                                           float s, uint32_t cw, uint64_t i0, uint32_t step,
                                           uint32_t sid, Key key, TauK tk,
                                           float (&out)[N]) {
    constexpr int L = GridT<GRID>::L;
    NoiseFor<L, N> ns(i0, step, sid, key);
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
}

}  // namespace relax
}  // namespace gsq
