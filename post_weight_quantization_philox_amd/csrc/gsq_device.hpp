// Device helpers shared by the GSQ kernels (gfx950, wave64).
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gsq {

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11), written from the
// published round function: the products M0*c0 and M1*c2 (32x32 -> 64 bit),
// new counter (hi1^c1^k0, lo1, hi0^c3^k1, lo0), key bumped by the Weyl
// constants between rounds. The key is wave-uniform, so its schedule stays in
// scalar registers; each round costs two v_mad_u64_u32 and two three-input xors.
// ---------------------------------------------------------------------------
constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

struct Key { uint32_t k0, k1; };

// a ^ b ^ c in one VALU instruction: gfx950's three-input bitwise op with
// truth table 0x96 (the compiler emits two v_xor_b32 for the plain expression).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ void philox_block(uint64_t blk, uint32_t step, uint32_t sid,
                                             Key key, uint32_t out[4]) {
    uint32_t c0 = static_cast<uint32_t>(blk);
    uint32_t c1 = static_cast<uint32_t>(blk >> 32);
    uint32_t c2 = step;
    uint32_t c3 = sid;
    uint32_t k0 = key.k0, k1 = key.k1;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = static_cast<uint64_t>(kPhiloxM0) * c0;
        const uint64_t p1 = static_cast<uint64_t>(kPhiloxM1) * c2;
        const uint32_t n0 = xor3(static_cast<uint32_t>(p1 >> 32), c1, k0);
        const uint32_t n2 = xor3(static_cast<uint32_t>(p0 >> 32), c3, k1);
        c1 = static_cast<uint32_t>(p1);
        c3 = static_cast<uint32_t>(p0);
        c0 = n0;
        c2 = n2;
        k0 += kPhiloxW0;
        k1 += kPhiloxW1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

// Noise of the N consecutive coordinates i0..i0+N-1 of a grid with L logits
// (N*L a multiple of 4, i0 a multiple of N): stream elements e = i*L + k, i.e.
// the N*L/4 whole Philox blocks starting at block i0*L/4. Coordinate C
// (0..N-1) takes words C*L .. C*L + L - 1 of that block sequence. Blocks are
// generated on demand, in order, with at most two live (the last two), so the
// words of all N coordinates never occupy registers at once. Which blocks are
// new for coordinate C is known at compile time.
template <int L, int N>
struct NoiseStream {
    static_assert((L * N) % 4 == 0, "coordinates per thread must cover whole Philox blocks");
    uint64_t b0;
    uint32_t step, sid;
    Key key;
    uint32_t cur[4], nxt[4];   // after words<C>(): blocks hi(C) - 1 and hi(C)

    __device__ __forceinline__ NoiseStream(uint64_t i0, uint32_t step_, uint32_t sid_, Key key_)
        : b0((i0 * L) >> 2), step(step_), sid(sid_), key(key_) {}

    // Calls must come in order C = 0, 1, ..., N - 1.
    template <int C>
    __device__ __forceinline__ void words(uint32_t (&w)[L]) {
        constexpr int first = C * L;
        constexpr int hi = (first + L - 1) / 4;          // last block this coordinate uses
        constexpr int done = C == 0 ? -1 : (first - 1) / 4;   // last block generated before
#pragma unroll
        for (int b = done + 1; b <= hi; ++b) {
#pragma unroll
            for (int j = 0; j < 4; ++j) cur[j] = nxt[j];
            philox_block(b0 + b, step, sid, key, nxt);
        }
#pragma unroll
        for (int j = 0; j < L; ++j) {
            const int word = first + j;
            w[j] = (word / 4 == hi) ? nxt[word & 3] : cur[word & 3];
        }
    }
};

// The same noise when N*L is 2 mod 4 (i0 a multiple of N, so i0*L is even):
// the thread's N*L words start at word 0 or 2 of block i0*L/4 ("shifted").
// Blocks are generated on demand as in NoiseStream, at most two live; both
// placements of coordinate C's words lie in the same two blocks, and each
// word is selected from its block for the thread's placement.
template <int L, int N>
struct NoiseStreamU {
    static_assert((L * N) % 4 == 2, "for N*L = 2 mod 4");
    uint64_t b0;
    bool shifted;
    uint32_t step, sid;
    Key key;
    uint32_t cur[4], nxt[4];

    __device__ __forceinline__ NoiseStreamU(uint64_t i0, uint32_t step_, uint32_t sid_, Key key_)
        : b0((i0 * L) >> 2), shifted(((i0 * L) & 3u) != 0), step(step_), sid(sid_), key(key_) {}

    template <int C>
    __device__ __forceinline__ void words(uint32_t (&w)[L]) {
        constexpr int first = C * L;
        constexpr int hi = (first + L - 1 + 2) / 4;            // last block (shifted)
        constexpr int done = C == 0 ? -1 : (first - 1 + 2) / 4;  // last block generated before
        static_assert(first / 4 >= hi - 1, "a coordinate's words span at most two blocks");
#pragma unroll
        for (int b = done + 1; b <= hi; ++b) {
#pragma unroll
            for (int j = 0; j < 4; ++j) cur[j] = nxt[j];
            philox_block(b0 + b, step, sid, key, nxt);
        }
#pragma unroll
        for (int j = 0; j < L; ++j) {
            const int u = first + j, v = u + 2;
            const uint32_t a = (u / 4 == hi) ? nxt[u & 3] : cur[u & 3];
            const uint32_t c = (v / 4 == hi) ? nxt[v & 3] : cur[v & 3];
            w[j] = shifted ? c : a;
        }
    }
};

template <int L, int N>
using NoiseFor = typename std::conditional<(L * N) % 4 == 0, NoiseStream<L, N>,
                                           NoiseStreamU<L, N>>::type;

// Uniform in (0,1): top 24 bits forced odd, times 2^-24 (exact in fp32).
__device__ __forceinline__ float uniform24(uint32_t x) {
    return static_cast<float>((x >> 8) | 1u) * 0x1p-24f;
}

// Hardware base-2 logarithm and exponential (v_log_f32 / v_exp_f32). Their
// arguments here are never denormal: uniforms are >= 2^-24 and -log2(u) is
// >= 8.6e-8.
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Gumbel noise in base-2 units up to a constant: a standard Gumbel g equals
// -ln(-ln u) = -ln2 * (log2(-log2 u) + log2(ln 2)), so g*log2(e) =
// -log2(-log2 u) - log2(ln 2). The constant is the same for every logit of a
// coordinate and cancels in the softmax, so kernels use t = log2(-log2 u) and
// form y_k = (l_k*log2e - eta*t_k)/tau.
__device__ __forceinline__ float gumbel_t(uint32_t word) {
    return hw_log2(-hw_log2(uniform24(word)));
}

// Standard logistic noise in base-2 units: n*log2(e) = log2(u) - log2(1-u)
// (1-u is exact in fp32 for the 24-bit uniforms).
__device__ __forceinline__ float logistic_b2(uint32_t word) {
    const float u = uniform24(word);
    return hw_log2(u) - hw_log2(1.0f - u);
}

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// Conversions
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    _Float16 h = static_cast<_Float16>(x);
    return __builtin_bit_cast(uint16_t, h);
}

// ---------------------------------------------------------------------------
// Reductions within the P lanes (P = 32 or 64) that share a scale group: with
// 4 coordinates per thread the two halves of a wave hold two groups, with 2
// the whole wave holds one. Butterfly: every lane ends with the full result;
// callers let one fixed lane write it, so the stored value is deterministic.
// ---------------------------------------------------------------------------
template <int P>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(P == 32 || P == 64, "a scale group spans half a wave or a whole wave");
#pragma unroll
    for (int m = P / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

template <int P>
__device__ __forceinline__ float group_max(float v) {
    static_assert(P == 32 || P == 64, "a scale group spans half a wave or a whole wave");
#pragma unroll
    for (int m = P / 2; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

// First lane of the P-lane group that holds this lane.
template <int P>
__device__ __forceinline__ int group_lane0() { return static_cast<int>(threadIdx.x) & (64 - P); }

// Lion on one fp32 parameter (Chen et al. 2023). The sign is taken on
// c = fma(beta1, m, fp32((1-beta1)*g)); theta <- theta - lr*sign(c) - lr*wd*theta;
// m = fma(beta2, m, fp32((1-beta2)*g)).
struct LionK {
    float lr, b1, omb1, b2, omb2, nlrwd;   // nlrwd = -lr * wd (fp32)
};

// theta - lr*sign(c) is formed as theta - copysign(lr, c) (v_bfi_b32 on the
// sign bit), zero when c == 0; the decay term is then one fma with
// -lr*wd, which leaves the value unchanged when wd = 0.
__device__ __forceinline__ void lion_update(float& theta, float& m, float g, const LionK& k) {
    const float c = __builtin_fmaf(k.b1, m, __fmul_rn(k.omb1, g));
    const float step = __uint_as_float((__float_as_uint(k.lr) & 0x7FFFFFFFu) |
                                       (__float_as_uint(c) & 0x80000000u));
    const float moved = __fsub_rn(theta, c != 0.0f ? step : 0.0f);
    theta = __builtin_fmaf(k.nlrwd, theta, moved);
    m = __builtin_fmaf(k.b2, m, __fmul_rn(k.omb2, g));
}

}  // namespace gsq
