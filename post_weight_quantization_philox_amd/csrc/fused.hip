// The second reconstruction product fused with the relaxed backward, Lion and
// the next step's forward (gfx950).
//
// G = 2 R^T X, the gradient of the output reconstruction objective with
// respect to the soft weights (agihunt.info summary, method paragraph), is
// consumed by the backward and nothing else. For experts that each see a few
// hundred tokens the product is a short contraction with a large output: as a
// separate kernel it writes G (4 bytes per weight) at the memory system's
// rate and the backward reads it back. Here each workgroup forms one 128x128
// tile of G on the matrix cores and runs backward + Lion + next forward on it
// at once, so G never reaches HBM.
//
// Every G value is the same MFMA chain, in the same k order, as in the
// stand-alone product (gemm.hip): v_mfma_f32_16x16x32_bf16 over 32-wide
// slices in order, lane quarter q holding k = 32 s + 8 q .. + 7 of slice s.
// So G, and everything computed from it, is bit-identical to the two-kernel
// path.
//
// Workgroup: 4 waves over a tile of 32 rows x 512 columns; wave w owns
// columns 128w .. 128w+127 (one scale group per row) of all 32 rows (2 x 8
// blocks of 16x16, 64 accumulators per lane). Fragments come straight from
// global memory (R^T and X^T are small next to the state and stay in the
// caches). A wave's accumulators pass through its own LDS slab (32 x 128 fp32,
// rows padded to 132 floats so the four lane quarters' stores land 16 banks
// apart) into the relax
// layout: per row, lane l owns columns 2l and 2l+1, so one row of the wave's
// block is one scale group over the whole wave, as in the stand-alone
// backward (relax_device.hpp). The four waves walk the same rows, so a
// workgroup streams 2 KiB of each plane per row and neighbouring workgroups
// (the next 512 columns) continue it. Rows of inputs are loaded a few rows
// ahead of their arithmetic. 68 KiB of LDS per workgroup: two workgroups
// (eight waves) per compute unit.
#include <type_traits>

#include "relax_device.hpp"

namespace gsq {

namespace {

using namespace relax;

constexpr int kFT = 256;                 // threads per workgroup
constexpr int kTileRows = 32;
constexpr int kGroup = 128;              // columns per wave: one scale group
constexpr int kTileCols = 4 * kGroup;
constexpr int kSlabStride = kGroup + 4;  // floats per slab row
constexpr int kFusedMaxExperts = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Experts of one launch: expert e (expert0 + e of the batch) owns rows
// [e*rpe, (e+1)*rpe) of the layer, R^T block e at element rpe*tok[e]
// ([rpe][n_e]), X^T block e at element cols*tok[e] ([cols][n_e]); its
// workgroups are [wg0[e], wg0[e+1]), tiles_i row tiles by tiles_j column
// tiles, column tiles fastest.
struct FusedBatch {
    int n, rpe, cols, expert0, tiles_i, tiles_j;
    const uint16_t* RT;
    const uint16_t* XT;
    int tok[kFusedMaxExperts + 1];
    int wg0[kFusedMaxExperts + 1];
    // Workgroup 0 first sums fin_n loss partials into *fin_loss (fixed order,
    // fp64), as the stand-alone second product does.
    const float* fin_partials;
    int fin_n;
    double* fin_loss;
};

struct RelaxArgs {
    float* logits;
    float* mom;
    float* scales;
    float* scale_mom;
    const uint8_t* codes;
    const void* W;
    uint16_t* dW;
    uint64_t mk;
    uint32_t step, sid, next_step;
    Key key;
    TauK tk, tk_next;
    LionK lkl, lks;
};

// One row's worth of one thread's step inputs (two coordinates).
template <int GRID>
struct RowIn {
    float l[GridT<GRID>::L][GridT<GRID>::N];
    float m[GridT<GRID>::L][GridT<GRID>::N];
    float w[GridT<GRID>::N];
    uint32_t cw;
    float s, sm;
};

// Rows whose inputs are in flight per wave: a ring of ring_rows(L) rows,
// the next ones loading while one is computed; fewer rows for the grids with
// more logits per weight, whose rows take more registers.
constexpr int ring_rows(int L) { return L <= 2 ? 6 : (L <= 4 ? 4 : 2); }

template <int GRID, bool FWD_NEXT, bool WBF16, bool O32>
__global__ __launch_bounds__(kFT, 2) void recon_relax_kernel(FusedBatch fb, RelaxArgs ra) {
    constexpr int L = GridT<GRID>::L;
    constexpr int N = GridT<GRID>::N;
    constexpr int kRing = ring_rows(L);
    static_assert(N == 2, "one tile row is one scale group over the 64 lanes");
    __shared__ float slab[4 * 32 * kSlabStride];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    if (fb.fin_loss != nullptr && blockIdx.x == 0) {
        double* fred = reinterpret_cast<double*>(slab);
        double fs = 0.0;
        for (int i = tid; i < fb.fin_n; i += kFT) fs += static_cast<double>(fb.fin_partials[i]);
        fred[tid] = fs;
        __syncthreads();
        for (int w = kFT / 2; w >= 1; w >>= 1) {
            if (tid < w) fred[tid] += fred[tid + w];
            __syncthreads();
        }
        if (tid == 0) *fb.fin_loss = fred[0];
        __syncthreads();
    }

    // Tile of this workgroup; consecutive logical indices share an XCD (the
    // dispatcher deals workgroups round-robin over the 8 XCDs).
    const int nwg = gridDim.x;
    const int wg = blockIdx.x;
    const int logical = (nwg & 7) == 0 ? (wg & 7) * (nwg >> 3) + (wg >> 3) : wg;
    // The expert: how many later starts lie at or below `logical` (wg0 is
    // nondecreasing), unrolled so the table is read with wide scalar loads.
    int e = 0;
#pragma unroll
    for (int k = 1; k < kFusedMaxExperts; ++k) e += (k < fb.n && logical >= fb.wg0[k]) ? 1 : 0;
    e = __builtin_amdgcn_readfirstlane(e);   // uniform: keeps the addressing scalar
    const int local = logical - fb.wg0[e];
    const int ti = local / fb.tiles_j, tj = local % fb.tiles_j;
    const int ne = fb.tok[e + 1] - fb.tok[e];
    const int row0 = ti * kTileRows;              // first row within the expert
    const int col0 = tj * kTileCols + kGroup * wave;
    // A wave past the layer's last column has nothing to do (no workgroup
    // barrier follows).
    if (col0 >= fb.cols) return;
    const int frow = lane & 15, fq = lane >> 4;

    // Backward + Lion (+ next forward), one row (scale group) at a time.
    const int nrows = min(kTileRows, fb.rpe - row0);
    const uint64_t grow0 = static_cast<uint64_t>(fb.expert0 + e) * fb.rpe + row0;
    const uint64_t cols = static_cast<uint64_t>(fb.cols);
    const uint64_t mk = ra.mk;
    auto coord0 = [&](int j) { return (grow0 + j) * cols + col0 + 2 * lane; };
    auto load_in = [&](int j, RowIn<GRID>& in) {
        const uint64_t i0 = coord0(j);
        const Idx<O32> ix{i0};
#pragma unroll
        for (int k = 0; k < L; ++k) {
            loadv<N>(ix.at(ra.logits, mk, k), in.l[k]);
            loadv<N>(ix.at(ra.mom, mk, k), in.m[k]);
        }
        in.s = ra.scales[i0 >> 7];
        in.sm = ra.scale_mom[i0 >> 7];
        in.cw = 0;
        if constexpr (GRID == GSQ_GRID_INT3_LOCAL) in.cw = load_codes<N>(ra.codes, ix);
        if constexpr (FWD_NEXT) load_w<N>(ra.W, WBF16, ix, in.w);
    };
    // Rows of this wave are fetched kRing - 1 ahead; the first ones before
    // the matrix-core phase, whose time then hides their latency.
    RowIn<GRID> ring[kRing];
#pragma unroll
    for (int q = 0; q < kRing - 1; ++q)
        if (q < nrows) load_in(q, ring[q]);

    f32x4 acc[2][8];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[a][b][r] = 0.0f;

    // G tile = R^T[rows] X^T[cols]^T over the expert's tokens. An expert
    // without tokens has an empty contraction: G = 0.
    if (ne > 0) {
        const uint16_t* A = fb.RT + static_cast<int64_t>(fb.rpe) * fb.tok[e];
        const uint16_t* B = fb.XT + static_cast<int64_t>(fb.cols) * fb.tok[e];
        // A row past the expert reads a valid row; its results are dropped.
        const bf16x8* pa[2];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const int arow = min(row0 + 16 * a + frow, fb.rpe - 1);
            pa[a] = reinterpret_cast<const bf16x8*>(A + static_cast<int64_t>(arow) * ne + 8 * fq);
        }
        const bf16x8* pb[8];
#pragma unroll
        for (int b = 0; b < 8; ++b)
            pb[b] = reinterpret_cast<const bf16x8*>(
                B + static_cast<int64_t>(col0 + 16 * b + frow) * ne + 8 * fq);
        // Slice s starts 32 s elements (four 8-element vectors) further on.
        bf16x8 fa[2][2], fbv[2][8];
        auto ld = [&](int s, int slot) {
#pragma unroll
            for (int a = 0; a < 2; ++a) fa[slot][a] = pa[a][4 * s];
#pragma unroll
            for (int b = 0; b < 8; ++b) fbv[slot][b] = pb[b][4 * s];
        };
        auto mm = [&](int slot) {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 8; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[slot][a], fbv[slot][b],
                                                                        acc[a][b], 0, 0, 0);
        };
        const int S = ne / 32;   // even (ne is a multiple of 64)
        ld(0, 0);
        for (int s = 0; s < S; s += 2) {
            ld(s + 1, 1);
            mm(0);
            if (s + 2 < S) ld(s + 2, 0);
            mm(1);
        }
    }

    // Accumulators -> slab: register r of block (a, b) is
    // G[16a + 4q + r][16b + frow].
    float* my = slab + wave * 32 * kSlabStride;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                my[(16 * a + 4 * fq + r) * kSlabStride + 16 * b + frow] = acc[a][b][r];
    // The slab is the wave's own: its LDS operations complete in order, so
    // the reads below see these stores; the empty asm keeps the compiler from
    // moving memory accesses across.
    asm volatile("" ::: "memory");

    for (int jb = 0; jb < nrows; jb += kRing) {
#pragma unroll
        for (int q = 0; q < kRing; ++q) {
            const int j = jb + q;
            if (j >= nrows) break;
            if (j + kRing - 1 < nrows) load_in(j + kRing - 1, ring[(q + kRing - 1) % kRing]);
            RowIn<GRID>& cur = ring[q];
            const uint64_t i0 = coord0(j);
            const Idx<O32> ix{i0};
            float g[N];
            const float2 gv = *reinterpret_cast<const float2*>(my + j * kSlabStride + 2 * lane);
            g[0] = 2.0f * gv.x;
            g[1] = 2.0f * gv.y;
            float gsum = bwd_lion_coords<GRID, false, O32>(g, cur.l, cur.m, cur.s, cur.cw, i0,
                                                           ra.step, ra.sid, ra.key, ra.tk, ra.lkl,
                                                           nullptr, ix, mk);
#pragma unroll
            for (int k = 0; k < L; ++k) {
                storev<N>(ix.at(ra.logits, mk, k), cur.l[k]);
                storev<N>(ix.at(ra.mom, mk, k), cur.m[k]);
            }
            // The group is the whole wave; every lane applies lane 0's sum.
            gsum = __shfl(group_sum<64>(gsum), 0, 64);
            float sn = cur.s, smn = cur.sm;
            lion_update(sn, smn, gsum, ra.lks);
            if (lane == 0) {
                ra.scales[i0 >> 7] = sn;
                ra.scale_mom[i0 >> 7] = smn;
            }
            if constexpr (FWD_NEXT) {
                float out[N];
                fwd_coords<GRID>(cur.l, sn, cur.cw, i0, ra.next_step, ra.sid, ra.key, ra.tk_next,
                                 out);
                store_dw<N>(ra.dW, ix, out, cur.w);
            }
        }
    }
}

inline int cdiv(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }

}  // namespace

hipError_t launch_recon_relax(const LayerDesc& d, int32_t n_experts, const int64_t* tok_offsets,
                              int64_t rows_per_expert, const uint16_t* XT, const uint16_t* RT,
                              const float* partials, size_t n_partials, double* loss,
                              float* logits, float* mom, float* scales, float* scale_mom,
                              const uint8_t* codes, uint32_t step, TauK tk, LionK lkl, LionK lks,
                              const void* W, uint32_t next_step, TauK tk_next, uint16_t* dW_next,
                              hipStream_t st) {
    RelaxArgs ra{};
    ra.logits = logits; ra.mom = mom; ra.scales = scales; ra.scale_mom = scale_mom;
    ra.codes = codes; ra.W = W; ra.dW = dW_next; ra.mk = d.mk;
    ra.step = step; ra.sid = d.sid; ra.next_step = next_step; ra.key = d.key;
    ra.tk = tk; ra.tk_next = tk_next; ra.lkl = lkl; ra.lks = lks;
    const bool fwd = dW_next != nullptr;
    const bool o32 = d.mk * 4 <= 0xFFFFFFF0ull;
    const int tiles_i = cdiv(rows_per_expert, kTileRows);
    const int tiles_j = cdiv(static_cast<int64_t>(d.cols), kTileCols);
    const int per_expert = tiles_i * tiles_j;
    for (int e0 = 0; e0 < n_experts; e0 += kFusedMaxExperts) {
        const int e1 = e0 + kFusedMaxExperts < n_experts ? e0 + kFusedMaxExperts : n_experts;
        FusedBatch fb{};
        fb.n = e1 - e0;
        fb.rpe = static_cast<int>(rows_per_expert);
        fb.cols = static_cast<int>(d.cols);
        fb.expert0 = e0;
        fb.tiles_i = tiles_i;
        fb.tiles_j = tiles_j;
        fb.RT = RT;
        fb.XT = XT;
        for (int e = 0; e <= fb.n; ++e) {
            fb.tok[e] = static_cast<int>(tok_offsets[e0 + e]);
            fb.wg0[e] = e * per_expert;
        }
        if (e0 == 0) {
            fb.fin_partials = partials;
            fb.fin_n = static_cast<int>(n_partials);
            fb.fin_loss = loss;
        }
        const dim3 grid(fb.n * per_expert), block(kFT);
#define GSQ_FUSED(G_, FW, WB, O) hipLaunchKernelGGL((recon_relax_kernel<G_, FW, WB, O>), grid, block, 0, st, fb, ra)
#define GSQ_FUSED_O(G_, FW, WB) if (o32) GSQ_FUSED(G_, FW, WB, true); else GSQ_FUSED(G_, FW, WB, false);
#define GSQ_FUSED_G(G_)                                                    \
        if (!fwd) { GSQ_FUSED_O(G_, false, true); }                       \
        else if (d.w_bf16) { GSQ_FUSED_O(G_, true, true); }               \
        else { GSQ_FUSED_O(G_, true, false); }
        switch (d.grid) {
            case GSQ_GRID_INT2: GSQ_FUSED_G(GSQ_GRID_INT2); break;
            case GSQ_GRID_INT3: GSQ_FUSED_G(GSQ_GRID_INT3); break;
            case GSQ_GRID_TERNARY: GSQ_FUSED_G(GSQ_GRID_TERNARY); break;
            default: GSQ_FUSED_G(GSQ_GRID_INT3_LOCAL); break;
        }
#undef GSQ_FUSED_G
#undef GSQ_FUSED_O
#undef GSQ_FUSED
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace gsq
