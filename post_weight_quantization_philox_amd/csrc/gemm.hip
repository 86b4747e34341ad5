// Reconstruction contractions of the GSQ step on the gfx950 matrix cores.
//
// Both products are "NT": C[i][j] = alpha * sum_r A[i][r] * B[j][r] with the
// contraction index r contiguous in both operands.
//   GEMM1  R^T = dW X^T      A = dW [M][K],   B = X   [N][K]  -> R^T [M][N] bf16,
//                            plus the per-tile partial sum of R^2 (the loss);
//   GEMM2  G   = 2 R^T X     A = R^T [M][N],  B = X^T [K][N]  -> G [M][K] fp32;
//                            its first workgroup also sums GEMM1's partials
//                            into the loss (fixed order, fp64).
// For a batch of experts each product is one grouped launch over all the
// experts' tiles. The same kernel also forms the Gram matrix H = X^T X (bf16
// or fp32 output), the Gram-form step G = 2 dW H with the loss sum dW * dW H
// taken in its epilogue, and the plain bf16 products of the block forward.
//
// Tiling: 256x256 output tile per workgroup of 4 waves (2x2), each wave a
// 128x128 sub-tile of 8x8 v_mfma_f32_16x16x32_bf16 blocks (256 fp32
// accumulators per lane). The 16x16 blocks, rather than 4x4 blocks of
// 32x32x16, move the same LDS bytes per flop and hold a higher shader clock
// under sustained matrix load. K advances 64 at a time; the A tiles (32 KiB
// a step) alternate between two LDS buffers and the B tiles rotate through
// three, 160 KiB in all: global loads run a step ahead of the fragment reads,
// and half of a step's B loads can be issued a slice before the A buffer they
// wait behind is free, which spreads the loads over more of the step. LDS
// rows are 128 bytes; the 16-byte chunk
// index is XOR-swizzled with the row so both the stores (8 threads per row)
// and the fragment reads (16 rows x 16 bytes per quarter-wave) are free of bank
// conflicts. Workgroups are renumbered so that consecutive tiles share an XCD
// (the dispatcher deals workgroups round-robin over the 8 XCDs) and tiles are
// ordered in groups of 4 tile-rows, which keeps each XCD's A and B panels in
// its own L2. A product that does not fill its last round of 256 tiles runs
// whole rounds of full tiles on a column or row block and the rest as 256x128
// tiles (same kernel, waves of 128x64), with unchanged summation order.
#include <type_traits>

#include "gsq_internal.hpp"

namespace gsq {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NT = 256;
constexpr int kChunks = BK / 8;   // 16-byte chunks per tile row
constexpr int kGroupM = 4;
// Byte offset past every operand buffer (their sizes are checked to stay below
// it), so a load there is out of range and returns zeros.
constexpr uint32_t kOob = 0x7FFFFF00u;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Epilogues: bf16 output plus the tile's sum of squares (GEMM1); fp32 output
// times alpha (GEMM2); plain bf16 output (the Gram matrix); fp32 output times
// alpha plus the tile's sum of D[i][j] * C[i][j] before scaling (the Gram-form
// step, where D = dW and C = dW H, so the sum is the loss); and GEMM1 with a
// fixed bf16 offset D added to C before the square and the rounding (the
// residual R^T = dW X^T + E0^T of a layer fitted to a target downstream).
enum { EPI_BF16_LOSS = 0, EPI_F32_SCALED = 1, EPI_BF16 = 2, EPI_F32_GRAM = 3,
       EPI_BF16_LOSS_OFF = 4 };

struct GemmArgs {
    const uint16_t* A;
    const uint16_t* B;
    int64_t lda, ldb, ldc;
    int I, J, Rd;
    int a_bytes, b_bytes;   // operand buffer sizes for the range check
    int tiles_i, tiles_j;
    void* C;
    float alpha;
    float* partials;   // EPI_BF16_LOSS(_OFF), EPI_F32_GRAM: one float per workgroup
    const uint16_t* D; // EPI_F32_GRAM, EPI_BF16_LOSS_OFF: bf16 [I][ldd] paired with the output
    int64_t ldd;
    // Optional: workgroup 0 first sums fin_n loss partials of an earlier
    // launch into *fin_loss (the same order as loss_finalize_kernel), which
    // saves that launch.
    const float* fin_partials;
    int fin_n;
    double* fin_loss;
};

// Experts of one grouped launch (at most kMaxGroups). Expert e of the launch
// (expert0 + e of the batch) owns rows [e*rpe, (e+1)*rpe) of dW, R^T's block
// and G, and the token block [tok[e], tok[e+1]) of X (absolute offsets,
// multiples of 64); its workgroups are [wg0[e], wg0[e+1]).
constexpr int kMaxGroups = 64;
struct ExpertBatch {
    int n;            // experts in this launch
    int stage;        // 0: R_e^T = dW_e X_e^T;  1: G_e = 2 R_e^T X_e
    int rpe, cols, expert0;
    const uint16_t* dW;
    const uint16_t* X;
    const uint16_t* XT;
    uint16_t* RT;
    float* G;
    int tok[kMaxGroups + 1];
    int wg0[kMaxGroups + 1];
};

// Workgroups are renumbered so that consecutive logical indices share an XCD
// (the dispatcher deals workgroups round-robin over the 8 XCDs).
__device__ __forceinline__ int logical_wg() {
    const int nwg = gridDim.x;
    const int wg = blockIdx.x;
    return (nwg & 7) == 0 ? (wg & 7) * (nwg >> 3) + (wg >> 3) : wg;
}

// Tile of a logical index inside a tiles_i x tiles_j grid, in groups of
// kGroupM tile-rows.
__device__ __forceinline__ void tile_of(int logical, int tiles_i, int tiles_j, int& ti, int& tj) {
    const int width = kGroupM * tiles_j;
    const int grp = logical / width;
    const int first = grp * kGroupM;
    const int gm = min(tiles_i - first, kGroupM);
    const int in = logical - grp * width;
    ti = first + in % gm;
    tj = in / gm;
}

// The product this workgroup's expert computes, and the workgroup's index
// within it.
__device__ __forceinline__ int resolve(const ExpertBatch& eb, int logical, GemmArgs& g) {
    // wg0 is nondecreasing, so the expert is the number of later starts at or
    // below `logical`. Unrolled over the table's fixed size, the starts are
    // read with a few wide scalar loads instead of one dependent load per
    // expert (2.6 us per workgroup for 64 experts).
    int e = 0;
#pragma unroll
    for (int k = 1; k < kMaxGroups; ++k) e += (k < eb.n && logical >= eb.wg0[k]) ? 1 : 0;
    e = __builtin_amdgcn_readfirstlane(e);   // uniform: keeps the addressing scalar
    const int64_t t0 = eb.tok[e];
    const int ne = eb.tok[e + 1] - eb.tok[e];
    const int64_t rows0 = static_cast<int64_t>(eb.expert0 + e) * eb.rpe;
    if (eb.stage == 0) {
        g.A = eb.dW + rows0 * eb.cols; g.lda = eb.cols;
        g.B = eb.X + t0 * eb.cols;     g.ldb = eb.cols;
        g.I = eb.rpe; g.J = ne; g.Rd = eb.cols;
        g.C = eb.RT + static_cast<int64_t>(eb.rpe) * t0; g.ldc = ne;
        g.a_bytes = eb.rpe * eb.cols * 2; g.b_bytes = ne * eb.cols * 2;
    } else {
        g.A = eb.RT + static_cast<int64_t>(eb.rpe) * t0; g.lda = ne;
        g.B = eb.XT + static_cast<int64_t>(eb.cols) * t0; g.ldb = ne;
        g.I = eb.rpe; g.J = eb.cols; g.Rd = ne;
        g.C = eb.G + rows0 * eb.cols; g.ldc = eb.cols;
        g.a_bytes = eb.rpe * ne * 2; g.b_bytes = eb.cols * ne * 2;
    }
    g.tiles_i = (g.I + BM - 1) / BM;
    g.tiles_j = (g.J + BN - 1) / BN;
    return logical - eb.wg0[e];
}

typedef __attribute__((address_space(3))) void lds_void;

// LDS swizzle: logical 16-byte chunk c of tile row r sits at physical chunk
// c ^ ((r >> 1) & 7). A ds_read_b128 is served 16 lanes at a time across 64
// four-byte banks (256 bytes); a 128-byte row covers half of them, so rows of
// equal parity share banks. Fragment reads take 16 consecutive rows at one
// logical chunk: the 8 even and the 8 odd rows each land on 8 distinct
// physical chunks, which makes the access conflict-free.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// One K-step of one operand tile: 32 Q rows x 64 bf16 (32 KiB for 256 rows),
// written by direct global->LDS loads. Wave w, load q fills tile rows R0..R0+7 with
// R0 = 8*(4q + w); lane l lands at LDS row R0 + l/8, physical chunk l%8, and
// therefore fetches logical chunk (l%8) ^ swz(row) of its row.
template <int Q>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rs, const uint32_t* off, uint32_t koff,
                                         uint4* tile, int wave) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int r0 = 8 * (4 * q + wave);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(tile + r0 * kChunks), 16,
                                                 off[q], koff, 0, 0);
    }
}

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier without a memory fence (the explicit waits give the
// ordering); the empty asm statements keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void bar() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// GROUPED: one launch over the experts of `eb` (its product replaces the
// operand fields of g); otherwise g is one product and eb is unused. TBN is
// the tile width: 256, or 128 (each wave 128x64) for the tiles of a launch's
// last, partial round, which then finish in about half the time.
template <int EPI, bool GROUPED, int TBN>
__global__ __launch_bounds__(NT) void gemm_nt_kernel(GemmArgs g, ExpertBatch eb) {
    static_assert(TBN == 256 || TBN == 128, "tile width 256 or 128");
    static_assert(!GROUPED || TBN == BN, "expert batches use the full tile");
    constexpr int WN = TBN / 2;      // wave tile width
    constexpr int NB = WN / 16;      // 16-column MFMA blocks per wave
    constexpr int QB = TBN / 32;     // DMA row groups of the B tile
    // A tiles in two buffers, B tiles in a ring of three (a 128-wide tile
    // uses the first half of each): 160 KiB, the whole LDS.
    __shared__ uint4 sA0[BM * kChunks];
    __shared__ uint4 sA1[BM * kChunks];
    __shared__ uint4 sBr[3 * BN * kChunks];
    uint4* const sB0 = sBr;
    uint4* const sB1 = sBr + BN * kChunks;
    uint4* const sB2 = sBr + 2 * BN * kChunks;

    if (g.fin_loss != nullptr && blockIdx.x == 0) {
        // In the third B buffer, which no load writes before the prologue's
        // barrier.
        double* fred = reinterpret_cast<double*>(sB2);
        double fs = 0.0;
        for (int i = threadIdx.x; i < g.fin_n; i += NT) fs += static_cast<double>(g.fin_partials[i]);
        fred[threadIdx.x] = fs;
        __syncthreads();
        for (int w = NT / 2; w >= 1; w >>= 1) {
            if (static_cast<int>(threadIdx.x) < w) fred[threadIdx.x] += fred[threadIdx.x + w];
            __syncthreads();
        }
        if (threadIdx.x == 0) *g.fin_loss = fred[0];
    }
    int local = logical_wg();
    if constexpr (GROUPED) local = resolve(eb, local, g);
    int ti, tj;
    tile_of(local, g.tiles_i, g.tiles_j, ti, tj);
    const int i0 = ti * BM, j0 = tj * TBN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // Wave index as a scalar: LDS destinations of the DMA loads (the M0
    // operand) then come from scalar arithmetic.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wi = wave >> 1, wj = wave & 1;

    // Per-lane byte offsets of the rows this lane fetches. Rows past the edge
    // get an offset beyond the buffer: the hardware range check returns zeros.
    const __amdgpu_buffer_rsrc_t ra_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(g.A), 0, g.a_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(g.B), 0, g.b_bytes, 0x00020000);
    const int lrow = lane >> 3;
    uint32_t oa[8], ob[8];   // ob: the first QB entries are used
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int row = 8 * (4 * q + wave) + lrow;
        const int lch = (lane & 7) ^ swz(row);
        const int rowa = i0 + row, rowb = j0 + row;
        oa[q] = rowa < g.I ? static_cast<uint32_t>((static_cast<int64_t>(rowa) * g.lda + lch * 8) * 2) : kOob;
        if (q < QB)
            ob[q] = rowb < g.J ? static_cast<uint32_t>((static_cast<int64_t>(rowb) * g.ldb + lch * 8) * 2) : kOob;
    }

    // Block (a, b) of the wave's accumulators is the 16x16 output block at
    // rows 16a, columns 16b of its sub-tile.
    f32x4 acc[8][NB];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[a][b][r] = 0.0f;

    // Fragment addressing: lane reads row (lane & 15) of a 16-row block at
    // chunk 4s + (lane >> 4) of the 64-wide K-step, i.e. k = 32s + 8 (lane >> 4)
    // .. + 7 of slice s; block rows start at multiples of 16, so the swizzle
    // term is swz(lane & 15).
    const int frow = lane & 15;
    const int fq = lane >> 4;
    const int fsw = swz(frow);
    const int rowA = wi * 128 + frow;
    const int rowB = wj * WN + frow;

    // Fragment registers: slot s holds slice s of a K-step (8 A blocks, NB B
    // blocks); slice 1 is fetched during slice 0's MFMAs and the next step's
    // slice 0 during slice 1's.
    bf16x8 fa[2][8], fb[2][NB];
    auto read_a = [&](const uint4* t, int s, int a) {
        return __builtin_bit_cast(bf16x8, t[(rowA + 16 * a) * kChunks + ((4 * s + fq) ^ fsw)]);
    };
    auto read_b = [&](const uint4* t, int s, int b) {
        return __builtin_bit_cast(bf16x8, t[(rowB + 16 * b) * kChunks + ((4 * s + fq) ^ fsw)]);
    };
    // Fragment read q of a slice: the B blocks first, then the A blocks, in
    // the order the MFMAs consume them.
    constexpr int kReads = 8 + NB;
    auto fetch1 = [&](const uint4* tA, const uint4* tB, int s, int q) {
        if (q < NB) fb[s][q] = read_b(tB, s, q);
        else fa[s][q - NB] = read_a(tA, s, q - NB);
    };
    // DMA load d (0..15) of a K-step: A loads q = 0..7, then B's QB loads
    // (a 128-wide tile has 4: its last four slots load nothing).
    auto dma1 = [&](int d, uint32_t koff, uint4* nA, uint4* nB) {
        const int q = d & 7;
        const int r0 = 8 * (4 * q + wave);
        if (d < 8)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra_rs, (lds_void*)(nA + r0 * kChunks), 16,
                                                     oa[q], koff, 0, 0);
        else if (q < QB)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb_rs, (lds_void*)(nB + r0 * kChunks), 16,
                                                     ob[q], koff, 0, 0);
    };
    // Work item i of n spread over `parts` sub-groups: sub-group p takes
    // items [first(p), first(p + 1)).
    auto first = [](int p, int n, int parts) { return (p * n + parts - 1) / parts; };
    // Sub-group of slice 1 at which the workgroup hands this step's buffer
    // over to the DMA: the fragment reads of slice 1 have had two sub-groups
    // of MFMAs to land.
    constexpr int kBar = 2;
    // B-tile loads of step k+2 issued in step k's first slice, half of them:
    // the B tiles rotate through three buffers, so these have their buffer
    // free a slice before the barrier frees the A buffer for the rest.
    constexpr int kB0 = QB / 2;

    // One K-step: two 32-wide slices, each issued as 8 sub-groups (A block a:
    // NB MFMAs) with their share of fragment reads and DMA loads, pinned in
    // this order by scheduling barriers so memory instructions drain between
    // MFMAs. Slice 0 fetches slice 1 of this step and issues kB0 of step
    // k+2's B-tile loads into the B ring. At sub-group kBar of slice 1, once
    // every read of this step's buffers has landed, the next step has landed
    // and the workgroup has synced, the remaining sub-groups fetch the next
    // step's slice 0 and issue step k+2's other loads (its A tile into this
    // step's A buffer), about a full K-step ahead.
    // Every step is the same code, which keeps the accumulators in their
    // registers: the last step also syncs and fetches from the other buffer,
    // and the last two load the contraction's final K-step again (in range)
    // in place of steps k+2 past its end; neither result is read.
    auto kstep = [&](const uint4* tA, const uint4* tB, const uint4* nA,
                     const uint4* nB, uint4* bB2, uint32_t knext2) {
#pragma unroll
        for (int a = 0; a < 8; ++a) {
#pragma unroll
            for (int q = 0; q < kReads; ++q)
                if (q >= first(a, kReads, 8) && q < first(a + 1, kReads, 8)) fetch1(tA, tB, 1, q);
            // The last kB0 B-tile loads of step k+2, one per sub-group, into
            // the ring buffer that step k-1 used (free since its barrier).
#pragma unroll
            for (int d = 8 + QB - kB0; d < 8 + QB; ++d)
                if (a == d - (8 + QB - kB0)) dma1(d, knext2, nullptr, bB2);
#pragma unroll
            for (int b = 0; b < NB; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[0][a], fb[0][b], acc[a][b], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int a = 0; a < 8; ++a) {
            if (a == kBar) {
                // Step k+1 has landed; the kB0 loads of step k+2 issued in
                // slice 0 may still be in flight.
                if constexpr (kB0 == 4) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)" ::: "memory");
                else asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)" ::: "memory");
                bar();
            }
            if (a >= kBar) {
                const int p = a - kBar;
#pragma unroll
                for (int q = 0; q < kReads; ++q)
                    if (q >= first(p, kReads, 8 - kBar) && q < first(p + 1, kReads, 8 - kBar))
                        fetch1(nA, nB, 0, q);
                // The other loads of step k+2: the A tile into this step's
                // buffer, the rest of the B tile into the ring.
                uint4* fA = const_cast<uint4*>(tA);
                constexpr int kD1 = 8 + QB - kB0;
#pragma unroll
                for (int d = 0; d < kD1; ++d)
                    if (d >= first(p, kD1, 8 - kBar) && d < first(p + 1, kD1, 8 - kBar))
                        dma1(d, knext2, fA, bB2);
            }
#pragma unroll
            for (int b = 0; b < NB; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[1][a], fb[1][b], acc[a][b], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    const int nk = g.Rd / BK;
    constexpr uint32_t kStep = BK * 2;   // bytes of one K-step along a row
    // An expert without tokens has an empty contraction: its output is zero.
    if (nk > 0) {
        // Prologue: step 0 (waited for) and step 1 in flight; slice 0 fetched.
        dma_tile<8>(ra_rs, oa, 0, sA0, wave);
        dma_tile<QB>(rb_rs, ob, 0, sB0, wave);
        if (nk > 1) {
            wait_dma();
            dma_tile<8>(ra_rs, oa, kStep, sA1, wave);
            dma_tile<QB>(rb_rs, ob, kStep, sB1, wave);
            if constexpr (QB == 8) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
            else asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
        } else {
            wait_dma();
        }
        bar();
#pragma unroll
        for (int q = 0; q < kReads; ++q) fetch1(sA0, sB0, 0, q);
        uint4* b0 = sB0;   // B ring: steps kt, kt+1, kt+2
        uint4* b1 = sB1;
        uint4* b2 = sB2;
        for (int kt = 0; kt < nk; ++kt) {
            const bool odd = kt & 1;
            kstep(odd ? sA1 : sA0, b0, odd ? sA0 : sA1, b1, b2,
                  static_cast<uint32_t>(min(kt + 2, nk - 1)) * kStep);
            uint4* const t = b0;
            b0 = b1; b1 = b2; b2 = t;
        }
    }
    // The last steps' DMA loads have landed and all waves are done with the
    // operand buffers before the epilogue reuses them.
    wait_dma();
    __syncthreads();

    // Epilogue, one 32-row slab of the wave's 128x128 sub-tile at a time:
    // accumulators go to a private 32x128 fp32 LDS slab (register r of block
    // (a, b) is C[16a + 4*(lane/16) + r][16b + lane%16]), then each
    // lane reads back 8 (bf16 output) or 4 (fp32 output) consecutive values of
    // one row and stores them as one 16-byte vector. N and K are multiples of
    // 8, so a vector is entirely inside or outside the matrix.
    constexpr int kSlab = WN + 4;      // padded row: the two half-waves' rows
                                        // start 16 bytes apart in the banks
    // One 32 KiB buffer per wave.
    float* slab = reinterpret_cast<float*>(wave == 0 ? sA0 : wave == 1 ? sB0 : wave == 2 ? sA1 : sB1);
    float* red = reinterpret_cast<float*>(sB2);   // the loss partial's wave sums
    const int grow0 = i0 + wi * 128;
    const int gcol0 = j0 + wj * WN;
    float lsum = 0.0f;
    // Gram form: the dW values a slab pairs with, loaded one slab ahead so
    // their latency overlaps the previous slab's work (zero outside the
    // matrix).
    // Same lane -> (row, 4 columns) map as the fp32 store below.
    uint2 dv[2][16];
    auto load_dv = [&](int a, uint2 (&d)[16]) {
        constexpr int LPR = WN / 4;
#pragma unroll
        for (int t = 0; t < 32 * LPR / 64; ++t) {
            const int c = lane + 64 * t;
            const int grow = grow0 + a * 32 + c / LPR, gcol = gcol0 + (c % LPR) * 4;
            d[t] = (grow < g.I && gcol < g.J)
                       ? *reinterpret_cast<const uint2*>(g.D + static_cast<int64_t>(grow) * g.ldd + gcol)
                       : make_uint2(0u, 0u);
        }
    };
    if constexpr (EPI == EPI_F32_GRAM) load_dv(0, dv[0]);
    // Slab a of the wave (a compile-time index, so the accumulators stay in
    // place).
    auto slab_out = [&](auto slab_index) {
        constexpr int a = decltype(slab_index)::value;
        if constexpr (EPI == EPI_F32_GRAM) {
            if (a + 1 < 4) load_dv(a + 1, dv[(a + 1) & 1]);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    slab[(16 * h + 4 * fq + r) * kSlab + 16 * b + frow] = acc[2 * a + h][b][r];
        __syncthreads();
        if constexpr (EPI == EPI_BF16_LOSS || EPI == EPI_BF16 || EPI == EPI_BF16_LOSS_OFF) {
            // 16 lanes per 128-value row: 8 values -> one 16-byte bf16 store.
            constexpr int LPR = WN / 8;   // lanes per row
#pragma unroll
            for (int t = 0; t < 32 * LPR / 64; ++t) {
                const int c = lane + 64 * t;
                const int row = c / LPR, col = (c % LPR) * 8;
                float4 v0 = *reinterpret_cast<const float4*>(slab + row * kSlab + col);
                float4 v1 = *reinterpret_cast<const float4*>(slab + row * kSlab + col + 4);
                const int grow = grow0 + a * 32 + row, gcol = gcol0 + col;
                if (grow < g.I && gcol < g.J) {
                    const int64_t off = static_cast<int64_t>(grow) * g.ldc + gcol;
                    if constexpr (EPI == EPI_BF16_LOSS_OFF) {
                        const uint4 e = *reinterpret_cast<const uint4*>(
                            g.D + static_cast<int64_t>(grow) * g.ldd + gcol);
                        v0.x += bf16_lo(e.x); v0.y += bf16_hi(e.x);
                        v0.z += bf16_lo(e.y); v0.w += bf16_hi(e.y);
                        v1.x += bf16_lo(e.z); v1.y += bf16_hi(e.z);
                        v1.z += bf16_lo(e.w); v1.w += bf16_hi(e.w);
                    }
                    if constexpr (EPI == EPI_BF16_LOSS || EPI == EPI_BF16_LOSS_OFF) {
                        lsum = __builtin_fmaf(v0.x, v0.x, lsum); lsum = __builtin_fmaf(v0.y, v0.y, lsum);
                        lsum = __builtin_fmaf(v0.z, v0.z, lsum); lsum = __builtin_fmaf(v0.w, v0.w, lsum);
                        lsum = __builtin_fmaf(v1.x, v1.x, lsum); lsum = __builtin_fmaf(v1.y, v1.y, lsum);
                        lsum = __builtin_fmaf(v1.z, v1.z, lsum); lsum = __builtin_fmaf(v1.w, v1.w, lsum);
                    }
                    uint4 o;
                    o.x = pack_bf16x2(v0.x, v0.y); o.y = pack_bf16x2(v0.z, v0.w);
                    o.z = pack_bf16x2(v1.x, v1.y); o.w = pack_bf16x2(v1.z, v1.w);
                    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(g.C) + off) = o;
                }
            }
        } else {
            // 32 lanes per 128-value row: each store instruction writes two
            // whole 512-byte rows.
            constexpr int LPR = WN / 4;
#pragma unroll
            for (int t = 0; t < 32 * LPR / 64; ++t) {
                const int c = lane + 64 * t;
                const int row = c / LPR, col = (c % LPR) * 4;
                const float4 v = *reinterpret_cast<const float4*>(slab + row * kSlab + col);
                const int grow = grow0 + a * 32 + row, gcol = gcol0 + col;
                if (grow < g.I && gcol < g.J) {
                    const int64_t off = static_cast<int64_t>(grow) * g.ldc + gcol;
                    if constexpr (EPI == EPI_F32_GRAM) {
                        const uint2 d = dv[a & 1][t];
                        lsum = __builtin_fmaf(bf16_lo(d.x), v.x, lsum);
                        lsum = __builtin_fmaf(bf16_hi(d.x), v.y, lsum);
                        lsum = __builtin_fmaf(bf16_lo(d.y), v.z, lsum);
                        lsum = __builtin_fmaf(bf16_hi(d.y), v.w, lsum);
                    }
                    // G is read once, by the next kernel: a nontemporal
                    // store (the 64-expert recon 2.45 -> 2.26 ms).
                    __builtin_nontemporal_store(
                        f32x4{g.alpha * v.x, g.alpha * v.y, g.alpha * v.z, g.alpha * v.w},
                        reinterpret_cast<f32x4*>(static_cast<float*>(g.C) + off));
                }
            }
        }
        __syncthreads();
    };
    if constexpr (EPI == EPI_F32_SCALED && NB == 8) {
        // fp32 output (G) from full-width tiles: 16-row slabs in two buffers
        // of the wave's own region, no workgroup barriers (a wave only
        // touches its own region, and one wave's LDS operations complete in
        // order). Each of slab s's eight read-backs and 16-byte stores is
        // paired with the four LDS writes of one block of slab s+1, so the
        // writes issue while the stores drain instead of between them (the
        // compute unit's store path, about 70 GB/s, bounds this epilogue; on
        // the 64-expert batch both products 2.05 -> 2.01 ms).
        float* const sl0 = slab;
        float* const sl1 = slab + 16 * kSlab;
        constexpr int LPR = WN / 4;   // 32 lanes per 128-float row
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) sl0[(4 * fq + r) * kSlab + 16 * b + frow] = acc[0][b][r];
        auto step = [&](auto si) {
            constexpr int s = decltype(si)::value;
            const float* sl = (s & 1) ? sl1 : sl0;
            float* nx = (s & 1) ? sl0 : sl1;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int c = lane + 64 * t;
                const int row = c / LPR, col = (c % LPR) * 4;
                const float4 v = *reinterpret_cast<const float4*>(sl + row * kSlab + col);
                if constexpr (s + 1 < 8) {
                    // block b = t of slab s+1: its 4 values
#pragma unroll
                    for (int r = 0; r < 4; ++r) nx[(4 * fq + r) * kSlab + 16 * t + frow] = acc[s + 1][t][r];
                }
                const int grow = grow0 + s * 16 + row, gcol = gcol0 + col;
                if (grow < g.I && gcol < g.J) {
                    const int64_t off = static_cast<int64_t>(grow) * g.ldc + gcol;
                    __builtin_nontemporal_store(
                        f32x4{g.alpha * v.x, g.alpha * v.y, g.alpha * v.z, g.alpha * v.w},
                        reinterpret_cast<f32x4*>(static_cast<float*>(g.C) + off));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        step(std::integral_constant<int, 0>{}); step(std::integral_constant<int, 1>{});
        step(std::integral_constant<int, 2>{}); step(std::integral_constant<int, 3>{});
        step(std::integral_constant<int, 4>{}); step(std::integral_constant<int, 5>{});
        step(std::integral_constant<int, 6>{}); step(std::integral_constant<int, 7>{});
    } else {
        slab_out(std::integral_constant<int, 0>{});
        slab_out(std::integral_constant<int, 1>{});
        slab_out(std::integral_constant<int, 2>{});
        slab_out(std::integral_constant<int, 3>{});
    }
    if constexpr (EPI == EPI_BF16_LOSS || EPI == EPI_F32_GRAM || EPI == EPI_BF16_LOSS_OFF) {
        // Fixed-order reduction: wave butterfly, then waves 0..3 in order.
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) lsum += __shfl_xor(lsum, m, 64);
        if (lane == 0) red[wave] = lsum;
        __syncthreads();
        if (tid == 0) g.partials[blockIdx.x] = ((red[0] + red[1]) + red[2]) + red[3];
    }
}

__global__ __launch_bounds__(256) void loss_finalize_kernel(const float* __restrict__ partials,
                                                            int n, double* __restrict__ loss) {
    __shared__ double red[256];
    double s = 0.0;
    for (int i = threadIdx.x; i < n; i += 256) s += static_cast<double>(partials[i]);
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if (static_cast<int>(threadIdx.x) < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) *loss = red[0];
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

// X [n][cols] -> XT [cols][n], 64x64 tiles through LDS (n % 64 == 0,
// cols % 64 == 0).
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ X,
                                                        uint16_t* __restrict__ XT, int64_t n,
                                                        int64_t cols) {
    __shared__ uint16_t t[64][66];
    const int64_t c0 = static_cast<int64_t>(blockIdx.x) * 64;
    const int64_t r0 = static_cast<int64_t>(blockIdx.y) * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int r = ty; r < 64; r += 4) t[r][tx] = X[(r0 + r) * cols + c0 + tx];
    __syncthreads();
    for (int c = ty; c < 64; c += 4) XT[(c0 + c) * n + r0 + tx] = t[tx][c];
}

inline int cdiv(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }

// One launch of the product over rows [r0, r0 + I) and columns [c0, c0 + J)
// of the full product, tiles TBN wide.
template <int EPI, int TBN>
void launch_part(GemmArgs g, int r0, int c0, int I, int J, float* partials, hipStream_t st) {
    g.A += static_cast<int64_t>(r0) * g.lda;
    g.B += static_cast<int64_t>(c0) * g.ldb;
    if (g.D) g.D += static_cast<int64_t>(r0) * g.ldd + c0;
    g.I = I; g.J = J;
    g.a_bytes = static_cast<int>(static_cast<int64_t>(I) * g.lda * 2);
    g.b_bytes = static_cast<int>(static_cast<int64_t>(J) * g.ldb * 2);
    constexpr int esz = (EPI == EPI_BF16_LOSS || EPI == EPI_BF16 || EPI == EPI_BF16_LOSS_OFF) ? 2 : 4;
    g.C = static_cast<char*>(g.C) + (static_cast<int64_t>(r0) * g.ldc + c0) * esz;
    g.partials = partials;
    g.tiles_i = cdiv(I, BM); g.tiles_j = cdiv(J, TBN);
    ExpertBatch none{};
    hipLaunchKernelGGL((gemm_nt_kernel<EPI, false, TBN>), dim3(g.tiles_i * g.tiles_j), dim3(NT), 0,
                       st, g, none);
}

constexpr int kCUs = 256;   // MI355X compute units: one workgroup each per round

// How one product of ti x tj full tiles is launched. A partial last round
// leaves compute units idle while its tiles run, so whole rounds of full tiles
// go to a column block (COLS) or a row block (ROWS) of `at` tiles, and the rest
// of the product to 128-wide tiles, which finish in about half the time; a
// product under half a round uses 128-wide tiles throughout (NARROW).
struct Split {
    enum Kind { FULL, NARROW, COLS, ROWS } kind;
    int at;
};

Split plan_split(int I, int J) {
    const int ti = cdiv(I, BM), tj = cdiv(J, BN), T = ti * tj;
    if (T % kCUs == 0) return {Split::FULL, 0};
    if (T * 2 <= kCUs) return {Split::NARROW, 0};
    auto gcd = [](int a, int b) { while (b) { const int t = a % b; a = b; b = t; } return a; };
    const int n0 = kCUs / gcd(ti, kCUs), jm = (tj / n0) * n0;
    if (jm > 0 && jm < tj && ti * (tj - jm) * 2 <= kCUs) return {Split::COLS, jm};
    const int m0 = kCUs / gcd(tj, kCUs), im = (ti / m0) * m0;
    if (im > 0 && im < ti && (ti - im) * tj * 2 <= kCUs) return {Split::ROWS, im};
    return {Split::FULL, 0};
}

// Workgroups (and loss partials) of one product of I x J outputs.
int product_workgroups(int I, int J) {
    const Split sp = plan_split(I, J);
    const int ti = cdiv(I, BM), tj = cdiv(J, BN);
    switch (sp.kind) {
        case Split::NARROW: return ti * cdiv(J, 128);
        case Split::COLS: return ti * sp.at + ti * cdiv(J - sp.at * BN, 128);
        case Split::ROWS: return sp.at * tj + (ti - sp.at) * cdiv(J, 128);
        default: return ti * tj;
    }
}

// C[I][J] = alpha * A[I][Rd] B[J][Rd]^T (EPI selects the output form). With
// fin_loss set, the first workgroup also sums fin_n earlier loss partials
// into *fin_loss; partials (loss epilogues) receive product_workgroups(I, J)
// values.
template <int EPI>
hipError_t run_gemm(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int I, int J,
                    int Rd, void* C, int64_t ldc, float alpha, float* partials, hipStream_t st,
                    const uint16_t* D = nullptr, int64_t ldd = 0,
                    const float* fin_partials = nullptr, int fin_n = 0, double* fin_loss = nullptr) {
    GemmArgs g{};
    g.D = D; g.ldd = ldd;
    g.fin_partials = fin_partials; g.fin_n = fin_n; g.fin_loss = fin_loss;
    g.A = A; g.B = B; g.lda = lda; g.ldb = ldb; g.ldc = ldc;
    g.I = I; g.J = J; g.Rd = Rd;
    const int64_t ab = static_cast<int64_t>(I) * lda * 2, bb = static_cast<int64_t>(J) * ldb * 2;
    // Valid offsets plus the largest K offset stay below kOob, and kOob plus
    // that offset stays below 2^32, so the range check separates the two.
    if (Rd <= 0 || Rd % BK != 0 || ab > static_cast<int64_t>(kOob) - 2 * static_cast<int64_t>(Rd) ||
        bb > static_cast<int64_t>(kOob) - 2 * static_cast<int64_t>(Rd))
        return hipErrorInvalidValue;
    g.C = C; g.alpha = alpha;
    const Split sp = plan_split(I, J);
    const int ti = cdiv(I, BM), tj = cdiv(J, BN);
    float* tail_partials = nullptr;
    switch (sp.kind) {
        case Split::NARROW:
            launch_part<EPI, 128>(g, 0, 0, I, J, partials, st);
            break;
        case Split::COLS:
            launch_part<EPI, BN>(g, 0, 0, I, sp.at * BN, partials, st);
            g.fin_loss = nullptr;
            if (partials) tail_partials = partials + ti * sp.at;
            launch_part<EPI, 128>(g, 0, sp.at * BN, I, J - sp.at * BN, tail_partials, st);
            break;
        case Split::ROWS:
            launch_part<EPI, BN>(g, 0, 0, sp.at * BM, J, partials, st);
            g.fin_loss = nullptr;
            if (partials) tail_partials = partials + sp.at * tj;
            launch_part<EPI, 128>(g, sp.at * BM, 0, I - sp.at * BM, J, tail_partials, st);
            break;
        default:
            launch_part<EPI, BN>(g, 0, 0, I, J, partials, st);
    }
    return hipGetLastError();
}

// Both products of every expert in [e0, e1) (at most kMaxGroups), one grouped
// launch per product; stage-0 partials start at `partials`. Returns the
// number of partials written.
hipError_t run_expert_batch(int e0, int e1, const int64_t* tok_offsets, int64_t rpe, int64_t cols,
                            const uint16_t* X, const uint16_t* XT, const uint16_t* dW,
                            float* partials, uint16_t* RT, float* G, hipStream_t st,
                            size_t* n_partials, const float* fin_base = nullptr,
                            size_t fin_prior = 0, double* fin_loss = nullptr) {
    ExpertBatch eb{};
    eb.n = e1 - e0;
    eb.rpe = static_cast<int>(rpe);
    eb.cols = static_cast<int>(cols);
    eb.expert0 = e0;
    eb.dW = dW; eb.X = X; eb.XT = XT; eb.RT = RT; eb.G = G;
    // Per-expert operands are addressed like run_gemm's: 32-bit byte offsets
    // that must stay below kOob minus the contraction length.
    const int64_t lim = static_cast<int64_t>(kOob) - 2 * cols - 2 * tok_offsets[e1];
    if (rpe * cols * 2 > lim) return hipErrorInvalidValue;
    for (int e = e0; e < e1; ++e) {
        const int64_t ne = tok_offsets[e + 1] - tok_offsets[e];
        if (ne * cols * 2 > lim || rpe * ne * 2 > lim) return hipErrorInvalidValue;
    }
    const int ti = cdiv(rpe, BM);
    int wg1 = 0, wg2 = 0;
    int wg0_2[kMaxGroups + 1];
    for (int e = 0; e <= eb.n; ++e) eb.tok[e] = static_cast<int>(tok_offsets[e0 + e]);
    for (int e = 0; e < eb.n; ++e) {
        eb.wg0[e] = wg1;
        wg0_2[e] = wg2;
        wg1 += ti * cdiv(eb.tok[e + 1] - eb.tok[e], BN);
        wg2 += ti * cdiv(cols, BN);
    }
    eb.wg0[eb.n] = wg1;
    wg0_2[eb.n] = wg2;
    GemmArgs g{};
    g.alpha = 1.0f;
    g.partials = partials;
    *n_partials = static_cast<size_t>(wg1);
    if (wg1 > 0) {
        eb.stage = 0;
        hipLaunchKernelGGL((gemm_nt_kernel<EPI_BF16_LOSS, true, BN>), dim3(wg1), dim3(NT), 0, st, g, eb);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    eb.stage = 1;
    for (int e = 0; e <= eb.n; ++e) eb.wg0[e] = wg0_2[e];
    g.alpha = 2.0f;
    g.partials = nullptr;
    if (fin_loss != nullptr) {
        // The loss over every chunk's partials, this chunk's included.
        g.fin_partials = fin_base;
        g.fin_n = static_cast<int>(fin_prior + *n_partials);
        g.fin_loss = fin_loss;
    }
    hipLaunchKernelGGL((gemm_nt_kernel<EPI_F32_SCALED, true, BN>), dim3(wg2), dim3(NT), 0, st, g, eb);
    return hipGetLastError();
}

}  // namespace

size_t recon_partials(int32_t n_experts, const int64_t* tok_offsets, int64_t rows_per_expert) {
    size_t n = 0;
    for (int e = 0; e < n_experts; ++e) {
        const int64_t ne = tok_offsets[e + 1] - tok_offsets[e];
        if (ne == 0) continue;
        // A dense layer's GEMM1 may split its last round (product_workgroups);
        // expert batches launch whole tiles.
        n += n_experts == 1 ? static_cast<size_t>(product_workgroups(static_cast<int>(rows_per_expert),
                                                                     static_cast<int>(ne)))
                            : static_cast<size_t>(cdiv(rows_per_expert, BM)) * cdiv(ne, BN);
    }
    return n;
}

hipError_t launch_recon(int32_t n_experts, const int64_t* tok_offsets, int64_t rows_per_expert,
                        int64_t cols, const uint16_t* X, const uint16_t* XT, const uint16_t* dW,
                        float* partials, uint16_t* RT, float* G, double* loss, hipStream_t st) {
    size_t slot = 0;
    hipError_t err = hipSuccess;
    if (n_experts == 1) {
        // One dense layer: two plain launches.
        const int64_t ne = tok_offsets[1];
        if (ne == 0) {
            const int64_t n = rows_per_expert * cols;
            hipLaunchKernelGGL(fill_zero_kernel, dim3(cdiv(n, 256)), dim3(256), 0, st, G, n);
            err = hipGetLastError();
        } else {
            err = run_gemm<EPI_BF16_LOSS>(dW, cols, X, cols, static_cast<int>(rows_per_expert),
                                          static_cast<int>(ne), static_cast<int>(cols), RT, ne,
                                          1.0f, partials, st);
            if (err == hipSuccess) {
                slot = static_cast<size_t>(product_workgroups(static_cast<int>(rows_per_expert),
                                                              static_cast<int>(ne)));
                // GEMM2's first workgroup also sums GEMM1's loss partials.
                err = run_gemm<EPI_F32_SCALED>(RT, ne, XT, ne, static_cast<int>(rows_per_expert),
                                               static_cast<int>(cols), static_cast<int>(ne), G,
                                               cols, 2.0f, nullptr, st, nullptr, 0, partials,
                                               static_cast<int>(slot), loss);
                return err;
            }
        }
    } else {
        // Expert batches: every expert's tiles in one launch per product
        // (an expert's own products are too small to fill the GPU).
        for (int e0 = 0; e0 < n_experts && err == hipSuccess; e0 += kMaxGroups) {
            const int e1 = e0 + kMaxGroups < n_experts ? e0 + kMaxGroups : n_experts;
            size_t np = 0;
            // The last chunk's GEMM2 also sums every chunk's loss partials.
            const bool last = e1 == n_experts;
            err = run_expert_batch(e0, e1, tok_offsets, rows_per_expert, cols, X, XT, dW,
                                   partials + slot, RT, G, st, &np, partials, slot,
                                   last ? loss : nullptr);
            slot += np;
        }
        return err;
    }
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(loss_finalize_kernel, dim3(1), dim3(256), 0, st, partials,
                       static_cast<int>(slot), loss);
    return hipGetLastError();
}

hipError_t launch_recon_gemm1(int32_t n_experts, const int64_t* tok_offsets, int64_t rows_per_expert,
                              int64_t cols, const uint16_t* X, const uint16_t* dW, float* partials,
                              uint16_t* RT, size_t* n_partials, hipStream_t st) {
    *n_partials = 0;
    if (n_experts == 1) {
        const int64_t ne = tok_offsets[1];
        if (ne == 0) return hipSuccess;
        *n_partials = static_cast<size_t>(product_workgroups(static_cast<int>(rows_per_expert),
                                                            static_cast<int>(ne)));
        return run_gemm<EPI_BF16_LOSS>(dW, cols, X, cols, static_cast<int>(rows_per_expert),
                                       static_cast<int>(ne), static_cast<int>(cols), RT, ne, 1.0f,
                                       partials, st);
    }
    for (int e0 = 0; e0 < n_experts; e0 += kMaxGroups) {
        const int e1 = e0 + kMaxGroups < n_experts ? e0 + kMaxGroups : n_experts;
        ExpertBatch eb{};
        eb.n = e1 - e0;
        eb.stage = 0;
        eb.rpe = static_cast<int>(rows_per_expert);
        eb.cols = static_cast<int>(cols);
        eb.expert0 = e0;
        eb.dW = dW; eb.X = X; eb.RT = RT;
        const int64_t lim = static_cast<int64_t>(kOob) - 2 * cols - 2 * tok_offsets[e1];
        if (rows_per_expert * cols * 2 > lim) return hipErrorInvalidValue;
        const int ti = cdiv(rows_per_expert, BM);
        int wg = 0;
        for (int e = 0; e <= eb.n; ++e) eb.tok[e] = static_cast<int>(tok_offsets[e0 + e]);
        for (int e = 0; e < eb.n; ++e) {
            const int64_t ne = eb.tok[e + 1] - eb.tok[e];
            if (ne * cols * 2 > lim) return hipErrorInvalidValue;
            eb.wg0[e] = wg;
            wg += ti * cdiv(ne, BN);
        }
        eb.wg0[eb.n] = wg;
        if (wg > 0) {
            GemmArgs g{};
            g.alpha = 1.0f;
            g.partials = partials + *n_partials;
            hipLaunchKernelGGL((gemm_nt_kernel<EPI_BF16_LOSS, true, BN>), dim3(wg), dim3(NT), 0, st, g, eb);
            const hipError_t err = hipGetLastError();
            if (err != hipSuccess) return err;
        }
        *n_partials += static_cast<size_t>(wg);
    }
    return hipSuccess;
}

hipError_t launch_recon_offset(int64_t rows, int64_t cols, int64_t tokens, const uint16_t* X,
                               const uint16_t* XT, const uint16_t* dW, const uint16_t* E0T,
                               float* partials, uint16_t* RT, float* G, double* loss,
                               hipStream_t st) {
    hipError_t err = run_gemm<EPI_BF16_LOSS_OFF>(dW, cols, X, cols, static_cast<int>(rows),
                                                 static_cast<int>(tokens), static_cast<int>(cols), RT,
                                                 tokens, 1.0f, partials, st, E0T, tokens);
    if (err != hipSuccess) return err;
    const int slot = product_workgroups(static_cast<int>(rows), static_cast<int>(tokens));
    return run_gemm<EPI_F32_SCALED>(RT, tokens, XT, tokens, static_cast<int>(rows),
                                    static_cast<int>(cols), static_cast<int>(tokens), G, cols, 2.0f,
                                    nullptr, st, nullptr, 0, partials, slot, loss);
}

size_t gram_partials(int64_t rows, int64_t cols) {
    return static_cast<size_t>(product_workgroups(static_cast<int>(rows), static_cast<int>(cols)));
}

hipError_t launch_gram(int64_t tokens, int64_t cols, const uint16_t* XT, uint16_t* H,
                       hipStream_t st) {
    // H[i][j] = sum_n XT[i][n] XT[j][n]: an NT product of X^T with itself.
    return run_gemm<EPI_BF16>(XT, tokens, XT, tokens, static_cast<int>(cols), static_cast<int>(cols),
                              static_cast<int>(tokens), H, cols, 1.0f, nullptr, st);
}

hipError_t launch_matmul_nt_bf16(int64_t I, int64_t J, int64_t Rd, const uint16_t* A, int64_t lda,
                                 const uint16_t* B, int64_t ldb, uint16_t* C, int64_t ldc,
                                 hipStream_t st) {
    return run_gemm<EPI_BF16>(A, lda, B, ldb, static_cast<int>(I), static_cast<int>(J),
                              static_cast<int>(Rd), C, ldc, 1.0f, nullptr, st);
}

hipError_t launch_gram_f32(int64_t tokens, int64_t cols, const uint16_t* XT, float* H32,
                           hipStream_t st) {
    return run_gemm<EPI_F32_SCALED>(XT, tokens, XT, tokens, static_cast<int>(cols),
                                    static_cast<int>(cols), static_cast<int>(tokens), H32, cols, 1.0f,
                                    nullptr, st);
}

hipError_t launch_recon_gram(int64_t rows, int64_t cols, const uint16_t* H, const uint16_t* dW,
                             float* partials, float* G, double* loss, hipStream_t st) {
    // C = dW H^T = dW H (H is symmetric); G = 2 C; loss = sum dW * C.
    hipError_t err = run_gemm<EPI_F32_GRAM>(dW, cols, H, cols, static_cast<int>(rows),
                                            static_cast<int>(cols), static_cast<int>(cols), G, cols,
                                            2.0f, partials, st, dW, cols);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(loss_finalize_kernel, dim3(1), dim3(256), 0, st, partials,
                       static_cast<int>(gram_partials(rows, cols)), loss);
    return hipGetLastError();
}

hipError_t launch_transpose_tokens(int32_t n_experts, const int64_t* tok_offsets, int64_t cols,
                                   const uint16_t* X, uint16_t* XT, hipStream_t st) {
    for (int e = 0; e < n_experts; ++e) {
        const int64_t t0 = tok_offsets[e];
        const int64_t ne = tok_offsets[e + 1] - t0;
        if (ne == 0) continue;
        hipLaunchKernelGGL(transpose_kernel, dim3(cdiv(cols, 64), cdiv(ne, 64)), dim3(256), 0, st,
                           X + t0 * cols, XT + cols * t0, ne, cols);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace gsq
