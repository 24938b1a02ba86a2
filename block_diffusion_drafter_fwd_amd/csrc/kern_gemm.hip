// GEMMs of the drafter forward: C (+)= A . B^T with A = activations [M, K]
// and B = a weight [N, K] (row-major, out x in), several weights per launch
// as column segments (q|k|v|g, gate|up, every layer's k|v).
//
//  * k_gemm_skinny   M <= 16 (block path).  A workgroup owns 16 output
//    columns and streams their weight rows straight from HBM into MFMA
//    operands (v_mfma_f32_16x16x32_bf16), its 8 waves splitting K; weights
//    are read exactly once, so the kernel is HBM-bound.
//  * k_gemm_tiled    M > 16 (256-row flushes, batched blocks).  64|128 x 128
//    tiles, 4 waves as 2x2, A and B staged through LDS with double buffering.
//  * k_gemm_f32      the fp32 configuration (tiny shapes), plain FMA.
//
// Split-K partials of the tiled kernel go to a workspace slice and a reduce
// kernel writes C; the skinny kernel reduces inside the workgroup.
#include "kernels.h"

namespace dflash {
namespace kern {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;   // 16-byte operand piece
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ f32x4_t mfma32(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <class GA>
__device__ __forceinline__ int find_seg(const GA& a, int tile) {
    int s = 0;
    for (int j = 1; j < a.nseg; ++j)
        if (tile >= a.seg[j].tile0) s = j;
    return s;
}

template <class GA>
__device__ __forceinline__ void store_out(const GA& a, int split, int m, int col, float v) {
    if (a.splits == 1) {
        float* p = a.C + (size_t)m * a.ldc + col;
        *p = a.accumulate ? *p + v : v;
    } else {
        a.part[((size_t)split * a.M + m) * a.ldc + col] = v;
    }
}

// ---------------------------------------------------------------------------
// skinny: M <= 16.  A 512-thread workgroup owns TPW 16-column tiles (two
// tiles: the same A fragments feed both, halving activation traffic per
// weight byte; paired mode puts the gate tile and the up tile of the same
// columns side by side and the epilogue writes silu(gate) * up).  Its 8 waves
// take interleaved 64-wide k steps of the workgroup's K slice (kPartial mode
// splits K over gridDim.y workgroups), read the weight rows straight from HBM
// into MFMA operands, and reduce through LDS in a fixed order.
// ---------------------------------------------------------------------------
constexpr int kSkWaves = 8;

template <int TPW, int TAG, class GA, int BATCH>
__global__ __launch_bounds__(512) void k_gemm_skinny(GA a) {
    // BATCH: k steps per wave whose loads are in flight together (the launcher
    // picks the steps each wave has, up to 4, so a wave makes one round trip)
    __shared__ float red[kSkWaves][TPW][256];
    const int b = blockIdx.x, split = blockIdx.y, S = gridDim.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, q = lane >> 4;
    const bool pair = a.mode == kSwiGLU;
    const bool aval = r < a.M;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    const uint16_t* Bp[TPW];
    bool bval[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
        int n0;
        const GemmSeg* g;
        bool valid = true;
        if (pair) {
            g = &a.seg[j];
            n0 = b * 16;
        } else {
            const int tile = b * TPW + j;
            valid = tile < a.ntiles;
            g = &a.seg[find_seg(a, valid ? tile : a.ntiles - 1)];
            n0 = ((valid ? tile : a.ntiles - 1) - g->tile0) * 16;
        }
        bval[j] = valid && n0 + r < g->N;
        Bp[j] = (const uint16_t*)g->B + (size_t)(bval[j] ? n0 + r : 0) * g->ldb + q * 16;
    }
    // every tile of a workgroup reads the same A (the launcher guarantees it)
    const GemmSeg& g0 = a.seg[pair ? 0 : find_seg(a, min(b * TPW, a.ntiles - 1))];
    const int arow = aval ? (a.a_rows ? a.a_rows[r] : r) : 0;
    const uint16_t* Ap = (const uint16_t*)g0.A + (size_t)arow * g0.lda + q * 16;
    f32x4_t acc0[TPW], acc1[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) acc0[j] = acc1[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // this split's 64-wide k steps, interleaved over the waves
    const int nsteps_all = a.K >> 6;
    const int per = (nsteps_all + S - 1) / S;
    const int s_lo = split * per, s_hi = min(nsteps_all, s_lo + per);
    int st = s_lo + wave;
    for (; st + (BATCH - 1) * kSkWaves < s_hi; st += BATCH * kSkWaves) {
        u32x4_t bv[TPW][2 * BATCH], av[2 * BATCH];
#pragma unroll
        for (int j = 0; j < TPW; ++j)
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int k = (st + u * kSkWaves) << 6;
                bv[j][2 * u] = *(const u32x4_t*)(Bp[j] + k);
                bv[j][2 * u + 1] = *(const u32x4_t*)(Bp[j] + k + 8);
            }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int k = (st + u * kSkWaves) << 6;
            av[2 * u] = *(const u32x4_t*)(Ap + k);
            av[2 * u + 1] = *(const u32x4_t*)(Ap + k + 8);
        }
#pragma unroll
        for (int u = 0; u < 2 * BATCH; ++u) {
            av[u] = aval ? av[u] : zero;
#pragma unroll
            for (int j = 0; j < TPW; ++j) bv[j][u] = bval[j] ? bv[j][u] : zero;
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u)
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
                if (u & 1) {
                    acc1[j] = mfma32(av[2 * u], bv[j][2 * u], acc1[j]);
                    acc1[j] = mfma32(av[2 * u + 1], bv[j][2 * u + 1], acc1[j]);
                } else {
                    acc0[j] = mfma32(av[2 * u], bv[j][2 * u], acc0[j]);
                    acc0[j] = mfma32(av[2 * u + 1], bv[j][2 * u + 1], acc0[j]);
                }
            }
    }
    for (; st < s_hi; st += kSkWaves) {
        const int k = st << 6;
        u32x4_t a0 = *(const u32x4_t*)(Ap + k), a1 = *(const u32x4_t*)(Ap + k + 8);
        a0 = aval ? a0 : zero;
        a1 = aval ? a1 : zero;
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            u32x4_t b0 = *(const u32x4_t*)(Bp[j] + k), b1 = *(const u32x4_t*)(Bp[j] + k + 8);
            b0 = bval[j] ? b0 : zero;
            b1 = bval[j] ? b1 : zero;
            acc0[j] = mfma32(a0, b0, acc0[j]);
            acc0[j] = mfma32(a1, b1, acc0[j]);
        }
    }
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
        const f32x4_t acc = acc0[j] + acc1[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) red[wave][j][lane * 4 + e] = acc[e];
    }
    __syncthreads();
    // output (m, nn) of a tile lives at lane nn + 16 (m / 4), element m % 4;
    // threads 256 j' .. 256 j' + 255 finish tiles j', j' + 2, ...
    const int t = threadIdx.x;
    const int m = (t & 255) >> 4, nn = t & 15;
    if (m >= a.M) return;
    const int idx = (nn + 16 * (m >> 2)) * 4 + (m & 3);
    if (pair) {
        if (t >= 256 || b * 16 + nn >= a.seg[0].N) return;
        float gt = 0.f, up = 0.f;
        for (int w = 0; w < kSkWaves; ++w) {
            gt += red[w][0][idx];
            up += red[w][TPW - 1][idx];
        }
        const float v = gt / (1.f + __expf(-gt)) * up;
        const size_t o = (size_t)m * a.ldo + b * 16 + nn;
        if (a.out_bf16) {
            uint32_t u = __float_as_uint(v);
            u += 0x7FFFu + ((u >> 16) & 1u);
            ((uint16_t*)a.out)[o] = (uint16_t)(u >> 16);
        } else {
            ((float*)a.out)[o] = v;
        }
        return;
    }
    for (int j = t >> 8; j < TPW; j += 2) {
        const int tile = b * TPW + j;
        if (tile >= a.ntiles) return;
        const GemmSeg& g = a.seg[find_seg(a, tile)];
        const int n = (tile - g.tile0) * 16 + nn;
        if (n >= g.N) continue;
        float s0 = 0.f;
        for (int w = 0; w < kSkWaves; ++w) s0 += red[w][j][idx];
        if (a.mode == kPartial) {
            // this split's share; the consumer of C sums the splits
            a.C[((size_t)split * a.M + m) * a.ldc + g.c_col0 + n] = s0;
            continue;
        }
        float* p = a.C + (size_t)m * a.ldc + g.c_col0 + n;
        *p = a.mode == kAccumulate ? *p + s0 : s0;
    }
}

// ---------------------------------------------------------------------------
// skinny, persistent: the same work split, but each workgroup keeps its waves'
// A fragments in registers (STEPS 64-wide k steps per wave) and walks column
// tiles blockIdx.x, blockIdx.x + gridDim.x, ...  The activations are then read
// once per workgroup instead of once per 16 columns, which is what limits the
// per-tile kernel when N is large (the unembedding reads 622 MB of weights
// against 64 KB of activations).
// ---------------------------------------------------------------------------
template <int STEPS, int TAG, class GA, int TPI, int NW>
__global__ __launch_bounds__(64 * NW) void k_gemm_skinny_p(GA a) {
    // TPI adjacent 16-column tiles per iteration (2: the plain store form,
    // e.g. the unembedding; the reduction and its barriers then serve twice
    // the bytes); the paired SwiGLU form takes one
    static_assert(TPI == 1 || TPI == 2, "tiles per iteration");
    static_assert(NW == 8 || NW == 16, "waves");
    __shared__ float red[NW][TPI][64 * 4];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const bool pair = TPI == 1 && NW == kSkWaves && a.mode == kSwiGLU;
    const int nw = pair ? NW / 2 : NW;
    const int wv = pair ? (wave & (NW / 2 - 1)) : wave;
    const int r = lane & 15, q = lane >> 4;
    const bool aval = r < a.M;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    // this wave's k steps are wv, wv + nw, ... (STEPS of them: K = 64 * nw * STEPS)
    u32x4_t av[2 * STEPS];
    {
        const int arow = aval ? (a.a_rows ? a.a_rows[r] : r) : 0;
        const uint16_t* Ap = (const uint16_t*)a.seg[0].A + (size_t)arow * a.seg[0].lda + q * 16;
#pragma unroll
        for (int j = 0; j < STEPS; ++j) {
            const int k = (wv + j * nw) << 6;
            av[2 * j] = *(const u32x4_t*)(Ap + k);
            av[2 * j + 1] = *(const u32x4_t*)(Ap + k + 8);
        }
#pragma unroll
        for (int j = 0; j < 2 * STEPS; ++j) av[j] = aval ? av[j] : zero;
    }
    const int t = threadIdx.x;
    for (int tile0 = blockIdx.x * TPI; tile0 < a.ntiles; tile0 += gridDim.x * TPI) {
        const uint16_t* Bp[TPI];
        bool bval[TPI];
        int n0[TPI];
        GemmSeg gs[TPI];
#pragma unroll
        for (int i = 0; i < TPI; ++i) {
            const int tile = min(tile0 + i, a.ntiles - 1);
            gs[i] = pair ? a.seg[wave / (NW / 2)] : a.seg[find_seg(a, tile)];
            n0[i] = (tile - gs[i].tile0) * 16;
            bval[i] = tile0 + i < a.ntiles && n0[i] + r < gs[i].N;
            Bp[i] = (const uint16_t*)gs[i].B + (size_t)(bval[i] ? n0[i] + r : 0) * gs[i].ldb + q * 16;
        }
        f32x4_t acc0[TPI], acc1[TPI];
#pragma unroll
        for (int i = 0; i < TPI; ++i) acc0[i] = acc1[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j0 = 0; j0 < STEPS; j0 += 4) {
            u32x4_t bv[TPI][8];
#pragma unroll
            for (int i = 0; i < TPI; ++i)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int k = (wv + (j0 + u) * nw) << 6;
                    bv[i][2 * u] = *(const u32x4_t*)(Bp[i] + k);
                    bv[i][2 * u + 1] = *(const u32x4_t*)(Bp[i] + k + 8);
                }
#pragma unroll
            for (int i = 0; i < TPI; ++i)
#pragma unroll
                for (int u = 0; u < 8; ++u) bv[i][u] = bval[i] ? bv[i][u] : zero;
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int i = 0; i < TPI; ++i) {
                    if (u & 1) {
                        acc1[i] = mfma32(av[2 * (j0 + u)], bv[i][2 * u], acc1[i]);
                        acc1[i] = mfma32(av[2 * (j0 + u) + 1], bv[i][2 * u + 1], acc1[i]);
                    } else {
                        acc0[i] = mfma32(av[2 * (j0 + u)], bv[i][2 * u], acc0[i]);
                        acc0[i] = mfma32(av[2 * (j0 + u) + 1], bv[i][2 * u + 1], acc0[i]);
                    }
                }
        }
#pragma unroll
        for (int i = 0; i < TPI; ++i) {
            const f32x4_t acc = acc0[i] + acc1[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) red[wave][i][lane * 4 + e] = acc[e];
        }
        __syncthreads();
        // threads 256 i .. 256 i + 255 finish tile i of the iteration
        const int i = t >> 8, m = (t & 255) >> 4, nn = t & 15;
        if (i < TPI && m < a.M && tile0 + i < a.ntiles) {
            // (selects, not a runtime index into the per-tile arrays, which
            // would put them in scratch memory)
            const int gN = (TPI == 2 && i) ? gs[TPI - 1].N : gs[0].N;
            const int gcol = (TPI == 2 && i) ? gs[TPI - 1].c_col0 : gs[0].c_col0;
            const int ni = (TPI == 2 && i) ? n0[TPI - 1] : n0[0];
            const int idx = (nn + 16 * (m >> 2)) * 4 + (m & 3);
            float s0 = 0.f;
            for (int w = 0; w < nw; ++w) s0 += red[w][i][idx];
            if (pair) {
                if (n0[0] + nn < a.seg[0].N) {
                    float s1 = 0.f;
                    for (int w = nw; w < NW; ++w) s1 += red[w][0][idx];
                    const float v = s0 / (1.f + __expf(-s0)) * s1;
                    const size_t o = (size_t)m * a.ldo + n0[0] + nn;
                    if (a.out_bf16) {
                        uint32_t u = __float_as_uint(v);
                        u += 0x7FFFu + ((u >> 16) & 1u);
                        ((uint16_t*)a.out)[o] = (uint16_t)(u >> 16);
                    } else {
                        ((float*)a.out)[o] = v;
                    }
                }
            } else if (ni + nn < gN) {
                float* p = a.C + (size_t)m * a.ldc + gcol + ni + nn;   // kPartial: split 0 of 1
                *p = a.mode == kAccumulate ? *p + s0 : s0;
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// tiled, pipelined (M > 16, K a multiple of 256): 128 x 128 output tiles, 4
// waves as 2 x 2 owning 64 x 64 each (4 x 4 MFMA tiles).  64-wide k tiles of
// A and B are copied straight into LDS (global_load_lds, no registers) into
// four stages, three ahead of the one being multiplied; each 128-byte row of
// a stage has its 16-byte pieces XOR-permuted by (row / 2) mod 8, so the 16
// rows of a fragment read fall on distinct banks.  The stages are separate
// LDS objects and the k loop is unrolled over them, so the compiler sees the
// copies into one stage as independent of the reads from another.
// ---------------------------------------------------------------------------
constexpr int kMtBM = 128, kMtBN = 128;

// per lane: the source rows (already offset to the lane's 16-byte piece) of
// the A and B pieces it copies into every stage
template <int BK>
struct MtRows {
    static constexpr int kInst = BK / 16;              // copy instructions per operand per wave
    const uint16_t* pa[kInst];
    const uint16_t* pb[kInst];
};

// 16-byte pieces of a BK-wide row are XOR-permuted by row / 2, so that the
// fragment reads (16 rows, one piece each) are free of bank conflicts: with
// 64-byte rows, row / 4 as the key left a two-way conflict in every read
// (rocprofv3 SQ_LDS_BANK_CONFLICT: 4.0 stall cycles per LDS instruction,
// 0 with row / 2)
template <int BK>
__device__ __forceinline__ int mt_swz(int row) {
    constexpr int P = BK / 8;                           // pieces per row
    return (row >> 1) & (P - 1);
}

template <int BK>
__device__ __forceinline__ int mt_off(int row, int piece) {
    return row * BK + ((piece ^ mt_swz<BK>(row)) << 3);
}

// one 16-byte piece per lane from global memory straight into LDS (the LDS
// destination is wave-uniform; lane l lands at dst + 16 l).  Kept out of the
// kernel templates: their host-side pass cannot compile the builtin.
__device__ __forceinline__ void dma16(const uint16_t* src, uint16_t* dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_void_t*)dst, 16, 0, 0);
}

__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)p;
}

__device__ __forceinline__ u32x4_t lds_read16(uint32_t addr) {
    u32x4_t v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}

// Work item (column tile, row tile, K split) of this workgroup.  Workgroups
// are dispatched round-robin over the 8 XCDs, each with its own L2; when the
// grid divides evenly, consecutive items (column tiles first, then row tiles,
// then splits: the items that share A rows) are gathered onto one XCD, so an
// XCD reads its K slice of A once from HBM and then from its L2.
struct TileItem {
    int tile, mt, split;
};
__device__ __forceinline__ TileItem tile_item(int xcd_remap) {
    const int nx = gridDim.x, ny = gridDim.y, total = nx * ny * gridDim.z;
    int l = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
    if (xcd_remap && (total & 7) == 0) l = (l & 7) * (total >> 3) + (l >> 3);
    const int r = l / nx;
    return TileItem{l - r * nx, r % ny, r / ny};
}

// PAIR: the gate|up projection with its SwiGLU epilogue.  Tile t covers gate
// columns [64 t, 64 t + 64) (segment 0, the waves with wn = 0) and the same
// up columns (segment 1, wn = 1); the up products pass through LDS and the
// gate waves store silu(gate) * up to the activation buffer.  One split.
template <int TAG, class GA, int BK, bool PAIR = false>
__global__ __launch_bounds__(256) void k_gemm_mt(GA a) {
    constexpr int KS = BK / 32;                         // 32-wide MFMA k steps per stage
    constexpr int NI = MtRows<BK>::kInst;
    __shared__ __attribute__((aligned(16))) uint16_t sA0[kMtBM * BK], sA1[kMtBM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sA2[kMtBM * BK], sA3[kMtBM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sB0[kMtBN * BK], sB1[kMtBN * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sB2[kMtBN * BK], sB3[kMtBN * BK];
    const TileItem it = tile_item(a.xcd_remap);
    const int tile = it.tile, mt = it.mt, split = it.split;
    const GemmSeg g = a.seg[find_seg(a, tile)];
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int wm = wave >> 1, wn = wave & 1, r = lane & 15, q = lane >> 4;
    const int m0 = mt * kMtBM, n0 = (tile - g.tile0) * kMtBN;
    MtRows<BK> c;
    {
        // lane l of a block stores piece position l % P of the block's row
        // l / P, which holds the logical piece that position maps to; rows
        // past M or N repeat the last one (computed, never stored)
        constexpr int P = BK / 8;
        const int rl = lane / P, pp = lane % P;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int row = (wave * NI + i) * (64 / P) + rl;
            const int lp = pp ^ mt_swz<BK>(row);
            const int am = min(m0 + row, a.M - 1);
            const int ar = a.a_rows ? a.a_rows[am] : am;
            c.pa[i] = (const uint16_t*)g.A + (size_t)ar * g.lda + lp * 8;
            if (PAIR) {   // rows 0..63 of the B tile: gate weights, 64..127: up weights
                const bool up = row >= 64;
                const uint16_t* Bb = (const uint16_t*)(up ? a.seg[1].B : a.seg[0].B);
                const int ldb = up ? a.seg[1].ldb : a.seg[0].ldb, nb = up ? a.seg[1].N : a.seg[0].N;
                c.pb[i] = Bb + (size_t)min(tile * 64 + (row & 63), nb - 1) * ldb + lp * 8;
            } else {
                c.pb[i] = (const uint16_t*)g.B + (size_t)min(n0 + row, g.N - 1) * g.ldb + lp * 8;
            }
        }
    }
    const int kb = split * a.kc, ke = min(a.K, kb + a.kc);
    const int nk = (ke - kb) / BK;
    // copy one BK-wide k tile of A and B into a stage: per operand 128 rows x
    // BK/8 pieces, i.e. BK/4 wave instructions of 64 pieces, NI per wave
    auto mt_load = [&](int k0, uint16_t* sA, uint16_t* sB) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int b = wave * NI + i;               // 1 KiB block of the stage
            dma16(c.pa[i] + k0, &sA[b * 512]);
            dma16(c.pb[i] + k0, &sB[b * 512]);
        }
    };

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // fragment reads are issued as inline asm: the compiler, which cannot tell
    // the stage being read from the stages being copied into, would otherwise
    // wait for every copy in flight before each read; here the reads of one
    // 32-wide k step are waited for (lgkmcnt) explicitly, tied to their values
    uint32_t offA[4], offB[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        offA[i] = (uint32_t)mt_off<BK>(wm * 64 + i * 16 + r, q) * 2;
        offB[i] = (uint32_t)mt_off<BK>(wn * 64 + i * 16 + r, q) * 2;
    }
    auto compute = [&](const uint16_t* tA, const uint16_t* tB) {
        const uint32_t baseA = lds_addr(tA), baseB = lds_addr(tB);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            // piece kk * 4 + q sits at (q ^ swz) ^ (kk * 4): the kk = 1 pieces
            // are the kk = 0 ones with bit 2 of the position flipped
            u32x4_t af[4], bf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = lds_read16(baseA + (offA[i] ^ (kk * 64)));
#pragma unroll
            for (int j = 0; j < 4; ++j) bf[j] = lds_read16(baseB + (offB[j] ^ (kk * 64)));
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(af[0]), "+v"(af[1]), "+v"(af[2]), "+v"(af[3]), "+v"(bf[0]), "+v"(bf[1]),
                           "+v"(bf[2]), "+v"(bf[3]));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
        }
    };
    // step kt: wait for its stage (the two stages after it stay in flight:
    // 2 NI copy instructions each per wave), then start the copy of tile
    // kt + 3 into the stage tile kt - 1 used, then multiply.  Copies are
    // issued unconditionally (past the end the last tile is fetched again,
    // unused) so the count of copies in flight is the same at every step.
    auto step = [&](int kt, const uint16_t* tA, const uint16_t* tB, uint16_t* nA, uint16_t* nB) {
        if constexpr (NI == 4) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        // a bare barrier: a fenced one would also wait for the later stages'
        // copies (the LDS reads of the previous step completed before their
        // MFMAs issued, so the stage refilled below is free)
        __builtin_amdgcn_s_barrier();
        mt_load(kb + min(kt + 3, nk - 1) * BK, nA, nB);
        compute(tA, tB);
    };
    if (nk > 0) {
        mt_load(kb, sA0, sB0);
        mt_load(kb + min(1, nk - 1) * BK, sA1, sB1);
        mt_load(kb + min(2, nk - 1) * BK, sA2, sB2);
    }
    for (int kt = 0; kt < nk; kt += 4) {          // nk is a multiple of 4 (the launcher's split)
        step(kt, sA0, sB0, sA3, sB3);
        step(kt + 1, sA1, sB1, sA0, sB0);
        step(kt + 2, sA2, sB2, sA1, sB1);
        step(kt + 3, sA3, sB3, sA2, sB2);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no copy may land after the workgroup ends
    if constexpr (PAIR) {
        // up products of wave (wm, 1) -> LDS (a finished stage per wm), then the
        // gate wave (wm, 0) of the same rows and columns applies SwiGLU
        __syncthreads();                                // every wave is done reading the stages
        float* xs = (float*)(wm == 0 ? sA0 : sA1);      // 64 x 64 floats = one 16 KiB stage
        if (wn == 1) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) xs[(i * 16 + 4 * q + e) * 64 + j * 16 + r] = acc[i][j][e];
        }
        __syncthreads();
        if (wn == 0) {
            const int I = a.seg[0].N;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int n = tile * 64 + j * 16 + r;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int m = m0 + wm * 64 + i * 16 + 4 * q + e;
                        if (n >= I || m >= a.M) continue;
                        const float gt = acc[i][j][e], up = xs[(i * 16 + 4 * q + e) * 64 + j * 16 + r];
                        const float v = gt / (1.f + __expf(-gt)) * up;
                        const size_t o = (size_t)m * a.ldo + n;
                        if (a.out_bf16) {
                            uint32_t u = __float_as_uint(v);
                            u += 0x7FFFu + ((u >> 16) & 1u);
                            ((uint16_t*)a.out)[o] = (uint16_t)(u >> 16);
                        } else {
                            ((float*)a.out)[o] = v;
                        }
                    }
                }
        }
        return;
    }
    // output (m, n) of MFMA tile (i, j): lane (r, q) holds rows 4 q + e of column r
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + wn * 64 + j * 16 + r;
            const bool nok = n < g.N;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + wm * 64 + i * 16 + 4 * q + e;
                if (nok && m < a.M) store_out(a, split, m, g.c_col0 + n, acc[i][j][e]);
            }
        }
}

// ---------------------------------------------------------------------------
// tiled, pipelined, 8 waves (M > 16): 256 x 128 output tiles, waves as 4 x 2
// owning 64 x 64 each.  A CU's L2 read rate grows with the waves issuing
// loads (about 45 GB/s with 4 waves, 85 with 8), and a 256 x 128 tile needs
// fewer bytes per flop than 128 x 128, so this form feeds the MFMAs better.
// 32-wide k tiles of A (16 KiB) and B (8 KiB) are copied straight into LDS,
// four stages, three in flight; pieces of a 64-byte row are XOR-permuted by
// (row / 2) mod 4.  Same read/wait scheme as k_gemm_mt.
// ---------------------------------------------------------------------------
constexpr int kW8BN = 128, kW8BK = 32;

// MI: 16-row MFMA tiles per wave along M (waves as 4 x 2): MI = 4 gives
// 256 x 128 output tiles (64 x 64 per wave), MI = 8 gives 512 x 128 (128 x 64
// per wave: all the rows of a batched unembedding in one tile, so every
// weight byte is read from HBM once, and twice the products per A/B byte in
// LDS).  Stages: 4 x (BM x 32 + 128 x 32) bf16 = 96 KiB (MI 4) or 160 KiB.
template <int MI>
struct W8 {
    static constexpr int BM = 64 * MI;
    static constexpr int ABLK = MI / 2;   // 1 KiB copies of A per wave per stage
};

template <int TAG, class GA, int MI>
__global__ __launch_bounds__(512) void k_gemm_w8(GA a) {
    constexpr int BM = W8<MI>::BM, ABLK = W8<MI>::ABLK;
    __shared__ __attribute__((aligned(16))) uint16_t sA0[BM * kW8BK], sA1[BM * kW8BK];
    __shared__ __attribute__((aligned(16))) uint16_t sA2[BM * kW8BK], sA3[BM * kW8BK];
    __shared__ __attribute__((aligned(16))) uint16_t sB0[kW8BN * kW8BK], sB1[kW8BN * kW8BK];
    __shared__ __attribute__((aligned(16))) uint16_t sB2[kW8BN * kW8BK], sB3[kW8BN * kW8BK];
    const TileItem it = tile_item(a.xcd_remap);
    const int tile = it.tile, mt = it.mt, split = it.split;
    const GemmSeg g = a.seg[find_seg(a, tile)];
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int wm = wave >> 1, wn = wave & 1, r = lane & 15, q = lane >> 4;
    const int m0 = mt * BM, n0 = (tile - g.tile0) * kW8BN;
    // copies per stage: A BM / 16 blocks of 16 rows (ABLK per wave), B 8
    // blocks (1 per wave); lane l of a block stores position l % 4 of row
    // l / 4, holding the logical piece (l % 4) ^ ((row / 2) % 4); rows past M
    // or N repeat the last
    const uint16_t* pa[ABLK];
    const uint16_t* pb;
    {
        const int rl = lane >> 2, pp = lane & 3;
#pragma unroll
        for (int i = 0; i < ABLK; ++i) {
            const int row = (wave * ABLK + i) * 16 + rl;
            const int am = min(m0 + row, a.M - 1);
            const int ar = a.a_rows ? a.a_rows[am] : am;
            pa[i] = (const uint16_t*)g.A + (size_t)ar * g.lda + ((pp ^ mt_swz<32>(row)) << 3);
        }
        const int row = wave * 16 + rl;
        pb = (const uint16_t*)g.B + (size_t)min(n0 + row, g.N - 1) * g.ldb + ((pp ^ mt_swz<32>(row)) << 3);
    }
    const int kb = split * a.kc, ke = min(a.K, kb + a.kc);
    const int nk = (ke - kb) / kW8BK;
    auto load = [&](int k0, uint16_t* sA, uint16_t* sB) {
#pragma unroll
        for (int i = 0; i < ABLK; ++i) dma16(pa[i] + k0, &sA[(wave * ABLK + i) * 512]);
        dma16(pb + k0, &sB[wave * 512]);
    };

    f32x4_t acc[MI][4];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    uint32_t offA[MI], offB[4];
#pragma unroll
    for (int i = 0; i < MI; ++i) offA[i] = (uint32_t)mt_off<32>(wm * (16 * MI) + i * 16 + r, q) * 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) offB[j] = (uint32_t)mt_off<32>(wn * 64 + j * 16 + r, q) * 2;
    auto compute = [&](const uint16_t* tA, const uint16_t* tB) {
        const uint32_t baseA = lds_addr(tA), baseB = lds_addr(tB);
        u32x4_t bf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) bf[j] = lds_read16(baseB + offB[j]);
        // A fragments four at a time (MI = 8: the second four are read while
        // the first four's products run)
#pragma unroll
        for (int i0 = 0; i0 < MI; i0 += 4) {
            u32x4_t af[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = lds_read16(baseA + offA[i0 + i]);
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(af[0]), "+v"(af[1]), "+v"(af[2]), "+v"(af[3]), "+v"(bf[0]), "+v"(bf[1]), "+v"(bf[2]),
                           "+v"(bf[3]));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i0 + i][j] = mfma32(af[i], bf[j], acc[i0 + i][j]);
        }
    };
    // step kt: its stage landed when at most the two later stages' copies
    // (ABLK + 1 instructions each per wave) are in flight; refill the stage of kt - 1
    auto step = [&](int kt, const uint16_t* tA, const uint16_t* tB, uint16_t* nA, uint16_t* nB) {
        if constexpr (ABLK == 2) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        load(kb + min(kt + 3, nk - 1) * kW8BK, nA, nB);
        compute(tA, tB);
    };
    static_assert(ABLK == 2 || ABLK == 4, "copy waits are written for 2 or 4 A blocks per wave");
    if (nk > 0) {
        load(kb, sA0, sB0);
        load(kb + min(1, nk - 1) * kW8BK, sA1, sB1);
        load(kb + min(2, nk - 1) * kW8BK, sA2, sB2);
    }
    for (int kt = 0; kt < nk; kt += 4) {          // nk is a multiple of 4 (the launcher's split)
        step(kt, sA0, sB0, sA3, sB3);
        step(kt + 1, sA1, sB1, sA0, sB0);
        step(kt + 2, sA2, sB2, sA1, sB1);
        step(kt + 3, sA3, sB3, sA2, sB2);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no copy may land after the workgroup ends
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + wn * 64 + j * 16 + r;
            const bool nok = n < g.N;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + wm * (16 * MI) + i * 16 + 4 * q + e;
                if (nok && m < a.M) store_out(a, split, m, g.c_col0 + n, acc[i][j][e]);
            }
        }
}

// ---------------------------------------------------------------------------
// k_gemm_w8 (256 x 128 tiles, 8 waves of 64 x 64) with 64-wide k tiles:
// every copy instruction moves whole 128-byte rows (8 rows x 128 bytes
// instead of 16 x 64), three stages of 48 KiB, two in flight; pieces of a
// row XOR-permuted by (row / 2) mod 8 as in k_gemm_mt.
// ---------------------------------------------------------------------------
constexpr int kW8KBK = 64, kW8KStage = (256 + kW8BN) * kW8KBK;

template <int TAG, class GA>
__global__ __launch_bounds__(512) void k_gemm_w8k(GA a) {
    constexpr int BM = 256, NA = 4, NB = 2;        // copy instructions per wave per stage (A, B)
    __shared__ __attribute__((aligned(16))) uint16_t smem[3 * kW8KStage];
    const TileItem it = tile_item(a.xcd_remap);
    const int tile = it.tile, mt = it.mt, split = it.split;
    const GemmSeg g = a.seg[find_seg(a, tile)];
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int wm = wave >> 1, wn = wave & 1, r = lane & 15, q = lane >> 4;
    const int m0 = mt * BM, n0 = (tile - g.tile0) * kW8BN;
    // lane l of a 1 KiB copy block stores position l % 8 of the block's row
    // l / 8, holding the logical piece (l % 8) ^ swz(row); rows past M or N
    // repeat the last one (computed, never stored)
    const uint16_t* pa[NA];
    const uint16_t* pb[NB];
    {
        const int rl = lane >> 3, pp = lane & 7;
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int row = (wave * NA + i) * 8 + rl;
            const int am = min(m0 + row, a.M - 1);
            const int ar = a.a_rows ? a.a_rows[am] : am;
            pa[i] = (const uint16_t*)g.A + (size_t)ar * g.lda + ((pp ^ mt_swz<kW8KBK>(row)) << 3);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int row = (wave * NB + i) * 8 + rl;
            pb[i] = (const uint16_t*)g.B + (size_t)min(n0 + row, g.N - 1) * g.ldb + ((pp ^ mt_swz<kW8KBK>(row)) << 3);
        }
    }
    const int kb = split * a.kc, ke = min(a.K, kb + a.kc);
    const int nk = (ke - kb) / kW8KBK;
    auto load = [&](int kt) {
        uint16_t* st = smem + (kt % 3) * kW8KStage;
        const int k0 = kb + min(kt, nk - 1) * kW8KBK;
#pragma unroll
        for (int i = 0; i < NA; ++i) dma16(pa[i] + k0, st + (wave * NA + i) * 512);
#pragma unroll
        for (int i = 0; i < NB; ++i) dma16(pb[i] + k0, st + BM * kW8KBK + (wave * NB + i) * 512);
    };
    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    uint32_t offA[4], offB[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        offA[i] = (uint32_t)mt_off<kW8KBK>(wm * 64 + i * 16 + r, q) * 2;
        offB[i] = (uint32_t)mt_off<kW8KBK>(BM + wn * 64 + i * 16 + r, q) * 2;
    }
    if (nk > 0) {
        load(0);
        load(1);
    }
    for (int kt = 0; kt < nk; ++kt) {
        // stage kt landed when only stage kt + 1's copies (6 per wave) are in
        // flight; the barrier also tells that every wave is done reading the
        // stage of kt - 1, which the copy of kt + 2 refills
        asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        load(kt + 2);
        const uint32_t base = lds_addr(smem + (kt % 3) * kW8KStage);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            // piece kk * 4 + q sits at (q ^ swz) ^ (kk * 4)
            u32x4_t af[4], bf[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) bf[j] = lds_read16(base + (offB[j] ^ (kk * 64)));
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = lds_read16(base + (offA[i] ^ (kk * 64)));
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(af[0]), "+v"(af[1]), "+v"(af[2]), "+v"(af[3]), "+v"(bf[0]), "+v"(bf[1]), "+v"(bf[2]),
                           "+v"(bf[3]));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no copy may land after the workgroup ends
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + wn * 64 + j * 16 + r;
            const bool nok = n < g.N;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + wm * 64 + i * 16 + 4 * q + e;
                if (nok && m < a.M) store_out(a, split, m, g.c_col0 + n, acc[i][j][e]);
            }
        }
}

// ---------------------------------------------------------------------------
// 8 waves on 256 x 256 tiles (waves as 2 x 4, 128 x 64 each: the wave tile
// of k_gemm_w8<8>).  Per 32-wide k step a workgroup copies 32 KiB (A and B
// 16 KiB each) for the products that cost k_gemm_w8<8> 40 KiB, and these
// GEMMs are bound by the copies into LDS.  Used for the batched unembedding:
// the row tiles of one column tile are consecutive work items (dispatched
// together, so the weight tile is fetched from HBM once), and the grid is
// padded to a multiple of 8 so that they share an XCD.  Four stages of
// 32 KiB, three in flight; same read/wait scheme as k_gemm_mt.
// ---------------------------------------------------------------------------
constexpr int kSqB = 256;

template <int TAG, class GA>
__global__ __launch_bounds__(512) void k_gemm_sq(GA a) {
    constexpr int BK = kW8BK, MI = 8, SA = kSqB * BK;
    __shared__ __attribute__((aligned(16))) uint16_t sA0[SA], sA1[SA], sA2[SA], sA3[SA];
    __shared__ __attribute__((aligned(16))) uint16_t sB0[SA], sB1[SA], sB2[SA], sB3[SA];
    // item l: row tile fastest, then column tile; consecutive items on one XCD
    const int mtiles = (a.M + kSqB - 1) / kSqB, items = a.ntiles * mtiles;
    const int total = gridDim.x;   // items rounded up to a multiple of 8
    int l = blockIdx.x;
    l = (l & 7) * (total >> 3) + (l >> 3);
    if (l >= items) return;
    const int mt = l % mtiles, tile = l / mtiles;
    const GemmSeg g = a.seg[find_seg(a, tile)];
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int wm = wave >> 2, wn = wave & 3, r = lane & 15, q = lane >> 4;
    const int m0 = mt * kSqB, n0 = (tile - g.tile0) * kSqB;
    // copies per stage: A and B 16 blocks of 16 rows each, two of each per
    // wave; lane l of a block stores position l % 4 of row l / 4, holding the
    // logical piece (l % 4) ^ ((row / 2) % 4); rows past M or N repeat the last
    const uint16_t* pa[2];
    const uint16_t* pb[2];
    {
        const int rl = lane >> 2, pp = lane & 3;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = (wave * 2 + i) * 16 + rl;
            const int am = min(m0 + row, a.M - 1);
            const int ar = a.a_rows ? a.a_rows[am] : am;
            pa[i] = (const uint16_t*)g.A + (size_t)ar * g.lda + ((pp ^ mt_swz<32>(row)) << 3);
            pb[i] = (const uint16_t*)g.B + (size_t)min(n0 + row, g.N - 1) * g.ldb + ((pp ^ mt_swz<32>(row)) << 3);
        }
    }
    const int nk = a.K / BK;   // the launcher checks K % 128 == 0
    auto load = [&](int k0, uint16_t* sA, uint16_t* sB) {
#pragma unroll
        for (int i = 0; i < 2; ++i) dma16(pa[i] + k0, &sA[(wave * 2 + i) * 512]);
#pragma unroll
        for (int i = 0; i < 2; ++i) dma16(pb[i] + k0, &sB[(wave * 2 + i) * 512]);
    };
    f32x4_t acc[MI][4];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    uint32_t offA[MI], offB[4];
#pragma unroll
    for (int i = 0; i < MI; ++i) offA[i] = (uint32_t)mt_off<32>(wm * (16 * MI) + i * 16 + r, q) * 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) offB[j] = (uint32_t)mt_off<32>(wn * 64 + j * 16 + r, q) * 2;
    auto compute = [&](const uint16_t* tA, const uint16_t* tB) {
        const uint32_t baseA = lds_addr(tA), baseB = lds_addr(tB);
        u32x4_t bf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) bf[j] = lds_read16(baseB + offB[j]);
#pragma unroll
        for (int i0 = 0; i0 < MI; i0 += 4) {
            u32x4_t af[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = lds_read16(baseA + offA[i0 + i]);
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(af[0]), "+v"(af[1]), "+v"(af[2]), "+v"(af[3]), "+v"(bf[0]), "+v"(bf[1]), "+v"(bf[2]),
                           "+v"(bf[3]));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i0 + i][j] = mfma32(af[i], bf[j], acc[i0 + i][j]);
        }
    };
    // step kt: its stage landed when at most the two later stages' copies (4
    // instructions each per wave) are in flight; refill the stage of kt - 1
    auto step = [&](int kt, const uint16_t* tA, const uint16_t* tB, uint16_t* nA, uint16_t* nB) {
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        load(min(kt + 3, nk - 1) * BK, nA, nB);
        compute(tA, tB);
    };
    if (nk > 0) {
        load(0, sA0, sB0);
        load(min(1, nk - 1) * BK, sA1, sB1);
        load(min(2, nk - 1) * BK, sA2, sB2);
    }
    for (int kt = 0; kt < nk; kt += 4) {          // nk is a multiple of 4
        step(kt, sA0, sB0, sA3, sB3);
        step(kt + 1, sA1, sB1, sA0, sB0);
        step(kt + 2, sA2, sB2, sA1, sB1);
        step(kt + 3, sA3, sB3, sA2, sB2);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no copy may land after the workgroup ends
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + wn * 64 + j * 16 + r;
            const bool nok = n < g.N;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + wm * (16 * MI) + i * 16 + 4 * q + e;
                if (nok && m < a.M) store_out(a, 0, m, g.c_col0 + n, acc[i][j][e]);
            }
        }
}

// ---------------------------------------------------------------------------
// tiled: MT x 128 tiles, KT = 64, LDS double buffer
// ---------------------------------------------------------------------------
template <int MT, int TAG, class GA>
__global__ __launch_bounds__(256) void k_gemm_tiled(GA a) {
    constexpr int NT = 128, KT = 64, LDS_LD = KT + 8;
    constexpr int AL = MT / 32, BL = NT / 32;      // 16-byte loads per thread
    constexpr int TM = MT / 32, TN = 4;            // 16x16 tiles per wave
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][MT * LDS_LD];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][NT * LDS_LD];

    const int tile = blockIdx.x, mt = blockIdx.y, split = blockIdx.z;
    const GemmSeg g = a.seg[find_seg(a, tile)];
    const int n0 = (tile - g.tile0) * NT, m0 = mt * MT;
    const int kb = split * a.kc, ke = min(a.K, kb + a.kc);
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int wm = wave >> 1, wn = wave & 1, r = lane & 15, q = lane >> 4;
    const int lrow = t >> 3, lcol = (t & 7) * 8;
    const u32x4_t zero = {0u, 0u, 0u, 0u};

    const uint16_t* Ag = (const uint16_t*)g.A;
    const uint16_t* Bg = (const uint16_t*)g.B;
    u32x4_t ra[AL], rb[BL];
#define DF_LOAD_TILE(k)                                                                         \
    do {                                                                                        \
        _Pragma("unroll") for (int i = 0; i < AL; ++i) {                                        \
            const int row_ = m0 + lrow + 32 * i;                                                \
            const int ar_ = min(row_, a.M - 1);                                                 \
            const u32x4_t v_ = *(const u32x4_t*)(Ag + (size_t)(a.a_rows ? a.a_rows[ar_] : ar_) * g.lda + (k) + lcol); \
            ra[i] = row_ < a.M ? v_ : zero;                                                     \
        }                                                                                       \
        _Pragma("unroll") for (int i = 0; i < BL; ++i) {                                        \
            const int row_ = n0 + lrow + 32 * i;                                                \
            const u32x4_t v_ = *(const u32x4_t*)(Bg + (size_t)min(row_, g.N - 1) * g.ldb + (k) + lcol); \
            rb[i] = row_ < g.N ? v_ : zero;                                                     \
        }                                                                                       \
    } while (0)
#define DF_STORE_TILE(buf)                                                                      \
    do {                                                                                        \
        _Pragma("unroll") for (int i = 0; i < AL; ++i)                                          \
            *(u32x4_t*)&sA[buf][(lrow + 32 * i) * LDS_LD + lcol] = ra[i];                         \
        _Pragma("unroll") for (int i = 0; i < BL; ++i)                                          \
            *(u32x4_t*)&sB[buf][(lrow + 32 * i) * LDS_LD + lcol] = rb[i];                         \
    } while (0)

    f32x4_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nk = (ke - kb + KT - 1) / KT;
    if (nk > 0) {
        DF_LOAD_TILE(kb);
        DF_STORE_TILE(0);
    }
    __syncthreads();
    for (int it = 0; it < nk; ++it) {
        const int buf = it & 1;
        if (it + 1 < nk) DF_LOAD_TILE(kb + (it + 1) * KT);
#pragma unroll
        for (int kk = 0; kk < KT; kk += 32) {
            u32x4_t af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = *(const u32x4_t*)&sA[buf][(wm * (MT / 2) + i * 16 + r) * LDS_LD + kk + q * 8];
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bf[j] = *(const u32x4_t*)&sB[buf][(wn * 64 + j * 16 + r) * LDS_LD + kk + q * 8];
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
        }
        if (it + 1 < nk) DF_STORE_TILE(buf ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = n0 + wn * 64 + j * 16 + r;
            const bool nok = n < g.N;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + wm * (MT / 2) + i * 16 + 4 * q + e;
                if (nok && m < a.M) store_out(a, split, m, g.c_col0 + n, acc[i][j][e]);
            }
        }
#undef DF_LOAD_TILE
#undef DF_STORE_TILE
}

// ---------------------------------------------------------------------------
// fp32: one thread per output element
// ---------------------------------------------------------------------------
template <class GA>
__global__ __launch_bounds__(64) void k_gemm_f32(GA a) {
    const int col = a.col_lo + blockIdx.x * 64 + threadIdx.x;
    const int m = blockIdx.y;
    if (col >= a.col_hi) return;
    int s = 0;
    for (int j = 1; j < a.nseg; ++j)
        if (col >= a.seg[j].c_col0) s = j;
    const GemmSeg g = a.seg[s];
    const int n = col - g.c_col0;
    if (n < 0 || n >= g.N) return;
    const float* A = (const float*)g.A + (size_t)(a.a_rows ? a.a_rows[m] : m) * g.lda;
    const float* B = (const float*)g.B + (size_t)n * g.ldb;
    float acc = 0.f;
    for (int k = 0; k < a.K; ++k) acc = fmaf(A[k], B[k], acc);
    float* p = a.C + (size_t)m * a.ldc + col;
    *p = a.accumulate ? *p + acc : acc;
}

template <class GA>
__global__ __launch_bounds__(256) void k_splitk_reduce(GA a) {
    const int width = a.col_hi - a.col_lo;
    const size_t total = (size_t)a.M * width;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
        const int m = (int)(i / width), col = a.col_lo + (int)(i % width);
        float s = 0.f;
        for (int sp = 0; sp < a.splits; ++sp) s += a.part[((size_t)sp * a.M + m) * a.ldc + col];
        float* p = a.C + (size_t)m * a.ldc + col;
        *p = a.accumulate ? *p + s : s;
    }
}

// ---------------------------------------------------------------------------
// launcher: tiles, split-K choice, reduce
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_swiglu(const float* in, int32_t ld, int32_t I, void* out, int32_t ldo,
                                                int32_t out_bf16, int32_t rows) {
    const size_t total = (size_t)rows * I;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
        const int r = (int)(i / I), j = (int)(i % I);
        const float gt = in[(size_t)r * ld + j];
        const float up = in[(size_t)r * ld + I + j];
        const float v = gt / (1.f + __expf(-gt)) * up;
        const size_t o = (size_t)r * ldo + j;
        if (out_bf16) {
            uint32_t u = __float_as_uint(v);
            u += 0x7FFFu + ((u >> 16) & 1u);
            ((uint16_t*)out)[o] = (uint16_t)(u >> 16);
        } else {
            ((float*)out)[o] = v;
        }
    }
}

template <class GA, int TPW, int TAG>
static void launch_skinny_b(int batch, dim3 grid, hipStream_t st, const GA& a) {
    switch (batch) {
        case 1: hipLaunchKernelGGL((k_gemm_skinny<TPW, TAG, GA, 1>), grid, dim3(512), 0, st, a); break;
        case 2: hipLaunchKernelGGL((k_gemm_skinny<TPW, TAG, GA, 2>), grid, dim3(512), 0, st, a); break;
        case 3: hipLaunchKernelGGL((k_gemm_skinny<TPW, TAG, GA, 3>), grid, dim3(512), 0, st, a); break;
        default: hipLaunchKernelGGL((k_gemm_skinny<TPW, TAG, GA, 4>), grid, dim3(512), 0, st, a); break;
    }
}

template <class GA>
static hipError_t launch_skinny(int tpw, int tag, int batch, dim3 grid, hipStream_t st, const GA& a) {
    if (tpw == 2) {
        if (tag == 1) launch_skinny_b<GA, 2, 1>(batch, grid, st, a);
        else launch_skinny_b<GA, 2, 0>(batch, grid, st, a);
    } else {
        if (tag == 1) launch_skinny_b<GA, 1, 1>(batch, grid, st, a);
        else launch_skinny_b<GA, 1, 0>(batch, grid, st, a);
    }
    return hipGetLastError();
}

template <class GA>
static hipError_t gemm_impl(GA a, bool bf16, size_t part_cap_floats, int num_cus, hipStream_t st, int tag,
                            int* splits_out) {
    if (a.M <= 0 || a.nseg <= 0) return hipSuccess;
    a.accumulate = a.mode == kAccumulate;
    a.col_lo = a.seg[0].c_col0;
    a.col_hi = a.seg[a.nseg - 1].c_col0 + a.seg[a.nseg - 1].N;
    const bool swiglu = a.mode == kSwiGLU;
    const bool skinny = bf16 && a.M <= 16;
    if (skinny) {
        int ntiles = 0;
        if (swiglu) {
            ntiles = (a.seg[0].N + 15) / 16;
            a.seg[0].tile0 = a.seg[1].tile0 = 0;
        } else {
            for (int s = 0; s < a.nseg; ++s) {
                a.seg[s].tile0 = ntiles;
                ntiles += (a.seg[s].N + 15) / 16;
            }
        }
        a.ntiles = ntiles;
        a.splits = 1;
        a.kc = a.K;
        // persistent form when every segment shares one A and each wave's k
        // share fits in registers (4 or 8 steps of 64)
        bool shared_a = true;
        for (int s = 1; s < a.nseg; ++s) shared_a &= a.seg[s].A == a.seg[0].A && a.seg[s].lda == a.seg[0].lda;
        const int nw = swiglu ? kSkWaves / 2 : kSkWaves;
        const int steps = (a.K % (64 * nw)) ? 0 : a.K / (64 * nw);
        const int grid = std::min(ntiles, 2 * num_cus);   // persistent grid
        // (only when every workgroup gets at least two tiles; otherwise the
        // per-tile kernel, with more workgroups in flight, is faster)
        if (shared_a && (steps == 4 || steps == 8) && ntiles >= 2 * grid) {
            if (splits_out) *splits_out = 1;
            // two tiles per iteration (the reduction and its barriers serve
            // twice the bytes): four k steps per wave on 8 waves (K = 2048:
            // the 151936-token unembedding 124.2 -> 122.1 us); at K = 4096 the
            // 8-wave form would need eight steps (172 VGPRs with two tiles, one
            // workgroup per CU), so 16 waves of four steps, one workgroup per
            // CU resident at once (the 262144-token unembedding 369 -> 345 us);
            // the paired SwiGLU form takes one tile on 8 waves
            if (steps == 4 && !swiglu) {
                const dim3 g2((unsigned)std::min(2 * num_cus, (ntiles + 1) / 2));
                if (tag == 1) hipLaunchKernelGGL((k_gemm_skinny_p<4, 1, GA, 2, 8>), g2, dim3(512), 0, st, a);
                else hipLaunchKernelGGL((k_gemm_skinny_p<4, 0, GA, 2, 8>), g2, dim3(512), 0, st, a);
            } else if (steps == 4) {
                hipLaunchKernelGGL((k_gemm_skinny_p<4, 0, GA, 1, 8>), dim3(grid), dim3(512), 0, st, a);
            } else if (!swiglu) {
                const dim3 g16((unsigned)std::min(num_cus, (ntiles + 1) / 2));
                if (tag == 1) hipLaunchKernelGGL((k_gemm_skinny_p<4, 1, GA, 2, 16>), g16, dim3(1024), 0, st, a);
                else hipLaunchKernelGGL((k_gemm_skinny_p<4, 0, GA, 2, 16>), g16, dim3(1024), 0, st, a);
            } else {
                hipLaunchKernelGGL((k_gemm_skinny_p<8, 0, GA, 1, 8>), dim3(grid), dim3(512), 0, st, a);
            }
            return hipGetLastError();
        }
        // two tiles per workgroup when they share A (the A loads of a k step
        // serve both); kPartial: split K over workgroups while the grid stays
        // within four workgroups per CU and every wave keeps a k step (measured
        // on the M = 16 block shapes: more, shorter workgroups beat fewer, longer
        // ones until the splits leave waves idle)
        const int tpw = swiglu ? 2 : (shared_a ? 2 : 1);
        const int nwg = swiglu ? ntiles : (ntiles + tpw - 1) / tpw;
        int splits = 1;
        const int nsteps = a.K / 64;
        while (a.mode == kPartial && nwg * splits * 2 <= 4 * num_cus && nsteps / (splits * 2) >= kSkWaves &&
               splits * 2 <= a.max_splits)
            splits *= 2;
        a.splits = splits;
        if (splits_out) *splits_out = splits;
        const dim3 grid2(nwg, splits);
        const int spw = ((nsteps + splits - 1) / splits + kSkWaves - 1) / kSkWaves;   // k steps per wave
        const int batch = std::max(1, std::min(4, spw));
        return launch_skinny<GA>(tpw, tag, batch, grid2, st, a);
    }
    // larger M (or fp32): plain GEMM into C, then the SwiGLU pass if asked;
    // kPartial leaves the split partials [splits][M][ldc] in C
    if (swiglu) a.accumulate = 0;
    if (splits_out) *splits_out = 1;
    hipError_t e = hipSuccess;
    if (!bf16) {
        a.splits = 1;
        a.kc = a.K;
        a.accumulate = a.mode == kAccumulate;
        dim3 grid((a.col_hi - a.col_lo + 63) / 64, a.M);
        hipLaunchKernelGGL(k_gemm_f32<GA>, grid, dim3(64), 0, st, a);
        e = hipGetLastError();
    } else {
        // kernels: k_gemm_w8 (256 x 128 tiles, 8 waves) when the column tiles
        // alone give at least half a workgroup per CU, with 512 x 128 tiles
        // when M fits one and there are two column tiles per CU or more (a
        // batched unembedding: the weights are read once); else k_gemm_mt
        // (128 x 128, 4 waves) with K split to about one workgroup per CU;
        // all take K in groups of four stages.  k_gemm_tiled otherwise.
        // 257..512 rows over many columns (the batched unembedding): 256 x 256
        // tiles, each weight tile fetched once for both row tiles
        if (a.M > kSqB && a.M <= 2 * kSqB && a.K % 128 == 0 && (a.mode == kStore || a.mode == kAccumulate)) {
            int nt = 0;
            for (int s = 0; s < a.nseg; ++s) nt += (a.seg[s].N + kSqB - 1) / kSqB;
            if (nt >= num_cus) {
                nt = 0;
                for (int s = 0; s < a.nseg; ++s) {
                    a.seg[s].tile0 = nt;
                    nt += (a.seg[s].N + kSqB - 1) / kSqB;
                }
                a.ntiles = nt;
                a.splits = 1;
                a.kc = a.K;
                const int items = nt * 2;
                const dim3 grid((items + 7) / 8 * 8);
                if (tag == 1) hipLaunchKernelGGL((k_gemm_sq<1, GA>), grid, dim3(512), 0, st, a);
                else hipLaunchKernelGGL((k_gemm_sq<0, GA>), grid, dim3(512), 0, st, a);
                return hipGetLastError();
            }
        }
        const bool pipelined = a.K % 256 == 0;
        const int NT = 128;
        int ntiles = 0;
        for (int s = 0; s < a.nseg; ++s) {
            a.seg[s].tile0 = ntiles;
            ntiles += (a.seg[s].N + NT - 1) / NT;
        }
        a.ntiles = ntiles;
        // gate|up with SwiGLU: 128-row tiles pairing 64 gate and 64 up columns,
        // the epilogue writing the activations (no fp32 gate|up round trip
        // and no separate SwiGLU pass), when the pairs alone give at least one
        // workgroup per CU (no K split)
        if (swiglu && pipelined && a.nseg == 2 && a.seg[0].A == a.seg[1].A && a.seg[0].N == a.seg[1].N) {
            const int pt = (a.seg[0].N + 63) / 64, mtl = (a.M + kMtBM - 1) / kMtBM;
            if (pt * mtl >= num_cus) {
                a.seg[0].tile0 = a.seg[1].tile0 = 0;
                a.ntiles = pt;
                a.splits = 1;
                a.kc = a.K;
                a.xcd_remap = 1;
                const dim3 grid3(pt, mtl, 1);
                if (tag == 1) hipLaunchKernelGGL((k_gemm_mt<1, GA, 64, true>), grid3, dim3(256), 0, st, a);
                else hipLaunchKernelGGL((k_gemm_mt<0, GA, 64, true>), grid3, dim3(256), 0, st, a);
                return hipGetLastError();
            }
        }
        const bool w8big = pipelined && a.M > W8<4>::BM && a.M <= W8<8>::BM && ntiles >= 2 * num_cus;
        const size_t cap = a.mode == kPartial ? (size_t)a.max_splits * a.M * a.ldc : part_cap_floats;
        const int max_s = a.mode == kPartial ? a.max_splits : 1 << 30;
        // power-of-two K splits while the grid stays within one workgroup per
        // CU and a split keeps >= 512 k-values, within the partial slices
        auto pow2_splits = [&](int base) {
            int sp = 1;
            while (base * sp * 2 <= num_cus && a.K / (sp * 2) >= 512) sp *= 2;
            while (sp > 1 && ((size_t)sp * a.M * a.ldc > cap || sp > max_s)) sp /= 2;
            return sp;
        };
        // the tile form: 128 x 128 (k_gemm_mt, 4 waves) or 256 x 128
        // (k_gemm_w8, 8 waves; K slices of any count in kPartial mode) by a
        // cost model that fits the measured shapes: one workgroup per CU is
        // resident, so a launch takes rounds of resident workgroups x (a
        // fixed start-up of ~1e7 multiply-adds' time + the multiply-adds of
        // a workgroup), the 8-wave form ~7% faster per multiply-add.  It keeps
        // 128-row tiles where 256-row ones would be mostly padding (a
        // 551-row block: qkv 35.5 us on 256-row tiles) or too few, and takes
        // 256-row tiles where K slices fill the CUs (the context k|v
        // projection, 24.3 vs 26.5 us; the 4096-wide fc, 66 vs 70 us)
        auto cost = [&](int BM, int sp, int kq_, double rate) {
            const int kc_ = ((a.K + sp - 1) / sp + kq_ - 1) / kq_ * kq_;
            const int n_sp = (a.K + kc_ - 1) / kc_;
            const long wgs = (long)ntiles * ((a.M + BM - 1) / BM) * n_sp;
            const long rounds = (wgs + num_cus - 1) / num_cus;
            return (double)rounds * (1e7 + (double)BM * 128 * kc_ / rate);
        };
        bool w8 = false;
        int MT, kq, splits;
        if (w8big) {
            MT = W8<8>::BM;
            kq = 256;
            splits = pow2_splits(ntiles * ((a.M + MT - 1) / MT));
        } else if (!pipelined) {
            MT = a.M <= 64 ? 64 : 128;
            kq = 64;
            splits = pow2_splits(ntiles * ((a.M + MT - 1) / MT));
        } else {
            MT = kMtBM;
            kq = 256;
            splits = pow2_splits(ntiles * ((a.M + kMtBM - 1) / kMtBM));
            if (a.M > kMtBM) {
                const int b8 = ntiles * ((a.M + W8<4>::BM - 1) / W8<4>::BM);
                int s8 = pow2_splits(b8);
                if (a.mode == kPartial) {
                    s8 = std::max(1, std::min(a.max_splits, num_cus / b8));
                    while (s8 > 1 && a.K / s8 < 512) --s8;
                }
                const double c_mt = cost(kMtBM, splits, 256, 1.0), c_w8 = cost(W8<4>::BM, s8, 128, 1.07);
                if (c_w8 < c_mt || (c_w8 == c_mt && s8 <= splits)) {
                    w8 = true;
                    MT = W8<4>::BM;
                    kq = 128;
                    splits = s8;
                }
            }
        }
        const int mtiles = (a.M + MT - 1) / MT;
        int kc = ((a.K + splits - 1) / splits + kq - 1) / kq * kq;
        splits = (a.K + kc - 1) / kc;
        a.splits = splits;
        a.kc = kc;
        a.xcd_remap = 1;
        if (a.mode == kPartial) {
            a.part = a.C;            // the partial slices are the output
            if (splits_out) *splits_out = splits;
        }
        const dim3 blk(256), grid3(ntiles, mtiles, splits);
        if (w8big) {
            if (tag == 1) hipLaunchKernelGGL((k_gemm_w8<1, GA, 8>), grid3, dim3(512), 0, st, a);
            else hipLaunchKernelGGL((k_gemm_w8<0, GA, 8>), grid3, dim3(512), 0, st, a);
        } else if (w8 && kc >= 1024) {
            // K slices of 16 or more 64-wide steps: whole 128-byte rows per
            // copy (the long flush's fc 66.9 -> 57.9 us, k|v 40.1 -> 37.0 by
            // events; at 8-12 steps the extra pipeline fill loses: 18.0 ->
            // 18.8 us at 487 x 4096 -> 2048, qwen's k|v 26.6 -> 27.4)
            if (tag == 1) hipLaunchKernelGGL((k_gemm_w8k<1, GA>), grid3, dim3(512), 0, st, a);
            else hipLaunchKernelGGL((k_gemm_w8k<0, GA>), grid3, dim3(512), 0, st, a);
        } else if (w8) {
            if (tag == 1) hipLaunchKernelGGL((k_gemm_w8<1, GA, 4>), grid3, dim3(512), 0, st, a);
            else hipLaunchKernelGGL((k_gemm_w8<0, GA, 4>), grid3, dim3(512), 0, st, a);
        } else if (pipelined) {
            if (tag == 1) hipLaunchKernelGGL((k_gemm_mt<1, GA, 64>), grid3, blk, 0, st, a);
            else hipLaunchKernelGGL((k_gemm_mt<0, GA, 64>), grid3, blk, 0, st, a);
        } else if (MT == 64) {
            if (tag == 1) hipLaunchKernelGGL((k_gemm_tiled<64, 1, GA>), grid3, blk, 0, st, a);
            else hipLaunchKernelGGL((k_gemm_tiled<64, 0, GA>), grid3, blk, 0, st, a);
        } else {
            if (tag == 1) hipLaunchKernelGGL((k_gemm_tiled<128, 1, GA>), grid3, blk, 0, st, a);
            else hipLaunchKernelGGL((k_gemm_tiled<128, 0, GA>), grid3, blk, 0, st, a);
        }
        e = hipGetLastError();
        if (e == hipSuccess && splits > 1 && a.mode != kPartial) {
            const size_t total = (size_t)a.M * (a.col_hi - a.col_lo);
            const int blocks = (int)std::min<size_t>((total + 255) / 256, (size_t)num_cus * 8);
            hipLaunchKernelGGL(k_splitk_reduce<GA>, dim3(blocks), dim3(256), 0, st, a);
            e = hipGetLastError();
        }
    }
    if (e != hipSuccess || !swiglu) return e;
    const int I = a.seg[0].N;
    const size_t total = (size_t)a.M * I;
    const int blocks = (int)std::min<size_t>((total + 255) / 256, 4096);
    hipLaunchKernelGGL(k_swiglu, dim3(blocks), dim3(256), 0, st, a.C, a.ldc, I, a.out, a.ldo, a.out_bf16, a.M);
    return hipGetLastError();
}

hipError_t gemm(GemmArgs a, bool bf16, size_t part_cap_floats, int num_cus, hipStream_t st, int tag,
                int* splits_out) {
    if (a.nseg > kFewSeg) return gemm_impl(a, bf16, part_cap_floats, num_cus, st, tag, splits_out);
    GemmArgsT<kFewSeg> b{};
    static_cast<GemmHead&>(b) = a;
    for (int s = 0; s < kFewSeg; ++s) b.seg[s] = a.seg[s];
    return gemm_impl(b, bf16, part_cap_floats, num_cus, st, tag, splits_out);
}

}  // namespace kern
}  // namespace dflash
