// GEMMs of the drafter forward: C (+)= A . B^T with A = activations [M, K]
// and B = a weight [N, K] (row-major, out x in), several weights per launch
// as column segments (q|k|v|g, gate|up, every layer's k|v).
//
//  * k_gemm_skinny   M <= 16 (block path).  Each wave owns 16 output columns
//    and streams its weight rows straight from HBM into MFMA operands
//    (v_mfma_f32_16x16x32_bf16); weights are read exactly once, so the kernel
//    is HBM-bound and split-K supplies enough waves to fill 256 CUs.
//  * k_gemm_tiled    M > 16 (256-row flushes, batched blocks).  64|128 x 128
//    tiles, 4 waves as 2x2, A and B staged through LDS with double buffering.
//  * k_gemm_f32      the fp32 configuration (tiny shapes), plain FMA.
//
// Split-K partials go to a workspace slice and a reduce kernel writes C.
#include "kernels.h"

namespace dflash {
namespace kern {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;   // 16-byte operand piece

__device__ __forceinline__ f32x4_t mfma32(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ int find_seg(const GemmArgs& a, int tile) {
    int s = 0;
    for (int j = 1; j < a.nseg; ++j)
        if (tile >= a.seg[j].tile0) s = j;
    return s;
}

__device__ __forceinline__ void store_out(const GemmArgs& a, int split, int m, int col, float v) {
    if (a.splits == 1) {
        float* p = a.C + (size_t)m * a.ldc + col;
        *p = a.accumulate ? *p + v : v;
    } else {
        a.part[((size_t)split * a.M + m) * a.ldc + col] = v;
    }
}

// ---------------------------------------------------------------------------
// skinny: M <= 16, 64 columns per workgroup (16 per wave)
// ---------------------------------------------------------------------------
template <int TAG>
__global__ __launch_bounds__(256) void k_gemm_skinny(GemmArgs a) {
    const int tile = blockIdx.x, split = blockIdx.y;
    const GemmSeg g = a.seg[find_seg(a, tile)];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n0 = (tile - g.tile0) * 64 + wave * 16;
    if (n0 >= g.N) return;
    const int r = lane & 15, q = lane >> 4;
    const bool bval = n0 + r < g.N, aval = r < a.M;
    const int kb = split * a.kc, ke = min(a.K, kb + a.kc);
    // lane (r, q) reads 32 contiguous bytes of row r at k + 16q: both MFMAs of
    // a 64-wide k step see the same k assignment for A and B
    const uint16_t* Bp = (const uint16_t*)g.B + (size_t)(bval ? n0 + r : 0) * g.ldb + q * 16;
    const uint16_t* Ap = (const uint16_t*)g.A + (size_t)(aval ? r : 0) * g.lda + q * 16;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
    int k = kb;
    for (; k + 256 <= ke; k += 256) {
        u32x4_t bv[8], av[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            bv[2 * u] = *(const u32x4_t*)(Bp + k + 64 * u);
            bv[2 * u + 1] = *(const u32x4_t*)(Bp + k + 64 * u + 8);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            av[2 * u] = *(const u32x4_t*)(Ap + k + 64 * u);
            av[2 * u + 1] = *(const u32x4_t*)(Ap + k + 64 * u + 8);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (!bval) bv[u] = zero;
            if (!aval) av[u] = zero;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (u & 1) {
                acc1 = mfma32(av[2 * u], bv[2 * u], acc1);
                acc1 = mfma32(av[2 * u + 1], bv[2 * u + 1], acc1);
            } else {
                acc0 = mfma32(av[2 * u], bv[2 * u], acc0);
                acc0 = mfma32(av[2 * u + 1], bv[2 * u + 1], acc0);
            }
        }
    }
    for (; k < ke; k += 64) {
        u32x4_t b0 = *(const u32x4_t*)(Bp + k), b1 = *(const u32x4_t*)(Bp + k + 8);
        u32x4_t a0 = *(const u32x4_t*)(Ap + k), a1 = *(const u32x4_t*)(Ap + k + 8);
        if (!bval) b0 = b1 = zero;
        if (!aval) a0 = a1 = zero;
        acc0 = mfma32(a0, b0, acc0);
        acc0 = mfma32(a1, b1, acc0);
    }
    const f32x4_t acc = acc0 + acc1;
    if (!bval) return;
    const int col = g.c_col0 + n0 + r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int m = 4 * q + e;
        if (m < a.M) store_out(a, split, m, col, acc[e]);
    }
}

// ---------------------------------------------------------------------------
// tiled: MT x 128 tiles, KT = 64, LDS double buffer
// ---------------------------------------------------------------------------
template <int MT, int TAG>
__global__ __launch_bounds__(256) void k_gemm_tiled(GemmArgs a) {
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
            const u32x4_t v_ = *(const u32x4_t*)(Ag + (size_t)min(row_, a.M - 1) * g.lda + (k) + lcol); \
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
__global__ __launch_bounds__(64) void k_gemm_f32(GemmArgs a) {
    const int col = a.col_lo + blockIdx.x * 64 + threadIdx.x;
    const int m = blockIdx.y;
    if (col >= a.col_hi) return;
    int s = 0;
    for (int j = 1; j < a.nseg; ++j)
        if (col >= a.seg[j].c_col0) s = j;
    const GemmSeg g = a.seg[s];
    const int n = col - g.c_col0;
    if (n < 0 || n >= g.N) return;
    const float* A = (const float*)g.A + (size_t)m * g.lda;
    const float* B = (const float*)g.B + (size_t)n * g.ldb;
    float acc = 0.f;
    for (int k = 0; k < a.K; ++k) acc = fmaf(A[k], B[k], acc);
    float* p = a.C + (size_t)m * a.ldc + col;
    *p = a.accumulate ? *p + acc : acc;
}

__global__ __launch_bounds__(256) void k_splitk_reduce(GemmArgs a) {
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
hipError_t gemm(GemmArgs a, bool bf16, size_t part_cap_floats, int num_cus, hipStream_t st, int tag) {
    if (a.M <= 0 || a.nseg <= 0) return hipSuccess;
    a.col_lo = a.seg[0].c_col0;
    a.col_hi = a.seg[a.nseg - 1].c_col0 + a.seg[a.nseg - 1].N;
    if (!bf16) {
        a.splits = 1;
        a.kc = a.K;
        dim3 grid((a.col_hi - a.col_lo + 63) / 64, a.M);
        hipLaunchKernelGGL(k_gemm_f32, grid, dim3(64), 0, st, a);
        return hipGetLastError();
    }
    const bool skinny = a.M <= 16;
    const int NT = skinny ? 64 : 128;
    const int MT = skinny ? 16 : (a.M <= 64 ? 64 : 128);
    int ntiles = 0;
    for (int s = 0; s < a.nseg; ++s) {
        a.seg[s].tile0 = ntiles;
        ntiles += (a.seg[s].N + NT - 1) / NT;
    }
    a.ntiles = ntiles;
    const int mtiles = (a.M + MT - 1) / MT;
    const int base = ntiles * mtiles;
    // enough workgroups for ~2 per CU; keep a split at >= 512 k-values
    int splits = 1;
    const int target = 2 * num_cus;
    while (base * splits < target && a.K / (splits * 2) >= 512) splits *= 2;
    while (splits > 1 && (size_t)splits * a.M * a.ldc > part_cap_floats) splits /= 2;
    int kc = ((a.K + splits - 1) / splits + 63) / 64 * 64;
    splits = (a.K + kc - 1) / kc;
    a.splits = splits;
    a.kc = kc;
    const dim3 blk(256);
    if (skinny) {
        if (tag == 1) hipLaunchKernelGGL(k_gemm_skinny<1>, dim3(ntiles, splits), blk, 0, st, a);
        else hipLaunchKernelGGL(k_gemm_skinny<0>, dim3(ntiles, splits), blk, 0, st, a);
    } else if (MT == 64) {
        if (tag == 1) hipLaunchKernelGGL((k_gemm_tiled<64, 1>), dim3(ntiles, mtiles, splits), blk, 0, st, a);
        else hipLaunchKernelGGL((k_gemm_tiled<64, 0>), dim3(ntiles, mtiles, splits), blk, 0, st, a);
    } else {
        if (tag == 1) hipLaunchKernelGGL((k_gemm_tiled<128, 1>), dim3(ntiles, mtiles, splits), blk, 0, st, a);
        else hipLaunchKernelGGL((k_gemm_tiled<128, 0>), dim3(ntiles, mtiles, splits), blk, 0, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    const size_t total = (size_t)a.M * (a.col_hi - a.col_lo);
    const int blocks = (int)std::min<size_t>((total + 255) / 256, (size_t)num_cus * 8);
    hipLaunchKernelGGL(k_splitk_reduce, dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace kern
}  // namespace dflash
