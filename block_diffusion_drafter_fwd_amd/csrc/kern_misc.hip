// Row-wise kernels of the drafter forward: RMSNorm, the per-head q/k norm +
// RoPE + slot-indexed K/V cache writer, embedding gather, descriptor upload,
// row gather, cache readback, and the batched sampler.
#include <climits>
#include <cmath>

#include "kernels.h"

namespace dflash {
namespace kern {

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f2bf(float x) {   // round to nearest, ties to even
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float ld_any(const void* p, size_t i, int bf16) {
    return bf16 ? bf2f(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}

__device__ __forceinline__ void st_any(void* p, size_t i, float v, int bf16) {
    if (bf16) ((uint16_t*)p)[i] = f2bf(v);
    else ((float*)p)[i] = v;
}

// Sums by DPP lane moves (no LDS round trip): quad swaps, half-row and row
// mirrors give every lane of a 16-lane row its row's sum (the row uniformly
// active); two row broadcasts (lanes left out add 0) carry rows 0-2 into
// row 3, whose lane 63 then holds the wave's sum.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float v) {
    v = dpp_add<0xB1, 0xF>(v);    // quad_perm [1, 0, 3, 2]
    v = dpp_add<0x4E, 0xF>(v);    // quad_perm [2, 3, 0, 1]
    v = dpp_add<0x141, 0xF>(v);   // row_half_mirror
    return dpp_add<0x140, 0xF>(v);   // row_mirror
}
__device__ __forceinline__ float wave_sum(float v) {   // the whole wave; every lane gets lane 63's sum
    v = row16_sum(v);
    v = dpp_add<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
    v = dpp_add<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float block_sum(float v, float* sh) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    __syncthreads();
    if (l == 0) sh[w] = v;
    __syncthreads();
    float s = 0.f;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += sh[i];
    return s;
}

// ---------------------------------------------------------------------------
// RMSNorm: y = x / sqrt(mean(x^2) + eps) * gain, per row and per group of
// width/groups columns; one input, up to kMaxOut (gain, output) pairs.  x may
// be the sum of a residual row and K-slices of a GEMM (then written back).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) void k_rmsnorm(NormArgs a) {
    __shared__ float sh[8];
    __shared__ float xs[kNormMaxW];
    const int orow = blockIdx.x, grp = blockIdx.y;
    const int irow = a.row_src ? a.row_src[orow] : orow;
    const int W = a.width / a.groups;
    const size_t ibase = (size_t)irow * a.in_stride + (size_t)grp * W;
    // gather x (residual + slices) into LDS: every load is independent of the
    // stores, which come after the reduction
    float ss = 0.f;
    for (int i = threadIdx.x; i < W; i += 512) {
        float x = a.in ? ld_any(a.in, ibase + i, a.in_bf16) : 0.f;
        const float* __restrict__ p = a.part + ibase + i;
        for (int sp = 0; sp < a.nsplit; ++sp) x += p[(size_t)sp * a.part_stride];
        xs[i] = x;
        ss += x * x;
    }
    ss = block_sum(ss, sh);
    const float rstd = 1.f / sqrtf(ss / (float)W + a.eps);
    if (a.writeback)
        for (int i = threadIdx.x; i < W; i += 512) a.writeback[ibase + i] = xs[i];
    const size_t obase = (size_t)orow * a.out_stride + (size_t)grp * W;
    const size_t gbase = (size_t)grp * a.gain_group_stride;
    for (int o = 0; o < a.nout; ++o)
        for (int i = threadIdx.x; i < W; i += 512) {
            const float gn = ld_any(a.gain[o], gbase + i, a.gain_bf16);
            st_any(a.out[o], obase + i, xs[i] * rstd * gn, a.out_bf16);
        }
}

// four consecutive elements, fp32 or bf16 (16- or 8-byte aligned)
__device__ __forceinline__ float4 ld4_any(const void* p, size_t i, int bf16) {
    if (bf16) {
        const uint2 u = *(const uint2*)((const uint16_t*)p + i);
        return float4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u), __uint_as_float(u.y << 16),
                      __uint_as_float(u.y & 0xFFFF0000u)};
    }
    return *(const float4*)((const float*)p + i);
}

__device__ __forceinline__ void st4_any(void* p, size_t i, float4 v, int bf16) {
    if (bf16) {
        const uint2 u = {(uint32_t)f2bf(v.x) | ((uint32_t)f2bf(v.y) << 16),
                         (uint32_t)f2bf(v.z) | ((uint32_t)f2bf(v.w) << 16)};
        *(uint2*)((uint16_t*)p + i) = u;
    } else {
        *(float4*)((float*)p + i) = v;
    }
}

// The same norm with every operand read and written four elements at a time
// (the launcher checks widths, strides and alignment).  The slice loads of a
// chunk are issued together, eight at a time (the latency of one L2 round
// trip, not of one per slice), and added in slice order.
constexpr int kNormSliceBatch = 8;
// NT threads per row: 1024 when the row has more than 512 four-element
// columns, so that every thread's loads go out in one batch
template <int NT>
__global__ __launch_bounds__(NT) void k_rmsnorm4(NormArgs a) {
    __shared__ float sh[NT / 64];
    __shared__ float4 xs[kNormMaxW / 4];
    const int orow = blockIdx.x, grp = blockIdx.y;
    const int irow = a.row_src ? a.row_src[orow] : orow;
    const int W = a.width / a.groups, W4 = W >> 2;
    const size_t ibase = (size_t)irow * a.in_stride + (size_t)grp * W;
    const size_t gbase = (size_t)grp * a.gain_group_stride;
    // the first output's gains go out with the other loads, not after the
    // writeback stores (a load issued after a store would wait for it)
    constexpr int kIt = kNormMaxW / 4 / NT;
    float4 g0[kIt];
    if (a.nout > 0)
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int i = threadIdx.x + it * NT;
            if (i < W4) g0[it] = ld4_any(a.gain[0], gbase + 4 * i, a.gain_bf16);
        }
    float ss = 0.f;
    for (int i = threadIdx.x; i < W4; i += NT) {
        float4 x = a.in ? ld4_any(a.in, ibase + 4 * i, a.in_bf16) : float4{0.f, 0.f, 0.f, 0.f};
        const float* __restrict__ p = a.part + ibase + 4 * i;
        for (int s0 = 0; s0 < a.nsplit; s0 += kNormSliceBatch) {
            float4 v[kNormSliceBatch];
#pragma unroll
            for (int j = 0; j < kNormSliceBatch; ++j)   // past the last slice: re-read it, add nothing
                v[j] = *(const float4*)(p + (size_t)min(s0 + j, a.nsplit - 1) * a.part_stride);
#pragma unroll
            for (int j = 0; j < kNormSliceBatch; ++j)
                if (s0 + j < a.nsplit) {
                    x.x += v[j].x;
                    x.y += v[j].y;
                    x.z += v[j].z;
                    x.w += v[j].w;
                }
        }
        xs[i] = x;
        ss += x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
    }
    ss = block_sum(ss, sh);
    const float rstd = 1.f / sqrtf(ss / (float)W + a.eps);
    if (a.writeback)
        for (int i = threadIdx.x; i < W4; i += NT) *(float4*)(a.writeback + ibase + 4 * i) = xs[i];
    const size_t obase = (size_t)orow * a.out_stride + (size_t)grp * W;
    for (int o = 0; o < a.nout; ++o)
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int i = threadIdx.x + it * NT;
            if (i >= W4) break;
            const float4 gn = o == 0 ? g0[it] : ld4_any(a.gain[o], gbase + 4 * i, a.gain_bf16);
            const float4 x = xs[i];
            st4_any(a.out[o], obase + 4 * i,
                    float4{x.x * rstd * gn.x, x.y * rstd * gn.y, x.z * rstd * gn.z, x.w * rstd * gn.w}, a.out_bf16);
        }
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

#ifndef DFLASH_NORM_WIDE
#define DFLASH_NORM_WIDE 1
#endif
constexpr bool kNormWide = DFLASH_NORM_WIDE;

hipError_t rmsnorm(const NormArgs& a, hipStream_t st) {
    if (a.rows <= 0) return hipSuccess;
    const int W = a.width / a.groups;
    bool v4 = W % 4 == 0 && a.in_stride % 4 == 0 && (a.nsplit == 0 || a.part_stride % 4 == 0) &&
              a.out_stride % 4 == 0 && a.gain_group_stride % 4 == 0 && aligned16(a.in) && aligned16(a.part) &&
              aligned16(a.writeback);
    for (int o = 0; o < a.nout; ++o) v4 = v4 && aligned16(a.gain[o]) && aligned16(a.out[o]);
    if (v4 && W / 4 > 512 && kNormWide)
        hipLaunchKernelGGL(k_rmsnorm4<1024>, dim3(a.rows, a.groups), dim3(1024), 0, st, a);
    else if (v4)
        hipLaunchKernelGGL(k_rmsnorm4<512>, dim3(a.rows, a.groups), dim3(512), 0, st, a);
    else hipLaunchKernelGGL(k_rmsnorm, dim3(a.rows, a.groups), dim3(512), 0, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-head finish of a projection row: q and k get RMSNorm over the head and
// rotate-half RoPE at the row's position (angle pos * theta^(-2d/D) in fp64,
// cos/sin rounded to fp32); q goes to the query buffer, k and v to the
// session's cache at the row's slot.  Grid (row, task group, layer); each
// wave finishes one head (tasks: q heads, then k heads, then v heads).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_head_finish(HeadArgs a) {
    __shared__ float s_cos[64], s_sin[64];
    const int row = blockIdx.x, li = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nq = (a.q_col >= 0) ? a.Hq : 0;
    const int task = blockIdx.y * 4 + wave;
    const bool live = task < nq + 2 * a.Hkv;
    const int half = a.D >> 1;
    const bool act = lane < half;
    const int layer = a.layer[li];
    int kind, head, col;   // kind 0 q, 1 k, 2 v
    if (task < nq) { kind = 0; head = task; col = a.q_col + head * a.D; }
    else if (task < nq + a.Hkv) { kind = 1; head = task - nq; col = a.k_col[li] + head * a.D; }
    else { kind = 2; head = task - nq - a.Hkv; col = a.v_col[li] + head * a.D; }
    // the loads that do not depend on the row's position go out first: the
    // first kNormSliceBatch slices and the head norm's gains
    const float* src = a.src + (size_t)row * a.ld + col + lane;
    const void* gnp = kind == 0 ? a.q_norm : a.k_norm[li];
    const bool use_norm = kind != 2 && a.qk_norm;
    float v1[kNormSliceBatch], v2[kNormSliceBatch];
    float gn1 = 0.f, gn2 = 0.f;
    if (live && act) {
#pragma unroll
        for (int j = 0; j < kNormSliceBatch; ++j) {
            const size_t o = (size_t)min(j, a.nsplit - 1) * a.src_stride;
            v1[j] = src[o];
            v2[j] = src[o + half];
        }
        if (use_norm) {
            gn1 = ld_any(gnp, lane, a.w_bf16);
            gn2 = ld_any(gnp, lane + half, a.w_bf16);
        }
    }
    int pos, cap, ring;
    void* cache;
    if (a.rows) {
        const RowInfo ri = a.rows[row];
        const SeqDesc sd = a.seqs[ri.seq];
        pos = ri.pos;
        cap = sd.cap;
        ring = sd.ring;
        cache = sd.cache;
    } else {
        pos = a.pos0 + row;
        cap = a.cap0;
        ring = a.ring0;
        cache = a.cache0;
    }
    // the row's rotation angles once for the workgroup's four heads (fp64,
    // rounded to fp32), not once per head
    if (threadIdx.x < half) {
        double sn_, cs_;
        sincos((double)pos * a.inv_freq[threadIdx.x], &sn_, &cs_);
        s_cos[threadIdx.x] = (float)cs_;
        s_sin[threadIdx.x] = (float)sn_;
    }
    __syncthreads();
    if (!live) return;
    const int slot = ring ? pos % cap : pos;
    float x1 = 0.f, x2 = 0.f;
    if (act)   // slices added in order; past the first batch, kNormSliceBatch loads per round trip
        for (int s0 = 0; s0 < a.nsplit; s0 += kNormSliceBatch) {
            if (s0) {
#pragma unroll
                for (int j = 0; j < kNormSliceBatch; ++j) {
                    const size_t o = (size_t)min(s0 + j, a.nsplit - 1) * a.src_stride;
                    v1[j] = src[o];
                    v2[j] = src[o + half];
                }
            }
#pragma unroll
            for (int j = 0; j < kNormSliceBatch; ++j)
                if (s0 + j < a.nsplit) {
                    x1 += v1[j];
                    x2 += v2[j];
                }
        }
    if (kind != 2) {
        if (use_norm) {
            const float ss = wave_sum(x1 * x1 + x2 * x2);
            const float rstd = 1.f / sqrtf(ss / (float)a.D + a.eps);
            if (act) {
                x1 = x1 * rstd * gn1;
                x2 = x2 * rstd * gn2;
            }
        }
        if (act) {
            const float cs = s_cos[lane], sn = s_sin[lane];
            const float y1 = x1 * cs - x2 * sn;
            const float y2 = x2 * cs + x1 * sn;
            x1 = y1;
            x2 = y2;
        }
    }
    if (!act) return;
    if (kind == 0) {
        const size_t o = ((size_t)row * a.Hq + head) * a.D;
        st_any(a.q_out, o + lane, x1, a.q_bf16);
        st_any(a.q_out, o + lane + half, x2, a.q_bf16);
    } else {
        const size_t o = ((((size_t)layer * 2 + (kind - 1)) * a.Hkv + head) * cap + slot) * a.D;
        st_any(cache, o + lane, x1, a.cache_bf16);
        st_any(cache, o + lane + half, x2, a.cache_bf16);
    }
}

// The same finish for 128-wide heads with 16-byte accesses: 16 lanes per
// head, four heads per wave, lane l holding dims 4l .. 4l + 3 and their
// rotation partners 64 + 4l .. (a quarter of the load instructions, each
// four times wider; the flush's 256-row context pass reads 31.5 MB of K
// slices here).  The slice sums and the rotation are those of k_head_finish
// element by element; the head norm's sum of squares runs over 16 lanes.
__global__ __launch_bounds__(256) void k_head_finish4(HeadArgs a) {
    __shared__ float4 s_cs[16], s_sn[16];   // cos, sin of dims 4i .. 4i + 3
    const int row = blockIdx.x, li = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l = lane & 15;
    const int nq = (a.q_col >= 0) ? a.Hq : 0;
    const int task = blockIdx.y * 16 + wave * 4 + (lane >> 4);
    const bool live = task < nq + 2 * a.Hkv;   // (uniform over each 16-lane group)
    const int layer = a.layer[li];
    int kind, head, col;   // kind 0 q, 1 k, 2 v
    if (task < nq) { kind = 0; head = task; col = a.q_col + head * 128; }
    else if (task < nq + a.Hkv) { kind = 1; head = task - nq; col = a.k_col[li] + head * 128; }
    else { kind = 2; head = task - nq - a.Hkv; col = a.v_col[li] + head * 128; }
    // position-independent loads first: a batch of slices and the gains
    constexpr int kB = 4;
    const float* src = a.src + (size_t)row * a.ld + col + 4 * l;
    const void* gnp = kind == 0 ? a.q_norm : a.k_norm[li];
    const bool use_norm = kind != 2 && a.qk_norm;
    float4 v1[kB], v2[kB];
    float4 g1 = {0.f, 0.f, 0.f, 0.f}, g2 = {0.f, 0.f, 0.f, 0.f};
    if (live) {
#pragma unroll
        for (int j = 0; j < kB; ++j) {
            const size_t o = (size_t)min(j, a.nsplit - 1) * a.src_stride;
            v1[j] = *(const float4*)(src + o);
            v2[j] = *(const float4*)(src + o + 64);
        }
        if (use_norm) {
            g1 = ld4_any(gnp, 4 * l, a.w_bf16);
            g2 = ld4_any(gnp, 64 + 4 * l, a.w_bf16);
        }
    }
    int pos, cap, ring;
    void* cache;
    if (a.rows) {
        const RowInfo ri = a.rows[row];
        const SeqDesc sd = a.seqs[ri.seq];
        pos = ri.pos;
        cap = sd.cap;
        ring = sd.ring;
        cache = sd.cache;
    } else {
        pos = a.pos0 + row;
        cap = a.cap0;
        ring = a.ring0;
        cache = a.cache0;
    }
    if (threadIdx.x < 64) {
        double sn_, cs_;
        sincos((double)pos * a.inv_freq[threadIdx.x], &sn_, &cs_);
        ((float*)s_cs)[threadIdx.x] = (float)cs_;
        ((float*)s_sn)[threadIdx.x] = (float)sn_;
    }
    __syncthreads();
    if (!live) return;
    float4 x1 = {0.f, 0.f, 0.f, 0.f}, x2 = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < a.nsplit; s0 += kB) {
        if (s0) {
#pragma unroll
            for (int j = 0; j < kB; ++j) {
                const size_t o = (size_t)min(s0 + j, a.nsplit - 1) * a.src_stride;
                v1[j] = *(const float4*)(src + o);
                v2[j] = *(const float4*)(src + o + 64);
            }
        }
#pragma unroll
        for (int j = 0; j < kB; ++j)
            if (s0 + j < a.nsplit) {
                x1 = float4{x1.x + v1[j].x, x1.y + v1[j].y, x1.z + v1[j].z, x1.w + v1[j].w};
                x2 = float4{x2.x + v2[j].x, x2.y + v2[j].y, x2.z + v2[j].z, x2.w + v2[j].w};
            }
    }
    if (kind != 2) {
        if (use_norm) {
            float ss = x1.x * x1.x + x1.y * x1.y + x1.z * x1.z + x1.w * x1.w + x2.x * x2.x + x2.y * x2.y +
                       x2.z * x2.z + x2.w * x2.w;
            ss = row16_sum(ss);   // the head's 16 lanes are one DPP row
            const float rstd = 1.f / sqrtf(ss / 128.f + a.eps);
            x1 = float4{x1.x * rstd * g1.x, x1.y * rstd * g1.y, x1.z * rstd * g1.z, x1.w * rstd * g1.w};
            x2 = float4{x2.x * rstd * g2.x, x2.y * rstd * g2.y, x2.z * rstd * g2.z, x2.w * rstd * g2.w};
        }
        const float4 cs = s_cs[l], sn = s_sn[l];
        const float4 y1 = {x1.x * cs.x - x2.x * sn.x, x1.y * cs.y - x2.y * sn.y, x1.z * cs.z - x2.z * sn.z,
                           x1.w * cs.w - x2.w * sn.w};
        const float4 y2 = {x2.x * cs.x + x1.x * sn.x, x2.y * cs.y + x1.y * sn.y, x2.z * cs.z + x1.z * sn.z,
                           x2.w * cs.w + x1.w * sn.w};
        x1 = y1;
        x2 = y2;
    }
    if (kind == 0) {
        const size_t o = ((size_t)row * a.Hq + head) * 128;
        st4_any(a.q_out, o + 4 * l, x1, a.q_bf16);
        st4_any(a.q_out, o + 64 + 4 * l, x2, a.q_bf16);
    } else {
        const int slot = ring ? pos % cap : pos;
        const size_t o = ((((size_t)layer * 2 + (kind - 1)) * a.Hkv + head) * cap + slot) * 128;
        st4_any(cache, o + 4 * l, x1, a.cache_bf16);
        st4_any(cache, o + 64 + 4 * l, x2, a.cache_bf16);
    }
}

hipError_t head_finish(const HeadArgs& a, int nlayer, hipStream_t st) {
    if (a.nrows <= 0 || nlayer <= 0) return hipSuccess;
    const int ntask = (a.q_col >= 0 ? a.Hq : 0) + 2 * a.Hkv;
    // 128-wide heads with every slice row and column 16-byte aligned: the
    // vector form (the cache and query rows are 256-byte multiples)
    bool v4 = a.D == 128 && a.ld % 4 == 0 && a.src_stride % 4 == 0 && aligned16(a.src) && (a.q_col < 0 || a.q_col % 4 == 0) &&
              aligned16(a.q_out) && aligned16(a.q_norm);
    for (int j = 0; j < nlayer; ++j) v4 = v4 && a.k_col[j] % 4 == 0 && a.v_col[j] % 4 == 0 && aligned16(a.k_norm[j]);
    if (v4)
        hipLaunchKernelGGL(k_head_finish4, dim3(a.nrows, (ntask + 15) / 16, nlayer), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(k_head_finish, dim3(a.nrows, (ntask + 3) / 4, nlayer), dim3(256), 0, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Block embedding: row i of a sequence's block is the anchor (i = 0) or the
// mask token.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_embed(EmbedArgs a) {
    __shared__ float sh[4];
    __shared__ float xs[kNormMaxW];
    const int row = blockIdx.x;
    int tok;
    if (a.rows) {
        const RowInfo ri = a.rows[row];
        const SeqDesc sd = a.seqs[ri.seq];
        tok = ri.pos == sd.F ? sd.current : a.mask_id;
    } else {
        tok = row == 0 ? a.current : a.mask_id;
    }
    const size_t src = (size_t)tok * a.H;
    float ss = 0.f;
    if (a.vec4) {
        // four elements at j = 4 (t + 256 c): the table row and the gains are
        // all loaded before the first store (a load after a store to h or out
        // would wait for the loads before it)
        constexpr int kC = kNormMaxW / 1024;
        float4 v[kC], gn[kC];
#pragma unroll
        for (int c = 0; c < kC; ++c) {
            const int j = 4 * (threadIdx.x + 256 * c);
            if (j < a.H) v[c] = ld4_any(a.table, src + j, a.w_bf16);
        }
        if (a.gain)
#pragma unroll
            for (int c = 0; c < kC; ++c) {
                const int j = 4 * (threadIdx.x + 256 * c);
                if (j < a.H) gn[c] = ld4_any(a.gain, j, a.w_bf16);
            }
#pragma unroll
        for (int c = 0; c < kC; ++c) {
            const int j = 4 * (threadIdx.x + 256 * c);
            if (j < a.H) {
                ss += v[c].x * v[c].x + v[c].y * v[c].y + v[c].z * v[c].z + v[c].w * v[c].w;
                *(float4*)(a.h + (size_t)row * a.H + j) = v[c];
            }
        }
        if (!a.gain) return;                           // uniform over the launch
        ss = block_sum(ss, sh);
        const float rstd = 1.f / sqrtf(ss / (float)a.H + a.eps);
#pragma unroll
        for (int c = 0; c < kC; ++c) {
            const int j = 4 * (threadIdx.x + 256 * c);
            if (j < a.H)
                st4_any(a.out, (size_t)row * a.H + j,
                        float4{v[c].x * rstd * gn[c].x, v[c].y * rstd * gn[c].y, v[c].z * rstd * gn[c].z,
                               v[c].w * rstd * gn[c].w},
                        a.out_bf16);
        }
        return;
    }
    for (int j = threadIdx.x; j < a.H; j += 256) {
        const float v = ld_any(a.table, src + j, a.w_bf16);
        xs[j] = v;
        ss += v * v;
    }
    __syncthreads();
    for (int j = threadIdx.x; j < a.H; j += 256) a.h[(size_t)row * a.H + j] = xs[j];
    if (!a.gain) return;                               // uniform over the launch
    ss = block_sum(ss, sh);
    const float rstd = 1.f / sqrtf(ss / (float)a.H + a.eps);
    for (int j = threadIdx.x; j < a.H; j += 256)
        st_any(a.out, (size_t)row * a.H + j, xs[j] * rstd * ld_any(a.gain, j, a.w_bf16), a.out_bf16);
}

hipError_t embed(const EmbedArgs& args, hipStream_t st) {
    if (args.nrows <= 0) return hipSuccess;
    EmbedArgs a = args;
    a.vec4 = a.H % 4 == 0 && a.H <= kNormMaxW && aligned16(a.table) && aligned16(a.h) && aligned16(a.gain) &&
             aligned16(a.out);
    hipLaunchKernelGGL(k_embed, dim3(a.nrows), dim3(256), 0, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Descriptor upload (payload travels in the kernel arguments), row gather,
// cache readback.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_upload(UploadArgs a) {
    for (int i = threadIdx.x; i < a.nwords; i += 256) a.dst[i] = a.data[i];
}

hipError_t upload(void* dst, const void* host, size_t bytes, hipStream_t st) {
    const uint32_t* src = (const uint32_t*)host;
    size_t words = (bytes + 3) / 4;
    UploadArgs a;
    for (size_t off = 0; off < words; off += kUploadWords) {
        const int n = (int)std::min<size_t>(kUploadWords, words - off);
        a.dst = (uint32_t*)dst + off;
        a.nwords = n;
        a.pad = 0;
        for (int i = 0; i < n; ++i) a.data[i] = src[off + i];
        hipLaunchKernelGGL(k_upload, dim3(1), dim3(256), 0, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

__global__ __launch_bounds__(256) void k_commit(CommitArgs a) {
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i < a.count; i += 256) a.hist[i] = a.tokens[i];
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < a.n16; i += (int64_t)gridDim.x * 256)
        a.dst[i] = a.src[i];
}

hipError_t commit_rows(int32_t* hist, const int32_t* tokens, int32_t count, void* dst, const void* src, size_t bytes,
                       hipStream_t st) {
    if (count < 0 || count > kCommitTokens || bytes % 16 || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15))
        return hipErrorInvalidValue;
    CommitArgs a;
    a.hist = hist;
    a.src = (const uint4*)src;
    a.dst = (uint4*)dst;
    a.n16 = (int64_t)(bytes / 16);
    a.count = count;
    a.pad = 0;
    for (int i = 0; i < count; ++i) a.tokens[i] = tokens[i];
    const int64_t wgs = std::min<int64_t>(1024, std::max<int64_t>(1, (a.n16 + 255) / 256));
    hipLaunchKernelGGL(k_commit, dim3((unsigned)wgs), dim3(256), 0, st, a);
    return hipGetLastError();
}

// grid (items, copy blocks): block (i, 0) also writes item i's history tokens
__global__ __launch_bounds__(256) void k_commit_batch(CommitBatchArgs a) {
    const CommitItemArgs& it = a.item[blockIdx.x];
    if (blockIdx.y == 0)
        for (int j = threadIdx.x; j < it.count; j += 256) it.hist[(it.slot0 + j) % kHistRing] = a.tokens[it.tok0 + j];
    for (int64_t i = (int64_t)blockIdx.y * 256 + threadIdx.x; i < it.n16; i += (int64_t)gridDim.y * 256)
        it.dst[i] = it.src[i];
}

hipError_t commit_batch(const CommitBatchArgs& a, hipStream_t st) {
    if (a.n <= 0) return hipSuccess;
    if (a.n > kCommitItems) return hipErrorInvalidValue;
    int64_t most = 1;
    for (int i = 0; i < a.n; ++i) {
        const CommitItemArgs& it = a.item[i];
        if (it.count < 0 || it.tok0 < 0 || it.tok0 + it.count > kCommitBatchTokens || it.n16 < 0 ||
            ((uintptr_t)it.src & 15) || ((uintptr_t)it.dst & 15))
            return hipErrorInvalidValue;
        most = std::max(most, it.n16);
    }
    const unsigned gy = (unsigned)std::min<int64_t>(16, (most + 255) / 256);
    hipLaunchKernelGGL(k_commit_batch, dim3(a.n, gy), dim3(256), 0, st, a);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_gather_rows(uint4* dst, const uint64_t* src, size_t row_words) {
    const int row = blockIdx.x;
    const uint4* s = (const uint4*)src[row];
    for (size_t i = threadIdx.x; i < row_words; i += 256) dst[(size_t)row * row_words + i] = s[i];
}

hipError_t gather_rows(void* dst, const uint64_t* src_ptrs, int32_t rows, size_t row_bytes, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_gather_rows, dim3(rows), dim3(256), 0, st, (uint4*)dst, src_ptrs, row_bytes / 16);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_cache_read(const void* cache, int32_t cap, int32_t ring, int32_t Hkv,
                                                    int32_t D, int32_t layer, int32_t pos0, int32_t count,
                                                    int32_t bf16, float* k_out, float* v_out) {
    const size_t per = (size_t)Hkv * D;
    const size_t total = (size_t)count * per;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
        const int c = (int)(i / per);
        const int h = (int)((i % per) / D), d = (int)(i % D);
        const int pos = pos0 + c;
        const int slot = ring ? pos % cap : pos;
        const size_t kk = ((((size_t)layer * 2 + 0) * Hkv + h) * cap + slot) * D + d;
        const size_t vv = ((((size_t)layer * 2 + 1) * Hkv + h) * cap + slot) * D + d;
        k_out[i] = ld_any(cache, kk, bf16);
        v_out[i] = ld_any(cache, vv, bf16);
    }
}

hipError_t cache_read(const void* cache, int32_t cap, int32_t ring, int32_t Hkv, int32_t D, int32_t layer,
                      int32_t pos0, int32_t count, int32_t bf16, float* k_out, float* v_out, hipStream_t st) {
    const size_t total = (size_t)count * Hkv * D;
    const int blocks = (int)std::min<size_t>((total + 255) / 256, 4096);
    hipLaunchKernelGGL(k_cache_read, dim3(blocks), dim3(256), 0, st, cache, cap, ring, Hkv, D, layer, pos0,
                       count, bf16, k_out, v_out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Sampler.  Penalties (CTRL repetition penalty over the distinct tokens of the
// session's committed history) -> temperature -> softmax probabilities and a
// Gumbel-max draw, u from Philox4x64-10 (Salmon et al., SC'11) at counter
// (t div 8, row, round, 0) under key (seed, stream), word (t mod 8) div 2,
// bits 63..41 for even t and 40..18 for odd t.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += W0;
            k1 += W1;
        }
        const uint64_t hi0 = __umul64hi(M0, c[0]), lo0 = M0 * c[0];
        const uint64_t hi1 = __umul64hi(M1, c[2]), lo1 = M1 * c[2];
        const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = lo1;
        c[2] = n2;
        c[3] = lo0;
    }
}

// ONE: a one-session call, whose descriptor rides in the arguments (no
// tables; row r is the session's row r).  A compile-time switch: choosing
// between the two sources at run time moved the descriptor (the Philox key)
// into vector registers and cut the occupancy of the sampling kernel.
template <bool ONE>
__device__ __forceinline__ RowInfo sample_row(const SampleArgs& a, int r) {
    if constexpr (ONE) return RowInfo{0, r};
    else return a.rows[r];
}
template <bool ONE>
__device__ __forceinline__ SeqDesc sample_seq(const SampleArgs& a, int k) {
    if constexpr (ONE) return a.seq0;
    else return a.seqs[k];
}

template <bool ONE>
__global__ __launch_bounds__(256) void k_hist_bitmap(SampleArgs a) {
    const SeqDesc sd = sample_seq<ONE>(a, blockIdx.x);
    uint32_t* bm = a.bitmap + (size_t)blockIdx.x * a.words;
    for (int i = threadIdx.x; i < a.words; i += 256) bm[i] = 0u;
    __syncthreads();
    for (int j = threadIdx.x; j < sd.hist_n; j += 256) {
        const int tok = sd.hist[(sd.hist_head - sd.hist_n + j + 2 * kHistRing) % kHistRing];
        if (tok >= 0 && tok < a.V) atomicOr(&bm[tok >> 5], 1u << (tok & 31));
    }
}

struct Stat {
    float m, l, best;
    int idx;
};

__device__ __forceinline__ void stat_merge(Stat& a, const Stat& b) {
    if (b.m > a.m) {
        a.l = a.l * (a.m == -INFINITY ? 0.f : __expf(a.m - b.m)) + b.l;
        a.m = b.m;
    } else if (b.m != -INFINITY) {
        a.l += b.l * __expf(b.m - a.m);
    }
    if (b.best > a.best || (b.best == a.best && b.idx < a.idx)) {
        a.best = b.best;
        a.idx = b.idx;
    }
}

// The repetition penalty of a token in the history: a positive logit times
// 1 / rho, any other times rho (a multiply and two selects, no branch; the
// sampling pass and the probability pass use this same form)
__device__ __forceinline__ float penalize(float z, bool hit, float rho, float inv_rho) {
    return hit ? z * (z > 0.f ? inv_rho : rho) : z;
}
__device__ __forceinline__ float penalized(const SampleArgs& a, const uint32_t* bm, int r, int t) {
    const float z = a.logits[(size_t)r * a.V + t];
    return a.use_penalty ? penalize(z, (bm[t >> 5] >> (t & 31)) & 1u, a.rho, 1.f / a.rho) : z;
}

// A lane's Stat moved by DPP (no LDS round trip); a lane with no source in
// the move (rows left out of a row broadcast) gets the empty Stat, which
// merges as nothing
template <int CTRL, int ROWS>
__device__ __forceinline__ Stat stat_dpp(const Stat& s) {
    return Stat{__int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(-INFINITY), __float_as_int(s.m), CTRL, ROWS,
                                                           0xF, false)),
                __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s.l), CTRL, ROWS, 0xF, false)),
                __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(-INFINITY), __float_as_int(s.best), CTRL,
                                                           ROWS, 0xF, false)),
                __builtin_amdgcn_update_dpp(0x7fffffff, s.idx, CTRL, ROWS, 0xF, false)};
}

// The wave's Stat, every lane getting lane 63's: quad swaps, half-row and
// row mirrors merge each 16-lane row, two row broadcasts carry rows 0-2
// into row 3.  The whole wave must be active.
__device__ __forceinline__ Stat wave_stat(Stat s) {
    stat_merge(s, stat_dpp<0xB1, 0xF>(s));    // quad_perm [1, 0, 3, 2]
    stat_merge(s, stat_dpp<0x4E, 0xF>(s));    // quad_perm [2, 3, 0, 1]
    stat_merge(s, stat_dpp<0x141, 0xF>(s));   // row_half_mirror
    stat_merge(s, stat_dpp<0x140, 0xF>(s));   // row_mirror
    stat_merge(s, stat_dpp<0x142, 0xA>(s));   // row_bcast:15 into rows 1 and 3
    stat_merge(s, stat_dpp<0x143, 0xC>(s));   // row_bcast:31 into rows 2 and 3
    return Stat{__int_as_float(__builtin_amdgcn_readlane(__float_as_int(s.m), 63)),
                __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s.l), 63)),
                __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s.best), 63)),
                __builtin_amdgcn_readlane(s.idx, 63)};
}

__device__ Stat block_stat(Stat s) {
    __shared__ float sm[4], sl[4], sb[4];
    __shared__ int si[4];
    s = wave_stat(s);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    __syncthreads();
    if (l == 0) {
        sm[w] = s.m;
        sl[w] = s.l;
        sb[w] = s.best;
        si[w] = s.idx;
    }
    __syncthreads();
    Stat t{sm[0], sl[0], sb[0], si[0]};
    for (int i = 1; i < 4; ++i) stat_merge(t, Stat{sm[i], sl[i], sb[i], si[i]});
    return t;
}

// -ln(-ln u) on the hardware base-2 logarithm (u in [2^-24, 1 - 2^-24], so
// both arguments are normal floats)
__device__ __forceinline__ float gumbel(float u) {
    constexpr float kLn2 = 0.6931471805599453f;
    return -__builtin_amdgcn_logf(-__builtin_amdgcn_logf(u) * kLn2) * kLn2;
}

// Per (row, vocabulary chunk): max and sum-exp of z'/T (online), and the
// Gumbel-max candidate (or the argmax when greedy).  Eight consecutive tokens
// per thread: two 16-byte logits loads, one history-bitmap word, one Philox
// call whose four words carry the eight draws (two 23-bit fields a word).
// FULL: every group of eight tokens lies inside the vocabulary (V and the
// chunk bounds multiples of 8), so no token needs a bounds check.  A
// thread visits its tokens in ascending id, so on equal keys it keeps the
// one it holds unless it holds none yet.  The running max and sum of
// exponentials serve the probabilities only and are skipped without them
// (a -inf logit adds nothing to the sum).
template <bool ONE, bool FULL>
__global__ __launch_bounds__(256) void k_sample_stats(SampleArgs a) {
    const int c = blockIdx.x, r = blockIdx.y;
    const RowInfo ri = sample_row<ONE>(a, r);
    const SeqDesc sd = sample_seq<ONE>(a, ri.seq);
    const uint32_t* bm = a.bitmap + (size_t)ri.seq * a.words;
    const int t_lo = c * a.chunk, t_hi = min(a.V, t_lo + a.chunk);
    Stat s{-INFINITY, 0.f, -INFINITY, 0x7fffffff};
    const bool greedy = a.temperature == 0.f;
    const bool want_l = a.probs != nullptr;
    const float inv_t = greedy ? 0.f : 1.f / a.temperature;
    const float inv_rho = 1.f / a.rho;
    const float* zr = a.logits + (size_t)r * a.V;
    for (int oc = (t_lo >> 3) + threadIdx.x; oc * 8 < t_hi; oc += 256) {
        const int t0 = oc * 8;
        float z[8];
        if constexpr (FULL) {
            const float4 v0 = *(const float4*)(zr + t0), v1 = *(const float4*)(zr + t0 + 4);
            z[0] = v0.x;
            z[1] = v0.y;
            z[2] = v0.z;
            z[3] = v0.w;
            z[4] = v1.x;
            z[5] = v1.y;
            z[6] = v1.z;
            z[7] = v1.w;
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) z[j] = t0 + j < t_hi ? zr[t0 + j] : -INFINITY;
        }
        if (a.use_penalty) {
            const uint32_t word = bm[t0 >> 5] >> (t0 & 31);   // the eight tokens share one word
#pragma unroll
            for (int j = 0; j < 8; ++j) z[j] = penalize(z[j], (word >> j) & 1u, a.rho, inv_rho);
        }
        if (greedy) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const bool take = (FULL || t0 + j < t_hi) &&
                                  (z[j] > s.best || (z[j] == s.best && s.idx == 0x7fffffff));
                s.best = take ? z[j] : s.best;
                s.idx = take ? t0 + j : s.idx;
            }
            continue;
        }
        uint64_t w[4] = {(uint64_t)oc, (uint64_t)ri.pos, (uint64_t)a.round, 0};
        philox4x64_10(w, sd.seed, sd.stream);
        float sv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) sv[j] = (FULL || t0 + j < t_hi) ? z[j] * inv_t : -INFINITY;
        if (want_l) {
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < 8; ++j) mx = fmaxf(mx, sv[j]);
            if (mx > s.m) {
                s.l = s.m == -INFINITY ? 0.f : s.l * __expf(s.m - mx);
                s.m = mx;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) s.l += sv[j] == -INFINITY ? 0.f : __expf(sv[j] - s.m);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint64_t wj = w[j >> 1];
            const uint32_t bits = (j & 1) ? (uint32_t)((wj >> 18) & 0x7FFFFFu) : (uint32_t)(wj >> 41);
            const float u = ((float)bits + 0.5f) * 0x1p-23f;
            const float key = sv[j] + gumbel(u);
            const bool take = (FULL || t0 + j < t_hi) && (key > s.best || (key == s.best && s.idx == 0x7fffffff));
            s.best = take ? key : s.best;
            s.idx = take ? t0 + j : s.idx;
        }
    }
    s = block_stat(s);
    if (threadIdx.x == 0) {
        float* o = a.stats + ((size_t)r * a.nchunk + c) * 4;
        o[0] = s.m;
        o[1] = s.l;
        o[2] = s.best;
        o[3] = __int_as_float(s.idx);
    }
}

template <bool ONE>
__global__ __launch_bounds__(256) void k_sample_final(SampleArgs a) {
    __shared__ float tot[4];
    const int c = blockIdx.x, r = blockIdx.y;
    if (threadIdx.x < 64) {
        Stat s{-INFINITY, 0.f, -INFINITY, 0x7fffffff};
        for (int j = threadIdx.x; j < a.nchunk; j += 64) {
            const float* o = a.stats + ((size_t)r * a.nchunk + j) * 4;
            stat_merge(s, Stat{o[0], o[1], o[2], __float_as_int(o[3])});
        }
        s = wave_stat(s);
        if (threadIdx.x == 0) {
            tot[0] = s.m;
            tot[1] = s.l;
            if (c == 0) a.ids[r] = s.idx;
        }
    }
    if (!a.probs || a.temperature == 0.f) return;
    __syncthreads();
    const float M = tot[0], Z = tot[1];
    const RowInfo ri = sample_row<ONE>(a, r);
    const uint32_t* bm = a.bitmap + (size_t)ri.seq * a.words;
    const int t_lo = c * a.chunk, t_hi = min(a.V, t_lo + a.chunk);
    const float inv_t = 1.f / a.temperature, inv_z = 1.f / Z;
    for (int t = t_lo + threadIdx.x; t < t_hi; t += 256) {
        const float sv = penalized(a, bm, r, t) * inv_t;   // as in k_sample_stats
        a.probs[(size_t)r * a.V + t] = __expf(sv - M) * inv_z;
    }
}

template <bool ONE>
static hipError_t sample_launch(const SampleArgs& a, hipStream_t st) {
    if (a.use_penalty) {
        hipLaunchKernelGGL(k_hist_bitmap<ONE>, dim3(a.nseq), dim3(256), 0, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if ((a.V & 7) == 0 && (a.chunk & 7) == 0)
        hipLaunchKernelGGL((k_sample_stats<ONE, true>), dim3(a.nchunk, a.R), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((k_sample_stats<ONE, false>), dim3(a.nchunk, a.R), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const bool probs = a.probs && a.temperature != 0.f;
    hipLaunchKernelGGL(k_sample_final<ONE>, dim3(probs ? a.nchunk : 1, a.R), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t sample(const SampleArgs& a, hipStream_t st) {
    if (a.R <= 0) return hipSuccess;
    if (!a.rows && a.nseq != 1) return hipErrorInvalidValue;   // no tables: exactly one session
    return a.rows ? sample_launch<false>(a, st) : sample_launch<true>(a, st);
}

// ---------------------------------------------------------------------------
// Speculative verification.  Pass 1, per (row, 4096-token chunk): max and
// sum-exp of row / T and the argmax.  Pass 2 (T > 0), per (row, chunk): the
// Gumbel-max candidate of the draw that the row would emit, with the row's
// normaliser from pass 1: over log(max(0, p - q)) on a drafted position,
// over row / T on the bonus position.  Pass 3, per session: walk the drafted
// tokens (argmax match, or u * q(x) <= p(x)) to the first rejection and take
// that row's draw (or argmax).  Draws: Philox4x64-10 under (seed, stream),
// counters (0, i, round, 1) for the acceptance uniforms and
// (t div 4, i, round, 2) for the Gumbel draws of row i.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float u23(uint64_t w) { return ((float)(w >> 41) + 0.5f) * 0x1p-23f; }

__global__ __launch_bounds__(256) void k_verify_stats(VerifyArgs a) {
    const int c = blockIdx.x, r = blockIdx.y;
    const int t_lo = c * a.chunk, t_hi = min(a.V, t_lo + a.chunk);
    const float* z = a.target + (size_t)r * a.V;
    const float inv_t = a.temperature > 0.f ? 1.f / a.temperature : 1.f;
    Stat s{-INFINITY, 0.f, -INFINITY, 0x7fffffff};
    // the thread's tokens t_lo + threadIdx.x + 256 i, kVerBatch loads issued
    // together (one round trip), then the online pass in ascending order
    constexpr int kVerBatch = 16;
    for (int b0 = t_lo + threadIdx.x; b0 < t_hi; b0 += 256 * kVerBatch) {
        float zb[kVerBatch];
#pragma unroll
        for (int i = 0; i < kVerBatch; ++i) {
            const int t = b0 + 256 * i;
            zb[i] = t < t_hi ? z[t] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < kVerBatch; ++i) {
        const int t = b0 + 256 * i;
        if (t >= t_hi) break;
        const float zt = zb[i];
        if (a.temperature > 0.f) {
            const float sv = zt * inv_t;
            if (sv > s.m) {
                s.l = s.l * (s.m == -INFINITY ? 0.f : __expf(s.m - sv)) + 1.f;
                s.m = sv;
            } else if (sv != -INFINITY) {   // (a -inf logit adds nothing, also before any finite one)
                s.l += __expf(sv - s.m);
            }
        }
        if (zt > s.best) {      // threads walk ascending ids: a tie keeps the lower one
            s.best = zt;
            s.idx = t;
        }
        }
    }
    s = block_stat(s);
    if (threadIdx.x == 0) {
        float* o = a.stats + ((size_t)r * a.nchunk + c) * 4;
        o[0] = s.m;
        o[1] = s.l;
        o[2] = s.best;
        o[3] = __int_as_float(s.idx);
    }
}

// the row's statistics over all chunks, merged by the first 64 threads
__device__ Stat row_stat(const float* stats, int nchunk, int r) {
    Stat s{-INFINITY, 0.f, -INFINITY, 0x7fffffff};
    for (int j = threadIdx.x & 63; j < nchunk; j += 64) {
        const float* o = stats + ((size_t)r * nchunk + j) * 4;
        stat_merge(s, Stat{o[0], o[1], o[2], __float_as_int(o[3])});
    }
    return wave_stat(s);
}

// ONE: a one-session call (descriptor and draft count in the arguments, no
// tables), chosen at compile time as for the sampler
template <bool ONE>
__device__ __forceinline__ RowInfo verify_row(const VerifyArgs& a, int r) {
    if constexpr (ONE) return RowInfo{0, r};
    else return a.rows[r];
}
template <bool ONE>
__device__ __forceinline__ int verify_off(const VerifyArgs& a, int k) {
    if constexpr (ONE) return k == 0 ? 0 : a.n0;
    else return a.offs[k];
}
template <bool ONE>
__device__ __forceinline__ SeqDesc verify_seq(const VerifyArgs& a, int k) {
    if constexpr (ONE) return a.seq0;
    else return a.seqs[k];
}

template <bool ONE>
__global__ __launch_bounds__(256) void k_verify_next(VerifyArgs a) {
    __shared__ float tot[2];
    const int c = blockIdx.x, r = blockIdx.y;
    if (threadIdx.x < 64) {
        const Stat s = row_stat(a.stats, a.nchunk, r);
        if (threadIdx.x == 0) {
            tot[0] = s.m;
            tot[1] = s.l;
        }
    }
    __syncthreads();
    const float M = tot[0], inv_z = 1.f / tot[1], inv_t = 1.f / a.temperature;
    const RowInfo ri = verify_row<ONE>(a, r);
    const SeqDesc sd = verify_seq<ONE>(a, ri.seq);
    const int n = verify_off<ONE>(a, ri.seq + 1) - verify_off<ONE>(a, ri.seq);
    const int i = ri.pos;                      // row within the block: i < n drafted, i == n bonus
    const float* z = a.target + (size_t)r * a.V;
    const float* q = i < n ? a.draft_probs + (size_t)(verify_off<ONE>(a, ri.seq) + i) * a.V : nullptr;
    const int t_lo = c * a.chunk, t_hi = min(a.V, t_lo + a.chunk);
    Stat s{-INFINITY, 0.f, -INFINITY, 0x7fffffff};
    // the thread's groups of four tokens qd = t_lo / 4 + threadIdx.x + 256 u:
    // kNextBatch groups' target and draft loads issued together
    constexpr int kNextBatch = 4;
    for (int qb = (t_lo >> 2) + threadIdx.x; qb * 4 < t_hi; qb += 256 * kNextBatch) {
    float zb[kNextBatch][4], qb_[kNextBatch][4];
#pragma unroll
    for (int u = 0; u < kNextBatch; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = (qb + 256 * u) * 4 + j;
            zb[u][j] = t < t_hi ? z[t] : 0.f;
            qb_[u][j] = (q && t < t_hi) ? q[t] : 0.f;
        }
#pragma unroll
    for (int u = 0; u < kNextBatch; ++u) {
        const int qd = qb + 256 * u;
        if (qd * 4 >= t_hi) break;
        uint64_t w[4] = {(uint64_t)qd, (uint64_t)i, (uint64_t)a.round, 2};
        philox4x64_10(w, sd.seed, sd.stream);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = qd * 4 + j;
            if (t >= t_hi) break;
            const float sv = zb[u][j] * inv_t;
            float key;
            if (q) {
                const float d = __expf(sv - M) * inv_z - qb_[u][j];
                // (the hardware base-2 logarithm, as for the Gumbel noise)
                key = d > 0.f ? __builtin_amdgcn_logf(d) * 0.6931471805599453f : -INFINITY;
            } else {
                key = sv;
            }
            key += gumbel(u23(w[j]));
            if (key > s.best || (key == s.best && t < s.idx)) {
                s.best = key;
                s.idx = t;
            }
        }
    }
    }
    s = block_stat(s);
    if (threadIdx.x == 0) {
        float* o = a.stats2 + ((size_t)r * a.nchunk + c) * 4;
        o[0] = -INFINITY;
        o[1] = 0.f;
        o[2] = s.best;
        o[3] = __int_as_float(s.idx);
    }
}

// Acceptance: every drafted row's test is independent of the others (its own
// counter), so each wave takes rows wave, wave + kVerWaves, ... (statistics
// merge, draft id, the accept draw), the tests land in LDS, and the accepted
// run is their first failure; next is the rejected (or bonus) row's draw.
constexpr int kVerWaves = 16;
constexpr int kVerMaxRows = 512;       // n_k + 1 <= blockSize <= 512
template <bool ONE>
__global__ __launch_bounds__(64 * kVerWaves) void k_verify_final(VerifyArgs a) {
    __shared__ uint8_t s_ok[kVerMaxRows];
    __shared__ int s_next[kVerMaxRows];
    const int k = blockIdx.x, wave = threadIdx.x >> 6;
    const int off = verify_off<ONE>(a, k), r0 = off + k;
    const int n = min(verify_off<ONE>(a, k + 1) - off, kVerMaxRows - 1);   // (the API bounds it by blockSize - 1)
    const SeqDesc sd = verify_seq<ONE>(a, k);
    for (int j = wave; j <= n; j += kVerWaves) {
        const Stat s = row_stat(a.stats, a.nchunk, r0 + j);
        bool ok = false;
        if (j < n) {
            const int x = a.draft_ids[off + j];
            if (x < 0 || x >= a.V) {
                ok = false;              // outside the vocabulary: never accepted, nothing loaded
            } else if (a.temperature == 0.f) {
                ok = s.idx == x;
            } else {
                const float p = __expf(a.target[(size_t)(r0 + j) * a.V + x] / a.temperature - s.m) / s.l;
                const float q = a.draft_probs[(size_t)(off + j) * a.V + x];
                uint64_t w[4] = {0, (uint64_t)j, (uint64_t)a.round, 1};
                philox4x64_10(w, sd.seed, sd.stream);
                ok = u23(w[0]) * q <= p;
            }
        }
        const int nx = a.temperature == 0.f ? s.idx : row_stat(a.stats2, a.nchunk, r0 + j).idx;
        if ((threadIdx.x & 63) == 0) {
            s_ok[j] = ok;
            s_next[j] = nx;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int acc = 0;
        while (acc < n && s_ok[acc]) ++acc;
        a.accepted[k] = acc;
        a.next[k] = s_next[acc];
    }
}

// ---------------------------------------------------------------------------
// DFlash2 candidate selector.  Pass 1, per (row, 4096-token chunk): the
// chunk's K best logits (value descending, id ascending), by K rounds of a
// workgroup argmax over the 16 values each thread holds; with dense output
// the chunk of the row's dense distribution is zeroed on the way.  Pass 2,
// per row: merge the chunks' candidates into the row's K best and, as the
// row's predecessor is one of the K candidates of the row before (the
// anchor first), the bigram term <P[p], Q[c]> of every predecessor
// candidate p and candidate c.  Pass 3, per session, its rows in order:
// candidate c scores z(c) + the term of the row before's choice, softmax
// over the K candidates at temperature T and a Gumbel-max draw (u of rank j
// from Philox4x64-10 counter (j div 4, position, round, 3), word j mod 4),
// or the best score when T = 0; the choice is the next row's predecessor.
// ---------------------------------------------------------------------------
// Order-preserving int32 image of a float (-0 taken as +0, as the float
// comparison does): a > b as floats iff key(a) > key(b); -inf maps above
// INT_MIN, which therefore marks a slot holding no token.
__device__ __forceinline__ int sel_key(float f) {
    const int u = __float_as_int(f + 0.f);
    return u >= 0 ? u : u ^ 0x7FFFFFFF;
}
__device__ __forceinline__ float sel_unkey(int k) { return __int_as_float(k >= 0 ? k : k ^ 0x7FFFFFFF); }
constexpr int kSelGone = INT_MIN;
// (key, id) as one int64 whose order is key first, then the lower id
__device__ __forceinline__ long long sel_pack(int key, int id) {
    return (long long)(((unsigned long long)(unsigned)key << 32) | (unsigned)(0x7FFFFFFF - id));
}
__device__ __forceinline__ int sel_pack_key(long long b) { return (int)(b >> 32); }
__device__ __forceinline__ int sel_pack_id(long long b) { return 0x7FFFFFFF - (int)(unsigned)(b & 0xFFFFFFFFll); }
constexpr long long kSelNone = -0x7FFFFFFFFFFFFFFFll - 1;   // sel_pack(kSelGone, INT_MAX): below every real entry

// Wave maxima of packed entries by DPP lane moves (no LDS round trip per
// step): quad swaps, half-row and row mirrors give every lane of a 16-lane
// row its row's maximum; two row broadcasts carry rows 0-2 into row 3.  The
// whole wave must be active.
template <int CTRL, int ROWS>
__device__ __forceinline__ long long sel_dpp_max(long long v) {
    const int lo = (int)(unsigned)v, hi = (int)(v >> 32);
    const int lo2 = __builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWS, 0xF, false);
    const int hi2 = __builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWS, 0xF, false);
    const long long o = (long long)(((unsigned long long)(unsigned)hi2 << 32) | (unsigned)lo2);
    return o > v ? o : v;
}
__device__ __forceinline__ long long sel_lane(long long v, int l) {
    const int lo = __builtin_amdgcn_readlane((int)(unsigned)v, l), hi = __builtin_amdgcn_readlane((int)(v >> 32), l);
    return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ long long sel_row_max(long long v) {   // lanes 0..15, returned to every lane
    v = sel_dpp_max<0xB1, 0xF>(v);      // quad_perm [1, 0, 3, 2]
    v = sel_dpp_max<0x4E, 0xF>(v);      // quad_perm [2, 3, 0, 1]
    v = sel_dpp_max<0x141, 0xF>(v);     // row_half_mirror
    v = sel_dpp_max<0x140, 0xF>(v);     // row_mirror
    return sel_lane(v, 0);
}
__device__ __forceinline__ long long sel_wave_max(long long v) {  // all 64 lanes, returned to every lane
    v = sel_dpp_max<0xB1, 0xF>(v);
    v = sel_dpp_max<0x4E, 0xF>(v);
    v = sel_dpp_max<0x141, 0xF>(v);
    v = sel_dpp_max<0x140, 0xF>(v);
    v = sel_dpp_max<0x142, 0xA>(v);     // row_bcast:15 into rows 1 and 3
    v = sel_dpp_max<0x143, 0xC>(v);     // row_bcast:31 into rows 2 and 3
    return sel_lane(v, 63);
}

template <bool DENSE>
__global__ __launch_bounds__(256) void k_sel_topk(SelectArgs a) {
    __shared__ long long sw[4];
    const int c = blockIdx.x, r = blockIdx.y, tid = threadIdx.x, wave = tid >> 6;
    const int t_lo = c * a.chunk, t_hi = min(a.V, t_lo + a.chunk);
    const float* z = a.logits + (size_t)r * a.V;
    // every token of the chunk stays eligible, -inf included (a NaN logit
    // counts as -inf), so each chunk hands out min(K, its tokens) real ids
    // and a row's K best are always real tokens; slots past the vocabulary
    // and tokens already taken hold kSelGone, which no comparison picks
    int kv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int t = t_lo + tid + 256 * j;
        const float x = t < t_hi ? z[t] : 0.f;
        kv[j] = t < t_hi ? sel_key(x == x ? x : -INFINITY) : kSelGone;
        if (DENSE && t < t_hi) a.dense[(size_t)r * a.V + t] = 0.f;
    }
    for (int k = 0; k < a.K; ++k) {
        int bk = kSelGone, bi = INT_MAX;
#pragma unroll
        for (int j = 0; j < 16; ++j)                     // ids ascend with j: ties keep the lower id
            if (kv[j] > bk) {
                bk = kv[j];
                bi = t_lo + tid + 256 * j;
            }
        long long b = sel_wave_max(sel_pack(bk, bi));
        if ((tid & 63) == 0) sw[wave] = b;
        __syncthreads();
        b = sw[0];
#pragma unroll
        for (int w = 1; w < 4; ++w) b = sw[w] > b ? sw[w] : b;
        __syncthreads();
        const int wk = sel_pack_key(b), wi = sel_pack_id(b);
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (wi == t_lo + tid + 256 * j) kv[j] = kSelGone;
        if (tid == 0) {
            float* o = a.cand + (((size_t)r * a.nchunk + c) * kSelMaxK + k) * 2;
            o[0] = wk == kSelGone ? -INFINITY : sel_unkey(wk);   // no token left: sorts last in the merge
            o[1] = __int_as_float(wk == kSelGone ? INT_MAX : wi);
        }
    }
}

// The K best of row r over its chunks' candidates (rank j held by lane j of
// the calling wave; ties to the lower id).  The whole wave calls it.
__device__ __forceinline__ void sel_merge_row(const SelectArgs& a, int r, int lane, int& cid, float& cz) {
    const float* ent = a.cand + (size_t)r * a.nchunk * kSelMaxK * 2;
    const int E = a.nchunk * a.K;                        // <= kSelMaxEntries: 16 entries per lane
    long long eb[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int e = lane + 64 * u;
        eb[u] = kSelNone;
        if (e < E) {
            const float* o = ent + ((size_t)(e / a.K) * kSelMaxK + e % a.K) * 2;
            const int id = __float_as_int(o[1]);
            if (id != INT_MAX) eb[u] = sel_pack(sel_key(o[0]), id);
        }
    }
    cid = INT_MAX;
    cz = -INFINITY;
    for (int j = 0; j < a.K; ++j) {
        long long b = kSelNone;
#pragma unroll
        for (int u = 0; u < 16; ++u) b = eb[u] > b ? eb[u] : b;
        b = sel_wave_max(b);
#pragma unroll
        for (int u = 0; u < 16; ++u) eb[u] = eb[u] == b ? kSelNone : eb[u];
        if (lane == j) {
            cid = sel_pack_id(b);
            cz = sel_unkey(sel_pack_key(b));
        }
    }
}

// a call's sessions: from its tables, or one session from the arguments
__device__ __forceinline__ int sel_off(const SelectArgs& a, int k) { return a.offs ? a.offs[k] : (k == 0 ? 0 : a.R); }
__device__ __forceinline__ SeqDesc sel_seq(const SelectArgs& a, int k) { return a.seqs ? a.seqs[k] : a.seq0; }
__device__ __forceinline__ int sel_anchor(const SelectArgs& a, int k) {
    return a.anchors ? a.anchors[k] : a.seq0.current;
}

// Pass 2, one workgroup per drafted row (session k, position i): nothing a
// row's choice depends on except its predecessor, and that is one of the
// K candidates of the row before (the anchor at i = 0), so every row's
// candidates and the bigram terms <P[p], Q[c]> for each predecessor
// candidate p and candidate c are computed here, all rows at once.
__global__ __launch_bounds__(256) void k_sel_prep(SelectArgs a) {
    __shared__ int s_cid[kSelMaxK], s_pid[kSelMaxK];
    __shared__ float s_cz[kSelMaxK];
    __shared__ float s_p[kSelMaxK][kSelMaxDs + 1], s_q[kSelMaxK][kSelMaxDs + 1];
    __shared__ int s_k;
    const int r = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (wave == 0) {   // the row's session: offs[k] <= r < offs[k + 1]
        int k = 0;
        for (int k0 = 0; a.offs && k0 < a.nseq; k0 += 64) {
            const int kk = k0 + lane;
            const bool hit = kk < a.nseq && a.offs[kk] <= r && r < a.offs[kk + 1];
            const uint64_t m = __ballot(hit);
            if (m) {
                k = k0 + __ffsll((unsigned long long)m) - 1;
                break;
            }
        }
        if (lane == 0) s_k = k;
    }
    __syncthreads();
    const int k = s_k, i = r - sel_off(a, k);
    const int Kp = i == 0 ? 1 : a.K;                     // predecessor candidates
    if (wave == 0) {
        int cid;
        float cz;
        sel_merge_row(a, r, lane, cid, cz);
        if (lane < a.K) {
            s_cid[lane] = cid;
            s_cz[lane] = cz;
        }
    } else if (wave == 1) {
        if (i == 0) {
            if (lane == 0) s_pid[0] = sel_anchor(a, k);
        } else {
            int cid;
            float cz;
            sel_merge_row(a, r - 1, lane, cid, cz);
            if (lane < a.K) s_pid[lane] = cid;
        }
    }
    __syncthreads();
    // the predecessor rows of P and the candidate rows of Q, as fp32 in LDS
    for (int e = tid; e < (Kp + a.K) * a.Ds; e += 256) {
        const int row = e / a.Ds, d = e - row * a.Ds;
        if (row < Kp) s_p[row][d] = ld_any(a.P, (size_t)s_pid[row] * a.Ds + d, a.w_bf16);
        else s_q[row - Kp][d] = ld_any(a.Q, (size_t)s_cid[row - Kp] * a.Ds + d, a.w_bf16);
    }
    __syncthreads();
    float* o = a.prep + (size_t)r * kSelPrepStride;
    if (tid < a.K) {
        o[tid] = __int_as_float(s_cid[tid]);
        o[kSelMaxK + tid] = s_cz[tid];
    }
    for (int pc = tid; pc < Kp * a.K; pc += 256) {
        const int pi = pc / a.K, c = pc - pi * a.K;
        float t = 0.f;
        for (int d = 0; d < a.Ds; ++d) t += s_p[pi][d] * s_q[c][d];
        o[2 * kSelMaxK + pi * kSelMaxK + c] = t;
    }
}

// Pass 3, one workgroup per session, its rows kSelWalkRows at a time: the
// prepared rows are staged in LDS and the Gumbel noise of every (row, rank)
// is drawn at once (u of rank j from Philox4x64-10 counter (j div 4, i + 1,
// round, 3), word j mod 4); then one wave walks the rows in order, lane c
// scoring candidate c as z + <P[prev], Q[c]> (the term of the rank chosen at
// the row before), at T > 0 divided by T plus its noise, and the best by a
// DPP maximum (the lower rank on a tie): that maximum is all the chain from
// one row to the next holds.  All threads then write the rows' outputs: the
// candidate ids, the chosen token and, at T > 0, the softmax over the K of
// score / T as probabilities and dense rows.
constexpr int kSelWalkRows = 32;
__global__ __launch_bounds__(256) void k_sel_walk(SelectArgs a) {
    __shared__ float sp[kSelWalkRows * kSelPrepStride];
    __shared__ float sg[kSelWalkRows * kSelMaxK];
    __shared__ int sch[kSelWalkRows + 1];   // rank chosen at each row of the chunk; [0]: at the row before it
    const int k = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const SeqDesc sd = sel_seq(a, k);
    const int r0 = sel_off(a, k), n = sel_off(a, k + 1) - r0;
    const bool sampling = a.temperature > 0.f;
    const float inv_t = sampling ? 1.f / a.temperature : 0.f;
    const int K = a.K, nq = (K + 3) >> 2;
    int p = 0;                                           // rank of the row before's choice (the anchor: 0)
    for (int i0 = 0; i0 < n; i0 += kSelWalkRows) {
        const int m = min(kSelWalkRows, n - i0);
        __syncthreads();
        for (int e = tid; e < m * kSelPrepStride; e += 256) sp[e] = a.prep[(size_t)(r0 + i0) * kSelPrepStride + e];
        if (sampling)
            for (int e = tid; e < m * nq; e += 256) {
                const int ii = e / nq, qd = e - ii * nq;
                uint64_t w[4] = {(uint64_t)qd, (uint64_t)(i0 + ii + 1), (uint64_t)a.round, 3};
                philox4x64_10(w, sd.seed, sd.stream);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    if (4 * qd + jj < K) sg[ii * kSelMaxK + 4 * qd + jj] = -logf(-logf(u23(w[jj])));
            }
        if (tid == 0) sch[0] = p;
        __syncthreads();
        if (wave == 0) {                                 // the whole wave: the DPP maximum needs every lane
            const bool act = lane < K;
            for (int ii = 0; ii < m; ++ii) {
                const float* q = sp + ii * kSelPrepStride;
                long long b = kSelNone;
                if (act) {
                    const float sc = q[kSelMaxK + lane] + q[2 * kSelMaxK + p * kSelMaxK + lane];
                    b = sel_pack(sel_key(sampling ? sc * inv_t + sg[ii * kSelMaxK + lane] : sc), lane);
                }
                p = sel_pack_id(sel_row_max(b));
                if (lane == 0) sch[ii + 1] = p;
            }
        }
        __syncthreads();
        for (int e = tid; e < m * K; e += 256) {
            const int ii = e / K, c = e - ii * K, r = r0 + i0 + ii;
            const float* q = sp + ii * kSelPrepStride;
            const int cid = __float_as_int(q[c]);
            a.cand_ids[(size_t)r * K + c] = cid;
            if (c == sch[ii + 1]) a.tokens[r] = cid;
            if (sampling && (a.cand_probs || a.dense)) {
                const float* tz = q + kSelMaxK;
                const float* tb = q + 2 * kSelMaxK + sch[ii] * kSelMaxK;
                float mx = -INFINITY;
                for (int c2 = 0; c2 < K; ++c2) mx = fmaxf(mx, (tz[c2] + tb[c2]) * inv_t);
                float sum = 0.f;
                for (int c2 = 0; c2 < K; ++c2) sum += __expf((tz[c2] + tb[c2]) * inv_t - mx);
                const float prob = __expf((tz[c] + tb[c]) * inv_t - mx) / sum;
                if (a.cand_probs) a.cand_probs[(size_t)r * K + c] = prob;
                if (a.dense) a.dense[(size_t)r * a.V + cid] = prob;
            }
        }
        p = sch[m];
    }
}

hipError_t select(const SelectArgs& a, hipStream_t st) {
    if (a.R <= 0 || a.nseq <= 0) return hipSuccess;
    if (a.K < 1 || a.K > kSelMaxK || a.Ds < 1 || a.Ds > kSelMaxDs || a.nchunk * a.K > kSelMaxEntries ||
        a.chunk != 4096 || !a.prep || (a.seqs ? !a.offs || !a.anchors : a.nseq != 1 || a.offs || a.anchors))
        return hipErrorInvalidValue;
    if (a.dense) hipLaunchKernelGGL(k_sel_topk<true>, dim3(a.nchunk, a.R), dim3(256), 0, st, a);
    else hipLaunchKernelGGL(k_sel_topk<false>, dim3(a.nchunk, a.R), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_sel_prep, dim3(a.R), dim3(256), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_sel_walk, dim3(a.nseq), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <bool ONE>
static hipError_t verify_launch(const VerifyArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(k_verify_stats, dim3(a.nchunk, a.Rt), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.temperature > 0.f) {
        hipLaunchKernelGGL(k_verify_next<ONE>, dim3(a.nchunk, a.Rt), dim3(256), 0, st, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_verify_final<ONE>, dim3(a.nseq), dim3(64 * kVerWaves), 0, st, a);
    return hipGetLastError();
}

hipError_t verify(const VerifyArgs& a, hipStream_t st) {
    if (a.nseq <= 0) return hipSuccess;
    if (!a.rows && a.nseq != 1) return hipErrorInvalidValue;   // no tables: exactly one session
    return a.rows ? verify_launch<false>(a, st) : verify_launch<true>(a, st);
}

}  // namespace kern
}  // namespace dflash
