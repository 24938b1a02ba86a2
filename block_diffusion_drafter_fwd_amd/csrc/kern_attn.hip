// Short-query attention of the block rows over the draft KV cache.
//
// Row i of a block sits at position p = F + i; key position s is visible iff
// s < F + M, s <= p when the in-block mask is causal, and p - s < W when a
// sliding window is set (mlxcel PR "add the Laguna DFlash drafter": a
// per-query window over [context | block]).  GQA maps q head h to kv head
// h / (Hq / Hkv).
//
// bf16 path (flash-decoding split over the context):
//   k_attn_partial  one workgroup per (context chunk, kv head).  The G q heads
//                   of that kv head times M block rows form up to 64 query rows
//                   (4 waves x 16).  Per 64-key tile: K and V^T staged in LDS,
//                   S^T = K . Q^T with v_mfma_f32_16x16x32_bf16 (its output
//                   layout holds, per lane, the 4 keys the next product's B
//                   operand needs; two key tiles fill one k = 32 step),
//                   online softmax in fp32, O^T += V^T . P^T.
//                   Writes unnormalised O with its running max and sum.
//   k_attn_combine  merges the chunks of each (row, q head) with weights
//                   staged in LDS, applies the per-head sigmoid gate.
// fp32 path (tiny configurations): k_attn_f32, one workgroup per (row, head).
#include "kernels.h"

namespace dflash {
namespace kern {

typedef __attribute__((ext_vector_type(4))) float f32x4_t;

__device__ __forceinline__ uint16_t f2bf(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ int find_item_seq(const SeqDesc* seqs, int nseq, int item) {
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {                       // last seq with item0 <= item
        const int mid = (lo + hi + 1) >> 1;
        if (seqs[mid].item0 <= item) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ bool visible(int s, int p, int kend, int causal, int window) {
    return s < kend && (!causal || s <= p) && (!window || p - s < window);
}

constexpr int kKT = 64;                 // keys per tile
constexpr int kD = 128;                 // head dim of the bf16 path
constexpr int kKLD = kD + 8;            // LDS row stride of K (elements)
constexpr int kVLD = kKT + 8;           // LDS row stride of V^T

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

__device__ __forceinline__ f32x4_t mfma32(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// V^T is stored with its 4-key groups XOR-swizzled by the row's 8-row band,
// which makes the transposing stores conflict-free and keeps every 4-key group
// contiguous (8-byte aligned) for the fragment reads.
__device__ __forceinline__ int vt_index(int d, int key) { return d * kVLD + (key ^ (((d >> 3) & 15) << 2)); }

__global__ __launch_bounds__(256) void k_attn_partial(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sK[kKT * kKLD];
    __shared__ __attribute__((aligned(16))) uint16_t sVt[kD * kVLD];

    const int item = blockIdx.x, g = blockIdx.y;
    const SeqDesc sd = a.seqs[find_item_seq(a.seqs, a.nseq, item)];
    const int c = item - sd.item0;
    const int kend = sd.F + sd.M;
    const int kb = sd.key_lo + c * a.chunk;
    const int ke = min(kend, kb + a.chunk);
    const int G = a.Hq / a.Hkv;
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63, r = lane & 15, q = lane >> 4;
    const int row = wave * 16 + r;
    const bool rvalid = row < sd.M * G;
    const int qi = rvalid ? row / G : 0;
    const int hq = g * G + (rvalid ? row % G : 0);
    const int p = sd.F + qi;
    const int p_last = sd.F + sd.M - 1;

    // Q^T as the B operand of S^T = K Q^T: lane (r, q) holds Q[row r][32 j + 8 q .. +8]
    u32x4_t qf[4];
    {
        const uint16_t* Qp = (const uint16_t*)a.Q + ((size_t)(sd.q_row0 + qi) * a.Hq + hq) * kD;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            qf[j] = rvalid ? *(const u32x4_t*)(Qp + j * 32 + 8 * q) : u32x4_t{0u, 0u, 0u, 0u};
    }
    const size_t headsz = (size_t)sd.cap * kD;
    const uint16_t* Kc = (const uint16_t*)sd.cache + ((size_t)(a.layer * 2 + 0) * a.Hkv + g) * headsz;
    const uint16_t* Vc = (const uint16_t*)sd.cache + ((size_t)(a.layer * 2 + 1) * a.Hkv + g) * headsz;

    float m_run = -INFINITY, l_run = 0.f;
    f32x4_t o[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // 64-key tiles: the next tile's K and V are loaded into registers while
    // the current one is multiplied out of LDS
    uint4 kreg[4], vreg[4];
#define DF_ATTN_LOAD(T0)                                                        \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                             \
        const int idx_ = t + 256 * i;                                           \
        const int kp_ = (T0) + (idx_ >> 4), dc_ = (idx_ & 15) * 8;               \
        kreg[i] = uint4{0u, 0u, 0u, 0u};                                        \
        vreg[i] = uint4{0u, 0u, 0u, 0u};                                        \
        if (kp_ < ke) {                                                         \
            const int slot_ = sd.ring ? kp_ % sd.cap : kp_;                     \
            kreg[i] = *(const uint4*)(Kc + (size_t)slot_ * kD + dc_);           \
            vreg[i] = *(const uint4*)(Vc + (size_t)slot_ * kD + dc_);           \
        }                                                                       \
    }
    DF_ATTN_LOAD(kb)
    for (int t0 = kb; t0 < ke; t0 += kKT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = t + 256 * i;
            const int key = idx >> 4, dc = (idx & 15) * 8;
            *(uint4*)&sK[key * kKLD + dc] = kreg[i];
            const uint16_t* ve = (const uint16_t*)&vreg[i];
#pragma unroll
            for (int e = 0; e < 8; ++e) sVt[vt_index(dc + e, key)] = ve[e];
        }
        __syncthreads();
        if (t0 + kKT < ke) {
            DF_ATTN_LOAD(t0 + kKT)
        }

        // S^T[key][row] for 4 key tiles of 16 (4 MFMAs of k = 32 over D)
        f32x4_t s[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4_t kf = *(const u32x4_t*)&sK[(kt * 16 + r) * kKLD + j * 32 + 8 * q];
                s[kt] = mfma32(kf, qf[j], s[kt]);
            }
        }
        // scale and mask; a tile every row sees whole (all context, inside
        // every row's window) skips the per-element test
        const bool full = t0 + kKT <= ke && t0 + kKT <= sd.F && (!a.window || p_last - t0 < a.window);
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int kp = t0 + kt * 16 + 4 * q + e;
                const bool ok = full || (rvalid && visible(kp, p, ke, a.causal, a.window));
                s[kt][e] = ok ? s[kt][e] * a.scale : -INFINITY;
                mx = fmaxf(mx, s[kt][e]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_run == -INFINITY ? 0.f : __expf(m_run - m_new);
        float sum = 0.f;
        uint2 pf[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            float pe[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pe[e] = s[kt][e] == -INFINITY ? 0.f : __expf(s[kt][e] - m_new);
                sum += pe[e];
            }
            pf[kt].x = (uint32_t)f2bf(pe[0]) | ((uint32_t)f2bf(pe[1]) << 16);
            pf[kt].y = (uint32_t)f2bf(pe[2]) | ((uint32_t)f2bf(pe[3]) << 16);
        }
        sum += __shfl_xor(sum, 16);
        sum += __shfl_xor(sum, 32);
        l_run = l_run * alpha + sum;
        m_run = m_new;
        // O^T[d][row] = alpha * O^T + V^T . P^T, k = 32 per MFMA: element e of
        // lane q stands for key 4q + e of tile 2h (e < 4) or tile 2h + 1 (e >= 4),
        // for both operands
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            o[dt] *= alpha;
            const int d = dt * 16 + r;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const uint2 v0 = *(const uint2*)&sVt[vt_index(d, (2 * h2) * 16 + 4 * q)];
                const uint2 v1 = *(const uint2*)&sVt[vt_index(d, (2 * h2 + 1) * 16 + 4 * q)];
                const u32x4_t vf = {v0.x, v0.y, v1.x, v1.y};
                const u32x4_t pp = {pf[2 * h2].x, pf[2 * h2].y, pf[2 * h2 + 1].x, pf[2 * h2 + 1].y};
                o[dt] = mfma32(vf, pp, o[dt]);
            }
        }
        __syncthreads();
    }
#undef DF_ATTN_LOAD
    if (!rvalid) return;
    const size_t base = ((size_t)item * a.Hkv + g) * 64 + row;
    float* po = a.part_o + base * kD;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
        *(float4*)(po + dt * 16 + 4 * q) = float4{o[dt][0], o[dt][1], o[dt][2], o[dt][3]};
    if (q == 0) {
        a.part_ml[base * 2] = m_run;
        a.part_ml[base * 2 + 1] = l_run;
    }
}

// One workgroup per (block row, q head), one thread per output dim.  The
// chunk maxima and sums are staged in LDS (independent loads), turned into
// weights exp(m_c - M), and the partial outputs are summed with those
// weights; chunks are taken 1024 at a time with a running merge.
constexpr int kCombItems = 1024;

__global__ __launch_bounds__(128) void k_attn_combine(AttnArgs a) {
    __shared__ float sw[kCombItems];
    __shared__ float red[2][2];
    const int brow = blockIdx.x, hq = blockIdx.y, t = threadIdx.x;
    const RowInfo ri = a.rows[brow];
    const SeqDesc sd = a.seqs[ri.seq];
    const int G = a.Hq / a.Hkv, g = hq / G;
    const int row = (ri.pos - sd.F) * G + hq % G;
    const size_t stride = (size_t)a.Hkv * 64;                    // between items
    const size_t base0 = ((size_t)sd.item0 * a.Hkv + g) * 64 + row;
    float M_run = -INFINITY, L_run = 0.f, acc = 0.f;
    for (int c0 = 0; c0 < sd.nitems; c0 += kCombItems) {
        const int nc = min(kCombItems, sd.nitems - c0);
        float mx = -INFINITY;
        for (int c = t; c < nc; c += 128) {
            const float m = a.part_ml[(base0 + (size_t)(c0 + c) * stride) * 2];
            sw[c] = m;
            mx = fmaxf(mx, m);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        if ((t & 63) == 0) red[0][t >> 6] = mx;
        __syncthreads();
        const float M = fmaxf(fmaxf(red[0][0], red[0][1]), M_run);
        float lsum = 0.f;
        for (int c = t; c < nc; c += 128) {
            const float m = sw[c];
            const float w = m == -INFINITY ? 0.f : __expf(m - M);
            sw[c] = w;
            lsum += w * a.part_ml[(base0 + (size_t)(c0 + c) * stride) * 2 + 1];
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o);
        if ((t & 63) == 0) red[1][t >> 6] = lsum;
        __syncthreads();
        const float sc = M_run == -INFINITY ? 0.f : __expf(M_run - M);
        float part = 0.f;
        const float* po = a.part_o + (base0 + (size_t)c0 * stride) * kD + t;
#pragma unroll 8
        for (int c = 0; c < nc; ++c) part += sw[c] * po[(size_t)c * stride * kD];
        acc = acc * sc + part;
        L_run = L_run * sc + red[1][0] + red[1][1];
        M_run = M;
        __syncthreads();
    }
    float out = acc / L_run;
    if (a.gate) {
        float gv = 0.f;
        for (int sp = 0; sp < a.gate_nsplit; ++sp)
            gv += a.gate_src[(size_t)sp * a.gate_stride + (size_t)brow * a.gate_ld + a.gate_col + hq];
        out *= 1.f / (1.f + __expf(-gv));
    }
    const size_t o = (size_t)brow * a.Hq * kD + (size_t)hq * kD + t;
    if (a.out_bf16) ((uint16_t*)a.out)[o] = f2bf(out);
    else ((float*)a.out)[o] = out;
}

// fp32: one workgroup of 64 threads per (block row, q head); D <= 64
__global__ __launch_bounds__(64) void k_attn_f32(AttnArgs a) {
    __shared__ float sq[64];
    __shared__ float sm[64], sl[64];
    __shared__ float so[64][65];
    const int brow = blockIdx.x, hq = blockIdx.y, t = threadIdx.x;
    const RowInfo ri = a.rows[brow];
    const SeqDesc sd = a.seqs[ri.seq];
    const int G = a.Hq / a.Hkv, g = hq / G, D = a.D;
    const int p = ri.pos;
    const int kend = sd.F + sd.M;
    if (t < D) sq[t] = ((const float*)a.Q)[((size_t)brow * a.Hq + hq) * D + t];
    __syncthreads();
    const size_t headsz = (size_t)sd.cap * D;
    const float* Kc = (const float*)sd.cache + ((size_t)(a.layer * 2 + 0) * a.Hkv + g) * headsz;
    const float* Vc = (const float*)sd.cache + ((size_t)(a.layer * 2 + 1) * a.Hkv + g) * headsz;
    float m = -INFINITY, l = 0.f, o[64];
    for (int d = 0; d < 64; ++d) o[d] = 0.f;
    for (int s = sd.key_lo + t; s < kend; s += 64) {
        if (!visible(s, p, kend, a.causal, a.window)) continue;
        const int slot = sd.ring ? s % sd.cap : s;
        const float* kr = Kc + (size_t)slot * D;
        const float* vr = Vc + (size_t)slot * D;
        float dot = 0.f;
        for (int d = 0; d < D; ++d) dot = fmaf(sq[d], kr[d], dot);
        dot *= a.scale;
        const float mn = fmaxf(m, dot);
        const float al = m == -INFINITY ? 0.f : expf(m - mn);
        const float pe = expf(dot - mn);
        l = l * al + pe;
        for (int d = 0; d < D; ++d) o[d] = o[d] * al + pe * vr[d];
        m = mn;
    }
    sm[t] = m;
    sl[t] = l;
    for (int d = 0; d < D; ++d) so[t][d] = o[d];
    __syncthreads();
    if (t >= D) return;
    float M = -INFINITY;
    for (int j = 0; j < 64; ++j) M = fmaxf(M, sm[j]);
    float L = 0.f, acc = 0.f;
    for (int j = 0; j < 64; ++j) {
        if (sm[j] == -INFINITY) continue;
        const float w = expf(sm[j] - M);
        L += sl[j] * w;
        acc += so[j][t] * w;
    }
    float out = acc / L;
    if (a.gate) {
        float gv = 0.f;
        for (int sp = 0; sp < a.gate_nsplit; ++sp)
            gv += a.gate_src[(size_t)sp * a.gate_stride + (size_t)brow * a.gate_ld + a.gate_col + hq];
        out *= 1.f / (1.f + expf(-gv));
    }
    ((float*)a.out)[(size_t)brow * a.Hq * D + (size_t)hq * D + t] = out;
}

hipError_t attention(const AttnArgs& a, bool bf16, hipStream_t st) {
    if (a.nrows <= 0) return hipSuccess;
    if (!bf16) {
        hipLaunchKernelGGL(k_attn_f32, dim3(a.nrows, a.Hq), dim3(64), 0, st, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_attn_partial, dim3(a.total_items, a.Hkv), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_attn_combine, dim3(a.nrows, a.Hq), dim3(kD), 0, st, a);
    return hipGetLastError();
}

}  // namespace kern
}  // namespace dflash
