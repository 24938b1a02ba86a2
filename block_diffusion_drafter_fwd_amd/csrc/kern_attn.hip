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
//                   S^T = K . Q^T with v_mfma_f32_16x16x16_bf16 (its output
//                   layout is exactly the B-operand layout the next product
//                   needs), online softmax in fp32, O^T += V^T . P^T.
//                   Writes unnormalised O with its running max and sum.
//   k_attn_combine  merges the chunks of each (row, q head), applies the
//                   per-head sigmoid gate, stores the attention output.
// fp32 path (tiny configurations): k_attn_f32, one workgroup per (row, head).
#include "kernels.h"

namespace dflash {
namespace kern {

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

__device__ __forceinline__ f32x4_t mfma16(uint2 a, uint2 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, a),
                                                     __builtin_bit_cast(bf16x4_t, b), c, 0, 0, 0);
}

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

    // Q^T as the B operand: lane (r, q) holds Q[row r][16 d + 4 q .. +4]
    uint2 qf[8];
    {
        const uint16_t* Qp = (const uint16_t*)a.Q + ((size_t)(sd.q_row0 + qi) * a.Hq + hq) * kD;
#pragma unroll
        for (int d = 0; d < 8; ++d)
            qf[d] = rvalid ? *(const uint2*)(Qp + d * 16 + 4 * q) : uint2{0u, 0u};
    }
    const size_t headsz = (size_t)sd.cap * kD;
    const uint16_t* Kc = (const uint16_t*)sd.cache + ((size_t)(a.layer * 2 + 0) * a.Hkv + g) * headsz;
    const uint16_t* Vc = (const uint16_t*)sd.cache + ((size_t)(a.layer * 2 + 1) * a.Hkv + g) * headsz;

    float m_run = -INFINITY, l_run = 0.f;
    f32x4_t o[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int t0 = kb; t0 < ke; t0 += kKT) {
        // stage 64 keys: 1024 16-byte pieces each of K and V
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = t + 256 * i;
            const int key = idx >> 4, dc = (idx & 15) * 8;
            const int kp = t0 + key;
            uint4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
            if (kp < ke) {
                const int slot = sd.ring ? kp % sd.cap : kp;
                kv = *(const uint4*)(Kc + (size_t)slot * kD + dc);
                vv = *(const uint4*)(Vc + (size_t)slot * kD + dc);
            }
            *(uint4*)&sK[key * kKLD + dc] = kv;
            const uint16_t* ve = (const uint16_t*)&vv;
#pragma unroll
            for (int e = 0; e < 8; ++e) sVt[(dc + e) * kVLD + key] = ve[e];
        }
        __syncthreads();

        // S^T[key][row] for 4 key tiles of 16
        f32x4_t s[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                const uint2 kf = *(const uint2*)&sK[(kt * 16 + r) * kKLD + d * 16 + 4 * q];
                s[kt] = mfma16(kf, qf[d], s[kt]);
            }
        }
        // mask, scale, running max of this lane's row r
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int kp = t0 + kt * 16 + 4 * q + e;
                const bool ok = rvalid && visible(kp, p, ke, a.causal, a.window);
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
        // O^T[d][row] = alpha * O^T + V^T . P^T
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            o[dt] *= alpha;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const uint2 vf = *(const uint2*)&sVt[(dt * 16 + r) * kVLD + kt * 16 + 4 * q];
                o[dt] = mfma16(vf, pf[kt], o[dt]);
            }
        }
        __syncthreads();
    }
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

__global__ __launch_bounds__(128) void k_attn_combine(AttnArgs a) {
    const int brow = blockIdx.x, hq = blockIdx.y, d = threadIdx.x;
    const RowInfo ri = a.rows[brow];
    const SeqDesc sd = a.seqs[ri.seq];
    const int G = a.Hq / a.Hkv, g = hq / G;
    const int row = (ri.pos - sd.F) * G + hq % G;
    float M = -INFINITY;
    for (int c = 0; c < sd.nitems; ++c)
        M = fmaxf(M, a.part_ml[(((size_t)(sd.item0 + c) * a.Hkv + g) * 64 + row) * 2]);
    float L = 0.f, acc = 0.f;
    for (int c = 0; c < sd.nitems; ++c) {
        const size_t base = ((size_t)(sd.item0 + c) * a.Hkv + g) * 64 + row;
        const float m = a.part_ml[base * 2];
        if (m == -INFINITY) continue;
        const float w = __expf(m - M);
        L += a.part_ml[base * 2 + 1] * w;
        acc += a.part_o[base * kD + d] * w;
    }
    float out = acc / L;
    if (a.gate) {
        const float gv = a.gate_src[(size_t)brow * a.gate_ld + a.gate_col + hq];
        out *= 1.f / (1.f + __expf(-gv));
    }
    const size_t o = (size_t)brow * a.Hq * kD + (size_t)hq * kD + d;
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
        const float gv = a.gate_src[(size_t)brow * a.gate_ld + a.gate_col + hq];
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
