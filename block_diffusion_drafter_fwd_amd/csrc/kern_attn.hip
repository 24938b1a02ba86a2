// Short-query attention of the block rows over the draft KV cache.
//
// Row i of a block sits at position p = F + i; key position s is visible iff
// s < F + M, s <= p when the in-block mask is causal, and p - s < W when a
// sliding window is set (mlxcel PR "add the Laguna DFlash drafter": a
// per-query window over [context | block]).  GQA maps q head h to kv head
// h / (Hq / Hkv).
//
// bf16 path (flash-decoding split over the context):
//   k_attn_partial  one workgroup (4 waves) per (context chunk, kv head); a
//                   chunk is a run of keys or (chunks of 256 keys and more)
//                   every nitems-th 64-key tile of the sequence.  The
//                   G q heads of that kv head times M block rows form up to 64
//                   query rows, 16 per wave.  64-key tiles of K and V are
//                   copied from the cache straight into LDS (global_load_lds,
//                   double-buffered one tile ahead) with their 16-byte pieces
//                   XOR-permuted per key; S^T = K . Q^T with
//                   v_mfma_f32_16x16x32_bf16 (its output layout holds, per
//                   lane, the 4 keys the next product's B operand needs; two
//                   key tiles fill one k = 32 step); online softmax in fp32 on
//                   the base-2 exponential; O^T += V^T . P^T with the V^T
//                   operand read from the row-major tile by the transposing
//                   LDS read (ds_read_b64_tr_b16).  Writes unnormalised O with
//                   its running max and sum.
//   k_attn_combine  merges the chunks of each (row, q head) with weights
//                   staged in LDS, applies the per-head sigmoid gate.
// fp32 path (tiny configurations): k_attn_f32, one workgroup per (row, head).
#include "kernels.h"

namespace dflash {
namespace kern {

typedef __attribute__((ext_vector_type(4))) float f32x4_t;

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// two floats to packed bf16 (round to nearest even, one conversion instruction)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// (bitwise, not short-circuit: keeps the masking branch-free)
__device__ __forceinline__ bool visible(int s, int p, int kend, int causal, int window) {
    return (s < kend) & ((causal == 0) | (s <= p)) & ((window == 0) | (p - s < window));
}

constexpr int kKT = 64;                 // keys per tile
constexpr int kD = 128;                 // head dim of the bf16 path

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

__device__ __forceinline__ f32x4_t mfma32(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

constexpr int kAttnWaves = 4;               // waves per workgroup
constexpr int kRG = 4 / kAttnWaves;         // 16-row groups per wave (64 query rows per workgroup)
constexpr int kAttnThreads = 64 * kAttnWaves;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;

// K and V tiles sit in LDS row-major (64 keys x 256 bytes), with the 16-byte
// pieces of each row XOR-permuted by the key so that the fragment reads hit
// distinct banks: K reads take 16 keys of one piece, V reads (transposing,
// ds_read_b64_tr_b16) take 8 keys of two adjacent pieces.
__device__ __forceinline__ int k_piece(int key, int c) { return key * 16 + (c ^ (key & 15)); }
__device__ __forceinline__ int v_piece(int key, int c) { return key * 16 + (c ^ ((key & 7) << 1)); }

// The waves share each 64-key tile; each owns kRG 16-row groups of the 64
// query rows (every K and V fragment read from LDS feeds kRG MFMAs).  Tiles
// are copied from the cache straight into LDS (global_load_lds, no registers)
// one tile ahead, into a second buffer; V^T fragments come from the
// row-major V tile through the transposing LDS read.
__global__ __launch_bounds__(kAttnThreads) void k_attn_partial(AttnArgs a) {
    // two buffers per operand, as separate objects: the copy into one must be
    // seen by the compiler as independent of the reads from the other, or it
    // waits for the copy before every read
    __shared__ __attribute__((aligned(16))) uint16_t sK0[kKT * kD];
    __shared__ __attribute__((aligned(16))) uint16_t sK1[kKT * kD];
    __shared__ __attribute__((aligned(16))) uint16_t sV0[kKT * kD];
    __shared__ __attribute__((aligned(16))) uint16_t sV1[kKT * kD];

    // work items in the host's order (largest chunks first, so the short
    // ones fill the end of the launch), every kv head of an item together
    // (one session, rows == nullptr: its descriptor in the arguments, items in order)
    const int rank = blockIdx.x / a.Hkv, g = blockIdx.x - rank * a.Hkv;
    int item = rank;
    SeqDesc sd = a.seq0;
    if (a.rows) {
        const uint32_t od = a.order[rank];
        item = (int)(od & 0xffffu);
        sd = a.seqs[od >> 16];
    }
    const int c = item - sd.item0;
    const int kend = sd.F + sd.M;
    // the item's tiles: one run of chunk keys, or (strided) every nitems-th
    // 64-key tile of the sequence's keys, so that the items of a kv head
    // stream neighbouring tiles at the same time
    const int kb = sd.key_lo + c * (a.strided ? kKT : a.chunk);
    const int ke = a.strided ? kend : min(kend, kb + a.chunk);
    const int kstep = a.strided ? sd.nitems * kKT : kKT;
    const int G = a.Hq / a.Hkv;
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63, r = lane & 15, q = lane >> 4;
    const int p_last = sd.F + sd.M - 1;

    // per row group: query row, validity, position; Q^T as the B operand of
    // S^T = K Q^T: lane (r, q) holds Q[row][32 j + 8 q .. +8]
    int row[kRG], pos[kRG];
    bool rvalid[kRG];
    u32x4_t qf[kRG][4];
#pragma unroll
    for (int gi = 0; gi < kRG; ++gi) {
        row[gi] = (wave * kRG + gi) * 16 + r;
        rvalid[gi] = row[gi] < sd.M * G;
        const int qi = rvalid[gi] ? row[gi] / G : 0;
        const int hq = g * G + (rvalid[gi] ? row[gi] % G : 0);
        pos[gi] = sd.F + qi;
        const uint16_t* Qp = (const uint16_t*)a.Q + ((size_t)(sd.q_row0 + qi) * a.Hq + hq) * kD;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4_t v = *(const u32x4_t*)(Qp + j * 32 + 8 * q);   // row qi is in range either way
            qf[gi][j] = rvalid[gi] ? v : u32x4_t{0u, 0u, 0u, 0u};
        }
    }
    const size_t headsz = (size_t)sd.cap * kD;
    const uint16_t* Kc = (const uint16_t*)sd.cache + ((size_t)(a.layer * 2 + 0) * a.Hkv + g) * headsz;
    const uint16_t* Vc = (const uint16_t*)sd.cache + ((size_t)(a.layer * 2 + 1) * a.Hkv + g) * headsz;

    float m_run[kRG], l_run[kRG];   // raw-score max, running sum
#pragma unroll
    for (int gi = 0; gi < kRG; ++gi) {
        m_run[gi] = -INFINITY;
        l_run[gi] = 0.f;
    }
    const float c2 = a.scale * 1.4426950408889634f;
    f32x4_t o[kRG][8];
#pragma unroll
    for (int gi = 0; gi < kRG; ++gi)
#pragma unroll
        for (int d = 0; d < 8; ++d) o[gi][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // tile copy: instruction i of this wave fills LDS pieces (8 wave + i) * 64
    // + lane, i.e. key 4 (8 wave + i) + lane / 16, position lane % 16, with the
    // piece the XOR permutation puts there.  Keys past the end copy the last
    // key (masked below, probability zero).
    auto load_tile = [&](int t0, uint16_t* dK, uint16_t* dV) {
#pragma unroll
        for (int i = 0; i < 16 / kAttnWaves; ++i) {
            const int b = wave * (16 / kAttnWaves) + i;
            const int key = 4 * b + (lane >> 4), cpos = lane & 15;
            const int kk = min(t0 + key, ke - 1);
            const int slot = sd.ring ? kk % sd.cap : kk;
            const uint16_t* krow = Kc + (size_t)slot * kD;
            const uint16_t* vrow = Vc + (size_t)slot * kD;
            __builtin_amdgcn_global_load_lds(krow + 8 * (cpos ^ (key & 15)), (lds_void_t*)&dK[b * 512], 16, 0, 0);
            __builtin_amdgcn_global_load_lds(vrow + 8 * (cpos ^ ((key & 7) << 1)), (lds_void_t*)&dV[b * 512], 16, 0, 0);
        }
    };
    auto tile = [&](int t0, const uint16_t* tK, const uint16_t* tV, uint16_t* nK, uint16_t* nV) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's copies of the tile landed
        __syncthreads();                                    // everyone's have; the other buffer is free
        if (t0 + kstep < ke) load_tile(t0 + kstep, nK, nV);

        // S^T[key][row] for 4 key tiles of 16 (4 MFMAs of k = 32 over D) per row group
        f32x4_t s[kRG][4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
            for (int gi = 0; gi < kRG; ++gi) s[gi][kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4_t kf = *(const u32x4_t*)&tK[8 * k_piece(kt * 16 + r, 4 * j + q)];
#pragma unroll
                for (int gi = 0; gi < kRG; ++gi) s[gi][kt] = mfma32(kf, qf[gi][j], s[gi][kt]);
            }
        }
        // mask; a tile every row sees whole (all context, inside every row's
        // window) skips the per-element test (the branch is uniform)
        const bool full = t0 + kKT <= ke && t0 + kKT <= sd.F && (!a.window || p_last - t0 < a.window);
        if (!full) {
#pragma unroll
            for (int gi = 0; gi < kRG; ++gi)
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int kp = t0 + kt * 16 + 4 * q + e;
                        s[gi][kt][e] = (rvalid[gi] & visible(kp, pos[gi], ke, a.causal, a.window)) ? s[gi][kt][e]
                                                                                                   : -INFINITY;
                    }
        }
        // online softmax on the raw scores in base 2: p = 2^(c s - c m) with
        // c = scale * log2(e), i.e. exp(scale s - scale m)
        uint2 pf[kRG][4];
        float alpha[kRG];
        bool rescale = false;
#pragma unroll
        for (int gi = 0; gi < kRG; ++gi) {
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
                mx = fmaxf(fmaxf(mx, fmaxf(s[gi][kt][0], s[gi][kt][1])), fmaxf(s[gi][kt][2], s[gi][kt][3]));
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run[gi], mx);
            alpha[gi] = m_run[gi] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_run[gi] - m_new) * c2);
            const float mc = m_new == -INFINITY ? 0.f : m_new * c2;   // a row with nothing visible yet: p = 0
            float sum = 0.f;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                float pe[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pe[e] = __builtin_amdgcn_exp2f(fmaf(s[gi][kt][e], c2, -mc));   // masked (-inf) scores give 0
                    sum += pe[e];
                }
                pf[gi][kt].x = pack_bf16(pe[0], pe[1]);
                pf[gi][kt].y = pack_bf16(pe[2], pe[3]);
            }
            sum += __shfl_xor(sum, 16);
            sum += __shfl_xor(sum, 32);
            l_run[gi] = l_run[gi] * alpha[gi] + sum;
            m_run[gi] = m_new;
            rescale |= alpha[gi] != 1.f;
        }
        // the accumulators are still zero on the chunk's first tile, and a
        // wave whose rows all kept their maximum needs no rescale
        if (t0 != kb && __any(rescale)) {
#pragma unroll
            for (int gi = 0; gi < kRG; ++gi)
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) o[gi][dt] *= alpha[gi];
        }
        // O^T[d][row] += V^T . P^T, k = 32 per MFMA: element e of lane q
        // stands for key 4q + e of tile 2h (e < 4) or tile 2h + 1 (e >= 4),
        // for both operands.  Transposing read: lane r of group q points at
        // 4 dims (4 (r % 4) ..) of key 4q + r / 4 and receives the 4 keys of
        // dim r.
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                u32x4_t vf;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int key = (2 * h2 + hh) * 16 + 4 * q + (r >> 2);
                    const int d = dt * 16 + 4 * (r & 3);
                    const uint16_t* src = &tV[8 * v_piece(key, d >> 3) + (d & 7)];
                    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4_t*)(src));
                    const uint2 u = __builtin_bit_cast(uint2, v);
                    vf[2 * hh] = u.x;
                    vf[2 * hh + 1] = u.y;
                }
#pragma unroll
                for (int gi = 0; gi < kRG; ++gi) {
                    const u32x4_t pp = {pf[gi][2 * h2].x, pf[gi][2 * h2].y, pf[gi][2 * h2 + 1].x,
                                        pf[gi][2 * h2 + 1].y};
                    o[gi][dt] = mfma32(vf, pp, o[gi][dt]);
                }
            }
        }
    };
    load_tile(kb, sK0, sV0);
    for (int t0 = kb; t0 < ke; t0 += 2 * kstep) {
        tile(t0, sK0, sV0, sK1, sV1);
        if (t0 + kstep < ke) tile(t0 + kstep, sK1, sV1, sK0, sV0);
    }
#pragma unroll
    for (int gi = 0; gi < kRG; ++gi) {
        if (!rvalid[gi]) continue;
        const size_t base = ((size_t)item * a.Hkv + g) * 64 + row[gi];
        float* po = a.part_o + base * kD;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
            *(float4*)(po + dt * 16 + 4 * q) = float4{o[gi][dt][0], o[gi][dt][1], o[gi][dt][2], o[gi][dt][3]};
        if (q == 0) {
            a.part_ml[base * 2] = m_run[gi] * a.scale;   // the combine works in natural-log units
            a.part_ml[base * 2 + 1] = l_run[gi];
        }
    }
}

// One workgroup per (block row, 4 q heads): 32 threads per head, four
// output dims each (float4 partial loads), so a batched launch is one
// resident round of workgroups instead of several rounds of one thread per
// dim.  The chunk maxima and sums are staged in LDS (independent loads),
// turned into weights exp(m_c - M), and the partial outputs are summed with
// those weights; chunks are taken kCombItems at a time with a running merge.
constexpr int kCombItems = 1024;
constexpr int kCombHeads = 4;
#ifndef DFLASH_COMB_WIDE_BELOW
#define DFLASH_COMB_WIDE_BELOW 512
#endif
constexpr int kCombWideBelow = DFLASH_COMB_WIDE_BELOW;   // workgroups of the form below under which the wide form runs

__global__ __launch_bounds__(32 * kCombHeads) void k_attn_combine(AttnArgs a) {
    __shared__ float sw[kCombHeads][kCombItems], sl[kCombHeads][kCombItems];
    const int brow = blockIdx.x, t = threadIdx.x, hl = t >> 5, lane = t & 31;
    const int hq = blockIdx.y * kCombHeads + hl;
    const bool act = hq < a.Hq;
    SeqDesc sd = a.seq0;                                         // rows == nullptr: one session
    int pos = sd.F + brow;
    if (a.rows) {
        const RowInfo ri = a.rows[brow];
        sd = a.seqs[ri.seq];
        pos = ri.pos;
    }
    const int G = a.Hq / a.Hkv, hqc = act ? hq : 0, g = hqc / G;
    const int row = (pos - sd.F) * G + hqc % G;
    const size_t stride = (size_t)a.Hkv * 64;                    // between items
    const size_t base0 = ((size_t)sd.item0 * a.Hkv + g) * 64 + row;
    // the output gate's pre-activation (the sum of the projection's K slices),
    // loaded first so that its latency hides under the combine
    float gv = 0.f;
    if (a.gate && act) {
        const float* gs = a.gate_src + (size_t)brow * a.gate_ld + a.gate_col + hq;
        for (int s0 = 0; s0 < a.gate_nsplit; s0 += 8) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = gs[(size_t)min(s0 + j, a.gate_nsplit - 1) * a.gate_stride];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (s0 + j < a.gate_nsplit) gv += v[j];
        }
    }
    float M_run = -INFINITY, L_run = 0.f;
    float4 acc = float4{0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < sd.nitems; c0 += kCombItems) {
        const int nc = min(kCombItems, sd.nitems - c0);
        float mx = -INFINITY;
        if (act)
            for (int c = lane; c < nc; c += 32) {
                const float2 ml = *(const float2*)&a.part_ml[(base0 + (size_t)(c0 + c) * stride) * 2];
                sw[hl][c] = ml.x;
                sl[hl][c] = ml.y;
                mx = fmaxf(mx, ml.x);
            }
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));   // within the head's 32 lanes
        __syncthreads();
        const float M = fmaxf(mx, M_run);
        float lsum = 0.f;
        for (int c = lane; c < nc; c += 32) {
            const float m = sw[hl][c];
            const float w = m == -INFINITY ? 0.f : __expf(m - M);
            sw[hl][c] = w;
            lsum += w * sl[hl][c];
        }
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o);
        __syncthreads();
        const float sc = M_run == -INFINITY ? 0.f : __expf(M_run - M);
        float4 part = float4{0.f, 0.f, 0.f, 0.f};
        if (act) {
            const float* po = a.part_o + (base0 + (size_t)c0 * stride) * kD + 4 * lane;
#pragma unroll 8
            for (int c = 0; c < nc; ++c) {
                const float w = sw[hl][c];
                const float4 v = *(const float4*)(po + (size_t)c * stride * kD);
                part.x += w * v.x;
                part.y += w * v.y;
                part.z += w * v.z;
                part.w += w * v.w;
            }
        }
        acc.x = acc.x * sc + part.x;
        acc.y = acc.y * sc + part.y;
        acc.z = acc.z * sc + part.z;
        acc.w = acc.w * sc + part.w;
        L_run = L_run * sc + lsum;
        M_run = M;
        __syncthreads();
    }
    if (!act) return;
    float f = 1.f / L_run;
    if (a.gate) f *= 1.f / (1.f + __expf(-gv));
    const size_t o = (size_t)brow * a.Hq * kD + (size_t)hq * kD + 4 * lane;
    if (a.out_bf16) {
        *(uint2*)((uint16_t*)a.out + o) = uint2{pack_bf16(acc.x * f, acc.y * f), pack_bf16(acc.z * f, acc.w * f)};
    } else {
        *(float4*)((float*)a.out + o) = float4{acc.x * f, acc.y * f, acc.z * f, acc.w * f};
    }
}

// The combine for launches with few rows (one session's block): one
// workgroup per (block row, q head), 8 groups of 32 lanes (four dims per
// lane); group j merges items j, j + 8, ... on the fly (all its loads issued
// together), then group 0 merges the 8 groups through LDS.  The form above
// gives such launches only a few dozen workgroups, each walking every item.
constexpr int kCombGroups = 8;

__global__ __launch_bounds__(32 * kCombGroups) void k_attn_combine_w(AttnArgs a) {
    __shared__ float gm[kCombGroups], gl[kCombGroups];
    __shared__ float4 go[kCombGroups][32];
    const int brow = blockIdx.x, hq = blockIdx.y, t = threadIdx.x, grp = t >> 5, lane = t & 31;
    SeqDesc sd = a.seq0;                                         // rows == nullptr: one session
    int pos = sd.F + brow;
    if (a.rows) {
        const RowInfo ri = a.rows[brow];
        sd = a.seqs[ri.seq];
        pos = ri.pos;
    }
    const int G = a.Hq / a.Hkv, g = hq / G;
    const int row = (pos - sd.F) * G + hq % G;
    const size_t stride = (size_t)a.Hkv * 64;                    // between items
    const size_t base0 = ((size_t)sd.item0 * a.Hkv + g) * 64 + row;
    float gv = 0.f;
    if (a.gate && grp == 0) {
        const float* gs = a.gate_src + (size_t)brow * a.gate_ld + a.gate_col + hq;
        for (int sp = 0; sp < a.gate_nsplit; ++sp) gv += gs[(size_t)sp * a.gate_stride];
    }
    float M = -INFINITY, L = 0.f;
    float4 acc = float4{0.f, 0.f, 0.f, 0.f};
    for (int c0 = grp; c0 < sd.nitems; c0 += 4 * kCombGroups) {
        float2 ml[4];
        float4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {                            // the group's next four items, loads first
            const int c = min(c0 + u * kCombGroups, sd.nitems - 1);
            const size_t b = base0 + (size_t)c * stride;
            ml[u] = *(const float2*)&a.part_ml[b * 2];
            v[u] = *(const float4*)(a.part_o + b * kD + 4 * lane);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (c0 + u * kCombGroups >= sd.nitems || ml[u].x == -INFINITY) continue;
            const float mn = fmaxf(M, ml[u].x);
            const float so = M == -INFINITY ? 0.f : __expf(M - mn), sn = __expf(ml[u].x - mn);
            acc = float4{acc.x * so + v[u].x * sn, acc.y * so + v[u].y * sn, acc.z * so + v[u].z * sn,
                         acc.w * so + v[u].w * sn};
            L = L * so + ml[u].y * sn;
            M = mn;
        }
    }
    if (lane == 0) {
        gm[grp] = M;
        gl[grp] = L;
    }
    go[grp][lane] = acc;
    __syncthreads();
    if (grp != 0) return;
    float Mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < kCombGroups; ++j) Mt = fmaxf(Mt, gm[j]);
    float Lt = 0.f;
    float4 out = float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kCombGroups; ++j) {
        if (gm[j] == -INFINITY) continue;
        const float w = __expf(gm[j] - Mt);
        Lt += gl[j] * w;
        const float4 o = go[j][lane];
        out = float4{out.x + o.x * w, out.y + o.y * w, out.z + o.z * w, out.w + o.w * w};
    }
    float f = 1.f / Lt;
    if (a.gate) f *= 1.f / (1.f + __expf(-gv));
    const size_t o = (size_t)brow * a.Hq * kD + (size_t)hq * kD + 4 * lane;
    if (a.out_bf16) {
        *(uint2*)((uint16_t*)a.out + o) = uint2{pack_bf16(out.x * f, out.y * f), pack_bf16(out.z * f, out.w * f)};
    } else {
        *(float4*)((float*)a.out + o) = float4{out.x * f, out.y * f, out.z * f, out.w * f};
    }
}

// fp32: one workgroup (one wave) per (block row, q head); D <= 64.  Keys go
// in tiles of 64, one per lane: the lane's score, the tile's maximum and sum
// by wave reductions (online softmax), then lane d < D accumulates output
// dimension d over the tile's values.  Every per-lane quantity is a scalar.
__global__ __launch_bounds__(64) void k_attn_f32(AttnArgs a) {
    __shared__ float sq[64];
    __shared__ float sp[64];
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
    float m = -INFINITY, l = 0.f, o = 0.f;
    for (int s0 = sd.key_lo; s0 < kend; s0 += 64) {
        const int s = s0 + t;
        float dot = -INFINITY;
        if (s < kend && visible(s, p, kend, a.causal, a.window)) {
            const float* kr = Kc + (size_t)(sd.ring ? s % sd.cap : s) * D;
            dot = 0.f;
            for (int d = 0; d < D; ++d) dot = fmaf(sq[d], kr[d], dot);
            dot *= a.scale;
        }
        float tm = dot;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) tm = fmaxf(tm, __shfl_xor(tm, off));
        const float mn = fmaxf(m, tm);
        if (mn == -INFINITY) continue;                 // nothing visible yet (the same on every lane)
        const float al = m == -INFINITY ? 0.f : expf(m - mn);
        const float pe = dot == -INFINITY ? 0.f : expf(dot - mn);
        float ts = pe;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) ts += __shfl_xor(ts, off);
        l = l * al + ts;
        sp[t] = pe;
        __syncthreads();
        if (t < D) {
            float acc = o * al;
            const int n = min(64, kend - s0);
            for (int j = 0; j < n; ++j) {
                const float pj = sp[j];
                if (pj != 0.f) {
                    const int sj = s0 + j;
                    acc = fmaf(pj, Vc[(size_t)(sd.ring ? sj % sd.cap : sj) * D + t], acc);
                }
            }
            o = acc;
        }
        m = mn;
        __syncthreads();
    }
    if (t >= D) return;
    float out = o / l;
    if (a.gate) {
        float gv = 0.f;
        for (int sp2 = 0; sp2 < a.gate_nsplit; ++sp2)
            gv += a.gate_src[(size_t)sp2 * a.gate_stride + (size_t)brow * a.gate_ld + a.gate_col + hq];
        out *= 1.f / (1.f + expf(-gv));
    }
    ((float*)a.out)[(size_t)brow * a.Hq * D + (size_t)hq * D + t] = out;
}

hipError_t attention(const AttnArgs& a, bool bf16, hipStream_t st, int part) {
    if (a.nrows <= 0) return hipSuccess;
    if (!bf16) {
        if (part == 2) return hipSuccess;
        hipLaunchKernelGGL(k_attn_f32, dim3(a.nrows, a.Hq), dim3(64), 0, st, a);
        return hipGetLastError();
    }
    if (part != 2) {
        hipLaunchKernelGGL(k_attn_partial, dim3(a.total_items * a.Hkv), dim3(kAttnThreads), 0, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || part == 1) return e;
    }
    // few rows (one session's block): the wide form, one workgroup per (row, q head)
    if (a.nrows * ((a.Hq + kCombHeads - 1) / kCombHeads) < kCombWideBelow)
        hipLaunchKernelGGL(k_attn_combine_w, dim3(a.nrows, a.Hq), dim3(32 * kCombGroups), 0, st, a);
    else
        hipLaunchKernelGGL(k_attn_combine, dim3(a.nrows, (a.Hq + kCombHeads - 1) / kCombHeads),
                           dim3(32 * kCombHeads), 0, st, a);
    return hipGetLastError();
}

}  // namespace kern
}  // namespace dflash
