// Decode attention on gfx950: 256-slot chunk partials, merged in chunk order.
//
// Method: TensorFold PR #1183 "cuda gemma4: images on the 12B ...", squashed
// commit bodies (window_rows notes): a head's keys split into 256-key chunks,
// each leaving a partial (max, sum, accumulator), merged in chunk order; at
// head dim 512 a block serves several query heads and a warp a run of keys.
// PR #975 "Gemma 4 12B on the native Metal engine", decode attention commits:
// a KV head's query heads form one 16-row tile so every key and value is read
// once per token; chunks spread over workgroups and leave partials for a merge.
//
// MI355X design.  One wave64 per (stream, KV head, chunk).  The 16 rows of
// the matrix-core tile are the G <= 16 query heads of the KV head (rows past
// G hold zero queries and are never stored).  The wave walks its chunk in
// 16-key tiles with an online softmax:
//   S^T[key][head] = K . Q^T   on v_mfma_f32_16x16x32_bf16; each lane loads
//                               16 contiguous bytes of a K row straight from
//                               HBM (four lanes cover 64 contiguous bytes of
//                               one row per load), Q^T sits in registers;
//   O^T[d][head] += V^T . P^T  on v_mfma_f32_16x16x4_f32 with p in fp32, so
//                               p is never rounded; each lane loads 16 bytes
//                               of a V row (sixteen lanes cover 256 contiguous
//                               bytes), widening bf16 to fp32 in registers.
// With S^T as the score layout, lane l always owns query head l % 16: its row
// maximum, rescale factor and accumulator stay in the lane, and only the four
// lanes of one head (l, l^16, l^32, l^48) exchange maxima and sums.
// Keys that are not attended (outside the window, beyond the row, never
// written, past the cache end) get p = 0 and their V values are replaced by
// zeros before the products, so NaN in such slots cannot reach the output.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int CHUNK = 256;
constexpr int TILE = 16;

// position held by `slot` for a row at position t, and whether it is attended
ATTN_DEV bool slot_attended(int slot, int t, int cap, int ring, int window) {
    if (slot >= cap || t < 0) return false;
    int p;
    if (ring) {
        int d = (t - slot) % cap;
        if (d < 0) d += cap;
        p = t - d;
    } else {
        p = slot;
    }
    if (p < 0 || p > t) return false;
    if (window > 0 && t - p >= window) return false;
    return true;
}

template <int D>
__global__ __launch_bounds__(64)
void decode_partial_kernel(const uint16_t* __restrict__ q,
                           const uint16_t* __restrict__ kc,
                           const uint16_t* __restrict__ vc,
                           const int32_t* __restrict__ pos,
                           float* __restrict__ part_acc,
                           float* __restrict__ part_ml,
                           int Hq, int Hkv, int G, int cap, int nch,
                           int ring, int window, float c) {
    constexpr int QST = D / 32;     // 32-wide reduction steps of Q.K
    constexpr int SPANS = D / 128;  // 128-wide d spans of the accumulator
    const int chunk = blockIdx.x;
    const int g = blockIdx.y;
    const int s = blockIdx.z;
    const int lane = threadIdx.x;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int t = pos[s];

    const size_t head_base = ((size_t)s * Hkv + g) * (size_t)cap;
    const uint16_t* K = kc + head_base * D;
    const uint16_t* V = vc + head_base * D;

    // Q^T operand: lane holds Q[head col][32 st + 8 grp .. +7]
    u32x4 qreg[QST];
    {
        const bool hv = col < G;
        const uint16_t* qrow = q + ((size_t)s * Hq + (size_t)g * G + (hv ? col : 0)) * D;
#pragma unroll
        for (int st = 0; st < QST; ++st) {
            u32x4 z = {0u, 0u, 0u, 0u};
            qreg[st] = hv ? ld16(qrow + 32 * st + 8 * grp) : z;
        }
    }

    f32x4 acc[SPANS][8];
#pragma unroll
    for (int sp = 0; sp < SPANS; ++sp)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[sp][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    float m_run = -INFINITY;
    float l_run = 0.f;
    const int slot0 = chunk * CHUNK;

    for (int tt = 0; tt < CHUNK / TILE; ++tt) {
        const int sb = slot0 + tt * TILE;
        // attended keys of this tile: lane's K row (sb + col) and its four
        // score keys (sb + 4 grp + i)
        const bool krow_ok = slot_attended(sb + col, t, cap, ring, window);
        if (!__any(krow_ok)) continue;   // uniform: nothing attended here

        u32x4 kreg[QST];
        const uint16_t* krow = K + (size_t)(sb + col) * D + 8 * grp;
#pragma unroll
        for (int st = 0; st < QST; ++st) {
            u32x4 z = {0u, 0u, 0u, 0u};
            kreg[st] = krow_ok ? ld16(krow + 32 * st) : z;
        }
        // V rows (sb + 4 grp + r), d = 128 sp + 8 col .. +7
        bool vok[4];
        u32x4 vreg[4][SPANS];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            vok[r] = slot_attended(sb + 4 * grp + r, t, cap, ring, window);
            const uint16_t* vrow = V + (size_t)(sb + 4 * grp + r) * D + 8 * col;
#pragma unroll
            for (int sp = 0; sp < SPANS; ++sp) {
                u32x4 z = {0u, 0u, 0u, 0u};
                vreg[r][sp] = vok[r] ? ld16(vrow + 128 * sp) : z;
            }
        }

        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < QST; ++st) sc = mfma_bf16_16x16x32(kreg[st], qreg[st], sc);

        float tv[4];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            tv[i] = vok[i] ? sc[i] * c : -INFINITY;
            mx = fmaxf(mx, tv[i]);
        }
        mx = xmax4(mx);
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - m_new);   // 0 when m_run = -inf
        float pv[4];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pv[i] = vok[i] ? fast_exp2(tv[i] - m_new) : 0.f;
            psum += pv[i];
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        if (__any(alpha != 1.f)) {
#pragma unroll
            for (int sp = 0; sp < SPANS; ++sp)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[sp][j] *= alpha;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int sp = 0; sp < SPANS; ++sp) {
                const u32x4 w = vreg[r][sp];
                acc[sp][0] = mfma_f32_16x16x4(bf16lo_to_f32(w.x), pv[r], acc[sp][0]);
                acc[sp][1] = mfma_f32_16x16x4(bf16hi_to_f32(w.x), pv[r], acc[sp][1]);
                acc[sp][2] = mfma_f32_16x16x4(bf16lo_to_f32(w.y), pv[r], acc[sp][2]);
                acc[sp][3] = mfma_f32_16x16x4(bf16hi_to_f32(w.y), pv[r], acc[sp][3]);
                acc[sp][4] = mfma_f32_16x16x4(bf16lo_to_f32(w.z), pv[r], acc[sp][4]);
                acc[sp][5] = mfma_f32_16x16x4(bf16hi_to_f32(w.z), pv[r], acc[sp][5]);
                acc[sp][6] = mfma_f32_16x16x4(bf16lo_to_f32(w.w), pv[r], acc[sp][6]);
                acc[sp][7] = mfma_f32_16x16x4(bf16hi_to_f32(w.w), pv[r], acc[sp][7]);
            }
        }
    }

    const float l_tot = xsum4(l_run);
    if (col >= G) return;
    const int h = g * G + col;
    const size_t pidx = ((size_t)s * Hq + h) * (size_t)nch + chunk;
    if (grp == 0) {
        part_ml[2 * pidx + 0] = m_run;
        part_ml[2 * pidx + 1] = l_tot;
    }
    float* dst = part_acc + pidx * D;
    // lane holds d = 128 sp + 32 grp + 8 i + j in acc[sp][j][i]
#pragma unroll
    for (int sp = 0; sp < SPANS; ++sp) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float* p = dst + 128 * sp + 32 * grp + 8 * i;
            f32x4 lo = {acc[sp][0][i], acc[sp][1][i], acc[sp][2][i], acc[sp][3][i]};
            f32x4 hi = {acc[sp][4][i], acc[sp][5][i], acc[sp][6][i], acc[sp][7][i]};
            *reinterpret_cast<f32x4*>(p) = lo;
            *reinterpret_cast<f32x4*>(p + 4) = hi;
        }
    }
}

// Merge of chunk partials in ascending chunk order: M = max over live chunks,
// out = bf16(sum e^(m_c - M) acc_c / sum e^(m_c - M) l_c).  A chunk with no
// attended key (m = -inf) is skipped, never multiplied.  Block: 64 threads,
// four consecutive d each (256 d); grid (Hq, S, D / 256).
template <int D>
__global__ __launch_bounds__(64)
void decode_merge_kernel(uint16_t* __restrict__ out,
                         const float* __restrict__ part_acc,
                         const float* __restrict__ part_ml,
                         int Hq, int nch) {
    const int h = blockIdx.x;
    const int s = blockIdx.y;
    const int d0 = blockIdx.z * 256 + threadIdx.x * 4;
    const size_t base = ((size_t)s * Hq + h) * (size_t)nch;
    const float2* ml = reinterpret_cast<const float2*>(part_ml) + base;

    float M = -INFINITY;
    for (int cidx = 0; cidx < nch; ++cidx) M = fmaxf(M, ml[cidx].x);

    float L = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
        for (int cidx = 0; cidx < nch; ++cidx) {
            const float2 e = ml[cidx];
            if (e.x == -INFINITY) continue;
            const float w = fast_exp2(e.x - M);
            L += w * e.y;
            const f32x4 a = *reinterpret_cast<const f32x4*>(part_acc + (base + cidx) * D + d0);
            o += w * a;
        }
    }
    uint32_t b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = (L != 0.f || L != L) ? f32_to_bf16_bits(o[i] / L) : 0u;
    u32x2 packed = {pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
    *reinterpret_cast<u32x2*>(out + ((size_t)s * Hq + h) * D + d0) = packed;
}

}  // namespace

size_t decode_workspace_bytes(int S, int Hq, int D, int cap) {
    const size_t nch = ((size_t)cap + CHUNK - 1) / CHUNK;
    return (size_t)S * Hq * nch * ((size_t)D + 2) * sizeof(float);
}

hipError_t launch_decode(uint16_t* out, const uint16_t* q, const uint16_t* kc,
                         const uint16_t* vc, const int32_t* pos, int S, int Hq,
                         int Hkv, int D, int cap, int ring, int window,
                         float scale, void* ws, hipStream_t stream) {
    const int nch = (cap + CHUNK - 1) / CHUNK;
    const int G = Hq / Hkv;
    float* part_acc = reinterpret_cast<float*>(ws);
    float* part_ml = part_acc + (size_t)S * Hq * nch * D;
    const float c = scale * ATTN_LOG2E;
    dim3 g1(nch, Hkv, S);
    dim3 g2(Hq, S, D / 256);
    if (D == 256) {
        decode_partial_kernel<256><<<g1, 64, 0, stream>>>(q, kc, vc, pos, part_acc, part_ml,
                                                          Hq, Hkv, G, cap, nch, ring, window, c);
        decode_merge_kernel<256><<<g2, 64, 0, stream>>>(out, part_acc, part_ml, Hq, nch);
    } else {
        decode_partial_kernel<512><<<g1, 64, 0, stream>>>(q, kc, vc, pos, part_acc, part_ml,
                                                          Hq, Hkv, G, cap, nch, ring, window, c);
        decode_merge_kernel<512><<<g2, 64, 0, stream>>>(out, part_acc, part_ml, Hq, nch);
    }
    return hipGetLastError();
}
