// Prompt (prefill) attention on gfx950 for one stream's chunk of rows.
//
// Method: TensorFold PR #975 "Gemma 4 12B on the native Metal engine", prompt
// attention commits: 16 query rows of a head per tile, causal and sliding-
// window masks, an online softmax whose row maxima and probabilities are
// settled once per key block, value reads that stop at the last written key;
// the key/value cache is written before attention and read from it.  PR #1183
// "cuda gemma4: images on the 12B ...", window_rows notes: prompt tiles score
// over 128-dim slices (the score accumulates 32-wide steps in ascending d, so
// 128-wide slices add in slice order) and P may be kept as two bf16 halves.
//
// MI355X design (v1).  A workgroup of four waves takes one 16-row tile of the
// chunk and four query heads of one KV group; wave w owns head w: 16 rows x
// the whole head dim, so its softmax state never leaves the wave.  The four
// heads share every K/V block, staged once in LDS and double-buffered: while
// the waves multiply block b, the next block's 16-byte global loads are in
// flight in registers and land in the other LDS stage after the products.
//   S^T[key][row] = K . Q^T  v_mfma_f32_16x16x32_bf16, K rows from LDS,
//                            Q^T resident in registers for the whole walk;
//   O^T[d][row] += V^T . P^T v_mfma_f32_16x16x32_bf16 with P (or its bf16 hi
//                            and lo halves, two products) as the B operand;
//                            V is written to LDS transposed, in a key order
//                            that matches the lanes' P registers, so each A
//                            operand is one 16-byte LDS read.
// Lane l always owns query row l % 16 (the S^T and O^T column), so the row's
// maximum, rescale and sum stay in its four lanes (l, l^16, l^32, l^48).
// Key blocks are KB keys aligned to absolute positions; the running maximum
// moves once per block and p is rounded against it.  Keys of a block outside
// the tile's attended span [lo, hi] are stored as zeros, never loaded.
#include "common.h"
#include "kernels.h"

namespace {

template <int D> struct PrefillCfg;
template <> struct PrefillCfg<256> { static constexpr int KB = 64; };
template <> struct PrefillCfg<512> { static constexpr int KB = 32; };

template <int D, int PM>
__global__ __launch_bounds__(256)
void prefill_kernel(uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
                    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
                    int pos0, int n_rows, int Hq, int Hkv, int G, int HG, int cap,
                    int ring, int window, float c) {
    constexpr int KB = PrefillCfg<D>::KB;
    constexpr int KP = D + 8;                // K row stride in LDS (elements)
    constexpr int VP = KB + 8;               // V^T row stride in LDS
    constexpr int K_ELEMS = KB * KP;
    constexpr int STAGE = K_ELEMS + D * VP;
    constexpr int QST = D / 32;              // reduction steps of a score
    constexpr int KT = KB / 16;              // 16-key score tiles per block
    constexpr int KS = KB / 32;              // 32-key steps of P.V per block
    constexpr int DT = D / 16;               // 16-wide d tiles of the output
    constexpr int VEC_ROW = D / 8;           // 16-byte vectors per cache row
    constexpr int K_VECS = KB * VEC_ROW / 256;       // per thread
    constexpr int V_UNITS = (KB / 4) * VEC_ROW / 256; // 4-key units per thread
    static_assert(K_VECS * 256 == KB * VEC_ROW, "K staging");
    static_assert(V_UNITS * 256 == (KB / 4) * VEC_ROW, "V staging");

    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int col = lane & 15;
    const int grp = lane >> 4;

    const int r0 = blockIdx.x * 16;
    const int g = blockIdx.y / HG;
    const int hl = (blockIdx.y % HG) * 4 + wave;
    const bool head_ok = hl < G;
    const int h = g * G + (head_ok ? hl : 0);
    const int nvalid = min(16, n_rows - r0);
    const int t_first = pos0 + r0;
    const int t_last = pos0 + r0 + nvalid - 1;
    const int lo_tile = window > 0 ? max(0, t_first - window + 1) : 0;
    const int hi_tile = t_last;
    const int b_lo = lo_tile / KB;
    const int b_hi = hi_tile / KB;

    const bool row_ok = col < nvalid;
    const int t_row = pos0 + r0 + col;
    const int lo_row = window > 0 ? max(0, t_row - window + 1) : 0;

    // Q^T operand: lane holds Q[row col][head h][32 st + 8 grp .. +7]
    u32x4 qreg[QST];
    {
        const uint16_t* qrow = q + ((size_t)(r0 + (row_ok ? col : 0)) * Hq + h) * D + 8 * grp;
#pragma unroll
        for (int st = 0; st < QST; ++st) {
            u32x4 z = {0u, 0u, 0u, 0u};
            qreg[st] = (row_ok && head_ok) ? ld16(qrow + 32 * st) : z;
        }
    }

    const uint16_t* Kg = kc + (size_t)g * cap * D;
    const uint16_t* Vg = vc + (size_t)g * cap * D;

    u32x4 kst[K_VECS];
    u32x4 vst[V_UNITS][4];

    auto slot_of = [&](int p) -> size_t { return (size_t)(ring ? p % cap : p); };

    auto gload = [&](int b) {
        const int p0 = b * KB;
#pragma unroll
        for (int it = 0; it < K_VECS; ++it) {
            const int vi = tid + 256 * it;
            const int key = vi / VEC_ROW;
            const int dv = vi % VEC_ROW;
            const int p = p0 + key;
            u32x4 z = {0u, 0u, 0u, 0u};
            kst[it] = (p >= lo_tile && p <= hi_tile) ? ld16(Kg + slot_of(p) * D + dv * 8) : z;
        }
#pragma unroll
        for (int u = 0; u < V_UNITS; ++u) {
            const int ui = tid + 256 * u;
            const int k4 = ui % (KB / 4);
            const int dv = ui / (KB / 4);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int p = p0 + 4 * k4 + kk;
                u32x4 z = {0u, 0u, 0u, 0u};
                vst[u][kk] = (p >= lo_tile && p <= hi_tile) ? ld16(Vg + slot_of(p) * D + dv * 8) : z;
            }
        }
    };

    auto lstore = [&](int stg) {
        uint16_t* Kl = lds + stg * STAGE;
        uint16_t* Vl = Kl + K_ELEMS;
#pragma unroll
        for (int it = 0; it < K_VECS; ++it) {
            const int vi = tid + 256 * it;
            st16(Kl + (vi / VEC_ROW) * KP + (vi % VEC_ROW) * 8, kst[it]);
        }
#pragma unroll
        for (int u = 0; u < V_UNITS; ++u) {
            const int ui = tid + 256 * u;
            const int k4 = ui % (KB / 4);
            const int dv = ui / (KB / 4);
            // keys 4 k4 .. +3 of the 32-key group k4 / 8 go to the columns
            // where the P.V step expects them: lane group g' reads columns
            // 8 g' .. 8 g' + 7 = keys 4 g' .. +3 and 16 + 4 g' .. +3
            const int k4l = k4 & 7;
            const int cst = 32 * (k4 >> 3) + (k4l < 4 ? 8 * k4l : 8 * (k4l - 4) + 4);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int w = j >> 1;
                const int sh = (j & 1) * 16;
                const uint32_t e0 = (vst[u][0][w] >> sh) & 0xFFFFu;
                const uint32_t e1 = (vst[u][1][w] >> sh) & 0xFFFFu;
                const uint32_t e2 = (vst[u][2][w] >> sh) & 0xFFFFu;
                const uint32_t e3 = (vst[u][3][w] >> sh) & 0xFFFFu;
                u32x2 pk = {e0 | (e1 << 16), e2 | (e3 << 16)};
                *reinterpret_cast<u32x2*>(Vl + (dv * 8 + j) * VP + cst) = pk;
            }
        }
    };

    f32x4 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;
    float l_run = 0.f;

    gload(b_lo);
    lstore(0);
    __syncthreads();

    for (int b = b_lo; b <= b_hi; ++b) {
        const int stg = (b - b_lo) & 1;
        const bool more = b < b_hi;
        if (more) gload(b + 1);
        if (head_ok) {
            const uint16_t* Kl = lds + stg * STAGE;
            const uint16_t* Vl = Kl + K_ELEMS;
            const int p0 = b * KB;
            // scores: tile kt holds keys 16 kt + (0..15) in natural order;
            // lane has keys 16 kt + 4 grp + i for its row
            float sv[KT][4];
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                f32x4 a = {0.f, 0.f, 0.f, 0.f};
                const uint16_t* krow = Kl + (16 * kt + col) * KP + 8 * grp;
#pragma unroll
                for (int st = 0; st < QST; ++st) a = mfma_bf16_16x16x32(ld16(krow + 32 * st), qreg[st], a);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int p = p0 + 16 * kt + 4 * grp + i;
                    const bool ok = row_ok && p <= t_row && p >= lo_row;
                    sv[kt][i] = ok ? a[i] * c : -INFINITY;
                }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sv[kt][i]);
            mx = xmax4(mx);
            const float m_new = fmaxf(m_run, mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_use);
            float psum = 0.f;
            u32x4 phi[KS];
            u32x4 plo[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                uint32_t hb[8], lb[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int kt = 2 * ks + (e >> 2);
                    const float p = fast_exp2(sv[kt][e & 3] - m_use);
                    psum += p;
                    hb[e] = f32_to_bf16_bits(p);
                    if (PM == ATTN_P_BF16X2) lb[e] = f32_to_bf16_bits(p - __uint_as_float(hb[e] << 16));
                }
                phi[ks] = u32x4{pack_bf16x2(hb[0], hb[1]), pack_bf16x2(hb[2], hb[3]),
                                pack_bf16x2(hb[4], hb[5]), pack_bf16x2(hb[6], hb[7])};
                if (PM == ATTN_P_BF16X2)
                    plo[ks] = u32x4{pack_bf16x2(lb[0], lb[1]), pack_bf16x2(lb[2], lb[3]),
                                    pack_bf16x2(lb[4], lb[5]), pack_bf16x2(lb[6], lb[7])};
            }
            l_run = l_run * alpha + psum;
            m_run = m_new;
            if (__any(alpha != 1.f)) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const u32x4 a = ld16(Vl + (16 * dt + col) * VP + 32 * ks + 8 * grp);
                    oacc[dt] = mfma_bf16_16x16x32(a, phi[ks], oacc[dt]);
                    if (PM == ATTN_P_BF16X2) oacc[dt] = mfma_bf16_16x16x32(a, plo[ks], oacc[dt]);
                }
            }
        }
        if (more) lstore(stg ^ 1);
        __syncthreads();
    }

    const float l_tot = xsum4(l_run);
    if (!(row_ok && head_ok)) return;
    uint16_t* orow = out + ((size_t)(r0 + col) * Hq + h) * D + 4 * grp;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        uint32_t b0 = f32_to_bf16_bits(oacc[dt][0] / l_tot);
        uint32_t b1 = f32_to_bf16_bits(oacc[dt][1] / l_tot);
        uint32_t b2 = f32_to_bf16_bits(oacc[dt][2] / l_tot);
        uint32_t b3 = f32_to_bf16_bits(oacc[dt][3] / l_tot);
        u32x2 pk = {pack_bf16x2(b0, b1), pack_bf16x2(b2, b3)};
        *reinterpret_cast<u32x2*>(orow + 16 * dt) = pk;
    }
}

}  // namespace

int prefill_key_block(int D, int p_mode) {
    (void)p_mode;
    return D == 256 ? PrefillCfg<256>::KB : PrefillCfg<512>::KB;
}

hipError_t launch_prefill(uint16_t* out, const uint16_t* q, const uint16_t* kc,
                          const uint16_t* vc, int pos0, int n_rows, int Hq,
                          int Hkv, int D, int cap, int ring, int window,
                          float scale, int p_mode, hipStream_t stream) {
    const int G = Hq / Hkv;
    const int HG = (G + 3) / 4;
    const float c = scale * ATTN_LOG2E;
    dim3 grid((n_rows + 15) / 16, Hkv * HG);
#define PREFILL_LAUNCH(DD, PMV)                                                        \
    prefill_kernel<DD, PMV><<<grid, 256, 0, stream>>>(out, q, kc, vc, pos0, n_rows, Hq, \
                                                      Hkv, G, HG, cap, ring, window, c)
    if (D == 256) {
        if (p_mode == ATTN_P_BF16X2) PREFILL_LAUNCH(256, ATTN_P_BF16X2);
        else PREFILL_LAUNCH(256, ATTN_P_BF16);
    } else {
        if (p_mode == ATTN_P_BF16X2) PREFILL_LAUNCH(512, ATTN_P_BF16X2);
        else PREFILL_LAUNCH(512, ATTN_P_BF16);
    }
#undef PREFILL_LAUNCH
    return hipGetLastError();
}
