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
// MI355X design.  A workgroup of four waves takes one 16-row tile of the
// chunk and four query heads of one KV group; wave w owns head w: 16 rows x
// the whole head dim, so its softmax state never leaves the wave.  The four
// heads share every key block: K and V rows land in LDS by direct
// global->LDS loads (1 KiB of whole rows per instruction, no registers, no
// VALU), two stages, the next block in flight while the current one is
// multiplied.  Rows are padded in LDS (K by 16 bytes, V by 32) so that the
// score reads (eight rows, one 16-byte chunk each) and the transpose reads
// (four rows, 32 bytes each) fall on distinct banks, and every LDS address
// is a per-lane base plus a constant offset.  At head dim 256 one DMA
// instruction moves two 512-byte rows back to back; it takes rows r and
// r + 8 of a 16-row group, which no read phase uses together, and the
// padding sits between such pairs.
//   S^T[key][row] = K . Q^T   v_mfma_f32_16x16x32_bf16: K rows from LDS,
//                             Q^T resident in registers for the whole walk;
//   O^T[d][row] += V^T . P^T  v_mfma_f32_16x16x32_bf16 with P (or its bf16
//                             hi and lo halves, two products) as B; the V^T
//                             operand comes straight from the row-major V
//                             block through two transpose reads.
// Lane l always owns query row l % 16 (the S^T and O^T column), so the row's
// maximum, rescale and sum stay in its four lanes (l, l^16, l^32, l^48).
// Key blocks are KB keys aligned to absolute positions; the running maximum
// moves once per block and p is rounded against it.  Key slots of a block
// outside the tile's attended span [lo, hi] are fetched from a position
// inside the span instead: their scores are masked, and their V rows are
// finite, so they add exactly zero (a never-written row is never read).
#include "common.h"
#include "kernels.h"

namespace {

template <int D> struct PrefillCfg;
template <> struct PrefillCfg<256> { static constexpr int KB = 64; };
template <> struct PrefillCfg<512> { static constexpr int KB = 32; };

// element offset of block row r in LDS (PADP: padding elements per unit)
template <int D, int PADP>
ATTN_DEV constexpr int row_pos(int r) {
    if constexpr (D == 512) {
        return r * (D + PADP);
    } else {
        return ((r >> 4) * 8 + (r & 7)) * (2 * D + PADP) + ((r >> 3) & 1) * D;
    }
}

template <int D, int PM>
__global__ __launch_bounds__(256)
void prefill_kernel(uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
                    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
                    int pos0, int n_rows, int Hq, int Hkv, int G, int HG, int cap,
                    int ring, int window, float c) {
    constexpr int KB = PrefillCfg<D>::KB;
    constexpr int KPADP = 8;                 // K padding per row (pair at 256)
    constexpr int VPADP = 16;                // V padding per row (pair at 256)
    constexpr int KBLK = row_pos<D, KPADP>(KB);
    constexpr int VBLK = row_pos<D, VPADP>(KB);
    constexpr int QST = D / 32;              // reduction steps of a score
    constexpr int KT = KB / 16;              // 16-key score tiles per block
    constexpr int KS = KB / 32;              // 32-key steps of P.V per block
    constexpr int DT = D / 16;               // 16-wide d tiles of the output
    constexpr int LPR = D / 8;               // lanes that move one row
    constexpr int INSTR = KB * LPR / 64;     // DMA instructions per K (or V) block
    constexpr int IPW = INSTR / 4;           // ... per wave
    static_assert(IPW * 4 == INSTR, "DMA split");
    constexpr int K16 = row_pos<D, KPADP>(16);     // offset of the next 16 rows
    constexpr int V16 = row_pos<D, VPADP>(16);

    // two K stages and two V stages: K runs one block ahead of V
    __shared__ __attribute__((aligned(16))) uint16_t ks_lds[2][KBLK];
    __shared__ __attribute__((aligned(16))) uint16_t vs_lds[2][VBLK];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lane = tid & 63;
    const int col = lane & 15;
    const int grp = lane >> 4;

    // XCD-aware tile order: the hardware deals workgroup L to XCD L % 8, so
    // L is renumbered to put each XCD on a contiguous range of tiles ordered
    // KV group, head group, row tile: the workgroups sharing one L2 then
    // stream the same K/V blocks at about the same time
    const int n_rt = (n_rows + 15) / 16;
    const int nwg = n_rt * Hkv * HG;
    const int L = blockIdx.x;
    const int lam = (nwg % 8 == 0) ? (L % 8) * (nwg / 8) + L / 8 : L;
    const int rt = lam % n_rt;
    const int gh = lam / n_rt;                       // g * HG + head group
    const int r0 = rt * 16;
    const int g = gh / HG;
    const int hl = (gh % HG) * 4 + wave;
    const bool head_ok = hl < G;
    const int h = g * G + (head_ok ? hl : 0);
    const int nvalid = min(16, n_rows - r0);
    const int t_first = pos0 + r0;
    const int t_last = pos0 + r0 + nvalid - 1;
    const int lo_tile = window > 0 ? max(0, t_first - window + 1) : 0;
    const int lo_last = window > 0 ? max(0, t_last - window + 1) : 0;
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

    // DMA of one K or V block: instruction j (wave w issues [w IPW, (w+1) IPW))
    // moves 1 KiB: block row j at D=512, rows 16 (j >> 3) + (j & 7) and +8 at
    // D=256 (lanes 0..31 and 32..63).  A block whose KB positions all lie in
    // the tile's span and do not wrap the ring takes a uniform row base plus
    // per-lane constant offsets; other blocks clamp each position into the span.
    int lane_row[IPW];          // block row this lane moves in instruction i
    int lane_dst[IPW];          // LDS row base (elements) of instruction i, for K
    int lane_dstv[IPW];         // ... for V
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int j = wave * IPW + i;
        const int r0i = (LPR == 64) ? j : 16 * (j >> 3) + (j & 7);
        lane_row[i] = (LPR == 64) ? j : r0i + 8 * (lane >> 5);
        lane_dst[i] = row_pos<D, KPADP>(r0i);
        lane_dstv[i] = row_pos<D, VPADP>(r0i);
    }
    const int lane_col = (lane % LPR) * 8;
    auto dma = [&](const uint16_t* base, uint16_t* stage, const int* dsts, int b) {
        const int p0 = b * KB;
        const int s0 = ring ? p0 % cap : p0;
        if (p0 >= lo_tile && p0 + KB - 1 <= hi_tile && s0 + KB <= cap) {
            const uint16_t* src = base + (size_t)s0 * D + lane_col;
#pragma unroll
            for (int i = 0; i < IPW; ++i)
                ATTN_DMA16(src + lane_row[i] * D, stage + dsts[i]);
        } else {
#pragma unroll
            for (int i = 0; i < IPW; ++i) {
                const int p = min(max(p0 + lane_row[i], lo_tile), hi_tile);
                const int slot = ring ? p % cap : p;
                ATTN_DMA16(base + (size_t)slot * D + lane_col, stage + dsts[i]);
            }
        }
    };

    f32x4 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;
    float l_run = 0.f;

    const int kofs = row_pos<D, KPADP>(col) + 8 * grp;
    const int vofs = row_pos<D, VPADP>(4 * grp + (col >> 2)) + 4 * (col & 3);

    // scores of block b from K stage kl; then the block's softmax: P of the
    // block in phi / plo, the row sum, and the accumulator rescale
    u32x4 phi[KS], plo[KS];
    auto scores_softmax = [&](int b, const uint16_t* kl) {
        const int p0 = b * KB;
        const bool interior = p0 >= lo_last && p0 + KB - 1 <= t_first;
        float sv[KT][4];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            // K operands run PF reads ahead of the products that use them
            constexpr int PF = 4;
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
            u32x4 kb[PF];
#pragma unroll
            for (int st = 0; st < PF; ++st) kb[st] = ld16(kl + kofs + kt * K16 + 32 * st);
#pragma unroll
            for (int st = 0; st < QST; ++st) {
                a = mfma_bf16_16x16x32(kb[st % PF], qreg[st], a);
                if (st + PF < QST) kb[st % PF] = ld16(kl + kofs + kt * K16 + 32 * (st + PF));
            }
            if (interior) {
#pragma unroll
                for (int i = 0; i < 4; ++i) sv[kt][i] = a[i] * c;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int p = p0 + 16 * kt + 4 * grp + i;
                    const bool ok = row_ok && p <= t_row && p >= lo_row;
                    sv[kt][i] = ok ? a[i] * c : -INFINITY;
                }
            }
        }
        float mx = sv[0][0];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sv[kt][i]);
        mx = xmax4(mx);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float psum = 0.f;
        // P.V step ks: lane's k-slots (grp, e) are keys 32 ks + 4 grp + e
        // (e < 4) and 32 ks + 16 + 4 grp + (e - 4), from tiles 2 ks, 2 ks + 1
#pragma unroll
        for (int k2 = 0; k2 < KS; ++k2) {
            float pe[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pe[e] = fast_exp2(sv[2 * k2 + (e >> 2)][e & 3] - m_use);
                psum += pe[e];
            }
            uint32_t hw[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) hw[u] = cvt_pk_bf16(pe[2 * u], pe[2 * u + 1]);
            phi[k2] = u32x4{hw[0], hw[1], hw[2], hw[3]};
            if (PM == ATTN_P_BF16X2) {
                uint32_t lw[4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    lw[u] = cvt_pk_bf16(pe[2 * u] - bf16lo_to_f32(hw[u]),
                                        pe[2 * u + 1] - bf16hi_to_f32(hw[u]));
                plo[k2] = u32x4{lw[0], lw[1], lw[2], lw[3]};
            }
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        if (__any(alpha != 1.f)) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
        }
    };

    // O^T += V^T P^T for the block in V stage vl with the P in phi / plo.
    // V^T operand by transpose reads: lane j of a 16-lane group points at V
    // row (key of k-slot j >> 2), columns 16 dt + 4 (j & 3) .. +3
    auto pv = [&](const uint16_t* vl) {
#pragma unroll
        for (int k2 = 0; k2 < KS; ++k2) {
            // V^T operands run PF d-tiles ahead of the products that use them
            constexpr int PF = 4;
            u32x4 vb[PF];
            auto rd = [&](int dt) -> u32x4 {
                const u32x2 x0 = lds_read_tr16(vl + vofs + 2 * k2 * V16 + 16 * dt);
                const u32x2 x1 = lds_read_tr16(vl + vofs + (2 * k2 + 1) * V16 + 16 * dt);
                return u32x4{x0.x, x0.y, x1.x, x1.y};
            };
#pragma unroll
            for (int dt = 0; dt < PF; ++dt) vb[dt] = rd(dt);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const u32x4 a = vb[dt % PF];
                if (dt + PF < DT) vb[dt % PF] = rd(dt + PF);
                oacc[dt] = mfma_bf16_16x16x32(a, phi[k2], oacc[dt]);
                if (PM == ATTN_P_BF16X2) oacc[dt] = mfma_bf16_16x16x32(a, plo[k2], oacc[dt]);
            }
        }
    };

    // prologue: K(b_lo), V(b_lo) and K(b_lo + 1) in flight; scores of b_lo
    dma(Kg, ks_lds[0], lane_dst, b_lo);
    dma(Vg, vs_lds[0], lane_dstv, b_lo);
    if (b_lo < b_hi) dma(Kg, ks_lds[1], lane_dst, b_lo + 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (head_ok) scores_softmax(b_lo, ks_lds[0]);
    __syncthreads();                             // K(b_lo) read by every wave

    for (int b = b_lo; b <= b_hi; ++b) {
        const int st = (b - b_lo) & 1;
        // in LDS now: V(b) in vs[st], K(b + 1) in ks[st ^ 1]; P(b) in registers
        if (b + 2 <= b_hi) dma(Kg, ks_lds[st], lane_dst, b + 2);
        if (b + 1 <= b_hi) dma(Vg, vs_lds[st ^ 1], lane_dstv, b + 1);
        if (head_ok) {
            pv(vs_lds[st]);
            if (b < b_hi) scores_softmax(b + 1, ks_lds[st ^ 1]);
        }
        __builtin_amdgcn_s_waitcnt(0);          // this wave's DMAs of K(b+2), V(b+1)
        __syncthreads();                         // everyone's; K(b+1), V(b) free
    }

    const float l_tot = xsum4(l_run);
    if (!(row_ok && head_ok)) return;
    uint16_t* orow = out + ((size_t)(r0 + col) * Hq + h) * D + 4 * grp;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        u32x2 pk = {cvt_pk_bf16(oacc[dt][0] / l_tot, oacc[dt][1] / l_tot),
                    cvt_pk_bf16(oacc[dt][2] / l_tot, oacc[dt][3] / l_tot)};
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
    dim3 grid(((n_rows + 15) / 16) * Hkv * HG);
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
