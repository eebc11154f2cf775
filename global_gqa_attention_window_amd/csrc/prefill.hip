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
// multiplied.  Rows are padded in LDS by 32 bytes so that the score reads
// (sixteen rows, one 16-byte chunk each) and the transpose reads (four rows,
// 32 bytes each) fall on distinct banks, and every LDS address is a per-lane
// base plus a constant offset.  At head dim 256 one DMA instruction moves two
// 512-byte rows back to back; it takes rows r and r + 8 of a 16-row group,
// and the padding sits between such pairs.
//   S^T[key][row] = K . Q^T   v_mfma_f32_16x16x32_bf16: K rows from LDS,
//                             Q^T resident in AGPRs for the whole walk;
//   O^T[d][row] += V^T . P^T  v_mfma_f32_16x16x32_bf16 with P (or its bf16
//                             hi and lo halves, two products) as B; the V^T
//                             operand comes straight from the row-major V
//                             block through two transpose reads.
// One wave runs per SIMD, so the wave itself must keep its matrix unit fed:
// an iteration issues the scores of block b + 1 (K operands eight products
// ahead, with the accumulator rescale that block b needs in the VALU slots
// beside them), then block b's P.V with block b + 1's mask and softmax cut
// into slices between its products.  Both phases are fenced step by step so
// the compiler keeps that order.
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
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_kernel(uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
                    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
                    int pos0, int n_rows, int Hq, int Hkv, int G, int HG, int cap,
                    int ring, int window, float c) {
    constexpr int KB = PrefillCfg<D>::KB;
    constexpr int KPADP = 16;                // K padding per row (pair at 256)
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
            // Q lives in AGPRs (the products read their B operand from
            // there), which leaves the VGPRs to the accumulators and to the
            // operand reads in flight
            asm volatile("" : "+a"(qreg[st]));
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
        const uint32_t lds0 = lds_addr(stage);
        if (p0 >= lo_tile && p0 + KB - 1 <= hi_tile && s0 + KB <= cap) {
            const uint16_t* src = base + (size_t)s0 * D + lane_col;
#pragma unroll
            for (int i = 0; i < IPW; ++i)
                dma16_asm(src + lane_row[i] * D, lds0 + 2 * dsts[i]);
        } else {
#pragma unroll
            for (int i = 0; i < IPW; ++i) {
                const int p = min(max(p0 + lane_row[i], lo_tile), hi_tile);
                const int slot = ring ? p % cap : p;
                dma16_asm(base + (size_t)slot * D + lane_col, lds0 + 2 * dsts[i]);
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

    constexpr int NS = KT * QST;                 // score products per block
    constexpr int KPF = 8;                       // K operand reads in flight
    constexpr int NPV = KS * DT;                 // V^T operands per block
    constexpr int VPF = 4;                       // V^T operands in flight
    constexpr int NE = 8 * KS;                   // probabilities per lane per block
    static_assert(KPF == 2 * VPF, "the V^T reads fill the last KPF score steps");

    // K operand of score product j: tile j % KT, reduction step j / KT
    auto rd_k = [&](const uint16_t* kl, int j) {
        return ld16(kl + kofs + (j % KT) * K16 + 32 * (j / KT));
    };
    // V^T operand i (P.V step i / DT, d tile i % DT) by two transpose reads:
    // lane j of a 16-lane group points at V row (key of k-slot j >> 2),
    // columns 16 dt + 4 (j & 3) .. +3
    auto rd_v = [&](const uint16_t* vl, int i) -> u32x4 {
        const int k2 = i / DT, dt = i % DT;
        const u32x2 x0 = lds_read_tr16(vl + vofs + 2 * k2 * V16 + 16 * dt);
        const u32x2 x1 = lds_read_tr16(vl + vofs + (2 * k2 + 1) * V16 + 16 * dt);
        return u32x4{x0.x, x0.y, x1.x, x1.y};
    };

    // Score phase of a block: S^T from K stage kl into sacc (lane: keys
    // 16 kt + 4 grp + i of tile kt, query row col), the accumulator taken to
    // the running maximum of the previous block (factor alpha; exactly 1
    // keeps the bits), and the first VPF V^T operands of the P.V that
    // follows, from V stage vl.  Step j issues product j, the LDS read KPF
    // products ahead (K operands, then the V^T halves) and its share of the
    // rescale, fenced so that the products never wait on LDS and the
    // multiplies fill the VALU slots beside them.
    constexpr int RPS = 4 * DT / NS;             // rescale multiplies per step
    static_assert(RPS * NS == 4 * DT, "rescale split");
    auto score_phase = [&](const uint16_t* kl, const uint16_t* vl, f32x4 (&sacc)[KT],
                           u32x4 (&vb)[VPF], float alpha) {
        u32x4 kb[KPF];
#pragma unroll
        for (int j = 0; j < KPF; ++j) kb[j] = rd_k(kl, j);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) sacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        u32x2 vhalf = {0u, 0u};
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            sacc[j % KT] = mfma_bf16_16x16x32(kb[j % KPF], qreg[j / KT], sacc[j % KT]);
            const int r = j + KPF;               // the read issued at this step
            if (r < NS) {
                kb[j % KPF] = rd_k(kl, r);
            } else {
                const int h = r - NS;            // V^T operand h / 2, half h & 1
                const int i = h >> 1, k2 = i / DT, dt = i % DT;
                const u32x2 x = lds_read_tr16(vl + vofs + (2 * k2 + (h & 1)) * V16 + 16 * dt);
                if ((h & 1) == 0) vhalf = x;
                else vb[i] = u32x4{vhalf.x, vhalf.y, x.x, x.y};
            }
#pragma unroll
            for (int u = 0; u < RPS; ++u) {
                const int e = j * RPS + u;       // accumulator element e
                oacc[e / 4][e % 4] *= alpha;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Softmax of block b from its raw scores, in slices that the P.V of the
    // previous block interleaves: the causal / window mask, P in qh (and the
    // low halves in ql), the row sum folded into l_run, and the factor that
    // takes the accumulator to the new running maximum.  A key p of the
    // block is attended when lo_row <= p <= t_row, one unsigned compare of
    // p - lo_row against t_row - lo_row; rows past the chunk end score finite
    // values against finite keys and are never stored.  The scale c > 0 is
    // applied inside the exponent: the row maximum of c s is c times that of
    // s (rounding is monotone), and exp2(c s - m) takes one fused rounding.
    // Probability e sits in tile e >> 2, element e & 3: P.V step e >> 3,
    // k-slot (grp, e & 7), i.e. keys 32 ks + 4 grp + (e & 3) + 16 ((e >> 2) & 1).
    constexpr int SL_MAX = KT;                   // slices 0 .. KT-1 mask a tile each
    constexpr int SL_EXP = KT + 4;
    constexpr int SL_CVT = SL_EXP + NE;
    constexpr int NSLICE = SL_CVT + NE / 2;      // the row sum rides on the last one
    const uint32_t span = (uint32_t)(t_row - lo_row);
    float sm_mx = 0.f, sm_mnew = 0.f, sm_muse = 0.f, sm_alpha = 1.f, sm_psum = 0.f;
    float sm_pe[NE];
    auto softmax_slice = [&](int sl, int b, f32x4 (&sacc)[KT], u32x4 (&qh)[KS],
                             u32x4 (&ql)[KS]) {
        if (sl < SL_MAX) {
            const int kt = sl;
            const int d0 = b * KB + 16 * kt + 4 * grp - lo_row;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sacc[kt][i] = ((uint32_t)(d0 + i) <= span) ? sacc[kt][i] : -INFINITY;
        } else if (sl == SL_MAX) {
            float mx = sacc[0][0];
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[kt][i]);
            sm_mx = mx;
        } else if (sl == SL_MAX + 1) {
            float a, b2;
            pair16(sm_mx, a, b2);
            sm_mx = fmaxf(a, b2);
        } else if (sl == SL_MAX + 2) {
            float a, b2;
            pair32(sm_mx, a, b2);
            sm_mnew = fmaxf(m_run, fmaxf(a, b2) * c);
            sm_muse = (sm_mnew == -INFINITY) ? 0.f : sm_mnew;
            sm_psum = 0.f;
        } else if (sl == SL_MAX + 3) {
            sm_alpha = fast_exp2(m_run - sm_muse);
        } else if (sl < SL_CVT) {
            const int e = sl - SL_EXP;
            sm_pe[e] = fast_exp2(fmaf(sacc[e >> 2][e & 3], c, -sm_muse));
            sm_psum += sm_pe[e];
        } else if (sl < NSLICE) {
            const int u = sl - SL_CVT;
            const uint32_t hw = cvt_pk_bf16(sm_pe[2 * u], sm_pe[2 * u + 1]);
            qh[u / 4][u % 4] = hw;
            if (PM == ATTN_P_BF16X2)
                ql[u / 4][u % 4] = cvt_pk_bf16(sm_pe[2 * u] - bf16lo_to_f32(hw),
                                               sm_pe[2 * u + 1] - bf16hi_to_f32(hw));
            if (sl == NSLICE - 1) {
                l_run = l_run * sm_alpha + sm_psum;
                m_run = sm_mnew;
            }
        }
    };
    static_assert(NSLICE <= NPV, "the softmax fits beside one P.V");

    // P.V of a block (V stage vl, first VPF operands already in vb, P in
    // ph / pl) with the next block's softmax beside it: step i issues the
    // products of operand i, the read of operand i + VPF and one softmax
    // slice, fenced so that the order holds.
    auto pv_phase = [&](const uint16_t* vl, u32x4 (&vb)[VPF], const u32x4 (&ph)[KS],
                        const u32x4 (&pl)[KS], int bn, f32x4 (&sacc)[KT], u32x4 (&qh)[KS],
                        u32x4 (&ql)[KS]) {
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
            const int k2 = i / DT, dt = i % DT;
            const u32x4 a = vb[i % VPF];
            if (i + VPF < NPV) vb[i % VPF] = rd_v(vl, i + VPF);
            oacc[dt] = mfma_bf16_16x16x32(a, ph[k2], oacc[dt]);
            if (PM == ATTN_P_BF16X2) oacc[dt] = mfma_bf16_16x16x32(a, pl[k2], oacc[dt]);
            softmax_slice(i, bn, sacc, qh, ql);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // P of the block whose P.V comes next, and the next block's
    u32x4 pch[KS], pcl[KS], pnh[KS], pnl[KS];
#pragma unroll
    for (int k2 = 0; k2 < KS; ++k2) {
        pch[k2] = u32x4{0u, 0u, 0u, 0u};
        pcl[k2] = u32x4{0u, 0u, 0u, 0u};
        pnh[k2] = u32x4{0u, 0u, 0u, 0u};
        pnl[k2] = u32x4{0u, 0u, 0u, 0u};
    }
    u32x4 vb[VPF];

    // prologue: K(b_lo), V(b_lo) and K(b_lo + 1) in flight; softmax of b_lo
    dma(Kg, ks_lds[0], lane_dst, b_lo);
    dma(Vg, vs_lds[0], lane_dstv, b_lo);
    if (b_lo < b_hi) dma(Kg, ks_lds[1], lane_dst, b_lo + 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (head_ok) {
        f32x4 sacc[KT];
        score_phase(ks_lds[0], vs_lds[0], sacc, vb, 1.f);
#pragma unroll
        for (int sl = 0; sl < NSLICE; ++sl) softmax_slice(sl, b_lo, sacc, pch, pcl);
    }
    __syncthreads();                             // K(b_lo) read by every wave

    // Iteration b: the scores of block b + 1 (with the rescale that block b
    // needs), then block b's P.V beside block b + 1's softmax.
    for (int b = b_lo; b < b_hi; ++b) {
        const int st = (b - b_lo) & 1;
        // in LDS now: V(b) in vs[st], K(b + 1) in ks[st ^ 1]; P(b) in pch / pcl
        if (b + 2 <= b_hi) dma(Kg, ks_lds[st], lane_dst, b + 2);
        dma(Vg, vs_lds[st ^ 1], lane_dstv, b + 1);
        if (head_ok) {
            f32x4 sacc[KT];
            score_phase(ks_lds[st ^ 1], vs_lds[st], sacc, vb, sm_alpha);
            pv_phase(vs_lds[st], vb, pch, pcl, b + 1, sacc, pnh, pnl);
#pragma unroll
            for (int k2 = 0; k2 < KS; ++k2) {
                pch[k2] = pnh[k2];
                pcl[k2] = pnl[k2];
            }
        }
        __builtin_amdgcn_s_waitcnt(0);          // this wave's DMAs of K(b+2), V(b+1)
        __syncthreads();                         // everyone's; K(b+1), V(b) free
    }
    if (head_ok) {
        const uint16_t* vl = vs_lds[(b_hi - b_lo) & 1];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] *= sm_alpha;
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
            const int k2 = i / DT, dt = i % DT;
            const u32x4 a = rd_v(vl, i);
            oacc[dt] = mfma_bf16_16x16x32(a, pch[k2], oacc[dt]);
            if (PM == ATTN_P_BF16X2) oacc[dt] = mfma_bf16_16x16x32(a, pcl[k2], oacc[dt]);
        }
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
