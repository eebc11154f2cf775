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
// MI355X design.  A workgroup of NW waves (four, or eight in launches with
// enough tiles to fill the chip twice over) takes one 16-row tile of the
// chunk and NW query heads of one KV group; wave w owns head w: 16 rows x
// the whole head dim, so its softmax state never leaves the wave.  The
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
// One wave runs per SIMD (two at NW = 8, which hide one wave's LDS reads and
// softmax behind the other's products), so the wave itself must keep its
// matrix unit fed:
// an iteration issues the scores of block b + 1 (K operands eight products
// ahead, with the accumulator rescale that block b needs in the VALU slots
// beside them), then block b's P.V with block b + 1's mask and softmax cut
// into slices between its products.  Both phases are fenced step by step so
// the compiler keeps that order.
// Lane l always owns query row l % 16 (the S^T and O^T column), so the row's
// maximum, rescale and sum stay in its four lanes (l, l^16, l^32, l^48).
// Key blocks are KB keys aligned to absolute positions; the running maximum
// moves once per block and p is rounded against it.
// Split form (SPLIT): when one workgroup per tile leaves most of the chip
// idle (a short chunk of a sliding layer: 64 workgroups), S workgroups share
// a tile's key blocks, split into S consecutive ranges.  Workgroup s > 0
// first forms the scores of the blocks before its range (score products
// only, K alone staged) to reach the running maximum those blocks leave, so
// its p are rounded against exactly the maxima the unsplit walk uses; then it
// walks its own range and leaves a partial (maximum, row sum, accumulator)
// that a merge launch joins in range order.  The ranges are uneven
// (the first longest), so that every workgroup's walk, score-only blocks
// included, takes about the same time.  Key slots of a block
// outside the tile's attended span [lo, hi] are fetched from a position
// inside the span instead: their scores are masked, and their V rows are
// finite, so they add exactly zero (a never-written row is never read).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace {

template <int D> struct PrefillCfg;
template <> struct PrefillCfg<256> { static constexpr int KB = 64; };
template <> struct PrefillCfg<512> { static constexpr int KB = 32; };


// Operations per stage of the staged softmax (see the kernel) for NE
// probabilities per lane, and the P.V steps its plan takes at cap
// operations per step.
template <int NE, bool X2>
__host__ __device__ constexpr int sm_stage_ops(int k) {
    constexpr int NP = NE / 2;
    constexpr int NMX = (NE + 2) / 3;
    constexpr int NMX2 = (NMX + 2) / 3;
    switch (k) {
        case 0: return NMX;
        case 1: return NMX2;
        case 2: return NMX2 > 1 ? 1 : 0;
        case 3: case 4: case 5: case 6: case 7: return 1;
        case 8: return 2;
        case 9: case 10: return 1 + NE;
        case 11: return NE / 2 + NP;
        case 12: return NE / 4 + (X2 ? 2 * NP : 0);
        case 13: return NE / 8 + (X2 ? 2 * NP : 0);
        case 14: return NE / 16 + (X2 ? NP : 0);
        default: return 1;
    }
}
template <int NE, bool X2>
__host__ __device__ constexpr int sm_plan_steps(int cap, int nstg) {
    int t = 0;
    for (int k = 0; k < nstg; ++k) t += (sm_stage_ops<NE, X2>(k) + cap - 1) / cap;
    return t;
}

// First block of range s of S over a tile's n blocks: round(n F_s), F_s =
// (1 - x^s) / (1 - x^S), x = SPLIT_XN / SPLIT_XD the cost of a score-only
// block relative to a whole one subtracted from 1 (the ranges where every
// workgroup's walk costs the same).
// (measured on MI355X: a score-only block takes about 0.54 of a whole one)
constexpr int SPLIT_XN = 6, SPLIT_XD = 13;
ATTN_DEV int split_start(int n, int S, int s) {
    if (s <= 0) return 0;
    if (s >= S) return n;
    long long xs = 1, ds = 1, xS = 1, dS = 1;
    for (int i = 0; i < s; ++i) { xs *= SPLIT_XN; ds *= SPLIT_XD; }
    for (int i = 0; i < S; ++i) { xS *= SPLIT_XN; dS *= SPLIT_XD; }
    // F_s = (1 - xs/ds) / (1 - xS/dS) = (dS - xs dS / ds) / (dS - xS)
    const long long num = dS - xs * (dS / ds);
    const long long den = dS - xS;
    return (int)((2 * n * num + den) / (2 * den));
}

template <int D, int PM, bool SPLIT, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void prefill_kernel(uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
                    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
                    int pos0, int n_rows, int Hq, int Hkv, int G, int HG, int cap,
                    int ring, int window, float c,
                    const int32_t* __restrict__ last_key, int S,
                    float* __restrict__ part_acc, float* __restrict__ part_ml, int pos_base,
                    int clamp_rows, int rs, long long hs) {
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
    constexpr int IPW = INSTR / NW;          // ... per wave
    static_assert(IPW * NW == INSTR, "DMA split");
    constexpr int K16 = row_pos<D, KPADP>(16);     // offset of the next 16 rows
    constexpr int V16 = row_pos<D, VPADP>(16);

    // two K stages and two V stages: K runs one block ahead of V
    __shared__ __attribute__((aligned(16))) uint16_t ks_lds[2][KBLK];
    __shared__ __attribute__((aligned(16))) uint16_t vs_lds[2][VBLK];
    // landing row of the L2 prefetch loads (written, never read)
    __shared__ __attribute__((aligned(16))) uint16_t pf_lds[2][512];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lane = tid & 63;
    const int col = lane & 15;
    const int grp = lane >> 4;

    // XCD-aware tile order: the hardware deals workgroup L to XCD L % 8, so
    // L is renumbered to put each XCD on a contiguous range of tiles ordered
    // KV group, head group, row tile: the workgroups sharing one L2 then
    // stream the same K/V blocks at about the same time.  Row tiles go last
    // row first, so that in a long launch the longest walks start first
    // (SPLIT: the S workgroups of a tile are consecutive in that order)
    const int n_rt = (n_rows + 15) / 16;
    const int nwg = n_rt * Hkv * HG * (SPLIT ? S : 1);
    const int L = blockIdx.x;
    const int lam = (nwg % 8 == 0) ? (L % 8) * (nwg / 8) + L / 8 : L;
    const int sp = SPLIT ? lam % S : 0;              // range of the tile's blocks
    const int lt = SPLIT ? lam / S : lam;
    const int rt = n_rt - 1 - lt % n_rt;        // later (longer) tiles first
    const int gh = lt / n_rt;                        // g * HG + head group
    const int r0 = rt * 16;
    const int g = gh / HG;
    const int hl = (gh % HG) * NW + wave;
    const bool head_ok = hl < G;
    const int h = g * G + (head_ok ? hl : 0);
    const int nvalid = min(16, n_rows - r0);
    const int t_first = pos0 + r0;
    const int t_last = pos0 + r0 + nvalid - 1;
    const int lo_tile = window > 0 ? max(0, t_first - window + 1) : 0;
    const int lo_last = window > 0 ? max(0, t_last - window + 1) : 0;
    const bool row_ok = col < nvalid;
    const int t_row = pos0 + r0 + col;
    const int lo_row = window > 0 ? max(0, t_row - window + 1) : 0;
    // each row's last key: its own position, or last_key's value clamped to
    // [own position, the last row of the row's chunk of clamp_rows rows]; the
    // tile reads keys up to the largest of its rows' last keys (a
    // wave-uniform value)
    int t_hi = t_row;
    if (last_key != nullptr && row_ok) {
        const int r = r0 + col;
        const int c_end = (int)min((long long)n_rows, (long long)(r - r % clamp_rows) + clamp_rows);
        t_hi = min(max((int)last_key[r], t_row), pos0 + c_end - 1);
    }
    int hi_m = row_ok ? t_hi : t_first;
    hi_m = max(hi_m, __shfl_xor(hi_m, 1));
    hi_m = max(hi_m, __shfl_xor(hi_m, 2));
    hi_m = max(hi_m, __shfl_xor(hi_m, 4));
    hi_m = max(hi_m, __shfl_xor(hi_m, 8));
    const int hi_tile = __builtin_amdgcn_readfirstlane(hi_m);
    const int b_lo = lo_tile / KB;
    const int b_hi = hi_tile / KB;
    // this workgroup's blocks [b_beg, b_end] (all of them unless SPLIT; a
    // split range may be empty)
    int b_beg = b_lo, b_end = b_hi;
    if constexpr (SPLIT) {
        const int nb = b_hi - b_lo + 1;
        b_beg = b_lo + split_start(nb, S, sp);
        b_end = b_lo + split_start(nb, S, sp + 1) - 1;
    }

    // key rows of KV group g: slot s at Kg + s rs (a cache: rs = D, groups
    // cap D apart; a prompt's own k / v rows: rs = Hkv D, groups D apart)
    const uint16_t* Kg = kc + (size_t)g * (size_t)hs;
    const uint16_t* Vg = vc + (size_t)g * (size_t)hs;

    // DMA of one K or V block: instruction j (wave w issues [w IPW, (w+1) IPW))
    // moves 1 KiB: block row j at D=512, rows 16 (j >> 3) + (j & 7) and +8 at
    // D=256 (lanes 0..31 and 32..63).  dma_plan picks the sources of the
    // wave's IPW instructions (a wave-uniform base and per-lane 32-bit byte
    // offsets), dma_issue sends one, so the loop can spread them between its
    // products.  A block whose KB positions all lie in the tile's span and do
    // not wrap the ring takes the base of its first slot and per-lane constant
    // offsets; other blocks clamp each position into the span (a block past
    // the tile's last one reads its last key).
    // The workgroups of one XCD stream the same blocks at about the same
    // time; each starts its instructions at a different row (rotation by its
    // index on the XCD) so that their requests spread over the L2 channels
    // instead of queueing on the few that hold the same lines.
    int lane_row[IPW];          // block row this lane moves in instruction i
    int lane_dst[IPW];          // LDS row base (elements) of instruction i, for K
    int lane_dstv[IPW];         // ... for V
    const int rot = __builtin_amdgcn_readfirstlane((int)((blockIdx.x >> 3) * 7u) % INSTR);
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int j = (wave * IPW + i + rot) % INSTR;
        const int r0i = (LPR == 64) ? j : 16 * (j >> 3) + (j & 7);
        lane_row[i] = (LPR == 64) ? j : r0i + 8 * (lane >> 5);
        lane_dst[i] = row_pos<D, KPADP>(r0i);
        lane_dstv[i] = row_pos<D, VPADP>(r0i);
    }
    const int lane_col = (lane % LPR) * 8;
    uint32_t lane_off[IPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i) lane_off[i] = (uint32_t)(lane_row[i] * rs + lane_col) * 2u;
    auto dma_plan = [&](const uint16_t* g, uint16_t* stage, int b, const uint16_t*& base,
                        uint32_t (&voff)[IPW], uint32_t& lds0) {
        const int p0 = b * KB;
        const int s0 = ring ? p0 % cap : p0 - pos_base;
        lds0 = lds_addr(stage);
        if (p0 >= lo_tile && p0 + KB - 1 <= hi_tile && s0 + KB <= cap) {
            base = g + (size_t)s0 * rs;
#pragma unroll
            for (int i = 0; i < IPW; ++i) voff[i] = lane_off[i];
        } else {
            base = g;
#pragma unroll
            for (int i = 0; i < IPW; ++i) {
                const int p = min(max(p0 + lane_row[i], lo_tile), hi_tile);
                const int slot = ring ? p % cap : p - pos_base;
                voff[i] = (uint32_t)(slot * rs + lane_col) * 2u;
            }
        }
    };
    auto dma_issue = [&](const uint16_t* base, const uint32_t (&voff)[IPW], uint32_t lds0,
                         const int* dsts, int i) {
        dma16_asm_sbase(base, voff[i], lds0 + 2u * (uint32_t)dsts[i]);
    };
    auto dma = [&](const uint16_t* g, uint16_t* stage, const int* dsts, int b) {
        const uint16_t* base;
        uint32_t voff[IPW], lds0;
        dma_plan(g, stage, b, base, voff, lds0);
#pragma unroll
        for (int i = 0; i < IPW; ++i) dma_issue(base, voff, lds0, dsts, i);
    };
    constexpr int DMA_EVERY = 4;                 // fenced steps between DMA issues

    // The first K/V loads go out before Q's, so that the two latencies
    // overlap: the first three K blocks of SPLIT's score-only walk (all four
    // LDS stages take K there), else K(b_beg), V(b_beg) and K(b_beg + 1)
    const bool pre = SPLIT && b_beg > b_lo && b_beg <= b_end;    // a score-only walk first
    const bool walk = b_beg <= b_end;                            // (false: an empty range)
    static_assert(VBLK == KBLK, "K and V stages alike");
    auto kstage = [&](int i) -> uint16_t* { return i < 2 ? ks_lds[i] : vs_lds[i - 2]; };
    if (pre) {
        for (int i = 0; i < 3; ++i)
            if (b_lo + i < b_beg) dma(Kg, kstage(i), lane_dst, b_lo + i);
    } else if (walk) {
        dma(Kg, ks_lds[0], lane_dst, b_beg);
        dma(Vg, vs_lds[0], lane_dstv, b_beg);
        if (b_beg < b_end) dma(Kg, ks_lds[1], lane_dst, b_beg + 1);
    }

    // Q^T operand: lane holds Q[row col][head h][32 st + 8 grp .. +7]
    u32x4 qreg[QST];
    {
        const uint16_t* qrow = q + ((size_t)(r0 + (row_ok ? col : 0)) * Hq + h) * D + 8 * grp;
#pragma unroll
        for (int st = 0; st < QST; ++st) {
            u32x4 z = {0u, 0u, 0u, 0u};
            qreg[st] = (row_ok && head_ok) ? ld16(qrow + 32 * st) : z;
        }
        // Q lives in AGPRs (the products read their B operand from there),
        // which leaves the VGPRs to the accumulators and to the operand reads
        // in flight; all loads are issued before the first move
#pragma unroll
        for (int st = 0; st < QST; ++st) asm volatile("" : "+a"(qreg[st]));
    }


    // L2 prefetch.  Each XCD fetches every K/V block from memory once, and
    // its workgroups, which walk the blocks in step, would all wait on that
    // miss; so the workgroups of an XCD share out block b + PF_AHEAD one
    // 1 KiB slice each (row tile rt: K slice in wave 0, V slice in wave 1)
    // and load it early into a scratch row, making the block's DMAs L2 hits.
    constexpr int PF_AHEAD = 4;
    constexpr int PF_ROWS = 512 / D;             // block rows per 1 KiB slice
    auto l2_prefetch = [&](int b) {
        if (wave >= 2) return;
        const int r = (rt * PF_ROWS) % KB + (lane * 8) / D;
        const int p = max(min(b * KB + r, hi_tile), lo_tile);
        const int slot = ring ? p % cap : p - pos_base;
        const uint16_t* g = wave == 0 ? Kg : Vg;
        dma16_asm_sbase(g, (uint32_t)(slot * rs + (lane * 8) % D) * 2u,
                        lds_addr(pf_lds[wave]));
    };

    f32x4 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;
    float l_run = 0.f;

    const int kofs = row_pos<D, KPADP>(col) + 8 * grp;
    const int vofs = row_pos<D, VPADP>(4 * grp + (col >> 2)) + 4 * (col & 3);

    // a block needs no per-key mask when every row of the tile attends all
    // of its keys (a row's last key is never before its own position); the
    // others mask keys outside [lo_row, t_hi] with -inf
    auto is_interior = [&](int b) {
        const int p0 = b * KB;
        return p0 >= lo_last && p0 + KB - 1 <= t_first;
    };
    auto mask = [&](int b, f32x4 (&sacc)[KT]) {
        const int p0 = b * KB;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int p = p0 + 16 * kt + 4 * grp + i;
                sacc[kt][i] = (p >= lo_row && p <= t_hi) ? sacc[kt][i] : -INFINITY;
            }
    };

    constexpr int NS = KT * QST;                 // score products per block
    // K operand reads in flight (at two waves a SIMD the other wave covers
    // the read latency, and shallower prefetch keeps registers in VGPRs)
    constexpr int KPF = NW == 8 ? 2 : 8;
    constexpr int NPV = KS * DT;                 // V^T operands per block
    constexpr int VPF = KPF / 2;                 // V^T operands in flight
    constexpr int NE = 8 * KS;                   // probabilities per lane per block
    static_assert(KPF == 2 * VPF, "the V^T reads fill the last KPF score steps");
    static_assert(IPW * DMA_EVERY <= NS && IPW * DMA_EVERY <= NPV, "DMA issues fit the steps");

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

    // Scores alone (SPLIT's walk to its range): the score phase's products in
    // its order, so every score has the same bits
    auto score_only = [&](const uint16_t* kl, f32x4 (&sacc)[KT]) {
        u32x4 kb[KPF];
#pragma unroll
        for (int j = 0; j < KPF; ++j) kb[j] = rd_k(kl, j);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) sacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            sacc[j % KT] = mfma_bf16_16x16x32(kb[j % KPF], qreg[j / KT], sacc[j % KT]);
            if (j + KPF < NS) kb[j % KPF] = rd_k(kl, j + KPF);
            __builtin_amdgcn_sched_barrier(0);
        }
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
                           u32x4 (&vb)[VPF], float alpha, auto&& hook) {
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
            hook(j);
            __builtin_amdgcn_sched_barrier(0);
        }
        // the rescaled accumulator is used here, so the multiplies stay in
        // this phase rather than sinking past the mask branch
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) asm volatile("" :: "v"(oacc[dt]));
    };

    // Softmax of a block from its masked raw scores, cut into stages for
    // the P.V of the previous block to carry: P in qh (and the low halves in
    // ql), the row sum folded into l_run, and the factor sm_alpha that takes
    // the accumulator to the new running maximum.  The operations of a stage
    // are independent of one another and use only results of earlier
    // stages, and a stage spreads over ceil(ops / SM_CAP) P.V steps, so no
    // VALU instruction waits on its neighbour while products are due.  The
    // scale c > 0 is applied inside the exponent: the row maximum of c s is c
    // times that of s (rounding is monotone), and exp2(c s - m) takes one
    // fused rounding; m is clamped to -FLT_MAX so a fully masked row gives
    // exp2(-inf) = 0.  The row sum adds pairwise.  Probability e sits in
    // tile e >> 2, element e & 3: P.V step e >> 3, k-slot (grp, e & 7), i.e.
    // keys 32 ks + 4 grp + (e & 3) + 16 ((e >> 2) & 1).
    constexpr bool X2 = PM == ATTN_P_BF16X2;
    constexpr int NP = NE / 2;                   // packed pairs of P
    constexpr int NMX = (NE + 2) / 3;            // first-level max3 partials
    constexpr int NMX2 = (NMX + 2) / 3;
    constexpr int SM_CAP = X2 ? 6 : (NE > 8 ? 4 : 3);   // VALU ops per P.V step
    constexpr int NSTG = 16;
    constexpr int SM_STEPS = sm_plan_steps<NE, X2>(SM_CAP, NSTG);
    static_assert(NMX2 <= 2, "two second-level partial maxima at most");
    float sm_pm[NMX], sm_pm2[NMX2], sm_mx = 0.f, sm_mnew = 0.f, sm_muse = 0.f;
    float sm_aarg = 0.f, sm_alpha = 1.f;
    float sm_t[NE], sm_pe[NE], sm_ps1[NE / 2], sm_ps2[NE / 4], sm_ps3[(NE + 7) / 8];
    float sm_ps4 = 0.f, sm_a = 0.f, sm_b = 0.f;
    float sm_r[2 * NP];
    uint32_t sm_hw[NP];
    auto sm_op = [&](int k, int o, f32x4 (&sacc)[KT], u32x4 (&qh)[KS], u32x4 (&ql)[KS]) {
        auto sv = [&](int e) { return sacc[e >> 2][e & 3]; };
        if (k == 0) {                                  // partial maxima
            const int e = 3 * o;
            sm_pm[o] = (e + 2 < NE) ? fmaxf(fmaxf(sv(e), sv(e + 1)), sv(e + 2))
                     : (e + 1 < NE) ? fmaxf(sv(e), sv(e + 1)) : sv(e);
        } else if (k == 1) {
            const int e = 3 * o;
            sm_pm2[o] = (e + 2 < NMX) ? fmaxf(fmaxf(sm_pm[e], sm_pm[e + 1]), sm_pm[e + 2])
                      : (e + 1 < NMX) ? fmaxf(sm_pm[e], sm_pm[e + 1]) : sm_pm[e];
            if (NMX2 == 1) sm_mx = sm_pm2[0];
        } else if (k == 2) {
            sm_mx = (NMX2 > 1) ? fmaxf(sm_pm2[0], sm_pm2[NMX2 - 1]) : sm_pm2[0];
        } else if (k == 3) {
            pair16(sm_mx, sm_a, sm_b);
        } else if (k == 4) {
            sm_mx = fmaxf(sm_a, sm_b);
        } else if (k == 5) {
            pair32(sm_mx, sm_a, sm_b);
        } else if (k == 6) {
            sm_mx = fmaxf(sm_a, sm_b);
        } else if (k == 7) {
            sm_mx *= c;
        } else if (k == 8) {
            if (o == 0) sm_mnew = fmaxf(m_run, sm_mx);
            else sm_muse = fmaxf(fmaxf(m_run, sm_mx), -__FLT_MAX__);
        } else if (k == 9) {
            if (o == 0) sm_aarg = m_run - sm_muse;
            else sm_t[o - 1] = fmaf(sv(o - 1), c, -sm_muse);
        } else if (k == 10) {
            if (o == 0) sm_alpha = fast_exp2(sm_aarg);
            else sm_pe[o - 1] = fast_exp2(sm_t[o - 1]);
        } else if (k == 11) {
            if (o < NE / 2) {
                sm_ps1[o] = sm_pe[2 * o] + sm_pe[2 * o + 1];
            } else {
                const int u = o - NE / 2;
                sm_hw[u] = cvt_pk_bf16(sm_pe[2 * u], sm_pe[2 * u + 1]);
                qh[u / 4][u % 4] = sm_hw[u];
            }
        } else if (k == 12) {
            if (o < NE / 4) {
                sm_ps2[o] = sm_ps1[2 * o] + sm_ps1[2 * o + 1];
            } else {
                const int v = o - NE / 4;                  // hi halves back to fp32
                sm_r[v] = (v & 1) ? bf16hi_to_f32(sm_hw[v >> 1]) : bf16lo_to_f32(sm_hw[v >> 1]);
            }
        } else if (k == 13) {
            if (o < NE / 8) {
                sm_ps3[o] = sm_ps2[2 * o] + sm_ps2[2 * o + 1];
            } else {
                const int v = o - NE / 8;                  // residuals
                sm_r[v] = sm_pe[v] - sm_r[v];
            }
        } else if (k == 14) {
            if (o < NE / 16) {
                sm_ps4 = sm_ps3[0] + sm_ps3[(NE >= 16) ? 1 : 0];
            } else {
                const int u = o - NE / 16;
                ql[u / 4][u % 4] = cvt_pk_bf16(sm_r[2 * u], sm_r[2 * u + 1]);
            }
        } else if (k == 15) {
            const float psum = (NE >= 16) ? sm_ps4 : (NE >= 8) ? sm_ps3[0] : sm_ps2[0];
            l_run = fmaf(l_run, sm_alpha, psum);
            m_run = sm_mnew;
        }
    };
    // P.V step i carries the softmax operations the plan puts there
    auto sm_step = [&](int i, f32x4 (&sacc)[KT], u32x4 (&qh)[KS], u32x4 (&ql)[KS]) {
        int st0 = 0;
#pragma unroll
        for (int k = 0; k < NSTG; ++k) {
            const int n = sm_stage_ops<NE, X2>(k);
            const int ns = (n + SM_CAP - 1) / SM_CAP;
            if (i >= st0 && i < st0 + ns) {
#pragma unroll
                for (int o = (i - st0) * SM_CAP; o < n && o < (i - st0 + 1) * SM_CAP; ++o)
                    sm_op(k, o, sacc, qh, ql);
            }
            st0 += ns;
        }
    };

    // P.V of a block (V stage vl, first VPF operands already in vb, P in
    // ph / pl) with the next block's softmax beside it: step i issues the
    // products of operand i, the read of operand i + VPF and the softmax
    // operations planned for step i, fenced so that the order holds.
    auto pv_phase = [&](const uint16_t* vl, u32x4 (&vb)[VPF], const u32x4 (&ph)[KS],
                        const u32x4 (&pl)[KS], f32x4 (&sacc)[KT], u32x4 (&qh)[KS],
                        u32x4 (&ql)[KS], auto&& hook) {
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
            const int k2 = i / DT, dt = i % DT;
            const u32x4 a = vb[i % VPF];
            if (i + VPF < NPV) vb[i % VPF] = rd_v(vl, i + VPF);
            oacc[dt] = mfma_bf16_16x16x32(a, ph[k2], oacc[dt]);
            if (PM == ATTN_P_BF16X2) oacc[dt] = mfma_bf16_16x16x32(a, pl[k2], oacc[dt]);
            sm_step(i, sacc, qh, ql);
            hook(i);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = NPV; i < SM_STEPS; ++i) sm_step(i, sacc, qh, ql);
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

    // SPLIT: the running maximum the blocks before this range leave (their
    // masked scores' maxima, times c, as the softmax takes them), K alone
    // staged, the next block's K in flight beside each block's products
    // (all four LDS stages take K here, three blocks in flight behind the
    // one being scored)
    if constexpr (SPLIT) {
        if (pre) {
            for (int b = b_lo; b < b_beg; ++b) {
                const int st = (b - b_lo) & 3;
                // K(b), this wave's share (blocks b + 1, b + 2 may be in flight)
                if (b + 2 < b_beg) wait_vmcnt<2 * IPW>();
                else if (b + 1 < b_beg) wait_vmcnt<IPW>();
                else __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();                     // everyone's; K(b - 1) read
                if (b + 3 < b_beg) dma(Kg, kstage((st + 3) & 3), lane_dst, b + 3);
                if (head_ok) {
                    f32x4 sacc[KT];
                    score_only(kstage(st), sacc);
                    if (!is_interior(b)) mask(b, sacc);
                    float mx = -INFINITY;
#pragma unroll
                    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[kt][i]);
                    mx = xmax4(mx);
                    m_run = fmaxf(m_run, mx * c);
                }
            }
            __syncthreads();                         // the last K stage read
        }
    }
    // prologue: K(b_beg), V(b_beg) and K(b_beg + 1) in flight (issued at the
    // start unless a score-only walk came first); softmax of b_beg
    if (walk) {
    if (pre) {
        dma(Kg, ks_lds[0], lane_dst, b_beg);
        dma(Vg, vs_lds[0], lane_dstv, b_beg);
        if (b_beg < b_end) dma(Kg, ks_lds[1], lane_dst, b_beg + 1);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (head_ok) {
        f32x4 sacc[KT];
        score_phase(ks_lds[0], vs_lds[0], sacc, vb, 1.f, [](int) {});
        if (!is_interior(b_beg)) mask(b_beg, sacc);
#pragma unroll
        for (int i = 0; i < SM_STEPS; ++i) sm_step(i, sacc, pch, pcl);
    }
    __syncthreads();                             // K(b_beg) read by every wave
    }

    // Iteration b: the scores of block b + 1 (with the rescale that block b
    // needs), then block b's P.V beside block b + 1's softmax.
    for (int b = b_beg; b < b_end; ++b) {
        const int st = (b - b_beg) & 1;
        // in LDS now: V(b) in vs[st], K(b + 1) in ks[st ^ 1]; P(b) in pch / pcl.
        // K(b + 2) goes to ks[st] and V(b + 1) to vs[st ^ 1] beside the score
        // products, one instruction of each every DMA_EVERY steps, so both
        // have the whole P.V phase to land before the iteration's wait (past
        // b_hi the K stage takes filler rows that nothing reads).
        l2_prefetch(b + PF_AHEAD);
        const uint16_t *kbase, *vbase;
        uint32_t kvoff[IPW], vvoff[IPW], klds, vlds;
        dma_plan(Kg, ks_lds[st], b + 2, kbase, kvoff, klds);
        dma_plan(Vg, vs_lds[st ^ 1], b + 1, vbase, vvoff, vlds);
        auto k_hook = [&](int j) {
            if (j % DMA_EVERY == 0 && j / DMA_EVERY < IPW)
                dma_issue(kbase, kvoff, klds, lane_dst, j / DMA_EVERY);
            if (j % DMA_EVERY == DMA_EVERY / 2 && j / DMA_EVERY < IPW)
                dma_issue(vbase, vvoff, vlds, lane_dstv, j / DMA_EVERY);
        };
        auto v_hook = [](int) {};
        if (head_ok) {
            f32x4 sacc[KT];
            // with eight waves, each SIMD's second (younger) wave issues its
            // score products at wave priority 1, so it keeps pace with the
            // first, which the barrier would otherwise make wait for it
            // (8k prompt about 1% less time; the arithmetic is unchanged)
            if (NW == 8 && wave >= 4) __builtin_amdgcn_s_setprio(1);
            score_phase(ks_lds[st ^ 1], vs_lds[st], sacc, vb, sm_alpha, k_hook);
            if (NW == 8 && wave >= 4) __builtin_amdgcn_s_setprio(0);
            if (!is_interior(b + 1)) mask(b + 1, sacc);
            pv_phase(vs_lds[st], vb, pch, pcl, sacc, pnh, pnl, v_hook);
#pragma unroll
            for (int k2 = 0; k2 < KS; ++k2) {
                pch[k2] = pnh[k2];
                pcl[k2] = pnl[k2];
            }
        } else {
#pragma unroll
            for (int i = 0; i < IPW; ++i) {
                dma_issue(kbase, kvoff, klds, lane_dst, i);
                dma_issue(vbase, vvoff, vlds, lane_dstv, i);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);          // this wave's DMAs of K(b+2), V(b+1)
        __syncthreads();                         // everyone's; K(b+1), V(b) free
    }
    if (head_ok && walk) {
        const uint16_t* vl = vs_lds[(b_end - b_beg) & 1];
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
    if constexpr (SPLIT) {
        // the range's partial: (m, l) and the accumulator, for the merge
        const size_t pidx = ((size_t)(r0 + col) * Hq + h) * S + sp;
        if (grp == 0) {
            part_ml[2 * pidx + 0] = m_run;
            part_ml[2 * pidx + 1] = l_tot;
        }
        float* dst = part_acc + pidx * D + 4 * grp;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(dst + 16 * dt) = oacc[dt];
        return;
    }
    uint16_t* orow = out + ((size_t)(r0 + col) * Hq + h) * D + 4 * grp;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        u32x2 pk = {cvt_pk_bf16(oacc[dt][0] / l_tot, oacc[dt][1] / l_tot),
                    cvt_pk_bf16(oacc[dt][2] / l_tot, oacc[dt][3] / l_tot)};
        *reinterpret_cast<u32x2*>(orow + 16 * dt) = pk;
    }
}

// Merge of a split launch's S range partials, one lane per 4 d of a (row,
// head): M = the largest range maximum; range s weighted by 2^(m_s - M) (0
// for a range with no attended key), acc and l summed in range order with one
// rounding each (fmaf); out = bf16(acc / l).
template <int D>
ATTN_DEV void prefill_merge_unit(uint16_t* __restrict__ out, const float* __restrict__ part_acc,
                                 const float* __restrict__ part_ml, int n_rh, int S,
                                 long long i) {
    const long long rh = i / (D / 4);
    if (rh >= n_rh) return;
    const int d = (int)(i % (D / 4)) * 4;
    const float* ml = part_ml + 2 * rh * S;
    // every range's loads go out before any is used (S <= PREFILL_MAX_SPLIT;
    // a range past S repeats the last, weighted 0)
    float2 mlv[PREFILL_MAX_SPLIT];
    f32x4 av[PREFILL_MAX_SPLIT];
#pragma unroll
    for (int s = 0; s < PREFILL_MAX_SPLIT; ++s) {
        const int sc = min(s, S - 1);
        mlv[s] = *reinterpret_cast<const float2*>(ml + 2 * sc);
        av[s] = *reinterpret_cast<const f32x4*>(part_acc + (rh * S + sc) * D + d);
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < PREFILL_MAX_SPLIT; ++s) M = fmaxf(M, mlv[s].x);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
        for (int s = 0; s < PREFILL_MAX_SPLIT; ++s) {
            if (s >= S || mlv[s].x == -INFINITY) continue;
            const float w = fast_exp2(mlv[s].x - M);
            l = fmaf(w, mlv[s].y, l);
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[k] = fmaf(w, av[s][k], acc[k]);
        }
    }
    uint32_t b[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) b[k] = (l != 0.f || l != l) ? f32_to_bf16_bits(acc[k] / l) : 0u;
    *reinterpret_cast<u32x2*>(out + rh * D + d) = u32x2{pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
}

template <int D>
__global__ __launch_bounds__(256)
void prefill_merge_kernel(uint16_t* __restrict__ out, const float* __restrict__ part_acc,
                          const float* __restrict__ part_ml, int n_rh, int S) {
    prefill_merge_unit<D>(out, part_acc, part_ml, n_rh, S, (long long)blockIdx.x * 256 + threadIdx.x);
}

// A prompt's keys and values as one linear span for a single launch: unit i
// of Hkv * L * D / 8 copies eight bf16 of position base + l (l < L) of KV
// head g into [g][l][D] of sk and sv, from the ring (slot p mod cap) below
// pos0, from the prompt's k and v ([row][Hkv][D]) from pos0 on.
__global__ __launch_bounds__(256)
void stage_kernel(uint16_t* __restrict__ sk, uint16_t* __restrict__ sv,
                  const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
                  const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int pos0,
                  int base, int L, int n_rows, int Hkv, int D, int cap) {
    const int vpr = D / 8;
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)Hkv * L * vpr) return;
    const int dv = (int)(i % vpr);
    const size_t gl = i / vpr;
    const int l = (int)(gl % L);
    const int g = (int)(gl / L);
    const int p = base + l;
    size_t src;
    const uint16_t *ks, *vs;
    if (p < pos0) {
        src = ((size_t)g * cap + (size_t)(p % cap)) * D;
        ks = kc;
        vs = vc;
    } else {
        src = ((size_t)(p - pos0) * Hkv + g) * D;
        ks = k;
        vs = v;
    }
    const size_t dst = gl * D + (size_t)dv * 8;
    st16(sk + dst, ld16(ks + src + (size_t)dv * 8));
    st16(sv + dst, ld16(vs + src + (size_t)dv * 8));
}

}  // namespace

int prefill_key_block(int D, int p_mode) {
    (void)p_mode;
    return D == 256 ? PrefillCfg<256>::KB : PrefillCfg<512>::KB;
}

int prefill_split_count(int n_rows, int Hq, int Hkv, int D) {
    if (D != 256 || n_rows <= 0) return 1;
    const long long base = (long long)((n_rows + 15) / 16) * Hkv * ((Hq / Hkv + 3) / 4);
    // up to PREFILL_MAX_SPLIT workgroups a tile while the grid stays within
    // one round of the chip (one workgroup a CU)
    long long S = 256 / base;
    return (int)(S < 1 ? 1 : (S > PREFILL_MAX_SPLIT ? PREFILL_MAX_SPLIT : S));
}

size_t prefill_partials_bytes(int n_rows, int Hq, int D, int S) {
    return (size_t)n_rows * Hq * S * (D + 2) * sizeof(float);
}

namespace {

// a split launch's partials, left for its merge
struct PrefillParts {
    int S = 1;
    float* acc = nullptr;
    float* ml = nullptr;
};

// The attention launch over n_rows rows; with S > 1 in parts, its merge is
// still to come.  base: the position of slot 0 of a linear cache (a staged
// copy of a span of positions); clamp_rows: the chunk length whose last row
// bounds each row's last key.
hipError_t launch_prefill_attend(uint16_t* out, const uint16_t* q, const uint16_t* kc,
                                 const uint16_t* vc, int pos0, int n_rows, int Hq, int Hkv,
                                 int D, int cap, int ring, int window, float scale,
                                 int p_mode, const int32_t* last_key, void* ws, int base,
                                 int clamp_rows, hipStream_t stream, PrefillParts& parts,
                                 int rs = 0, long long hs = 0) {
    parts = PrefillParts{};
    // key row and KV group strides (elements): a cache's unless given
    if (rs == 0) {
        rs = D;
        hs = (long long)cap * D;
    }
    if (D == 512) {
        if (rs != D) return hipErrorInvalidValue;   // that kernel reads caches only
        return launch_prefill_512(out, q, kc, vc, pos0, n_rows, Hq, Hkv, cap, ring, window,
                                  scale, p_mode, last_key, base, clamp_rows, stream);
    }
    const int G = Hq / Hkv;
    const float c = scale * ATTN_LOG2E;
    const int S = ws ? prefill_split_count(n_rows, Hq, Hkv, D) : 1;
    const int n_rt = (n_rows + 15) / 16;
    // eight waves (heads) a workgroup when a group has more than four heads
    // and the launch still fills every CU with such workgroups (a wave's
    // arithmetic does not depend on the workgroup's width)
    const bool wide = S == 1 && G > 4 && (long long)n_rt * Hkv * ((G + 7) / 8) >= 256;
    const int HG = wide ? (G + 7) / 8 : (G + 3) / 4;
    dim3 grid(n_rt * Hkv * HG * S);
    float* part_acc = static_cast<float*>(ws);
    float* part_ml = S > 1 ? part_acc + (size_t)n_rows * Hq * S * D : nullptr;
#define PF_LAUNCH(PP, SP, NN)                                                                 \
    prefill_kernel<256, PP, SP, NN><<<grid, 64 * NN, 0, stream>>>(                            \
        out, q, kc, vc, pos0, n_rows, Hq, Hkv, G, HG, cap, ring, window, c, last_key, S,      \
        part_acc, part_ml, base, clamp_rows, rs, hs)
    if (S > 1) {
        if (p_mode == ATTN_P_BF16X2) PF_LAUNCH(ATTN_P_BF16X2, true, 4);
        else PF_LAUNCH(ATTN_P_BF16, true, 4);
    } else if (wide) {
        if (p_mode == ATTN_P_BF16X2) PF_LAUNCH(ATTN_P_BF16X2, false, 8);
        else PF_LAUNCH(ATTN_P_BF16, false, 8);
    } else {
        if (p_mode == ATTN_P_BF16X2) PF_LAUNCH(ATTN_P_BF16X2, false, 4);
        else PF_LAUNCH(ATTN_P_BF16, false, 4);
    }
#undef PF_LAUNCH
    parts.S = S;
    parts.acc = part_acc;
    parts.ml = part_ml;
    return hipGetLastError();
}

// The merge of a split launch's range partials into the rows of out
// (nothing when the launch did not split; splits happen at head dim 256).
hipError_t launch_prefill_merge(uint16_t* out, int n_rows, int Hq, const PrefillParts& parts,
                                hipStream_t stream) {
    if (parts.S <= 1) return hipSuccess;
    const long long n_rh = (long long)n_rows * Hq;
    prefill_merge_kernel<256><<<(unsigned)((n_rh * (256 / 4) + 255) / 256), 256, 0, stream>>>(
        out, parts.acc, parts.ml, (int)n_rh, parts.S);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(uint16_t* out, const uint16_t* q, const uint16_t* kc,
                          const uint16_t* vc, int pos0, int n_rows, int Hq,
                          int Hkv, int D, int cap, int ring, int window,
                          float scale, int p_mode, const int32_t* last_key,
                          void* ws, hipStream_t stream) {
    PrefillParts parts;
    const hipError_t e = launch_prefill_attend(out, q, kc, vc, pos0, n_rows, Hq, Hkv, D, cap,
                                               ring, window, scale, p_mode, last_key, ws, 0,
                                               n_rows > 0 ? n_rows : 1, stream, parts);
    if (e != hipSuccess) return e;
    return launch_prefill_merge(out, n_rows, Hq, parts, stream);
}

size_t prefill_prompt_stage_bytes(int pos0, int n_rows, int Hkv, int D, int ring, int window) {
    if (!ring) return 0;
    const long long base = std::max(0, pos0 - window + 1);
    const long long L = (long long)pos0 + n_rows - base;
    return (size_t)2 * Hkv * L * D * sizeof(uint16_t);
}

hipError_t launch_prefill_prompt(uint16_t* out, const uint16_t* q, const uint16_t* k,
                                 const uint16_t* v, uint16_t* kc, uint16_t* vc, int pos0,
                                 int n_rows, int chunk, int Hq, int Hkv, int D, int cap,
                                 int ring, int window, float scale, int p_mode,
                                 const int32_t* last_key, void* ws, hipStream_t stream) {
    PrefillParts parts;                          // (one launch, no split)
    if (!ring) {
        // every row into the cache first: no chunk reads a slot another
        // chunk writes, so one launch attends the whole prompt
        hipError_t e = launch_cache_write(kc, vc, k, v, pos0, n_rows, Hkv, D, cap, ring, stream);
        if (e != hipSuccess) return e;
        return launch_prefill_attend(out, q, kc, vc, pos0, n_rows, Hq, Hkv, D, cap, 0, window,
                                     scale, p_mode, last_key, nullptr, 0, chunk, stream, parts);
    }
    // A ring: chunk c + 1's rows would overwrite keys chunk c still reads, so
    // one launch attends the whole prompt over a linear copy, in the
    // workspace, of every key it attends (the window before pos0 from the
    // ring, the prompt's own from k and v) -- or over k and v themselves when
    // it attends no key before pos0 -- and the prompt's last rows then enter
    // the ring (those the chunked path leaves there).
    const int base = std::max(0, pos0 - window + 1);
    hipError_t e;
    if (D == 256 && window > 0 && base == pos0 &&
        (long long)n_rows * Hkv * D * 2 < (1LL << 32)) {
        // no key before pos0 is attended (a prompt from position 0, or a
        // window of one): every key is one of the prompt's own rows, read in
        // place from k and v (rows Hkv D apart, groups D apart), no copy
        e = launch_prefill_attend(out, q, k, v, pos0, n_rows, Hq, Hkv, D, n_rows, 0, window,
                                  scale, p_mode, last_key, nullptr, pos0, chunk, stream, parts,
                                  Hkv * D, D);
    } else {
        const int L = pos0 + n_rows - base;
        uint16_t* sk = static_cast<uint16_t*>(ws);
        uint16_t* sv = sk + (size_t)Hkv * L * D;
        const size_t units = (size_t)Hkv * L * (D / 8);
        stage_kernel<<<(unsigned)((units + 255) / 256), 256, 0, stream>>>(
            sk, sv, kc, vc, k, v, pos0, base, L, n_rows, Hkv, D, cap);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = launch_prefill_attend(out, q, sk, sv, pos0, n_rows, Hq, Hkv, D, L, 0, window, scale,
                                  p_mode, last_key, nullptr, base, chunk, stream, parts);
    }
    if (e != hipSuccess) return e;
    const int tail = std::min(n_rows, cap);
    const size_t ko = (size_t)(n_rows - tail) * Hkv * D;
    return launch_cache_write(kc, vc, k + ko, v + ko, pos0 + n_rows - tail, tail, Hkv, D, cap,
                              ring, stream);
}
