// Prompt (prefill) attention on gfx950 for head dim 512 (the global layers).
//
// Method: as the general prompt kernel (TensorFold PR #975, prompt attention
// commits; PR #1183 window_rows notes): 16 query rows of a head per tile,
// causal (and window) masks, an online softmax whose running maximum moves
// once per key block of 32 keys aligned to absolute positions, P rounded to
// bf16 or kept as two bf16 halves, the key/value cache read after the chunk
// has been written into it.
//
// MI355X design.  Matrix products here are fed from LDS, and with one wave
// per SIMD a 16x16x32 product cannot hide a 1 KiB LDS read beside it: LDS
// bytes per product set the speed.  So a workgroup of four waves takes one
// 16-row tile and four query heads of one KV group as two head pairs x two
// halves of the head dim: wave (pair p, half e) holds Q of heads 2p, 2p + 1
// over dims [256 e, 256 e + 256), so every K operand it reads serves two
// products (one per head) and every V^T operand four (two heads, hi and lo
// halves of P).
//   S^T partial = K[:, half] . Q[:, half]^T   two heads per K operand;
//   the two halves of a head pair swap partials through LDS (4 KiB per wave
//   per block) and both add them (fp32 addition commutes, so both hold the
//   same bits) and run the same softmax for the pair's two heads;
//   O^T[half] += V^T[half] . P^T              each wave owns half of the
//   output dims of its two heads.
// K and V blocks reach LDS by direct global->LDS loads (two stages, rows
// padded by 32 bytes), spread one instruction every few steps between the
// products; an L2 prefetch four blocks ahead is shared out across the
// workgroups of an XCD.  Each iteration issues the scores of block b + 1,
// swaps the partials, then block b's P.V with block b + 1's softmax cut into
// stages between its products; the steps are fenced so the order holds.
// The accumulator is rescaled at the top of an iteration only when some row's
// maximum moved.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int P5_D = 512;
constexpr int P5_KB = 32;                // keys per block
constexpr int P5_H = 256;                // dims of Q and O a wave holds

// Operations per stage of the pair softmax, for each of the two heads
// (bf16x2: with the low halves of P).  Stages [0, P5_SPLIT) run beside the
// previous block's P.V (they need the scores); the rest, which turn the
// probabilities into P and the row sum, run in the block's own score phase,
// before its P.V reads P.
template <bool X2>
__host__ __device__ constexpr int p5_stage_ops(int k) {
    switch (k) {
        case 0: return 8;            // S = own + partner partial
        case 1: return 3;            // partial maxima (max3)
        case 2: return 1;            // the lane's maximum
        case 3: case 4: case 5: case 6: case 7: return 1;   // swap, max, swap, max, x c
        case 8: return 2;            // m_new, m_use
        case 9: case 10: return 9;   // exponent arguments; factor, exponentials
        case 11: return 1;           // maximum carried
        case 12: return 4;           // row sum level 1
        case 13: return 4;           // hi halves of P
        case 14: return 2 + (X2 ? 8 : 0);   // sum level 2, hi halves back to fp32
        case 15: return 1 + (X2 ? 8 : 0);   // sum level 3, residuals
        default: return 1 + (X2 ? 4 : 0);   // row sum carried, lo halves
    }
}
constexpr int P5_NSTG = 17;
constexpr int P5_SPLIT = 13;
template <bool X2>
__host__ __device__ constexpr int p5_plan_steps(int k0, int k1, int start, int cap) {
    int t = start;
    for (int k = k0; k < k1; ++k) t += (2 * p5_stage_ops<X2>(k) + cap - 1) / cap;
    return t;
}

template <int PM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_pair_kernel(uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
                         const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
                         int pos0, int n_rows, int Hq, int Hkv, int G, int HG, int cap,
                         int ring, int window, float c,
                         const int32_t* __restrict__ last_key) {
    constexpr int D = P5_D, KB = P5_KB, HD = P5_H;
    constexpr bool X2 = PM == ATTN_P_BF16X2;
    constexpr int KT = KB / 16;              // 16-key score tiles per block
    constexpr int QST = HD / 32;             // reduction steps over a half
    constexpr int DTH = HD / 16;             // output d tiles of a half
    constexpr int ROW = D + 16;              // LDS row (elements), 32 bytes of padding
    constexpr int BLK = KB * ROW;
    constexpr int INSTR = KB;                // DMA instructions (1 KiB rows) per block
    constexpr int IPW = INSTR / 4;
    constexpr int NS = KT * QST;             // K operands per block (two products each)
    constexpr int KPF = 6;                   // K operand reads in flight
    constexpr int VPF = KPF / 2;             // V^T operands read ahead
    constexpr int NPV = 2 * DTH;             // P.V half-steps: (d tile, head)
    constexpr int SM_START = 2;              // steps before the partner partials are used
    constexpr int SM_CAP = 4;                // softmax operations per step
    constexpr int SMA_STEPS = p5_plan_steps<X2>(0, P5_SPLIT, SM_START, SM_CAP);
    constexpr int SMB_STEPS = p5_plan_steps<X2>(P5_SPLIT, P5_NSTG, 0, SM_CAP);
    constexpr int DMA_K_EVERY = NS / IPW;    // score steps between K DMA issues
    constexpr int DMA_V_EVERY = NPV / IPW;   // P.V half-steps between V DMA issues
    static_assert(DMA_K_EVERY * IPW == NS && DMA_V_EVERY * IPW == NPV, "DMA spread");
    static_assert(SMA_STEPS <= NPV, "the first softmax stages fit beside one P.V");
    static_assert(SMB_STEPS <= NS, "the last softmax stages fit in one score phase");

    __shared__ __attribute__((aligned(16))) uint16_t ks_lds[2][BLK];
    __shared__ __attribute__((aligned(16))) uint16_t vs_lds[2][BLK];
    __shared__ __attribute__((aligned(16))) f32x4 xs_lds[4][2 * KT][64];   // S partials
    __shared__ __attribute__((aligned(16))) uint16_t pf_lds[2][512];      // prefetch landing

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int pr = wave >> 1;                // head pair
    const int dh = wave & 1;                 // half of the head dim

    // XCD-aware tile order (workgroup L runs on XCD L % 8): each XCD takes a
    // contiguous range of (KV group, head group, row tile), so the
    // workgroups sharing an L2 stream the same K/V blocks together
    const int n_rt = (n_rows + 15) / 16;
    const int nwg = n_rt * Hkv * HG;
    const int L = blockIdx.x;
    const int lam = (nwg % 8 == 0) ? (L % 8) * (nwg / 8) + L / 8 : L;
    const int rt = lam % n_rt;
    const int gh = lam / n_rt;
    const int r0 = rt * 16;
    const int g = gh / HG;
    const int hl0 = (gh % HG) * 4 + 2 * pr;
    const bool ok0 = hl0 < G, ok1 = hl0 + 1 < G;
    const bool pair_ok = ok0;                // both halves of a pair agree
    const int hh[2] = {g * G + (ok0 ? hl0 : 0), g * G + (ok1 ? hl0 + 1 : (ok0 ? hl0 : 0))};
    const int nvalid = min(16, n_rows - r0);
    const int t_first = pos0 + r0;
    const int t_last = pos0 + r0 + nvalid - 1;
    const int lo_tile = window > 0 ? max(0, t_first - window + 1) : 0;
    const int lo_last = window > 0 ? max(0, t_last - window + 1) : 0;
    const bool row_ok = col < nvalid;
    const int t_row = pos0 + r0 + col;
    const int lo_row = window > 0 ? max(0, t_row - window + 1) : 0;
    // each row's last key: its own position, or last_key's value clamped to
    // [own position, the chunk's last row]; the tile reads keys up to the
    // largest of its rows' last keys (a wave-uniform value)
    int t_hi = t_row;
    if (last_key != nullptr && row_ok)
        t_hi = min(max((int)last_key[r0 + col], t_row), pos0 + n_rows - 1);
    int hi_m = row_ok ? t_hi : t_first;
    hi_m = max(hi_m, __shfl_xor(hi_m, 1));
    hi_m = max(hi_m, __shfl_xor(hi_m, 2));
    hi_m = max(hi_m, __shfl_xor(hi_m, 4));
    hi_m = max(hi_m, __shfl_xor(hi_m, 8));
    const int hi_tile = __builtin_amdgcn_readfirstlane(hi_m);
    const int b_lo = lo_tile / KB;
    const int b_hi = hi_tile / KB;

    // Q^T operands of both heads over this wave's half, in AGPRs (the
    // products read their B operand there): Q[row col][head][256 dh + 32 st
    // + 8 grp .. +7]
    u32x4 qreg[2][QST];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const bool okk = (k == 0 ? ok0 : ok1) && row_ok;
        const uint16_t* qrow = q + ((size_t)(r0 + (row_ok ? col : 0)) * Hq + hh[k]) * D +
                               HD * dh + 8 * grp;
#pragma unroll
        for (int st = 0; st < QST; ++st) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            qreg[k][st] = okk ? ld16(qrow + 32 * st) : z;
        }
    }
    // (all loads issued before the first move, so they overlap)
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int st = 0; st < QST; ++st) asm volatile("" : "+a"(qreg[k][st]));

    const uint16_t* Kg = kc + (size_t)g * cap * D;
    const uint16_t* Vg = vc + (size_t)g * cap * D;

    // DMA of one K or V block: 32 rows of 1 KiB, instruction j moves row j;
    // wave w issues [w IPW, (w + 1) IPW) after a per-workgroup rotation that
    // spreads an XCD's concurrent requests over the L2 channels.  dma_plan
    // picks the wave's sources (uniform base, per-lane 32-bit byte offsets):
    // a block inside the tile's span that does not wrap the ring takes the
    // base of its first slot; others clamp each position into the span (a
    // block past the tile's last one reads its last key).
    const int rot = __builtin_amdgcn_readfirstlane((int)((blockIdx.x >> 3) * 7u) % INSTR);
    int lane_row[IPW];
    int lane_dst[IPW];
    uint32_t lane_off[IPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int j = (wave * IPW + i + rot) % INSTR;
        lane_row[i] = j;
        lane_dst[i] = j * ROW;
        lane_off[i] = (uint32_t)(j * D + lane * 8) * 2u;
    }
    auto dma_plan = [&](const uint16_t* gsrc, uint16_t* stage, int b, const uint16_t*& base,
                        uint32_t (&voff)[IPW], uint32_t& lds0) {
        const int p0 = b * KB;
        const int s0 = ring ? p0 % cap : p0;
        lds0 = lds_addr(stage);
        if (p0 >= lo_tile && p0 + KB - 1 <= hi_tile && s0 + KB <= cap) {
            base = gsrc + (size_t)s0 * D;
#pragma unroll
            for (int i = 0; i < IPW; ++i) voff[i] = lane_off[i];
        } else {
            base = gsrc;
#pragma unroll
            for (int i = 0; i < IPW; ++i) {
                const int p = min(max(p0 + lane_row[i], lo_tile), hi_tile);
                const int slot = ring ? p % cap : p;
                voff[i] = (uint32_t)(slot * D + lane * 8) * 2u;
            }
        }
    };
    auto dma_issue = [&](const uint16_t* base, const uint32_t (&voff)[IPW], uint32_t lds0, int i) {
        dma16_asm_sbase(base, voff[i], lds0 + 2u * (uint32_t)lane_dst[i]);
    };
    auto dma = [&](const uint16_t* gsrc, uint16_t* stage, int b) {
        const uint16_t* base;
        uint32_t voff[IPW], lds0;
        dma_plan(gsrc, stage, b, base, voff, lds0);
#pragma unroll
        for (int i = 0; i < IPW; ++i) dma_issue(base, voff, lds0, i);
    };
    // L2 prefetch of block b: the XCD's workgroups take one 1 KiB row each
    // (row tile rt), K in wave 0 and V in wave 1, landing in a scratch row
    auto l2_prefetch = [&](int b) {
        if (wave >= 2) return;
        const int p = min(b * KB + rt % KB, hi_tile);
        const int slot = ring ? p % cap : p;
        dma16_asm_sbase(wave == 0 ? Kg : Vg, (uint32_t)(slot * D + lane * 8) * 2u,
                        lds_addr(pf_lds[wave]));
    };

    f32x4 oacc[2][DTH];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int dt = 0; dt < DTH; ++dt) oacc[k][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.f, 0.f};

    const int kofs = col * ROW + 8 * grp + HD * dh;
    const int vofs = (4 * grp + (col >> 2)) * ROW + 4 * (col & 3) + HD * dh;
    auto rd_k = [&](const uint16_t* kl, int j) {
        return ld16(kl + kofs + (j % KT) * 16 * ROW + 32 * (j / KT));
    };
    // V^T operand of d tile dt: lane j of a 16-lane group points at the V
    // row of k-slot j >> 2 (keys 4 grp + (col >> 2), and + 16), columns
    // 16 dt + 4 (j & 3) .. +3 of the wave's half
    auto rd_v_half = [&](const uint16_t* vl, int dt, int half) {
        return lds_read_tr16(vl + vofs + half * 16 * ROW + 16 * dt);
    };

    // a block needs no per-key mask when every row of the tile attends all of
    // its keys (a row's last key is never before its own position)
    auto is_interior = [&](int b) {
        const int p0 = b * KB;
        return p0 >= lo_last && p0 + KB - 1 <= t_first;
    };
    // keys outside [lo_row, t_hi] score -inf; applied to the own partial
    // (-inf plus the partner's finite or -inf partial stays -inf)
    auto mask = [&](int b, f32x4 (&sacc)[2][KT]) {
        const int p0 = b * KB;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int p = p0 + 16 * kt + 4 * grp + i;
                const bool okp = p >= lo_row && p <= t_hi;
#pragma unroll
                for (int k = 0; k < 2; ++k) sacc[k][kt][i] = okp ? sacc[k][kt][i] : -INFINITY;
            }
    };

    // Score phase of a block from K stage kl: the wave's half of S^T for both
    // heads (sacc[head][tile]: keys 16 tile + 4 grp + i, query row col),
    // and the first VPF V^T operands of the P.V that follows (stage vl).
    // Step j issues the two products of K operand j, the LDS read KPF ahead
    // (K operands, then V^T halves), the step's DMA hook and softmax
    // operations, fenced.
    auto score_phase = [&](const uint16_t* kl, const uint16_t* vl, f32x4 (&sacc)[2][KT],
                           u32x4 (&vb)[VPF], auto&& hook, auto&& sm_hook) {
        u32x4 kb[KPF];
#pragma unroll
        for (int j = 0; j < KPF; ++j) kb[j] = rd_k(kl, j);
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) sacc[k][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        u32x2 vhalf = {0u, 0u};
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const int kt = j % KT, st = j / KT;
            const u32x4 a = kb[j % KPF];
            sacc[0][kt] = mfma_bf16_16x16x32(a, qreg[0][st], sacc[0][kt]);
            sacc[1][kt] = mfma_bf16_16x16x32(a, qreg[1][st], sacc[1][kt]);
            const int r = j + KPF;
            if (r < NS) {
                kb[j % KPF] = rd_k(kl, r);
            } else {
                const int h = r - NS;            // V^T operand h / 2, half h & 1
                const u32x2 x = rd_v_half(vl, h >> 1, h & 1);
                if ((h & 1) == 0) vhalf = x;
                else vb[h >> 1] = u32x4{vhalf.x, vhalf.y, x.x, x.y};
            }
            hook(j);
            sm_hook(j);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // the partials of a block: own half out to LDS, a barrier (LDS only: the
    // K/V loads stay in flight), the partner's half back (used from softmax
    // stage 0 on)
    auto exchange = [&](const f32x4 (&sacc)[2][KT], f32x4 (&part)[2][KT]) {
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) xs_lds[wave][k * KT + kt][lane] = sacc[k][kt];
        __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0) only
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) part[k][kt] = xs_lds[wave ^ 1][k * KT + kt][lane];
    };

    // Softmax of a block for both heads, in stages; a stage's operations are
    // independent (they alternate heads) and use only earlier stages'
    // results, and a phase carries ceil(2 ops / SM_CAP) steps of each.  As in
    // the general kernel: the scale c > 0 enters inside the exponent (max of
    // c s = c max s, one fused rounding in exp2(c s - m)); m is clamped to
    // -FLT_MAX so a fully masked row gives zeros; the row sum adds pairwise;
    // probability e is tile e >> 2, element e & 3, k-slot (grp, e), key
    // 4 grp + (e & 3) + 16 (e >> 2).  The factor sm_alpha of a block stays
    // until the next block's stage 10, past the rescale and row sum that use it.
    float sm_pm[2][3], sm_mx[2], sm_a[2], sm_b[2], sm_mnew[2], sm_muse[2], sm_aarg[2];
    float sm_alpha[2] = {1.f, 1.f};
    float sm_t[2][8], sm_pe[2][8], sm_ps1[2][4], sm_ps2[2][2], sm_ps3[2], sm_r[2][8];
    uint32_t sm_hw[2][4];
    auto sm_op = [&](int kst, int o, f32x4 (&sacc)[2][KT], const f32x4 (&part)[2][KT],
                     u32x4 (&qh)[2], u32x4 (&ql)[2]) {
        const int k = o & 1, oo = o >> 1;        // head, operation within the head
        auto sv = [&](int e) { return sacc[k][e >> 2][e & 3]; };
        if (kst == 0) {
            sacc[k][oo >> 2][oo & 3] += part[k][oo >> 2][oo & 3];
        } else if (kst == 1) {
            const int e = 3 * oo;
            sm_pm[k][oo] = (e + 2 < 8) ? fmaxf(fmaxf(sv(e), sv(e + 1)), sv(e + 2))
                                       : fmaxf(sv(e), sv(e + 1));
        } else if (kst == 2) {
            sm_mx[k] = fmaxf(fmaxf(sm_pm[k][0], sm_pm[k][1]), sm_pm[k][2]);
        } else if (kst == 3) {
            pair16(sm_mx[k], sm_a[k], sm_b[k]);
        } else if (kst == 4) {
            sm_mx[k] = fmaxf(sm_a[k], sm_b[k]);
        } else if (kst == 5) {
            pair32(sm_mx[k], sm_a[k], sm_b[k]);
        } else if (kst == 6) {
            sm_mx[k] = fmaxf(sm_a[k], sm_b[k]);
        } else if (kst == 7) {
            sm_mx[k] *= c;
        } else if (kst == 8) {
            if (oo == 0) sm_mnew[k] = fmaxf(m_run[k], sm_mx[k]);
            else sm_muse[k] = fmaxf(fmaxf(m_run[k], sm_mx[k]), -__FLT_MAX__);
        } else if (kst == 9) {
            if (oo == 0) sm_aarg[k] = m_run[k] - sm_muse[k];
            else sm_t[k][oo - 1] = fmaf(sv(oo - 1), c, -sm_muse[k]);
        } else if (kst == 10) {
            if (oo == 0) sm_alpha[k] = fast_exp2(sm_aarg[k]);
            else sm_pe[k][oo - 1] = fast_exp2(sm_t[k][oo - 1]);
        } else if (kst == 11) {
            m_run[k] = sm_mnew[k];
        } else if (kst == 12) {
            sm_ps1[k][oo] = sm_pe[k][2 * oo] + sm_pe[k][2 * oo + 1];
        } else if (kst == 13) {
            sm_hw[k][oo] = cvt_pk_bf16(sm_pe[k][2 * oo], sm_pe[k][2 * oo + 1]);
            qh[k][oo] = sm_hw[k][oo];
        } else if (kst == 14) {
            if (oo < 2) {
                sm_ps2[k][oo] = sm_ps1[k][2 * oo] + sm_ps1[k][2 * oo + 1];
            } else {
                const int v = oo - 2;            // hi halves back to fp32
                sm_r[k][v] = (v & 1) ? bf16hi_to_f32(sm_hw[k][v >> 1])
                                     : bf16lo_to_f32(sm_hw[k][v >> 1]);
            }
        } else if (kst == 15) {
            if (oo < 1) {
                sm_ps3[k] = sm_ps2[k][0] + sm_ps2[k][1];
            } else {
                const int v = oo - 1;            // residuals
                sm_r[k][v] = sm_pe[k][v] - sm_r[k][v];
            }
        } else {
            if (oo == 0) l_run[k] = fmaf(l_run[k], sm_alpha[k], sm_ps3[k]);
            else ql[k][oo - 1] = cvt_pk_bf16(sm_r[k][2 * (oo - 1)], sm_r[k][2 * (oo - 1) + 1]);
        }
    };
    // step i of a phase carries the operations of stages [k0, k1) the plan
    // puts there (plan starting at step start)
    auto sm_step = [&](int i, int k0, int k1, int start, f32x4 (&sacc)[2][KT],
                       const f32x4 (&part)[2][KT], u32x4 (&qh)[2], u32x4 (&ql)[2]) {
        int st0 = start;
#pragma unroll
        for (int kst = 0; kst < P5_NSTG; ++kst) {
            if (kst < k0 || kst >= k1) continue;
            const int n = 2 * p5_stage_ops<X2>(kst);
            const int ns = (n + SM_CAP - 1) / SM_CAP;
            if (i >= st0 && i < st0 + ns) {
#pragma unroll
                for (int u = 0; u < SM_CAP; ++u) {
                    const int o = (i - st0) * SM_CAP + u;
                    if (o < n) sm_op(kst, o, sacc, part, qh, ql);
                }
            }
            st0 += ns;
        }
    };

    // P.V of a block (V stage vl, first VPF operands in vb, P in ph / pl)
    // with the next block's first softmax stages beside it: half-step i =
    // (d tile i >> 1, head i & 1) issues that head's products, on even steps
    // the read of the operand VPF tiles ahead, the planned softmax
    // operations and the DMA hook.
    auto pv_phase = [&](const uint16_t* vl, u32x4 (&vb)[VPF], const u32x4 (&ph)[2],
                        const u32x4 (&pl)[2], f32x4 (&sacc)[2][KT], const f32x4 (&part)[2][KT],
                        auto&& hook) {
        u32x4 qh_unused[2], ql_unused[2];            // the first stages write no P
        u32x4 (&qh)[2] = qh_unused;
        u32x4 (&ql)[2] = ql_unused;
        u32x4 a = vb[0];
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
            const int dt = i >> 1, k = i & 1;
            if (k == 0) {
                a = vb[dt % VPF];
                if (dt + VPF < DTH) {
                    const u32x2 x0 = rd_v_half(vl, dt + VPF, 0);
                    const u32x2 x1 = rd_v_half(vl, dt + VPF, 1);
                    vb[dt % VPF] = u32x4{x0.x, x0.y, x1.x, x1.y};
                }
            }
            oacc[k][dt] = mfma_bf16_16x16x32(a, ph[k], oacc[k][dt]);
            if (X2) oacc[k][dt] = mfma_bf16_16x16x32(a, pl[k], oacc[k][dt]);
            sm_step(i, 0, P5_SPLIT, SM_START, sacc, part, qh, ql);
            hook(i);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // the accumulator to the running maximum, when some row's moved
    auto rescale = [&]() {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            if (__any(sm_alpha[k] != 1.f)) {
#pragma unroll
                for (int dt = 0; dt < DTH; ++dt) oacc[k][dt] *= sm_alpha[k];
            }
        }
    };

    u32x4 pch[2], pcl[2];                        // P of the block whose P.V is next
#pragma unroll
    for (int k = 0; k < 2; ++k) pch[k] = pcl[k] = u32x4{0u, 0u, 0u, 0u};
    u32x4 vb[VPF];
    f32x4 part[2][KT];
    // the last softmax stages of the block whose P.V is next, run whole
    auto sm_finish = [&](f32x4 (&sacc)[2][KT]) {
#pragma unroll
        for (int i = 0; i < SMB_STEPS; ++i) sm_step(i, P5_SPLIT, P5_NSTG, 0, sacc, part, pch, pcl);
    };

    // prologue: K(b_lo), V(b_lo), K(b_lo + 1) in flight; first softmax
    // stages of b_lo
    dma(Kg, ks_lds[0], b_lo);
    dma(Vg, vs_lds[0], b_lo);
    if (b_lo < b_hi) dma(Kg, ks_lds[1], b_lo + 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    {
        f32x4 sacc[2][KT] = {};
        if (pair_ok) {
            score_phase(ks_lds[0], vs_lds[0], sacc, vb, [](int) {}, [](int) {});
            if (!is_interior(b_lo)) mask(b_lo, sacc);
        }
        exchange(sacc, part);
        if (pair_ok) {
            u32x4 qh_unused[2], ql_unused[2];
#pragma unroll
            for (int i = 0; i < SMA_STEPS; ++i)
                sm_step(i, 0, P5_SPLIT, 0, sacc, part, qh_unused, ql_unused);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();                             // K(b_lo) and the partials read

    for (int b = b_lo; b < b_hi; ++b) {
        const int st = (b - b_lo) & 1;
        // in LDS: V(b) in vs[st], K(b + 1) in ks[st ^ 1]; block b's softmax
        // up to its exponentials done.  K(b + 2) goes to ks[st], V(b + 1) to
        // vs[st ^ 1] (past b_hi the K stage takes filler rows nothing reads)
        l2_prefetch(b + 4);
        const uint16_t *kbase, *vbase;
        uint32_t kvoff[IPW], vvoff[IPW], klds, vlds;
        dma_plan(Kg, ks_lds[st], b + 2, kbase, kvoff, klds);
        dma_plan(Vg, vs_lds[st ^ 1], b + 1, vbase, vvoff, vlds);
        auto k_hook = [&](int j) {
            if (j % DMA_K_EVERY == 0) dma_issue(kbase, kvoff, klds, j / DMA_K_EVERY);
        };
        auto v_hook = [&](int i) {
            if (i % DMA_V_EVERY == 0) dma_issue(vbase, vvoff, vlds, i / DMA_V_EVERY);
        };
        f32x4 sacc[2][KT];
        if (pair_ok) {
            rescale();                           // by block b's factor
            // scores of b + 1, with block b's P and row sum finished beside them
            auto smb_hook = [&](int j) {
                sm_step(j, P5_SPLIT, P5_NSTG, 0, sacc, part, pch, pcl);
            };
            score_phase(ks_lds[st ^ 1], vs_lds[st], sacc, vb, k_hook, smb_hook);
            if (!is_interior(b + 1)) mask(b + 1, sacc);
        } else {
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int kt = 0; kt < KT; ++kt) sacc[k][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < IPW; ++i) dma_issue(kbase, kvoff, klds, i);
        }
        exchange(sacc, part);
        if (pair_ok) {
            pv_phase(vs_lds[st], vb, pch, pcl, sacc, part, v_hook);
        } else {
#pragma unroll
            for (int i = 0; i < IPW; ++i) dma_issue(vbase, vvoff, vlds, i);
        }
        __builtin_amdgcn_s_waitcnt(0);          // this wave's DMAs of K(b+2), V(b+1)
        __syncthreads();                         // everyone's; K(b+1), V(b), partials free
    }

    if (!pair_ok) return;
    rescale();
    {
        f32x4 sacc_unused[2][KT] = {};
        sm_finish(sacc_unused);
        const uint16_t* vl = vs_lds[(b_hi - b_lo) & 1];
#pragma unroll
        for (int dt = 0; dt < DTH; ++dt) {
            const u32x2 x0 = rd_v_half(vl, dt, 0);
            const u32x2 x1 = rd_v_half(vl, dt, 1);
            const u32x4 a = {x0.x, x0.y, x1.x, x1.y};
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                oacc[k][dt] = mfma_bf16_16x16x32(a, pch[k], oacc[k][dt]);
                if (X2) oacc[k][dt] = mfma_bf16_16x16x32(a, pcl[k], oacc[k][dt]);
            }
        }
    }

#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const float l_tot = xsum4(l_run[k]);
        if (!(row_ok && (k == 0 ? ok0 : ok1))) continue;
        uint16_t* orow = out + ((size_t)(r0 + col) * Hq + hh[k]) * D + HD * dh + 4 * grp;
#pragma unroll
        for (int dt = 0; dt < DTH; ++dt) {
            u32x2 pk = {cvt_pk_bf16(oacc[k][dt][0] / l_tot, oacc[k][dt][1] / l_tot),
                        cvt_pk_bf16(oacc[k][dt][2] / l_tot, oacc[k][dt][3] / l_tot)};
            *reinterpret_cast<u32x2*>(orow + 16 * dt) = pk;
        }
    }
}

}  // namespace

hipError_t launch_prefill_512(uint16_t* out, const uint16_t* q, const uint16_t* kc,
                              const uint16_t* vc, int pos0, int n_rows, int Hq, int Hkv,
                              int cap, int ring, int window, float scale, int p_mode,
                              const int32_t* last_key, hipStream_t stream) {
    const int G = Hq / Hkv;
    const int HG = (G + 3) / 4;
    const float c = scale * ATTN_LOG2E;
    dim3 grid(((n_rows + 15) / 16) * Hkv * HG);
    if (p_mode == ATTN_P_BF16X2)
        prefill_pair_kernel<ATTN_P_BF16X2><<<grid, 256, 0, stream>>>(
            out, q, kc, vc, pos0, n_rows, Hq, Hkv, G, HG, cap, ring, window, c, last_key);
    else
        prefill_pair_kernel<ATTN_P_BF16><<<grid, 256, 0, stream>>>(
            out, q, kc, vc, pos0, n_rows, Hq, Hkv, G, HG, cap, ring, window, c, last_key);
    return hipGetLastError();
}
