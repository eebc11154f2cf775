// Prompt (prefill) attention on gfx950 for head dim 512 (the global layers).
//
// Method: as the general prompt kernel (TensorFold PR #975, prompt attention
// commits; PR #1183 window_rows notes): 16 query rows of a head per tile,
// causal (and window) masks, an online softmax whose running maximum moves
// once per key block of 32 keys aligned to absolute positions, P rounded to
// bf16 or kept as two bf16 halves, the key/value cache read after the chunk
// has been written into it.
//
// MI355X design.  A workgroup takes one 16-row tile and four query heads of
// one KV group with eight waves, two per SIMD, in two roles:
//   scorer w (waves 0-3): head w; S^T = K . Q^T over all 512 dims (Q in
//     AGPRs, each half of the head its own partial sum, the two added once),
//     masks, the online softmax, and P^T (bf16, or its two bf16 halves), the
//     block's rescale factor out to LDS;
//   P.V wave w (waves 4-7): heads 2 (w / 2), + 1 over half w % 2 of the head
//     dim; O^T += V^T . P^T, each V^T operand read once for four products.
// With one wave per SIMD a matrix product cannot hide the LDS reads and
// vector work of its own wave; with a scorer and a P.V wave on each SIMD the
// two roles' products, reads and softmax interleave.  A step is one barrier:
// the scorers take block i + 1 while the P.V waves take block i (P handed
// over through two LDS stages).  K and V blocks arrive by direct global->LDS
// loads issued from asm (two stages each, rows padded by 32 bytes), K by
// the scorers (one instruction every few score products) and V by the P.V
// waves (one beside each of the first d tiles' products); each workgroup
// rotates its row order so an XCD's concurrent requests spread over the L2
// channels.  Every step's arithmetic is the one the two-waves-per-head-pair
// layout gave (the same partial sums in the same order), so the outputs do
// not depend on the split.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int P5_D = 512;
constexpr int P5_KB = 32;                // keys per block
constexpr int P5_H = 256;                // dims of O a P.V wave holds

template <int PM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_roles_kernel(uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
                          const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
                          int pos0, int n_rows, int Hq, int Hkv, int G, int HG, int cap,
                          int ring, int window, float c,
                          const int32_t* __restrict__ last_key, int pos_base, int clamp_rows) {
    constexpr int D = P5_D, KB = P5_KB, HD = P5_H;
    constexpr bool X2 = PM == ATTN_P_BF16X2;
    constexpr int KT = KB / 16;              // 16-key score tiles per block
    constexpr int QS = D / 32;               // reduction steps over the head
    constexpr int DTH = HD / 16;             // output d tiles of a half
    constexpr int ROW = D + 16;              // LDS row (elements), 32 bytes of padding
    constexpr int BLK = KB * ROW;
    constexpr int IPW = KB / 4;              // DMA instructions (1 KiB rows) per wave per block
    constexpr int NS = KT * QS;              // K operands per block
    constexpr int KPF = 4;                   // K operand reads in flight
    constexpr int VPF = 4;                   // V^T operands read ahead
    // P.V waves issue at wave priority 1 over their first PV_PRIO d tiles of
    // a step, then at 0.  At equal priority the older scorer waves win the
    // SIMD's issue slots and finish early, and the P.V wave then runs alone
    // to the barrier; at priority 1 throughout it delays the scorers past
    // it (measured on the 32k prompt: 4 or 5 tiles -2.8%, 2 or 3 tiles
    // about -1%, all 16 +2%)
    constexpr int PV_PRIO = 4;
    constexpr int DMA_K_EVERY = NS / IPW;    // K rows: one every few score products
    // V rows: one beside each of the first IPW d tiles' products, so that
    // they land well before the step's end
    static_assert(DMA_K_EVERY * IPW == NS && IPW <= DTH, "DMA spread");

    __shared__ __attribute__((aligned(16))) uint16_t ks_lds[2][BLK];
    __shared__ __attribute__((aligned(16))) uint16_t vs_lds[2][BLK];
    __shared__ __attribute__((aligned(16))) u32x4 p_lds[2][4][2][64];   // P^T operands
    __shared__ float a_lds[2][4][16];                                    // rescale factors
    __shared__ float l_lds[4][16];                                       // row sums

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool scorer = wave < 4;
    const int rw = wave & 3;                 // wave within its role
    const int lane = tid & 63;
    const int col = lane & 15;
    const int grp = lane >> 4;

    // XCD-aware tile order (workgroup L runs on XCD L % 8): each XCD takes a
    // contiguous range of (KV group, head group, row tile), so the
    // workgroups sharing an L2 stream the same K/V blocks together; row tiles
    // go last row first, so that in a long launch the longest walks start
    // first
    const int n_rt = (n_rows + 15) / 16;
    const int nwg = n_rt * Hkv * HG;
    const int L = blockIdx.x;
    const int lam = (nwg % 8 == 0) ? (L % 8) * (nwg / 8) + L / 8 : L;
    const int rt = n_rt - 1 - lam % n_rt;       // later (longer) tiles first
    const int gh = lam / n_rt;
    const int r0 = rt * 16;
    const int g = gh / HG;
    const int hg0 = (gh % HG) * 4;           // the workgroup's first head within the group
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

    const uint16_t* Kg = kc + (size_t)g * cap * D;
    const uint16_t* Vg = vc + (size_t)g * cap * D;

    // DMA of one K or V block: 32 rows of 1 KiB, instruction j moves row j;
    // the four waves of a role issue [rw IPW, (rw + 1) IPW) after a
    // per-workgroup rotation that spreads an XCD's concurrent requests over
    // the L2 channels.  dma_plan picks the wave's sources (uniform base,
    // per-lane 32-bit byte offsets): a block inside the tile's span that
    // does not wrap the ring takes the base of its first slot; others clamp
    // each position into the span.
    const int rot = __builtin_amdgcn_readfirstlane((int)((blockIdx.x >> 3) * 7u) % KB);
    int lane_row[IPW];
    int lane_dst[IPW];
    uint32_t lane_off[IPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int j = (rw * IPW + i + rot) % KB;
        lane_row[i] = j;
        lane_dst[i] = j * ROW;
        lane_off[i] = (uint32_t)(j * D + lane * 8) * 2u;
    }
    auto dma_plan = [&](const uint16_t* gsrc, uint16_t* stage, int b, const uint16_t*& base,
                        uint32_t (&voff)[IPW], uint32_t& lds0) {
        const int p0 = b * KB;
        const int s0 = ring ? p0 % cap : p0 - pos_base;
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
                const int slot = ring ? p % cap : p - pos_base;
                voff[i] = (uint32_t)(slot * D + lane * 8) * 2u;
            }
        }
    };
    auto dma_issue = [&](const uint16_t* base, const uint32_t (&voff)[IPW], uint32_t lds0, int i) {
        dma16_asm_sbase(base, voff[i], lds0 + 2u * (uint32_t)lane_dst[i]);
    };
    auto end_step = [&]() {
        __builtin_amdgcn_s_waitcnt(0);           // this wave's DMAs and LDS traffic
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // Steps i = b_lo - 1 .. b_hi, one barrier each: the scorers take block
    // i + 1 (K(i + 1) in ks[(i + 1) & 1], P and factor out to stage
    // (i + 1) & 1) and load K(i + 2); the P.V waves take block i (V(i) in
    // vs[i & 1], P from stage i & 1) and load V(i + 1).
    if (scorer) {
        const int hl = hg0 + rw;
        const bool okh = hl < G;
        const int h = g * G + (okh ? hl : 0);
        // Q^T operands over the whole head, held in registers for the whole
        // pass: Q[row col][h][32 st + 8 grp .. +7]. Left to the allocator
        // (no AGPR pin), they take VGPRs with no spill at two waves per SIMD.
        u32x4 qreg[QS];
        {
            const uint16_t* qrow = q + ((size_t)(r0 + (row_ok ? col : 0)) * Hq + h) * D + 8 * grp;
#pragma unroll
            for (int st = 0; st < QS; ++st) {
                const u32x4 z = {0u, 0u, 0u, 0u};
                qreg[st] = (okh && row_ok) ? ld16(qrow + 32 * st) : z;
            }
        }
        const int kofs = col * ROW + 8 * grp;
        // K operand j: tile j & 1, dims 32 (j >> 1) + 8 grp .. +7
        auto rd_k = [&](const uint16_t* kl, int j) {
            return ld16(kl + kofs + (j % KT) * 16 * ROW + 32 * (j / KT));
        };
        float m_run = -INFINITY, l_run = 0.f;

        {
            const uint16_t* base;
            uint32_t voff[IPW], lds0;
            dma_plan(Kg, ks_lds[b_lo & 1], b_lo, base, voff, lds0);
#pragma unroll
            for (int i = 0; i < IPW; ++i) dma_issue(base, voff, lds0, i);
        }
        end_step();

        for (int i = b_lo - 1; i <= b_hi; ++i) {
            const int bs = i + 1;                // block scored in this step
            const uint16_t* kbase;
            uint32_t kvoff[IPW], klds;
            const bool more = i + 2 <= b_hi;
            dma_plan(Kg, ks_lds[i & 1], i + 2, kbase, kvoff, klds);
            if (bs <= b_hi && okh) {
                const uint16_t* kl = ks_lds[bs & 1];
                // S^T of block bs over each half of the head (the halves
                // add once, as two partial sums)
                f32x4 sacc[2][KT];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int kt = 0; kt < KT; ++kt) sacc[hf][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
                u32x4 kb[KPF];
#pragma unroll
                for (int j = 0; j < KPF; ++j) kb[j] = rd_k(kl, j);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < NS; ++j) {
                    const int kt = j % KT, st = j / KT, hf = st / (QS / 2);
                    sacc[hf][kt] = mfma_bf16_16x16x32(kb[j % KPF], qreg[st], sacc[hf][kt]);
                    if (j + KPF < NS) kb[j % KPF] = rd_k(kl, j + KPF);
                    if (more && j % DMA_K_EVERY == 0) dma_issue(kbase, kvoff, klds, j / DMA_K_EVERY);
                    __builtin_amdgcn_sched_barrier(0);
                }
                // scores s[e]: key 16 (e >> 2) + 4 grp + (e & 3), query row col
                float s[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) s[e] = sacc[0][e >> 2][e & 3] + sacc[1][e >> 2][e & 3];
                // keys outside [lo_row, t_hi] score -inf (blocks every row
                // attends whole skip this)
                const int p0 = bs * KB;
                if (!(p0 >= lo_last && p0 + KB - 1 <= t_first)) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int p = p0 + 16 * (e >> 2) + 4 * grp + (e & 3);
                        s[e] = (p >= lo_row && p <= t_hi) ? s[e] : -INFINITY;
                    }
                }
                // online softmax of the block: the scale c > 0 enters inside
                // the exponent (max of c s = c max s, one fused rounding in
                // exp2(c s - m)); m is clamped to -FLT_MAX so a fully masked
                // row gives zeros; the row sum adds pairwise
                const float pm0 = fmaxf(fmaxf(s[0], s[1]), s[2]);
                const float pm1 = fmaxf(fmaxf(s[3], s[4]), s[5]);
                const float pm2 = fmaxf(s[6], s[7]);
                float mx = fmaxf(fmaxf(pm0, pm1), pm2);
                float xa, xb;
                pair16(mx, xa, xb);
                mx = fmaxf(xa, xb);
                pair32(mx, xa, xb);
                mx = fmaxf(xa, xb);
                mx *= c;
                const float m_new = fmaxf(m_run, mx);
                const float m_use = fmaxf(fmaxf(m_run, mx), -__FLT_MAX__);
                const float aarg = m_run - m_use;
                float pe[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) pe[e] = fast_exp2(fmaf(s[e], c, -m_use));
                const float alpha = fast_exp2(aarg);
                m_run = m_new;
                const float ps1[4] = {pe[0] + pe[1], pe[2] + pe[3], pe[4] + pe[5], pe[6] + pe[7]};
                const float ps3 = (ps1[0] + ps1[1]) + (ps1[2] + ps1[3]);
                u32x4 ph, pl = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int o = 0; o < 4; ++o) ph[o] = cvt_pk_bf16(pe[2 * o], pe[2 * o + 1]);
                if constexpr (X2) {
                    float r[8];
#pragma unroll
                    for (int v = 0; v < 8; ++v)
                        r[v] = pe[v] - ((v & 1) ? bf16hi_to_f32(ph[v >> 1]) : bf16lo_to_f32(ph[v >> 1]));
#pragma unroll
                    for (int o = 0; o < 4; ++o) pl[o] = cvt_pk_bf16(r[2 * o], r[2 * o + 1]);
                }
                l_run = fmaf(l_run, alpha, ps3);
                p_lds[bs & 1][rw][0][lane] = ph;
                if constexpr (X2) p_lds[bs & 1][rw][1][lane] = pl;
                if (grp == 0) a_lds[bs & 1][rw][col] = alpha;
            } else if (more) {
#pragma unroll
                for (int i2 = 0; i2 < IPW; ++i2) dma_issue(kbase, kvoff, klds, i2);
            }
            end_step();
        }
        const float l_tot = xsum4(l_run);
        if (grp == 0) l_lds[rw][col] = l_tot;
        end_step();
        return;
    }

    // P.V waves: pair p of heads, half e of the head dim
    const int pr = rw >> 1;
    const int dh = rw & 1;
    const int hl0 = hg0 + 2 * pr;
    const bool ok0 = hl0 < G, ok1 = hl0 + 1 < G;
    const int hh[2] = {g * G + (ok0 ? hl0 : 0), g * G + (ok1 ? hl0 + 1 : (ok0 ? hl0 : 0))};
    f32x4 oacc[2][DTH];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int dt = 0; dt < DTH; ++dt) oacc[k][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // V^T operand of d tile dt: lane j of a 16-lane group points at the V
    // row of k-slot j >> 2 (keys 4 grp + (col >> 2), and + 16), columns
    // 16 dt + 4 (j & 3) .. +3 of the wave's half
    const int vofs = (4 * grp + (col >> 2)) * ROW + 4 * (col & 3) + HD * dh;
    auto rd_v = [&](const uint16_t* vl, int dt) {
        const u32x2 x0 = lds_read_tr16(vl + vofs + 16 * dt);
        const u32x2 x1 = lds_read_tr16(vl + vofs + 16 * ROW + 16 * dt);
        return u32x4{x0.x, x0.y, x1.x, x1.y};
    };
    end_step();                                  // the scorers' K(b_lo)

    for (int i = b_lo - 1; i <= b_hi; ++i) {
        const uint16_t* vbase;
        uint32_t vvoff[IPW], vlds;
        const bool more = i + 1 <= b_hi;
        dma_plan(Vg, vs_lds[(i + 1) & 1], i + 1, vbase, vvoff, vlds);
        if (i >= b_lo && ok0) {
            const int stg = i & 1;
            const uint16_t* vl = vs_lds[stg];
            u32x4 ph[2], pl[2];
            float alpha[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                ph[k] = p_lds[stg][2 * pr + k][0][lane];
                pl[k] = X2 ? p_lds[stg][2 * pr + k][1][lane] : u32x4{0u, 0u, 0u, 0u};
                alpha[k] = a_lds[stg][2 * pr + k][col];
            }
            u32x4 vb[VPF];
#pragma unroll
            for (int u = 0; u < VPF; ++u) vb[u] = rd_v(vl, u);
            // the accumulator to the running maximum, when some row's moved
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                if (__any(alpha[k] != 1.f)) {
#pragma unroll
                    for (int dt = 0; dt < DTH; ++dt) oacc[k][dt] *= alpha[k];
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int dt = 0; dt < DTH; ++dt) {
                if (dt == 0) __builtin_amdgcn_s_setprio(1);
                if (dt == PV_PRIO) __builtin_amdgcn_s_setprio(0);
                const u32x4 a = vb[dt % VPF];
                if (dt + VPF < DTH) vb[dt % VPF] = rd_v(vl, dt + VPF);
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    oacc[k][dt] = mfma_bf16_16x16x32(a, ph[k], oacc[k][dt]);
                    if (X2) oacc[k][dt] = mfma_bf16_16x16x32(a, pl[k], oacc[k][dt]);
                }
                if (more && dt < IPW) dma_issue(vbase, vvoff, vlds, dt);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else if (more) {
#pragma unroll
            for (int i2 = 0; i2 < IPW; ++i2) dma_issue(vbase, vvoff, vlds, i2);
        }
        end_step();
    }
    end_step();                                  // the scorers' row sums

    if (!ok0) return;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const float l_tot = l_lds[2 * pr + k][col];
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
                              const int32_t* last_key, int base, int clamp_rows,
                              hipStream_t stream) {
    const int G = Hq / Hkv;
    const int HG = (G + 3) / 4;
    const float c = scale * ATTN_LOG2E;
    dim3 grid(((n_rows + 15) / 16) * Hkv * HG);
    if (p_mode == ATTN_P_BF16X2)
        prefill_roles_kernel<ATTN_P_BF16X2><<<grid, 512, 0, stream>>>(
            out, q, kc, vc, pos0, n_rows, Hq, Hkv, G, HG, cap, ring, window, c, last_key, base,
            clamp_rows);
    else
        prefill_roles_kernel<ATTN_P_BF16><<<grid, 512, 0, stream>>>(
            out, q, kc, vc, pos0, n_rows, Hq, Hkv, G, HG, cap, ring, window, c, last_key, base,
            clamp_rows);
    return hipGetLastError();
}
