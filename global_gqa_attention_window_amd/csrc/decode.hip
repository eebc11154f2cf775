// Decode attention on gfx950: chunk partials over the KV cache, merged in
// chunk order, for one row or a window of up to 16 consecutive rows per
// stream.
//
// Method: TensorFold PR #1183 "cuda gemma4: images on the 12B ...", squashed
// commit bodies (window_rows notes): a head's keys split into 256-key chunks,
// each leaving a partial (max, sum, accumulator), merged in chunk order.
// PR #975 "Gemma 4 12B on the native Metal engine", decode attention commits:
// a KV head's query heads (and several decode rows) form one 16-row tile so
// every key and value is read once per window; chunks spread over
// workgroups and leave partials for a merge; every row keeps its bits at any
// window width.
#include <type_traits>

#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "prologue.h"

namespace {

constexpr int CHUNK = ATTN_DECODE_CHUNK;

// Decode windows: R <= 16 rows per stream, row r at position pos[s] + r
// (PR #975 decode attention commits: a key head's query heads and two decode
// rows fill one 16-row tile, so each key and value is read once for the
// window; PR #1183 engine note: windows of up to 16 rows a stream).
//
// A matrix-core column is one (row, query head) pair: a 16-column tile holds
// RPT = 16 / G rows of the G query heads of a KV head.  32-key blocks of K
// and V are staged in LDS by direct global->LDS loads shared by a
// workgroup's waves.  At head dim 512 a workgroup takes 4 / DS column tiles
// of one (stream, KV head, run of chunks); the DS waves of a tile split its
// output d range (all of them form the tile's scores, so a column's
// arithmetic is the same for every DS); two block stages.  At head dim 256
// a workgroup takes one tile: the run's even blocks go to waves 0 and 1 and
// its odd blocks to waves 2 and 3, each pair splitting d in two, so a
// block's K rows are read and its scores formed by two waves instead of
// four; each block set keeps its own online softmax and the two join once
// at the end (M = the larger reference maximum, each set weighted by
// 2^(m - M)); a pair of blocks lands while the previous pair is multiplied
// (four stages).  Windows of three or more tiles go, four tiles a
// workgroup, to decode_roles_kernel, which splits each tile's work between
// a scorer wave and a P.V wave with the same per-column arithmetic (at head
// dim 256 the same two block sets).  Per block and column:
//   S^T = K . Q^T               bf16 products, two 16-key tiles;
//   reference maximum           as in the one-row kernel (moves only when the
//                               block maximum passes it by 8), so p <= 2^8;
//   p = exp2(s c - m), fp32     never rounded: p = hi + mid + lo exactly,
//                               hi = bf16(p), mid = bf16(p - hi), lo =
//                               bf16(p - hi - mid) (24 significant bits in
//                               three 8-bit pieces), and
//   O^T += V^T . {hi, mid, lo}  three bf16 products per d tile, fp32
//                               accumulation: fp32 probabilities on the bf16
//                               matrix cores, at 3/16 of the fp32 path's
//                               matrix time.
// V^T comes from the staged rows by transpose reads.  A key no row of the
// workgroup attends is fetched from the slot of the window's last row
// instead (masked, finite: it adds exactly zero); a key some rows attend and
// others do not has p = 0 in the others.  Each (row, head) leaves one
// partial per run, merged by decode_merge_kernel.  The arithmetic of a
// column depends neither on the other columns of its tile nor on R, so a
// row keeps its bits at any window width.
constexpr int WKB = 32;        // keys per block (one P.V product)

// Slots per run: a workgroup carries one online softmax over a run of
// consecutive slots and leaves one partial for it.  Runs grow with the cache
// (fewer partials to write and merge) up to eight chunks, so that a 262144-key
// cache over two KV heads takes 256 workgroups, one round on the chip.  A
// cache of at most four chunks (1024 slots) takes half chunks, and one of at
// most two (512 slots) quarter chunks: its one-row decode is a few
// workgroups' chains of blocks, which shorter runs spread over more
// workgroups (8 streams over a 1024-slot ring: 13.5 against 15.4 us; one
// stream over 512 slots: 9.4 against 13.4 us).  Windows of many rows,
// already thousands of workgroups, would pay more partials for nothing; they
// take larger rings.  The length depends on the cache capacity alone, so a
// row's bits depend neither on the number of streams nor on the window width.
int decode_run_slots(int cap) {
    const int nch = (cap + CHUNK - 1) / CHUNK;
    if (nch <= 2) return CHUNK / 4;
    if (nch <= 4) return CHUNK / 2;
    const int r = nch / 16;
    return CHUNK * (r < 1 ? 1 : (r > 8 ? 8 : r));
}
int decode_run_count(int cap) {
    const int rs = decode_run_slots(cap);
    return (cap + rs - 1) / rs;
}
constexpr int WPAD = 16;       // LDS padding elements per row (per row pair at 256)
// K/V bytes above which a launch streams its K/V loads past the caches: the
// MI355X last-level (Infinity) cache holds 256 MiB
constexpr long long DECODE_STREAM_BYTES = 256ll << 20;

// Merge width: the merge kernel's waves per (row, head) and d slice; a
// workgroup that merges in place mirrors its summation order.
constexpr int MW = 16;

// The slots of one run (slot0 .. slot0 + run_slots - 1) that a workgroup's
// rows, at positions t0r .. t1, attend.  A slot one of them attends is one
// the last row attends under the window widened by t1 - max(t0r, 0).  t mod
// cap is taken once (t1m): a ring slot's position for a row at t is then
// t - ((t mod cap) - slot, plus cap when negative), with no division.  The
// tests are written with selects only, so callers' instruction order is
// never cut by branches.
struct RunKeys {
    int cap, ring, window, slot0, t0r, t1, t1m, w_all;
    ATTN_DEV RunKeys(int cap_, int ring_, int window_, int slot0_, int t_first, int t_last)
        : cap(cap_), ring(ring_), window(window_), slot0(slot0_), t0r(t_first), t1(t_last),
          t1m(t_last >= 0 ? t_last % cap_ : 0),
          w_all(window_ > 0 ? window_ + (t_last - max(t_first, 0)) : 0) {}
    // slot attended by a row at t (tm = t mod cap) under window w
    ATTN_DEV bool attended(int slot, int t, int tm, int w) const {
        int d = tm - slot;
        d += d < 0 ? cap : 0;
        const int p = ring ? t - d : slot;
        return (slot < cap) & (t >= 0) & (p >= 0) & (p <= t) & ((w <= 0) | (t - p < w));
    }
    // slot attended by some row of the workgroup
    ATTN_DEV bool any_row(int slot) const { return attended(slot, t1, t1m, w_all); }
    // first and last of the run's nblk blocks that hold a slot some row
    // attends (a wave-wide ballot; hi = -1 when there is none)
    ATTN_DEV void blocks(int nblk, int lane, int& lo, int& hi) const {
        lo = 0x7FFFFFFF;
        hi = -1;
        for (int b0 = 0; b0 < nblk; b0 += 8) {
            const int bb = b0 + (lane >> 3);     // lane covers 4 slots of block bb
            bool mine = false;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                mine |= (bb < nblk) & any_row(slot0 + bb * WKB + 4 * (lane & 7) + i);
            const uint64_t bal = __ballot(mine);
            if (bal != 0) {
                lo = min(lo, b0 + __builtin_ctzll(bal) / 8);
                hi = b0 + (63 - __builtin_clzll(bal)) / 8;
            }
        }
    }
    // block b: all its slots attended by the workgroup's rows, holding
    // consecutive positions (no ring wrap inside; almost every block)
    ATTN_DEV bool block_all(int b) const {
        const int sb = slot0 + b * WKB;
        const bool wrap = ring & (t1m >= sb) & (t1m < sb + WKB - 1);
        return ((int)(sb + WKB <= cap) & (int)!wrap & (int)any_row(sb) &
                (int)any_row(sb + WKB - 1)) != 0;
    }
    // block b needs no mask: every row attends it whole (its consecutive
    // positions within [last row - W + 1, first row])
    ATTN_DEV bool block_nomask(int b) const {
        const int sb = slot0 + b * WKB;
        int d = t1m - sb;
        d += d < 0 ? cap : 0;
        const int pl = ring ? t1 - d : sb;
        return block_all(b) && t0r >= 0 && pl + WKB - 1 <= t0r &&
               (window <= 0 || pl >= t1 - window + 1);
    }
    // Sources of block b's DMA rows row[k] as byte offsets (below 2^32) from
    // the head's K or V base; lane_elem is the lane's element offset in its
    // row.  A block_all block adds its offset to the fixed per-lane offsets
    // voff; any other block computes each lane's slot, fetching an unattended
    // one from slot sub instead.
    template <int D, int N>
    ATTN_DEV void dma_plan(int b, int sub, const int (&row)[N], const uint32_t (&voff)[N],
                           int lane_elem, uint32_t (&vo)[N]) const {
        if (block_all(b)) {
            const uint32_t boff = (uint32_t)(slot0 + b * WKB) * (uint32_t)D * 2u;
#pragma unroll
            for (int k = 0; k < N; ++k) vo[k] = boff + voff[k];
        } else {
#pragma unroll
            for (int k = 0; k < N; ++k) {
                int slot = slot0 + b * WKB + row[k];
                slot = any_row(slot) ? slot : sub;
                vo[k] = (uint32_t)(slot * D + lane_elem) * 2u;
            }
        }
    }
};

// FUSE: one launch.  With one run the workgroup writes the output itself
// (its weight e^(m - m) is 1); otherwise the last workgroup of a (stream, KV
// head, column group) to finish, found by a counter that it resets, merges
// that group's rows in the merge kernel's order, so the bits do not change.
// PREP (one row per stream): the queries come from the stacked projection
// row, normed and rotated in place, and the workgroup whose run holds the
// row's slot first writes the row's normed, rotated key and its value there
// (the functions of prologue.h, so the bits equal the standalone prologue).
// NTL: K/V blocks loaded nontemporal (streamed past the caches), for
// launches whose K/V span outgrows the last-level cache, so that nothing of
// it would be there for a later read anyway.
template <int D, int DS, bool FUSE, bool PREP, bool NTL, bool ONEP = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ONEP ? 2 : 1, ONEP ? 2 : 1)))
void decode_rows_kernel(const uint16_t* __restrict__ q,
                        const uint16_t* __restrict__ kc,
                        const uint16_t* __restrict__ vc,
                        const int32_t* __restrict__ pos,
                        float* __restrict__ part_acc,
                        float* __restrict__ part_ml,
                        uint16_t* __restrict__ out,
                        uint32_t* __restrict__ counters,
                        int R, int Hq, int Hkv, int G, int RPT, int NT, int CG,
                        int n_items, int cap, int nrun, int run_slots, int ring, int window,
                        float c, PrepArgs pa) {
    // Head dim 256: two block sets (KP).  A workgroup takes one column tile;
    // waves 0, 1 take the even blocks of the run and waves 2, 3 the odd ones,
    // each pair splitting the d range in two (DS = 2).  A wave reads only its
    // own blocks' K and V rows and forms their scores once, and the two sets
    // keep their own online softmax, joined once at the end.  Head dim 512
    // keeps one set: the DS waves of a tile all form its scores.
    constexpr bool KP = D == 256;
    static_assert(!KP || DS == 2, "two block sets take two d halves");
    constexpr int WC = KP ? 1 : 4 / DS;         // column tiles per workgroup
    constexpr int QST = D / 32;                 // reduction steps of a score
    constexpr int DTW = D / 16 / DS;            // 16-wide d tiles of this wave
    constexpr int LPR = D / 8;                  // lanes moving one row per DMA
    constexpr int NI = WKB * LPR / 64;          // DMA instructions per K (or V) block
    constexpr int NIW = NI / 4;                 // ... issued by each wave
    constexpr int BLK = row_pos<D, WPAD>(WKB);
    constexpr int K16 = row_pos<D, WPAD>(16);   // rows 16.. of a block
    constexpr int KPF = 4;                      // score steps of K reads in flight
    constexpr int VG = DTW < 4 ? DTW : 4;       // d tiles per P.V group
    constexpr int NG = DTW / VG;                // P.V groups
    // Memory-bound shapes (d split over the waves: one or two column tiles)
    // run K two blocks ahead of its use; a workgroup of four column tiles is
    // matrix-bound, and the single-launch form serves short runs where the
    // barrier inside each block costs more than the deeper prefetch gains:
    // those move K and V one block ahead, with no barrier inside a block
    constexpr bool K2 = DS >= 2 && !FUSE && !KP;
    // stages: two blocks (KP: two pairs of blocks, one in use, one landing)
    // ONEP (head dim 256, runs of one block pair): two stages, so that two
    // workgroups share a CU
    static_assert(!ONEP || (KP && !PREP), "one-pair runs");
    constexpr int NST = KP && !ONEP ? 4 : 2;
    static_assert(NIW * 4 == NI && NG * VG == DTW && QST >= KPF && (2 * NIW) % QST == 0,
                  "shapes");

    __shared__ __attribute__((aligned(16))) uint16_t ks[NST][BLK];
    __shared__ __attribute__((aligned(16))) uint16_t vs[NST][BLK];
    // the row's new key and value (PREP)
    __shared__ __attribute__((aligned(16))) uint16_t kv_new[PREP ? 2 : 1][PREP ? D : 8];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 15;
    const int grp = lane >> 4;

    // the CG workgroups of item u are consecutive on one XCD (the hardware
    // deals workgroup L to XCD L % 8), so its K/V blocks come from HBM once
    const int L = blockIdx.x;
    const int cgi = (L >> 3) % CG;
    const int u = ((L >> 3) / CG) * 8 + (L & 7);
    if (u >= n_items) return;
    const int run = u % nrun;
    const int g = (u / nrun) % Hkv;
    const int s = u / (nrun * Hkv);

    // this wave: column tile ct (RPT rows x G heads), d part dp
    const int ct = cgi * WC + (KP ? 0 : wave / DS);
    const int dp = KP ? (wave & 1) : wave % DS;
    const int set = KP ? (wave >> 1) : 0;       // block set (parity of the run's block)
    const int rr = ct * RPT + col / G;
    const int h = g * G + col % G;
    const bool cv = ct < NT && col < RPT * G && rr < R;
    const int p0 = pos[s];
    const int t_col = cv ? p0 + rr : -1;
    // the workgroup's rows and the run's slots they attend
    const int r_lo = cgi * WC * RPT;
    const int r_hi = min(R, (cgi + 1) * WC * RPT) - 1;
    const int slot0 = run * run_slots;
    const RunKeys rk(cap, ring, window, slot0, p0 + r_lo, p0 + r_hi);
    const int t1 = rk.t1;
    const size_t pidx = (((size_t)s * R + (cv ? rr : 0)) * Hq + h) * (size_t)nrun + run;
    const int tcm = t_col >= 0 ? t_col % cap : 0;

    const int nslot = min(run_slots, cap - slot0);
    const int nblk = (nslot + WKB - 1) / WKB;
    int bb_lo, bb_hi;
    rk.blocks(nblk, lane, bb_lo, bb_hi);
    f32x4 acc[DTW];
#pragma unroll
    for (int dt = 0; dt < DTW; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;
    float l_run = 0.f;

    // a run with no attended key leaves an empty partial (m = -inf, l = 0)
    if (bb_hi >= 0) {
    const size_t head_base = ((size_t)s * Hkv + g) * (size_t)cap * D;
    const uint16_t* Kh = kc + head_base;
    const uint16_t* Vh = vc + head_base;
    // Source of a slot no row of the workgroup attends: a slot the last row
    // attends (its contents are finite, or NaN that belongs in the output).
    // With PREP the row's own slot is written by this launch, so the source
    // is another attended slot of the run (its lowest, else its highest);
    // when the row's own slot is the run's only attended slot, every staged
    // row of that slot's block is overwritten with the new key and value
    // once the block has landed (fill_all).
    int sub = ring ? t1 % cap : min(t1, cap - 1);           // t1 >= 0 here
    [[maybe_unused]] bool fill_all = false;
    if constexpr (PREP) {
        // lowest or highest attended slot of block bb (which holds one; an
        // empty ballot would keep the last row's slot)
        auto ends = [&](int bb, bool lowest) {
            const bool a = lane < WKB && rk.any_row(slot0 + bb * WKB + lane);
            const uint64_t bal = __ballot(a);
            if (bal == 0) return sub;
            return slot0 + bb * WKB + (lowest ? __builtin_ctzll(bal) : 63 - __builtin_clzll(bal));
        };
        const int s_lo = ends(bb_lo, true);
        const int s_hi = ends(bb_hi, false);
        if (s_lo != sub) sub = s_lo;
        else if (s_hi != sub) sub = s_hi;
        else fill_all = true;
    }

    // DMA instruction i = wave + 4 k of a K or V block moves 1 KiB: block row
    // i at D = 512, rows 16 (i >> 3) + (i & 7) and + 8 at D = 256 (lanes
    // 0..31, 32..63).  The lane's source row and LDS offset per k are fixed.
    int dma_row[NIW];
    int dma_dst[NIW];
#pragma unroll
    for (int k = 0; k < NIW; ++k) {
        const int i = wave + 4 * k;
        const int r0 = (LPR == 64) ? i : 16 * (i >> 3) + (i & 7);
        dma_row[k] = (LPR == 64) ? r0 : r0 + 8 * (lane >> 5);
        dma_dst[k] = row_pos<D, WPAD>(r0);
    }
    // per-lane DMA source offsets of a block with consecutive slots (RunKeys::dma_plan)
    uint32_t dma_voff[NIW];
#pragma unroll
    for (int k = 0; k < NIW; ++k)
        dma_voff[k] = (uint32_t)(dma_row[k] * D + (lane % LPR) * 8) * 2u;
    // block b's DMA offsets from the heads' bases Kh, Vh
    auto dma_plan = [&](int b, uint32_t (&vo)[NIW]) {
        rk.dma_plan<D>(b, sub, dma_row, dma_voff, (lane % LPR) * 8, vo);
    };
    auto dma_one = [&](const uint16_t* base, uint16_t* stage, const uint32_t (&vo)[NIW], int k) {
        if constexpr (NTL) dma16_asm_sbase_nt(base, vo[k], lds_addr(stage + dma_dst[k]));
        else dma16_asm_sbase(base, vo[k], lds_addr(stage + dma_dst[k]));
    };

    // KP: block pair j (blocks 2 j, 2 j + 1 of the run, those the workgroup's
    // rows attend) into stages 2 ((j - jlo) & 1) + {0, 1}
    const int jlo = bb_lo >> 1, jhi = bb_hi >> 1;
    auto issue_pair = [&](int j) {
        const int sp = ONEP ? 0 : 2 * ((j - jlo) & 1);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int b = 2 * j + e;
            if (b >= bb_lo && b <= bb_hi) {
                uint32_t vo[NIW];
                dma_plan(b, vo);
#pragma unroll
                for (int k = 0; k < NIW; ++k) {
                    dma_one(Kh, ks[sp + e], vo, k);
                    dma_one(Vh, vs[sp + e], vo, k);
                }
            }
        }
    };
    // the first block's K and V go out before anything else, then the second
    // block's K (K runs two blocks ahead of its use, V one; with PREP the
    // second K stage holds the rotary table until the loop starts, so that
    // block's K goes out once the table has been read); KP: the first pair
    // (with PREP the table sits in the second pair's K stage)
    if constexpr (KP) {
        issue_pair(jlo);
    } else {
        uint32_t vo0[NIW];
        dma_plan(bb_lo, vo0);
#pragma unroll
        for (int k = 0; k < NIW; ++k) {
            dma_one(Kh, ks[0], vo0, k);
            dma_one(Vh, vs[0], vo0, k);
        }
        if (K2 && !PREP && bb_lo < bb_hi) {
            dma_plan(bb_lo + 1, vo0);
#pragma unroll
            for (int k = 0; k < NIW; ++k) dma_one(Kh, ks[1], vo0, k);
        }
    }

    // Q^T operand in AGPRs: Q[column][32 st + 8 grp .. +7]
    u32x4 qreg[QST];
    [[maybe_unused]] int b_slot = -1, r_slot = 0;          // the row's own slot, if in this run
    if constexpr (PREP) {
        // The workgroup whose run holds the row's slot writes the row's key
        // and value to the cache for later rows, and to LDS for this one
        // (copied over the staged slot once its block has landed).  Raw rows
        // are loaded first; the cos/sin table sits in the second K stage (its
        // first DMA goes out during block bb_lo's scores).
        const int slot_t = ring ? p0 % cap : p0;          // p0 >= 0 here (R = 1)
        const bool owner = slot_t >= slot0 && slot_t < slot0 + nslot && wave < 2;
        u32x4 kvx[QST];
        load_row<D>(qreg, pa.qkv + ((size_t)s * (Hq + 2 * Hkv) + h) * D, grp, cv);
        if (owner) load_kv<D>(kvx, pa, s, g, Hq, Hkv, lane, wave);
        float* cs = reinterpret_cast<float*>(&ks[KP ? 2 : 1][0]);
        rope_table<D>(cs, pa.inv_freq, p0, tid, 256);
        norm_row<D>(qreg, pa.q_w, grp, pa.eps);
        if (owner) norm_kv<D>(kvx, pa, lane, wave);
        __syncthreads();
        rope_row<D>(qreg, cs, grp);
        if (slot_t >= slot0 && slot_t < slot0 + nslot) {
            b_slot = (slot_t - slot0) / WKB;
            r_slot = (slot_t - slot0) % WKB;
        }
        if (owner)
            rope_store_kv<D>(kvx, pa, (((size_t)s * Hkv + g) * cap + slot_t) * D, cs, lane, wave,
                             kv_new[wave]);
    } else {
        const uint16_t* qrow = q + (((size_t)s * R + (cv ? rr : 0)) * Hq + h) * D + 8 * grp;
#pragma unroll
        for (int st = 0; st < QST; ++st) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            qreg[st] = cv ? ld16(qrow + 32 * st) : z;
        }
    }
#pragma unroll
    for (int st = 0; st < QST; ++st) asm volatile("" : "+a"(qreg[st]));

    const int kofs = row_pos<D, WPAD>(col) + 8 * grp;
    // V^T operand: lane j of a 16-lane group points at the row of k-slot
    // j >> 2 (keys 4 grp + (col >> 2), and + 16), columns 16 dt + 4 (j & 3)
    // of the wave's d part
    const int vofs = row_pos<D, WPAD>(4 * grp + (col >> 2)) + 4 * (col & 3) + dp * (D / DS);

    // One block from stage st.  With NEXT, block b + 1's V (and its K, unless
    // K2) moves into the other stage beside the score products; with NEXT2
    // (K2 only), once every wave has read K(b), block b + 2's K moves into
    // this K stage beside the softmax and P.V products, so about one and a
    // half blocks stay in flight.
    auto block = [&](int b, int st, auto next_c, auto next2_c) {
        constexpr bool NEXT = decltype(next_c)::value;
        constexpr bool NEXT2 = decltype(next2_c)::value;
        const uint16_t* kl = ks[st];
        const uint16_t* vl = vs[st];

        uint32_t nvo[NIW], kvo[NIW];             // DMA plans of V(b + 1), K(b + 2)
        if constexpr (NEXT) dma_plan(b + 1, nvo);
        if constexpr (NEXT2) dma_plan(b + 2, kvo);
        const bool nomask = rk.block_nomask(b);
        u32x4 kb[KPF][2];
#pragma unroll
        for (int j = 0; j < KPF; ++j) {
            kb[j][0] = ld16(kl + kofs + 32 * j);
            kb[j][1] = ld16(kl + K16 + kofs + 32 * j);
        }
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        // each step: two products, the reads KPF steps ahead, the step's
        // share of the DMA; fenced so the reads stay ahead of their use
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < QST; ++j) {
            s0 = mfma_bf16_16x16x32(kb[j % KPF][0], qreg[j], s0);
            s1 = mfma_bf16_16x16x32(kb[j % KPF][1], qreg[j], s1);
            if (j + KPF < QST) {
                kb[j % KPF][0] = ld16(kl + kofs + 32 * (j + KPF));
                kb[j % KPF][1] = ld16(kl + K16 + kofs + 32 * (j + KPF));
            }
            if constexpr (NEXT && K2) {
#pragma unroll
                for (int k = j * NIW / QST; k < (j + 1) * NIW / QST; ++k)
                    dma_one(Vh, vs[st ^ 1], nvo, k);
            } else if constexpr (NEXT) {
#pragma unroll
                for (int k = j * 2 * NIW / QST; k < (j + 1) * 2 * NIW / QST; ++k) {
                    if (k < NIW) dma_one(Kh, ks[st ^ 1], nvo, k);
                    else dma_one(Vh, vs[st ^ 1], nvo, k - NIW);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (NEXT2) {
            // every wave's K(b) reads are done (their products consumed them)
            __syncthreads();
#pragma unroll
            for (int k = 0; k < NIW; ++k) dma_one(Kh, ks[st], kvo, k);
            __builtin_amdgcn_sched_barrier(0);
        }
        // first V^T group's reads go out before the softmax
        u32x4 va[2][VG];
        auto rd_v = [&](int dt) -> u32x4 {
            const u32x2 x0 = lds_read_tr16(vl + vofs + 16 * dt);
            const u32x2 x1 = lds_read_tr16(vl + K16 + vofs + 16 * dt);
            return u32x4{x0.x, x0.y, x1.x, x1.y};
        };
#pragma unroll
        for (int e = 0; e < VG; ++e) va[0][e] = rd_v(e);

        const int sb = slot0 + b * WKB;
        float tv[8];
        float mx = -INFINITY;
        if (nomask) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                tv[i] = s0[i] * c;
                tv[4 + i] = s1[i] * c;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok0 = rk.attended(sb + 4 * grp + i, t_col, tcm, window);
                const bool ok1 = rk.attended(sb + 16 + 4 * grp + i, t_col, tcm, window);
                tv[i] = ok0 ? s0[i] * c : -INFINITY;
                tv[4 + i] = ok1 ? s1[i] * c : -INFINITY;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fmaxf(tv[i], tv[4 + i]));
        // reference maximum: moves only when the block maximum passes it by
        // more than 8 (p <= 2^8); a lane that keeps it keeps its bits
        mx = xmax4(mx);
        const bool grow = mx > m_run + 8.f;
        if (__any(grow)) {
            const float m_new = grow ? mx : m_run;
            const float alpha = grow ? fast_exp2(m_run - mx) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < DTW; ++dt) acc[dt] *= alpha;
            m_run = m_new;
        }
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
        float psum = 0.f;
        uint32_t ph[4], pm[4], pl[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            // B operand slots 2 k, 2 k + 1: slots 0..3 are keys 4 grp + i of
            // tile 0, slots 4..7 those of tile 1
            const float pa = fast_exp2(tv[2 * k] - m_use);
            const float pb = fast_exp2(tv[2 * k + 1] - m_use);
            psum += pa + pb;
            ph[k] = cvt_pk_bf16(pa, pb);
            const float ra = pa - bf16lo_to_f32(ph[k]);
            const float rb = pb - bf16hi_to_f32(ph[k]);
            pm[k] = cvt_pk_bf16(ra, rb);
            pl[k] = cvt_pk_bf16(ra - bf16lo_to_f32(pm[k]), rb - bf16hi_to_f32(pm[k]));
        }
        l_run += psum;
        const u32x4 bp[3] = {{ph[0], ph[1], ph[2], ph[3]}, {pm[0], pm[1], pm[2], pm[3]},
                             {pl[0], pl[1], pl[2], pl[3]}};

        // O^T += V^T . P^T in groups of VG d tiles: the group's products go
        // hi, mid, lo across its tiles (each accumulator's next product is VG
        // products later), the next group's reads beside them
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            if (gi + 1 < NG) {
#pragma unroll
                for (int e = 0; e < VG; ++e) va[(gi + 1) & 1][e] = rd_v((gi + 1) * VG + e);
            }
#pragma unroll
            for (int x = 0; x < 3; ++x)
#pragma unroll
                for (int e = 0; e < VG; ++e)
                    acc[gi * VG + e] = mfma_bf16_16x16x32(va[gi & 1][e], bp[x], acc[gi * VG + e]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    if constexpr (KP) {
        for (int j = jlo; j <= jhi; ++j) {
            // pair j has landed and every wave is done with pair j - 1, whose
            // stages take pair j + 1 (and, with PREP, the rotary table has
            // been read)
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            const int sp = ONEP ? 0 : 2 * ((j - jlo) & 1);
            if constexpr (PREP) {
                if (j == (b_slot >> 1) && b_slot >= 0) {
                    // the row's own key and value over the staged slot
                    // contents (over every row of the block with fill_all)
                    const int st = sp + (b_slot & 1);
                    const int n_fill = (fill_all ? WKB : 1) * 2 * (D / 8);
                    for (int idx = tid; idx < n_fill; idx += 256) {
                        const int r = fill_all ? idx / (2 * (D / 8)) : r_slot;
                        const int part = (idx / (D / 8)) & 1, piece = idx % (D / 8);
                        uint16_t* dst = (part ? vs[st] : ks[st]) + row_pos<D, WPAD>(r) + 8 * piece;
                        *reinterpret_cast<u32x4*>(dst) =
                            *reinterpret_cast<const u32x4*>(&kv_new[part][8 * piece]);
                    }
                    __syncthreads();
                }
            }
            if (!ONEP && j + 1 <= jhi) issue_pair(j + 1);
            const int b = 2 * j + set;
            if (b >= bb_lo && b <= bb_hi) block(b, sp + set, std::false_type{}, std::false_type{});
        }
    } else {
    for (int b = bb_lo; b <= bb_hi; ++b) {
        // block b has landed (every wave's share; only block b + 1's K, issued
        // last, may still be in flight), and every wave is done with block
        // b - 1's V stage
        if (K2 && b < bb_hi && (!PREP || b > bb_lo)) wait_vmcnt<NIW>();
        else __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if constexpr (PREP) {
            if (b == b_slot) {
                // the row's own key and value over the staged slot contents
                // (over every row of the block with fill_all: its other rows
                // were fetched from the slot being written)
                const int st = (b - bb_lo) & 1;
                const int n_fill = (fill_all ? WKB : 1) * 2 * (D / 8);
                for (int idx = tid; idx < n_fill; idx += 256) {
                    const int r = fill_all ? idx / (2 * (D / 8)) : r_slot;
                    const int part = (idx / (D / 8)) & 1, piece = idx % (D / 8);
                    uint16_t* dst = (part ? vs[st] : ks[st]) + row_pos<D, WPAD>(r) + 8 * piece;
                    *reinterpret_cast<u32x4*>(dst) =
                        *reinterpret_cast<const u32x4*>(&kv_new[part][8 * piece]);
                }
                __syncthreads();
            }
            if (K2 && b == bb_lo && bb_lo < bb_hi) {
                // the rotary table in the second K stage has been read
                uint32_t vo1[NIW];
                dma_plan(bb_lo + 1, vo1);
#pragma unroll
                for (int k = 0; k < NIW; ++k) dma_one(Kh, ks[1], vo1, k);
            }
        }
        const int st = (b - bb_lo) & 1;
        if (K2 && b + 1 < bb_hi) block(b, st, std::true_type{}, std::bool_constant<K2>{});
        else if (b < bb_hi) block(b, st, std::true_type{}, std::false_type{});
        else block(b, st, std::false_type{}, std::false_type{});
    }
    }
    }

    if constexpr (KP) {
        // the odd set hands its state to the even set through LDS (the
        // stages are free once every wave is past its last block); per lane
        // and element: M = max(m_even, m_odd), each set weighted by
        // 2^(m - M) (0 for a set with no attended key), the two terms added
        __syncthreads();
        float* xs = reinterpret_cast<float*>(&ks[0][0]);
        constexpr int XN = 4 * DTW + 2;
        float* xl = xs + dp * XN * 64 + lane;
        if (set == 1) {
#pragma unroll
            for (int dt = 0; dt < DTW; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) xl[(4 * dt + i) * 64] = acc[dt][i];
            xl[(4 * DTW) * 64] = m_run;
            xl[(4 * DTW + 1) * 64] = l_run;
        }
        __syncthreads();
        if (set == 0) {
#pragma clang fp contract(off)
            const float m1 = xl[(4 * DTW) * 64];
            const float l1 = xl[(4 * DTW + 1) * 64];
            const float M = fmaxf(m_run, m1);
            const float w0 = m_run == -INFINITY ? 0.f : fast_exp2(m_run - M);
            const float w1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - M);
#pragma unroll
            for (int dt = 0; dt < DTW; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float a0 = acc[dt][i] * w0;
                    const float a1 = xl[(4 * dt + i) * 64] * w1;
                    acc[dt][i] = a0 + a1;
                }
            const float l0w = l_run * w0;
            const float l1w = l1 * w1;
            l_run = l0w + l1w;
            m_run = M;
        }
    }
    // the waves that hold a column's final state (KP: the even set)
    const bool cvo = cv && set == 0;

    const float l_tot = xsum4(l_run);
    // lane holds d = dp D / DS + 16 dt + 4 grp + i of its column in acc[dt][i]
    const int dofs = dp * (D / DS) + 4 * grp;
    uint16_t* orow = out + (((size_t)s * R + (cv ? rr : 0)) * Hq + h) * D + dofs;
    auto store_out = [&](const f32x4 (&o)[DTW], float l) {
#pragma unroll
        for (int dt = 0; dt < DTW; ++dt) {
            uint32_t bb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                bb[i] = (l != 0.f || l != l) ? f32_to_bf16_bits(o[dt][i] / l) : 0u;
            *reinterpret_cast<u32x2*>(orow + 16 * dt) =
                u32x2{pack_bf16x2(bb[0], bb[1]), pack_bf16x2(bb[2], bb[3])};
        }
    };
    if constexpr (FUSE) {
        if (nrun == 1) {
            if (cvo) store_out(acc, l_tot);
            return;
        }
    }
    if (cvo) {
        if (dp == 0 && grp == 0) {
            part_ml[2 * pidx + 0] = m_run;
            part_ml[2 * pidx + 1] = l_tot;
        }
        float* dst = part_acc + pidx * D + dofs;
#pragma unroll
        for (int dt = 0; dt < DTW; ++dt) *reinterpret_cast<f32x4*>(dst + 16 * dt) = acc[dt];
    }
    if constexpr (FUSE) {
        // publish this run's partials, count the run; the last run's
        // workgroup merges (and leaves the counter at zero for the next call)
        // (the barrier orders every wave's stores before thread 0's release,
        // and thread 0's acquire before every wave's loads: one cache
        // write-back and one invalidate per workgroup)
        __shared__ int s_last;
        __syncthreads();
        if (tid == 0) {
            uint32_t* ctr = counters + ((size_t)s * Hkv + g) * CG + cgi;
            const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_ACQ_REL,
                                                        __HIP_MEMORY_SCOPE_AGENT);
            const int last = old == (uint32_t)(nrun - 1);
            if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_last = last;
        }
        __syncthreads();
        if (!s_last) return;
        if (!cvo) return;
        {
            // the merge kernel's arithmetic for nrun <= MW: M the largest run
            // maximum; each run's weighted sums round once (wt l and wt acc,
            // from zero) and add in ascending run order (the merge kernel's
            // waves hold one run or none, and adding its empty waves' zeros
            // changes nothing: no sum here is -0).  A run with m = -inf adds
            // zero (its partial holds zeros), so every load can go out at once
#pragma clang fp contract(off)
            const size_t base = (pidx - run);
            const float2* mlp = reinterpret_cast<const float2*>(part_ml) + base;
            float2 e[MW];
#pragma unroll
            for (int ci = 0; ci < MW; ++ci) e[ci] = mlp[min(ci, nrun - 1)];
            float M = -INFINITY;
#pragma unroll
            for (int ci = 0; ci < MW; ++ci) M = fmaxf(M, e[ci].x);
            // weights of the runs (0 for runs past nrun or with m = -inf)
            float wts[MW];
            float Lt = 0.f;
#pragma unroll
            for (int ci = 0; ci < MW; ++ci) {
                const bool use = ci < nrun && e[ci].x != -INFINITY;
                wts[ci] = use ? fast_exp2(e[ci].x - M) : 0.f;
                const float lw = wts[ci] * (use ? e[ci].y : 0.f);
                Lt = Lt + lw;
            }
            // d tiles in groups of DG, runs' accumulators loaded CB at a time
            constexpr int DG = DTW < 8 ? DTW : 8;
            constexpr int CB = 16 / DG;
#pragma unroll
            for (int d0 = 0; d0 < DTW; d0 += DG) {
                f32x4 ot[DG];
#pragma unroll
                for (int j = 0; j < DG; ++j) ot[j] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (M != -INFINITY) {
#pragma unroll
                    for (int c0 = 0; c0 < MW; c0 += CB) {
                        if (c0 >= nrun) break;
                        f32x4 av[CB][DG];
#pragma unroll
                        for (int u = 0; u < CB; ++u) {
                            const float* a = part_acc + (base + min(c0 + u, nrun - 1)) * D + dofs;
#pragma unroll
                            for (int j = 0; j < DG; ++j)
                                av[u][j] = *reinterpret_cast<const f32x4*>(a + 16 * (d0 + j));
                        }
#pragma unroll
                        for (int u = 0; u < CB; ++u) {
                            const int ci = c0 + u;
                            const bool use = ci < nrun && e[ci].x != -INFINITY;
#pragma unroll
                            for (int j = 0; j < DG; ++j)
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    const float ow = wts[ci] * (use ? av[u][j][i] : 0.f);
                                    ot[j][i] = ot[j][i] + ow;
                                }
                        }
                    }
                }
#pragma unroll
                for (int j = 0; j < DG; ++j) {
                    uint32_t bb[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        bb[i] = (Lt != 0.f || Lt != Lt) ? f32_to_bf16_bits(ot[j][i] / Lt) : 0u;
                    *reinterpret_cast<u32x2*>(orow + 16 * (d0 + j)) =
                        u32x2{pack_bf16x2(bb[0], bb[1]), pack_bf16x2(bb[2], bb[3])};
                }
            }
        }
    }
}

// Decode windows of four column tiles a workgroup (three or more tiles a
// window; fewer tiles go to the kernel above), in two roles on eight waves,
// two per SIMD, as the head-dim-512 prompt kernel splits its work: scorer w
// (waves 0-3) forms tile w's scores, reference maximum and probability
// pieces and hands the pieces and the rescale factor over through LDS; P.V
// wave w (waves 4-7) holds tile w's accumulator over all D dims and adds
// V^T . {hi, mid, lo} to it.  With one wave a SIMD a wave's K reads and
// softmax cannot hide behind its own products; here the scorer of block
// b + 1 and the P.V wave of block b share each SIMD.  A step is one
// barrier: scorers take block i + 1 (K(i + 1) in stage (i + 1) - lo,
// loading K(i + 2)) while the P.V waves take block i (V(i), loading
// V(i + 1)).  Every column's arithmetic is the kernel above's, step for step
// (the same score chains, the same lazy maximum, the same pieces, the same
// product order per accumulator; at head dim 256 its two block sets, the
// run's even and odd blocks, each with its own maximum, sum and
// accumulator, joined once at the end), so the bits are those of every
// other form and do not depend on the window width.
template <int D, bool NTL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_roles_kernel(const uint16_t* __restrict__ q,
                         const uint16_t* __restrict__ kc,
                         const uint16_t* __restrict__ vc,
                         const int32_t* __restrict__ pos,
                         float* __restrict__ part_acc,
                         float* __restrict__ part_ml,
                         int R, int Hq, int Hkv, int G, int RPT, int NT, int CG,
                         int n_items, int cap, int nrun, int run_slots, int ring, int window,
                         float c) {
    constexpr int QST = D / 32;                 // reduction steps of a score
    constexpr int DTW = D / 16;                 // 16-wide d tiles of a column
    constexpr int LPR = D / 8;                  // lanes moving one row per DMA
    constexpr int NIW = WKB * LPR / 64 / 4;     // DMA instructions per wave of a role per block
    constexpr int NSET = D == 256 ? 2 : 1;      // block sets (even and odd blocks at 256)
    constexpr int BLK = row_pos<D, WPAD>(WKB);
    constexpr int K16 = row_pos<D, WPAD>(16);
    constexpr int KPF = 4;                      // score steps of K reads in flight
    // d tiles per P.V group (at 256 the two sets' accumulators leave room for
    // fewer V^T operands in flight)
    constexpr int VG = D == 256 ? 2 : 4;
    constexpr int NG = DTW / VG;
    constexpr int DMA_K_EVERY = QST / NIW;      // K rows: one every few score products
    // V rows: half beside each of the first two P.V groups, so that they land
    // well before the step's end
    constexpr int DMA_V_GROUPS = 2;
    static_assert(DMA_K_EVERY * NIW == QST && NIW % DMA_V_GROUPS == 0 && DMA_V_GROUPS <= NG,
                  "DMA spread");

    __shared__ __attribute__((aligned(16))) uint16_t ks[2][BLK];
    __shared__ __attribute__((aligned(16))) uint16_t vs[2][BLK];
    __shared__ __attribute__((aligned(16))) u32x4 p_lds[2][4][3][64];   // P^T pieces
    __shared__ float a_lds[2][4][16];                                   // rescale factors
    __shared__ float j_lds[4][2][16];           // the block sets' weights (two sets)

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool scorer = wave < 4;
    const int rw = wave & 3;                    // the wave's column tile within the workgroup
    // the scorer's K reads and softmax gate the next step; its SIMD's P.V wave fills
    // the gaps (measured on 8 x 16 rows at 32k keys: 1-2% faster than equal priority)
    if (scorer) __builtin_amdgcn_s_setprio(1);
    const int lane = tid & 63;
    const int col = lane & 15;
    const int grp = lane >> 4;

    // workgroup -> item as in the kernel above
    const int L = blockIdx.x;
    const int cgi = (L >> 3) % CG;
    const int u = ((L >> 3) / CG) * 8 + (L & 7);
    if (u >= n_items) return;
    const int run = u % nrun;
    const int g = (u / nrun) % Hkv;
    const int s = u / (nrun * Hkv);

    const int ct = cgi * 4 + rw;
    const int rr = ct * RPT + col / G;
    const int h = g * G + col % G;
    const bool cv = ct < NT && col < RPT * G && rr < R;
    const int p0 = pos[s];
    const int t_col = cv ? p0 + rr : -1;
    const int r_lo = cgi * 4 * RPT;
    const int r_hi = min(R, (cgi + 1) * 4 * RPT) - 1;
    const int slot0 = run * run_slots;
    const RunKeys rk(cap, ring, window, slot0, p0 + r_lo, p0 + r_hi);
    const int t1 = rk.t1;
    const size_t pidx = (((size_t)s * R + (cv ? rr : 0)) * Hq + h) * (size_t)nrun + run;
    const int tcm = t_col >= 0 ? t_col % cap : 0;

    const int nslot = min(run_slots, cap - slot0);
    const int nblk = (nslot + WKB - 1) / WKB;
    int bb_lo, bb_hi;
    rk.blocks(nblk, lane, bb_lo, bb_hi);

    // a run with no attended key leaves an empty partial (m = -inf, l = 0)
    if (bb_hi < 0) {
        if (!cv) return;
        if (scorer) {
            if (grp == 0) {
                part_ml[2 * pidx + 0] = -INFINITY;
                part_ml[2 * pidx + 1] = 0.f;
            }
        } else {
            float* dst = part_acc + pidx * D + 4 * grp;
#pragma unroll
            for (int dt = 0; dt < DTW; ++dt)
                *reinterpret_cast<f32x4*>(dst + 16 * dt) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        return;
    }

    const size_t head_base = ((size_t)s * Hkv + g) * (size_t)cap * D;
    const uint16_t* Kh = kc + head_base;
    const uint16_t* Vh = vc + head_base;
    const int sub = ring ? t1 % cap : min(t1, cap - 1);     // t1 >= 0 here
    // DMA instruction i = rw + 4 k of a K or V block moves 1 KiB: block row
    // i at D = 512, rows 16 (i >> 3) + (i & 7) and + 8 at D = 256 (lanes
    // 0..31, 32..63); K by the scorers, V by the P.V waves
    int dma_row[NIW];
    int dma_dst[NIW];
    uint32_t dma_voff[NIW];
#pragma unroll
    for (int k = 0; k < NIW; ++k) {
        const int i = rw + 4 * k;
        const int r0 = (LPR == 64) ? i : 16 * (i >> 3) + (i & 7);
        dma_row[k] = (LPR == 64) ? r0 : r0 + 8 * (lane >> 5);
        dma_dst[k] = row_pos<D, WPAD>(r0);
        dma_voff[k] = (uint32_t)(dma_row[k] * D + (lane % LPR) * 8) * 2u;
    }
    auto dma_plan = [&](int b, uint32_t (&vo)[NIW]) {
        rk.dma_plan<D>(b, sub, dma_row, dma_voff, (lane % LPR) * 8, vo);
    };
    auto dma_one = [&](const uint16_t* base, uint16_t* stage, const uint32_t (&vo)[NIW], int k) {
        if constexpr (NTL) dma16_asm_sbase_nt(base, vo[k], lds_addr(stage + dma_dst[k]));
        else dma16_asm_sbase(base, vo[k], lds_addr(stage + dma_dst[k]));
    };
    auto step_sync = [&]() {
        __builtin_amdgcn_s_waitcnt(0);           // this wave's DMAs and LDS traffic
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    if (scorer) {
        // per block set: reference maximum and per-lane row sum
        float m_run[NSET], l_run[NSET];
#pragma unroll
        for (int e = 0; e < NSET; ++e) {
            m_run[e] = -INFINITY;
            l_run[e] = 0.f;
        }
        // Q^T operand: Q[column][32 st + 8 grp .. +7]
        u32x4 qreg[QST];
        const uint16_t* qrow = q + (((size_t)s * R + (cv ? rr : 0)) * Hq + h) * D + 8 * grp;
#pragma unroll
        for (int st = 0; st < QST; ++st) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            qreg[st] = cv ? ld16(qrow + 32 * st) : z;
        }
        const int kofs = row_pos<D, WPAD>(col) + 8 * grp;
        {
            uint32_t vo[NIW];
            dma_plan(bb_lo, vo);
#pragma unroll
            for (int k = 0; k < NIW; ++k) dma_one(Kh, ks[0], vo, k);
        }
        // block b with its set's maximum and sum
        auto score_block = [&](int b, float& m_cur, float& l_cur) {
            const int sb = (b - bb_lo) & 1;
            const bool more = b + 1 <= bb_hi;
            uint32_t kvo[NIW];
            if (more) dma_plan(b + 1, kvo);
            const bool nomask = rk.block_nomask(b);
            const uint16_t* kl = ks[sb];
            u32x4 kb[KPF][2];
#pragma unroll
            for (int j = 0; j < KPF; ++j) {
                kb[j][0] = ld16(kl + kofs + 32 * j);
                kb[j][1] = ld16(kl + K16 + kofs + 32 * j);
            }
            f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < QST; ++j) {
                s0 = mfma_bf16_16x16x32(kb[j % KPF][0], qreg[j], s0);
                s1 = mfma_bf16_16x16x32(kb[j % KPF][1], qreg[j], s1);
                if (j + KPF < QST) {
                    kb[j % KPF][0] = ld16(kl + kofs + 32 * (j + KPF));
                    kb[j % KPF][1] = ld16(kl + K16 + kofs + 32 * (j + KPF));
                }
                if (more && j % DMA_K_EVERY == 0) dma_one(Kh, ks[sb ^ 1], kvo, j / DMA_K_EVERY);
                __builtin_amdgcn_sched_barrier(0);
            }
            const int sbase = slot0 + b * WKB;
            float tv[8];
            float mx = -INFINITY;
            if (nomask) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    tv[e] = s0[e] * c;
                    tv[4 + e] = s1[e] * c;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool ok0 = rk.attended(sbase + 4 * grp + e, t_col, tcm, window);
                    const bool ok1 = rk.attended(sbase + 16 + 4 * grp + e, t_col, tcm, window);
                    tv[e] = ok0 ? s0[e] * c : -INFINITY;
                    tv[4 + e] = ok1 ? s1[e] * c : -INFINITY;
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fmaxf(tv[e], tv[4 + e]));
            // reference maximum: moves only when the block maximum passes it
            // by more than 8 (p <= 2^8); the factor goes to the P.V wave
            mx = xmax4(mx);
            const bool grow = mx > m_cur + 8.f;
            float alpha = 1.f;
            if (__any(grow)) {
                const float m_new = grow ? mx : m_cur;
                alpha = grow ? fast_exp2(m_cur - mx) : 1.f;
                l_cur *= alpha;
                m_cur = m_new;
            }
            const float m_use = (m_cur == -INFINITY) ? 0.f : m_cur;
            float psum = 0.f;
            uint32_t ph[4], pm[4], pl[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float pa = fast_exp2(tv[2 * k] - m_use);
                const float pb = fast_exp2(tv[2 * k + 1] - m_use);
                psum += pa + pb;
                ph[k] = cvt_pk_bf16(pa, pb);
                const float ra = pa - bf16lo_to_f32(ph[k]);
                const float rb = pb - bf16hi_to_f32(ph[k]);
                pm[k] = cvt_pk_bf16(ra, rb);
                pl[k] = cvt_pk_bf16(ra - bf16lo_to_f32(pm[k]), rb - bf16hi_to_f32(pm[k]));
            }
            l_cur += psum;
            p_lds[sb][rw][0][lane] = u32x4{ph[0], ph[1], ph[2], ph[3]};
            p_lds[sb][rw][1][lane] = u32x4{pm[0], pm[1], pm[2], pm[3]};
            p_lds[sb][rw][2][lane] = u32x4{pl[0], pl[1], pl[2], pl[3]};
            if (grp == 0) a_lds[sb][rw][col] = alpha;
        };
        // step k scores block bb_lo + k; the last step is the P.V waves'
        for (int b = bb_lo; b <= bb_hi; ++b) {
            step_sync();
            if (NSET == 2 && (b & 1)) score_block(b, m_run[NSET - 1], l_run[NSET - 1]);
            else score_block(b, m_run[0], l_run[0]);
        }
        step_sync();
        float m_fin = m_run[0], l_fin = l_run[0];
        if constexpr (NSET == 2) {
            // the two sets joined per lane: M = the larger maximum, each set
            // weighted by 2^(m - M) (0 for a set with no attended key); the
            // P.V wave applies the same weights to its two accumulators
#pragma clang fp contract(off)
            const float M = fmaxf(m_run[0], m_run[1]);
            const float w0 = m_run[0] == -INFINITY ? 0.f : fast_exp2(m_run[0] - M);
            const float w1 = m_run[1] == -INFINITY ? 0.f : fast_exp2(m_run[1] - M);
            const float l0w = l_run[0] * w0;
            const float l1w = l_run[1] * w1;
            l_fin = l0w + l1w;
            m_fin = M;
            if (grp == 0) {
                j_lds[rw][0][col] = w0;
                j_lds[rw][1][col] = w1;
            }
            step_sync();
        }
        const float l_tot = xsum4(l_fin);
        if (cv && grp == 0) {
            part_ml[2 * pidx + 0] = m_fin;
            part_ml[2 * pidx + 1] = l_tot;
        }
        return;
    }
    {
        // V^T operand as in the kernel above (one wave holds all D dims)
        const int vofs = row_pos<D, WPAD>(4 * grp + (col >> 2)) + 4 * (col & 3);
        f32x4 acc[NSET][DTW];
#pragma unroll
        for (int e = 0; e < NSET; ++e)
#pragma unroll
            for (int dt = 0; dt < DTW; ++dt) acc[e][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        // block i into its set's accumulator
        auto pv_block = [&](int i, f32x4 (&ac)[DTW]) {
            const bool more = i + 1 <= bb_hi;
            uint32_t vvo[NIW];
            if (more) dma_plan(i + 1, vvo);
            const int sn = (i + 1 - bb_lo) & 1;  // stage of V(i + 1)
            step_sync();
            const int sb = (i - bb_lo) & 1;
            const uint16_t* vl = vs[sb];
            auto rd_v = [&](int dt) -> u32x4 {
                const u32x2 x0 = lds_read_tr16(vl + vofs + 16 * dt);
                const u32x2 x1 = lds_read_tr16(vl + K16 + vofs + 16 * dt);
                return u32x4{x0.x, x0.y, x1.x, x1.y};
            };
            u32x4 va[2][VG];
#pragma unroll
            for (int e = 0; e < VG; ++e) va[0][e] = rd_v(e);
            const u32x4 bp[3] = {p_lds[sb][rw][0][lane], p_lds[sb][rw][1][lane],
                                 p_lds[sb][rw][2][lane]};
            const float alpha = a_lds[sb][rw][col];
            if (__any(alpha != 1.f)) {
#pragma unroll
                for (int dt = 0; dt < DTW; ++dt) ac[dt] *= alpha;
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                if (gi + 1 < NG) {
#pragma unroll
                    for (int e = 0; e < VG; ++e) va[(gi + 1) & 1][e] = rd_v((gi + 1) * VG + e);
                }
#pragma unroll
                for (int x = 0; x < 3; ++x)
#pragma unroll
                    for (int e = 0; e < VG; ++e)
                        ac[gi * VG + e] = mfma_bf16_16x16x32(va[gi & 1][e], bp[x], ac[gi * VG + e]);
                if (more && gi < DMA_V_GROUPS) {
#pragma unroll
                    for (int kk = 0; kk < NIW / DMA_V_GROUPS; ++kk)
                        dma_one(Vh, vs[sn], vvo, gi * (NIW / DMA_V_GROUPS) + kk);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // V(bb_lo) goes out while the scorers take block bb_lo; step k + 1
        // multiplies block bb_lo + k
        {
            uint32_t vo[NIW];
            dma_plan(bb_lo, vo);
#pragma unroll
            for (int k = 0; k < NIW; ++k) dma_one(Vh, vs[0], vo, k);
        }
        step_sync();
        for (int i = bb_lo; i <= bb_hi; ++i) {
            if (NSET == 2 && (i & 1)) pv_block(i, acc[NSET - 1]);
            else pv_block(i, acc[0]);
        }
        if constexpr (NSET == 2) {
            step_sync();                         // the scorer's set weights
            {
#pragma clang fp contract(off)
                const float w0 = j_lds[rw][0][col];
                const float w1 = j_lds[rw][1][col];
#pragma unroll
                for (int dt = 0; dt < DTW; ++dt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float a0 = acc[0][dt][i] * w0;
                        const float a1 = acc[1][dt][i] * w1;
                        acc[0][dt][i] = a0 + a1;
                    }
            }
        }
        if (!cv) return;
        float* dst = part_acc + pidx * D + 4 * grp;
#pragma unroll
        for (int dt = 0; dt < DTW; ++dt) *reinterpret_cast<f32x4*>(dst + 16 * dt) = acc[0][dt];
    }
}

// Merge of chunk partials in ascending chunk order.  A block of MW waves
// serves one (stream, head) and 64 VEC d (VEC per lane); wave w takes the
// contiguous chunk range [w nch / MW, (w + 1) nch / MW) in ascending order,
// then the waves' sums are added in ascending wave order.  M is the largest
// chunk maximum; chunks with no attended key (m = -inf) are skipped, never
// multiplied; out = bf16(sum e^(m_c - M) acc_c / sum e^(m_c - M) l_c), each
// weighted term added with one rounding (fmaf).  A wave loads MB chunks'
// partials before it adds them (in order), so that many loads are in flight,
// and its first MB go out before M is known (the loads do not depend on it);
// the d slice per block (VEC) only spreads the same per-element arithmetic
// over more blocks.  Registers stay within eight waves per SIMD, so two
// blocks share a CU.
template <int D, int VEC>
__global__ __launch_bounds__(64 * MW) __attribute__((amdgpu_waves_per_eu(8)))
void decode_merge_kernel(uint16_t* __restrict__ out,
                         const float* __restrict__ part_acc,
                         const float* __restrict__ part_ml,
                         int nch) {
    constexpr int MB = VEC == 4 ? 4 : 8;     // loads in flight per wave (two blocks a CU)
    static_assert(VEC == 1 || VEC == 2 || VEC == 4, "lane width");
    __shared__ float s_max[MW];
    __shared__ float s_l[MW];
    __shared__ __attribute__((aligned(16))) float s_o[MW][64 * VEC];
    const int sh = blockIdx.x;                 // s * Hq + h
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int d0 = blockIdx.y * (64 * VEC) + lane * VEC;
    const size_t base = (size_t)sh * (size_t)nch;
    const float2* ml = reinterpret_cast<const float2*>(part_ml) + base;
    const int c0 = (int)((long long)w * nch / MW);
    const int c1 = (int)((long long)(w + 1) * nch / MW);
    auto load = [&](int ci, float (&v)[VEC]) {
        const float* p = part_acc + (base + ci) * D + d0;
        if constexpr (VEC == 4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(p);
            v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
        } else if constexpr (VEC == 2) {
            const float2 x = *reinterpret_cast<const float2*>(p);
            v[0] = x.x; v[1] = x.y;
        } else {
            v[0] = *p;
        }
    };

    // the batch at cb: runs past c1 read as empty (m = -inf), never loaded
    float2 e[MB];
    float a[MB][VEC];
    auto fetch = [&](int cb) {
#pragma unroll
        for (int u = 0; u < MB; ++u) {
            if (cb + u < c1) {
                e[u] = ml[cb + u];
                load(cb + u, a[u]);
            } else {
                e[u] = float2{-INFINITY, 0.f};
#pragma unroll
                for (int i = 0; i < VEC; ++i) a[u][i] = 0.f;
            }
        }
    };
    fetch(c0);

    float mw = -INFINITY;
    for (int cidx = c0 + lane; cidx < c1; cidx += 64) mw = fmaxf(mw, ml[cidx].x);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mw = fmaxf(mw, __shfl_xor(mw, o));
    if (lane == 0) s_max[w] = mw;
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < MW; ++i) M = fmaxf(M, s_max[i]);

    float L = 0.f;
    float o[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) o[i] = 0.f;
    if (M != -INFINITY) {
        for (int cb = c0; cb < c1; cb += MB) {
            if (cb != c0) fetch(cb);
#pragma unroll
            for (int u = 0; u < MB; ++u) {
                if (e[u].x == -INFINITY) continue;
                const float wt = fast_exp2(e[u].x - M);
                L = fmaf(wt, e[u].y, L);
#pragma unroll
                for (int i = 0; i < VEC; ++i) o[i] = fmaf(wt, a[u][i], o[i]);
            }
        }
    }
    float* so = &s_o[w][lane * VEC];
    if constexpr (VEC == 4) *reinterpret_cast<f32x4*>(so) = f32x4{o[0], o[1], o[2], o[3]};
    else if constexpr (VEC == 2) *reinterpret_cast<float2*>(so) = float2{o[0], o[1]};
    else *so = o[0];
    if (lane == 0) s_l[w] = L;
    __syncthreads();
    if (w != 0) return;
    float Lt = 0.f;
    float ot[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) ot[i] = 0.f;
#pragma unroll 4
    for (int j = 0; j < MW; ++j) {
        Lt += s_l[j];
        const float* sj = &s_o[j][lane * VEC];
        float x[VEC];
        if constexpr (VEC == 4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(sj);
            x[0] = v[0]; x[1] = v[1]; x[2] = v[2]; x[3] = v[3];
        } else if constexpr (VEC == 2) {
            const float2 v = *reinterpret_cast<const float2*>(sj);
            x[0] = v.x; x[1] = v.y;
        } else {
            x[0] = *sj;
        }
#pragma unroll
        for (int i = 0; i < VEC; ++i) ot[i] += x[i];
    }
    uint32_t bb[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i)
        bb[i] = (Lt != 0.f || Lt != Lt) ? f32_to_bf16_bits(ot[i] / Lt) : 0u;
    uint16_t* orow = out + (size_t)sh * D + d0;
    if constexpr (VEC == 4) {
        *reinterpret_cast<u32x2*>(orow) = u32x2{pack_bf16x2(bb[0], bb[1]), pack_bf16x2(bb[2], bb[3])};
    } else if constexpr (VEC == 2) {
        *reinterpret_cast<uint32_t*>(orow) = pack_bf16x2(bb[0], bb[1]);
    } else {
        *orow = (uint16_t)bb[0];
    }
}

// Merge of at most MW runs: the merge kernel's arithmetic with one wave per
// (stream, head) and d slice.  There each wave holds one run or none, its
// sum being the run's weighted terms rounded once (fmaf from +0), and the
// waves' sums add in ascending order.  A sum that starts at +0 is never -0,
// so adding an empty wave's +0 changes nothing: here each run's terms add in
// ascending run order directly, every run's loads in flight at once and no
// exchange through LDS.
template <int D>
__global__ __launch_bounds__(64)
void decode_merge_few_kernel(uint16_t* __restrict__ out,
                             const float* __restrict__ part_acc,
                             const float* __restrict__ part_ml,
                             int nch) {
#pragma clang fp contract(off)
    const int sh = blockIdx.x;                 // s * Hq + h
    const int lane = threadIdx.x;
    const int d0 = blockIdx.y * 256 + lane * 4;
    const size_t base = (size_t)sh * (size_t)nch;
    const float2* ml = reinterpret_cast<const float2*>(part_ml) + base;
    float2 e[MW];
    f32x4 a[MW];
#pragma unroll
    for (int c = 0; c < MW; ++c) {
        if (c < nch) {
            e[c] = ml[c];
            a[c] = *reinterpret_cast<const f32x4*>(part_acc + (base + c) * D + d0);
        } else {
            e[c] = float2{-INFINITY, 0.f};
            a[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    float M = -INFINITY;
#pragma unroll
    for (int c = 0; c < MW; ++c) M = fmaxf(M, e[c].x);
    float Lt = 0.f;
    f32x4 ot = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
#pragma unroll
        for (int c = 0; c < MW; ++c) {
            if (e[c].x == -INFINITY) continue;
            const float wt = fast_exp2(e[c].x - M);
            Lt = Lt + fmaf(wt, e[c].y, 0.f);
#pragma unroll
            for (int i = 0; i < 4; ++i) ot[i] = ot[i] + fmaf(wt, a[c][i], 0.f);
        }
    }
    uint32_t bb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        bb[i] = (Lt != 0.f || Lt != Lt) ? f32_to_bf16_bits(ot[i] / Lt) : 0u;
    uint16_t* orow = out + (size_t)sh * D + d0;
    *reinterpret_cast<u32x2*>(orow) = u32x2{pack_bf16x2(bb[0], bb[1]), pack_bf16x2(bb[2], bb[3])};
}

}  // namespace

size_t decode_workspace_bytes(int S, int Hq, int D, int cap) {
    // one partial per chunk, or per run where runs are shorter (half chunks)
    const size_t nch = ((size_t)cap + CHUNK - 1) / CHUNK;
    const size_t nrun = (size_t)decode_run_count(cap);
    return (size_t)S * Hq * (nrun > nch ? nrun : nch) * ((size_t)D + 2) * sizeof(float);
}

size_t decode_partials_bytes(int S, int Hq, int D, int cap) {
    const size_t nrun = (size_t)decode_run_count(cap);
    return (size_t)S * Hq * nrun * ((size_t)D + 2) * sizeof(float);
}

hipError_t launch_decode(uint16_t* out, const uint16_t* q, const uint16_t* kc,
                         const uint16_t* vc, const int32_t* pos, int S, int Hq,
                         int Hkv, int D, int cap, int ring, int window,
                         float scale, void* ws, hipStream_t stream) {
    // one row per stream is a window of one row: the same kernel and bits
    return launch_decode_rows(out, q, kc, vc, pos, S, 1, Hq, Hkv, D, cap, ring, window, scale,
                              ws, false, nullptr, stream);
}

static hipError_t launch_decode_merge(uint16_t* out, const float* part_acc, const float* part_ml,
                               int n_rows_heads, int D, int nrun, hipStream_t stream) {
    // narrow d slices when few (stream, head) rows carry many runs each, so
    // the merge still spreads over the chip
    const long long wide = (long long)n_rows_heads * (D / 256);
    const int vec = (nrun < 64 || wide >= 512) ? 4 : (2 * wide >= 512 ? 2 : 1);
    const dim3 g2(n_rows_heads, D / (64 * vec));
    if (nrun <= MW) {
        // at most MW runs: one wave per (stream, head) and 256-wide d slice
        // (vec is 4 here)
        if (D == 256)
            decode_merge_few_kernel<256><<<g2, 64, 0, stream>>>(out, part_acc, part_ml, nrun);
        else
            decode_merge_few_kernel<512><<<g2, 64, 0, stream>>>(out, part_acc, part_ml, nrun);
        return hipGetLastError();
    }
#define MERGE_LAUNCH(DD, VV) \
    decode_merge_kernel<DD, VV><<<g2, 64 * MW, 0, stream>>>(out, part_acc, part_ml, nrun)
    if (D == 256) {
        if (vec == 4) MERGE_LAUNCH(256, 4);
        else if (vec == 2) MERGE_LAUNCH(256, 2);
        else MERGE_LAUNCH(256, 1);
    } else {
        if (vec == 4) MERGE_LAUNCH(512, 4);
        else if (vec == 2) MERGE_LAUNCH(512, 2);
        else MERGE_LAUNCH(512, 1);
    }
#undef MERGE_LAUNCH
    return hipGetLastError();
}

hipError_t launch_decode_rows(uint16_t* out, const uint16_t* q, const uint16_t* kc,
                              const uint16_t* vc, const int32_t* pos, int S, int R, int Hq,
                              int Hkv, int D, int cap, int ring, int window, float scale,
                              void* ws, bool fused, const PrepArgs* prep, hipStream_t stream) {
    const int G = Hq / Hkv;
    const int RPT = 16 / G;                      // rows per 16-column tile
    const int NT = (R + RPT - 1) / RPT;          // column tiles of a window
    const int run_slots = decode_run_slots(cap);
    const int nrun = decode_run_count(cap);
    // one launch when the merge fits a workgroup (at most MW runs); the
    // counters sit at the start of a fused call's workspace
    const bool one = fused && nrun <= MW;
    // windows of three or more tiles: four tiles a workgroup, eight waves in
    // two roles (three tiles leave a scorer and a P.V wave idle); at head dim
    // 256 only while that still gives 128 workgroups or more (a tile a
    // workgroup spreads a small window wider).  Otherwise four waves: at head
    // dim 512 one tile split four ways over d, two tiles two ways (or four
    // tiles in the single launch); at head dim 256 one tile, two block sets
    // by two d halves.  Every form gives the same bits.
    const long long n_items = (long long)nrun * Hkv * S;
    const bool roles = !one && !prep && NT >= 3 &&
                       (D == 512 || n_items * ((NT + 3) / 4) >= 128);
    const int DS = D == 256 ? 2 : (NT == 1 ? 4 : (NT == 2 ? 2 : 1));
    const int WC = roles ? 4 : (D == 256 ? 1 : 4 / DS);
    const int CG = (NT + WC - 1) / WC;           // workgroups per item
    const long long nwg = (n_items + 7) / 8 * 8 * CG;
    if (nwg > 0x7FFFFFFFLL || (long long)S * R * Hq > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    uint32_t* counters = reinterpret_cast<uint32_t*>(ws);
    float* part_acc = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                               (fused ? ATTN_DECODE_COUNTER_BYTES : 0));
    float* part_ml = part_acc + (size_t)S * R * Hq * nrun * D;
    const float c = scale * ATTN_LOG2E;
    const PrepArgs pa = prep ? *prep : PrepArgs{};
    // K/V bytes the launch can read: each stream's window (plus the rows
    // below its last) or its whole cache, per KV head
    const long long span = window > 0 ? std::min<long long>(cap, (long long)window + R - 1) : cap;
    const bool ntl = (double)S * Hkv * span * D * 4.0 > (double)DECODE_STREAM_BYTES;
#define ROWS_LAUNCH(DD, SS, FF, PP)                                                           \
    do {                                                                                      \
        if (ntl) ROWS_LAUNCH_NT(DD, SS, FF, PP, true);                                        \
        else ROWS_LAUNCH_NT(DD, SS, FF, PP, false);                                           \
    } while (0)
#define ROWS_LAUNCH_NT(DD, SS, FF, PP, NN)                                                    \
    decode_rows_kernel<DD, SS, FF, PP, NN><<<(unsigned)nwg, 256, 0, stream>>>(                \
        q, kc, vc, pos, part_acc, part_ml, out, counters, R, Hq, Hkv, G, RPT, NT, CG,         \
        (int)n_items, cap, nrun, run_slots, ring, window, c, pa)
#define ROWS_DS(DD, FF)                                                                       \
    do {                                                                                      \
        if (prep) ROWS_LAUNCH(DD, 4, FF, true);                                               \
        else if (DS == 4) ROWS_LAUNCH(DD, 4, FF, false);                                      \
        else if (DS == 2) ROWS_LAUNCH(DD, 2, FF, false);                                      \
        else ROWS_LAUNCH(DD, 1, FF, false);                                                   \
    } while (0)
    if (prep && R != 1) return hipErrorInvalidValue;       // the prologue serves one row
    // head dim 256, runs of one block pair: the two-stage form
#define ROWS_ONEP(FF)                                                                         \
    do {                                                                                      \
        if (ntl) decode_rows_kernel<256, 2, FF, false, true, true><<<(unsigned)nwg, 256, 0, stream>>>( \
            q, kc, vc, pos, part_acc, part_ml, out, counters, R, Hq, Hkv, G, RPT, NT, CG,     \
            (int)n_items, cap, nrun, run_slots, ring, window, c, pa);                         \
        else decode_rows_kernel<256, 2, FF, false, false, true><<<(unsigned)nwg, 256, 0, stream>>>( \
            q, kc, vc, pos, part_acc, part_ml, out, counters, R, Hq, Hkv, G, RPT, NT, CG,     \
            (int)n_items, cap, nrun, run_slots, ring, window, c, pa);                         \
    } while (0)
#define ROLES_LAUNCH(DD)                                                                      \
    do {                                                                                      \
        if (ntl) decode_roles_kernel<DD, true><<<(unsigned)nwg, 512, 0, stream>>>(            \
            q, kc, vc, pos, part_acc, part_ml, R, Hq, Hkv, G, RPT, NT, CG, (int)n_items, cap, \
            nrun, run_slots, ring, window, c);                                                \
        else decode_roles_kernel<DD, false><<<(unsigned)nwg, 512, 0, stream>>>(               \
            q, kc, vc, pos, part_acc, part_ml, R, Hq, Hkv, G, RPT, NT, CG, (int)n_items, cap, \
            nrun, run_slots, ring, window, c);                                                \
    } while (0)
    const bool onep = run_slots <= 2 * WKB && !prep;
    if (roles) {
        if (D == 256) ROLES_LAUNCH(256);
        else ROLES_LAUNCH(512);
    } else if (D == 256) {
        if (one) {
            if (prep) ROWS_LAUNCH(256, 2, true, true);
            else if (onep) ROWS_ONEP(true);
            else ROWS_LAUNCH(256, 2, true, false);
        } else {
            if (prep) ROWS_LAUNCH(256, 2, false, true);
            else if (onep) ROWS_ONEP(false);
            else ROWS_LAUNCH(256, 2, false, false);
        }
    } else {
        if (one) ROWS_DS(512, true);
        else ROWS_DS(512, false);
    }
#undef ROLES_LAUNCH
#undef ROWS_ONEP
#undef ROWS_DS
#undef ROWS_LAUNCH
#undef ROWS_LAUNCH_NT
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || one) return e;
    return launch_decode_merge(out, part_acc, part_ml, S * R * Hq, D, nrun, stream);
}

namespace {

// zero fill of a fused decode's counter area (a kernel, so a graph may hold it)
__global__ void zero_words_kernel(uint32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

}  // namespace

hipError_t launch_decode_counters_init(void* ws, hipStream_t stream) {
    constexpr int n = ATTN_DECODE_COUNTER_BYTES / 4;
    zero_words_kernel<<<(n + 255) / 256, 256, 0, stream>>>(static_cast<uint32_t*>(ws), n);
    return hipGetLastError();
}

// Standalone prologue: grid (S, ceil(Hq / 16) + 2 Hkv), one wave each: unit u
// < ceil(Hq / 16) norms and rotates 16 query heads into q_out; the next Hkv
// units write the rotated keys, the last Hkv the values, at the row's slot
// (skipped when the row's position has no slot: t < 0, or t >= cap linear).
namespace {

template <int D>
__global__ __launch_bounds__(64)
void qkv_prep_kernel(uint16_t* __restrict__ q_out, PrepArgs pa, const int32_t* __restrict__ pos,
                     int Hq, int Hkv, int cap, int ring) {
    __shared__ float cs[D];
    const int s = blockIdx.x;
    const int u = blockIdx.y;
    const int lane = threadIdx.x;
    const int col = lane & 15, grp = lane >> 4;
    const int t = pos[s];
    const int QT = (Hq + 15) / 16;
    rope_table<D>(cs, pa.inv_freq, t, lane, 64);
    __syncthreads();
    u32x4 x[D / 32];
    if (u < QT) {
        const int h = u * 16 + col;
        const bool ok = h < Hq;
        load_row<D>(x, pa.qkv + ((size_t)s * (Hq + 2 * Hkv) + (ok ? h : 0)) * D, grp, ok);
        norm_row<D>(x, pa.q_w, grp, pa.eps);
        rope_row<D>(x, cs, grp);
        if (ok) store_row<D>(q_out + ((size_t)s * Hq + h) * D, x, grp);
        return;
    }
    if (t < 0 || (!ring && t >= cap)) return;
    const int slot = ring ? t % cap : t;
    const int g = (u - QT) % Hkv;
    const int part = (u - QT) / Hkv;
    load_kv<D>(x, pa, s, g, Hq, Hkv, lane, part);
    norm_kv<D>(x, pa, lane, part);
    rope_store_kv<D>(x, pa, (((size_t)s * Hkv + g) * cap + slot) * D, cs, lane, part, nullptr);
}

}  // namespace

hipError_t launch_qkv_prep(uint16_t* q_out, const PrepArgs& pa, const int32_t* pos, int S,
                           int Hq, int Hkv, int D, int cap, int ring, hipStream_t stream) {
    const dim3 grid(S, (Hq + 15) / 16 + 2 * Hkv);
    if (D == 256)
        qkv_prep_kernel<256><<<grid, 64, 0, stream>>>(q_out, pa, pos, Hq, Hkv, cap, ring);
    else
        qkv_prep_kernel<512><<<grid, 64, 0, stream>>>(q_out, pa, pos, Hq, Hkv, cap, ring);
    return hipGetLastError();
}
