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
                           int Hq, int Hkv, int G, int cap, int nrun, int cpr,
                           int ring, int window, float c) {
    constexpr int QST = D / 32;       // 32-wide reduction steps of Q.K
    constexpr int SPANS = D / 128;    // 128-wide d spans of the accumulator
    constexpr int LPR = D / 8;        // lanes that move one K row per DMA
    constexpr int RPD = 64 / LPR;     // K rows per DMA instruction
    const int run = blockIdx.x;
    const int g = blockIdx.y;
    const int s = blockIdx.z;
    const int lane = threadIdx.x;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int t = pos[s];

    // K tiles land here by direct global->LDS loads, two stages
    __shared__ __attribute__((aligned(16))) uint16_t ks[2][TILE * D];

    const size_t head_base = ((size_t)s * Hkv + g) * (size_t)cap;
    const uint16_t* K = kc + head_base * D;
    const uint16_t* V = vc + head_base * D;
    const int h0 = g * G;
    const size_t pbase = ((size_t)s * Hq + h0) * (size_t)nrun + run;
    const int slot0 = run * cpr * CHUNK;
    const int nslot = min(cpr * CHUNK, cap - slot0);
    const int ntile = (nslot + TILE - 1) / TILE;

    // attended tiles of this run: [tt_lo, tt_hi]; a run with none writes an
    // empty partial (m = -inf, l = 0) that the merge skips
    int tt_lo = 0x7FFFFFFF, tt_hi = -1;
    for (int tb = 0; tb < ntile; tb += 16) {
        bool mine = false;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            mine |= slot_attended(slot0 + (tb + lane / 4) * TILE + 4 * (lane & 3) + i, t, cap, ring, window);
        const uint64_t bal = __ballot(mine);     // lane covers tile tb + lane / 4
        if (bal != 0) {
            tt_lo = min(tt_lo, tb + __builtin_ctzll(bal) / 4);
            tt_hi = tb + (63 - __builtin_clzll(bal)) / 4;
        }
    }
    if (tt_hi < 0) {
        if (col < G && grp == 0) {
            part_ml[2 * (pbase + (size_t)col * nrun) + 0] = -INFINITY;
            part_ml[2 * (pbase + (size_t)col * nrun) + 1] = 0.f;
        }
        return;
    }

    // Q^T operand: lane holds Q[head col][32 st + 8 grp .. +7]
    u32x4 qreg[QST];
    {
        const bool hv = col < G;
        const uint16_t* qrow = q + ((size_t)s * Hq + h0 + (hv ? col : 0)) * D;
#pragma unroll
        for (int st = 0; st < QST; ++st) {
            u32x4 z = {0u, 0u, 0u, 0u};
            qreg[st] = hv ? ld16(qrow + 32 * st + 8 * grp) : z;
        }
        // Q lives in AGPRs (the score products read their B operand there),
        // leaving the VGPRs to the accumulator and two tiles of V
#pragma unroll
        for (int st = 0; st < QST; ++st) asm volatile("" : "+a"(qreg[st]));
    }

    f32x4 acc[SPANS][8];
#pragma unroll
    for (int sp = 0; sp < SPANS; ++sp)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[sp][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // K tile: each DMA instruction moves 1 KiB of whole rows (one row at
    // D=512, two at 256).  16-byte chunk c of row r sits at chunk c ^ (r & 7)
    // of its LDS row, so the eight lanes of one LDS read phase (eight rows,
    // same chunk) hit eight different bank groups.  The slot is clamped in
    // range; a key that is not attended is masked out of the scores.
    // (issued from asm, one instruction at a time between the score
    // products: the compiler then adds no wait for it before the LDS reads
    // of the other stage; the tile loop waits for it explicitly)
    auto load_k_one = [&](int sb, int stage, int i) {
        const int row = i * RPD + lane / LPR;
        const int slot = min(sb + row, cap - 1);
        const int chunk = (lane % LPR) ^ (row & 7);
        dma16_asm(K + (size_t)slot * D + chunk * 8, lds_addr(&ks[stage][i * RPD * D]));
    };
    auto load_k = [&](int sb, int stage) {
#pragma unroll
        for (int i = 0; i < TILE / RPD; ++i) load_k_one(sb, stage, i);
    };
    // V rows (sb + 4 grp + r), d = 128 sp + 8 col .. +7: sixteen lanes read
    // 256 contiguous bytes of one row per load
    u32x4 vbuf0[4][SPANS];
    u32x4 vbuf1[4][SPANS];
    auto load_v = [&](int sb, u32x4 (&dst)[4][SPANS]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int slot = min(sb + 4 * grp + r, cap - 1);
            const uint16_t* vrow = V + (size_t)slot * D + 8 * col;
#pragma unroll
            for (int sp = 0; sp < SPANS; ++sp) dst[r][sp] = ld16(vrow + 128 * sp);
        }
    };

    float m_run = -INFINITY;
    float l_run = 0.f;

    // One 16-key tile; V of this tile in vc, the next tile's V goes to vn.
    static_assert(TILE / RPD == QST, "one K DMA instruction per score product");
    auto tile = [&](int tt, const u32x4 (&vc)[4][SPANS], u32x4 (&vn)[4][SPANS]) {
        const int stage = (tt - tt_lo) & 1;
        const int sb = slot0 + tt * TILE;
        const bool more = tt < tt_hi;
        // K(tt) in LDS and V(tt) in registers have landed
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (more) load_v(sb + TILE, vn);         // in flight through this tile

        // scores: the two halves of the head dim accumulate separately (two
        // independent product chains) and are added at the end; the next
        // tile's K moves in beside them, one DMA instruction per product
        const uint16_t* kt = &ks[stage][0];
        f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < QST; ++st) {
            const u32x4 kop = ld16(kt + col * D + 8 * ((4 * st + grp) ^ (col & 7)));
            if (st < QST / 2) sa = mfma_bf16_16x16x32(kop, qreg[st], sa);
            else sb2 = mfma_bf16_16x16x32(kop, qreg[st], sb2);
            if (more) load_k_one(sb + TILE, stage ^ 1, st);
        }
        const f32x4 sc = sa + sb2;

        float tv[4];
        uint32_t vmask[4], vsel[4];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = slot_attended(sb + 4 * grp + i, t, cap, ring, window);
            tv[i] = ok ? sc[i] * c : -INFINITY;
            mx = fmaxf(mx, tv[i]);
            // bf16 -> fp32 of V with unattended keys forced to +0 (a NaN
            // there must not meet its zero probability)
            vmask[i] = ok ? 0xFFFF0000u : 0u;
            vsel[i] = ok ? 0x01000C0Cu : 0x0C0C0C0Cu;
        }
        // Reference maximum.  Decode keeps p in fp32 and never rounds it
        // against the maximum, so the maximum only keeps exp2 in range: it
        // moves (and the accumulator is rescaled) only when a tile's maximum
        // passes it by more than 8, so p <= 2^8 and a run's row sum stays
        // below 2^18, far inside fp32; the partial carries the reference it
        // used, which the merge takes as the chunk maximum.
        mx = xmax4(mx);
        const bool grow = mx > m_run + 8.f;       // first attended tile: m_run = -inf
        if (__any(grow)) {
            const float m_new = grow ? mx : m_run;
            // 0 when growing from -inf; exactly 1 for a lane that keeps its
            // reference (also one still at -inf, where the difference is NaN)
            const float alpha = grow ? fast_exp2(m_run - mx) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int sp = 0; sp < SPANS; ++sp)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[sp][j] *= alpha;
            m_run = m_new;
        }
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
        float pv[4];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pv[i] = fast_exp2(tv[i] - m_use);              // 0 for masked keys
            psum += pv[i];
        }
        l_run += psum;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int sp = 0; sp < SPANS; ++sp) {
                const u32x4 w = vc[r][sp];
                const float p = pv[r];
                const uint32_t sl = vsel[r], mk = vmask[r];
#define LO(x) __uint_as_float(__builtin_amdgcn_perm(0u, (x), sl))
#define HI(x) __uint_as_float((x) & mk)
                acc[sp][0] = mfma_f32_16x16x4(LO(w.x), p, acc[sp][0]);
                acc[sp][1] = mfma_f32_16x16x4(HI(w.x), p, acc[sp][1]);
                acc[sp][2] = mfma_f32_16x16x4(LO(w.y), p, acc[sp][2]);
                acc[sp][3] = mfma_f32_16x16x4(HI(w.y), p, acc[sp][3]);
                acc[sp][4] = mfma_f32_16x16x4(LO(w.z), p, acc[sp][4]);
                acc[sp][5] = mfma_f32_16x16x4(HI(w.z), p, acc[sp][5]);
                acc[sp][6] = mfma_f32_16x16x4(LO(w.w), p, acc[sp][6]);
                acc[sp][7] = mfma_f32_16x16x4(HI(w.w), p, acc[sp][7]);
#undef LO
#undef HI
            }
        }
    };

    load_k(slot0 + tt_lo * TILE, 0);
    load_v(slot0 + tt_lo * TILE, vbuf0);
    for (int tt = tt_lo; tt <= tt_hi; ++tt) {
        tile(tt, vbuf0, vbuf1);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int sp = 0; sp < SPANS; ++sp) vbuf0[r][sp] = vbuf1[r][sp];
    }

    const float l_tot = xsum4(l_run);
    if (col >= G) return;
    const size_t pidx = pbase + (size_t)col * nrun;
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

// Merge of chunk partials in ascending chunk order.  A block of MW waves
// serves one (stream, head) and 256 d (four per lane); wave w takes the
// contiguous chunk range [w nch / MW, (w + 1) nch / MW) in ascending order,
// then the waves' sums are added in ascending wave order.  M is the largest
// chunk maximum; chunks with no attended key (m = -inf) are skipped, never
// multiplied; out = bf16(sum e^(m_c - M) acc_c / sum e^(m_c - M) l_c).
constexpr int MW = 16;

template <int D>
__global__ __launch_bounds__(64 * MW)
void decode_merge_kernel(uint16_t* __restrict__ out,
                         const float* __restrict__ part_acc,
                         const float* __restrict__ part_ml,
                         int Hq, int nch) {
    __shared__ float s_max[MW];
    __shared__ float s_l[MW];
    __shared__ f32x4 s_o[MW][64];
    const int sh = blockIdx.x;                 // s * Hq + h
    const int d0 = blockIdx.y * 256 + (threadIdx.x & 63) * 4;
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const size_t base = (size_t)sh * (size_t)nch;
    const float2* ml = reinterpret_cast<const float2*>(part_ml) + base;
    const int c0 = (int)((long long)w * nch / MW);
    const int c1 = (int)((long long)(w + 1) * nch / MW);

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
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
        int cidx = c0;
        for (; cidx + 4 <= c1; cidx += 4) {
            f32x4 a[4];
            float2 e[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                e[u] = ml[cidx + u];
                a[u] = *reinterpret_cast<const f32x4*>(part_acc + (base + cidx + u) * D + d0);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (e[u].x == -INFINITY) continue;
                const float wt = fast_exp2(e[u].x - M);
                L += wt * e[u].y;
                o += wt * a[u];
            }
        }
        for (; cidx < c1; ++cidx) {
            const float2 e = ml[cidx];
            if (e.x == -INFINITY) continue;
            const float wt = fast_exp2(e.x - M);
            L += wt * e.y;
            o += wt * *reinterpret_cast<const f32x4*>(part_acc + (base + cidx) * D + d0);
        }
    }
    s_o[w][lane] = o;
    if (lane == 0) s_l[w] = L;
    __syncthreads();
    if (w != 0) return;
    float Lt = 0.f;
    f32x4 ot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < MW; ++i) {
        Lt += s_l[i];
        ot += s_o[i][lane];
    }
    uint32_t b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = (Lt != 0.f || Lt != Lt) ? f32_to_bf16_bits(ot[i] / Lt) : 0u;
    u32x2 packed = {pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
    *reinterpret_cast<u32x2*>(out + (size_t)sh * D + d0) = packed;
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
    // a workgroup carries its softmax over a run of consecutive chunks; runs
    // of two when there are chunks for more than one wave per SIMD
    const long long waves = (long long)nch * Hkv * S;
    const int cpr = waves > 1536 ? 2 : 1;
    const int nrun = (nch + cpr - 1) / cpr;
    const int G = Hq / Hkv;
    float* part_acc = reinterpret_cast<float*>(ws);
    float* part_ml = part_acc + (size_t)S * Hq * nrun * D;
    const float c = scale * ATTN_LOG2E;
    dim3 g1(nrun, Hkv, S);
    dim3 g2(S * Hq, D / 256);
    if (D == 256) {
        decode_partial_kernel<256><<<g1, 64, 0, stream>>>(q, kc, vc, pos, part_acc, part_ml,
                                                          Hq, Hkv, G, cap, nrun, cpr, ring, window, c);
        decode_merge_kernel<256><<<g2, 64 * MW, 0, stream>>>(out, part_acc, part_ml, Hq, nrun);
    } else {
        decode_partial_kernel<512><<<g1, 64, 0, stream>>>(q, kc, vc, pos, part_acc, part_ml,
                                                          Hq, Hkv, G, cap, nrun, cpr, ring, window, c);
        decode_merge_kernel<512><<<g2, 64 * MW, 0, stream>>>(out, part_acc, part_ml, Hq, nrun);
    }
    return hipGetLastError();
}
