// Decode prologue of a stacked projection row, shared by the standalone
// prologue kernel and the decode kernel that runs it in place, so that both
// produce the same bits.
//
// Method: TensorFold PR #1183, squashed commit bodies (the qk_rows note): q
// and k are normed as bf16(w * bf16(x * inv)) with inv = 1 / sqrt(mean(x^2) +
// eps), then rotated; v may be normed by a unit RMS norm (bf16(x * inv)).
// PR #975, decode attention commits: the decode kernel norms and ropes its
// query heads from the stacked row and the workgroup holding the row's slot
// writes its key and value to the cache.
//
// Layout: a head row sits in the lanes of one matrix-core column, as the
// decode kernel's Q operand: lane (col, grp) holds elements 32 st + 8 grp ..
// +7 in x[st] (eight bf16 in a u32x4).  The rotary pairs are (i, i + D/2),
// i.e. x[st] and x[st + D/64] of the same lane; the angle of pair i is
// fp32(fp32(t) * inv_freq[i]), its cosine and sine taken once per row into
// an LDS table.
#pragma once

#include "common.h"

struct PrepArgs {
    const uint16_t* qkv;        // [S][(Hq + 2 Hkv) D] stacked rows (bf16)
    const uint16_t* q_w;        // [D] q norm scale (bf16)
    const uint16_t* k_w;        // [D] k norm scale (bf16)
    const float* inv_freq;      // [D/2] rotary frequencies
    float eps;
    int v_norm;                 // 1: v <- bf16(v * inv); 0: v as given
    uint16_t* kc;               // caches written at the row's slot
    uint16_t* vc;
};

ATTN_DEV float bf16_elem(const u32x4& v, int j) {
    const uint32_t w = v[j >> 1];
    return (j & 1) ? bf16hi_to_f32(w) : bf16lo_to_f32(w);
}

// cos and sin of the row's D/2 angles: cs[i] = cos, cs[D/2 + i] = sin
template <int D>
ATTN_DEV void rope_table(float* cs, const float* inv_freq, int t, int tid, int nthreads) {
    const float ft = (float)t;
    for (int i = tid; i < D / 2; i += nthreads) {
        const float a = ft * inv_freq[i];
        float s, c;
        sincosf(a, &s, &c);
        cs[i] = c;
        cs[D / 2 + i] = s;
    }
}

// RMS norm of the column's row in place: bf16(w * bf16(x * inv)), or
// bf16(x * inv) without w.  The sum of squares runs over the lane's
// elements in order, then over the column's four lanes (xsum4).
template <int D>
ATTN_DEV void norm_row(u32x4 (&x)[D / 32], const uint16_t* w, int grp, float eps) {
    constexpr int QST = D / 32;
    float ss = 0.f;
#pragma unroll
    for (int st = 0; st < QST; ++st)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float v = bf16_elem(x[st], j);
            ss = fmaf(v, v, ss);
        }
    ss = xsum4(ss);
    const float inv = 1.f / sqrtf(fmaf(ss, 1.f / D, eps));
#pragma unroll
    for (int st = 0; st < QST; ++st) {
        u32x4 o;
        const u32x4 wv = w ? ld16(w + 32 * st + 8 * grp) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t t1 = cvt_pk_bf16(bf16_elem(x[st], 2 * k) * inv,
                                      bf16_elem(x[st], 2 * k + 1) * inv);
            if (w)
                t1 = cvt_pk_bf16(bf16lo_to_f32(wv[k]) * bf16lo_to_f32(t1),
                                 bf16hi_to_f32(wv[k]) * bf16hi_to_f32(t1));
            o[k] = t1;
        }
        x[st] = o;
    }
}

// rotary embedding of the column's row in place from the cos/sin table
template <int D>
ATTN_DEV void rope_row(u32x4 (&x)[D / 32], const float* cs, int grp) {
    constexpr int H = D / 64;                   // st offset of the upper half
#pragma unroll
    for (int st = 0; st < H; ++st) {
        u32x4 lo, hi;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float rl[2], rh[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int j = 2 * k + e;
                const int i = 32 * st + 8 * grp + j;
                const float a = bf16_elem(x[st], j);
                const float b = bf16_elem(x[st + H], j);
                const float c = cs[i], s = cs[D / 2 + i];
                const float bs = b * s, as = a * s;
                rl[e] = fmaf(a, c, -bs);
                rh[e] = fmaf(b, c, as);
            }
            lo[k] = cvt_pk_bf16(rl[0], rl[1]);
            hi[k] = cvt_pk_bf16(rh[0], rh[1]);
        }
        x[st] = lo;
        x[st + H] = hi;
    }
}

// one head row from global memory in the column layout (zeros when !ok)
template <int D>
ATTN_DEV void load_row(u32x4 (&x)[D / 32], const uint16_t* row, int grp, bool ok) {
#pragma unroll
    for (int st = 0; st < D / 32; ++st) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        x[st] = ok ? ld16(row + 32 * st + 8 * grp) : z;
    }
}

template <int D>
ATTN_DEV void store_row(uint16_t* row, const u32x4 (&x)[D / 32], int grp) {
#pragma unroll
    for (int st = 0; st < D / 32; ++st)
        *reinterpret_cast<u32x4*>(row + 32 * st + 8 * grp) = x[st];
}

// The row's key (part 0) or value (part 1) of KV head g, in three steps so
// the loads can go out early: load (column 0 of the tile holds the row),
// norm (k with its scale; v by the unit norm when asked), then rotate (k)
// and store to the cache slot, and to lds_row [D] when given.
template <int D>
ATTN_DEV void load_kv(u32x4 (&x)[D / 32], const PrepArgs& pa, int s, int g, int Hq, int Hkv,
                      int lane, int part) {
    const size_t row = (size_t)s * (Hq + 2 * Hkv) + Hq + part * Hkv + g;
    load_row<D>(x, pa.qkv + row * D, lane >> 4, (lane & 15) == 0);
}

template <int D>
ATTN_DEV void norm_kv(u32x4 (&x)[D / 32], const PrepArgs& pa, int lane, int part) {
    if (part == 0) norm_row<D>(x, pa.k_w, lane >> 4, pa.eps);
    else if (pa.v_norm) norm_row<D>(x, nullptr, lane >> 4, pa.eps);
}

template <int D>
ATTN_DEV void rope_store_kv(u32x4 (&x)[D / 32], const PrepArgs& pa, size_t slot_off,
                            const float* cs, int lane, int part, uint16_t* lds_row) {
    const int grp = lane >> 4;
    const bool c0 = (lane & 15) == 0;
    if (part == 0) rope_row<D>(x, cs, grp);
    if (c0) store_row<D>((part == 0 ? pa.kc : pa.vc) + slot_off, x, grp);
    if (lds_row && c0) store_row<D>(lds_row, x, grp);
}
