// Device helpers shared by the gfx950 attention kernels.
//
// Matrix-core conventions (CDNA3/CDNA4 16x16 MFMA, wave64):
//   v_mfma_f32_16x16x32_bf16  A 16x32, B 32x16: lane l supplies row/column
//       l % 16 and eight reduction indices picked by l / 16; the reduction
//       index a lane supplies is the same slot for A and B, so any one-to-one
//       assignment of reduction indices to (l / 16, element) is a valid dot
//       product.  C 16x16: lane l holds rows 4 * (l / 16) + i, column l % 16.
//   v_mfma_f32_16x16x4_f32    A 16x4: lane l holds A[l % 16][l / 16];
//       B 4x16: B[l / 16][l % 16]; C as above.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define ATTN_DEV __device__ __forceinline__

ATTN_DEV float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
ATTN_DEV float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
ATTN_DEV uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

ATTN_DEV float bf16_round_f32(float f) {
    return __uint_as_float(f32_to_bf16_bits(f) << 16);
}

ATTN_DEV uint32_t pack_bf16x2(uint32_t lo_bits, uint32_t hi_bits) {
    return (lo_bits & 0xFFFFu) | (hi_bits << 16);
}

ATTN_DEV bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// two fp32 -> packed bf16 pair (lo, hi) with v_cvt_pk_bf16_f32: round to
// nearest even, NaN stays NaN
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
ATTN_DEV uint32_t cvt_pk_bf16(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

ATTN_DEV f32x4 mfma_bf16_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

ATTN_DEV f32x4 mfma_f32_16x16x4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

ATTN_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16 bytes per lane from global memory straight into LDS (global_load_lds
// dwordx4): lane i writes lds_base + 16 i; lds_base must be wave-uniform.
// The host compilation pass sees no body (the builtin exists only on gfx950).
#if defined(__HIP_DEVICE_COMPILE__)
#define ATTN_DMA16(src, lds_base) __builtin_amdgcn_global_load_lds((src), (lds_base), 16, 0, 0)
#else
#define ATTN_DMA16(src, lds_base) ((void)(src), (void)(lds_base))
#endif

// LDS byte address of a __shared__ pointer (the low half of its flat address)
ATTN_DEV uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)p;
}

// The same global->LDS load issued from asm.  The compiler then does not see
// an LDS write, so it adds no wait on the load before later LDS reads (it
// cannot tell which bytes the load writes and would wait before every read);
// the caller waits for vmcnt and synchronises before any wave reads the
// bytes.  lds_byte must be wave-uniform; M0 carries it, with the one wait
// state an SALU write of M0 needs before an LDS DMA.  Nothing else in a
// kernel that uses this may rely on M0.
ATTN_DEV void dma16_asm(const void* src, uint32_t lds_byte) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(src), "s"(lds_byte) : "memory");
#else
    (void)src;
    (void)lds_byte;
#endif
}
// ... with a wave-uniform base address and a per-lane 32-bit byte offset
// (both wave-uniform by construction; readfirstlane puts them in SGPRs where
// the compiler cannot prove it)
ATTN_DEV void dma16_asm_sbase(const void* base, uint32_t voff, uint32_t lds_byte) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint64_t b64 = (uint64_t)(uintptr_t)base;
    const uint64_t bu = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b64);
    const uint32_t lu = __builtin_amdgcn_readfirstlane(lds_byte);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(bu), "s"(lu) : "memory");
#else
    (void)base;
    (void)voff;
    (void)lds_byte;
#endif
}

// ... the same, nontemporal (nt: the lines are streamed, not kept for reuse),
// for data a launch reads once
ATTN_DEV void dma16_asm_sbase_nt(const void* base, uint32_t voff, uint32_t lds_byte) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint64_t b64 = (uint64_t)(uintptr_t)base;
    const uint64_t bu = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b64);
    const uint32_t lu = __builtin_amdgcn_readfirstlane(lds_byte);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :: "v"(voff), "s"(bu), "s"(lu) : "memory");
#else
    (void)base;
    (void)voff;
    (void)lds_byte;
#endif
}

// Wait until at most N of this wave's vector memory loads are outstanding
// (loads complete in issue order for the count), with no wait on LDS or
// export counters: the N most recent global->LDS loads may stay in flight.
template <int N>
ATTN_DEV void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Element offset of row r of a K or V block staged in LDS.  D = 512: rows of
// 1 KiB, each followed by PADP padding elements.  D = 256: rows r and r + 8
// of each 16-row group share one 1 KiB unit (the two halves of a DMA
// instruction's 64 lanes), units followed by PADP padding elements.
template <int D, int PADP>
ATTN_DEV constexpr int row_pos(int r) {
    if constexpr (D == 512) {
        return r * (D + PADP);
    } else {
        return ((r >> 4) * 8 + (r & 7)) * (2 * D + PADP) + ((r >> 3) & 1) * D;
    }
}

// Whether a cache slot is attended by a decode row at position t, and the
// position it holds: a linear cache holds position `slot`; a ring of cap
// slots the latest position p <= t with p = slot (mod cap).  Attended: 0 <=
// p <= t and, with a window W > 0, t - p < W.  Slots at or past cap, and
// rows at t < 0, attend nothing.
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

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane j points at four consecutive 16-bit elements M[j][0..3]; lane i gets
// back M[4 k + (i >> 2)][i & 3] for k = 0..3 (measured on gfx950).  Pointing
// lane j at row kappa(j >> 2), column c0 + 4 (j & 3) of a row-major matrix
// therefore hands lane i the four rows kappa(0..3) at column c0 + i.
typedef short s16x4 __attribute__((ext_vector_type(4)));
ATTN_DEV u32x2 lds_read_tr16(const uint16_t* p) {
#if defined(__HIP_DEVICE_COMPILE__)
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p));
    return __builtin_bit_cast(u32x2, v);
#else
    (void)p;
    return u32x2{0u, 0u};
#endif
}

// Butterfly over the four lanes l, l^16, l^32, l^48 (same l % 16), in VALU
// without an LDS round trip.  v_permlane16_swap_b32 with both operands x
// hands back (x[l & ~16], x[l | 16]) and v_permlane32_swap_b32 likewise for
// bit 5, so both lanes of a pair combine the same two values in the same
// order and end with identical bits.
ATTN_DEV void pair16(float x, float& a, float& b) {
#if defined(__HIP_DEVICE_COMPILE__)
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
#else
    a = x; b = x;
#endif
}
ATTN_DEV void pair32(float x, float& a, float& b) {
#if defined(__HIP_DEVICE_COMPILE__)
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
#else
    a = x; b = x;
#endif
}
ATTN_DEV float xmax4(float x) {
    float a, b;
    pair16(x, a, b);
    x = fmaxf(a, b);
    pair32(x, a, b);
    return fmaxf(a, b);
}
ATTN_DEV float xsum4(float x) {
    float a, b;
    pair16(x, a, b);
    x = a + b;
    pair32(x, a, b);
    return a + b;
}

// Pinned instruction order inside one scheduling region: each call opens a
// group of up to n instructions of one kind, groups issue in call order.
#define ATTN_SG_VALU 0x0002
#define ATTN_SG_MFMA 0x0008
#define ATTN_SG_DS_READ 0x0100
#if defined(__HIP_DEVICE_COMPILE__)
#define ATTN_SCHED(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)
#else
#define ATTN_SCHED(mask, n) ((void)0)
#endif

ATTN_DEV u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
ATTN_DEV void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Cache write, unit i of n_rows * Hkv * D / 8: eight bf16 of one (row, KV
// head) of k and of v into the row's slot (pos0 + row of a linear cache,
// (pos0 + row) mod cap of a ring); consecutive units walk d, so a wave reads
// and writes 1 KiB of contiguous memory.  Units past the end do nothing.
ATTN_DEV void cache_write_unit(uint16_t* __restrict__ kc, uint16_t* __restrict__ vc,
                               const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                               int pos0, int n_rows, int Hkv, int D, int cap, int ring,
                               size_t i) {
    const int vec_per_row = D / 8;
    const size_t total = (size_t)n_rows * Hkv * vec_per_row;
    if (i >= total) return;
    const int dv = (int)(i % vec_per_row);
    const size_t rg = i / vec_per_row;
    const int g = (int)(rg % Hkv);
    const int r = (int)(rg / Hkv);
    const long long p = (long long)pos0 + r;
    const long long slot = ring ? p % cap : p;
    const size_t src = rg * D + (size_t)dv * 8;
    const size_t dst = ((size_t)g * cap + (size_t)slot) * D + (size_t)dv * 8;
    st16(kc + dst, ld16(k + src));
    st16(vc + dst, ld16(v + src));
}

// log2(e) as float: scores are scaled by scale * log2(e) and exponentiated
// with exp2, so exp(scale * s - m) = exp2(scale * log2e * s - m').
#define ATTN_LOG2E 1.4426950408889634f
