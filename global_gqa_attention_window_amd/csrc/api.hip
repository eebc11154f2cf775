// C ABI of the attention library: argument checks, then launches on the
// caller's stream.  Declarations and the meaning of every argument are in
// include/gqa_attn.h.  Every check runs before any HIP call, so a refused call
// touches neither the device nor the stream (the pages' practice of refusing
// unsupported geometries by name, and of validating sizes before any cast:
// TensorFold PR #975, owner review).
#include "../../include/gqa_attn.h"

#include <math.h>

#include <algorithm>

#include "kernels.h"

namespace {

constexpr long long kMaxBytes = 1LL << 46;   // 64 TiB: far past any device

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_heads(int Hq, int Hkv, int D) {
    if (D != 256 && D != 512) return ATTN_E_HEAD_DIM;
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Hq / Hkv > 16) return ATTN_E_GQA;
    return ATTN_OK;
}

// bytes of one [n][h][len][D] bf16 tensor, or -1 past kMaxBytes
long long tensor_bytes(long long n, long long h, long long len, long long D) {
    if (n < 0 || h < 0 || len < 0) return -1;
    long long b = 2 * D;
    for (long long f : {n, h, len}) {
        if (f != 0 && b > kMaxBytes / f) return -1;
        b *= f;
    }
    return b;
}

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ATTN_OK";
        case ATTN_E_NULL: return "ATTN_E_NULL";
        case ATTN_E_HEAD_DIM: return "ATTN_E_HEAD_DIM";
        case ATTN_E_GQA: return "ATTN_E_GQA";
        case ATTN_E_WINDOW: return "ATTN_E_WINDOW";
        case ATTN_E_CACHE: return "ATTN_E_CACHE";
        case ATTN_E_ALIGN: return "ATTN_E_ALIGN";
        case ATTN_E_WORKSPACE: return "ATTN_E_WORKSPACE";
        case ATTN_E_P_MODE: return "ATTN_E_P_MODE";
        case ATTN_E_RANGE: return "ATTN_E_RANGE";
        case ATTN_E_LAUNCH: return "ATTN_E_LAUNCH";
        case ATTN_E_UNSUPPORTED: return "ATTN_E_UNSUPPORTED";
        default: return "ATTN_E_UNKNOWN";
    }
}

size_t attn_decode_workspace_bytes(int n_seq, int n_q_heads, int head_dim,
                                   int cache_cap) {
    if (n_seq < 0 || cache_cap < 1 || n_q_heads < 1 || (head_dim != 256 && head_dim != 512))
        return 0;
    const long long nch = ((long long)cache_cap + ATTN_DECODE_CHUNK - 1) / ATTN_DECODE_CHUNK;
    const long long units = (long long)n_seq * n_q_heads * nch;
    if (units > kMaxBytes / (4 * (head_dim + 2))) return 0;
    return decode_workspace_bytes(n_seq, n_q_heads, head_dim, cache_cap);
}

}  // extern "C"

// Checks of attn_decode's arguments other than its workspace, in the order
// the call makes them; ATTN_OK with n_seq == 0 means "nothing to launch".
int decode_args_status(const void* out, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* pos, int n_seq, int n_q_heads,
                       int n_kv_heads, int head_dim, int cache_cap, int ring, int window,
                       float scale) {
    int st = check_heads(n_q_heads, n_kv_heads, head_dim);
    if (st != ATTN_OK) return st;
    if (n_seq < 0 || (ring != 0 && ring != 1) || !isfinite(scale)) return ATTN_E_RANGE;
    if (cache_cap < 1) return ATTN_E_CACHE;
    if (window < 0 || (ring && window > cache_cap)) return ATTN_E_WINDOW;
    if (tensor_bytes(n_seq, n_kv_heads, cache_cap, head_dim) < 0 ||
        tensor_bytes(n_seq, n_q_heads, 1, head_dim) < 0)
        return ATTN_E_RANGE;
    // one head's cache slice is addressed with 32-bit byte offsets
    if ((long long)cache_cap * head_dim * 2 >= (1LL << 32)) return ATTN_E_RANGE;
    if (n_seq == 0) return ATTN_OK;
    if (!out || !q || !k_cache || !v_cache || !pos) return ATTN_E_NULL;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
        (reinterpret_cast<uintptr_t>(pos) & 3u) != 0)
        return ATTN_E_ALIGN;
    if (n_seq > 65535 || n_kv_heads > 65535 ||
        (cache_cap + ATTN_DECODE_CHUNK - 1) / ATTN_DECODE_CHUNK > 0x7FFFFFFF / 2)
        return ATTN_E_RANGE;
    return ATTN_OK;
}

extern "C" {

int attn_decode(void* out, const void* q, const void* k_cache,
                const void* v_cache, const int32_t* pos, int n_seq,
                int n_q_heads, int n_kv_heads, int head_dim, int cache_cap,
                int ring, int window, float scale, void* workspace,
                size_t workspace_bytes, void* stream) {
    const int st = decode_args_status(out, q, k_cache, v_cache, pos, n_seq, n_q_heads,
                                      n_kv_heads, head_dim, cache_cap, ring, window, scale);
    if (st != ATTN_OK || n_seq == 0) return st;
    if (!workspace) return ATTN_E_WORKSPACE;
    if (!aligned16(workspace)) return ATTN_E_ALIGN;
    const size_t need = attn_decode_workspace_bytes(n_seq, n_q_heads, head_dim, cache_cap);
    if (need == 0) return ATTN_E_RANGE;
    if (workspace_bytes < need) return ATTN_E_WORKSPACE;
    hipError_t e = launch_decode(
        static_cast<uint16_t*>(out), static_cast<const uint16_t*>(q),
        static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache),
        pos, n_seq, n_q_heads, n_kv_heads, head_dim, cache_cap, ring, window,
        scale, workspace, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

size_t attn_decode_rows_workspace_bytes(int n_seq, int rows, int n_q_heads, int head_dim,
                                        int cache_cap) {
    if (rows < 1 || rows > ATTN_DECODE_MAX_ROWS || n_seq < 0 ||
        (long long)n_seq * rows > 0x7FFFFFFFLL)
        return 0;
    return attn_decode_workspace_bytes(n_seq * rows, n_q_heads, head_dim, cache_cap);
}

namespace {

// checks of the prologue's own arguments (stacked rows, scales, frequencies)
static int check_prep(const PrepArgs& pa) {
    if (!pa.qkv || !pa.q_w || !pa.k_w || !pa.inv_freq) return ATTN_E_NULL;
    if (!aligned16(pa.qkv) || !aligned16(pa.q_w) || !aligned16(pa.k_w) ||
        (reinterpret_cast<uintptr_t>(pa.inv_freq) & 3u) != 0)
        return ATTN_E_ALIGN;
    if (!isfinite(pa.eps) || pa.eps < 0.f || (pa.v_norm != 0 && pa.v_norm != 1))
        return ATTN_E_RANGE;
    return ATTN_OK;
}

static int decode_rows_call(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* pos, int n_seq, int rows, int n_q_heads, int n_kv_heads,
                     int head_dim, int cache_cap, int ring, int window, float scale,
                     void* workspace, size_t workspace_bytes, bool fused,
                     const PrepArgs* prep, void* stream) {
    int st = check_heads(n_q_heads, n_kv_heads, head_dim);
    if (st != ATTN_OK) return st;
    if (n_seq < 0 || rows < 1 || rows > ATTN_DECODE_MAX_ROWS || (ring != 0 && ring != 1) ||
        !isfinite(scale))
        return ATTN_E_RANGE;
    if (cache_cap < 1) return ATTN_E_CACHE;
    if (window < 0) return ATTN_E_WINDOW;
    if (ring && (window < 1 || (long long)window + rows - 1 > cache_cap)) return ATTN_E_WINDOW;
    if (tensor_bytes(n_seq, n_kv_heads, cache_cap, head_dim) < 0 ||
        tensor_bytes((long long)n_seq * rows, n_q_heads, 1, head_dim) < 0)
        return ATTN_E_RANGE;
    // one head's cache slice is addressed with 32-bit byte offsets
    if ((long long)cache_cap * head_dim * 2 >= (1LL << 32)) return ATTN_E_RANGE;
    // sixteen counters per (stream, KV head) in the fused counter area (one
    // per workgroup of the item: up to 16 column tiles at head dim 256)
    if (fused && (long long)n_seq * n_kv_heads * 16 * 4 > ATTN_DECODE_COUNTER_BYTES)
        return ATTN_E_RANGE;
    if (n_seq == 0) return ATTN_OK;
    if (prep) {
        st = check_prep(*prep);
        if (st != ATTN_OK) return st;
        q = prep->qkv;                           // the queries come from the stacked rows
    }
    if (!out || !q || !k_cache || !v_cache || !pos) return ATTN_E_NULL;
    if (!workspace) return ATTN_E_WORKSPACE;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) ||
        !aligned16(v_cache) || !aligned16(workspace) ||
        (reinterpret_cast<uintptr_t>(pos) & 3u) != 0)
        return ATTN_E_ALIGN;
    const size_t need =
        attn_decode_rows_workspace_bytes(n_seq, rows, n_q_heads, head_dim, cache_cap);
    if (need == 0) return ATTN_E_RANGE;
    if (workspace_bytes < need + (fused ? ATTN_DECODE_COUNTER_BYTES : 0)) return ATTN_E_WORKSPACE;
    if (n_seq > 65535 || n_kv_heads > 65535 ||
        (cache_cap + ATTN_DECODE_CHUNK - 1) / ATTN_DECODE_CHUNK > 0x7FFFFFFF / 2)
        return ATTN_E_RANGE;
    hipError_t e = launch_decode_rows(
        static_cast<uint16_t*>(out), static_cast<const uint16_t*>(q),
        static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache),
        pos, n_seq, rows, n_q_heads, n_kv_heads, head_dim, cache_cap, ring, window,
        scale, workspace, fused, prep, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

}  // namespace

int attn_decode_rows(void* out, const void* q, const void* k_cache,
                     const void* v_cache, const int32_t* pos, int n_seq, int rows,
                     int n_q_heads, int n_kv_heads, int head_dim, int cache_cap,
                     int ring, int window, float scale, void* workspace,
                     size_t workspace_bytes, void* stream) {
    return decode_rows_call(out, q, k_cache, v_cache, pos, n_seq, rows, n_q_heads, n_kv_heads,
                            head_dim, cache_cap, ring, window, scale, workspace,
                            workspace_bytes, false, nullptr, stream);
}

int attn_decode_rows_fused(void* out, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* pos, int n_seq, int rows,
                           int n_q_heads, int n_kv_heads, int head_dim, int cache_cap,
                           int ring, int window, float scale, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return decode_rows_call(out, q, k_cache, v_cache, pos, n_seq, rows, n_q_heads, n_kv_heads,
                            head_dim, cache_cap, ring, window, scale, workspace,
                            workspace_bytes, true, nullptr, stream);
}

int attn_decode_prep_fused(void* out, const void* qkv, const void* q_norm_w,
                           const void* k_norm_w, const float* inv_freq, float eps, int v_norm,
                           void* k_cache, void* v_cache, const int32_t* pos, int n_seq,
                           int n_q_heads, int n_kv_heads, int head_dim, int cache_cap,
                           int ring, int window, float scale, void* workspace,
                           size_t workspace_bytes, void* stream) {
    const PrepArgs pa = {static_cast<const uint16_t*>(qkv), static_cast<const uint16_t*>(q_norm_w),
                         static_cast<const uint16_t*>(k_norm_w), inv_freq, eps, v_norm,
                         static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache)};
    return decode_rows_call(out, qkv, k_cache, v_cache, pos, n_seq, 1, n_q_heads, n_kv_heads,
                            head_dim, cache_cap, ring, window, scale, workspace,
                            workspace_bytes, true, &pa, stream);
}

int attn_qkv_prep(void* q_out, void* k_cache, void* v_cache, const void* qkv,
                  const void* q_norm_w, const void* k_norm_w, const float* inv_freq, float eps,
                  int v_norm, const int32_t* pos, int n_seq, int n_q_heads, int n_kv_heads,
                  int head_dim, int cache_cap, int ring, void* stream) {
    int st = check_heads(n_q_heads, n_kv_heads, head_dim);
    if (st != ATTN_OK) return st;
    if (n_seq < 0 || (ring != 0 && ring != 1)) return ATTN_E_RANGE;
    if (cache_cap < 1) return ATTN_E_CACHE;
    if (tensor_bytes(n_seq, n_kv_heads, cache_cap, head_dim) < 0 ||
        tensor_bytes(n_seq, n_q_heads + 2LL * n_kv_heads, 1, head_dim) < 0 || n_seq > 65535)
        return ATTN_E_RANGE;
    if (n_seq == 0) return ATTN_OK;
    const PrepArgs pa = {static_cast<const uint16_t*>(qkv), static_cast<const uint16_t*>(q_norm_w),
                         static_cast<const uint16_t*>(k_norm_w), inv_freq, eps, v_norm,
                         static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache)};
    st = check_prep(pa);
    if (st != ATTN_OK) return st;
    if (!q_out || !k_cache || !v_cache || !pos) return ATTN_E_NULL;
    if (!aligned16(q_out) || !aligned16(k_cache) || !aligned16(v_cache) ||
        (reinterpret_cast<uintptr_t>(pos) & 3u) != 0)
        return ATTN_E_ALIGN;
    const hipError_t e = launch_qkv_prep(static_cast<uint16_t*>(q_out), pa, pos, n_seq,
                                         n_q_heads, n_kv_heads, head_dim, cache_cap, ring,
                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

int attn_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
    if (!workspace) return ATTN_E_WORKSPACE;
    if (!aligned16(workspace)) return ATTN_E_ALIGN;
    if (workspace_bytes < ATTN_DECODE_COUNTER_BYTES) return ATTN_E_WORKSPACE;
    const hipError_t e = launch_decode_counters_init(workspace, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

int attn_prefill_key_block(int head_dim, int p_mode) {
    if (head_dim != 256 && head_dim != 512) return ATTN_E_HEAD_DIM;
    if (p_mode != ATTN_P_BF16 && p_mode != ATTN_P_BF16X2) return ATTN_E_P_MODE;
    return prefill_key_block(head_dim, p_mode);
}

namespace {

// Argument checks of attn_prefill, up to (not including) the n_rows == 0
// early return and the pointer checks.
static int check_prefill(int pos0, int n_rows, int n_q_heads, int n_kv_heads, int head_dim,
                  int cache_cap, int ring, int window, float scale, int p_mode) {
    int st = check_heads(n_q_heads, n_kv_heads, head_dim);
    if (st != ATTN_OK) return st;
    if (p_mode != ATTN_P_BF16 && p_mode != ATTN_P_BF16X2) return ATTN_E_P_MODE;
    if (n_rows < 0 || pos0 < 0 || (ring != 0 && ring != 1) || !isfinite(scale))
        return ATTN_E_RANGE;
    if (cache_cap < 1) return ATTN_E_CACHE;
    if (window < 0) return ATTN_E_WINDOW;
    if (ring) {
        if (window == 0 || window > cache_cap) return ATTN_E_WINDOW;
        if ((long long)cache_cap < (long long)window + n_rows - 1) return ATTN_E_CACHE;
    } else if ((long long)pos0 + n_rows > cache_cap) {
        return ATTN_E_CACHE;
    }
    if (tensor_bytes(1, n_kv_heads, cache_cap, head_dim) < 0 ||
        tensor_bytes(n_rows, n_q_heads, 1, head_dim) < 0)
        return ATTN_E_RANGE;
    // one head's cache slice is addressed with 32-bit byte offsets
    if ((long long)cache_cap * head_dim * 2 >= (1LL << 32)) return ATTN_E_RANGE;
    // the kernels form positions up to the last row's plus one key block in
    // 32-bit ints (a ring's positions are not bounded by its capacity)
    if ((long long)pos0 + n_rows + 64 > 0x7FFFFFFFLL) return ATTN_E_RANGE;
    return ATTN_OK;
}

}  // namespace

int attn_prefill(void* out, const void* q, const void* k_cache,
                 const void* v_cache, int pos0, int n_rows, int n_q_heads,
                 int n_kv_heads, int head_dim, int cache_cap, int ring,
                 int window, float scale, int p_mode,
                 const int32_t* last_key, void* stream) {
    const int st = check_prefill(pos0, n_rows, n_q_heads, n_kv_heads, head_dim, cache_cap,
                                 ring, window, scale, p_mode);
    if (st != ATTN_OK) return st;
    if (n_rows == 0) return ATTN_OK;
    if (!out || !q || !k_cache || !v_cache) return ATTN_E_NULL;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return ATTN_E_ALIGN;
    if (last_key && (reinterpret_cast<uintptr_t>(last_key) & 3u)) return ATTN_E_ALIGN;
    hipError_t e = launch_prefill(
        static_cast<uint16_t*>(out), static_cast<const uint16_t*>(q),
        static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache),
        pos0, n_rows, n_q_heads, n_kv_heads, head_dim, cache_cap, ring, window,
        scale, p_mode, last_key, nullptr, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

size_t attn_prefill_workspace_bytes(int n_rows, int n_q_heads, int head_dim) {
    if (n_rows < 0 || n_q_heads < 1 || (head_dim != 256 && head_dim != 512)) return 0;
    // (bf16 count: twice as many entries gives the fp32 partials' bytes)
    if (tensor_bytes(n_rows, n_q_heads, 2 * PREFILL_MAX_SPLIT, head_dim + 2) < 0) return 0;
    return prefill_partials_bytes(n_rows, n_q_heads, head_dim, PREFILL_MAX_SPLIT);
}

int attn_prefill_ws(void* out, const void* q, const void* k_cache,
                    const void* v_cache, int pos0, int n_rows, int n_q_heads,
                    int n_kv_heads, int head_dim, int cache_cap, int ring,
                    int window, float scale, int p_mode,
                    const int32_t* last_key, void* workspace, size_t workspace_bytes,
                    void* stream) {
    if (workspace == nullptr)
        return attn_prefill(out, q, k_cache, v_cache, pos0, n_rows, n_q_heads, n_kv_heads,
                            head_dim, cache_cap, ring, window, scale, p_mode, last_key, stream);
    const int st = check_prefill(pos0, n_rows, n_q_heads, n_kv_heads, head_dim, cache_cap,
                                 ring, window, scale, p_mode);
    if (st != ATTN_OK) return st;
    if (n_rows == 0) return ATTN_OK;
    if (!out || !q || !k_cache || !v_cache) return ATTN_E_NULL;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
        !aligned16(workspace))
        return ATTN_E_ALIGN;
    if (last_key && (reinterpret_cast<uintptr_t>(last_key) & 3u)) return ATTN_E_ALIGN;
    const size_t need = attn_prefill_workspace_bytes(n_rows, n_q_heads, head_dim);
    if (need == 0) return ATTN_E_RANGE;
    if (workspace_bytes < need) return ATTN_E_WORKSPACE;
    hipError_t e = launch_prefill(
        static_cast<uint16_t*>(out), static_cast<const uint16_t*>(q),
        static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache),
        pos0, n_rows, n_q_heads, n_kv_heads, head_dim, cache_cap, ring, window,
        scale, p_mode, last_key, workspace, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

size_t attn_prefill_prompt_workspace_bytes(int pos0, int n_rows, int n_kv_heads, int head_dim,
                                           int ring, int window) {
    if (pos0 < 0 || n_rows < 0 || n_kv_heads < 1 || (head_dim != 256 && head_dim != 512) ||
        (ring != 0 && ring != 1) || window < 0 || (ring && window == 0))
        return 0;
    if ((long long)pos0 + n_rows + 64 > 0x7FFFFFFFLL) return 0;
    const long long span = (long long)pos0 + n_rows - std::max(0, pos0 - window + 1);
    if (ring && tensor_bytes(2 * n_kv_heads, 1, span, head_dim) < 0) return 0;
    return prefill_prompt_stage_bytes(pos0, n_rows, n_kv_heads, head_dim, ring, window);
}

int attn_prefill_prompt(void* out, const void* q, const void* k, const void* v,
                        void* k_cache, void* v_cache, int pos0, int n_rows, int chunk,
                        int n_q_heads, int n_kv_heads, int head_dim, int cache_cap, int ring,
                        int window, float scale, int p_mode, const int32_t* last_key,
                        void* workspace, size_t workspace_bytes, void* stream) {
    if (chunk < 1) return ATTN_E_RANGE;
    // every chunk meets attn_prefill's checks if the first (longest) does and
    // the whole prompt fits the positions and the linear cache
    const int first = n_rows < chunk ? n_rows : chunk;
    const int st = check_prefill(pos0, first, n_q_heads, n_kv_heads, head_dim, cache_cap,
                                 ring, window, scale, p_mode);
    if (st != ATTN_OK) return st;
    if (n_rows < 0) return ATTN_E_RANGE;
    if (!ring && (long long)pos0 + n_rows > cache_cap) return ATTN_E_CACHE;
    if ((long long)pos0 + n_rows + 64 > 0x7FFFFFFFLL ||
        tensor_bytes(n_rows, n_q_heads, 1, head_dim) < 0 ||
        tensor_bytes(n_rows, n_kv_heads, 1, head_dim) < 0)
        return ATTN_E_RANGE;
    if (n_rows == 0) return ATTN_OK;
    if (!out || !q || !k || !v || !k_cache || !v_cache) return ATTN_E_NULL;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k) || !aligned16(v) ||
        !aligned16(k_cache) || !aligned16(v_cache) || (workspace && !aligned16(workspace)))
        return ATTN_E_ALIGN;
    if (last_key && (reinterpret_cast<uintptr_t>(last_key) & 3u)) return ATTN_E_ALIGN;
    if (ring) {
        // the attended span's linear copy: one head's slice in 32-bit offsets
        const long long span = (long long)pos0 + n_rows - std::max(0, pos0 - window + 1);
        if (span * head_dim * 2 >= (1LL << 32)) return ATTN_E_RANGE;
        const size_t need = attn_prefill_prompt_workspace_bytes(pos0, n_rows, n_kv_heads,
                                                                head_dim, ring, window);
        if (need == 0) return ATTN_E_RANGE;
        if (!workspace || workspace_bytes < need) return ATTN_E_WORKSPACE;
    }
    const hipError_t e = launch_prefill_prompt(
        static_cast<uint16_t*>(out), static_cast<const uint16_t*>(q),
        static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
        static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), pos0, n_rows, chunk,
        n_q_heads, n_kv_heads, head_dim, cache_cap, ring, window, scale, p_mode, last_key,
        workspace, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

int attn_cache_write(void* k_cache, void* v_cache, const void* k,
                     const void* v, int pos0, int n_rows, int n_kv_heads,
                     int head_dim, int cache_cap, int ring, void* stream) {
    if (head_dim != 256 && head_dim != 512) return ATTN_E_HEAD_DIM;
    if (n_kv_heads < 1) return ATTN_E_GQA;
    if (n_rows < 0 || pos0 < 0 || (ring != 0 && ring != 1)) return ATTN_E_RANGE;
    if (cache_cap < 1) return ATTN_E_CACHE;
    if (ring ? n_rows > cache_cap : (long long)pos0 + n_rows > cache_cap)
        return ATTN_E_CACHE;
    if (tensor_bytes(1, n_kv_heads, cache_cap, head_dim) < 0 ||
        tensor_bytes(n_rows, n_kv_heads, 1, head_dim) < 0)
        return ATTN_E_RANGE;
    if (n_rows == 0) return ATTN_OK;
    if (!k_cache || !v_cache || !k || !v) return ATTN_E_NULL;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k) || !aligned16(v))
        return ATTN_E_ALIGN;
    hipError_t e = launch_cache_write(
        static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
        static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), pos0,
        n_rows, n_kv_heads, head_dim, cache_cap, ring, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

}  // extern "C"
