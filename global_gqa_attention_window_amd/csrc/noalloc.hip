// One-row decode whose chunk-run partials live in a fixed device array of
// this library instead of a caller's workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops that
// forbid allocation).  The kernels and the arithmetic are attn_decode's, so
// the outputs are its bits.
#include <mutex>

#include "../../include/gqa_attn.h"
#include "kernels.h"

namespace {

// The partials of every call on a device.  Each device that runs the library
// holds its own copy until the process ends; host code never passes this
// name to a kernel (on the host it is only a stand-in for the symbol), only
// the device address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[ATTN_DECODE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};      // device address of `scratch` per device

// The current device's address of `scratch`, looked up once per device with
// that device current; NULL (and the runtime's error) on failure.
void* scratch_for_current_device(hipError_t* err) {
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess || p == nullptr) {
            if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
            return nullptr;
        }
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" int attn_decode_noalloc(void* out, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* pos, int n_seq,
                                   int n_q_heads, int n_kv_heads, int head_dim, int cache_cap,
                                   int ring, int window, float scale, void* stream) {
    const int st = decode_args_status(out, q, k_cache, v_cache, pos, n_seq, n_q_heads,
                                      n_kv_heads, head_dim, cache_cap, ring, window, scale);
    if (st != ATTN_OK || n_seq == 0) return st;
    if (decode_partials_bytes(n_seq, n_q_heads, head_dim, cache_cap) > ATTN_DECODE_SCRATCH_BYTES)
        return ATTN_E_WORKSPACE;
    hipError_t e;
    void* ws = scratch_for_current_device(&e);
    if (ws == nullptr) return ATTN_E_LAUNCH;
    e = launch_decode(static_cast<uint16_t*>(out), static_cast<const uint16_t*>(q),
                      static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache),
                      pos, n_seq, n_q_heads, n_kv_heads, head_dim, cache_cap, ring, window, scale,
                      ws, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}
