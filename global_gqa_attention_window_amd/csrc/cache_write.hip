// Cache write before attention (TensorFold PR #975 "Gemma 4 12B on the native
// Metal engine", the cache-before-attention commit: a window's keys and values
// enter the cache first, and attention reads every key from the cache).
//
// Row r of the chunk (position pos0 + r) goes to slot pos0 + r of a linear
// cache, or (pos0 + r) mod cap of a ring.  Pure 16-byte copies: one thread
// moves eight bf16 of one (row, KV head), consecutive threads walk d, so each
// wave reads and writes 1 KiB of contiguous memory (cache_write_unit).
#include "common.h"
#include "kernels.h"

namespace {

__global__ __launch_bounds__(256)
void cache_write_kernel(uint16_t* __restrict__ kc, uint16_t* __restrict__ vc,
                        const uint16_t* __restrict__ k,
                        const uint16_t* __restrict__ v, int pos0, int n_rows,
                        int Hkv, int D, int cap, int ring) {
    cache_write_unit(kc, vc, k, v, pos0, n_rows, Hkv, D, cap, ring,
                     (size_t)blockIdx.x * blockDim.x + threadIdx.x);
}

}  // namespace

hipError_t launch_cache_write(uint16_t* kc, uint16_t* vc, const uint16_t* k,
                              const uint16_t* v, int pos0, int n_rows, int Hkv,
                              int D, int cap, int ring, hipStream_t stream) {
    const size_t total = (size_t)n_rows * Hkv * (D / 8);
    const unsigned blocks = (unsigned)((total + 255) / 256);
    cache_write_kernel<<<blocks, 256, 0, stream>>>(kc, vc, k, v, pos0, n_rows,
                                                   Hkv, D, cap, ring);
    return hipGetLastError();
}
