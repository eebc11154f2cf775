// Calibration kernels for the benchmark (a separate library, not part of the
// attention ABI): the HBM read bandwidth and the bf16 matrix-core rate this
// part attains, measured beside the published peaks.
//
//   calib_read_stream   every byte of a buffer read once with 16-byte loads,
//                       a grid-stride walk over the whole chip; each thread
//                       folds what it read into one word, written out so the
//                       loads cannot be dropped
//   calib_read_chunks   the same read with each workgroup walking a
//                       contiguous share of the buffer, loads nontemporal
//                       (streamed past the caches)
//   calib_mfma_loop     waves that issue only v_mfma_f32_16x16x32_bf16 from
//                       register operands (eight independent accumulators),
//                       two waves per SIMD on every CU
//   calib_clock         the shader clock, from the cycle counter against the
//                       100 MHz real-time counter over a matrix-core loop
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// each thread walks contiguous runs of U 16-byte words (U loads in flight),
// runs strided by the whole grid
template <int U>
__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4* __restrict__ src,
                                                          size_t n16, uint32_t* __restrict__ sink) {
    const size_t nthr = (size_t)gridDim.x * blockDim.x;
    const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    size_t i = (size_t)blockIdx.x * blockDim.x * U + threadIdx.x;
    for (; i + (U - 1) * 256 < n16; i += nthr * U) {
        u32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = src[i + (size_t)u * 256];
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
    }
    for (; i < n16; i += 256) {
        const u32x4 a = src[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    sink[tid] = acc;
}

// each workgroup reads its contiguous share (n16 / grid words, a multiple
// of 256 U) with nontemporal loads, U in flight per thread
template <int U>
__global__ __launch_bounds__(256) void read_chunks_kernel(const u32x4* __restrict__ src,
                                                          size_t n16, uint32_t* __restrict__ sink) {
    const size_t per = n16 / gridDim.x;
    const u32x4* p = src + (size_t)blockIdx.x * per;
    uint32_t acc = 0;
    for (size_t i = threadIdx.x; i + (U - 1) * 256 < per; i += 256 * U) {
        u32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = __builtin_nontemporal_load(p + i + (size_t)u * 256);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
    }
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// shader clock against the 100 MHz real-time counter over a matrix-core
// loop: each workgroup's thread 0 writes (cycles, real-time ticks)
__global__ __launch_bounds__(256) void clock_kernel(int iters, uint64_t* __restrict__ out) {
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    const u32x4 a = {0x3F803F80u ^ threadIdx.x, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    const bf16x8 av = __builtin_bit_cast(bf16x8, a);
    f32x4 c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, av, c[j], 0, 0, 0);
    }
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    const float s = c[0][0] + c[1][1] + c[2][2] + c[3][3];
    if (threadIdx.x == 0) {
        out[3 * blockIdx.x] = c1 - c0;
        out[3 * blockIdx.x + 1] = r1 - r0;
        out[3 * blockIdx.x + 2] = __float_as_uint(s);
    }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mfma_loop_kernel(int iters, float* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const u32x4 a = {0x3F803F80u ^ (uint32_t)lane, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    const u32x4 b = {0x3F803F80u, 0x3F803F80u ^ (uint32_t)threadIdx.x, 0x3F803F80u, 0x3F803F80u};
    const bf16x8 av = __builtin_bit_cast(bf16x8, a);
    const bf16x8 bv = __builtin_bit_cast(bf16x8, b);
    f32x4 c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Reads n_bytes (a multiple of 16) at src once, `unroll` (4, 8 or 16)
// 16-byte loads in flight per thread; sink holds grid * 256 words.  Returns a
// hipError_t.
int calib_read_stream(const void* src, size_t n_bytes, void* sink, int grid, int unroll,
                      void* stream) {
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const u32x4* p = static_cast<const u32x4*>(src);
    uint32_t* k = static_cast<uint32_t*>(sink);
    if (unroll == 16) read_stream_kernel<16><<<grid, 256, 0, st>>>(p, n_bytes / 16, k);
    else if (unroll == 8) read_stream_kernel<8><<<grid, 256, 0, st>>>(p, n_bytes / 16, k);
    else read_stream_kernel<4><<<grid, 256, 0, st>>>(p, n_bytes / 16, k);
    return (int)hipGetLastError();
}

// Reads n_bytes at src once, workgroup b its contiguous share, nontemporal;
// n_bytes must be a multiple of grid * 256 * 16 * unroll (8 or 16); sink
// holds grid * 256 words.  Returns a hipError_t (hipErrorInvalidValue for a
// size that does not split so).
int calib_read_chunks(const void* src, size_t n_bytes, void* sink, int grid, int unroll,
                      void* stream) {
    if (grid < 1 || (unroll != 8 && unroll != 16) ||
        n_bytes % ((size_t)grid * 256 * 16 * unroll) != 0)
        return (int)hipErrorInvalidValue;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const u32x4* p = static_cast<const u32x4*>(src);
    uint32_t* k = static_cast<uint32_t*>(sink);
    if (unroll == 16) read_chunks_kernel<16><<<grid, 256, 0, st>>>(p, n_bytes / 16, k);
    else read_chunks_kernel<8><<<grid, 256, 0, st>>>(p, n_bytes / 16, k);
    return (int)hipGetLastError();
}

// grid workgroups each time `iters` x 4 matrix products with the shader
// cycle counter and the 100 MHz real-time counter; out holds 3 * grid words
// (cycles, ticks, a word that keeps the products).  Returns a hipError_t.
int calib_clock(int iters, void* out, int grid, void* stream) {
    clock_kernel<<<grid, 256, 0, static_cast<hipStream_t>(stream)>>>(iters,
                                                                     static_cast<uint64_t*>(out));
    return (int)hipGetLastError();
}

// grid workgroups of four waves, each wave iters x 8 products of 16x16x32
// (16384 flops each); sink holds grid * 256 floats.  Returns a hipError_t.
int calib_mfma_loop(int iters, void* sink, int grid, void* stream) {
    mfma_loop_kernel<<<grid, 256, 0, static_cast<hipStream_t>(stream)>>>(
        iters, static_cast<float*>(sink));
    return (int)hipGetLastError();
}

}  // extern "C"
