// synth_gpu.hip -- device implementation of the synthetic-input definitions in
// synth/gen.py, for workloads too large to generate on the host.  It holds no
// arithmetic of the MoE layer: SplitMix64 stream words, Irwin-Hall normal-like
// values, fp64 -> fp16 round-to-nearest-even, and an ascending sort of each parent
// LUT row.  Every output is bit-identical to the numpy generator.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp16_rne.h"

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__device__ inline uint64_t mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// element idx of the stream with key `key`
__device__ inline uint64_t stream(uint64_t key, uint64_t idx) { return mix(key + (idx + 1) * kGolden); }

// normal-like value number idx: sum of twelve 16-bit chunks of stream elements
// 3idx..3idx+2, minus 393210, times 2^-16 (exact)
__device__ inline double normal(uint64_t key, uint64_t idx)
{
    int64_t acc = 0;
    for (int i = 0; i < 3; ++i) {
        const uint64_t u = stream(key, 3 * idx + i);
        acc += (int64_t)(u & 0xFFFF) + (int64_t)((u >> 16) & 0xFFFF) + (int64_t)((u >> 32) & 0xFFFF) +
               (int64_t)(u >> 48);
    }
    return (double)(acc - 393210) * (1.0 / 65536.0);
}

__global__ void planes_kernel(uint64_t key, uint64_t nwords, uint32_t *__restrict__ out)
{
    const uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j * 2 >= nwords)
        return;
    const uint64_t v = stream(key, j);
    out[2 * j] = (uint32_t)v;
    if (2 * j + 1 < nwords)
        out[2 * j + 1] = (uint32_t)(v >> 32);
}

__global__ void fp16_normal_kernel(uint64_t key, uint64_t n, double std, uint16_t *__restrict__ out)
{
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        out[i] = apmoe_d2h_rne(normal(key, i) * std);
}

// order-preserving key of a non-NaN fp16 bit pattern (+0 after canonicalisation)
__device__ inline uint32_t sort_key(uint16_t h) { return (h & 0x8000) ? (uint32_t)(~h & 0xFFFF) : (uint32_t)(h | 0x8000); }

// One 256-thread workgroup per row: generate 256 values, canonicalise -0 to +0,
// bitonic sort ascending in LDS.
__global__ void __launch_bounds__(256) parent_lut_kernel(uint64_t key, int rows, double std,
                                                         uint16_t *__restrict__ out)
{
    __shared__ uint16_t v[256];
    const int row = blockIdx.x;
    const int t = threadIdx.x;
    if (row >= rows)
        return;
    uint16_t h = apmoe_d2h_rne(normal(key, (uint64_t)row * 256 + t) * std);
    if (h == 0x8000)
        h = 0;
    v[t] = h;
    __syncthreads();
    for (int k = 2; k <= 256; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            const int p = t ^ j;
            if (p > t) {
                const bool up = (t & k) == 0;
                const uint16_t a = v[t], b = v[p];
                if ((sort_key(a) > sort_key(b)) == up) {
                    v[t] = b;
                    v[p] = a;
                }
            }
            __syncthreads();
        }
    }
    out[(size_t)row * 256 + t] = v[t];
}

}  // namespace

extern "C" {

// All pointers are device pointers; calls are asynchronous on `stream`.
int synth_gpu_planes(uint64_t key, uint64_t nwords, uint32_t *out, void *stream)
{
    const uint64_t threads = (nwords + 1) / 2;
    if (threads == 0)
        return 0;
    hipLaunchKernelGGL(planes_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), key, nwords, out);
    return (int)hipGetLastError();
}

int synth_gpu_fp16_normal(uint64_t key, uint64_t n, double std, uint16_t *out, void *stream)
{
    if (n == 0)
        return 0;
    hipLaunchKernelGGL(fp16_normal_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), key, n, std, out);
    return (int)hipGetLastError();
}

int synth_gpu_parent_lut(uint64_t key, int rows, double std, uint16_t *out, void *stream)
{
    if (rows <= 0)
        return 0;
    hipLaunchKernelGGL(parent_lut_kernel, dim3(rows), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), key,
                       rows, std, out);
    return (int)hipGetLastError();
}

}  // extern "C"
