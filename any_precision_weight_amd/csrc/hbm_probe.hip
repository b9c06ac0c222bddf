// hbm_probe.hip -- a plain HBM read stream, the practical read ceiling the benchmark
// reports beside the published peak.  Not part of the layer: libhbmprobe.so is a
// separate library that only the benchmark loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Grid-stride 16-byte loads (non-temporal: read once), folded into one word per
// thread so that no load can be dropped.
__global__ void __launch_bounds__(256) read_stream_kernel(const u32x4 *__restrict__ src, size_t n16,
                                                          uint32_t *__restrict__ sink)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        const u32x4 b = __builtin_nontemporal_load(src + i + stride);
        const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16, 16-byte aligned) from device memory src once;
// sink is device memory of blocks * 256 words.  Returns a hipError_t.
extern "C" int hbm_read_probe(const void *src, size_t bytes, uint32_t *sink, int blocks, void *stream)
{
    if (!src || !sink || blocks < 1 || (bytes & 15) || ((uintptr_t)src & 15))
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(read_stream_kernel, dim3(blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       reinterpret_cast<const u32x4 *>(src), bytes / 16, sink);
    return (int)hipGetLastError();
}
