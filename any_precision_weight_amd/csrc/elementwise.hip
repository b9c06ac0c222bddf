// elementwise.hip -- expert activation, output accumulation and the format tools
// (PagedWeight, Section 3.3: "expert activation ... output accumulation"; Section 3
// / Figure 3 caption: per-bitwidth centroid LUTs over overlaid bit-planes).
#include "fp16_rne.h"
#include "internal.h"

namespace apmoe {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));

// a[r][f] = SiLU(h[r][f]) * h[r][F+f], SiLU(z) = z / (1 + e^-z), fp32 math, fp16 out.
__global__ void __launch_bounds__(256) act_kernel(const uint16_t *__restrict__ h, int R, int F,
                                                  uint16_t *__restrict__ a)
{
    const size_t per_row = (size_t)F / 8;
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)R * per_row)
        return;
    const size_t r = idx / per_row, f = (idx % per_row) * 8;
    const half8 g = __builtin_bit_cast(half8, *reinterpret_cast<const uint4 *>(h + r * 2 * F + f));
    const half8 u = __builtin_bit_cast(half8, *reinterpret_cast<const uint4 *>(h + r * 2 * F + F + f));
    half8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        o[i] = silu_mul(g[i], u[i]);
    }
    *reinterpret_cast<uint4 *>(a + r * F + f) = __builtin_bit_cast(uint4, o);
}

// out[t][n] = sum_j w[t][j] * y[inv_perm[t*k+j]][n], fp32, j ascending, fp16 out.
template <bool F32>
__global__ void __launch_bounds__(256) combine_kernel(const void *__restrict__ y, const float *__restrict__ w,
                                                      const int32_t *__restrict__ inv_perm, int T, int topk, int H,
                                                      uint16_t *__restrict__ out)
{
    const size_t per_row = (size_t)H / 8;
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)T * per_row)
        return;
    const size_t t = idx / per_row, n = (idx % per_row) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < topk; ++j) {
        const float wj = w[t * topk + j];
        const size_t r = (size_t)inv_perm[t * topk + j];
        if (F32) {
            const float4 *yp = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(y) + r * H + n);
            const float4 y0 = yp[0], y1 = yp[1];
            // one fused multiply-add per term (the down product's fused accumulation does
            // the same, for the same bits)
            acc[0] = __builtin_fmaf(wj, y0.x, acc[0]);
            acc[1] = __builtin_fmaf(wj, y0.y, acc[1]);
            acc[2] = __builtin_fmaf(wj, y0.z, acc[2]);
            acc[3] = __builtin_fmaf(wj, y0.w, acc[3]);
            acc[4] = __builtin_fmaf(wj, y1.x, acc[4]);
            acc[5] = __builtin_fmaf(wj, y1.y, acc[5]);
            acc[6] = __builtin_fmaf(wj, y1.z, acc[6]);
            acc[7] = __builtin_fmaf(wj, y1.w, acc[7]);
        } else {
            const half8 yv = __builtin_bit_cast(
                half8, *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(y) + r * H + n));
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[i] = __builtin_fmaf(wj, (float)yv[i], acc[i]);
        }
    }
    half8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        o[i] = (_Float16)acc[i];
    *reinterpret_cast<uint4 *>(out + t * H + n) = __builtin_bit_cast(uint4, o);
}

struct LevelPtrs {
    uint16_t *lv[APMOE_MAX_BITS + 1];
};

// One thread per row: level b = RNE(mean of entries 2c, 2c+1 of level b+1), b = 7..3.
__global__ void __launch_bounds__(256) lut_build_kernel(const uint16_t *__restrict__ parent, int n, LevelPtrs L)
{
    const int row = blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= n)
        return;
    uint16_t cur[256];
    const uint4 *src = reinterpret_cast<const uint4 *>(parent + (size_t)row * 256);
#pragma unroll 4
    for (int i = 0; i < 32; ++i) {
        const uint4 v = src[i];
        cur[8 * i + 0] = v.x & 0xFFFF;
        cur[8 * i + 1] = v.x >> 16;
        cur[8 * i + 2] = v.y & 0xFFFF;
        cur[8 * i + 3] = v.y >> 16;
        cur[8 * i + 4] = v.z & 0xFFFF;
        cur[8 * i + 5] = v.z >> 16;
        cur[8 * i + 6] = v.w & 0xFFFF;
        cur[8 * i + 7] = v.w >> 16;
    }
    for (int b = 7; b >= 3; --b) {
        for (int c = 0; c < (1 << b); ++c) {
            const double m = ((double)__builtin_bit_cast(_Float16, cur[2 * c]) +
                              (double)__builtin_bit_cast(_Float16, cur[2 * c + 1])) * 0.5;
            cur[c] = apmoe_d2h_rne(m);
        }
        if (L.lv[b]) {
            uint16_t *dst = L.lv[b] + (size_t)row * (1u << b);
            for (int c = 0; c < (1 << b); ++c)
                dst[c] = cur[c];
        }
    }
}

// One thread per (row, 32-column word): plane p bit j = bit (7-p) of code 32w+j.
__global__ void __launch_bounds__(256) pack_planes_kernel(const uint8_t *__restrict__ codes, int n, int k,
                                                          uint32_t *__restrict__ planes)
{
    const int kw = k / 32;
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)n * kw)
        return;
    const size_t row = idx / kw, w = idx % kw;
    const uint8_t *c = codes + row * k + w * 32;
    uint32_t out[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = 0; j < 32; ++j) {
        const uint32_t v = c[j];
#pragma unroll
        for (int p = 0; p < 8; ++p)
            out[p] |= ((v >> (7 - p)) & 1u) << j;
    }
#pragma unroll
    for (int p = 0; p < 8; ++p)
        planes[((size_t)p * n + row) * kw + w] = out[p];
}

// Canonical planes uint32 [8][n][k/32] -> tiled planes, 8 x tiled_words(n, k).
// Tile (rt, kt) of a plane covers rows 32rt..32rt+31 and columns 128kt..128kt+127
// in 128 words; lane slot L = 32g + i holds row i, columns 64g..64g+63 in words
// 2L (columns 64g..64g+31) and 2L+1.  Rows past n are zero.
__global__ void __launch_bounds__(256) tile_planes_kernel(const uint32_t *__restrict__ canon, int n, int k,
                                                          uint32_t *__restrict__ tiled, size_t plane_words)
{
    const int kw = k / 32, kt_count = k / 128, rt_count = (n + 31) / 32;
    const size_t per_plane = (size_t)rt_count * kt_count * 64;  // lane slots per plane
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= 8 * per_plane)
        return;
    const int p = (int)(idx / per_plane);
    const size_t rem = idx % per_plane;
    const size_t tile = rem / 64;
    const int L = (int)(rem % 64);
    const int rt = (int)(tile / kt_count), kt = (int)(tile % kt_count);
    const int i = L & 31, g = L >> 5;
    const int row = 32 * rt + i;
    uint32_t w0 = 0, w1 = 0;
    if (row < n) {
        const uint32_t *src = canon + ((size_t)p * n + row) * kw + 4 * kt + 2 * g;
        w0 = src[0];
        w1 = src[1];
    }
    uint32_t *dst = tiled + (size_t)p * plane_words + tile * 128 + 2 * L;
    dst[0] = w0;
    dst[1] = w1;
}

inline unsigned blocks_for(size_t work, unsigned threads) { return (unsigned)((work + threads - 1) / threads); }

}  // namespace

hipError_t launch_act(const uint16_t *h, int R, int F, uint16_t *a, hipStream_t s)
{
    const size_t work = (size_t)R * (F / 8);
    if (work == 0)
        return hipSuccess;
    hipLaunchKernelGGL(act_kernel, dim3(blocks_for(work, 256)), dim3(256), 0, s, h, R, F, a);
    return hipGetLastError();
}

hipError_t launch_combine(const void *y, int y_f32, const float *w, const int32_t *inv_perm, int T, int topk, int H,
                          uint16_t *out, hipStream_t s)
{
    const size_t work = (size_t)T * (H / 8);
    if (work == 0)
        return hipSuccess;
    if (y_f32)
        hipLaunchKernelGGL(combine_kernel<true>, dim3(blocks_for(work, 256)), dim3(256), 0, s, y, w, inv_perm, T,
                           topk, H, out);
    else
        hipLaunchKernelGGL(combine_kernel<false>, dim3(blocks_for(work, 256)), dim3(256), 0, s, y, w, inv_perm, T,
                           topk, H, out);
    return hipGetLastError();
}

hipError_t launch_lut_build(const uint16_t *parent, int n, uint16_t *const *levels, hipStream_t s)
{
    if (n == 0)
        return hipSuccess;
    LevelPtrs L;
    for (int b = 0; b <= APMOE_MAX_BITS; ++b)
        L.lv[b] = (b >= 3 && b <= 7) ? levels[b] : nullptr;
    hipLaunchKernelGGL(lut_build_kernel, dim3(blocks_for((size_t)n, 256)), dim3(256), 0, s, parent, n, L);
    return hipGetLastError();
}

hipError_t launch_tile_planes(const uint32_t *canon, int n, int k, uint32_t *tiled, hipStream_t s)
{
    const size_t per_plane = (size_t)((n + 31) / 32) * (k / 128) * 64;
    const size_t work = 8 * per_plane;
    if (work == 0)
        return hipSuccess;
    hipLaunchKernelGGL(tile_planes_kernel, dim3(blocks_for(work, 256)), dim3(256), 0, s, canon, n, k, tiled,
                       per_plane * 2);
    return hipGetLastError();
}

hipError_t launch_pack_planes(const uint8_t *codes, int n, int k, uint32_t *planes, hipStream_t s)
{
    const size_t work = (size_t)n * (k / 32);
    if (work == 0)
        return hipSuccess;
    hipLaunchKernelGGL(pack_planes_kernel, dim3(blocks_for(work, 256)), dim3(256), 0, s, codes, n, k, planes);
    return hipGetLastError();
}

}  // namespace apmoe
