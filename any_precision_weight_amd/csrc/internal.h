// internal.h -- declarations shared by the libapmoe HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "apmoe.h"

namespace apmoe {

// One committed linear-block as the kernels see it (device table entry).
// plane[p] (tiled layout, see apmoe_tile_planes) is valid for p < q; lut points at
// level q, fp16 [n][2^q].
struct DevBlock {
    const uint32_t *plane[APMOE_PLANES];
    const uint16_t *lut;
    int32_t q;
    int32_t n;
    int32_t k;
    int32_t present;
};

// Rows of the weight matrix handled by one workgroup of the decode product.
constexpr int kGemmRowsPerBlock = 64;
// Experts with at most kDecodeMaxRows rows use the decode product (one or two passes
// of its token buffers); up to kMidMaxRows the mid product (each weight decoded once
// for two 32-token tiles); larger ones the MFMA tile product.
constexpr int kDecodeMaxRows = 32;
constexpr int kMidMaxRows = 64;

// Expert activation of one (gate, up) pair of fp16 values: SiLU(g) * u with
// SiLU(z) = z / (1 + e^-z), fp32 math (the hardware reciprocal, 1 ulp, instead of a
// correctly rounded divide), fp16 result (RNE).  The activation launch and the
// products' fused epilogue both call this, so the two give identical bits.
__device__ __attribute__((always_inline)) inline _Float16 silu_mul(_Float16 g, _Float16 u)
{
    const float z = (float)g;
    return (_Float16)(z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)) * (float)u);
}
// Token rows per tile of the MFMA tile product.
constexpr int kTileTokens = 256;

// Words of one tiled plane: 32-row x 128-column tiles of 128 words.
inline size_t tiled_plane_words(int n, int k) { return (size_t)((n + 31) / 32) * (k / 128) * 128; }

hipError_t launch_route_topk(const uint16_t *x, const uint16_t *wr, const float *bias, int T, int H, int E, int topk,
                             int n_shared, int renormalize, int32_t *ids, float *w, hipStream_t s);
hipError_t launch_route_sort(const int32_t *ids, int R, int E, int32_t *counts, int32_t *offsets, int32_t *perm,
                             int32_t *inv_perm, hipStream_t s);
hipError_t launch_route_fused(const uint16_t *x, const uint16_t *wr, const float *bias, int T, int H, int E,
                              int topk, int n_shared, int renormalize, int32_t *ids, float *w, int32_t *counts,
                              int32_t *offsets, int32_t *perm, int32_t *inv_perm, int32_t *done, hipStream_t s);
hipError_t launch_route_stats(const float *w, const int32_t *perm, const int32_t *offsets, int E, double *mass,
                              double *total, int64_t *selections, hipStream_t s);

// table points at the (layer) slice: entry for expert e and kind u is table[2*e + u].
// in_bytes: size of `in` (rows x K fp16); must be below 2^31.
// R = T * topk rows in total; experts are split between the decode and the tile
// product by their row count (read on the device).
// act = 1 (gate_up only, F = N/2 a multiple of 64): the epilogue applies silu_mul to
// the fp16-rounded gate row f and up row F + f and writes fp16 a[R][F] to out.
// A stream of the context beside the caller's, and the events that fork work onto it
// from the caller's stream and join it back.
struct SideStream {
    hipStream_t stream = nullptr;
    hipEvent_t fork = nullptr;
    hipEvent_t join = nullptr;
};

int tile_grid(int N, int E, int R);

// order: the E experts by committed q, highest first, lower index on ties (a
// scheduling hint: the decode and mid products of a launch with more than 16 experts start
// the experts in this order; any permutation gives the same result).
// The output accumulation fused into the down product (decode product only: the call
// must have no expert above kDecodeMaxRows rows, i.e. R / topk <= kDecodeMaxRows tokens).
// cnt: (R / topk) x ceil(N / 64) device counters, zero before the call and after it.
struct CombineArgs {
    const float *w = nullptr;          // routing weights [T][topk]
    const int32_t *inv_perm = nullptr;  // [T * topk]
    uint16_t *out = nullptr;           // fp16 [T][N]; NULL: no fused accumulation
    int32_t *cnt = nullptr;
};

hipError_t launch_gemm(const DevBlock *table, int kind, int E, int N, int K, int max_q, const uint8_t *order,
                       const uint16_t *in, size_t in_bytes, int gather, const int32_t *perm, const int32_t *offsets,
                       int topk, int R, void *out, int out_f32, int act, const CombineArgs *comb, hipStream_t s,
                       int cus, const SideStream &side);
// The one-launch decode layer: gate_up with the activation and down with the output
// accumulation in one persistent launch (gemm.hip, layer_kernel), for batches of at most
// kDecodeMaxRows tokens over at most 16 experts whose separate launches would take two
// column parts for gate_up and four for down (the same bits).  Its counters, at `sync`
// (int32, zero before the first launch; every launch leaves them zero except the fault
// flag): the next work item, the workgroups that have finished, and a sticky flag set
// when a wait gave up (a broken count; never expected); at `done`, per expert the
// gate_up pairs done, kLsDoneStride words (4 KB) apart, zero between launches.
constexpr int kLsNext = 0, kLsExit = 1, kLsFault = 2, kLsWords = 4;
constexpr int kLsDoneStride = 1024;
bool layer_launch_fits(int E, int H, int F, int T);
hipError_t launch_layer(const DevBlock *table, int E, int H, int F, const uint16_t *x, const int32_t *perm,
                        const int32_t *offsets, int topk, int T, uint16_t *a, float *y, const CombineArgs &comb,
                        int32_t *sync, int32_t *done, hipStream_t s);
hipError_t launch_gemm_tile(const DevBlock *table, int kind, int E, int N, int K, const uint16_t *in, size_t in_bytes,
                            int gather, const int32_t *perm, const int32_t *offsets, int topk, void *out, int out_f32,
                            int act, int R, hipStream_t s);

hipError_t launch_act(const uint16_t *h, int R, int F, uint16_t *a, hipStream_t s);
hipError_t launch_combine(const void *y, int y_f32, const float *w, const int32_t *inv_perm, int T, int topk, int H,
                          uint16_t *out, hipStream_t s);
hipError_t launch_lut_build(const uint16_t *parent, int n, uint16_t *const *levels, hipStream_t s);
hipError_t launch_tile_planes(const uint32_t *canon, int n, int k, uint32_t *tiled, hipStream_t s);
hipError_t launch_pack_planes(const uint8_t *codes, int n, int k, uint32_t *planes, hipStream_t s);

}  // namespace apmoe
