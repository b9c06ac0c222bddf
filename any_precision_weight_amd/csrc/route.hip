// route.hip -- router of the MoE layer (PagedWeight, Section 2.1: the router
// weights E experts per token and selects the top K) and the expert-grouped
// ordering of the selected (token, slot) assignments that the expert products
// consume.
//
// Logits are accumulated in fp64: every product of two fp16 values is exact in
// fp64, so the only rounding is in the additions.  All experts of a token are
// summed in the same order, which makes identical router rows give identical
// logits and lets ties resolve to the lower expert index deterministically.
#include "internal.h"

namespace apmoe {
namespace {

constexpr int kWave = 64;

__device__ inline double h2d(uint16_t h) { return (double)__builtin_bit_cast(_Float16, h); }

// (z, e) ordering: larger logit first, lower expert index on ties.
__device__ inline bool better(double za, int ea, double zb, int eb)
{
    return (za > zb) || (za == zb && ea < eb);
}

// One workgroup per token.  Thread (e, c) sums chunk c of expert e's dot product
// over 8-column units c, c + nch, c + 2*nch, ...; expert e's logit is then the sum of
// its nch partial sums in ascending c.  Every expert uses the same order.
constexpr int kRouteThreads = 256;

template <bool COHERENT>
__device__ __attribute__((always_inline)) inline void route_token(const uint16_t *__restrict__ x,
                                                                 const uint16_t *__restrict__ wr,
                                                                 const float *__restrict__ bias, int t, int H, int E,
                                                                 int topk, int n_shared, int renormalize,
                                                                 int32_t *__restrict__ ids, float *__restrict__ wout)
{
    __shared__ double part[kRouteThreads];
    __shared__ double zs[APMOE_MAX_EXPERTS];
    const int tid = threadIdx.x;
    int nch = 1;
    while (nch * 2 * E <= kRouteThreads)
        nch *= 2;
    const int units = H / 8;
    const uint16_t *xr = x + (size_t)t * H;
    if (tid < E * nch) {
        const int e = tid / nch, c = tid % nch;
        const uint16_t *wrow = wr + (size_t)e * H;
        double acc = 0.0;
#pragma unroll 4
        for (int u = c; u < units; u += nch) {
            const uint4 xv = *reinterpret_cast<const uint4 *>(xr + 8 * u);
            const uint4 wv = *reinterpret_cast<const uint4 *>(wrow + 8 * u);
            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
            const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc += h2d((uint16_t)(xw[i] & 0xFFFFu)) * h2d((uint16_t)(ww[i] & 0xFFFFu));
                acc += h2d((uint16_t)(xw[i] >> 16)) * h2d((uint16_t)(ww[i] >> 16));
            }
        }
        part[tid] = acc;
    }
    __syncthreads();
    for (int e = tid; e < E; e += kRouteThreads) {
        double z = 0.0;
        for (int c = 0; c < nch; ++c)
            z += part[e * nch + c];
        zs[e] = z + (bias ? (double)bias[e] : 0.0);
    }
    __syncthreads();
    if (tid >= kWave)
        return;
    const int lane = tid;

    // top-k: each lane owns experts lane, lane+64, ...
    unsigned taken = 0;  // bit i: expert lane + 64*i selected
    double zsel[APMOE_MAX_TOPK];
    int esel[APMOE_MAX_TOPK];
    for (int j = 0; j < topk; ++j) {
        double bz = -INFINITY;
        int be = 0x7FFFFFFF;
        for (int i = 0; i * kWave + lane < E; ++i) {
            const int e = i * kWave + lane;
            if (taken & (1u << i))
                continue;
            const double z = zs[e];
            if (be == 0x7FFFFFFF || better(z, e, bz, be)) {
                bz = z;
                be = e;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const double oz = __shfl_xor(bz, off, kWave);
            const int oe = __shfl_xor(be, off, kWave);
            if (oe != 0x7FFFFFFF && (be == 0x7FFFFFFF || better(oz, oe, bz, be))) {
                bz = oz;
                be = oe;
            }
        }
        if (be % kWave == lane)
            taken |= 1u << (be / kWave);
        zsel[j] = bz;
        esel[j] = be;
    }
    // Softmax weights, one lane per term: lane j < topk takes choice j's exponential;
    // the denominator is those (renormalize) or every expert's exponential, lane u
    // summing experts u, u + 64, ..., reduced in a fixed tree and taken from lane 0.
    const double zmax = zsel[0];
    double zl = zsel[0];
    int el = esel[0];
#pragma unroll
    for (int j = 1; j < APMOE_MAX_TOPK; ++j)
        if (j < topk && j == lane) {
            zl = zsel[j];
            el = esel[j];
        }
    const double ex = lane < topk ? exp(zl - zmax) : 0.0;
    double term = 0.0;
    if (renormalize) {
        term = ex;
    } else {
        for (int e = lane; e < E; e += kWave)
            term += exp(zs[e] - zmax);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        term += __shfl_xor(term, off, kWave);
    const double den = __shfl(term, 0, kWave);  // lane 0's sum: the same value in every lane
    const int kt = topk + n_shared;  // row: routed choices, then the shared experts (weight 1)
    if (lane < kt) {
        const bool routed = lane < topk;
        const int id = routed ? el : E + (lane - topk);
        if (COHERENT)  // read by the grouping workgroup, maybe on another XCD
            __hip_atomic_store(ids + (size_t)t * kt + lane, id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
            ids[(size_t)t * kt + lane] = id;
        wout[(size_t)t * kt + lane] = routed ? (float)(ex / den) : 1.0f;
    }
}

__global__ void __launch_bounds__(kRouteThreads) route_topk_kernel(const uint16_t *__restrict__ x,
                                                                   const uint16_t *__restrict__ wr,
                                                                   const float *__restrict__ bias, int H, int E,
                                                                   int topk, int n_shared, int renormalize,
                                                                   int32_t *__restrict__ ids,
                                                                   float *__restrict__ wout)
{
    route_token<false>(x, wr, bias, (int)blockIdx.x, H, E, topk, n_shared, renormalize, ids, wout);
}

// Stable counting sort of the R = T*topk assignments by expert, in one
// workgroup of NT threads: per-expert counts, their prefix sums (one wave, 64 experts
// per scan), then per NT-assignment chunk every wave ranks its lanes inside each
// expert with one ballot per distinct expert in the wave, and waves are ordered by a
// prefix over per-wave counts.
template <int NT, bool COHERENT>
__device__ __attribute__((always_inline)) inline void sort_assignments(const int32_t *__restrict__ ids, int R, int E,
                                                                       int32_t *__restrict__ counts,
                                                                       int32_t *__restrict__ offsets,
                                                                       int32_t *__restrict__ perm,
                                                                       int32_t *__restrict__ inv_perm)
{
    constexpr int kWaves = NT / kWave;
    __shared__ int cnt[APMOE_MAX_EXPERTS];
    __shared__ int off[APMOE_MAX_EXPERTS + 1];
    __shared__ int wcnt[kWaves][APMOE_MAX_EXPERTS];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;

    for (int e = tid; e < E; e += NT)
        cnt[e] = 0;
    __syncthreads();
    auto load_id = [&](int a) {
        return COHERENT ? __hip_atomic_load(ids + a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : ids[a];
    };
    // with at most NT assignments each thread reads its one id once for both passes
    const int own = R <= NT && tid < R ? load_id(tid) : -1;
    auto id = [&](int a) { return R <= NT ? own : load_id(a); };
    for (int a = tid; a < R; a += NT) {
        const int e = id(a);
        if (e >= 0 && e < E)
            atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    if (wave == 0) {  // off[e + 1] = cnt[0] + ... + cnt[e]: inclusive scans of 64 experts
        int carry = 0;
        for (int c0 = 0; c0 < E; c0 += kWave) {
            const int e = c0 + lane;
            int x = e < E ? cnt[e] : 0;
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                const int y = __shfl_up(x, d, kWave);
                if (lane >= d)
                    x += y;
            }
            if (e < E)
                off[e + 1] = carry + x;
            carry += __shfl(x, kWave - 1, kWave);
        }
        if (lane == 0)
            off[0] = 0;
    }
    __syncthreads();
    for (int e = tid; e <= E; e += NT) {
        offsets[e] = off[e];
        if (e < E)
            counts[e] = cnt[e];
    }
    __syncthreads();
    for (int e = tid; e < E; e += NT)
        cnt[e] = 0;  // running position inside each expert
    __syncthreads();

    for (int base = 0; base < R; base += NT) {
        const int a = base + tid;
        int e = a < R ? id(a) : -1;
        if (e < 0 || e >= E)
            e = -1;  // never produced by the router; keeps every index in range
        // rank among lower lanes of this wave with the same expert, and whether
        // this lane is the last of its expert in the wave: one ballot per distinct
        // expert (lanes without an assignment form one more group, unused)
        uint64_t same = 0;
        uint64_t todo = __ballot(1);
        while (todo) {
            const int u = __builtin_amdgcn_readlane(e, (int)__builtin_ctzll(todo));
            const uint64_t m = __ballot(e == u);
            if (e == u)
                same = m;
            todo &= ~m;
        }
        const uint64_t below = (1ull << lane) - 1ull;
        const int rank = (int)__builtin_popcountll(same & below);
        const int after = (int)__builtin_popcountll(same & ~below) - 1;
        for (int i = lane; i < E; i += kWave)
            wcnt[wave][i] = 0;
        __syncthreads();
        if (e >= 0 && after == 0)
            wcnt[wave][e] = rank + 1;
        __syncthreads();
        if (e >= 0) {
            int pos = off[e] + cnt[e] + rank;
            for (int w = 0; w < wave; ++w)
                pos += wcnt[w][e];
            perm[pos] = a;
            inv_perm[a] = pos;
        }
        __syncthreads();
        for (int i = tid; i < E; i += NT) {
            int s = 0;
            for (int w = 0; w < kWaves; ++w)
                s += wcnt[w][i];
            cnt[i] += s;
        }
        __syncthreads();
    }
}

constexpr int kSortThreads = 1024;

__global__ void __launch_bounds__(kSortThreads) route_sort_kernel(const int32_t *__restrict__ ids, int R, int E,
                                                                  int32_t *__restrict__ counts,
                                                                  int32_t *__restrict__ offsets,
                                                                  int32_t *__restrict__ perm,
                                                                  int32_t *__restrict__ inv_perm)
{
    sort_assignments<kSortThreads, false>(ids, R, E, counts, offsets, perm, inv_perm);
}

// Route in one launch: workgroup t selects token t's experts as route_topk_kernel
// does, then counts itself done on `done` (a device counter that is zero between
// launches); the workgroup that counts last -- every token's selection is then
// stored -- groups the assignments as route_sort_kernel does and sets `done` back to
// zero.  Each XCD has its own L2: the selected ids are stored and read with
// agent-scope (device-coherent, sc1) accesses, a workgroup's waves wait for those
// stores to complete before the barrier that precedes its count, and the last
// workgroup reads them after its count has returned -- no L2 is written back or
// invalidated.  Same bits as the two launches: the selections are the same code, and
// the grouping is a stable sort, whose result does not depend on the thread count.
__global__ void __launch_bounds__(kRouteThreads) route_fused_kernel(const uint16_t *__restrict__ x,
                                                                    const uint16_t *__restrict__ wr,
                                                                    const float *__restrict__ bias, int T, int H,
                                                                    int E, int topk, int n_shared, int renormalize,
                                                                    int32_t *__restrict__ ids,
                                                                    float *__restrict__ wout, int Et,
                                                                    int32_t *__restrict__ counts,
                                                                    int32_t *__restrict__ offsets,
                                                                    int32_t *__restrict__ perm,
                                                                    int32_t *__restrict__ inv_perm,
                                                                    int32_t *__restrict__ done)
{
    __shared__ int last;
    route_token<true>(x, wr, bias, (int)blockIdx.x, H, E, topk, n_shared, renormalize, ids, wout);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's selections are stored (device-coherent)
    __syncthreads();
    if (threadIdx.x == 0)
        last = __hip_atomic_fetch_add(done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == T - 1;
    __syncthreads();
    if (!last)
        return;
    sort_assignments<kRouteThreads, true>(ids, T * (topk + n_shared), Et, counts, offsets, perm, inv_perm);
    if (threadIdx.x == 0)
        __hip_atomic_store(done, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// Routing statistics (PagedWeight, Section 2.1, Eq. 1 and Section 3.2 "Routing
// statistics"): per expert, the sum of the routing weights of the assignments it
// received and the number of those assignments, plus the sum of all routing
// weights, accumulated into caller-owned fp64 / int64 arrays across calls (the
// routing mass of expert e is mass[e] / total).  One workgroup walks the experts in
// order; each expert's contiguous perm segment is reduced with a fixed thread-strided
// partial sum and a fixed tree, so every call is deterministic.
constexpr int kStatsThreads = 256;

__global__ void __launch_bounds__(kStatsThreads) route_stats_kernel(const float *__restrict__ w,
                                                                    const int32_t *__restrict__ perm,
                                                                    const int32_t *__restrict__ offsets, int E,
                                                                    double *__restrict__ mass, double *__restrict__ total,
                                                                    int64_t *__restrict__ selections)
{
    __shared__ double part[kStatsThreads];
    const int tid = threadIdx.x;
    double batch_total = 0.0;  // thread 0 only
    for (int e = 0; e < E; ++e) {
        const int r0 = offsets[e], r1 = offsets[e + 1];
        double s = 0.0;
        for (int r = r0 + tid; r < r1; r += kStatsThreads)
            s += (double)w[perm[r]];
        part[tid] = s;
        __syncthreads();
        for (int h = kStatsThreads / 2; h > 0; h >>= 1) {
            if (tid < h)
                part[tid] += part[tid + h];
            __syncthreads();
        }
        if (tid == 0) {
            mass[e] += part[0];
            selections[e] += (int64_t)(r1 - r0);
            batch_total += part[0];
        }
        __syncthreads();
    }
    if (tid == 0)
        total[0] += batch_total;
}

}  // namespace

hipError_t launch_route_topk(const uint16_t *x, const uint16_t *wr, const float *bias, int T, int H, int E, int topk,
                             int n_shared, int renormalize, int32_t *ids, float *w, hipStream_t s)
{
    if (T <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(route_topk_kernel, dim3(T), dim3(kRouteThreads), 0, s, x, wr, bias, H, E, topk, n_shared,
                       renormalize, ids, w);
    return hipGetLastError();
}

hipError_t launch_route_fused(const uint16_t *x, const uint16_t *wr, const float *bias, int T, int H, int E,
                              int topk, int n_shared, int renormalize, int32_t *ids, float *w, int32_t *counts,
                              int32_t *offsets, int32_t *perm, int32_t *inv_perm, int32_t *done, hipStream_t s)
{
    hipLaunchKernelGGL(route_fused_kernel, dim3(T), dim3(kRouteThreads), 0, s, x, wr, bias, T, H, E, topk, n_shared,
                       renormalize, ids, w, E + n_shared, counts, offsets, perm, inv_perm, done);
    return hipGetLastError();
}

hipError_t launch_route_stats(const float *w, const int32_t *perm, const int32_t *offsets, int E, double *mass,
                              double *total, int64_t *selections, hipStream_t s)
{
    hipLaunchKernelGGL(route_stats_kernel, dim3(1), dim3(kStatsThreads), 0, s, w, perm, offsets, E, mass, total,
                       selections);
    return hipGetLastError();
}

hipError_t launch_route_sort(const int32_t *ids, int R, int E, int32_t *counts, int32_t *offsets, int32_t *perm,
                             int32_t *inv_perm, hipStream_t s)
{
    hipLaunchKernelGGL(route_sort_kernel, dim3(1), dim3(kSortThreads), 0, s, ids, R, E, counts, offsets, perm,
                       inv_perm);
    return hipGetLastError();
}

}  // namespace apmoe
