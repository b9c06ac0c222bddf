// gemm.hip -- any-precision expert product for every expert of one
// (layer, gate_up|down) in one launch (PagedWeight, Section 3.3: the fused MoE
// kernel reads the bit-planes and LUTs directly and follows the bitwidth of each
// linear-block; Section 3 / Figure 3 caption: a b-bit weight is a subset of the
// overlaid bit-planes plus a per-bitwidth centroid LUT).
//
//   out[r][n] = sum_c in_row(r)[c] * LUT_q[n][code_q(n, c)],  fp32 accumulation,
//   code_q(n, c) = bits of planes 0..q-1 at column c, plane 0 most significant.
//
// Workgroup = 2 x KP waves = 64 weight rows of one expert.  Wave w covers rows
// 32*(w&1) .. +31 and every KP-th 128-column step (w>>1 picks the column part);
// the parts are summed through LDS at the end in a fixed order.  Planes are read in the tiled layout
// (32-row x 128-column tiles of 512 bytes, one tile per wave step and plane).  For
// each step a lane loads, for its row, two words (64 columns) of each of the q
// needed planes (only planes p < q are touched), turns them into 8-bit codes with an 8x8 bit transpose, looks the
// codes up in the row's LUT level q staged in LDS, and feeds the fp16 centroids as
// the A operand of v_mfma_f32_32x32x16_f16 against the expert's tokens (B operand).
// The reduction over columns is a sum, so the order in which columns are assigned
// to MFMA k-slots is free as long as A and B agree.  Plane words of the next step
// are requested one step ahead.  For the down product of a batch whose experts all
// take this product, the workgroups also accumulate the layer output
// (combine_epilogue below).
//
// Token rows reach the B operand through LDS.  A workgroup step is one step of each
// column part; its token tile (2 parts x TOKL token rows x 128 columns, fp16) is
// copied global -> LDS by buffer_load ... lds one step ahead into a second buffer,
// and the four waves share it, so each token chunk is requested once per workgroup
// instead of once per wave with 64 scattered 16-byte pieces per request.  A step ends
// with a wait for the token copy and a workgroup barrier.  Token row jb stores its
// 16-byte chunk c at position c ^ jb, so 16 lanes reading one chunk of 16 rows hit
// distinct banks.
//
// LDS LUT layouts.  Single lookups (q = 5..8; q = 4 with the small LUT region): the
// transposed code byte v has bit p = plane p's bit, i.e. v is the q-bit code with its
// bits reversed; entry LUT_q[n][code] is stored at v*256 + 4*(32*g + i) + 2*t, where
// i is the row within the 32-row tile t and g the lane half.  The 256-byte stride
// lets one v_perm place v above the lane's constant byte to form the address; the
// second copy fills the rest of each 256-byte row.  Gathers are conflict-free: the
// LDS serves a wave in two halves of 32 lanes (lanes 0-31, 32-63), and within a half
// the 32 rows i fall in 32 distinct banks.  With the small (32 KB) region q = 8 keeps
// one copy at (v & 127)*256 + (v & 128) + 4*i + 2*t: bits 0-6 of v in the second
// byte of the address, bit 7 in the first beside the lane's constant (< 128), so one
// v_perm still forms each address from two words masked once per four codes; the
// large (64 KB) region holds both copies at every q.
//
// Pair lookups (q = 3; q = 4 with the large region): one ds_read_b32 returns the
// centroids of two adjacent columns, packed as the A operand needs them.  Two stages
// of bit-field inserts (2-bit digits, then nibbles) turn the q plane words of 32
// columns into 16 pair indices, one per byte: bit 2p + s of index v is plane p's bit
// of column 2m + s (m the pair).  Entry v of row (t, i) sits at v*256 + 128*t + 4*i
// and holds LUT_q[code of the even column] in its low half and the odd column's in
// its high half; its address is again one v_perm.  This replaces the three-stage
// 8x8 transpose, the per-weight address and the packing of two 16-bit gathers.
#include <algorithm>

#include "device.h"

namespace apmoe {
namespace {

// KP: column parts of a workgroup (waves: 2 row tiles x KP), 2 or 4
template <int KP>
constexpr int kThreadsOf = 2 * KP * 64;
constexpr int kRows = kGemmRowsPerBlock;  // 64
constexpr int kStepCols = 128;            // columns per wave step (2 lane halves x 64)
constexpr int kTokTile = 32;
constexpr int kLptExperts = 16;           // launches with at most this many experts rank them on the device
constexpr int kSmallLut = 32 * 1024;      // LUT region sizes (LUTB): q = 4 single lookups, q = 8 one copy
constexpr int kLargeLut = 64 * 1024;      //   q = 4 pair lookups, q = 8 two copies
template <int KP>
constexpr int kRedBytesOf = (KP - 1) * 2 * 16 * kWave * sizeof(float);  // column-part reduction
constexpr int kXRowBytes = kStepCols * 2;                   // one token row of one step (fp16)
constexpr uint32_t kNoWord = 0x20000000u;  // plane word offset past every plane (byte offset 2^31)

struct GemmParams {
    const DevBlock *table;  // layer slice; entry 2*e + kind
    const uint16_t *in;
    const int32_t *perm;
    const int32_t *offsets;
    void *out;
    int kind, E, N, K, topk, gather, out_f32, row_blocks;
    int act;               // gate_up with the activation fused: out = a [rows][N/2] fp16
    CombineArgs comb;      // down product with the output accumulation fused (comb.out != NULL)
    int max_rows;          // decode product: experts with more rows belong to the mid / tile products
    int min_rows;          // mid product: experts with at most this many rows belong to the decode product
    int tokl;              // token rows per pass (8 or 16): the LDS token buffers' size
    uint32_t in_bytes;     // bytes of `in` (buffer range of the B-operand loads)
    uint32_t plane_bytes;  // bytes of one tiled plane
    uint8_t order[APMOE_MAX_EXPERTS];  // experts by committed q, highest first (launches with E > 16)
};

// Work list of the one-launch decode layer (layer_kernel): both products' parameters
// and its counters in the context (LayerSync offsets in internal.h).
struct LayerParams {
    // [APMOE_GATE_UP]: gate_up with the activation fused (act = 1), out = a;
    // [APMOE_DOWN]: down with the output accumulation fused (comb.out set), in = a
    GemmParams p[2];
    int32_t *sync;
    int32_t *done;  // per expert the gate_up pairs done, kLsDoneStride words apart
    int items_gu, items_dn;
};

constexpr int max_i(int a, int b) { return a > b ? a : b; }

// Plane bases are wave-uniform (scalar registers); the per-lane part is a 32-bit
// word offset into the tiled plane, so each load is one buffer_load_dwordx2 with a
// scalar base and a wave reads 512 contiguous bytes per plane.  Plane words are used
// once: the requests are non-temporal (cache policy NT), so the stream does not push
// the token rows, which every row block of the expert reads again, out of the caches.
constexpr int kLoadNT = 2;  // buffer-load cache policy bits: NT
template <int Q>
__device__ inline void load_planes(u32x2 (&w)[Q], const __amdgpu_buffer_rsrc_t (&rs)[Q], uint32_t word)
{
#pragma unroll
    for (int p = 0; p < Q; ++p)
        w[p] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs[p], (int)(word * 4u), 0, kLoadNT));
}

__device__ inline uint32_t bfi32(uint32_t m, uint32_t a, uint32_t b) { return (m & a) | (~m & b); }

// 4 MFMAs over one 32-column word of each needed plane, q = 3 or 4, pair lookups:
// digits of planes 0/1 and 2/3 interleaved into nibbles, nibbles into bytes; p[r]
// byte k is the index of pair 4k + r' (r' = 0, 1, 2, 3 for r = 0, 1, 2, 3 below), the
// columns 8k + 2r', 8k + 2r' + 1.  MFMA b takes the pairs of byte b in column order,
// so its A operand holds columns 8b .. 8b + 7 like the B fragment.
template <int Q, int W, int XOFF>
__device__ inline void group_product_pairs(const u32x2 (&w)[Q], const uint32_t (&xaddr)[8], uint32_t lut_base,
                                           uint32_t lane_const, float16v &acc)
{
    static_assert(Q == 3 || Q == 4, "pair lookups");
    u32x4 xg[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
        xg[b] = lds_b128(xaddr[4 * W + b] + XOFF);
    const uint32_t w0 = w[0][W], w1 = w[1][W], w2 = w[2][W];
    // nibble i of a0 / a1: digit 2i / 2i+1 of planes 0 (bits 0-1) and 1 (bits 2-3)
    const uint32_t a0 = bfi32(0x33333333u, w0, w1 << 2);
    const uint32_t a1 = bfi32(0x33333333u, w0 >> 2, w1);
    uint32_t h0, h1;  // the same for planes 2 and 3 (plane 3 absent at q = 3)
    if constexpr (Q == 4) {
        const uint32_t w3 = w[Q == 4 ? 3 : 0][W];
        h0 = bfi32(0x33333333u, w2, w3 << 2);
        h1 = bfi32(0x33333333u, w2 >> 2, w3);
    } else {
        h0 = w2 & 0x33333333u;
        h1 = (w2 >> 2) & 0x33333333u;
    }
    uint32_t p[4];
    p[0] = bfi32(0x0F0F0F0Fu, a0, h0 << 4);  // digit 4k     -> columns 8k, 8k+1
    p[1] = bfi32(0x0F0F0F0Fu, a1, h1 << 4);  // digit 4k + 1 -> 8k+2, 8k+3
    p[2] = bfi32(0x0F0F0F0Fu, a0 >> 4, h0);  // digit 4k + 2 -> 8k+4, 8k+5
    p[3] = bfi32(0x0F0F0F0Fu, a1 >> 4, h1);  // digit 4k + 3 -> 8k+6, 8k+7
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        u32x4 a;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t addr = __builtin_amdgcn_perm(p[r], lane_const, 0x0C0C0000u | ((4u + b) << 8));
            a[r] = *reinterpret_cast<const __attribute__((address_space(3))) uint32_t *>((uintptr_t)(lut_base + addr));
        }
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, xg[b]), acc,
                                                     0, 0, 0);
    }
}

// 4 MFMAs over one 32-column word of each needed plane, single lookups: 8x8 bit
// transpose, one gather per weight, two gathers packed per A register.
template <int Q, int W, int XOFF, int LUTB>
__device__ inline void group_product(const u32x2 (&w)[Q], const uint32_t (&xaddr)[8], uint32_t lut_base,
                                     uint32_t lane_const, float16v &acc)
{
    u32x4 xg[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
        xg[b] = lds_b128(xaddr[4 * W + b] + XOFF);
    uint32_t d[8];
#pragma unroll
    for (int p = 0; p < 8; ++p)
        d[p] = p < Q ? w[p < Q ? p : 0][W] : 0u;
    transpose_codes<Q>(d);
    // q = 8 in the small region: bits 0-6 of each code byte go to the address's second
    // byte, bit 7 to bit 7 of its first byte beside the lane's constant (replicated in
    // every byte of lane_const): two masks per four codes, then one v_perm per address
    constexpr bool kSplit = Q == 8 && LUTB == kSmallLut;
    uint32_t lo[8];
    if constexpr (kSplit) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            lo[j] = (d[j] & 0x80808080u) | lane_const;
            d[j] &= 0x7F7F7F7Fu;
        }
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        half8 a;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t addr;
            if constexpr (kSplit)
                addr = __builtin_amdgcn_perm(d[j], lo[j], 0x0C0C0000u | ((4u + b) << 8) | (uint32_t)b);
            else
                addr = __builtin_amdgcn_perm(d[j], lane_const, 0x0C0C0000u | ((4u + b) << 8));
            a[j] = *reinterpret_cast<const __attribute__((address_space(3))) _Float16 *>((uintptr_t)(lut_base + addr));
        }
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, __builtin_bit_cast(half8, xg[b]), acc, 0, 0, 0);
    }
}

template <int Q, int LUTB>
constexpr bool kPairs = Q == 3 || (Q == 4 && LUTB == kLargeLut);

// LUT level Q of the block's two 32-row tiles (first rows nA, nB) into LDS (layouts
// in the file header).  first_loads() runs once the LUT requests are out and before
// their data is written, so the caller's first weight requests overlap the LUT's
// latency.
template <int Q, int KP, int LUTB, typename F>
__device__ __attribute__((always_inline)) inline void stage_lut(const __amdgpu_buffer_rsrc_t rl, int nA, int nB,
                                                                int N, int tid, char *smem, F &&first_loads)
{
    if constexpr (kPairs<Q, LUTB>) {
        // pair table: entry (row nl = 32t + i, index v(ce, co)) at v*256 + 4*nl holds
        // LUT[ce] | LUT[co] << 16.  Thread -> row nl = tid % 64 with its row's 2^Q
        // centroids in registers; wave wv writes the entries of the odd-column codes
        // co = wv (mod waves), every even-column code ce: 64 consecutive rows per
        // store, all indices compile-time constants.
        constexpr int C = 1 << Q, NW = kThreadsOf<KP> / kWave;
        const int nl = tid % kRows;
        const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
        const int n = (nl < 32 ? nA : nB) + (nl & 31);
        u32x4 lv[C / 8];
#pragma unroll
        for (int h = 0; h < C / 8; ++h)
            lv[h] = n < N ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                          rl, (int)((((uint32_t)n << Q) + 8u * h) * 2u), 0, 0))
                          : u32x4{0, 0, 0, 0};
        first_loads();
        char *row = smem + 4 * nl;
#pragma unroll
        for (int co = 0; co < C; ++co) {
            if (co % NW != wv)
                continue;
            const uint32_t hi = (lv[co >> 3][(co >> 1) & 3] >> (16 * (co & 1))) << 16;
#pragma unroll
            for (int ce = 0; ce < C; ++ce) {
                const uint32_t lo = (lv[ce >> 3][(ce >> 1) & 3] >> (16 * (ce & 1))) & 0xFFFFu;
                *reinterpret_cast<uint32_t *>(row + pair_index<Q>(ce, co) * 256) = lo | hi;
            }
        }
    } else {
        // 16-byte loads (8 entries of one row); thread -> (row il of both 32-row tiles,
        // chunk ch), so the two tiles' entries of one code, which share a word, are one
        // 32-bit store; the 32 lanes of each half of a wave take 32 consecutive rows
        // (distinct banks)
        constexpr int kItems = 32 * ((1 << Q) / 8);
        constexpr int kPer = (kItems + kThreadsOf<KP> - 1) / kThreadsOf<KP>;
        constexpr int kBatch = kPer < 4 ? kPer : 4;  // items (two loads each) in flight per batch
#pragma unroll
        for (int j0 = 0; j0 < kPer; j0 += kBatch) {
            u32x4 la[kBatch], lb[kBatch];
#pragma unroll
            for (int jj = 0; jj < kBatch; ++jj) {
                const int idx = tid + (j0 + jj) * kThreadsOf<KP>;
                const int il = idx % 32, ch = idx / 32;
                const bool ok = idx < kItems;
                la[jj] = ok && nA + il < N ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rl, (int)((((uint32_t)(nA + il) << Q) + 8u * ch) * 2u), 0, 0))
                                           : u32x4{0, 0, 0, 0};
                lb[jj] = ok && nB + il < N ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rl, (int)((((uint32_t)(nB + il) << Q) + 8u * ch) * 2u), 0, 0))
                                           : u32x4{0, 0, 0, 0};
            }
            if (j0 == 0)
                first_loads();
#pragma unroll
            for (int jj = 0; jj < kBatch; ++jj) {
                const int idx = tid + (j0 + jj) * kThreadsOf<KP>;
                if (idx >= kItems)
                    break;
                const int il = idx % 32, ch = idx / 32;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t sh = 16 * (e & 1);
                    const uint32_t w = ((la[jj][e >> 1] >> sh) & 0xFFFFu) | (((lb[jj][e >> 1] >> sh) & 0xFFFFu) << 16);
                    const uint32_t vp = bitrev((uint32_t)(8 * ch + e), Q);
                    if (Q < 8 || LUTB == kLargeLut) {
                        *reinterpret_cast<uint32_t *>(smem + vp * 256 + 4 * il) = w;
                        *reinterpret_cast<uint32_t *>(smem + vp * 256 + 4 * (32 + il)) = w;
                    } else {
                        *reinterpret_cast<uint32_t *>(smem + (vp & 0x7Fu) * 256 + (vp & 0x80u) + 4 * il) = w;
                    }
                }
            }
        }
    }
}

// Output accumulation fused into the down product (PagedWeight, Section 3.3: the fused
// kernel ends with the output accumulation), for calls whose experts all take the
// decode product.  A workgroup has written rows r0 .. r0 + Me - 1 of y for output
// columns 64 rb .. 64 rb + 63 (fp32).  Token t's output at those columns needs the kt
// rows inv_perm[t kt + j], written by the workgroups of t's kt experts with the same rb,
// which count themselves on cnt[t][rb]; the one that counts last sums
//   out[t][n] = sum_{j < kt} w[t kt + j] * y[inv_perm[t kt + j]][n]
// in j order with one fp32 fma per term from zero and stores it fp16 -- the arithmetic
// of the separate combine launch, so the same bits -- then sets the counter back to
// zero for the next call.
// Each XCD has its own L2.  The rows of y are stored and read with agent-scope
// (device-coherent, sc1) accesses, so no L2 is written back or invalidated: a writing
// wave waits for its stores to complete before the workgroup barrier, the count is an
// agent-scope atomic issued after that barrier, and the last workgroup issues its
// reads after the count has returned.  (Agent-scope release and acquire fences instead
// write back and invalidate a whole L2 per workgroup; the layer was 12-20% slower.)
__device__ __attribute__((always_inline)) inline void combine_epilogue(const GemmParams &P, int rb, int r0, int Me,
                                                                       char *smem)
{
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int N = P.N, kt = P.topk;
    const int NB = (N + kRows - 1) / kRows;
    int *fin = reinterpret_cast<int *>(smem);  // [0]: tokens this workgroup finishes, then their ids
    __builtin_amdgcn_s_waitcnt(wait_vm<0>());  // this wave's rows of y are stored (device-coherent)
    __syncthreads();
    if (wave == 0) {
        const bool mine = lane < Me;  // Me <= kDecodeMaxRows <= 64
        int t = 0, old = -1;
        if (mine) {
            t = P.perm[r0 + lane] / kt;
            old = __hip_atomic_fetch_add(P.comb.cnt + (size_t)t * NB + rb, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
        }
        const bool last = mine && old == kt - 1;
        const uint64_t m = __ballot(last);
        if (last)
            fin[1 + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] = t;
        if (lane == 0)
            fin[0] = (int)__builtin_popcountll(m);
    }
    __syncthreads();
    const int nf = fin[0];
    if (nf == 0)
        return;
    float *y = reinterpret_cast<float *>(P.out);
    for (int o = tid; o < nf * kRows; o += (int)blockDim.x) {
        const int t = fin[1 + o / kRows];
        const int n = rb * kRows + o % kRows;
        if (n < N) {
            float acc = 0.f;
            for (int j = 0; j < kt; ++j) {
                const int a = t * kt + j;
                const float yv = __hip_atomic_load(y + (size_t)P.comb.inv_perm[a] * N + n, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
                acc = __builtin_fmaf(P.comb.w[a], yv, acc);
            }
            reinterpret_cast<_Float16 *>(P.comb.out)[(size_t)t * N + n] = (_Float16)acc;
        }
    }
    if (tid < nf)
        __hip_atomic_store(P.comb.cnt + (size_t)fin[1 + tid] * NB + rb, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Where a block's waves sit in their workgroup and its LDS.  HALVES = 1: a workgroup
// of its own.  HALVES = 2: half HALF of a paired workgroup that runs two 64-row blocks
// of one expert in lockstep (the same steps, token passes and barriers): each half
// stages its own LUT at HALF * LUTB and keeps its own part-sum slots, and the two
// share the token buffers after both LUTs, copied by all of the workgroup's waves.
// COH: the activation epilogue stores `a` device-coherently (sc1), for a later work
// item of the same launch that reads it, maybe on another XCD.
template <int HALVES, int HALF, bool COH>
struct Seat {
    static constexpr int kHalves = HALVES, kHalf = HALF;
    static constexpr bool kCoherent = COH;
};
using Alone = Seat<1, 0, false>;

template <int Q, int TOKL, int KP, int LUTB, typename S = Alone>
__device__ void gemm_block(const GemmParams &P, const DevBlock &blk, int rb, int r0, int Me, char *smem)
{
    const int gtid = threadIdx.x;
    const int tid = gtid - S::kHalf * kThreadsOf<KP>;  // thread of this block
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform (scalar)
    const int gwave = __builtin_amdgcn_readfirstlane(gtid / kWave);  // wave of the workgroup
    const int t = wave & 1, part = wave >> 1;  // row tile, column part
    const int i = lane & 31, g = lane >> 5;
    const int N = P.N, K = P.K;
    // first rows of the block's two 32-row tiles: consecutive, or with the activation
    // fused, gate rows 32rb.. and the matching up rows F + 32rb..
    const int nA = P.act ? 32 * rb : rb * kRows;
    const int nB = P.act ? (N >> 1) + 32 * rb : rb * kRows + 32;
    const int nt = t ? nB : nA;  // this wave's tile
    const int nsteps = K / kStepCols;  // K % 128 == 0
    // a part past the last step (K < 128 KP) must not touch planes or token rows at all
    const bool has_steps = part < nsteps;
    // tiled planes: tile (rt, kt) = rows 32rt.., columns 128kt.., 128 words; this lane
    // reads words 2*lane, 2*lane+1 of each tile.  A row tile past the end (N % 64 in
    // (0, 32]) reads tile row 0; its outputs are not written.
    const int RT = (N + 31) / 32, KT = K / kStepCols;
    const int rt = nt / 32;
    const uint32_t lane_word = ((uint32_t)(rt < RT ? rt : 0) * (uint32_t)KT + (uint32_t)part) * 128u + 2u * lane;
    constexpr uint32_t kNextWords = KP * 128;  // this wave's next step: KP tiles on
    __amdgpu_buffer_rsrc_t rs[Q];
#pragma unroll
    for (int p = 0; p < Q; ++p)
        rs[p] = make_rsrc(blk.plane[p], P.plane_bytes);
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(blk.lut, (uint32_t)N << (Q + 1));
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(P.in, P.in_bytes);

    // a wave whose part has no step here reads nothing: its plane requests fall past the
    // buffer (zeros, no memory traffic), and it still takes part in the barriers
    const uint32_t first_word = has_steps ? lane_word : kNoWord;
    u32x2 wc[Q];
    stage_lut<Q, KP, LUTB>(rl, nA, nB, N, tid, smem + S::kHalf * LUTB, [&] { load_planes<Q>(wc, rs, first_word); });
    __syncthreads();

    // LDS byte addresses (compile-time constants for the static array)
    const uint32_t lds_base = lds_addr(smem) + S::kHalf * LUTB;  // this block's LUT
    const uint32_t lane_const = kPairs<Q, LUTB>             ? (uint32_t)(128 * t + 4 * i)
                                : Q < 8 || LUTB == kLargeLut ? (uint32_t)(4 * (32 * g + i) + 2 * t)
                                                             : (uint32_t)(4 * i + 2 * t) * 0x01010101u;
    char *xs = smem + S::kHalves * LUTB;
    const uint32_t xs_base = lds_addr(smem) + S::kHalves * LUTB;
    // part-sum slots of this block, used after the last token tile is read
    float *red = reinterpret_cast<float *>(xs) + S::kHalf * (kRedBytesOf<KP> / (int)sizeof(float));
    constexpr int kXBuf = KP * TOKL * kXRowBytes;  // one token buffer: KP parts x TOKL rows
    constexpr int kCopies = KP * TOKL / 4;         // copy instructions per buffer (4 token rows each)
    constexpr int kNW = S::kHalves * 2 * KP;       // the waves that share them
    constexpr int kDma = (kCopies + kNW - 1) / kNW;  // token copies per wave and workgroup step
    const int nws = (nsteps + KP - 1) / KP;         // workgroup steps: part p takes step KP s + p

    for (int tp = 0; tp < Me; tp += TOKL) {
        const int j = lane & 31;  // token column of this lane in the B operand and in D
        const bool tok_ok = j < TOKL && tp + j < Me;
        // token copies: instruction u = gwave + kNW k < kCopies fills rows 4u .. 4u+3 of a
        // buffer; lane L writes 16-byte position L % 16 of row 4u + L / 16 (part row / TOKL,
        // token row % TOKL) and fetches the chunk stored there, chunk = position ^ token row
        uint32_t doff[kDma];
#pragma unroll
        for (int k = 0; k < kDma; ++k) {
            // (an instruction number past kCopies is not issued; its row is never used)
            const int row = 4 * (kDma * kNW == kCopies ? gwave + kNW * k : (gwave + kNW * k) % kCopies) + (lane >> 4);
            const int pu = row / TOKL, jj = row % TOKL;
            const int c = (lane & 15) ^ jj;
            const int tok = tp + jj;
            const int src = tok < Me ? (P.gather ? P.perm[r0 + tok] / P.topk : r0 + tok) : 0;
            // rows past the expert's last token request an offset beyond the buffer
            doff[k] = tok < Me ? ((uint32_t)src * (uint32_t)K + (uint32_t)(pu * kStepCols + 8 * c)) * 2u : 0x80000000u;
        }
        // token tile of workgroup step s (columns 128 KP s .. +128 KP - 1) into buffer b;
        // the step is part of the lane offset, so the buffer's range check covers it
        auto copy_tokens = [&](int s, int b) {
#pragma unroll
            for (int k = 0; k < kDma; ++k)
                if (kDma * kNW == kCopies || gwave + kNW * k < kCopies)  // wave-uniform
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rx, (__attribute__((address_space(3))) void *)(xs + b * kXBuf + 1024 * (gwave + kNW * k)),
                        16, doff[k] + (uint32_t)s * (uint32_t)(KP * kStepCols * 2), 0, 0, 0);
        };
        // B-operand addresses in buffer 0: fragment f of word W is chunk 8g + 4W + f of this
        // lane's token row in its part; lanes of token columns >= TOKL repeat a row (their
        // D columns are not written)
        const int jb = j & (TOKL - 1);
        uint32_t xaddr[8];
#pragma unroll
        for (int f = 0; f < 8; ++f)
            xaddr[f] = xs_base + (uint32_t)((part * TOKL + jb) * kXRowBytes + (((8 * g + f) ^ jb) << 4));

        if (tp > 0)
            load_planes<Q>(wc, rs, first_word);
        copy_tokens(0, 0);
        __builtin_amdgcn_s_waitcnt(kWaitAll);
        __syncthreads();

        float16v acc;
#pragma unroll
        for (int v = 0; v < 16; ++v)
            acc[v] = 0.f;
        uint32_t word = first_word;
        // workgroup step s: request the next token tile and this wave's next plane words,
        // multiply, then wait for the token tile only (the plane words stay in flight)
        // and pass the barrier that frees the buffer just read
        auto step_body = [&](const u32x2 (&cur)[Q], u32x2 (&nxt)[Q], int s, auto buf) {
            constexpr int B = decltype(buf)::value;
            const int step = KP * s + part;
            // the wait below counts on the plane requests being issued after the token
            // copies: keep the scheduler from reordering them
            copy_tokens(s + 1 < nws ? s + 1 : s, B ^ 1);
            __builtin_amdgcn_sched_barrier(0);
            word = step + KP < nsteps ? word + kNextWords : kNoWord;
            load_planes<Q>(nxt, rs, word);
            __builtin_amdgcn_sched_barrier(0);
            if (step < nsteps) {
                if constexpr (kPairs<Q, LUTB>) {
                    group_product_pairs<Q, 0, B * kXBuf>(cur, xaddr, lds_base, lane_const, acc);
                    group_product_pairs<Q, 1, B * kXBuf>(cur, xaddr, lds_base, lane_const, acc);
                } else {
                    group_product<Q, 0, B * kXBuf, LUTB>(cur, xaddr, lds_base, lane_const, acc);
                    group_product<Q, 1, B * kXBuf, LUTB>(cur, xaddr, lds_base, lane_const, acc);
                }
            }
            __builtin_amdgcn_s_waitcnt(wait_vm<Q>());
            asm volatile("s_barrier" ::: "memory");
        };
        // two steps per iteration with the plane registers and token buffers in swapped roles
        u32x2 wd[Q];
        for (int s = 0; s < nws; s += 2) {
            step_body(wc, wd, s, std::integral_constant<int, 0>{});
            if (s + 1 >= nws)
                break;
            step_body(wd, wc, s + 1, std::integral_constant<int, 1>{});
        }

        // ---- sum the column parts (fixed order), write rows of this pass ---------
        // every token copy has landed and every wave has passed the last barrier, so the
        // token buffers are free for the part sums
        // part p >= 1 of row tile t writes slot (p - 1, t)
        auto slot = [&](int p, int tt, int v) { return (((p - 1) * 2 + tt) * 16 + v) * kWave + lane; };
        if (part > 0) {
#pragma unroll
            for (int v = 0; v < 16; ++v)
                red[slot(part, t, v)] = acc[v];
        }
        __syncthreads();
        if (part == 0) {
#pragma unroll
            for (int p = 1; p < KP; ++p)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    acc[v] += red[slot(p, t, v)];
        }
        // D layout of the 32x32 MFMA: column j = lane%32, row = 8*(v/4) + 4*(lane/32) + v%4
        if (!P.act) {
            if (part == 0 && tok_ok) {
                // rows nt + 4g + 8(v/4) + v%4 of token row r0 + tp + j: one base, constant offsets
                const size_t o0 = (size_t)(r0 + tp + j) * N + (size_t)(nt + 4 * g);
                const int nleft = N - (nt + 4 * g);
                float *of = reinterpret_cast<float *>(P.out) + o0;
                _Float16 *oh = reinterpret_cast<_Float16 *>(P.out) + o0;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int d = 8 * (v >> 2) + (v & 3);
                    if (d < nleft) {
                        if (P.comb.out)  // read by another workgroup, maybe on another XCD
                            __hip_atomic_store(of + d, acc[v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        else if (P.out_f32)
                            of[d] = acc[v];
                        else
                            oh[d] = (_Float16)acc[v];
                    }
                }
            }
        } else {
            // the up wave hands its fp16-rounded rows to the gate wave of the same lanes
            // through slot (1, up tile) (already read by it; no other wave touches it
            // after the barrier); the gate wave writes a = SiLU(gate) * up
            if (part == 0 && t == 1) {
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    red[slot(1, 1, v)] = (float)(_Float16)acc[v];
            }
            __syncthreads();
            if (part == 0 && t == 0 && tok_ok) {
                // rows f = nA + 4g + 8(v/4) + v%4 < F of token row r0 + tp + j
                _Float16 *oa = reinterpret_cast<_Float16 *>(P.out) + (size_t)(r0 + tp + j) * (size_t)(N >> 1) +
                               (size_t)(nA + 4 * g);
                if constexpr (S::kCoherent) {
                    // the four rows 8(v/4) .. +3 in one 8-byte device-coherent store
#pragma unroll
                    for (int v4 = 0; v4 < 4; ++v4) {
                        half4 h;
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            h[u] = silu_mul((_Float16)acc[4 * v4 + u], (_Float16)red[slot(1, 1, 4 * v4 + u)]);
                        __hip_atomic_store(reinterpret_cast<uint64_t *>(oa + 8 * v4), __builtin_bit_cast(uint64_t, h),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                } else {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const _Float16 up = (_Float16)red[slot(1, 1, v)];
                        oa[8 * (v >> 2) + (v & 3)] = silu_mul((_Float16)acc[v], up);
                    }
                }
            }
        }
        __syncthreads();
    }
    if (P.comb.out)
        combine_epilogue(P, rb, r0, Me, smem);
}

template <int TOKL, int KP, int LUTB, typename S = Alone>
__device__ __attribute__((always_inline)) inline void dispatch_q(const GemmParams &P, const DevBlock &blk, int rb,
                                                                 int r0, int Me, char *smem)
{
    switch (blk.q) {
    case 3: gemm_block<3, TOKL, KP, LUTB, S>(P, blk, rb, r0, Me, smem); break;
    case 4: gemm_block<4, TOKL, KP, LUTB, S>(P, blk, rb, r0, Me, smem); break;
    case 5: gemm_block<5, TOKL, KP, LUTB, S>(P, blk, rb, r0, Me, smem); break;
    case 6: gemm_block<6, TOKL, KP, LUTB, S>(P, blk, rb, r0, Me, smem); break;
    case 7: gemm_block<7, TOKL, KP, LUTB, S>(P, blk, rb, r0, Me, smem); break;
    case 8: gemm_block<8, TOKL, KP, LUTB, S>(P, blk, rb, r0, Me, smem); break;
    default: break;  // unreachable: commit validates q
    }
}

// KIND (APMOE_GATE_UP / APMOE_DOWN) only names the launch, so profiles tell them apart.
// The LDS region is a static array (its address is a compile-time constant, so LUT
// gathers need no base add): LUT, then the token buffers, which the part sums reuse.
template <int TOKL, int KP, int LUTB>
constexpr int kLdsBytes = LUTB + (kRedBytesOf<KP> > 2 * KP * TOKL * kXRowBytes ? kRedBytesOf<KP>
                                                                               : 2 * KP * TOKL * kXRowBytes);

// Workgroup -> (expert e, row block rb).  Workgroup b runs on XCD b % 8, and XCD x
// takes the x-th eighth of every expert's row blocks, so every XCD streams an equal
// share of every expert.  (With e = b % E and E = 8, each expert would run on one
// XCD, and the launch would wait for the XCD with the most planes or token passes.)
// XCD x runs its row blocks expert by expert, longest workgroups first, so the last
// workgroups of the launch (a partial round) are the shortest.  With at most 16
// experts the ranks come from key_of(u), the estimated workgroup length of expert u
// (0 when this launch does not serve it), then the lower index: lane u holds expert
// u's key and every wave computes the ranks.  Above 16 experts the host's order of
// the committed q map is used.  Returns false for grid padding.
// The expert of rank j (0 = longest key first, lower index on ties): with at most 16
// experts lane u holds key_of(u) and every wave computes the ranks; above 16 the host's
// order of the committed q map.  Wave-uniform.
template <typename KeyOf>
__device__ __attribute__((always_inline)) inline int expert_of_rank(const GemmParams &P, const KeyOf &key_of, int j)
{
    if (P.E <= kLptExperts) {
        const int lane = (int)(threadIdx.x % kWave);
        const int key = lane < P.E ? key_of(lane) : 0;
        int rank = 0;
#pragma unroll
        for (int v = 0; v < kLptExperts; ++v) {
            const int kv = __builtin_amdgcn_readlane(key, v);
            rank += v < P.E && (kv > key || (kv == key && v < lane));
        }
        const uint64_t hit = __ballot(lane < P.E && rank == j);  // exactly one lane: ranks are distinct
        return __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
    }
    return P.order[j];
}

template <typename KeyOf>
__device__ __attribute__((always_inline)) inline bool work_item(const GemmParams &P, const KeyOf &key_of, int &e,
                                                                int &rb)
{
    const int r8 = (P.row_blocks + kXcds - 1) / kXcds;
    const int l = (int)(blockIdx.x / kXcds);
    const int j = l / r8;  // rank of the expert
    rb = (int)(blockIdx.x % kXcds) * r8 + l % r8;
    if (j >= P.E || rb >= P.row_blocks)
        return false;
    e = expert_of_rank(P, key_of, j);
    return true;
}

template <int KIND, int TOKL, int KP, int LUTB>
__global__ void __launch_bounds__(kThreadsOf<KP>) __attribute__((amdgpu_waves_per_eu(3))) gemm_kernel(GemmParams P)
{
    __shared__ __attribute__((aligned(16))) char smem[kLdsBytes<TOKL, KP, LUTB>];
    int e, rb;
    const auto key_of = [&](int u) {
        // passes over the weights x (2q + 7), a fit of the measured time per q
        const int mu = P.offsets[u + 1] - P.offsets[u];
        return mu > 0 && mu <= P.max_rows ? (mu + TOKL - 1) / TOKL * (2 * P.table[2 * u + P.kind].q + 7) : 0;
    };
    if (!work_item(P, key_of, e, rb))
        return;  // grid padding
    const int r0 = P.offsets[e];
    const int Me = P.offsets[e + 1] - r0;
    if (Me <= 0 || Me > P.max_rows)
        return;  // expert without tokens (no weight reads), or one for the tile product
    const DevBlock blk = P.table[2 * e + P.kind];
    dispatch_q<TOKL, KP, LUTB>(P, blk, rb, r0, Me, smem);
}

// ---------------------------------------------------------------------------
// Mid product: experts with kDecodeMaxRows + 1 .. kMidMaxRows rows (33..64: experts
// of a skewed decode batch, shared experts of a small batch).  Same result as the
// decode product.  Each weight is decoded once per expert and its fp16 centroids stay
// in registers as the A operand of two MFMAs, one per 32-token tile of the expert.
// (Four token tiles, for experts up to 128 rows, measured slower than the tile
// product there: with one workgroup per CU the waves are bound by LDS latency.)
//
// Workgroup = 8 waves = 128 weight rows (four 32-row tiles) of one expert.  Wave w
// takes row tile w % 4 and word w / 4 of every 128-column step (lane slot 32g + i of
// the tiled layout holds row i's columns 64g .. 64g + 63 in two words), so the two
// waves of a row tile split its columns and are summed through LDS at the end in a
// fixed order.  All eight waves read the same token tile, which is copied global ->
// LDS by buffer_load ... lds.
//
// LDS (112 KB: one workgroup per CU, two waves per SIMD; or, for launches with many
// row blocks, 80 KB for the blocks at q <= 7 -- two workgroups per CU -- and a second
// launch for those at q = 8):
//   [0, L)        LUT level q of the 128 rows (L = 64 KB, or 32 KB for q <= 7 only): entry (row nl, code) at
//                 v*256 + 4*(nl % 64) + 2*(nl / 64), v = the code with its q bits
//                 reversed (the transposed code byte); one v_perm forms an address
//                 for every q (v < 256, lane constant < 256).  Within a 32-lane half
//                 of a wave the 32 rows fall in 32 distinct banks.
//   [L, L + 48 KB) three token buffers of 64 rows x 128 columns fp16; token row r
//                 stores its 16-byte chunk c at position c ^ (r % 16).
// Step s requests the token tile of step s + 2 and the plane words of step s + 2,
// so two steps of plane requests are in flight per wave.
// ---------------------------------------------------------------------------
constexpr int kMidWaves = 8;
constexpr int kMidThreads = kMidWaves * kWave;
constexpr int kMidRows = 128;                              // weight rows per workgroup
// Launch modes: kMidAll takes every q with a 64 KB LUT region (112 KB of LDS: one
// workgroup per CU); kMidLow takes q <= 7 with a 32 KB region (80 KB: two per CU) and
// kMidQ8 the blocks at q = 8 (112 KB), as two launches.
constexpr int kMidAll = 0, kMidLow = 1, kMidQ8 = 2;
template <int MODE>
constexpr int kMidLutBytes = MODE == kMidLow ? 32 * 1024 : 64 * 1024;
constexpr int kMidTT = kMidMaxRows / kTokTile;             // token tiles (2)
constexpr int kMidXBuf = kMidMaxRows * kXRowBytes;         // 16 KB token buffer
constexpr int kMidNxb = 3;                                 // token buffers (steps in flight + 1)
template <int MODE>
constexpr int kMidLds = kMidLutBytes<MODE> + kMidNxb * kMidXBuf;
static_assert(kMidMaxRows % kTokTile == 0 && kMidTT <= 4, "whole 32-token tiles");

// One word of each needed plane (32 columns of the lane's row), non-temporal.
template <int Q>
__device__ inline void load_words(uint32_t (&w)[Q], const __amdgpu_buffer_rsrc_t (&rs)[Q], uint32_t word)
{
#pragma unroll
    for (int p = 0; p < Q; ++p)
        w[p] = __builtin_amdgcn_raw_buffer_load_b32(rs[p], (int)(word * 4u), 0, kLoadNT);
}

// One wave step: the lane's 32 weights (word `cur` of each plane) -> codes -> four
// fp16 A fragments, each multiplied by the B fragments of TT token tiles.  With two
// waves per SIMD the LDS latency must be hidden inside the wave: the lookups and B
// fragments of k-group b + 2 are requested before k-group b multiplies.
template <int Q, int TT, int XOFF>
__device__ inline void mid_group(const uint32_t (&cur)[Q], const uint32_t (&xaddr)[4], uint32_t lut_base,
                                 uint32_t lane_const, float16v (&acc)[TT])
{
    uint32_t d[8];
#pragma unroll
    for (int p = 0; p < 8; ++p)
        d[p] = p < Q ? cur[p < Q ? p : 0] : 0u;
    transpose_codes<Q>(d);
    half8 a[4];
    u32x4 xb[4][TT];
    auto request = [&](auto bb) {
        constexpr int b = decltype(bb)::value;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t addr = __builtin_amdgcn_perm(d[j], lane_const, 0x0C0C0000u | ((4u + b) << 8));
            a[b][j] = *reinterpret_cast<const __attribute__((address_space(3))) _Float16 *>((uintptr_t)(lut_base + addr));
        }
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
            xb[b][tt] = lds_b128(xaddr[b] + (uint32_t)(XOFF + tt * kTokTile * kXRowBytes));
    };
    auto multiply = [&](auto bb) {
        constexpr int b = decltype(bb)::value;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
            acc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[b], __builtin_bit_cast(half8, xb[b][tt]), acc[tt], 0, 0, 0);
    };
    request(std::integral_constant<int, 0>{});
    request(std::integral_constant<int, 1>{});
    __builtin_amdgcn_sched_barrier(0);
    multiply(std::integral_constant<int, 0>{});
    request(std::integral_constant<int, 2>{});
    __builtin_amdgcn_sched_barrier(0);
    multiply(std::integral_constant<int, 1>{});
    request(std::integral_constant<int, 3>{});
    __builtin_amdgcn_sched_barrier(0);
    multiply(std::integral_constant<int, 2>{});
    multiply(std::integral_constant<int, 3>{});
}

template <int Q, int TT, int MODE>
__device__ __attribute__((always_inline)) inline void mid_block(const GemmParams &P, const DevBlock &blk, int rb, int r0,
                                                               int Me, char *smem)
{
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int rt = wave & 3, W = wave >> 2;  // row tile, word of every step
    const int i = lane & 31, g = lane >> 5, j = lane & 31;
    const int N = P.N, K = P.K;
    const int nsteps = K / kStepCols;
    // first rows of the workgroup's two 64-row halves: consecutive, or with the
    // activation fused, gate rows 64rb.. and the matching up rows F + 64rb..
    const int rowA0 = P.act ? 64 * rb : kMidRows * rb;
    const int rowB0 = P.act ? (N >> 1) + 64 * rb : kMidRows * rb + 64;
    const int nt = (rt < 2 ? rowA0 : rowB0) + 32 * (rt & 1);  // this wave's row tile
    // tiled planes: tile (rt, kt) = rows 32rt.., columns 128kt.., 128 words; this lane
    // reads word 2*lane + W of each tile.  A row tile past the end reads tile row 0;
    // its outputs are not written.
    const int RT = (N + 31) / 32, rtg = nt / 32;
    const uint32_t lane_word = (uint32_t)(rtg < RT ? rtg : 0) * (uint32_t)nsteps * 128u + 2u * lane + (uint32_t)W;
    __amdgpu_buffer_rsrc_t rs[Q];
#pragma unroll
    for (int p = 0; p < Q; ++p)
        rs[p] = make_rsrc(blk.plane[p], P.plane_bytes);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(P.in, P.in_bytes);
    const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char *)smem);
    char *xs = smem + kMidLutBytes<MODE>;
    const uint32_t xs_base = lds_base + kMidLutBytes<MODE>;

    // token copies: instruction u = wave + 8k fills rows 4u .. 4u+3 of a buffer; lane L
    // writes 16-byte position L % 16 of row 4u + L / 16 and fetches the chunk stored
    // there, chunk = position ^ (row % 16).  Rows past the expert's last token request
    // an offset beyond the buffer (zeros, no memory traffic).
    uint32_t doff[TT];
#pragma unroll
    for (int k = 0; k < TT; ++k) {
        const int row = 4 * (wave + kMidWaves * k) + (lane >> 4);
        const int c = (lane & 15) ^ (row & 15);
        const int src = row < Me ? (P.gather ? P.perm[r0 + row] / P.topk : r0 + row) : 0;
        doff[k] = row < Me ? ((uint32_t)src * (uint32_t)K + 8u * (uint32_t)c) * 2u : 0x80000000u;
    }
    auto copy_tokens = [&](int s, int b) {
#pragma unroll
        for (int k = 0; k < TT; ++k)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rx, (__attribute__((address_space(3))) void *)(xs + b * kMidXBuf + 1024 * (wave + kMidWaves * k)), 16,
                doff[k] + (uint32_t)s * (uint32_t)(kStepCols * 2), 0, 0, 0);
    };
    // B fragment of k-group b in buffer 0, token tile 0: chunk 8g + 4W + b of token row j
    uint32_t xaddr[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
        xaddr[b] = xs_base + (uint32_t)(j * kXRowBytes + (((8 * g + 4 * W + b) ^ (j & 15)) << 4));

    // plane words of steps 0 and 1 and token tiles of steps 0 and 1 (clamped) first
    uint32_t wr[kMidNxb][Q];
    load_words<Q>(wr[0], rs, lane_word);
    load_words<Q>(wr[1], rs, nsteps > 1 ? lane_word + 128u : kNoWord);
    copy_tokens(0, 0);
    copy_tokens(nsteps > 1 ? 1 : 0, 1);
    // ---- LUT level Q of the 128 rows -> LDS (row pair (pr, pr + 64) shares a word) ----
    {
        const __amdgpu_buffer_rsrc_t rl = make_rsrc(blk.lut, (uint32_t)N << (Q + 1));
        constexpr int kChunksPerRow = (1 << Q) / 8;  // 16-byte chunks of one LUT row
        constexpr int kPairChunks = 64 * kChunksPerRow;
        constexpr int kPer = (kPairChunks + kMidThreads - 1) / kMidThreads;
#pragma unroll
        for (int jj = 0; jj < kPer; ++jj) {
            const int pc = tid + jj * kMidThreads;
            if (pc < kPairChunks) {
                const int pr = pc % 64, ch = pc / 64;
                const int na = rowA0 + pr, nb = rowB0 + pr;
                const u32x4 za = {0, 0, 0, 0};
                const u32x4 la = na < N ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                     rl, (int)((((uint32_t)na << Q) + 8u * ch) * 2u), 0, 0))
                                        : za;
                const u32x4 lb = nb < N ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                     rl, (int)((((uint32_t)nb << Q) + 8u * ch) * 2u), 0, 0))
                                        : za;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t lo = (la[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                    const uint32_t hi = (lb[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                    const uint32_t v = bitrev((uint32_t)(8 * ch + e), Q);
                    *reinterpret_cast<uint32_t *>(smem + v * 256 + 4 * pr) = lo | (hi << 16);
                }
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    __syncthreads();

    const uint32_t lane_const = (uint32_t)(4 * (32 * (rt & 1) + i) + 2 * (rt >> 1));
    float16v acc[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            acc[tt][v] = 0.f;
    // step s (plane set and token buffer s % 3): request the token tile and the plane
    // words of step s + 2 (the token request first), multiply, then wait for the token
    // tile of step s + 1 -- requested one step earlier, before the plane words of step
    // s + 1, the token tile of step s + 2 and the plane words of step s + 2, which stay
    // in flight -- and pass the barrier that frees buffer s % 3 for step s + 3
    auto step_body = [&](int s, auto uu) {
        constexpr int U = decltype(uu)::value;
        constexpr int U2 = (U + 2) % kMidNxb;
        const int s2 = s + U + 2;
        copy_tokens(s2 < nsteps ? s2 : nsteps - 1, U2);
        __builtin_amdgcn_sched_barrier(0);  // the wait below counts on this order
        load_words<Q>(wr[U2], rs, s2 < nsteps ? lane_word + 128u * (uint32_t)s2 : kNoWord);
        __builtin_amdgcn_sched_barrier(0);
        mid_group<Q, TT, U * kMidXBuf>(wr[U], xaddr, lds_base, lane_const, acc);
        __builtin_amdgcn_s_waitcnt(wait_vm<2 * Q + TT>());
        asm volatile("s_barrier" ::: "memory");
    };
    for (int s = 0; s < nsteps; s += kMidNxb) {
        step_body(s, std::integral_constant<int, 0>{});
        if (s + 1 >= nsteps)
            break;
        step_body(s, std::integral_constant<int, 1>{});
        if (s + 2 >= nsteps)
            break;
        step_body(s, std::integral_constant<int, 2>{});
    }
    __builtin_amdgcn_s_waitcnt(kWaitAll);  // the last (repeated) token copy has landed
    __syncthreads();

    // ---- sum the two words of each row tile (word 0 + word 1), write ---------------
    float *red = reinterpret_cast<float *>(xs);
    auto slot = [&](int r, int tt, int v) { return ((r * TT + tt) * 16 + v) * kWave + lane; };
    if (W == 1) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                red[slot(rt, tt, v)] = acc[tt][v];
    }
    __syncthreads();
    if (W == 0) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[tt][v] += red[slot(rt, tt, v)];
    }
    // D layout of the 32x32 MFMA: column j = lane%32, row = 8*(v/4) + 4*(lane/32) + v%4
    if (!P.act) {
        if (W == 0) {
            const int nleft = N - (nt + 4 * g);
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                const int tok = kTokTile * tt + j;
                if (tok < Me) {
                    const size_t o0 = (size_t)(r0 + tok) * N + (size_t)(nt + 4 * g);
                    float *of = reinterpret_cast<float *>(P.out) + o0;
                    _Float16 *oh = reinterpret_cast<_Float16 *>(P.out) + o0;
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int d = 8 * (v >> 2) + (v & 3);
                        if (d < nleft) {
                            if (P.out_f32)
                                of[d] = acc[tt][v];
                            else
                                oh[d] = (_Float16)acc[tt][v];
                        }
                    }
                }
            }
        }
    } else {
        // the up waves (row tiles 2, 3) hand their fp16-rounded rows to the gate waves
        // of the same rows (tiles 0, 1) through the LUT region, no longer read; the gate
        // waves write a = SiLU(gate) * up for rows f = nt + 4g + 8(v/4) + v%4 < F
        float *xch = reinterpret_cast<float *>(smem);
        if (W == 0 && rt >= 2) {
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    xch[slot(rt - 2, tt, v)] = (float)(_Float16)acc[tt][v];
        }
        __syncthreads();
        if (W == 0 && rt < 2) {
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                const int tok = kTokTile * tt + j;
                if (tok < Me) {
                    _Float16 *oa = reinterpret_cast<_Float16 *>(P.out) + (size_t)(r0 + tok) * (size_t)(N >> 1) +
                                   (size_t)(nt + 4 * g);
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        oa[8 * (v >> 2) + (v & 3)] = silu_mul((_Float16)acc[tt][v], (_Float16)xch[slot(rt, tt, v)]);
                }
            }
        }
    }
}

template <int MODE, int TT>
__device__ __attribute__((always_inline)) inline void mid_dispatch_q(const GemmParams &P, const DevBlock &blk, int rb,
                                                                     int r0, int Me, char *smem)
{
    if constexpr (MODE == kMidQ8) {
        if (blk.q == 8)
            mid_block<8, TT, MODE>(P, blk, rb, r0, Me, smem);
    } else {
        switch (blk.q) {
        case 3: mid_block<3, TT, MODE>(P, blk, rb, r0, Me, smem); break;
        case 4: mid_block<4, TT, MODE>(P, blk, rb, r0, Me, smem); break;
        case 5: mid_block<5, TT, MODE>(P, blk, rb, r0, Me, smem); break;
        case 6: mid_block<6, TT, MODE>(P, blk, rb, r0, Me, smem); break;
        case 7: mid_block<7, TT, MODE>(P, blk, rb, r0, Me, smem); break;
        case 8:
            if constexpr (MODE == kMidAll)
                mid_block<8, TT, MODE>(P, blk, rb, r0, Me, smem);
            break;  // kMidLow: the q = 8 launch
        default: break;  // unreachable: commit validates q
        }
    }
}

// P.row_blocks here counts 128-row blocks (with the activation fused: 64 gate rows
// and their 64 up rows).  Experts outside P.min_rows + 1 .. kMidMaxRows rows, and
// blocks of the other launch's bitwidths, return at once.
template <int KIND, int MODE>
__global__ void __launch_bounds__(kMidThreads)
__attribute__((amdgpu_waves_per_eu(MODE == kMidLow ? 4 : 2, MODE == kMidLow ? 4 : 2))) gemm_mid_kernel(GemmParams P)
{
    __shared__ __attribute__((aligned(16))) char smem[kMidLds<MODE>];
    int e, rb;
    const auto key_of = [&](int u) {
        const int mu = P.offsets[u + 1] - P.offsets[u];
        const int q = P.table[2 * u + P.kind].q;
        const bool mine = MODE == kMidAll || (MODE == kMidQ8) == (q == 8);
        return mu > P.min_rows && mu <= kMidMaxRows && mine ? 2 * q + 7 : 0;
    };
    if (!work_item(P, key_of, e, rb))
        return;  // grid padding
    const int r0 = P.offsets[e];
    const int Me = P.offsets[e + 1] - r0;
    if (Me <= P.min_rows || Me > kMidMaxRows)
        return;
    const DevBlock blk = P.table[2 * e + P.kind];
    mid_dispatch_q<MODE, kMidTT>(P, blk, rb, r0, Me, smem);
}

// LUT region of the decode launch.  The large region (pair lookups at q = 4, one
// instruction per q = 8 address) halves the workgroups per CU, and measured slower at
// every q but 4 (q = 5: 137 -> 166 us on the Mixtral decode gate_up): the small one is
// the default; a build may choose the large one (-DAPMOE_DECODE_LUTB=65536).
#ifndef APMOE_DECODE_LUTB
#define APMOE_DECODE_LUTB 32768
#endif
constexpr int kDecodeLut = APMOE_DECODE_LUTB;
static_assert(kDecodeLut == kSmallLut || kDecodeLut == kLargeLut, "LUT region");

// ---------------------------------------------------------------------------
// One-launch decode layer (PagedWeight, Section 3.3: routing, expert activation, down
// projection and output accumulation in one fused kernel; here the launch after the
// one-launch route): the gate_up product with its activation epilogue, then the down
// product with the output accumulation in its epilogue, for batches whose experts all
// take the decode product.  Each 8-wave workgroup takes a ticket from a device counter
// when it starts and runs work item `ticket`:
//   [0, G)      gate_up: expert rank j = i / P2, row-block pair i % P2 (P2 = F / 64).
//               The workgroup's two halves run the pair's two 64-row blocks in
//               lockstep, each as the 4-wave decode workgroup (KP = 2, its own LUT,
//               the token buffers shared), store a device-coherently and count the
//               pair on done[e];
//   [G, G + D)  down: expert rank j = i' / NB, row block i' % NB (NB = H / 64): the
//               8-wave decode workgroup (KP = 4) with the output accumulation, once
//               done[e] = P2 (every row of a the expert reads is stored).
// So the down blocks fill the slots that the last gate_up blocks leave, with no
// launch boundary between the products.  A workgroup waits only for gate_up items,
// which never wait, and a down ticket is drawn only after every gate_up ticket has
// gone to a workgroup that is running, so every wait ends, in whatever order the
// hardware starts the workgroups.  (A bound on the wait far above any item's length
// turns a broken count into a fault flag instead of a hang.)  Rows of a are read only
// after the wait, by plain loads: the launch starts with no line of a in any cache,
// and each 128-byte line of a is written by one workgroup (a pair covers 128 bytes of
// each token row).  The last workgroup to finish sets the counters back to zero.  Each
// block does the arithmetic of the separate gate_up (KP = 2) and down (KP = 4)
// launches, so the bits are theirs.
// ---------------------------------------------------------------------------
template <int TOKL>
constexpr int kLayerLds = max_i(2 * kDecodeLut + max_i(2 * kRedBytesOf<2>, 2 * 2 * TOKL * kXRowBytes),
                                kLdsBytes<TOKL, 4, kDecodeLut>);
constexpr int kLayerSpin = 1 << 21;  // polls before a wait gives up (about a second)

template <int TOKL>
__global__ void __launch_bounds__(kThreadsOf<4>) __attribute__((amdgpu_waves_per_eu(4)))
layer_kernel(LayerParams L)
{
    __shared__ __attribute__((aligned(16))) char smem[kLayerLds<TOKL>];
    // the item number, read by every wave before the item's first barrier: the last 16
    // bytes of the region, which an item first writes after that barrier (token buffers)
    // or not at all
    int *item = reinterpret_cast<int *>(smem + kLayerLds<TOKL> - 16);
    if (threadIdx.x == 0)
        *item = __hip_atomic_fetch_add(L.sync + kLsNext, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int it = __builtin_amdgcn_readfirstlane(*item);
    const int pairs = L.p[APMOE_GATE_UP].row_blocks / 2;
    const int kind = it < L.items_gu ? APMOE_GATE_UP : APMOE_DOWN;
    // the item's parameters, indexed by a kind the compiler cannot see through: one set of
    // scalar registers holds the fields of whichever product the item is
    int ko = __builtin_amdgcn_readfirstlane(kind);
    asm volatile("" : "+s"(ko));
    const GemmParams &P = L.p[ko];
    const int i2 = kind == APMOE_GATE_UP ? it : it - L.items_gu;
    const int nb = kind == APMOE_GATE_UP ? pairs : P.row_blocks;  // work items per expert
    const auto key_of = [&](int u) {
        const int mu = P.offsets[u + 1] - P.offsets[u];
        return mu > 0 && mu <= P.max_rows ? (mu + TOKL - 1) / TOKL * (2 * P.table[2 * u + P.kind].q + 7) : 0;
    };
    if (i2 < P.E * nb) {
        const int e = expert_of_rank(P, key_of, i2 / nb);
        const int rb = i2 % nb;
        const int r0 = P.offsets[e];
        const int Me = P.offsets[e + 1] - r0;
        const DevBlock blk = P.table[2 * e + P.kind];
        if (Me <= 0 || Me > P.max_rows) {
            // no rows: no work, and no down item of this expert waits
        } else if (kind == APMOE_GATE_UP) {
            if (threadIdx.x < kThreadsOf<2>)
                dispatch_q<TOKL, 2, kDecodeLut, Seat<2, 0, true>>(P, blk, 2 * rb, r0, Me, smem);
            else
                dispatch_q<TOKL, 2, kDecodeLut, Seat<2, 1, true>>(P, blk, 2 * rb + 1, r0, Me, smem);
            __builtin_amdgcn_s_waitcnt(wait_vm<0>());  // this wave's rows of a are stored (device-coherent)
            __syncthreads();
            if (threadIdx.x == 0)
                __hip_atomic_fetch_add(L.done + kLsDoneStride * e, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            if (threadIdx.x == 0) {
                // many down workgroups may wait at once: polls back off to one per ~2 k clk,
                // and each expert's count sits on its own 4 KB, so they do not crowd the
                // memory requests of the gate_up workgroups still running
                int n = 0, nap = 1;
                while (__hip_atomic_load(L.done + kLsDoneStride * e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                       pairs) {
                    for (int i = 0; i < nap; ++i)
                        __builtin_amdgcn_s_sleep(8);
                    nap = nap < 4 ? 2 * nap : 4;
                    if (++n >= kLayerSpin) {
                        __hip_atomic_store(L.sync + kLsFault, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                }
            }
            __syncthreads();
            dispatch_q<TOKL, 4, kDecodeLut>(P, blk, rb, r0, Me, smem);
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int old = __hip_atomic_fetch_add(L.sync + kLsExit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old == (int)gridDim.x - 1) {  // every other workgroup is done
            for (int u = 0; u < L.p[APMOE_GATE_UP].E; ++u)
                __hip_atomic_store(L.done + kLsDoneStride * u, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(L.sync + kLsNext, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(L.sync + kLsExit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}



// Gate_up (with the activation) with two 64-row blocks of one expert per 8-wave
// workgroup, the halves in lockstep sharing the token buffers (the layer launch's
// gate_up items, as a launch of its own): the work order of gemm_kernel over pairs
// (P.row_blocks counts pairs here), the arithmetic of its two-column-part workgroups,
// so the same bits.
template <int TOKL>
__global__ void __launch_bounds__(kThreadsOf<4>) __attribute__((amdgpu_waves_per_eu(4))) gemm_pair_kernel(GemmParams P)
{
    __shared__ __attribute__((aligned(16))) char smem[kLayerLds<TOKL>];
    int e, pr;
    const auto key_of = [&](int u) {
        const int mu = P.offsets[u + 1] - P.offsets[u];
        return mu > 0 && mu <= P.max_rows ? (mu + TOKL - 1) / TOKL * (2 * P.table[2 * u + P.kind].q + 7) : 0;
    };
    if (!work_item(P, key_of, e, pr))
        return;
    const int r0 = P.offsets[e];
    const int Me = P.offsets[e + 1] - r0;
    if (Me <= 0 || Me > P.max_rows)
        return;
    const DevBlock blk = P.table[2 * e + APMOE_GATE_UP];
    if (threadIdx.x < kThreadsOf<2>)
        dispatch_q<TOKL, 2, kDecodeLut, Seat<2, 0, false>>(P, blk, 2 * pr, r0, Me, smem);
    else
        dispatch_q<TOKL, 2, kDecodeLut, Seat<2, 1, false>>(P, blk, 2 * pr + 1, r0, Me, smem);
}

template <int KIND, int KP>
void launch_kind(const GemmParams &P, hipStream_t s)
{
    const dim3 grid(kXcds * P.E * ((P.row_blocks + kXcds - 1) / kXcds));
    if (P.tokl == 8)
        hipLaunchKernelGGL((gemm_kernel<KIND, 8, KP, kDecodeLut>), grid, dim3(kThreadsOf<KP>), 0, s, P);
    else
        hipLaunchKernelGGL((gemm_kernel<KIND, 16, KP, kDecodeLut>), grid, dim3(kThreadsOf<KP>), 0, s, P);
}

}  // namespace

static hipError_t launch_mid(const GemmParams &P, int max_q, int act, int N, int E, bool beside, hipStream_t s);

static GemmParams gemm_params(const DevBlock *table, int kind, int E, int N, int K, const uint8_t *order,
                              const uint16_t *in, size_t in_bytes, int gather, const int32_t *perm,
                              const int32_t *offsets, int topk, void *out, int out_f32, int act,
                              const CombineArgs *comb)
{
    GemmParams P;
    P.comb = comb ? *comb : CombineArgs{};
    P.table = table;
    P.in = in;
    P.perm = perm;
    P.offsets = offsets;
    P.out = out;
    P.kind = kind;
    P.E = E;
    P.N = N;
    P.K = K;
    P.topk = topk;
    P.gather = gather;
    P.out_f32 = out_f32;
    P.act = act;
    // with the activation fused a block covers 32 gate rows and the matching 32 up rows
    P.row_blocks = act ? (N / 2) / 32 : (N + kRows - 1) / kRows;
    P.in_bytes = (uint32_t)in_bytes;
    P.plane_bytes = (uint32_t)(tiled_plane_words(N, K) * 4);
    for (int u = 0; u < E; ++u)
        P.order[u] = order ? order[u] : (uint8_t)u;
    P.max_rows = kDecodeMaxRows;
    P.min_rows = 0;
    return P;
}

// Token rows per pass of the decode product's LDS buffers for a batch of `tokens`.
static int decode_tokl(int tokens, int E) { return tokens <= 16 || (E > kLptExperts && tokens <= 64) ? 8 : 16; }

// Four column parts (8-wave workgroups) when the launch has few row blocks.
static bool decode_wide(int row_blocks, int E) { return (long)row_blocks * E <= 4 * 256; }

bool layer_launch_fits(int E, int H, int F, int T)
{
    return T >= 1 && T <= kDecodeMaxRows && E >= 1 && E <= kLptExperts && F % 64 == 0 && !decode_wide(F / 32, E) &&
           decode_wide((H + kRows - 1) / kRows, E);
}

hipError_t launch_layer(const DevBlock *table, int E, int H, int F, const uint16_t *x, const int32_t *perm,
                        const int32_t *offsets, int topk, int T, uint16_t *a, float *y, const CombineArgs &comb,
                        int32_t *sync, int32_t *done, hipStream_t s)
{
    if (!layer_launch_fits(E, H, F, T) || !comb.out)
        return hipErrorInvalidValue;
    const int R = T * topk;
    LayerParams L;
    GemmParams &gu = L.p[APMOE_GATE_UP], &dn = L.p[APMOE_DOWN];
    gu = gemm_params(table, APMOE_GATE_UP, E, 2 * F, H, nullptr, x, (size_t)T * H * 2, 1, perm, offsets, topk, a, 0, 1,
                     nullptr);
    dn = gemm_params(table, APMOE_DOWN, E, H, F, nullptr, a, (size_t)R * F * 2, 0, perm, offsets, topk, y, 1, 0, &comb);
    gu.tokl = dn.tokl = decode_tokl(T, E);
    L.sync = sync;
    L.done = done;
    L.items_gu = E * (gu.row_blocks / 2);
    L.items_dn = E * dn.row_blocks;
    const int grid = L.items_gu + L.items_dn;  // one item per workgroup, in the order they start
    if (gu.tokl == 8)
        hipLaunchKernelGGL(layer_kernel<8>, dim3(grid), dim3(kThreadsOf<4>), 0, s, L);
    else
        hipLaunchKernelGGL(layer_kernel<16>, dim3(grid), dim3(kThreadsOf<4>), 0, s, L);
    return hipGetLastError();
}

hipError_t launch_gemm(const DevBlock *table, int kind, int E, int N, int K, int max_q, const uint8_t *order,
                       const uint16_t *in, size_t in_bytes, int gather, const int32_t *perm, const int32_t *offsets,
                       int topk, int R, void *out, int out_f32, int act, const CombineArgs *comb, hipStream_t s,
                       int cus, const SideStream &side)
{
    GemmParams P = gemm_params(table, kind, E, N, K, order, in, in_bytes, gather, perm, offsets, topk, out, out_f32,
                               act, comb);
    // A token is routed to an expert at most once, so no expert has more rows than the
    // batch has tokens (R / topk; a shared expert has exactly that many).  The token
    // buffers hold 8 rows up to 16 tokens (40 KB of LDS: four workgroups per CU; with 16
    // tokens spread over the experts few have more than 8) and 16 rows above (48 KB,
    // three workgroups); an expert with more rows than the buffers takes further passes
    // over its weights.  The decode product takes experts with up to kDecodeMaxRows
    // rows, the mid product those up to kMidMaxRows, the tile product the rest; the
    // launches that no expert can need (by the token count) are skipped.  (Giving the
    // mid product the experts of 17..32 rows, one pass instead of two, measured slower
    // on a skewed 256-token batch.)
    // Layers with many experts (above 16) spread up to 64 tokens thinly enough that 8-row
    // buffers pay there too (the rare expert with more rows starts first): Qwen-like and
    // Gemma-like 64-token steps 1.6-1.8% faster; an 8-expert 32-token layer with them
    // was 30% slower.
    const int tokens = topk > 0 ? R / topk : R;
    if (P.comb.out && (kind != APMOE_DOWN || !out_f32 || act || tokens > kDecodeMaxRows))
        return hipErrorInvalidValue;  // the fused accumulation needs every expert on the decode product
    P.tokl = decode_tokl(tokens, E);
    // A tile launch of at most two tiles per CU (by its bound) cannot fill the GPU for
    // long, and each of its tiles is long: it runs on the context's side stream beside
    // the decode and mid launches (they serve other experts and write other rows),
    // forked from the caller's stream before them and joined back after, so the call
    // stays ordered on the caller's stream.
    const bool tile = tokens > kMidMaxRows;
    const bool beside = tile && cus > 0 && tile_grid(N, E, R) <= 2 * cus;
    hipError_t err = hipSuccess;
    if (beside) {
        err = hipEventRecord(side.fork, s);
        if (err == hipSuccess)
            err = hipStreamWaitEvent(side.stream, side.fork, 0);
        if (err == hipSuccess)
            err = launch_gemm_tile(table, kind, E, N, K, in, in_bytes, gather, perm, offsets, topk, out, out_f32, act, R,
                                   side.stream);
        if (err == hipSuccess)
            err = hipEventRecord(side.join, side.stream);
        if (err != hipSuccess)
            return err;
    }
    // Few workgroups (the down product's N / 64 row blocks) leave two per CU: four
    // column parts then give each CU four waves per SIMD instead of two.
    const bool wide = decode_wide(P.row_blocks, E);
    // gate_up with 16-row token buffers (above 16 tokens): two 64-row blocks per 8-wave
    // workgroup sharing the token buffers -- four waves per SIMD instead of three and
    // half the token copies per weight, which pays more than the halves' lockstep costs
    // (32-layer step, map A -1.0%, map B -1.3%; the 8x22B layer's decode experts
    // -1.8% of its gate_up); with 8-row buffers (up to 16 tokens, already four waves
    // per SIMD) it measured 8% slower
    const bool pairs = kind == APMOE_GATE_UP && act && !wide && P.tokl == 16 && P.row_blocks % 2 == 0 &&
                       E <= kLptExperts;
    if (pairs) {
        GemmParams Q = P;
        Q.row_blocks = P.row_blocks / 2;
        const dim3 grid(kXcds * E * ((Q.row_blocks + kXcds - 1) / kXcds));
        if (P.tokl == 8)
            hipLaunchKernelGGL(gemm_pair_kernel<8>, grid, dim3(kThreadsOf<4>), 0, s, Q);
        else
            hipLaunchKernelGGL(gemm_pair_kernel<16>, grid, dim3(kThreadsOf<4>), 0, s, Q);
    } else if (kind == APMOE_GATE_UP)
        wide ? launch_kind<APMOE_GATE_UP, 4>(P, s) : launch_kind<APMOE_GATE_UP, 2>(P, s);
    else
        wide ? launch_kind<APMOE_DOWN, 4>(P, s) : launch_kind<APMOE_DOWN, 2>(P, s);
    err = hipGetLastError();
    if (err == hipSuccess && tokens > P.max_rows)
        err = launch_mid(P, max_q, act, N, E, beside, s);
    if (err != hipSuccess || !tile)
        return err;
    if (beside)
        return hipStreamWaitEvent(s, side.join, 0);
    return launch_gemm_tile(table, kind, E, N, K, in, in_bytes, gather, perm, offsets, topk, out, out_f32, act, R, s);
}

// The mid product's launch(es) for the experts with kDecodeMaxRows + 1 .. kMidMaxRows rows.
static hipError_t launch_mid(const GemmParams &P, int max_q, int act, int N, int E, bool beside, hipStream_t s)
{
    hipError_t err = hipSuccess;
    const int kind = P.kind;
    GemmParams M = P;
    M.min_rows = P.max_rows;
    M.row_blocks = act ? (N / 2) / 64 : (N + kMidRows - 1) / kMidRows;
    const dim3 mgrid(kXcds * E * ((M.row_blocks + kXcds - 1) / kXcds));
    // Two workgroups per CU pay where an expert alone has many row blocks (the 8x22B
    // gate_up: 256), and where a tile launch beside this one holds part of the CUs (the
    // 8x22B down: 48 row blocks per expert on the CUs the tile launch leaves, one round
    // instead of two); with few row blocks on the whole GPU they measured slower than
    // one.  The q = 8 launch always follows: q is read from the device table when the
    // kernels run, and its workgroups exit at once when no expert of 33..64 rows is at
    // q = 8.
    (void)max_q;
    if (M.row_blocks >= 128 || beside) {
        if (kind == APMOE_GATE_UP)
            hipLaunchKernelGGL((gemm_mid_kernel<APMOE_GATE_UP, kMidLow>), mgrid, dim3(kMidThreads), 0, s, M);
        else
            hipLaunchKernelGGL((gemm_mid_kernel<APMOE_DOWN, kMidLow>), mgrid, dim3(kMidThreads), 0, s, M);
        err = hipGetLastError();
        if (err == hipSuccess) {
            if (kind == APMOE_GATE_UP)
                hipLaunchKernelGGL((gemm_mid_kernel<APMOE_GATE_UP, kMidQ8>), mgrid, dim3(kMidThreads), 0, s, M);
            else
                hipLaunchKernelGGL((gemm_mid_kernel<APMOE_DOWN, kMidQ8>), mgrid, dim3(kMidThreads), 0, s, M);
            err = hipGetLastError();
        }
    } else {
        if (kind == APMOE_GATE_UP)
            hipLaunchKernelGGL((gemm_mid_kernel<APMOE_GATE_UP, kMidAll>), mgrid, dim3(kMidThreads), 0, s, M);
        else
            hipLaunchKernelGGL((gemm_mid_kernel<APMOE_DOWN, kMidAll>), mgrid, dim3(kMidThreads), 0, s, M);
        err = hipGetLastError();
    }
    return err;
}

}  // namespace apmoe
