// gemm_tile.hip -- any-precision expert product, MFMA tile variant for experts with
// many rows (prefill, hot experts).  Same result as the decode product in gemm.hip
// (PagedWeight, Section 3.3: the fused kernel reads bit-planes and LUTs directly and
// follows each linear-block's bitwidth):
//
//   out[r][n] = sum_c in_row(r)[c] * LUT_q[n][code_q(n, c)],  fp32 accumulation.
//
// The weights are dequantised exactly (an fp16 LUT entry is the fp16 operand), so
// the product is an fp16 MFMA GEMM whose A operand is produced by lookups.
//
// Tile: 128 weight rows x 256 expert rows (tokens), one workgroup of 8 waves with
// split roles (two waves per SIMD, so the decoding VALU work of one overlaps the
// matrix pipe of the other):
//   producer wave p (waves 4..7) decodes weight rows 32p..32p+31: per 64-column
//     stage a lane loads, for each needed plane, one word of its row (same tiled
//     layout as the decode product), turns the 32 columns into codes with an 8x8 bit
//     transpose, looks them up in LUT_q (LDS) and writes the four fp16 A fragments to
//     the stage's A buffer; it also copies its quarter of a later stage's token rows
//     global -> LDS (buffer_load ... lds), one copy after each group of four lookups.
//   consumer wave c (waves 0..3) multiplies weight rows 64(c%2)..+63 (two A row
//     sets) by tokens 128(c/2)..+127 (four token tiles) with v_mfma_f32_32x32x16_f16,
//     2 x 4 x 16 fp32 accumulators per lane; each B fragment serves two A fragments.
// Stage n (word n%2 of 128-column step n/2) is produced in phase n and consumed in
// phase n+1; one workgroup barrier ends each phase, and stage buffers alternate.
//
// LDS (160 KB, one workgroup per CU), in this order (Layout below):
//   LUT_q of the tile's 128 rows, 2^q x 256 bytes (64 KB at q = 8): entry (row nl,
//     code) at v*256 + 4*(nl % 64) + 2*(nl / 64), v = code with its q bits reversed
//     (the transposed code byte), so a lookup address is one v_perm.  q = 3 instead
//     holds a pair table (32 KB): entry (row nl, pair index v) at (nl / 64)*16 KB +
//     v*256 + 4*(nl % 64) with the centroids of two adjacent columns, so one 32-bit
//     gather returns a packed A word (pair_indices3).
//   NXB token stages of 32 KB (three where the LUT leaves room, q <= 7; two at q = 8),
//     each 256 rows x 64 columns fp16; row tr holds eight 16-byte chunks (chunk c =
//     columns 64*(c/4) + 32*s + 8*(c%4) of the step, s the stage's word), stored at
//     chunk c ^ ((tr/2) % 8) so that 16 lanes reading one chunk of 16 consecutive rows
//     hit distinct banks.
//   two 16 KB A stages: fragment (producer p, k-group b) of lane L at
//     ((4p + b) * 64 + L) * 16.
//
// Tile order: weight-row groups of 8 tiles, each with the token tiles of every served
// expert; consecutive tiles run on the same XCD (workgroup b runs on XCD b % 8), so a
// group's weight and token tiles are shared through that XCD's L2, and every XCD
// runs tiles of every expert.
#include "device.h"

namespace apmoe {
namespace {

constexpr int kThreads = 512;  // 4 consumer + 4 producer waves
constexpr int kBN = 128;  // weight rows per tile
constexpr int kBM = kTileTokens;  // token rows per tile (256)
constexpr int kStepCols = 128;
constexpr int kLutBytes = 64 * 1024;
constexpr int kStageBytes = kBM * 64 * 2;  // 32 KB token stage
constexpr int kAStageBytes = 16 * 1024;     // A fragments of one stage
constexpr int kLdsBytes = 160 * 1024;
// q = 3: pair table, two 16 KB regions (the tile's two 64-row halves) of 64 pair
// indices x 256 bytes
constexpr int kPairLutBytes = 32 * 1024;

// LDS layout for bitwidth Q: LUT_Q (2^Q x 256 bytes), then NXB token buffers, then
// two A buffers.  NXB = 3 where the LUT leaves room (Q <= 7), else 2.  A token stage
// is requested D = NXB - 2 phases before the phase it must land in (one buffer is
// being read, one is landing).
template <int Q>
struct Layout {
    static constexpr int kLut = Q == 3 ? kPairLutBytes : (1 << Q) * 256;
    static_assert(kLut <= kLutBytes, "LUT region");
    static constexpr int kNxb = kLut <= 32 * 1024 ? 3 : 2;
    static constexpr int kD = kNxb - 2;
    static constexpr int kX = kLut;
    static constexpr int kA = kX + kNxb * kStageBytes;
    static_assert(kA + 2 * kAStageBytes <= kLdsBytes, "LDS budget");
};
constexpr int kGroupN = 8;  // weight-row tiles per group

struct TileParams {
    const DevBlock *table;  // layer slice; entry 2*e + kind
    const uint16_t *in;
    const int32_t *perm;
    const int32_t *offsets;
    void *out;
    int kind, E, N, K, topk, gather, out_f32, NT, min_rows;
    int act;               // gate_up with the activation fused: out = a [rows][N/2] fp16
    uint32_t in_bytes;     // bytes of `in`
    uint32_t plane_bytes;  // bytes of one tiled plane
};

struct Tile {
    int e, r0, m0, M, n0;
};

// Workgroup -> tile.  Every thread computes the same answer; E <= 256 < blockDim.
// Tile order: weight-row group k (kGroupN weight tiles; the last group the NT % 8
// left), then token tile u over all served experts (expert by expert), then the gs
// weight tiles of the group.  XCD x takes the x-th eighth of that order, so every XCD
// runs tiles of every expert (tile cost depends on the expert's q), and consecutive
// tiles on an XCD share a group's weight tiles and a token tile through its L2.
__device__ __attribute__((always_inline)) bool resolve_tile(const TileParams &P, int *scan, Tile &T)
{
    const int tid = threadIdx.x;
    int mt_e = 0;
    if (tid < P.E) {
        const int me = P.offsets[tid + 1] - P.offsets[tid];
        mt_e = me > P.min_rows ? (me + kBM - 1) / kBM : 0;
    }
    scan[tid] = mt_e;
    __syncthreads();
    for (int d = 1; d < kThreads; d <<= 1) {  // inclusive scan (Hillis-Steele)
        const int v = tid >= d ? scan[tid - d] : 0;
        __syncthreads();
        scan[tid] += v;
        __syncthreads();
    }
    const int MT = scan[kThreads - 1];  // token tiles of all served experts
    const int total = MT * P.NT;
    const int per_xcd = (total + kXcds - 1) / kXcds;
    const int b = blockIdx.x;
    const int local = b / kXcds;
    const int l = (b % kXcds) * per_xcd + local;
    if (local >= per_xcd || l >= total)
        return false;
    const int k = l / (kGroupN * MT);
    const int gs = min(kGroupN, P.NT - kGroupN * k);
    const int rem = l - k * kGroupN * MT;
    const int u = rem / gs;
    const int nt = k * kGroupN + rem % gs;
    // expert: the first e with scan[e] > u
    int e = 0;
    {
        int lo = 0, hi = P.E - 1;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (scan[mid] > u)
                hi = mid;
            else
                lo = mid + 1;
        }
        e = lo;
    }
    const int mt = u - (e > 0 ? scan[e - 1] : 0);
    const int r0 = P.offsets[e];
    const int me = P.offsets[e + 1] - r0;
    // identical in every lane: keep the tile in scalar registers
    T.e = __builtin_amdgcn_readfirstlane(e);
    T.r0 = __builtin_amdgcn_readfirstlane(r0);
    T.m0 = __builtin_amdgcn_readfirstlane(mt * kBM);
    T.M = __builtin_amdgcn_readfirstlane(min(kBM, me - mt * kBM));
    T.n0 = __builtin_amdgcn_readfirstlane(nt * kBN);
    return true;
}

// NT: request with the non-temporal cache policy.  Down-product plane words pass
// through once per token tile and are better kept out of the caches; gate_up ones
// measured faster with the default policy.
template <int Q, bool NT>
__device__ inline void load_planes(u32x2 (&w)[Q], const __amdgpu_buffer_rsrc_t (&rs)[Q], uint32_t word)
{
#pragma unroll
    for (int p = 0; p < Q; ++p)
        w[p] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs[p], (int)(word * 4u), 0, NT ? 2 : 0));
}

// Codes of word W (32 columns) of this lane's row: d[j] byte b = transposed code of
// column 8b + j of the word.
template <int Q, int W>
__device__ inline void word_codes(const u32x2 (&w)[Q], uint32_t (&d)[8])
{
#pragma unroll
    for (int p = 0; p < 8; ++p)
        d[p] = p < Q ? w[p < Q ? p : 0][W] : 0u;
    transpose_codes<Q>(d);
}

// Token stages are copied global -> LDS by the buffer unit (buffer_load ... lds):
// one instruction writes 64 x 16 bytes at consecutive LDS addresses, so producer p,
// instruction u fills rows 64p + 8u .. +7 of a stage, lane L the 16-byte slot L % 8
// of row 64p + 8u + L / 8, and fetches the token chunk stored in that slot.
struct XStage {
    uint32_t off[8];  // byte offset of the lane's chunk (token row + column) for instruction u
};

// Token stage n (word n % 2 of step n / 2, clamped to the last stage) into the LDS
// buffer at `dst` (this producer's quarter).
__device__ inline void x_stage(char *dst, __amdgpu_buffer_rsrc_t rx, const XStage &X, int n, int nst)
{
    n = n < nst ? n : nst - 1;
    const uint32_t step_off = (uint32_t)((n >> 1) * kStepCols * 2 + (n & 1) * 64);  // scalar offset
#pragma unroll
    for (int u = 0; u < 8; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void *)(dst + 1024 * u), 16,
                                                 X.off[u], step_off, 0, 0);
}

// Instruction u of x_stage alone.
__device__ inline void x_stage_u(char *dst, __amdgpu_buffer_rsrc_t rx, const XStage &X, int n, int nst, int u)
{
    n = n < nst ? n : nst - 1;
    const uint32_t step_off = (uint32_t)((n >> 1) * kStepCols * 2 + (n & 1) * 64);  // scalar offset
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void *)(dst + 1024 * u), 16,
                                             X.off[u], step_off, 0, 0);
}

// Workgroup barrier for the phase pipeline.  The wave's LDS accesses are complete
// (lgkmcnt 0) and at most VM vector-memory requests -- token copies into LDS among
// them -- are outstanding; a memory fence here would wait for every token copy, so
// the barrier is an s_barrier with a memory clobber (no compiler reordering of memory
// accesses across it) preceded by explicit waits.
template <int VM>
__device__ inline void phase_barrier()
{
    __builtin_amdgcn_s_waitcnt(wait_vm<VM>());
    asm volatile("s_barrier" ::: "memory");
}

// One LUT entry of the lane's row: code byte b of dj (transposed code) -> the fp16
// bits, zero-extended.  The LUT region starts at LDS address lut_base (a
// compile-time constant: the static array's address, folded into the instruction's
// offset).
__device__ inline uint32_t lookup1(uint32_t dj, int b, uint32_t lane_const, uint32_t lut_base)
{
    const uint32_t addr = __builtin_amdgcn_perm(dj, lane_const, 0x0C0C0000u | ((4u + b) << 8));
    return *(const __attribute__((address_space(3))) uint16_t *)(uintptr_t)(lut_base + addr);
}

// q = 3, pair lookups: the three plane words of the lane's 32 columns -> 16 pair
// indices, one per byte (two stages of bit-field inserts: 2-bit digits of planes 0
// and 1 into nibbles, then plane 2's digits beside them): bit 2p + s of an index is
// plane p's bit of column 2m + s (m the pair), and p[r] byte b indexes the columns
// 8b + 2r, 8b + 2r + 1.  `hsel` (bit 6 of every byte) selects the table region of
// the lane's 64-row half.
__device__ inline void pair_indices3(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t hsel, uint32_t (&p)[4])
{
    const uint32_t a0 = select_bits(0x33333333u, w0, w1 << 2);
    const uint32_t a1 = select_bits(0x33333333u, w0 >> 2, w1);
    const uint32_t h0 = w2 & 0x33333333u;
    const uint32_t h1 = (w2 >> 2) & 0x33333333u;
    p[0] = select_bits(0x0F0F0F0Fu, a0, h0 << 4) | hsel;
    p[1] = select_bits(0x0F0F0F0Fu, a1, h1 << 4) | hsel;
    p[2] = select_bits(0x0F0F0F0Fu, a0 >> 4, h0) | hsel;
    p[3] = select_bits(0x0F0F0F0Fu, a1 >> 4, h1) | hsel;
}

// Producer side of one stage: the lane's 32 weights of word W of `wc` -> four fp16 A
// fragments in the A buffer.  The 32 lookups land in registers of their own and are
// paired only after the last one is requested, so the wave waits for the LDS once;
// `issue` (the phase's vector-memory requests) is sent while they are in flight.
template <int Q, int W, class Issue>
__device__ inline void produce_a(const u32x2 (&wc)[Q], uint32_t lane_const, uint32_t lut_base, uint32_t a_dst,
                                 Issue &&issue)
{
    if constexpr (Q == 3) {
        // 16 gathers of packed pairs; byte 0 of lane_const is the lane's row slot,
        // bit 6 of its byte 1 the region (see pair_indices3)
        uint32_t p[4];
        pair_indices3(wc[0][W], wc[1][W], wc[Q == 3 ? 2 : 0][W], (lane_const >> 8) * 0x01010101u, p);
        const uint32_t slot = lane_const & 0xFFu;
        uint32_t v[4][4];
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int r = 2 * h; r < 2 * h + 2; ++r) {
                    const uint32_t addr = __builtin_amdgcn_perm(p[r], slot, 0x0C0C0000u | ((4u + b) << 8));
                    v[b][r] = *(const __attribute__((address_space(3))) uint32_t *)(uintptr_t)(lut_base + addr);
                }
                __builtin_amdgcn_sched_barrier(0);
                issue(2 * b + h);
                __builtin_amdgcn_sched_barrier(0);
            }
        issue(8);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < 4; ++b)
            lds_store_b128(a_dst + 1024u * b, u32x4{v[b][0], v[b][1], v[b][2], v[b][3]});
        return;
    }
    uint32_t d[8];
    word_codes<Q, W>(wc, d);
    uint32_t v[4][8];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int j = 4 * h; j < 4 * h + 4; ++j)
                v[b][j] = lookup1(d[j], b, lane_const, lut_base);
            __builtin_amdgcn_sched_barrier(0);
            issue(2 * b + h);  // request u of the phase after the u-th group of four gathers
            __builtin_amdgcn_sched_barrier(0);
        }
    issue(8);  // the plane words (even phases)
    __builtin_amdgcn_sched_barrier(0);  // every lookup is requested before the first is used
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        u32x4 a;
#pragma unroll
        for (int m = 0; m < 4; ++m)
            a[m] = v[b][2 * m] | (v[b][2 * m + 1] << 16);
        lds_store_b128(a_dst + 1024u * b, a);
    }
}

// Consumer side of one stage: 4 k-groups x 2 row sets x TTN token tiles.  A
// fragments of the stage and the B fragments of k-group 0 are requested first; the
// B fragments of k-group b+1 are requested while k-group b multiplies (fenced
// bundles of one MFMA and at most one LDS read).
template <int TTN>
__device__ inline void consume(uint32_t a_stage, uint32_t a_lane, uint32_t x_stage, const uint32_t (&bo)[4],
                               float16v (&acc)[2][TTN])
{
    // stage bases are wave-uniform; the per-lane parts are a_lane and bo
    const uint32_t a_src = __builtin_amdgcn_readfirstlane(a_stage) + a_lane;
    const uint32_t x_src = __builtin_amdgcn_readfirstlane(x_stage);
    half8 a[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int b = 0; b < 4; ++b)
            a[h][b] = __builtin_bit_cast(half8, lds_b128(a_src + 4096u * h + 1024u * b));
    uint32_t sb[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
        sb[b] = x_src + bo[b];
    u32x4 xb[2][TTN];
#pragma unroll
    for (int tt = 0; tt < TTN; ++tt)
        xb[0][tt] = lds_b128(sb[0] + 4096u * tt);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int tt = 0; tt < TTN; ++tt) {
                acc[h][tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[h][b], __builtin_bit_cast(half8, xb[b & 1][tt]),
                                                                    acc[h][tt], 0, 0, 0);
                if (h == 0 && b < 3)
                    xb[(b + 1) & 1][tt] = lds_b128(sb[b < 3 ? b + 1 : 3] + 4096u * tt);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
}

// TTN: token tiles per consumer (a power of two, at most 4); consumers whose token
// half holds no row of the tile skip their products.  Rows past the tile's last
// token repeat that token and are not written.
template <int Q, int TTN, int KIND>
__device__ __attribute__((always_inline)) void tile_block(const TileParams &P, const DevBlock &blk, const Tile &T,
                                                          char *smem)
{
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const bool producer = wave >= 4;
    const int pw = wave & 3;  // producer index / consumer index
    const int i = lane & 31, g = lane >> 5;
    const int N = P.N, K = P.K;
    const int KT = K / kStepCols;
    const int KT2 = (KT + 1) & ~1;  // steps rounded up to even (the pipeline runs two per loop)
    const int nst = 2 * KT;         // token stages (one per plane word)
    const uint32_t base = lds_addr(smem);
    // first rows of the tile's two 64-row halves: consecutive, or with the activation
    // fused, gate rows 64nt.. and the matching up rows F + 64nt..
    const int rowA0 = P.act ? (T.n0 >> 1) : T.n0;
    const int rowB0 = P.act ? (N >> 1) + (T.n0 >> 1) : T.n0 + 64;

    // ---- LUT level Q of the tile's rows -> LDS (row pairs nl, nl+64 share a word;
    //      lane -> row pair, so the writes of a wave hit distinct banks) ----------------
    if constexpr (Q == 3) {
        // pair table: entry (row pr of half h, index v(ce, co)) at h * 16 KB + v * 256 +
        // 4 * pr holds LUT[ce] | LUT[co] << 16.  Thread -> (row pr, half h, odd-column
        // codes 2k, 2k + 1): one 16-byte load of the row's 8 centroids, 16 stores, 64
        // consecutive rows per store instruction.
        const __amdgpu_buffer_rsrc_t rl = make_rsrc(blk.lut, (uint32_t)N << (Q + 1));
        const int pr = tid % 64, h = (tid / 64) % 2, k = tid / 128;
        const int n = (h ? rowB0 : rowA0) + pr;
        const u32x4 l = n < N ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       rl, (int)(((uint32_t)n << Q) * 2u), 0, 0))
                              : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int co = 2 * k; co < 2 * k + 2; ++co) {
            const uint32_t hi = (l[co >> 1] >> (16 * (co & 1))) << 16;
#pragma unroll
            for (int ce = 0; ce < 8; ++ce) {
                const uint32_t lo = (l[ce >> 1] >> (16 * (ce & 1))) & 0xFFFFu;
                *(__attribute__((address_space(3))) uint32_t *)(uintptr_t)(base + (uint32_t)h * 16384u +
                                                                           pair_index<3>(ce, co) * 256u + 4u * pr) = lo | hi;
            }
        }
    } else {
        const __amdgpu_buffer_rsrc_t rl = make_rsrc(blk.lut, (uint32_t)N << (Q + 1));
        constexpr int kChunksPerRow = (1 << Q) / 8;  // 16-byte chunks of one row
        constexpr int kPairChunks = 64 * kChunksPerRow;
        constexpr int kPer = (kPairChunks + kThreads - 1) / kThreads;
#pragma unroll
        for (int jj = 0; jj < kPer; ++jj) {
            const int pc = tid + jj * kThreads;
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
                    const uint32_t a = (la[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                    const uint32_t b = (lb[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                    const uint32_t v = bitrev((uint32_t)(8 * ch + e), Q);
                    *(__attribute__((address_space(3))) uint32_t *)(uintptr_t)(base + v * 256u + 4u * pr) = a | (b << 16);
                }
            }
        }
    }

    if (producer) {
        // ---------------------------------------------------------------- producer
        const int RT = (N + 31) / 32;
        const int rt = (pw < 2 ? rowA0 + 32 * pw : rowB0 + 32 * (pw - 2)) / 32;
        const uint32_t lane_word = (uint32_t)(rt < RT ? rt : 0) * (uint32_t)KT * 128u + 2u * lane;
        auto step_word = [&](int st) -> uint32_t { return lane_word + 128u * (uint32_t)(st < KT ? st : KT - 1); };
        __amdgpu_buffer_rsrc_t rs[Q];
#pragma unroll
        for (int p = 0; p < Q; ++p)
            rs[p] = make_rsrc(blk.plane[p], P.plane_bytes);
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(P.in, P.in_bytes);
        XStage X;
        {
            const int slot = lane & 7;
            // chunk c sits in slot c ^ ((tr / 2) % 8); for these rows (tr / 2) % 8 = 4 (u % 2) + lane / 16
            uint32_t col_off[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int c = slot ^ ((4 * h + (lane >> 4)) & 7);
                col_off[h] = (uint32_t)(64 * (c >> 2) + 8 * (c & 3)) * 2u;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int tr = 64 * pw + 8 * u + (lane >> 3);
                const int r = T.r0 + T.m0 + min(tr, T.M - 1);
                const int src = P.gather ? P.perm[r] / P.topk : r;
                X.off[u] = (uint32_t)src * (uint32_t)K * 2u + col_off[u & 1];
            }
        }
        const uint32_t lane_const = Q == 3 ? (uint32_t)(4 * (32 * (pw & 1) + i)) | ((uint32_t)(pw >> 1) << 14)
                                           : (uint32_t)(4 * (32 * (pw & 1) + i) + 2 * (pw >> 1));
        const uint32_t a_dst = base + Layout<Q>::kA + (uint32_t)(pw * 4 * 1024 + lane * 16);
        using L = Layout<Q>;
        constexpr int D = L::kD;
        char *x_dst = smem + L::kX + 8192 * pw;
        u32x2 pa[Q], pb[Q];  // plane words of even / odd steps
        // Phase n: produce A of stage n; request token stage n + D into buffer (n + D) % NXB
        // (last read by the consumers in phase n - 1) and, in even phases, the plane
        // words of step n/2 + 1, in that order.  The copies go out one after each group
        // of four LUT gathers and the plane words after the last gather: the four
        // producers' copies share the CU's vector-memory unit (≈64 B/clk), and issued as
        // one burst before the transpose they held a producer back for hundreds of clocks
        // per phase.  With D = 0 the copies go first, as they must land in the phase they
        // are sent in.  At the end of phase n token stage n must have landed;
        // the requests issued after it are the plane words of its own phase (if even),
        // then those of the D later phases, 8 copies each plus the plane words of the
        // even ones: wait until at most that many are outstanding.
        constexpr int kWaitOdd = 8 * D + Q * (D == 0 ? 0 : 1);
        constexpr int kWaitEven = 8 * D + Q;
        auto xbuf = [&](int n) -> char * { return x_dst + (n % L::kNxb) * kStageBytes; };
        auto phase = [&](auto wtag, const u32x2(&wc)[Q], uint32_t dst, int st, u32x2 *next, int next_step) {
            constexpr int W = decltype(wtag)::value;
            // request u < 8: copy instruction u of token stage st; request 8: the plane words
            auto iss = [&](int u) {
                if (u < 8)
                    x_stage_u(xbuf(st), rx, X, st, nst, u);
                else if (next)
                    load_planes<Q, KIND == APMOE_DOWN>(*reinterpret_cast<u32x2(*)[Q]>(next), rs, step_word(next_step));
            };
            if constexpr (D == 0) {
                for (int u = 0; u < 8; ++u)
                    iss(u);
                __builtin_amdgcn_sched_barrier(0);
                iss(8);
                produce_a<Q, W>(wc, lane_const, base, dst, [](int) {});
            } else {
                produce_a<Q, W>(wc, lane_const, base, dst, iss);
            }
        };
        using W0 = std::integral_constant<int, 0>;
        using W1 = std::integral_constant<int, 1>;
        load_planes<Q, KIND == APMOE_DOWN>(pa, rs, step_word(0));
#pragma unroll
        for (int n = 0; n < D; ++n)
            x_stage(xbuf(n), rx, X, n, nst);
        phase_barrier<Q + 8 * D>();  // the LUT written by all waves is visible
        // phase 0: stage 0 = word 0 of step 0
        phase(W0{}, pa, a_dst, D, pb, 1);
        phase_barrier<kWaitEven>();
        for (int m = 0; m < KT2 / 2; ++m) {
            const int n = 4 * m;
            // phase n+1: stage n+1 = word 1 of step 2m -> A buffer 1
            phase(W1{}, pa, a_dst + kAStageBytes, n + 1 + D, nullptr, 0);
            phase_barrier<kWaitOdd>();
            // phase n+2: stage n+2 = word 0 of step 2m+1 -> A buffer 0
            phase(W0{}, pb, a_dst, n + 2 + D, pa, 2 * m + 2);
            phase_barrier<kWaitEven>();
            // phase n+3: stage n+3 = word 1 of step 2m+1 -> A buffer 1
            phase(W1{}, pb, a_dst + kAStageBytes, n + 3 + D, nullptr, 0);
            phase_barrier<kWaitOdd>();
            // phase n+4: stage n+4 = word 0 of step 2m+2 -> A buffer 0
            phase(W0{}, pa, a_dst, n + 4 + D, pb, 2 * m + 3);
            phase_barrier<kWaitEven>();
        }
        if (P.act)
            __syncthreads();  // the consumers' activation exchange: every wave takes part
        return;
    }

    // -------------------------------------------------------------------- consumer
    const int c = pw;
    const int ntt = (T.M + 31) / 32;
    const bool active = 4 * (c >> 1) < ntt;  // this token half holds rows of the tile
    // B fragment (token tile tt of this half, k-group b): row 128(c/2) + 32tt + j, chunk 4g + b
    uint32_t bo[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
        bo[b] = (uint32_t)((128 * (c >> 1) + i) * 128 + 16 * ((4 * g + b) ^ ((i >> 1) & 7)));
    using L = Layout<Q>;
    const uint32_t a_stage = base + L::kA + (uint32_t)((2 * (c & 1)) * 4 * 1024);  // row sets 2(c%2), +1
    const uint32_t a_lane = (uint32_t)(lane * 16);
    auto xsrc = [&](int s) -> uint32_t { return base + L::kX + (uint32_t)((s % L::kNxb) * kStageBytes); };

    float16v acc[2][TTN];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int tt = 0; tt < TTN; ++tt)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[h][tt][v] = 0.f;

    phase_barrier<0>();  // the LUT written by all waves is visible
    phase_barrier<0>();  // phase 0: stage 0 is being produced
    for (int m = 0; m < KT2 / 2; ++m) {
        const int n = 4 * m;  // phases n+1 .. n+4 consume stages n .. n+3
        if (active)
            consume<TTN>(a_stage, a_lane, xsrc(n), bo, acc);
        phase_barrier<0>();
        if (active)
            consume<TTN>(a_stage + kAStageBytes, a_lane, xsrc(n + 1), bo, acc);
        phase_barrier<0>();
        if (active && n + 2 < nst)
            consume<TTN>(a_stage, a_lane, xsrc(n + 2), bo, acc);
        phase_barrier<0>();
        if (active && n + 3 < nst)
            consume<TTN>(a_stage + kAStageBytes, a_lane, xsrc(n + 3), bo, acc);
        phase_barrier<0>();
    }
    const int j = i;
    if (P.act) {
        // ---- activation fused: consumer c (odd, up rows) hands its fp16-rounded
        //      accumulators to consumer c - 1 (even, the matching gate rows) through the
        //      A buffers, idle after the last phase; the gate consumer writes
        //      a = SiLU(gate) * up for rows f = rowA0 + 32h + 8(v/4) + 4g + v%4 ---------
        _Float16 *xch = reinterpret_cast<_Float16 *>(smem + L::kA);
        auto xi = [&](int h, int tt, int v) { return ((((c >> 1) * 2 + h) * TTN + tt) * 16 + v) * kWave + lane; };
        if (active && (c & 1)) {
#pragma unroll
            for (int tt = 0; tt < TTN; ++tt)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        xch[xi(h, tt, v)] = (_Float16)acc[h][tt][v];
        }
        __syncthreads();
        if (active && !(c & 1)) {
            const int F = N >> 1;
#pragma unroll
            for (int tt = 0; tt < TTN; ++tt) {
                const int tok = 128 * (c >> 1) + 32 * tt + j;
                if (tok < T.M) {
                    const size_t orow = (size_t)(T.r0 + T.m0 + tok) * F;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
#pragma unroll
                        for (int a4 = 0; a4 < 4; ++a4) {
                            half4 hv;
#pragma unroll
                            for (int b = 0; b < 4; ++b)
                                hv[b] = silu_mul((_Float16)acc[h][tt][4 * a4 + b], xch[xi(h, tt, 4 * a4 + b)]);
                            const int f = rowA0 + 32 * h + 8 * a4 + 4 * g;
                            *reinterpret_cast<half4 *>(reinterpret_cast<_Float16 *>(P.out) + orow + f) = hv;
                        }
                    }
                }
            }
        }
        return;
    }
    if (!active)
        return;

    // ---- write: acc[h][tt][v] is token 128(c/2) + 32tt + (lane % 32), weight row
    //      64(c%2) + 32h + 8(v/4) + 4g + v%4; four consecutive rows per store ----------
#pragma unroll
    for (int tt = 0; tt < TTN; ++tt) {
        const int tok = 128 * (c >> 1) + 32 * tt + j;
        if (tok < T.M) {
            const size_t orow = (size_t)(T.r0 + T.m0 + tok) * N;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const int n = (c & 1 ? rowB0 : rowA0) + 32 * h + 8 * a4 + 4 * g;
                    const float16v &A = acc[h][tt];
                    if (P.out_f32) {
                        float *o = reinterpret_cast<float *>(P.out) + orow + n;
                        if ((N & 3) == 0 && n + 3 < N) {
                            *reinterpret_cast<float4 *>(o) = make_float4(A[4 * a4], A[4 * a4 + 1], A[4 * a4 + 2], A[4 * a4 + 3]);
                        } else {
#pragma unroll
                            for (int b = 0; b < 4; ++b)
                                if (n + b < N)
                                    o[b] = A[4 * a4 + b];
                        }
                    } else {
                        _Float16 *o = reinterpret_cast<_Float16 *>(P.out) + orow + n;
                        if ((N & 3) == 0 && n + 3 < N) {
                            half4 hv;
#pragma unroll
                            for (int b = 0; b < 4; ++b)
                                hv[b] = (_Float16)A[4 * a4 + b];
                            *reinterpret_cast<half4 *>(o) = hv;
                        } else {
#pragma unroll
                            for (int b = 0; b < 4; ++b)
                                if (n + b < N)
                                    o[b] = (_Float16)A[4 * a4 + b];
                        }
                    }
                }
            }
        }
    }
}

template <int TTN, int KIND>
__device__ __attribute__((always_inline)) void dispatch_q(const TileParams &P, const DevBlock &blk, const Tile &T,
                                                          char *smem)
{
    switch (blk.q) {
    case 3: tile_block<3, TTN, KIND>(P, blk, T, smem); break;
    case 4: tile_block<4, TTN, KIND>(P, blk, T, smem); break;
    case 5: tile_block<5, TTN, KIND>(P, blk, T, smem); break;
    case 6: tile_block<6, TTN, KIND>(P, blk, T, smem); break;
    case 7: tile_block<7, TTN, KIND>(P, blk, T, smem); break;
    case 8: tile_block<8, TTN, KIND>(P, blk, T, smem); break;
    default: break;  // unreachable: commit validates q
    }
}

template <int KIND>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) tile_kernel(TileParams P)
{
    __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
    Tile T;
    if (!resolve_tile(P, reinterpret_cast<int *>(smem + kLdsBytes - kThreads * sizeof(int)), T))
        return;
    __syncthreads();  // the scan scratch is reused as a token stage
    const DevBlock blk = P.table[2 * T.e + P.kind];
    const int ntt = (T.M + 31) / 32;  // token tiles of the tile (two halves of at most 4)
    if (ntt > 2)
        dispatch_q<4, KIND>(P, blk, T, smem);
    else if (ntt > 1)
        dispatch_q<2, KIND>(P, blk, T, smem);
    else
        dispatch_q<1, KIND>(P, blk, T, smem);
}

}  // namespace

int tile_grid(int N, int E, int R)
{
    const int NT = (N + kBN - 1) / kBN;
    // sum over experts with more than kMidMaxRows rows of ceil(M_e / 256) is at most
    // R / 256 + (number of such experts)
    const int big = min(E, R / (kMidMaxRows + 1));
    const long long tiles = (long long)NT * (R / kBM + big);
    return (int)((tiles + kXcds - 1) / kXcds * kXcds);
}

hipError_t launch_gemm_tile(const DevBlock *table, int kind, int E, int N, int K, const uint16_t *in, size_t in_bytes,
                            int gather, const int32_t *perm, const int32_t *offsets, int topk, void *out, int out_f32,
                            int act, int R, hipStream_t s)
{
    TileParams P;
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
    P.NT = (N + kBN - 1) / kBN;  // with the activation fused: F / 64 tiles of 64 gate + 64 up rows
    P.min_rows = kMidMaxRows;
    P.in_bytes = (uint32_t)in_bytes;
    P.plane_bytes = (uint32_t)(tiled_plane_words(N, K) * 4);
    const int grid = tile_grid(N, E, R);
    if (grid == 0)
        return hipSuccess;
    if (kind == APMOE_GATE_UP)
        hipLaunchKernelGGL(tile_kernel<APMOE_GATE_UP>, dim3(grid), dim3(kThreads), 0, s, P);
    else
        hipLaunchKernelGGL(tile_kernel<APMOE_DOWN>, dim3(grid), dim3(kThreads), 0, s, P);
    return hipGetLastError();
}

}  // namespace apmoe
