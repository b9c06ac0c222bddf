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
// are requested one step ahead.
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
// LDS LUT layout: the transposed code byte v has bit p = plane p's bit, i.e. v is
// the q-bit code with its bits reversed; entry LUT_q[n][code] is stored at
// v*256 + 4*(32*g + i) + 2*t for q <= 7, where i is the row within the 32-row tile
// t and g the lane half.  The 256-byte stride lets one v_perm place v above the
// lane's constant byte to form the address; the second copy fills the rest of
// each 256-byte row.  Gathers are conflict-free: the LDS serves a wave in two
// halves of 32 lanes (lanes 0-31, 32-63), and within a half the 32 rows i fall in
// 32 distinct banks.  For q = 8 one copy at v*128 + 4*i + 2*t keeps the region at
// 32 KB (two instructions per address).
#include "internal.h"

namespace apmoe {
namespace {

constexpr int kWave = 64;
// KP: column parts of a workgroup (waves: 2 row tiles x KP), 2 or 4
template <int KP>
constexpr int kThreadsOf = 2 * KP * 64;
constexpr int kRows = kGemmRowsPerBlock;  // 64
constexpr int kStepCols = 128;            // columns per wave step (2 lane halves x 64)
constexpr int kTokTile = 32;
constexpr int kXcds = 8;                  // accelerator complex dies; workgroup b runs on XCD b % 8
constexpr int kLutBytes = 32 * 1024;                       // LUT region, every q
template <int KP>
constexpr int kRedBytesOf = (KP - 1) * 2 * 16 * kWave * sizeof(float);  // column-part reduction
constexpr int kXRowBytes = kStepCols * 2;                   // one token row of one step (fp16)
constexpr uint32_t kNoWord = 0x20000000u;  // plane word offset past every plane (byte offset 2^31)
// s_waitcnt operands (vmcnt in bits 3:0 and 15:14, expcnt 6:4 left open, lgkmcnt 11:8)
constexpr int kWaitAll = 7 << 4;
template <int VM>
constexpr int wait_vm()
{
    static_assert(VM >= 0 && VM < 16, "vmcnt range");
    return VM | (7 << 4);
}

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource (base, byte range) in scalar registers: loads take a 32-bit lane
// offset and return zeros past the range.  Word 3 is the gfx9-family raw-buffer
// configuration.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ inline uint32_t bitrev(uint32_t c, int q) { return __builtin_bitreverse32(c) >> (32 - q); }

// In-place transpose of 4 independent 8x8 bit blocks: on input d[p] byte b bit j is
// plane p, column 8b+j; on output d[j] byte b bit p holds the same bit.
// Exchange the bits of b under m with the bits of a under m << s.  BFI: two
// bit-field inserts from the original pair (four instructions); otherwise the xor
// form (five), which the compiler folds further when some words are known zero.
template <bool BFI>
__device__ inline void swap_bits(uint32_t &a, uint32_t &b, int s, uint32_t m)
{
    if constexpr (BFI) {
        const uint32_t nb = (m & (a >> s)) | (~m & b);
        const uint32_t na = ((m << s) & (b << s)) | (~(m << s) & a);
        a = na;
        b = nb;
    } else {
        const uint32_t t = ((a >> s) ^ b) & m;
        b ^= t;
        a ^= t << s;
    }
}

template <bool BFI>
__device__ inline void transpose8x8(uint32_t (&d)[8])
{
    swap_bits<BFI>(d[0], d[4], 4, 0x0F0F0F0Fu);
    swap_bits<BFI>(d[1], d[5], 4, 0x0F0F0F0Fu);
    swap_bits<BFI>(d[2], d[6], 4, 0x0F0F0F0Fu);
    swap_bits<BFI>(d[3], d[7], 4, 0x0F0F0F0Fu);
    swap_bits<BFI>(d[0], d[2], 2, 0x33333333u);
    swap_bits<BFI>(d[1], d[3], 2, 0x33333333u);
    swap_bits<BFI>(d[4], d[6], 2, 0x33333333u);
    swap_bits<BFI>(d[5], d[7], 2, 0x33333333u);
    swap_bits<BFI>(d[0], d[1], 1, 0x55555555u);
    swap_bits<BFI>(d[2], d[3], 1, 0x55555555u);
    swap_bits<BFI>(d[4], d[5], 1, 0x55555555u);
    swap_bits<BFI>(d[6], d[7], 1, 0x55555555u);
}

struct GemmParams {
    const DevBlock *table;  // layer slice; entry 2*e + kind
    const uint16_t *in;
    const int32_t *perm;
    const int32_t *offsets;
    void *out;
    int kind, E, N, K, topk, gather, out_f32, row_blocks;
    int act;               // gate_up with the activation fused: out = a [rows][N/2] fp16
    int max_rows;          // experts with more rows belong to the tile product
    int tokl;              // token rows per pass (8 or 16): the LDS token buffers' size
    uint32_t in_bytes;     // bytes of `in` (buffer range of the B-operand loads)
    uint32_t plane_bytes;  // bytes of one tiled plane
};

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

// One B fragment (8 fp16 columns of one token row) from the LDS token buffer.
__device__ inline u32x4 lds_b128(uint32_t addr)
{
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4 *>((uintptr_t)addr);
}

// 4 MFMAs over one 32-column word of each needed plane: unpack, LUT gather, multiply.
// q = 3, two weights per lookup: the transpose input is the 3 plane words and the
// same words shifted down one column, so output byte b of d[j] (j even) holds the
// transposed codes of columns 8b+j (bits 0..2) and 8b+j+1 (bits 3..5) -- an index
// into the pair table of LUT_3 (entry = two fp16, the even column's in the low half).
// One ds_read_b32 per pair yields two A-operand elements with no repacking.
template <int W, int XOFF>
__device__ inline void group_product_pair3(const u32x2 (&w)[3], const uint32_t (&xaddr)[8], uint32_t lut_base,
                                           uint32_t lane_const, float16v &acc)
{
    u32x4 xg[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
        xg[b] = lds_b128(xaddr[4 * W + b] + XOFF);
    uint32_t d[8];
#pragma unroll
    for (int p = 0; p < 3; ++p) {
        d[p] = w[p][W];
        d[3 + p] = w[p][W] >> 1;
    }
    d[6] = d[7] = 0u;
    transpose8x8<true>(d);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        u32x4 a;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const uint32_t addr = __builtin_amdgcn_perm(d[2 * jj], lane_const, 0x0C0C0000u | ((4u + b) << 8));
            a[jj] = *reinterpret_cast<const __attribute__((address_space(3))) uint32_t *>((uintptr_t)(lut_base + addr));
        }
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, xg[b]), acc,
                                                     0, 0, 0);
    }
}

template <int Q, int W, int XOFF>
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
    transpose8x8<Q == 8>(d);  // the form with fewer instructions after folding (counted per q)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        half8 a;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t addr;
            if (Q < 8)
                addr = __builtin_amdgcn_perm(d[j], lane_const, 0x0C0C0000u | ((4u + b) << 8));
            else
                addr = (((d[j] >> (8 * b)) & 0xFFu) << 7) | lane_const;
            a[j] = *reinterpret_cast<const __attribute__((address_space(3))) _Float16 *>((uintptr_t)(lut_base + addr));
        }
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, __builtin_bit_cast(half8, xg[b]), acc, 0, 0, 0);
    }
}

// LUT level Q of the block's two 32-row tiles (first rows nA, nB) into LDS (layouts
// in the file header; q = 3 as the pair table).  first_loads() runs once the LUT
// requests are out and before their data is written, so the caller's first weight
// requests overlap the LUT's latency.
template <int Q, int KP, typename F>
__device__ __attribute__((always_inline)) inline void stage_lut(const __amdgpu_buffer_rsrc_t rl, int nA, int nB,
                                                                int N, int tid, char *smem, F &&first_loads)
{
    if constexpr (Q == 3) {
        // pair table of LUT_3: entry (row 32t+i, pair code v) at v*256 + 128t + 4i;
        // thread -> row tid % 64 and kPairsPer of the 64 pair codes
        constexpr int kPairsPer = 64 / (kThreadsOf<KP> / kRows);
        const int nl = tid % kRows, part = tid / kRows;
        const int n = (nl < 32 ? nA : nB) + (nl & 31);
        const u32x4 lv = n < N ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                         rl, (int)(((uint32_t)n << 3) * 2u), 0, 0))
                               : u32x4{0, 0, 0, 0};
        first_loads();
        const uint32_t slot = (uint32_t)(128 * (nl >> 5) + 4 * (nl & 31));
#pragma unroll
        for (int kk = 0; kk < kPairsPer; ++kk) {
            const uint32_t v = (uint32_t)(kPairsPer * part + kk);
            const uint32_t ce = bitrev(v & 7u, 3), co = bitrev(v >> 3, 3);  // codes of the even / odd column
            const uint32_t lo = (lv[ce >> 1] >> (16 * (ce & 1))) & 0xFFFFu;
            const uint32_t hi = (lv[co >> 1] >> (16 * (co & 1))) & 0xFFFFu;
            *reinterpret_cast<uint32_t *>(smem + v * 256 + slot) = lo | (hi << 16);
        }
    } else {
        // 16-byte loads (8 entries of one row), lane -> row so that one wave touches 64 rows
        constexpr int kLutU4 = (kRows << Q) / 8;
        constexpr int kPer = (kLutU4 + kThreadsOf<KP> - 1) / kThreadsOf<KP>;
        constexpr int kBatch = kPer < 4 ? kPer : 4;  // loads in flight per batch (register budget)
#pragma unroll
        for (int j0 = 0; j0 < kPer; j0 += kBatch) {
            u32x4 lv[kBatch];
#pragma unroll
            for (int jj = 0; jj < kBatch; ++jj) {
                const int idx = tid + (j0 + jj) * kThreadsOf<KP>;
                const int nl = idx % kRows, ch = idx / kRows;
                const int n = (nl < 32 ? nA : nB) + (nl & 31);
                const bool ok = idx < kLutU4 && n < N;
                lv[jj] = ok ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                  rl, (int)((((uint32_t)n << Q) + 8u * ch) * 2u), 0, 0))
                            : u32x4{0, 0, 0, 0};
            }
            if (j0 == 0)
                first_loads();
#pragma unroll
            for (int jj = 0; jj < kBatch; ++jj) {
                const int idx = tid + (j0 + jj) * kThreadsOf<KP>;
                if (idx >= kLutU4)
                    break;
                const int nl = idx % kRows, ch = idx / kRows;
                const int il = nl & 31, tl = nl >> 5;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint16_t v = (uint16_t)(lv[jj][e >> 1] >> (16 * (e & 1)));
                    const uint32_t vp = bitrev((uint32_t)(8 * ch + e), Q);
                    if (Q < 8) {
                        *reinterpret_cast<uint16_t *>(smem + vp * 256 + 4 * il + 2 * tl) = v;
                        *reinterpret_cast<uint16_t *>(smem + vp * 256 + 4 * (32 + il) + 2 * tl) = v;
                    } else {
                        *reinterpret_cast<uint16_t *>(smem + vp * 128 + 4 * il + 2 * tl) = v;
                    }
                }
            }
        }
    }
}

template <int Q, int TOKL, int KP>
__device__ void gemm_block(const GemmParams &P, const DevBlock &blk, int rb, int r0, int Me, char *smem)
{
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform (scalar)
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
    stage_lut<Q, KP>(rl, nA, nB, N, tid, smem, [&] { load_planes<Q>(wc, rs, first_word); });
    __syncthreads();

    // LDS byte addresses (compile-time constants for the static array)
    const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char *)smem);
    const uint32_t lane_const = Q == 3  ? (uint32_t)(128 * t + 4 * i)
                                : Q < 8 ? (uint32_t)(4 * (32 * g + i) + 2 * t)
                                        : (uint32_t)(4 * i + 2 * t);
    char *xs = smem + kLutBytes;
    const uint32_t xs_base = lds_base + kLutBytes;
    float *red = reinterpret_cast<float *>(xs);  // used after the last token tile is read
    constexpr int kXBuf = KP * TOKL * kXRowBytes;  // one token buffer: KP parts x TOKL rows
    constexpr int kDma = TOKL / 8;                 // token copies per wave and workgroup step
    const int nws = (nsteps + KP - 1) / KP;         // workgroup steps: part p takes step KP s + p

    for (int tp = 0; tp < Me; tp += TOKL) {
        const int j = lane & 31;  // token column of this lane in the B operand and in D
        const bool tok_ok = j < TOKL && tp + j < Me;
        // token copies: instruction u = wave + 2 KP k fills rows 4u .. 4u+3 of a buffer; lane L
        // writes 16-byte position L % 16 of row 4u + L / 16 (part row / TOKL, token row
        // % TOKL) and fetches the chunk stored there, chunk = position ^ token row
        uint32_t doff[kDma];
#pragma unroll
        for (int k = 0; k < kDma; ++k) {
            const int row = 4 * (wave + 2 * KP * k) + (lane >> 4);
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
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rx, (__attribute__((address_space(3))) void *)(xs + b * kXBuf + 1024 * (wave + 2 * KP * k)),
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
                if constexpr (Q == 3) {
                    group_product_pair3<0, B * kXBuf>(cur, xaddr, lds_base, lane_const, acc);
                    group_product_pair3<1, B * kXBuf>(cur, xaddr, lds_base, lane_const, acc);
                } else {
                    group_product<Q, 0, B * kXBuf>(cur, xaddr, lds_base, lane_const, acc);
                    group_product<Q, 1, B * kXBuf>(cur, xaddr, lds_base, lane_const, acc);
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
                        if (P.out_f32)
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
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const _Float16 up = (_Float16)red[slot(1, 1, v)];
                    oa[8 * (v >> 2) + (v & 3)] = silu_mul((_Float16)acc[v], up);
                }
            }
        }
        __syncthreads();
    }
}

template <int TOKL, int KP>
__device__ __attribute__((always_inline)) inline void dispatch_q(const GemmParams &P, const DevBlock &blk, int rb,
                                                                 int r0, int Me, char *smem)
{
    switch (blk.q) {
    case 3: gemm_block<3, TOKL, KP>(P, blk, rb, r0, Me, smem); break;
    case 4: gemm_block<4, TOKL, KP>(P, blk, rb, r0, Me, smem); break;
    case 5: gemm_block<5, TOKL, KP>(P, blk, rb, r0, Me, smem); break;
    case 6: gemm_block<6, TOKL, KP>(P, blk, rb, r0, Me, smem); break;
    case 7: gemm_block<7, TOKL, KP>(P, blk, rb, r0, Me, smem); break;
    case 8: gemm_block<8, TOKL, KP>(P, blk, rb, r0, Me, smem); break;
    default: break;  // unreachable: commit validates q
    }
}

// KIND (APMOE_GATE_UP / APMOE_DOWN) only names the launch, so profiles tell them apart.
// The LDS region is a static array (its address is a compile-time constant, so LUT
// gathers need no base add): LUT, then the token buffers, which the part sums reuse.
template <int TOKL, int KP>
constexpr int kLdsBytes = kLutBytes + (kRedBytesOf<KP> > 2 * KP * TOKL * kXRowBytes ? kRedBytesOf<KP>
                                                                                    : 2 * KP * TOKL * kXRowBytes);

template <int KIND, int TOKL, int KP>
__global__ void __launch_bounds__(kThreadsOf<KP>) __attribute__((amdgpu_waves_per_eu(3))) gemm_kernel(GemmParams P)
{
    __shared__ __attribute__((aligned(16))) char smem[kLdsBytes<TOKL, KP>];
    // Workgroup b runs on XCD b % 8.  XCD x takes the x-th eighth of the work items and
    // consecutive work items cycle over the experts, so every XCD streams an equal share
    // of every expert's rows.  (With e = b % E and E = 8, each expert would run on one
    // XCD, and the launch would wait for the XCD with the most planes or token passes.)
    const int per = (int)gridDim.x / kXcds;
    const int w = (int)(blockIdx.x % kXcds) * per + (int)(blockIdx.x / kXcds);
    if (w >= P.row_blocks * P.E)
        return;  // grid padding to a multiple of the XCD count
    const int e = w % P.E;
    const int rb = w / P.E;
    const int r0 = P.offsets[e];
    const int Me = P.offsets[e + 1] - r0;
    if (Me <= 0 || Me > P.max_rows)
        return;  // expert without tokens (no weight reads), or one for the tile product
    const DevBlock blk = P.table[2 * e + P.kind];
    dispatch_q<TOKL, KP>(P, blk, rb, r0, Me, smem);
}

template <int KIND, int KP>
void launch_kind(const GemmParams &P, hipStream_t s)
{
    const dim3 grid((P.row_blocks * P.E + kXcds - 1) / kXcds * kXcds);
    if (P.tokl == 8)
        hipLaunchKernelGGL((gemm_kernel<KIND, 8, KP>), grid, dim3(kThreadsOf<KP>), 0, s, P);
    else
        hipLaunchKernelGGL((gemm_kernel<KIND, 16, KP>), grid, dim3(kThreadsOf<KP>), 0, s, P);
}

}  // namespace

hipError_t launch_gemm(const DevBlock *table, int kind, int E, int N, int K, int max_q, const uint16_t *in,
                       size_t in_bytes, int gather, const int32_t *perm, const int32_t *offsets, int topk, int R,
                       void *out, int out_f32, int act, hipStream_t s)
{
    (void)max_q;
    GemmParams P;
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
    P.max_rows = kDecodeMaxRows;
    // A token is routed to an expert at most once, so no expert has more rows than the
    // batch has tokens (R / topk).  The token buffers hold 8 rows up to 16 tokens (40 KB
    // of LDS: four workgroups per CU; with 16 tokens spread over the experts few have
    // more than 8) and 16 rows above (48 KB, three workgroups); an expert with more rows
    // than the buffers takes further passes over its weights.
    const int tokens = topk > 0 ? R / topk : R;
    P.tokl = tokens <= 16 ? 8 : 16;
    // Few workgroups (the down product's N / 64 row blocks) leave two per CU: four
    // column parts then give each CU four waves per SIMD instead of two.
    const bool wide = (long)P.row_blocks * E <= 4 * 256;
    if (kind == APMOE_GATE_UP)
        wide ? launch_kind<APMOE_GATE_UP, 4>(P, s) : launch_kind<APMOE_GATE_UP, 2>(P, s);
    else
        wide ? launch_kind<APMOE_DOWN, 4>(P, s) : launch_kind<APMOE_DOWN, 2>(P, s);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || R <= kDecodeMaxRows)
        return err;  // no expert can have more rows than the decode product takes
    return launch_gemm_tile(table, kind, E, N, K, in, in_bytes, gather, perm, offsets, topk, out, out_f32, act, R, s);
}

}  // namespace apmoe
