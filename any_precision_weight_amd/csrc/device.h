// device.h -- device helpers shared by the expert-product kernels (not installed):
// buffer resources, the bit transpose that turns plane words into codes, LDS
// access, and the s_waitcnt immediates of the counted waits.
#pragma once

#include <type_traits>

#include "internal.h"

namespace apmoe {

constexpr int kWave = 64;
constexpr int kXcds = 8;  // accelerator complex dies; workgroup b runs on XCD b % 8

typedef _Float16 half4 __attribute__((ext_vector_type(4)));
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

// The low q bits of c in reverse order.
__device__ inline uint32_t bitrev(uint32_t c, int q) { return __builtin_bitreverse32(c) >> (32 - q); }

// (m & a) | (~m & b) in one v_bitop3_b32 (truth table 0xE4: the third operand
// selects between the first two).
__device__ inline uint32_t select_bits(uint32_t m, uint32_t a, uint32_t b)
{
    return __builtin_amdgcn_bitop3_b32(a, b, m, (unsigned char)0xE4);
}

// Transpose of 4 independent 8x8 bit blocks (the delta-swap method of Hacker's
// Delight, section 7-3) for codes of Q bits: on input d[p] byte b bit j is plane p,
// column 8b + j (planes p >= Q are zero); on output d[j] byte b bit p holds the same
// bit.  Each stage exchanges one bit of the word index with the same bit of the bit
// position (distance 1, 2, 4), so the three stages commute; the swaps whose words are
// known zero are folded at compile time.  A remaining swap is two shifts and two
// selects, a swap with a zero partner a mask and a shift-and-mask.  With the stages
// in the order 1, 2, 4 the zero words are paired longest: Q = 3..8 take 27, 28, 41,
// 42, 47, 48 instructions per 32 columns (39..48 in the order 4, 2, 1).
template <int Q>
__device__ inline void transpose_codes(uint32_t (&d)[8])
{
    // stage distance s: words (i, i + j) exchange the bits of i under m << s with the
    // bits of i + j under m
    auto stage = [&](auto jj, int s, uint32_t m, auto nz) {
        constexpr int J = decltype(jj)::value;
        constexpr uint32_t NZ = decltype(nz)::value;  // bit p: word p may be nonzero
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i & J)
                continue;
            const bool za = !((NZ >> i) & 1u), zb = !((NZ >> (i + J)) & 1u);
            const uint32_t a = d[i], b = d[i + J];
            if (za && zb)
                continue;
            if (zb) {
                d[i] = a & ~(m << s);
                d[i + J] = (a >> s) & m;
            } else if (za) {
                d[i] = (b << s) & (m << s);
                d[i + J] = b & ~m;
            } else {
                d[i] = select_bits(m << s, b << s, a);
                d[i + J] = select_bits(m, a >> s, b);
            }
        }
    };
    // after a stage of distance J, words i and i + J may be nonzero if either input was
    constexpr auto spread = [](uint32_t nz, int J) {
        uint32_t out = nz;
        for (int i = 0; i < 8; ++i)
            if (!(i & J) && (((nz >> i) | (nz >> (i + J))) & 1u))
                out |= (1u << i) | (1u << (i + J));
        return out;
    };
    constexpr uint32_t nz0 = (1u << Q) - 1u;
    constexpr uint32_t nz1 = spread(nz0, 1);
    constexpr uint32_t nz2 = spread(nz1, 2);
    stage(std::integral_constant<int, 1>{}, 1, 0x55555555u, std::integral_constant<uint32_t, nz0>{});
    stage(std::integral_constant<int, 2>{}, 2, 0x33333333u, std::integral_constant<uint32_t, nz1>{});
    stage(std::integral_constant<int, 4>{}, 4, 0x0F0F0F0Fu, std::integral_constant<uint32_t, nz2>{});
}

// Index of a pair of adjacent columns (codes ce of the even and co of the odd column)
// in a pair table: bit 2p + s is plane p's bit of the column of parity s (code bits
// with plane 0 most significant).
template <int Q>
__host__ __device__ constexpr uint32_t pair_index(int ce, int co)
{
    uint32_t v = 0;
    for (int p = 0; p < Q; ++p)
        v |= (uint32_t)((ce >> (Q - 1 - p)) & 1) << (2 * p) | (uint32_t)((co >> (Q - 1 - p)) & 1) << (2 * p + 1);
    return v;
}

// LDS byte address of a pointer into a __shared__ array.
__device__ inline uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

__device__ inline u32x4 lds_b128(uint32_t addr)
{
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4 *>((uintptr_t)addr);
}

__device__ inline void lds_store_b128(uint32_t addr, u32x4 v)
{
    *reinterpret_cast<__attribute__((address_space(3))) u32x4 *>((uintptr_t)addr) = v;
}

// s_waitcnt immediates: vmcnt in bits 3:0 and 15:14, expcnt (6:4) left open,
// lgkmcnt (11:8) zero.  The pipelines wait for exactly the vector-memory requests
// that must have landed and leave later ones in flight.  A build with
// APMOE_SAFE_WAITS defined counts every such wait down to zero instead: it drains
// every outstanding request (slower, never early), and must give identical bits.
#ifdef APMOE_SAFE_WAITS
constexpr bool kSafeWaits = true;
#else
constexpr bool kSafeWaits = false;
#endif
constexpr int kWaitAll = 7 << 4;
template <int VM>
constexpr int wait_vm()
{
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    constexpr int v = kSafeWaits ? 0 : VM;
    return (v & 15) | (7 << 4) | ((v >> 4) << 14);
}

}  // namespace apmoe
