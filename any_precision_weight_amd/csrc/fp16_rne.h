// fp16_rne.h -- fp64 -> IEEE 754 binary16 bits, round to nearest, ties to even,
// written from the two formats' encodings.  Used on the device by the child-LUT
// build of libapmoe and by the device input generator.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

__device__ inline uint16_t apmoe_d2h_rne(double d)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, d);
    const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
    const int ex = (int)((u >> 52) & 0x7FF);
    const uint64_t mant = u & ((1ull << 52) - 1);
    if (ex == 0x7FF)
        return sign | (mant ? 0x7E00 : 0x7C00);
    if (ex == 0)
        return sign;  // zero or an fp64 subnormal: far below fp16's range
    // value = 1.mant * 2^e
    const int e = ex - 1023;
    const uint64_t sig = mant | (1ull << 52);  // 53-bit significand
    int shift;
    uint32_t hexp;
    if (e >= -14) {
        if (e > 15)
            return sign | 0x7C00;
        shift = 52 - 10;  // keep 11 bits
        hexp = (uint32_t)(e + 15);
    } else {
        // subnormal half: quantum 2^-24, value / 2^-24 = sig * 2^(e - 52 + 24)
        shift = 52 - 10 + (-14 - e);
        hexp = 0;
        if (shift > 63)
            return sign;
    }
    uint64_t q = sig >> shift;
    const uint64_t rem = sig & ((1ull << shift) - 1);
    const uint64_t halfway = 1ull << (shift - 1);
    if (rem > halfway || (rem == halfway && (q & 1)))
        ++q;
    if (hexp == 0)
        return sign | (uint16_t)q;  // q == 1024 carries into the smallest normal
    if (q == 2048) {                // carry out of the significand
        q = 1024;
        if (++hexp >= 31)
            return sign | 0x7C00;
    }
    return sign | (uint16_t)((hexp << 10) | (uint32_t)(q - 1024));
}
