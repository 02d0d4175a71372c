// qsa_device.h -- device helpers shared by the attention kernels of
// libqsa.so (int8 -> fp16 conversion, vector types, wave-level LDS sync).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {
namespace dev {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

__device__ inline float half_bits_to_float(uint32_t bits16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// int8 -> fp16, exactly, from operations the compiler sees (no inline asm: the
// compiler inserts the wait states that an in-flight matrix instruction needs
// before a register it reads is overwritten, and it cannot do so for
// instructions hidden in an asm block). A byte b with its top bit flipped is
// b + 128 in [0, 255]; as the low byte of an fp16 whose high byte is 0x64
// (1024.0, where the fp16 step is 1) it reads 1152 + b, and subtracting 1152
// leaves b exactly.

// The same conversion can scale by 2^-k (0 <= k <= 7) at no cost: under a high
// byte 0x64 - 4k the fp16 exponent is 2^(10 - k), the half reads (1152 + b) *
// 2^-k, and subtracting 1152 * 2^-k leaves b * 2^-k, exactly (b has at most 7
// significant bits and b * 2^-k is a normal fp16 for b != 0).
struct I8Scale {
    uint32_t xr;      // xor: top bits of both bytes, and the exponent bytes
    uint32_t bias;    // fp16 bits of 1152 * 2^-k in both halves
};

// k must be uniform over the wave: both words are then kept in scalar
// registers. 1152 * 2^-k = 1.125 * 2^(10 - k) has the fp16 bits
// (25 - k) << 10 | 0x80.
__device__ inline I8Scale i8_scale(int k)
{
    const uint32_t hb = 0x64u - 4u * (uint32_t)k;
    const uint32_t b16 = ((25u - (uint32_t)k) << 10) | 0x80u;
    return I8Scale{(uint32_t)__builtin_amdgcn_readfirstlane((int)((hb << 24) | 0x00800000u | (hb << 8) | 0x80u)),
                   (uint32_t)__builtin_amdgcn_readfirstlane((int)((b16 << 16) | b16))};
}

// byte B of x into the low half and byte B of y into the high half, times
// 2^-k: the two bytes are placed over zero bytes, and one xor both flips their
// top bits and writes the exponent bytes above them
template <int B>
__device__ inline uint32_t cvt2_byte(uint32_t x, uint32_t y, const I8Scale &c)
{
    constexpr uint32_t sel = 0x0c000c00u | (uint32_t)(4 + B) << 16 | (uint32_t)B;   // [x_B, 0, y_B, 0]
    const uint32_t w = __builtin_amdgcn_perm(y, x, sel) ^ c.xr;
    const half2v h = __builtin_bit_cast(half2v, w) - __builtin_bit_cast(half2v, c.bias);
    return __builtin_bit_cast(uint32_t, h);
}

// Same with a byte index that is a constant once the caller's loop is unrolled.
__device__ inline uint32_t cvt2_sel(int b, uint32_t x, uint32_t y, const I8Scale &c)
{
    switch (b) {
    case 0: return cvt2_byte<0>(x, y, c);
    case 1: return cvt2_byte<1>(x, y, c);
    case 2: return cvt2_byte<2>(x, y, c);
    default: return cvt2_byte<3>(x, y, c);
    }
}

// Eight int8 values (little-endian in v) to fp16, exactly, in byte order: the
// top bits are flipped once per dword, then each pair of bytes is placed under
// two 0x64 bytes
__device__ inline half8 i8x8_to_half8(uint2 v)
{
    const uint32_t x = v.x ^ 0x80808080u, y = v.y ^ 0x80808080u;
    const half2v bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    const uint32_t w[4] = {__builtin_amdgcn_perm(0x64646464u, x, 0x04010400u),
                           __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u),
                           __builtin_amdgcn_perm(0x64646464u, y, 0x04010400u),
                           __builtin_amdgcn_perm(0x64646464u, y, 0x04030402u)};
    uint32_t r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, w[i]) - bias);
    return __builtin_bit_cast(half8, make_uint4(r[0], r[1], r[2], r[3]));
}

// v = hi + lo for eight fp32 values: hi the fp16 rounding of v (converted two
// values per instruction), lo the fp16 rounding of the residual v - hi. The
// residual is exact in fp32 for every v, so one fma that reads hi as fp16
// gives it without converting hi back: the same bits as the plain
// subtraction, in one instruction instead of two.
__device__ inline void split_half8(const float (&v)[8], half8 &hi, half8 &lo)
{
    // -1 kept opaque, so that the fma is not rewritten into a subtraction
    // (which would need hi converted back to fp32 first)
    float m1 = -1.0f;
    asm volatile("" : "+s"(m1));
#pragma unroll
    for (int s = 0; s < 8; s += 2) {
        // the pair is converted once, and the fmas read its two halves
        uint32_t hp = __builtin_bit_cast(uint32_t, (half2v){(_Float16)v[s], (_Float16)v[s + 1]});
        asm volatile("" : "+v"(hp));
        const _Float16 h0 = __builtin_bit_cast(_Float16, (uint16_t)(hp & 0xffffu));
        const _Float16 h1 = __builtin_bit_cast(_Float16, (uint16_t)(hp >> 16));
        hi[s] = h0;
        hi[s + 1] = h1;
        lo[s] = (_Float16)__builtin_fmaf((float)h0, m1, v[s]);
        lo[s + 1] = (_Float16)__builtin_fmaf((float)h1, m1, v[s + 1]);
    }
}

// sigmoid(g) = 1 / (1 + exp(-g)) in fp32, with a correctly rounded division:
// sigmoid(0) = 1/2, sigmoid(+inf) = 1 and sigmoid(-inf) = +0 exactly, and a
// NaN gate stays NaN. exp(-g) overflows to +inf below g = -88.7, where the
// exact sigmoid is already below the binary32 normal range.
__device__ inline float sigmoid_gate(float g)
{
    return 1.0f / (1.0f + __builtin_amdgcn_exp2f(-g * kLog2e));
}

// Four fp32 values rounded to fp16 (round to nearest even), packed in order.
__device__ inline uint2 pack_half4(float a, float b, float c, float d)
{
    const half2v lo = {(_Float16)a, (_Float16)b}, hi = {(_Float16)c, (_Float16)d};
    return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// Exact sum of the four fp16 values packed in v, as a double: each is an
// integer multiple of 2^-24 below 2^16, so sums of up to 2^9 of them are exact
// in binary64, in any order.
__device__ inline double half4_sum(uint2 v)
{
    const half2v lo = __builtin_bit_cast(half2v, v.x), hi = __builtin_bit_cast(half2v, v.y);
    return ((double)(float)lo[0] + (double)(float)lo[1]) + ((double)(float)hi[0] + (double)(float)hi[1]);
}

// One butterfly step: v plus the value of lane (lane ^ lane_xor). Steps over
// xor 1 and 2 leave each aligned group of four lanes holding the group's sum,
// which is exact for half4_sum values.
__device__ inline double xor_sum(double v, int lane_xor)
{
    return v + __shfl_xor(v, lane_xor, 64);
}

// Reductions over the lane pairs (l, l ^ 16) and (l, l ^ 32) through gfx950's
// row-swap permutes, which exchange values inside the VALU where a shuffle
// takes an LDS round trip. A swap of x with itself hands one lane of each pair
// the pair's first value and the other lane the second; both lanes then
// combine the same two values in the same order, so a pair ends with one
// result (the same result a shuffle-based exchange gives: max and + commute).
__device__ inline float xor16_max(float x)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ inline float xor32_max(float x)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ inline float xor16_sum(float x)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ inline float xor32_sum(float x)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ inline int xor16_max(int x)
{
    const auto p = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
    return max((int)p[0], (int)p[1]);
}
__device__ inline int xor32_max(int x)
{
    const auto p = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
    return max((int)p[0], (int)p[1]);
}

__device__ inline void wave_sync_lds()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

} // namespace dev
} // namespace qsa
