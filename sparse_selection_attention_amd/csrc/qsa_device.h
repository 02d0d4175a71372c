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

// byte B of x into the low half and byte B of y into the high half: the two
// bytes are placed over zero bytes, and one xor both flips their top bits and
// writes 0x64 above them
template <int B>
__device__ inline uint32_t cvt2_byte(uint32_t x, uint32_t y)
{
    constexpr uint32_t sel = 0x0c000c00u | (uint32_t)(4 + B) << 16 | (uint32_t)B;   // [x_B, 0, y_B, 0]
    const uint32_t w = __builtin_amdgcn_perm(y, x, sel) ^ 0x64806480u;
    const half2v h = __builtin_bit_cast(half2v, w) - (half2v){(_Float16)1152.0f, (_Float16)1152.0f};
    return __builtin_bit_cast(uint32_t, h);
}

// Same with a byte index that is a constant once the caller's loop is unrolled.
__device__ inline uint32_t cvt2_sel(int b, uint32_t x, uint32_t y)
{
    switch (b) {
    case 0: return cvt2_byte<0>(x, y);
    case 1: return cvt2_byte<1>(x, y);
    case 2: return cvt2_byte<2>(x, y);
    default: return cvt2_byte<3>(x, y);
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

__device__ inline void wave_sync_lds()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

} // namespace dev
} // namespace qsa
