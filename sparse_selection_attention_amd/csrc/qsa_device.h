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

// int8 -> fp16 (exact) with SDWA: byte BA of x into the low half, byte BB of y
// into the high half of one dword.
#define QSA_CVT2(out, x, ba, y, bb)                                                              \
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_" #ba  \
        "\n\tv_cvt_f16_i16_sdwa %0, sext(%2) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE "          \
        "src0_sel:BYTE_" #bb                                                                      \
        : "=&v"(out)                                                                             \
        : "v"(x), "v"(y))

template <int B>
__device__ inline uint32_t cvt2_byte(uint32_t x, uint32_t y)
{
    uint32_t r;
    if constexpr (B == 0)
        QSA_CVT2(r, x, 0, y, 0);
    else if constexpr (B == 1)
        QSA_CVT2(r, x, 1, y, 1);
    else if constexpr (B == 2)
        QSA_CVT2(r, x, 2, y, 2);
    else
        QSA_CVT2(r, x, 3, y, 3);
    return r;
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

// Eight int8 values (little-endian in v) to fp16, exactly, in byte order.
__device__ inline half8 i8x8_to_half8(uint2 v)
{
    uint32_t a, b, c, d;
    QSA_CVT2(a, v.x, 0, v.x, 1);
    QSA_CVT2(b, v.x, 2, v.x, 3);
    QSA_CVT2(c, v.y, 0, v.y, 1);
    QSA_CVT2(d, v.y, 2, v.y, 3);
    return __builtin_bit_cast(half8, make_uint4(a, b, c, d));
}

__device__ inline void wave_sync_lds()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

} // namespace dev
} // namespace qsa
