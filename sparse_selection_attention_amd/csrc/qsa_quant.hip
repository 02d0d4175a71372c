// qsa_quant.hip -- int8 cache rows with one fp16 scale per 32-element group.
//
// Writes the cache the attention reads ("round 11 track b: qsa attention and
// score", section "implementation and evaluator": a K row carries four scale
// groups), the kq/vq/ksc/vsc outputs of the pages' prep step, which is memory
// bound on the rows it reads and writes ("Round 36 Track C ...", section
// "Summary & Decision"). The pages do not print the quantisation rule; this
// library takes symmetric absmax per group:
//   a = max |x| over the 32 elements,  s = fp16_rne(a / 127),
//   code = clamp(rint(x / s), -127, 127), or 0 when s == 0,
// with both quotients correctly rounded binary32 divisions and rint rounding
// half to even. The integer codes and the fp16 scale are decided in binary32,
// so any implementation of the rule reproduces them bit for bit.
//
// Design on CDNA4: a streaming kernel. Each thread owns 8 consecutive
// elements (two 16-byte loads), four threads one group, sixteen one row, so a
// wave reads four 512-byte rows in one contiguous 2 KB sweep and writes four
// 128-byte code rows. The group maximum is two lane exchanges. Row tasks run
// over the K rows, then the V rows.
#include "qsa_internal.h"

#include <hip/hip_fp16.h>

namespace qsa {
namespace {

constexpr int kRowsPerBlock = 16;   // 256 threads, 16 per row

__device__ inline float absmax8(float4 a, float4 b)
{
    return fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                 fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
}

__device__ inline uint32_t code_byte(float x, float s)
{
    float c = 0.0f;
    if (s > 0.0f)
        c = fminf(fmaxf(rintf(__fdiv_rn(x, s)), -127.0f), 127.0f);
    return (uint32_t)(int32_t)c & 0xffu;
}

__device__ inline uint32_t pack4(float4 x, float s)
{
    return code_byte(x.x, s) | (code_byte(x.y, s) << 8) | (code_byte(x.z, s) << 16) | (code_byte(x.w, s) << 24);
}

__global__ __launch_bounds__(256) void quant_kernel(QuantArgs a)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int64_t task = (int64_t)blockIdx.x * kRowsPerBlock + (tid >> 4);
    // all 16 threads of a row share `task`, so a row is wholly in or out
    const bool active = task < 2 * (int64_t)a.n_rows;
    const bool is_v = task >= a.n_rows;
    const int64_t r = is_v ? task - a.n_rows : task;
    const int e0 = 8 * (tid & 15);

    float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
    if (active) {
        const float *src = (is_v ? a.v : a.k) + r * kD + e0;
        x0 = *(const float4 *)src;
        x1 = *(const float4 *)(src + 4);
    }
    float amax = absmax8(x0, x1);
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));        // the four threads of a group
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    const _Float16 s16 = (_Float16)__fdiv_rn(amax, 127.0f);    // binary32 quotient, then RNE to fp16
    const float s = (float)s16;

    const uint2 codes = make_uint2(pack4(x0, s), pack4(x1, s));
    // the row's four scales, from its threads 0, 4, 8 and 12
    const uint32_t sbits = (uint32_t)__builtin_bit_cast(uint16_t, s16);
    const int row_lane = lane & ~15;
    const uint32_t g0 = __shfl(sbits, row_lane + 0, 64), g1 = __shfl(sbits, row_lane + 4, 64);
    const uint32_t g2 = __shfl(sbits, row_lane + 8, 64), g3 = __shfl(sbits, row_lane + 12, 64);
    if (active) {
        const int64_t cell = (int64_t)a.cell0 + r;
        *(uint2 *)((is_v ? a.vq : a.kq) + cell * kD + e0) = codes;
        if ((tid & 15) == 0)
            *(uint2 *)((is_v ? a.vsc : a.ksc) + cell * (kD / kGroup)) = make_uint2(g0 | (g1 << 16), g2 | (g3 << 16));
    }
}

} // namespace

hipError_t launch_quant(const QuantArgs &a, hipStream_t stream)
{
    const int64_t tasks = 2 * (int64_t)a.n_rows;
    const int64_t blocks = (tasks + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL(quant_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

} // namespace qsa
