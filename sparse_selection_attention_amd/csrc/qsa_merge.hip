// qsa_merge.hip -- max-first merge of chunk records into fp16 output on gfx950.
//
// Follows "round 5 track b: cached residual norms and fused mtp attention",
// sections "preflight / ownership" and "mtp attention": the per-chunk records of
// 64-cell chunks are combined relative to the largest chunk maximum. For token
// t and head h, over the chunks whose max is finite:
//   M = max_k m_k, w_k = exp(m_k - M), L = sum_k w_k l_k,
//   out[d] = fp16_rne(sum_k w_k o_k[d] / L),
// and +0 when no chunk of the row had a valid slot. Records with m = -inf are
// skipped without reading their o, which qsa_attn leaves unwritten.
//
// The merge streams the partial records once, so it is bound by HBM reads.
// One 64-lane wave owns one (token, head) pair. The lanes first reduce the
// chunk maxima; then the wave walks the chunks in order, eight at a time, with
// each lane owning two dims, so every record row is one coalesced 512-byte read
// and eight of them are in flight per wave. The walk has no branches: records
// of empty chunks (or past the end) are still addressed, but their products are
// discarded by a select, so a stale o never reaches the sums.
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;

__global__ __launch_bounds__(64 * kWaves) void merge_kernel(MergeArgs a)
{
    constexpr int kUnroll = 8;
    const int lane = threadIdx.x & 63;
    const int64_t wv = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (wv >= (int64_t)a.T * a.H)
        return;
    const int t = (int)(wv / a.H);
    const int h = (int)(wv - (int64_t)t * a.H);
    const int64_t base = (int64_t)t * a.C * a.H + h;     // record (t, 0, h); chunk stride H

    float M = -INFINITY;
    for (int k0 = 0; k0 < a.C; k0 += 64) {
        const int k = k0 + lane;
        if (k < a.C)
            M = fmaxf(M, a.m[base + (int64_t)k * a.H]);
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1)
        M = fmaxf(M, __shfl_xor(M, s, 64));

    uint32_t res = 0u;              // two fp16 +0 values
    if (M != -INFINITY) {
        float L = 0.0f, O0 = 0.0f, O1 = 0.0f;
        for (int k0 = 0; k0 < a.C; k0 += kUnroll) {
            float mk[kUnroll], lk[kUnroll];
            float2 ov[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int k = min(k0 + u, a.C - 1);
                const int64_t r = base + (int64_t)k * a.H;
                mk[u] = a.m[r];
                lk[u] = a.l[r];
                ov[u] = *(const float2 *)(a.o + r * kD + 2 * lane);
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const bool use = (k0 + u < a.C) && (mk[u] != -INFINITY);
                const float wk = __builtin_amdgcn_exp2f((mk[u] - M) * kLog2e);
                L = use ? fmaf(wk, lk[u], L) : L;
                O0 = use ? fmaf(wk, ov[u].x, O0) : O0;
                O1 = use ? fmaf(wk, ov[u].y, O1) : O1;
            }
        }
        const _Float16 r0 = (_Float16)(O0 / L);
        const _Float16 r1 = (_Float16)(O1 / L);
        res = (uint32_t)__builtin_bit_cast(uint16_t, r0) | ((uint32_t)__builtin_bit_cast(uint16_t, r1) << 16);
    }
    *(uint32_t *)(a.out + ((int64_t)t * a.H + h) * kD + 2 * lane) = res;
}

} // namespace

hipError_t launch_merge(const MergeArgs &a, hipStream_t stream)
{
    const int64_t waves = (int64_t)a.T * a.H;
    dim3 grid((unsigned)((waves + kWaves - 1) / kWaves)), block(64 * kWaves);
    hipLaunchKernelGGL(merge_kernel, grid, block, 0, stream, a);
    return hipGetLastError();
}

} // namespace qsa
