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
// Each half of a 64-lane wave owns one (token, head) pair, so a wave covers two
// adjacent 512-byte head rows of a chunk record with one 16-byte load per lane.
// The lanes first reduce the chunk maxima; then the wave walks the chunks in
// order, eight at a time, so eight such loads are in flight. The records are
// read once and never again, so the loads are marked nontemporal. The walk has
// no branches: records of empty chunks (or past the end) are still addressed,
// but their products are discarded by a select, so a stale o never reaches the
// sums.
//
// The gated form (qsa_merge_gated) multiplies each merged value by sigmoid(g)
// of its own fp32 gate before the fp16 rounding, and can also write the exact
// sum of every block of 16 written values rounded once to fp32 ("round 5
// track b: cached residual norms and fused mtp attention", sections
// "preflight / ownership" and "actual verification": the sigmoid gate, fp32
// gates and the per-16 sums). A lane holds four consecutive dims, so two xor
// exchanges in binary64 give each block's sum exactly.
#include "qsa_internal.h"
#include "qsa_device.h"

namespace qsa {
namespace {

using dev::pack_half4;
using dev::half4_sum;
using dev::sigmoid_gate;
using dev::xor_sum;

typedef float f4v __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kUnroll = 8;          // chunks per batch of record reads
constexpr float kLog2e = 1.4426950408889634f;

// U chunks from k0 on (indexes past the last chunk re-read it; those are not
// added): their records are all read before the first is added, and they are
// added in chunk order with weights exp(m_k - M)
template <int U>
__device__ inline void combine(const MergeArgs &a, int64_t base, int k0, float M, int l32, float &L, float4 &O)
{
    float mk[U], lk[U];
    float4 ov[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int k = min(k0 + u, a.C - 1);
        const int64_t r = base + (int64_t)k * a.H;
        mk[u] = a.m[r];
        lk[u] = a.l[r];
        { f4v t4 = __builtin_nontemporal_load((const f4v *)(a.o + r * kD + 4 * l32)); ov[u] = make_float4(t4.x, t4.y, t4.z, t4.w); }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool use = (k0 + u < a.C) && (mk[u] != -INFINITY);
        const float wk = __builtin_amdgcn_exp2f((mk[u] - M) * kLog2e);
        L = use ? fmaf(wk, lk[u], L) : L;
        O.x = use ? fmaf(wk, ov[u].x, O.x) : O.x;
        O.y = use ? fmaf(wk, ov[u].y, O.y) : O.y;
        O.z = use ? fmaf(wk, ov[u].z, O.z) : O.z;
        O.w = use ? fmaf(wk, ov[u].w, O.w) : O.w;
    }
}

__global__ __launch_bounds__(64 * kWaves) void merge_kernel(MergeArgs a)
{
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5, l32 = lane & 31;
    const int64_t hv = ((int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6)) * 2 + half;   // (t, h) pair
    const bool live = hv < (int64_t)a.T * a.H;
    const int64_t hv2 = live ? hv : 0;
    const int t = (int)(hv2 / a.H);
    const int h = (int)(hv2 - (int64_t)t * a.H);
    const int64_t base = (int64_t)t * a.C * a.H + h;

    float M = -INFINITY;
    for (int k0 = 0; k0 < a.C; k0 += 32) {
        const int k = k0 + l32;
        if (k < a.C)
            M = fmaxf(M, a.m[base + (int64_t)k * a.H]);
    }
    // max over the 32 lanes of this half-wave, in the VALU: lane ^ 16 by the
    // row-swap permute, then lanes 8 and 4 apart by row rotations and lanes 2
    // and 1 apart by quad permutes
    M = dev::xor16_max(M);
    M = fmaxf(M, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(M), 0x128, 0xf, 0xf, false)));  // row_ror:8
    M = fmaxf(M, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(M), 0x124, 0xf, 0xf, false)));  // row_ror:4
    M = fmaxf(M, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(M), 0x4E, 0xf, 0xf, false)));   // lane ^ 2
    M = fmaxf(M, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(M), 0xB1, 0xf, 0xf, false)));   // lane ^ 1

    float4 y = make_float4(0.f, 0.f, 0.f, 0.f);  // +0 when no chunk of the row had a valid slot
    if (M != -INFINITY) {
        float L = 0.0f;
        float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
        // whole batches of kUnroll chunks, then the rest as one batch of the
        // smallest power of two that holds it (33 chunks: 4 x 8 + 1), so that
        // few loads re-read the last chunk
        const int c_full = a.C - a.C % kUnroll, rest = a.C - c_full;
        for (int k0 = 0; k0 < c_full; k0 += kUnroll)
            combine<kUnroll>(a, base, k0, M, l32, L, O);
        if (rest == 1)
            combine<1>(a, base, c_full, M, l32, L, O);
        else if (rest == 2)
            combine<2>(a, base, c_full, M, l32, L, O);
        else if (rest > 2 && rest <= 4)
            combine<4>(a, base, c_full, M, l32, L, O);
        else if (rest > 4)
            combine<kUnroll>(a, base, c_full, M, l32, L, O);
        y = make_float4(O.x / L, O.y / L, O.z / L, O.w / L);
    }
    const int64_t orow = ((int64_t)t * a.H + h) * kD + 4 * l32;
    if (a.gate) {                   // uniform: the gated entry point
        const float4 g = live ? *(const float4 *)(a.gate + orow) : make_float4(0.f, 0.f, 0.f, 0.f);
        y.x *= sigmoid_gate(g.x);
        y.y *= sigmoid_gate(g.y);
        y.z *= sigmoid_gate(g.z);
        y.w *= sigmoid_gate(g.w);
    }
    const uint2 res = pack_half4(y.x, y.y, y.z, y.w);
    if (live)
        *(uint2 *)(a.out + orow) = res;
    if (a.sums) {                   // uniform; every lane takes part in the exchanges
        const double s = xor_sum(xor_sum(half4_sum(res), 1), 2);   // dims 16b .. 16b+15, b = l32 / 4
        if (live && (l32 & 3) == 0)
            a.sums[((int64_t)t * a.H + h) * (kD / 16) + (l32 >> 2)] = (float)s;
    }
}

} // namespace

hipError_t launch_merge(const MergeArgs &a, hipStream_t stream)
{
    const int64_t pairs = (int64_t)a.T * a.H;
    const int64_t waves = (pairs + 1) / 2;
    dim3 grid((unsigned)((waves + kWaves - 1) / kWaves)), block(64 * kWaves);
    hipLaunchKernelGGL(merge_kernel, grid, block, 0, stream, a);
    return hipGetLastError();
}

} // namespace qsa
