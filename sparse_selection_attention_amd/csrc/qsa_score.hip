// qsa_score.hip -- fp32 causal q.K scores with a dead-key tail on gfx950.
//
// Follows "round 11 track b: qsa attention and score", sections
// "implementation and evaluator" (causal cells get scores, one constant marks
// the cells just past the causal edge, later cells are not written) and
// "score: valid negative result" (64 x 64 score tiles over a 128-deep
// contraction, summed over heads).
// For row t (p = pos0 + t):
//   scores[t][c] = scale * sum_h sum_d q[t][h][d] * k[c][d]      c <= p
//   scores[t][c] = dead        p < c < min(64 * ceil((p + 1) / 64), row_stride)
// and later cells are not written.
//
// Design on CDNA4. The head sum is linear, so sum_h (q_h . k) = (sum_h q_h) . k:
// the heads are added once while a 64-row q tile is staged in LDS, and the
// score tile becomes one 64 x 64 x 128 fp32 contraction regardless of the head
// count. A 256-thread workgroup owns one 64 x 64 tile; each wave computes a
// 32 x 32 quadrant as four 16 x 16 v_mfma_f32_16x16x4_f32 accumulators. Tiles
// that lie wholly beyond the last causal cell of their rows (and so hold no tail
// either, since the tail never crosses a 64-cell boundary) return at once.
#include "qsa_internal.h"

namespace qsa {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;
constexpr int kPitch = kD + 4;   // LDS row pitch in floats: rows 16 B apart in bank space

__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a)
{
    __shared__ float sq[kTile][kPitch];
    __shared__ float sk[kTile][kPitch];

    const int r0 = blockIdx.y * kTile;
    const int c0 = blockIdx.x * kTile;
    const int last_row = min(a.T, r0 + kTile) - 1;
    if ((int64_t)c0 > (int64_t)a.pos0 + last_row)
        return;                              // uniform over the workgroup

    const int tid = threadIdx.x;
    // stage q (summed over heads) and k, float4 per thread-step
    for (int idx = tid; idx < kTile * (kD / 4); idx += 256) {
        const int row = idx >> 5, c4 = idx & 31;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        const int t = r0 + row;
        if (t < a.T) {
            const float *qr = a.q + (int64_t)t * a.Hs * kD + 4 * c4;
            for (int h = 0; h < a.Hs; ++h) {
                const float4 v = *(const float4 *)(qr + (int64_t)h * kD);
                acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
            }
        }
        *(float4 *)&sq[row][4 * c4] = acc;
        float4 kv = make_float4(0.f, 0.f, 0.f, 0.f);
        const int c = c0 + row;
        if (c < a.n_cells)
            kv = *(const float4 *)(a.k + (int64_t)c * kD + 4 * c4);
        *(float4 *)&sk[row][4 * c4] = kv;
    }
    __syncthreads();

    const int lane = tid & 63, w = tid >> 6;
    const int j = lane >> 4, c16 = lane & 15;
    const int rq = 32 * (w >> 1), cq = 32 * (w & 1);   // this wave's quadrant
    floatx4 acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
            acc[mi][ni] = (floatx4){0.f, 0.f, 0.f, 0.f};

    // k-slot j of MFMA (u, e) is dim 4 * (4u + j) + e, for A and B alike
#pragma unroll 2
    for (int u = 0; u < 8; ++u) {
        float4 av[2], bv[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
            av[mi] = *(const float4 *)&sq[rq + 16 * mi + c16][4 * (4 * u + j)];
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
            bv[ni] = *(const float4 *)&sk[cq + 16 * ni + c16][4 * (4 * u + j)];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[mi].x, bv[ni].x, acc[mi][ni], 0, 0, 0);
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[mi].y, bv[ni].y, acc[mi][ni], 0, 0, 0);
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[mi].z, bv[ni].z, acc[mi][ni], 0, 0, 0);
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[mi].w, bv[ni].w, acc[mi][ni], 0, 0, 0);
            }
    }

    // D layout: lane (j, c16) holds rows 4j + r, column c16 of each 16 x 16 tile
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = r0 + rq + 16 * mi + 4 * j + r;
            if (t >= a.T)
                continue;
            const int64_t p = (int64_t)a.pos0 + t;
            int64_t tail_end = ((p + kTile) / kTile) * kTile;    // 64 * ceil((p + 1) / 64)
            if (tail_end > a.row_stride)
                tail_end = a.row_stride;
            float *row = a.scores + (int64_t)t * a.row_stride;
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                const int64_t c = c0 + cq + 16 * ni + c16;
                if (c <= p)
                    row[c] = a.scale * acc[mi][ni][r];
                else if (c < tail_end)
                    row[c] = a.dead;
            }
        }
}

} // namespace

hipError_t launch_score(const ScoreArgs &a, hipStream_t stream)
{
    const int64_t cells = (int64_t)a.pos0 + a.T;
    dim3 grid((unsigned)((cells + kTile - 1) / kTile), (unsigned)((a.T + kTile - 1) / kTile));
    hipLaunchKernelGGL(score_kernel, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

} // namespace qsa
