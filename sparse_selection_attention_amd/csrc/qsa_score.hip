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
// a 256-thread workgroup adds the heads of its 64 query rows once into LDS and
// then walks a run of consecutive 64-cell column tiles, each one a
// 64 x 64 x 128 fp32 contraction on v_mfma_f32_16x16x4_f32 (each wave a 32 x 32
// quadrant as four 16 x 16 accumulators). The next K tile is fetched into
// registers while the current one is multiplied. Tiles wholly beyond the last
// causal cell of their rows end the walk (such tiles hold no tail either, since
// the tail never crosses a 64-cell boundary). Workgroups are ordered so that
// each XCD (workgroup id mod 8) walks a contiguous range of column runs: the K
// rows one XCD reads stay within its own L2.
#include "qsa_internal.h"

#include <algorithm>

namespace qsa {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;
constexpr int kPitch = kD + 4;   // LDS row pitch in floats: rows 16 B apart in bank space
constexpr int kMaxRun = 32;      // column tiles per workgroup, at most

__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a, int n_row_tiles, int run_len, int n_runs, int blocks_per_xcd)
{
    __shared__ float sq[kTile][kPitch];
    __shared__ float sk[kTile][kPitch];

    const int lb = (blockIdx.x & 7) * blocks_per_xcd + (blockIdx.x >> 3);
    if (lb >= n_row_tiles * n_runs)
        return;                              // uniform over the workgroup
    const int run = lb / n_row_tiles;
    const int rt = lb - run * n_row_tiles;
    const int r0 = rt * kTile;
    const int last_row = min(a.T, r0 + kTile) - 1;
    const int64_t last_causal = (int64_t)a.pos0 + last_row;
    const int ct0 = run * run_len;
    if ((int64_t)ct0 * kTile > last_causal)
        return;

    const int tid = threadIdx.x;
    // q rows of this tile, summed over heads, float4 per thread-step
    for (int idx = tid; idx < kTile * (kD / 4); idx += 256) {
        const int row = idx >> 5, c4 = idx & 31;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        const int t = r0 + row;
        if (t < a.T) {
            // every head's read is issued before the first add (one round trip
            // per row, not one per few heads); the adds keep head order
            const float *qr = a.q + (int64_t)t * a.Hs * kD + 4 * c4;
            // (indexes past Hs re-read the last head, unconditionally, so that no
            // load is tied to a branch; those values are not added)
            float4 v[kMaxHeads];
#pragma unroll
            for (int h = 0; h < kMaxHeads; ++h)
                v[h] = *(const float4 *)(qr + (int64_t)min(h, a.Hs - 1) * kD);
#pragma unroll
            for (int h = 0; h < kMaxHeads; ++h)
                if (h < a.Hs) {
                    acc.x += v[h].x; acc.y += v[h].y; acc.z += v[h].z; acc.w += v[h].w;
                }
        }
        *(float4 *)&sq[row][4 * c4] = acc;
    }

    // K tile staging: thread tid moves 8 float4s, rows (tid >> 5) + 8i, column 4 * (tid & 31)
    floatx4 kreg[8];
    auto fetch = [&](int ct) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // a cell past the cache stages a copy of the last cell: a K row
            // feeds only its own score column, and such a column lies past
            // every row's causal edge (n_cells >= pos0 + T), so its value is
            // never written; the load stays unconditional, free of any branch
            const int c = min(ct * kTile + (tid >> 5) + 8 * i, a.n_cells - 1);
            kreg[i] = *(const floatx4 *)(a.k + (int64_t)c * kD + 4 * (tid & 31));
        }
    };
    fetch(ct0);

    const int lane = tid & 63, w = tid >> 6;
    const int j = lane >> 4, c16 = lane & 15;
    const int rq = 32 * (w >> 1), cq = 32 * (w & 1);   // this wave's quadrant

    for (int ct = ct0; ct < ct0 + run_len; ++ct) {
        const int c0 = ct * kTile;
        if ((int64_t)c0 > last_causal)
            break;                           // uniform: later tiles are further out
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *(floatx4 *)&sk[(tid >> 5) + 8 * i][4 * (tid & 31)] = kreg[i];
        __syncthreads();
        if (ct + 1 < ct0 + run_len && (int64_t)(c0 + kTile) <= last_causal)
            fetch(ct + 1);                   // in flight during the contraction

        floatx4 acc[2][2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                acc[mi][ni] = (floatx4){0.f, 0.f, 0.f, 0.f};
        // k-slot j of MFMA (u, e) is dim 4 * (4u + j) + e, for A and B alike
#pragma unroll 4
        for (int u = 0; u < 8; ++u) {
            float4 av[2], bv[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                av[mi] = *(const float4 *)&sq[rq + 16 * mi + c16][4 * (4 * u + j)];
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                bv[ni] = *(const float4 *)&sk[cq + 16 * ni + c16][4 * (4 * u + j)];
            // the four accumulators are independent: interleave them between steps
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[mi].x, bv[ni].x, acc[mi][ni], 0, 0, 0);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[mi].y, bv[ni].y, acc[mi][ni], 0, 0, 0);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[mi].z, bv[ni].z, acc[mi][ni], 0, 0, 0);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[mi].w, bv[ni].w, acc[mi][ni], 0, 0, 0);
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
        __syncthreads();                     // sk is rewritten next
    }
}

} // namespace

hipError_t launch_score(const ScoreArgs &a, hipStream_t stream)
{
    const int64_t cells = (int64_t)a.pos0 + a.T;
    const int n_col_tiles = (int)((cells + kTile - 1) / kTile);
    // longer runs share the head-summed q over more tiles; shorter runs spread
    // the short rows of a prompt start over more workgroups
    const int run_len = std::max(4, std::min(kMaxRun, (n_col_tiles + 15) / 16));
    const int n_runs = (n_col_tiles + run_len - 1) / run_len;
    const int n_row_tiles = (a.T + kTile - 1) / kTile;
    const int64_t blocks = (int64_t)n_runs * n_row_tiles;
    const int per_xcd = (int)((blocks + 7) / 8);
    hipLaunchKernelGGL(score_kernel, dim3(8 * per_xcd), dim3(256), 0, stream, a, n_row_tiles, run_len, n_runs, per_xcd);
    return hipGetLastError();
}

} // namespace qsa
