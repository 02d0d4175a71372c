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
// a 512-thread workgroup adds the heads of its 64 query rows once and then
// walks a run of consecutive 64-cell column tiles, each one a 64 x 64 x 128
// contraction; each of its eight waves owns a 16 x 32 strip as two 16 x 16
// accumulators, which holds it to 112 VGPRs, so two workgroups (16 waves)
// share a CU.
//
// The contraction runs on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16, 16
// times the fp32 MFMA rate) with both operands split into two bf16 parts,
// x = x_hi + x_lo, x_hi = bf16(x) and x_lo = bf16(x - x_hi), contracted as
// hi*hi + hi*lo + lo*hi with fp32 accumulation. bf16 keeps 8 significant bits,
// so |x - x_hi| <= 2^-8 |x| and |x - x_hi - x_lo| <= 2^-16 |x|; the dropped
// lo*lo term is at most 2^-16 |q||k| too, so every product is within
// 3 * 2^-16 |q||k| and a score within 4.6e-5 * scale * sum_d |q_d||k_d|. bf16
// has fp32's exponent range, so no scaling is needed; x_hi is taken from x
// clamped to the largest finite bf16, so an fp32 value beyond it splits into
// that maximum plus a finite remainder, and an infinity into the maximum plus
// an infinity, whose products are infinite exactly as in fp32. (A low part
// below 2^-126 is subnormal in bf16; scores of values that small lose it.)
//
// The score scale multiplies the head-summed q once, before its split
// (scale * (q . k) = (scale * q) . k up to rounding), and each wave keeps its
// 16 rows' split operands in registers for the whole walk. K tiles are split
// into bf16 parts as they are staged, into two LDS buffers used in turn: the
// next tile is read into registers before the current one is multiplied and
// staged into the other buffer after, so one barrier per tile suffices and
// the reads are issued ahead of the current tile's score stores (loads and
// stores share one completion counter, so a read issued after the stores
// could not be waited for without waiting for them too). Tiles wholly beyond
// the last causal cell of their rows end the walk (such tiles hold no tail
// either, since the tail never crosses a 64-cell boundary), and tiles wholly
// inside every row's causal range are stored without per-cell tests. Where
// every row starts 64-byte aligned (row_stride a multiple of 16), scores are
// written with nontemporal stores: a row of scores is written once and read by
// a later kernel, so it streams past the caches instead of evicting the K rows
// that the other workgroups are still reading. Rows that start inside a
// 64-byte segment have segments that two store instructions share; cached
// stores let L2 join them, which nontemporal stores would not.
// Workgroups are ordered so that each XCD (workgroup id mod 8) walks a
// contiguous range of column runs, and the K rows one XCD reads stay within
// its own L2; where that leaves the XCDs unbalanced (rows of very different
// lengths near the start of a sequence), each XCD takes every eighth row tile
// instead.
//
// Every workgroup that walks a run of a row tile sums that tile's heads, so q
// is read once per run (16 times at 1984 rows), in a burst when the launch
// starts, before any walk. With a workspace (qsa_score_ws) a first pass sums
// each 16-row strip's heads once, scales and splits them, and writes the
// operands in the order the walk's waves hold them; the walk then loads its
// operands with eight 16-byte reads per lane. Both paths add the heads in the
// same order and split the same values, so their scores are the same bits.
#include "qsa_internal.h"

#include <algorithm>

namespace qsa {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;
constexpr int kQPitch = kD + 4;  // fp32 q staging pitch (floats)
constexpr int kKPitch = kD + 8;  // bf16 K tile pitch (elements): 272-byte rows, so the
                                 // 16 rows of one operand read start 4 banks apart
constexpr int kScoreThreads = 512;  // 8 waves: 4 row strips of 16 x 2 column halves of 32
constexpr int kSlots = 512;      // resident workgroups: 256 CUs x 2 (LDS and VGPRs allow two)
constexpr int kQBytes = kTile * kQPitch * 4;
constexpr int kKBytes = 2 * kTile * kKPitch * 2;          // one K tile: hi rows, then lo rows
static_assert(kQBytes <= kKBytes, "the q staging fits in one K buffer");
constexpr int kLdsBytes = 2 * kKBytes;                     // two K buffers
constexpr float kBf16Max = 3.38953139e38f;   // largest finite bf16, 0x7f7f
constexpr int64_t kPrepareBytes = int64_t(4) << 20;   // q size from which qsa_score_ws sums heads first

typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// x = hi + lo as above, for two values (one packed conversion for each part).
// No contraction: x - hi is a subtraction of the rounded x, whatever product x
// came from, so every caller splits the same value the same way.
__device__ inline void split2(float x0, float x1, bf16x2 &hi, bf16x2 &lo)
{
#pragma clang fp contract(off)
    const float2v c = {__builtin_amdgcn_fmed3f(x0, -kBf16Max, kBf16Max),
                       __builtin_amdgcn_fmed3f(x1, -kBf16Max, kBf16Max)};
    hi = __builtin_convertvector(c, bf16x2);
    const float2v r = {x0 - (float)hi[0], x1 - (float)hi[1]};
    lo = __builtin_convertvector(r, bf16x2);
}

__device__ inline void split8(const float4 &a, const float4 &b, bf16x8 &hi, bf16x8 &lo)
{
    bf16x2 h[4], l[4];
    split2(a.x, a.y, h[0], l[0]);
    split2(a.z, a.w, h[1], l[1]);
    split2(b.x, b.y, h[2], l[2]);
    split2(b.z, b.w, h[3], l[3]);
    hi = (bf16x8){h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
    lo = (bf16x8){l[0][0], l[0][1], l[1][0], l[1][1], l[2][0], l[2][1], l[3][0], l[3][1]};
}

__device__ inline void split4(const floatx4 &a, bf16x4 &hi, bf16x4 &lo)
{
    bf16x2 h[2], l[2];
    split2(a.x, a.y, h[0], l[0]);
    split2(a.z, a.w, h[1], l[1]);
    hi = (bf16x4){h[0][0], h[0][1], h[1][0], h[1][1]};
    lo = (bf16x4){l[0][0], l[0][1], l[1][0], l[1][1]};
}

// q rows r0 .. r0 + R - 1 summed over heads into rows[0 .. R - 1] (zero for
// rows at or past T), by the NT threads of a workgroup, a float4 per
// thread-step
template <int R, int NT>
__device__ inline void sum_heads(const ScoreArgs &a, int r0, float (*rows)[kQPitch], int tid)
{
    for (int idx = tid; idx < R * (kD / 4); idx += NT) {
        const int row = idx >> 5, c4 = idx & 31;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        const int t = r0 + row;
        if (t < a.T) {
            // every head's read is issued before the first add (one round trip
            // per row, not one per few heads); the adds keep head order
            const float *qr = a.q + (int64_t)t * a.Hs * kD + 4 * c4;
            // (heads go in groups of four, each group behind one uniform branch;
            // inside a group, indexes past Hs re-read the last head, with no
            // branch per load; those values are not added)
            float4 v[kMaxHeads];
#pragma unroll
            for (int h4 = 0; h4 < kMaxHeads; h4 += 4)
                if (h4 < a.Hs) {                     // uniform: groups of four heads that hold a head
#pragma unroll
                    for (int h = h4; h < h4 + 4; ++h)
                        v[h] = *(const float4 *)(qr + (int64_t)min(h, a.Hs - 1) * kD);
                }
#pragma unroll
            for (int h = 0; h < kMaxHeads; ++h)
                if (h < a.Hs) {
                    acc.x += v[h].x; acc.y += v[h].y; acc.z += v[h].z; acc.w += v[h].w;
                }
        }
        *(float4 *)&rows[row][4 * c4] = acc;
    }
}

// the A operand of lane (j, c16) for k-step ks: the staged head sum of row
// c16 of `rows`, dims 32 ks + 8j .. +7, times the score scale (scale * (q . k)
// = (scale * q) . k), split into bf16 parts
__device__ inline void a_operand(const ScoreArgs &a, const float (*rows)[kQPitch], int ks, int j, int c16,
                                 bf16x8 &hi, bf16x8 &lo)
{
    const float *src = &rows[c16][32 * ks + 8 * j];
    float4 u = *(const float4 *)src, v = *(const float4 *)(src + 4);
    u.x *= a.scale; u.y *= a.scale; u.z *= a.scale; u.w *= a.scale;
    v.x *= a.scale; v.y *= a.scale; v.z *= a.scale; v.w *= a.scale;
    split8(u, v, hi, lo);
}

// Workspace of the prepared path: per 16-row strip, k-step and part (hi, lo),
// the 64 lanes' 16-byte operands: entry ((strip * 4 + ks) * 2 + part) * 64 + lane.
constexpr int kStripOperands = 4 * 2 * 64;       // uint4 entries per strip (8 KB)

// One 16-row strip: its heads summed into LDS, then wave ks writes the
// operands of k-step ks. Rows past T get zero operands (never multiplied
// into a written score).
__global__ __launch_bounds__(256) void prep_kernel(ScoreArgs a, uint4 *ws)
{
    __shared__ __align__(16) float sq[16][kQPitch];
    const int strip = blockIdx.x, tid = threadIdx.x;
    sum_heads<16, 256>(a, 16 * strip, sq, tid);
    __syncthreads();
    const int lane = tid & 63, ks = tid >> 6;
    bf16x8 hi, lo;
    a_operand(a, sq, ks, lane >> 4, lane & 15, hi, lo);
    uint4 *dst = ws + (int64_t)strip * kStripOperands + ks * 128 + lane;
    dst[0] = __builtin_bit_cast(uint4, hi);
    dst[64] = __builtin_bit_cast(uint4, lo);
}

// the thread's staged K values (rows (tid >> 5) + 16i, column 4 * (tid & 31))
// split into bf16 high and low parts, into the K buffer at `buf`
__device__ inline void stage_k(uint8_t *buf, const floatx4 (&kreg)[4], int tid)
{
    __bf16 (*kh)[kKPitch] = (__bf16 (*)[kKPitch])buf;
    __bf16 (*kl)[kKPitch] = (__bf16 (*)[kKPitch])(buf + kTile * kKPitch * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        bf16x4 h, l;
        split4(kreg[i], h, l);
        *(bf16x4 *)&kh[(tid >> 5) + 16 * i][4 * (tid & 31)] = h;
        *(bf16x4 *)&kl[(tid >> 5) + 16 * i][4 * (tid & 31)] = l;
    }
}

// A score store: nontemporal where every row starts 64-byte aligned (each
// store instruction then writes whole 64-byte segments that nothing else
// touches), cached otherwise, so that L2 joins the pieces of segments that
// straddle two instructions' rows before they go to memory.
template <bool kNT>
__device__ inline void put(float v, float *p)
{
    if constexpr (kNT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

template <bool kPrepared, bool kNT>
__global__ __launch_bounds__(kScoreThreads, 4) void score_kernel(ScoreArgs a, int n_row_tiles, int run_len, int n_runs, int blocks_per_xcd,
                                                                   int by_row, const uint4 *ws)
{
    // two bf16 K buffers (hi rows, then lo rows); the fp32 q staging shares the second
    __shared__ __align__(16) uint8_t lds[kLdsBytes];
    float (*sq)[kQPitch] = (float (*)[kQPitch])(lds + kKBytes);

    int run, rt;
    if (by_row) {
        // XCD x (workgroup id mod 8) takes row tiles x, x + 8, ..., each with all its runs
        const int i = blockIdx.x >> 3;
        const int m = i / n_runs;
        run = i - m * n_runs;
        rt = (blockIdx.x & 7) + 8 * m;
        if (rt >= n_row_tiles)
            return;                          // uniform over the workgroup
    } else {
        // XCD x takes a contiguous range of runs, each with all its row tiles
        const int lb = (blockIdx.x & 7) * blocks_per_xcd + (blockIdx.x >> 3);
        if (lb >= n_row_tiles * n_runs)
            return;
        run = lb / n_row_tiles;
        rt = lb - run * n_row_tiles;
    }
    const int r0 = rt * kTile;
    const int last_row = min(a.T, r0 + kTile) - 1;
    const int64_t last_causal = (int64_t)a.pos0 + last_row;
    const int64_t first_causal = (int64_t)a.pos0 + r0;    // the tile's first row's last causal cell
    const bool full_rows = r0 + kTile <= a.T;
    const int ct0 = run * run_len;
    if ((int64_t)ct0 * kTile > last_causal)
        return;

    const int tid = threadIdx.x;
    if constexpr (!kPrepared)
        sum_heads<kTile, kScoreThreads>(a, r0, sq, tid);   // q rows of this tile, summed over heads

    // K tile staging: thread tid moves 4 float4s, rows (tid >> 5) + 16i, column 4 * (tid & 31)
    floatx4 kreg[4];
    auto fetch = [&](int ct) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // a cell past the cache stages a copy of the last cell: a K row
            // feeds only its own score column, and such a column lies past
            // every row's causal edge (n_cells >= pos0 + T), so its value is
            // never written; the load stays unconditional, free of any branch
            const int c = min(ct * kTile + (tid >> 5) + 16 * i, a.n_cells - 1);
            kreg[i] = *(const floatx4 *)(a.k + (int64_t)c * kD + 4 * (tid & 31));
        }
    };
    fetch(ct0);

    const int lane = tid & 63, w = tid >> 6;
    const int j = lane >> 4, c16 = lane & 15;
    const int rq = 16 * (w >> 1), cq = 32 * (w & 1);   // this wave's 16 x 32 strip
    const bool live = r0 + rq < a.T;                     // uniform: a strip past the last row only stages

    // A operands, held for the whole walk: row rq + c16, dims 32 ks + 8j .. +7
    bf16x8 ah[4], al[4];
    if constexpr (kPrepared) {
        const uint4 *src = ws + (int64_t)(4 * rt + (w >> 1)) * kStripOperands + lane;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            ah[ks] = __builtin_bit_cast(bf16x8, src[ks * 128]);
            al[ks] = __builtin_bit_cast(bf16x8, src[ks * 128 + 64]);
        }
    } else {
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            a_operand(a, sq + rq, ks, j, c16, ah[ks], al[ks]);
    }
    stage_k(lds, kreg, tid);                 // the first tile into buffer 0
    __syncthreads();                         // buffer 0 complete; the q staging is free

    // Per tile: issue the next tile's reads, multiply this one, then wait for
    // the reads and stage the next tile into the other buffer before storing
    // this tile's scores. A wait for reads issued before the previous tile's
    // stores then finds those stores long finished (loads and stores share
    // one counter), and one barrier per tile suffices.
    int b = 0;
    for (int ct = ct0; ct < ct0 + run_len; ++ct, b ^= 1) {
        const int c0 = ct * kTile;
        if ((int64_t)c0 > last_causal)
            break;                           // uniform: later tiles are further out
        // the next tile, or (the walk's last tile) this one again: the reads and
        // the staging below run on every tile, with no branch around them
        const bool next = ct + 1 < ct0 + run_len && (int64_t)(c0 + kTile) <= last_causal;
        fetch(next ? ct + 1 : ct);
        __builtin_amdgcn_sched_barrier(0);   // the reads go out before the contraction
        const __bf16 (*kh)[kKPitch] = (const __bf16 (*)[kKPitch])(lds + b * kKBytes);
        const __bf16 (*kl)[kKPitch] = (const __bf16 (*)[kKPitch])(lds + b * kKBytes + kTile * kKPitch * 2);

        floatx4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        if (live) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                // B operand: cell cq + 16 ni + c16, dims 32 ks + 8j .. +7
                bf16x8 bh[2], bl[2];
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) {
                    bh[ni] = *(const bf16x8 *)&kh[cq + 16 * ni + c16][32 * ks + 8 * j];
                    bl[ni] = *(const bf16x8 *)&kl[cq + 16 * ni + c16][32 * ks + 8 * j];
                }
                // the two accumulators are independent: interleave them between steps
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[ks], bh[ni], acc[ni], 0, 0, 0);
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[ks], bl[ni], acc[ni], 0, 0, 0);
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[ks], bh[ni], acc[ni], 0, 0, 0);
            }
        }
        // the staging waits for the reads: keep it behind the contraction
        __builtin_amdgcn_sched_barrier(0);
        stage_k(lds + (b ^ 1) * kKBytes, kreg, tid);   // unread after the last tile

        // D layout: lane (j, c16) holds rows 4j + r, column c16 of each 16 x 16 tile
        if (live && full_rows && (int64_t)c0 + kTile - 1 <= first_causal) {
            // every cell of the tile is causal for every row of the tile
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float *row = a.scores + (int64_t)(r0 + rq + 4 * j + r) * a.row_stride + c0 + cq + c16;
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    put<kNT>(acc[ni][r], &row[16 * ni]);
            }
        } else if (live) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = r0 + rq + 4 * j + r;
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
                        put<kNT>(acc[ni][r], &row[c]);
                    else if (c < tail_end)
                        put<kNT>(a.dead, &row[c]);
                }
            }
        }
        __syncthreads();                     // the next tile is staged; this buffer is free
    }
}

} // namespace

hipError_t launch_score(const ScoreArgs &a, void *ws, hipStream_t stream)
{
    const int64_t cells = (int64_t)a.pos0 + a.T;
    const int n_col_tiles = (int)((cells + kTile - 1) / kTile);
    const int n_row_tiles = (a.T + kTile - 1) / kTile;
    // as many column runs per row tile as fill the chip's workgroup slots in
    // one round, so that few query rows still spread over the chip, but at
    // least four tiles per run to share each workgroup's head sum and split
    // (a call of at most 16 rows, such as a decode step, sums so few heads
    // that one tile per run is worth it: T = 1 and 8 at pos0 = 30000 run in
    // 7.7 and 8.6 us instead of 9.8 and 11.4)
    const int want_runs = std::max(1, std::min(n_col_tiles, kSlots / n_row_tiles));
    const int min_run = a.T <= 16 ? 1 : 4;
    const int run_len = std::max(min_run, (n_col_tiles + want_runs - 1) / want_runs);
    const int n_runs = (n_col_tiles + run_len - 1) / run_len;
    const int64_t blocks = (int64_t)n_runs * n_row_tiles;
    const int run_major_per_xcd = (int)((blocks + 7) / 8);

    // Column tiles per XCD under both workgroup orders. Runs on one XCD keep
    // the K rows it reads within its own L2, which long contexts need (each
    // XCD reads an eighth of K); but where row lengths differ (a causal
    // triangle near the start of a sequence) whole runs hold little or no
    // work, and XCDs that each take every eighth row tile balance it.
    int64_t by_runs[8] = {}, by_rows[8] = {};
    for (int rt = 0; rt < n_row_tiles; ++rt) {
        const int64_t last_tile = ((int64_t)a.pos0 + std::min(a.T, (rt + 1) * kTile) - 1) / kTile;
        for (int run = 0; run < n_runs; ++run) {
            const int64_t lo = (int64_t)run * run_len;
            const int64_t hi = std::min<int64_t>(lo + run_len, n_col_tiles) - 1;
            const int64_t w = std::max<int64_t>(0, std::min(hi, last_tile) - lo + 1);
            by_runs[((int64_t)run * n_row_tiles + rt) / run_major_per_xcd] += w;
            by_rows[rt & 7] += w;
        }
    }
    const int64_t max_runs = *std::max_element(by_runs, by_runs + 8);
    const int64_t max_rows = *std::max_element(by_rows, by_rows + 8);
    const int by_row = n_row_tiles >= 8 && 8 * max_rows < 7 * max_runs;
    const int per_xcd = by_row ? ((n_row_tiles + 7) / 8) * n_runs : run_major_per_xcd;
    // The first pass pays where the walk's workgroups would read q from beyond
    // L2 many times over: in the run-major order every XCD reads all of q
    // (eight times q's size in L2 misses, 96 MB at 1984 rows of 12 heads);
    // with a small q (decode steps, one head) or in the row-major order (each
    // XCD reads an eighth of q) the extra launch costs more than it saves.
    const bool prepare = ws && !by_row && (int64_t)a.T * a.Hs * kD * 4 >= kPrepareBytes;
    if (prepare)
        // one strip of operands per 16 rows of every row tile (the last tile's
        // rows past T included), so the walk's reads stay inside the workspace
        hipLaunchKernelGGL(prep_kernel, dim3(4 * n_row_tiles), dim3(256), 0, stream, a, (uint4 *)ws);
    // Nontemporal stores where every row starts 64-byte aligned; cached where
    // rows straddle segments, which nontemporal stores would write piecemeal
    // (T = 1984, pos0 = 30000: 80 us aligned; with an odd row stride 213 us
    // nontemporal against 106 us cached)
    const bool nt = ((uintptr_t)a.scores & 63) == 0 && a.row_stride % 16 == 0;
    const dim3 grid(8 * per_xcd), block(kScoreThreads);
    const uint4 *wsp = prepare ? (const uint4 *)ws : nullptr;
    if (prepare && nt)
        hipLaunchKernelGGL((score_kernel<true, true>), grid, block, 0, stream, a, n_row_tiles, run_len, n_runs,
                           run_major_per_xcd, by_row, wsp);
    else if (prepare)
        hipLaunchKernelGGL((score_kernel<true, false>), grid, block, 0, stream, a, n_row_tiles, run_len, n_runs,
                           run_major_per_xcd, by_row, wsp);
    else if (nt)
        hipLaunchKernelGGL((score_kernel<false, true>), grid, block, 0, stream, a, n_row_tiles, run_len, n_runs,
                           run_major_per_xcd, by_row, wsp);
    else
        hipLaunchKernelGGL((score_kernel<false, false>), grid, block, 0, stream, a, n_row_tiles, run_len, n_runs,
                           run_major_per_xcd, by_row, wsp);
    return hipGetLastError();
}

} // namespace qsa
