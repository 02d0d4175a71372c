// qsa_tile.hip -- implicit rows: a block of prompt queries shares each chunk's
// cells, so QK and PV become dense MFMA tile contractions.
//
// With implicit rows every query token t selects cells 0 .. p (p = pos0 + t),
// so chunk k (cells 64k .. 64k+63) is the same 64 cells for every token that
// reaches it ("round 11 track b: qsa attention and score", sections
// "boundaries and provenance" and "implementation and evaluator"; the chunk
// statistics and the merge relative to the largest chunk maximum follow
// "round 5 track b: cached residual norms and fused mtp attention", section
// "mtp attention"). The (token, head) pairs of consecutive tokens are the rows
// of one contraction: row r is token r / H, head r % H, which is also q's and
// the output's memory order.
//
// Design on CDNA4. A group of four waves owns 64 consecutive rows, 16 per
// wave, and walks the chunks up to its last token's causal edge:
//   * reads: the next chunk's K and V rows are read into registers while the
//     current chunk is contracted; each K read instruction covers whole
//     128-byte cache rows (eight lanes of 16 bytes per row), each V read gives
//     a lane 8 dims of one of four consecutive cells (the layout the
//     transposed tile is written in), and the K and V scales of the chunk's
//     64 cells are one contiguous 512-byte run each;
//   * staging, once per chunk for all four waves: K to LDS as fp16 (exact),
//     [cell][dim]; V transposed, [dim][position], as its int8 codes in fp16
//     (exact), cells permuted so that each PV operand read is one 16-byte
//     load; both tiles are XOR-swizzled in 16-byte granules for conflict-free
//     operand reads. The V scales go to LDS per scale group, each group times
//     its own power of two 2^kg, chosen from the chunk's largest scale of the
//     group so that p * vsc * 2^kg stays below 2^15;
//   * QK: v_mfma_f32_16x16x32_f16 with A = 16 cells x 32 dims of one scale
//     group and B = the wave's 16 q rows, one fp32 partial per scale group,
//     weighted by the cell's group scale; a lane then holds 16 of its row's
//     64 scores, so the row max and sum are lane folds plus two exchanges
//     (row-swap permutes, in the VALU).
//     Scores are kept in log2 units (the softmax scale is applied times
//     log2(e)), so p = exp2(S - max) needs no multiply;
//   * causality is a per-row mask: cell c counts for row r iff
//     c <= pos0 + r / H (and c < n_cells);
//   * PV: O^T = V^T P^T on the same MFMA. Each MFMA's 16 output dims lie in
//     one scale group, so the group's V scales fold into p: B = p * vsc * 2^kg
//     as fp16 high and low parts (high: the fp16 product; low: its residual
//     from one fp16 fma plus the low part of p times the scale), and A = the
//     exact V codes. Two MFMAs per tile carry about 22 bits of each product,
//     and 2^-kg comes back out exactly;
//   * chunk records (qsa_attn): one (m, l, o) per row and chunk, rows past
//     their causal edge writing the empty record (-inf, 0); the chunks of a
//     row block are split over workgroups of at most 8 chunks each, so the
//     long rows of late tokens do not serialise; fused (qsa_attn_merge): a
//     running max, denominator and output per row, rescaled as each chunk's
//     max (or a group's power of two) moves, divided once at the end. A fused
//     workgroup holds three such groups of four waves, each with its own LDS
//     tiles, walking every third chunk of the same rows; their states are
//     combined through LDS at the end (the same max-first rule), so the
//     longest row block walks a third as many chunks in sequence.
// The gated entry point multiplies each fused output by sigmoid(g) of its fp32
// gate before the fp16 rounding and may write the exact per-16 sums of the
// written values ("round 5 track b: cached residual norms and fused mtp
// attention", section "preflight / ownership").
// Workgroups start with the heaviest row blocks (the last tokens, with the most
// chunks).
#include "qsa_internal.h"
#include "qsa_device.h"

namespace qsa {
namespace {

using namespace dev;

constexpr int kTileRows = 64;                  // (token, head) rows per workgroup
constexpr int kTileThreads = 256;

// LDS layout of one group
constexpr int kLK = 0;                         // K fp16 [64 cells][128 dims], 256-byte rows
constexpr int kLV = kLK + kChunk * kD * 2;     // V^T codes fp16 [128 dims][64 positions], 128-byte rows
constexpr int kLKs = kLV + kD * kChunk * 2;    // K scales fp16 [64 cells][4]
constexpr int kVsRow = 144;                    // one group's 64 V scales (128 B) plus a 16-byte pad
constexpr int kLVs = kLKs + kChunk * 8;        // V scales times 2^kg, fp16 [4 groups][kVsRow bytes]
constexpr int kLE = kLVs + 4 * kVsRow;         // int[4 waves][4 groups]: largest V-scale exponents
constexpr int kGroupState = 4 * 64 * 36 * 4;   // end-of-walk (M, L, O) of the group's 256 lanes
constexpr int kTileLds = (kLE + 64 > kGroupState) ? kLE + 64 : kGroupState;
constexpr int kSplit = 8;                      // chunks per workgroup in the chunk-record kernel
constexpr int kFusedGroups = 3;                // groups of four waves per fused workgroup
static_assert(kTileLds % 16 == 0, "group regions stay 16-byte aligned");

// K tile: cell c's logical granule gi (dims 8gi .. 8gi+7) at gi ^ (c & 15)
__device__ inline int tk_offset(int c, int gi) { return kLK + c * 256 + ((gi ^ (c & 15)) << 4); }
// V^T tile: dim d's logical granule gp (positions 8gp .. 8gp+7) at gp ^ ((d >> 1) & 7)
__device__ inline int tv_offset(int d, int gp) { return kLV + d * 128 + ((gp ^ ((d >> 1) & 7)) << 4); }

// Position 32ks + 8j + s of a 64-cell chunk holds cell 32ks + 16(s/4) + 4j + s%4:
// the cells whose scores lane group j holds, in PV operand slot order. The
// inverse: cell c sits at position 32(c/32) + 8((c%16)/4) + 4((c%32)/16) + c%4.
__device__ inline int cell_pos(int c)
{
    return 32 * (c >> 5) + 8 * ((c >> 2) & 3) + 4 * ((c >> 4) & 1) + (c & 3);
}

// What each thread (wave w, lane L) reads of a chunk, into registers:
//   K: cells 16w + 8i + L/8 (i = 0, 1), dims 16(L%8) .. +15 -- eight lanes
//      per 128-byte row, eight rows per instruction;
//   V: dims 8db .. +7 (db = tid / 16) of the four consecutive cells at
//      positions 4pq .. 4pq + 3 (pq = tid % 16), in the layout the transposed
//      tile is written in: sixteen lanes then store one dim's sixteen 8-byte
//      pieces into distinct banks;
//   scales: cell 16w + L/4, group L%4, of K and of V -- the chunk's scales
//      are one contiguous 512-byte run.
__device__ inline int v_cell0(int pq) { return 32 * (pq >> 3) + 16 * (pq & 1) + 4 * ((pq >> 1) & 3); }

struct Raw {
    uint4 k[2];        // K: 16 bytes of each of two cells
    uint2 v[4];        // V: 8 dims of 4 consecutive cells
    uint32_t ks, vs;   // the K and V scale of one (cell, group), fp16 bits
};

// Issue the chunk's global reads. Every read is unconditional (cells past the
// cache read the last cached row) so that the reads stay in flight; the cells
// that do not exist are zeroed once the reads have landed (zero_missing). Byte
// offsets fit 32 bits: n_cells * 128 < 2^32.
__device__ inline void load_raw(const AttnArgs &a, int c0, int tid, Raw &R)
{
    const int last = a.n_cells - 1;     // >= 0 whenever a chunk is walked
    const int w = tid >> 6, L = tid & 63;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = c0 + 16 * w + 8 * i + (L >> 3);
        const uint32_t cc = (uint32_t)min(c, last);
        R.k[i] = *(const uint4 *)(a.kq + (cc * kD + 16 * (L & 7)));
    }
    const int cs = c0 + 16 * w + (L >> 2);
    const uint32_t ccs = (uint32_t)min(cs, last);
    R.ks = a.ksc[ccs * 4 + (L & 3)];
    R.vs = a.vsc[ccs * 4 + (L & 3)];
    const int db = tid >> 4, pq = tid & 15;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int c = c0 + v_cell0(pq) + s;
        const uint32_t cc = (uint32_t)min(c, last);
        R.v[s] = *(const uint2 *)(a.vq + (cc * kD + 8 * db));
    }
}

// Zero what load_raw read for cells at or past n_cells (it read the last
// cached row in their place): codes and scales, so that such a cell adds
// nothing to the tiles, the scores' weights or the V-scale exponents.
__device__ inline void zero_missing(Raw &R, int c0, int n_cells, int tid)
{
    const int w = tid >> 6, L = tid & 63;
#pragma unroll
    for (int i = 0; i < 2; ++i)
        if (c0 + 16 * w + 8 * i + (L >> 3) >= n_cells)
            R.k[i] = make_uint4(0u, 0u, 0u, 0u);
    if (c0 + 16 * w + (L >> 2) >= n_cells) {
        R.ks = 0u;
        R.vs = 0u;
    }
    const int pq = tid & 15;
#pragma unroll
    for (int s = 0; s < 4; ++s)
        if (c0 + v_cell0(pq) + s >= n_cells)
            R.v[s] = make_uint2(0u, 0u);
}

// Largest biased exponent of this thread's V scale over the lanes of the wave
// that hold the same scale group (lane % 4); a cell that does not exist has a
// zero scale (zero_missing), of exponent 0.
__device__ inline int group_max_exponent(const Raw &R)
{
    int e = (int)((R.vs >> 10) & 31u);
    // lanes l, l + 4, l + 8, l + 12 of a row: two row rotations (by 4, then 8)
    e = max(e, __builtin_amdgcn_update_dpp(0, e, 0x124, 0xf, 0xf, false));   // row_ror:4
    e = max(e, __builtin_amdgcn_update_dpp(0, e, 0x128, 0xf, 0xf, false));   // row_ror:8
    return xor32_max(xor16_max(e));
}

// The power of two that scale group g carries in this chunk: with eg the
// group's largest biased fp16 exponent, every scale is below 2^(eg - 14), so
// scale * 2^(29 - eg) < 2^15 and p * scale * 2^kg stays clear of the fp16
// limit. Scaling up is exact in fp16 (eg = 30 gives kg = -1, which may round
// scales below 2^-13 by the half of an fp16 subnormal step).
__device__ inline int group_shift(int eg) { return 29 - eg; }

// 2^k as a float (|k| < 126)
__device__ inline float pow2i(int k) { return __int_as_float((127 + k) << 23); }

// Convert the chunk's raw rows into the LDS tiles. kg[g] is scale group g's
// power of two for this chunk.
__device__ inline void stage_tiles(uint8_t *lds, int tid, const Raw &R, const int (&kg)[4])
{
    const int w = tid >> 6, L = tid & 63;
    // K: 16 dims (granules 2m and 2m + 1, m = L % 8) of each of two cells as
    // fp16 (exact)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = 16 * w + 8 * i + (L >> 3);
        const uint4 kr = R.k[i];
        *(half8 *)(lds + tk_offset(c, 2 * (L & 7))) = i8x8_to_half8(make_uint2(kr.x, kr.y));
        *(half8 *)(lds + tk_offset(c, 2 * (L & 7) + 1)) = i8x8_to_half8(make_uint2(kr.z, kr.w));
    }
    // the (cell, group) scales: K as read, V times 2^kg at the cell's position
    const int cs = 16 * w + (L >> 2), g = L & 3;
    *(uint16_t *)(lds + kLKs + cs * 8 + 2 * g) = (uint16_t)R.ks;
    const int kgs = g == 0 ? kg[0] : g == 1 ? kg[1] : g == 2 ? kg[2] : kg[3];
    const _Float16 vsn = (_Float16)(half_bits_to_float(R.vs) * pow2i(kgs));
    *(_Float16 *)(lds + kLVs + g * kVsRow + 2 * cell_pos(cs)) = vsn;
    // V: dims 8db .. +7 of positions 4pq .. +3 as fp16 codes (exact), transposed
    const uint2 (&v)[4] = R.v;
    const I8Scale cv = i8_scale(0);
    const int db = tid >> 4, pq = tid & 15;
    const int gp = pq >> 1, half = 8 * (pq & 1);
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
        const uint32_t x0 = dd < 4 ? v[0].x : v[0].y, x1 = dd < 4 ? v[1].x : v[1].y;
        const uint32_t x2 = dd < 4 ? v[2].x : v[2].y, x3 = dd < 4 ? v[3].x : v[3].y;
        const int d = 8 * db + dd;
        *(uint2 *)(lds + tv_offset(d, gp) + half) =
            make_uint2(cvt2_sel(dd & 3, x0, x1, cv), cvt2_sel(dd & 3, x2, x3, cv));
    }
}

// Scores of the chunk's 64 cells for this lane's row, in log2 units: the four
// group partials of QK weighted by the cells' K scales, times kmul (the
// softmax scale times log2(e)); with kMask, cells past the row's last valid
// cell get -inf (chunks that lie wholly inside every row's causal range skip
// the test).
template <bool kMask>
__device__ inline void qk_scores(const uint8_t *lds, const half8 (&qop)[4], int j, int c16, int c0, int lim,
                                 float kmul, float nz, float (&S)[4][4])
{
    const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        floatx4 acc[4];
        const int ca = 16 * b + c16;            // A operand row: cell ca, dims 32g + 8j .. +7
#pragma unroll
        for (int g = 0; g < 4; ++g)
            acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(*(const half8 *)(lds + tk_offset(ca, 4 * g + j)),
                                                            qop[g], zero, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int cell = 16 * b + 4 * j + r;
            const uint2 kb = *(const uint2 *)(lds + kLKs + cell * 8);
            float dot = __builtin_fmaf(acc[0][r], half_bits_to_float(kb.x & 0xffffu), nz);
            dot = __builtin_fmaf(acc[1][r], half_bits_to_float(kb.x >> 16), dot);
            dot = __builtin_fmaf(acc[2][r], half_bits_to_float(kb.y & 0xffffu), dot);
            dot = __builtin_fmaf(acc[3][r], half_bits_to_float(kb.y >> 16), dot);
            S[b][r] = (!kMask || c0 + cell <= lim) ? kmul * dot : -INFINITY;
        }
    }
}

// O[n] += the chunk's V codes weighted by p * vsc * 2^kg: O[n][r] is dim
// 16n + 4j + r of this lane's row, in units of 2^kg of its scale group n / 2.
__device__ inline void pv_accumulate(const uint8_t *lds, const float (&P)[4][4], int j, int c16, floatx4 (&O)[8])
{
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        // p of positions 32ks + 8j + s (cells 32ks + 16(s/4) + 4j + s%4) as
        // fp16 high and low parts, p = hi + lo to within 2^-22
        float pv[8];
#pragma unroll
        for (int s = 0; s < 8; ++s)
            pv[s] = P[2 * ks + (s >> 2)][s & 3];
        half8 ph, pl;
        split_half8(pv, ph, pl);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            // those positions' scales of group g (times 2^kg): B = p * scale as
            // the fp16 product, plus its exact residual and the low part of p
            const half8 sc = *(const half8 *)(lds + kLVs + g * kVsRow + 2 * (32 * ks + 8 * j));
            const half8 bh = ph * sc;
            const half8 bl = __builtin_elementwise_fma(pl, sc, __builtin_elementwise_fma(ph, sc, -bh));
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int n = 2 * g + u;
                const half8 va = *(const half8 *)(lds + tv_offset(16 * n + c16, 4 * ks + j));
                O[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, bh, O[n], 0, 0, 0);
                O[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, bl, O[n], 0, 0, 0);
            }
        }
    }
}

// Synchronisation of the four waves of one group. With one group per
// workgroup it is the workgroup barrier. With several, a workgroup barrier
// would also hold each group for the others, which walk other chunks, so the
// waves of a group meet on a counter in LDS instead: each wave adds one to it
// and waits until the group's four additions of this round are in. The
// counter only grows, and each wave compares it with its own running target.
// The wait polls the counter with LDS reads (a sleep between polls made the
// kernel 2% slower) and is bounded (kBarrierSpins polls, far longer than any
// chunk takes), so every wave always leaves it.
constexpr int kBarrierSpins = 1 << 16;

template <int G>
__device__ inline void group_sync(int *ctr, int &target)
{
    if constexpr (G == 1) {
        __syncthreads();
    } else {
        target += kTileThreads / 64;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");   // this wave's LDS writes are done
        if ((threadIdx.x & 63) == 0)
            __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll 1
        for (int spin = 0; spin < kBarrierSpins; ++spin) {
            const int seen = __builtin_amdgcn_readfirstlane(
                __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
            if (seen >= target)
                break;
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");   // the group's writes are visible
    }
}

// G groups of four waves share a workgroup's rows: group gi walks chunks
// k_lo + gi, k_lo + gi + G, ... with LDS tiles of its own, and the groups'
// running (max, denominator, output) are combined at the end (fused kernel).
template <bool kFused, int G>
__global__ __launch_bounds__(kTileThreads * G) void attn_tile_kernel(AttnArgs a, int n_parts)
{
    __shared__ __align__(16) uint8_t lds_all[G * kTileLds + (G > 1 ? 16 : 0)];
    const int gi = G == 1 ? (int)threadIdx.x / kTileThreads
                          : __builtin_amdgcn_readfirstlane((int)threadIdx.x / kTileThreads);   // uniform per wave
    uint8_t *lds = lds_all + gi * kTileLds;
    int *s_e = (int *)(lds + kLE);
    int *s_bar = (int *)(lds_all + G * kTileLds) + gi;   // this group's barrier counter (G > 1)
    int bar_target = 0;
    if constexpr (G > 1) {
        if (threadIdx.x < G)
            ((int *)(lds_all + G * kTileLds))[threadIdx.x] = 0;
        __syncthreads();
    }

    const int tid = (int)threadIdx.x % kTileThreads;    // thread within the group
    const int lane = tid & 63, w = tid >> 6;
    const int j = lane >> 4, c16 = lane & 15;
    const int n_rows = a.T * a.H;
    // workgroup -> (row block, chunk range); heaviest row blocks first. The
    // fused kernel walks every chunk of its rows (n_parts == 1); the record
    // kernel splits them into ranges of kSplit chunks.
    const int n_rb = (int)gridDim.x / n_parts;
    const int rb = n_rb - 1 - (int)blockIdx.x / n_parts;
    const int part = (int)blockIdx.x % n_parts;
    const int k_lo = kFused ? 0 : part * kSplit;
    const int k_hi = kFused ? a.C : min(a.C, k_lo + kSplit);    // exclusive
    const int row0 = rb * kTileRows;
    const int t_last = (min(n_rows, row0 + kTileRows) - 1) / a.H;   // the block's last token
    const int64_t lim_blk = min((int64_t)a.pos0 + t_last, (int64_t)a.n_cells - 1);
    const int kmax = lim_blk < 0 ? -1 : (int)min((int64_t)a.C - 1, lim_blk / kChunk);
    const int k_end = min(kmax, k_hi - 1);       // last chunk this workgroup walks

    // this lane's row (the MFMA column c16 of its wave)
    const int row = row0 + 16 * w + c16;
    const bool row_ok = row < n_rows;
    const int t = row_ok ? row / a.H : 0;
    const int h = row_ok ? row - t * a.H : 0;
    const int lim = row_ok ? (int)min((int64_t)a.pos0 + t, (int64_t)a.n_cells - 1) : -1;   // last valid cell
    const float kmul = a.scale * kLog2e;        // scores in log2 units
    // -0, from an argument the compiler cannot see through (n_cells >= 0): the
    // first product of each score is an fma with it, which reads the fp16
    // scale directly (x + -0 = x for every x, so it is the product's value),
    // where a constant -0 would be folded back into a multiply
    const float nz = __int_as_float((int)(0x80000000u | (uint32_t)(a.n_cells >> 31)));
    // the wave's smallest last valid cell: lane 0 holds the wave's first row
    // (rows past the end have lim = -1, and a wave whose first row is past
    // the end masks every chunk)
    const int lim_w = __builtin_amdgcn_readfirstlane(lim);

    half8 qop[4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
        qop[g] = row_ok ? *(const half8 *)(a.q + (int64_t)row * kD + 32 * g + 8 * j) : (half8)(_Float16)0.0f;

    Raw R;
    const int n_walk = k_end - k_lo + 1;
    const int n_iter = n_walk > 0 ? (n_walk + G - 1) / G : 0;
    if (k_lo + gi <= k_end)
        load_raw(a, (k_lo + gi) * kChunk, tid, R);

    float Mrun = -INFINITY, Lrun = 0.0f;
    int krun[4] = {0, 0, 0, 0};                 // the powers of two O carries per scale group
    floatx4 O[8];
#pragma unroll
    for (int n = 0; n < 8; ++n)
        O[n] = (floatx4){0.f, 0.f, 0.f, 0.f};

    for (int it = 0; it < n_iter; ++it) {
        const int k = k_lo + gi + it * G;
        const bool act = k <= k_end;            // uniform over the group: groups past the end idle
        const int c0 = k * kChunk;
        // every read issued so far (q, this chunk's rows) has landed: stated
        // here so that the contractions below wait on none of the next
        // chunk's reads, which are issued before them
        __builtin_amdgcn_s_waitcnt(0);
        if (act && c0 + kChunk > a.n_cells)     // uniform: only a chunk that reaches past the cache
            zero_missing(R, c0, a.n_cells, tid);
        if (act) {
            const int eg = group_max_exponent(R);
            if (lane < 4)
                s_e[4 * w + lane] = eg;         // lane l holds scale group l
        }
        group_sync<G>(s_bar, bar_target);       // the previous chunk's tiles are no longer read
        int kg[4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
            kg[g] = group_shift(max(max(s_e[g], s_e[4 + g]), max(s_e[8 + g], s_e[12 + g])));
        if (act)
            stage_tiles(lds, tid, R, kg);
        group_sync<G>(s_bar, bar_target);       // the chunk's tiles are in place
        if (!act)
            continue;
        if (k + G <= k_end) {
            // the next chunk's reads leave ahead of the other waves' compute on
            // this SIMD (records kernel 83.8 -> 80.4 us at the prompt start)
            __builtin_amdgcn_s_setprio(2);
            load_raw(a, c0 + G * kChunk, tid, R);   // in flight during this chunk's contractions
            __builtin_amdgcn_s_setprio(0);
        }

        // ---- QK: S[b][r] is cell 16b + 4j + r of this lane's row, log2 units ---
        float S[4][4];
        if (c0 + kChunk - 1 <= lim_w)           // uniform: every cell counts for every row of the wave
            qk_scores<false>(lds, qop, j, c16, c0, lim, kmul, nz, S);
        else
            qk_scores<true>(lds, qop, j, c16, c0, lim, kmul, nz, S);
        float mx = -INFINITY;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                mx = fmaxf(mx, S[b][r]);
        mx = xor32_max(xor16_max(mx));

        // reference max for p, and (fused) the factor on what came before
        float ref, alpha = 1.0f;
        if constexpr (kFused) {
            const float Mnew = fmaxf(Mrun, mx);
            ref = Mnew == -INFINITY ? 0.0f : Mnew;
            alpha = Mnew == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(Mrun - Mnew);  // 0 when Mrun = -inf
            Mrun = Mnew;
        } else {
            ref = mx == -INFINITY ? 0.0f : mx;
        }
        float P[4][4];
        float lsum = 0.0f;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                P[b][r] = __builtin_amdgcn_exp2f(S[b][r] - ref);    // exp2(-inf) = 0, exp2(0) = 1
                lsum += P[b][r];
            }
        lsum = xor32_sum(xor16_sum(lsum));
        if constexpr (kFused) {
            // what came before: times alpha, and moved to this chunk's powers of two
            Lrun = fmaf(alpha, Lrun, lsum);
            const bool same_k = kg[0] == krun[0] && kg[1] == krun[1] && kg[2] == krun[2] && kg[3] == krun[3];
            if (!same_k || __ballot(alpha != 1.0f) != 0) {   // uniform
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float f = alpha * pow2i(kg[g] - krun[g]);
                    O[2 * g] *= f;
                    O[2 * g + 1] *= f;
                    krun[g] = kg[g];
                }
            }
        } else {
#pragma unroll
            for (int n = 0; n < 8; ++n)
                O[n] = (floatx4){0.f, 0.f, 0.f, 0.f};
        }

        // ---- PV: O[n][r] is dim 16n + 4j + r of this lane's row -----------------
        pv_accumulate(lds, P, j, c16, O);

        if constexpr (!kFused) {
            if (row_ok) {
                const int64_t rec = ((int64_t)t * a.C + k) * a.H + h;
                if (j == 0) {
                    a.m[rec] = mx * kLn2;            // back from log2 units; -inf stays -inf
                    a.l[rec] = mx == -INFINITY ? 0.0f : lsum;
                }
                if (mx != -INFINITY) {          // an empty record leaves o alone
                    float *o = a.o + rec * kD + 4 * j;
#pragma unroll
                    for (int n = 0; n < 8; ++n)
                        *(floatx4 *)(o + 16 * n) = O[n] * pow2i(-kg[n >> 1]);
                }
            }
        }
    }

    if constexpr (kFused) {
        // back to plain units: each scale group's power of two comes out exactly
#pragma unroll
        for (int n = 0; n < 8; ++n)
            O[n] *= pow2i(-krun[n >> 1]);
    }
    if constexpr (kFused && G > 1) {
        // combine the groups: each lane's (M, L, O) has the same row and dims in
        // every group; groups 1.. publish theirs over their own tiles
        __syncthreads();
        // per lane: M, L, two pad words, then O as 8 x 4 floats (16-byte aligned), 144 bytes
        float *mine = (float *)lds + (w * 64 + lane) * 36;
        if (gi > 0) {
            mine[0] = Mrun;
            mine[1] = Lrun;
#pragma unroll
            for (int n = 0; n < 8; ++n)
                *(floatx4 *)(mine + 4 + 4 * n) = O[n];
        }
        __syncthreads();
        if (gi == 0) {
            for (int g2 = 1; g2 < G; ++g2) {
                const float *th = (const float *)(lds_all + g2 * kTileLds) + (w * 64 + lane) * 36;
                const float M2 = th[0], L2 = th[1];
                const float M = fmaxf(Mrun, M2);
                if (M == -INFINITY)
                    continue;                   // neither has seen a valid cell
                const float a1 = __builtin_amdgcn_exp2f(Mrun - M);   // 0 when Mrun = -inf (log2 units)
                const float a2 = __builtin_amdgcn_exp2f(M2 - M);
                Lrun = a1 * Lrun + a2 * L2;
#pragma unroll
                for (int n = 0; n < 8; ++n) {
                    const floatx4 o2 = *(const floatx4 *)(th + 4 + 4 * n);
                    O[n] = a1 * O[n] + a2 * o2;
                }
                Mrun = M;
            }
        }
    }
    if constexpr (kFused) {
        if (gi == 0) {                          // uniform per wave
            // O[n][r] is dim 16n + 4j + r: block n of 16 dims sits in the four
            // lanes c16, c16 + 16, c16 + 32, c16 + 48 (the same row)
            const int64_t obase = (int64_t)(row_ok ? row : 0) * kD + 4 * j;
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                float4 y = make_float4(0.f, 0.f, 0.f, 0.f);   // a row with no valid cell gives +0
                if (Lrun > 0.0f)
                    y = make_float4(O[n][0] / Lrun, O[n][1] / Lrun, O[n][2] / Lrun, O[n][3] / Lrun);
                if (a.gate && row_ok) {         // the gated entry point
                    const float4 g = *(const float4 *)(a.gate + obase + 16 * n);
                    y.x *= sigmoid_gate(g.x);
                    y.y *= sigmoid_gate(g.y);
                    y.z *= sigmoid_gate(g.z);
                    y.w *= sigmoid_gate(g.w);
                }
                const uint2 res = pack_half4(y.x, y.y, y.z, y.w);
                if (row_ok)
                    *(uint2 *)(a.out + obase + 16 * n) = res;
                if (a.sums) {                   // uniform; every lane takes part in the exchanges
                    const double sb = xor_sum(xor_sum(half4_sum(res), 16), 32);
                    if (row_ok && j == 0)
                        a.sums[(int64_t)row * (kD / 16) + n] = (float)sb;
                }
            }
        }
    } else {
        // chunks past the block's last causal cell: empty records for every row
        if (row_ok && j == 0)
            for (int k = max(kmax + 1, k_lo); k < k_hi; ++k) {
                const int64_t rec = ((int64_t)t * a.C + k) * a.H + h;
                a.m[rec] = -INFINITY;
                a.l[rec] = 0.0f;
            }
    }
}

} // namespace

hipError_t launch_attn_tile(const AttnArgs &a, hipStream_t stream)
{
    const int64_t n_rb = ((int64_t)a.T * a.H + kTileRows - 1) / kTileRows;
    const int n_parts = (a.C + kSplit - 1) / kSplit;
    hipLaunchKernelGGL((attn_tile_kernel<false, 1>), dim3((unsigned)(n_rb * n_parts)), dim3(kTileThreads), 0, stream,
                       a, n_parts);
    return hipGetLastError();
}

hipError_t launch_attn_merge_tile(const AttnArgs &a, hipStream_t stream)
{
    const int64_t n_rb = ((int64_t)a.T * a.H + kTileRows - 1) / kTileRows;
    hipLaunchKernelGGL((attn_tile_kernel<true, kFusedGroups>), dim3((unsigned)n_rb), dim3(kTileThreads * kFusedGroups),
                       0, stream, a, 1);
    return hipGetLastError();
}

} // namespace qsa
