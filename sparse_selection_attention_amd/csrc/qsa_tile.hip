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
// Design on CDNA4. A workgroup of four waves owns 64 consecutive rows, 16 per
// wave, and walks the chunks up to its last token's causal edge:
//   * staging, once per chunk for all four waves: half the threads read the
//     chunk's 64 K rows and write them to LDS as fp16 (exact), the other half
//     read the V rows and write V transposed (dims x cells) as fp16 high and
//     low parts with V_hi + V_lo = vq * vsc exactly, cells permuted so that
//     each PV operand read is one 16-byte load; both tiles are XOR-swizzled in
//     16-byte granules for conflict-free operand reads;
//   * QK: v_mfma_f32_16x16x32_f16 with A = 16 cells x 32 dims of one scale
//     group and B = the wave's 16 q rows, one fp32 partial per scale group,
//     weighted by the cell's group scale; a lane then holds 16 of its row's
//     64 scores, so the row max and sum are lane folds plus two exchanges;
//   * causality is a per-row mask: cell c counts for row r iff
//     c <= pos0 + r / H (and c < n_cells);
//   * PV: O^T = V^T P^T on the same MFMA, A = V^T from LDS, B = p straight
//     from the score registers, both split into fp16 high and low parts and
//     contracted as hi*hi + hi*lo + lo*hi (about 22 bits per product);
//   * chunk records (qsa_attn): one (m, l, o) per row and chunk, rows past
//     their causal edge writing the empty record (-inf, 0); the chunks of a
//     row block are split over workgroups of at most 8 chunks each, so the
//     long rows of late tokens do not serialise; fused
//     (qsa_attn_merge): a running max, denominator and output per row,
//     rescaled as each chunk's max arrives, divided once at the end. A fused
//     workgroup holds three such groups of four waves, each with its own LDS
//     tiles, walking every third chunk of the same rows; their states are
//     combined through LDS at the end (the same max-first rule), so the
//     longest row block walks a third as many chunks in sequence.
// The gated entry point multiplies each fused output by sigmoid(g) of its fp32
// gate before the fp16 rounding and may write the exact per-16 sums of the
// written values ("round 5 track b: cached residual norms and fused mtp
// attention", section "preflight / ownership").
// In a chunk whose largest V scale reaches 2^9 (vq * vsc could leave fp16
// range) the V codes are converted as vq * 2^-k, exactly and at no cost, and
// 2^k is taken back out exactly on p; the scales are never rounded. Workgroups start with the heaviest row blocks (the last
// tokens, with the most chunks).
#include "qsa_internal.h"
#include "qsa_device.h"

namespace qsa {
namespace {

using namespace dev;

constexpr int kTileRows = 64;                  // (token, head) rows per workgroup
constexpr int kTileThreads = 256;

// LDS layout
constexpr int kLK = 0;                         // K fp16 [64 cells][128 dims], 256-byte rows
constexpr int kLVh = kLK + kChunk * kD * 2;    // V^T hi fp16 [128 dims][64 positions], 128-byte rows
constexpr int kLVl = kLVh + kD * kChunk * 2;   // V^T lo
constexpr int kLKs = kLVl + kD * kChunk * 2;   // K scales fp16 [64 cells][4]
constexpr int kLE = kLKs + kChunk * 8;         // int[4]: largest V-scale exponent seen by each wave
constexpr int kTileLds = kLE + 16;
constexpr int kSplit = 8;                      // chunks per workgroup in the chunk-record kernel
constexpr int kFusedGroups = 3;                // groups of four waves per fused workgroup
static_assert(kTileLds % 16 == 0 && 4 * 64 * 36 * 4 <= kTileLds, "group state must fit a group's tiles");

// K tile: cell c's logical granule gi (dims 8gi .. 8gi+7) at gi ^ (c & 15)
__device__ inline int tk_offset(int c, int gi) { return kLK + c * 256 + ((gi ^ (c & 15)) << 4); }
// V^T tiles: dim d's logical granule gp (positions 8gp .. 8gp+7) at gp ^ ((d >> 1) & 7)
__device__ inline int tv_offset(int base, int d, int gp) { return base + d * 128 + ((gp ^ ((d >> 1) & 7)) << 4); }

// Position pos = 32ks + 8j + s of a 64-cell chunk holds cell 32ks + 16(s/4) + 4j + s%4:
// the cells whose scores lane group j holds, in PV operand slot order.
__device__ inline int pos_cell(int ks, int j, int s) { return 32 * ks + 16 * (s >> 2) + 4 * j + (s & 3); }

// Every thread stages 32 bytes of K and 32 bytes of V per chunk:
//   K: cell kc = tid / 4, dims 32 kg .. +31 (kg = tid % 4, one scale group);
//   V: dims 8 db .. +7 (db = tid / 16) of positions 4 pq .. 4 pq + 3
//      (pq = tid % 16), which are four consecutive cells.
struct Raw {
    uint4 k[2];        // K: 32 bytes of cell kc
    uint32_t ks;       // K: that cell's scale of group kg (fp16 bits)
    uint2 v[4];        // V: 8 dims of 4 cells
    uint32_t vs[4];    // V: the 4 cells' scales of dim group db / 4 (fp16 bits)
    uint32_t ok;       // bit 0: cell kc exists; bits 1..4: the V cells exist
};

__device__ inline int v_cell0(int pq) { return 32 * (pq >> 3) + 16 * (pq & 1) + 4 * ((pq >> 1) & 3); }

// Issue the chunk's global reads into registers. Every read is unconditional
// (cells past the cache read the last cached row) so that the reads stay in
// flight; the cells that do not exist are zeroed when the tiles are staged.
// Byte offsets fit 32 bits: n_cells * 128 < 2^32.
__device__ inline void load_raw(const AttnArgs &a, int c0, int tid, Raw &R)
{
    const int last = a.n_cells - 1;     // >= 0 whenever a chunk is walked
    const int kc = tid >> 2, kg = tid & 3;
    const int ck = c0 + kc;
    uint32_t ok = ck <= last ? 1u : 0u;
    const uint32_t kcc = (uint32_t)min(ck, last);
    const uint4 *src = (const uint4 *)(a.kq + (kcc * kD + 32 * kg));
    R.k[0] = src[0];
    R.k[1] = src[1];
    R.ks = a.ksc[kcc * 4 + kg];
    const int db = tid >> 4, pq = tid & 15;
    const int cv = c0 + v_cell0(pq);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        ok |= (cv + s <= last ? 1u : 0u) << (1 + s);
        const uint32_t vcc = (uint32_t)min(cv + s, last);
        R.v[s] = *(const uint2 *)(a.vq + (vcc * kD + 8 * db));
        R.vs[s] = a.vsc[vcc * 4 + (db >> 2)];
    }
    R.ok = ok;
}

// Largest biased V-scale exponent over this thread's existing V cells.
__device__ inline uint32_t vs_exponent(const Raw &R)
{
    uint32_t e = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s)
        e = max(e, ((R.ok >> (1 + s)) & 1u) ? (R.vs[s] >> 10) & 31u : 0u);
    return e;
}

// The same maximum over the wave, bit by bit with ballots (uniform result).
__device__ inline uint32_t wave_max_exponent(uint32_t ev)
{
    uint32_t e = 0;
#pragma unroll
    for (int bit = 4; bit >= 0; --bit) {
        const uint32_t c = e | (1u << bit);
        if (__ballot(ev >= c) != 0)
            e = c;
    }
    return e;
}

// Convert the chunk's raw rows into the LDS tiles. `e` is the chunk's largest
// biased V-scale exponent.
__device__ inline void stage_tiles(uint8_t *lds, int tid, const Raw &R, uint32_t e)
{
    // K: 32 dims of cell kc as fp16 (exact), and its group scale
    const int kc = tid >> 2, kg = tid & 3;
    const bool okk = (R.ok & 1u) != 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint4 kr = okk ? R.k[i] : make_uint4(0u, 0u, 0u, 0u);
        *(half8 *)(lds + tk_offset(kc, 4 * kg + 2 * i)) = i8x8_to_half8(make_uint2(kr.x, kr.y));
        *(half8 *)(lds + tk_offset(kc, 4 * kg + 2 * i + 1)) = i8x8_to_half8(make_uint2(kr.z, kr.w));
    }
    *(uint16_t *)(lds + kLKs + kc * 8 + 2 * kg) = okk ? (uint16_t)R.ks : (uint16_t)0;

    // V: dims 8db .. +7 of positions 4pq .. +3 as fp16 hi + lo, transposed
    const int db = tid >> 4, pq = tid & 15;
    uint2 v[4];
    uint32_t sb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const bool ok = ((R.ok >> (1 + s)) & 1u) != 0;
        v[s] = ok ? R.v[s] : make_uint2(0u, 0u);
        sb[s] = ok ? R.vs[s] : 0u;
    }
    const half2v sc[2] = {__builtin_bit_cast(half2v, sb[0] | (sb[1] << 16)),
                          __builtin_bit_cast(half2v, sb[2] | (sb[3] << 16))};
    // |vq| <= 127: no overflow below a scale of 2^9; above it the codes are
    // converted as vq * 2^-k, k = e - 23 <= 7 (exact), so |V| < 65024, and p
    // carries 2^k. V_lo is the residual of the fp16 product from one fp16
    // fma: exact, or (with the 2^-k) rounded by at most 2^-25 of the scaled value
    const I8Scale cv = i8_scale(e >= 24 ? (int)e - 23 : 0);
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
        uint32_t vh[2], vl[2];
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            const uint2 x = v[2 * sp], y = v[2 * sp + 1];
            const uint32_t xs = dd < 4 ? x.x : x.y, ys = dd < 4 ? y.x : y.y;
            const half2v vi = __builtin_bit_cast(half2v, cvt2_sel(dd & 3, xs, ys, cv));
            const half2v hi = vi * sc[sp];                                   // round to nearest
            const half2v lo = __builtin_elementwise_fma(vi, sc[sp], -hi);    // residual, one rounding
            vh[sp] = __builtin_bit_cast(uint32_t, hi);
            vl[sp] = __builtin_bit_cast(uint32_t, lo);
        }
        const int d = 8 * db + dd;
        const int half = 8 * (pq & 1);
        *(uint2 *)(lds + tv_offset(kLVh, d, pq >> 1) + half) = make_uint2(vh[0], vh[1]);
        *(uint2 *)(lds + tv_offset(kLVl, d, pq >> 1) + half) = make_uint2(vl[0], vl[1]);
    }
}

// G groups of four waves share a workgroup's rows: group gi walks chunks
// k_lo + gi, k_lo + gi + G, ... with LDS tiles of its own, and the groups'
// running (max, denominator, output) are combined at the end (fused kernel).
template <bool kFused, int G>
__global__ __launch_bounds__(kTileThreads * G) void attn_tile_kernel(AttnArgs a, int n_parts)
{
    __shared__ __align__(16) uint8_t lds_all[G * kTileLds];
    const int gi = (int)threadIdx.x / kTileThreads;
    uint8_t *lds = lds_all + gi * kTileLds;
    int *s_e = (int *)(lds + kLE);

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
        if (act) {
            const uint32_t ew = wave_max_exponent(vs_exponent(R));
            if (lane == 0)
                s_e[w] = (int)ew;
        }
        __syncthreads();                        // the previous chunk's tiles are no longer read
        const uint32_t e = (uint32_t)max(max(s_e[0], s_e[1]), max(s_e[2], s_e[3]));
        if (act)
            stage_tiles(lds, tid, R, e);
        __syncthreads();                        // the chunk's tiles are in place
        if (!act)
            continue;
        if (k + G <= k_end)
            load_raw(a, c0 + G * kChunk, tid, R);   // in flight during this chunk's contractions

        // ---- QK: S[b][r] is cell 16b + 4j + r of this lane's row ----------------
        float S[4][4];
        const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            floatx4 acc[4];
            const int ca = 16 * b + c16;        // A operand row: cell ca, dims 32g + 8j .. +7
#pragma unroll
            for (int g = 0; g < 4; ++g)
                acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(*(const half8 *)(lds + tk_offset(ca, 4 * g + j)),
                                                                qop[g], zero, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int cell = 16 * b + 4 * j + r;
                const uint2 kb = *(const uint2 *)(lds + kLKs + cell * 8);
                float dot = acc[0][r] * half_bits_to_float(kb.x & 0xffffu);
                dot = __builtin_fmaf(acc[1][r], half_bits_to_float(kb.x >> 16), dot);
                dot = __builtin_fmaf(acc[2][r], half_bits_to_float(kb.y & 0xffffu), dot);
                dot = __builtin_fmaf(acc[3][r], half_bits_to_float(kb.y >> 16), dot);
                const float sv = a.scale * dot;
                S[b][r] = c0 + cell <= lim ? sv : -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                mx = fmaxf(mx, S[b][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));

        // reference max for p, and (fused) the factor on what came before
        float ref, alpha = 1.0f;
        if constexpr (kFused) {
            const float Mnew = fmaxf(Mrun, mx);
            ref = Mnew == -INFINITY ? 0.0f : Mnew;
            alpha = Mnew == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f((Mrun - Mnew) * kLog2e);  // 0 when Mrun = -inf
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
                P[b][r] = __builtin_amdgcn_exp2f((S[b][r] - ref) * kLog2e);    // exp(-inf) = 0, exp(0) = 1
                lsum += P[b][r];
            }
        lsum += __shfl_xor(lsum, 16, 64);
        lsum += __shfl_xor(lsum, 32, 64);
        if constexpr (kFused) {
            Lrun = fmaf(alpha, Lrun, lsum);
#pragma unroll
            for (int n = 0; n < 8; ++n)
                O[n] *= alpha;
        } else {
#pragma unroll
            for (int n = 0; n < 8; ++n)
                O[n] = zero;
        }
        if (e >= 24) {                          // V carries 2^-(e - 23): put 2^(e - 23) on p
            const float down = __int_as_float((127 - 23 + (int)e) << 23);
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    P[b][r] *= down;
        }

        // ---- PV: O[n][r] is dim 16n + 4j + r of this lane's row -----------------
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            half8 pb_hi, pb_lo;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const float pv = P[2 * ks + (s >> 2)][s & 3];
                const _Float16 hi = (_Float16)pv;
                pb_hi[s] = hi;
                pb_lo[s] = (_Float16)(pv - (float)hi);
            }
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                const int d = 16 * n + c16;     // A operand row: dim d, positions 32ks + 8j .. +7
                const half8 va_hi = *(const half8 *)(lds + tv_offset(kLVh, d, 4 * ks + j));
                const half8 va_lo = *(const half8 *)(lds + tv_offset(kLVl, d, 4 * ks + j));
                O[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va_hi, pb_hi, O[n], 0, 0, 0);
                O[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va_hi, pb_lo, O[n], 0, 0, 0);
                O[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va_lo, pb_hi, O[n], 0, 0, 0);
            }
        }

        if constexpr (!kFused) {
            if (row_ok) {
                const int64_t rec = ((int64_t)t * a.C + k) * a.H + h;
                if (j == 0) {
                    a.m[rec] = mx;
                    a.l[rec] = mx == -INFINITY ? 0.0f : lsum;
                }
                if (mx != -INFINITY) {          // an empty record leaves o alone
                    float *o = a.o + rec * kD + 4 * j;
#pragma unroll
                    for (int n = 0; n < 8; ++n)
                        *(floatx4 *)(o + 16 * n) = O[n];
                }
            }
        }
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
                const float a1 = __builtin_amdgcn_exp2f((Mrun - M) * kLog2e);   // 0 when Mrun = -inf
                const float a2 = __builtin_amdgcn_exp2f((M2 - M) * kLog2e);
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
