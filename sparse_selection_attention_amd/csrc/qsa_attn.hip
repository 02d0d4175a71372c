// qsa_attn.hip -- chunk records of explicit-selection attention on gfx950.
//
// What is computed follows "round 11 track b: qsa attention and score",
// section "implementation and evaluator" (int8 K/V rows gathered by selected
// cell id, one scale per quarter of a K row, a last chunk that may be partly
// filled, empty slots that add nothing) and "round 5 track b: cached residual
// norms and fused mtp attention", section "mtp attention" (a max, a
// denominator and a partial output per chunk; each V value read once per cell
// for all heads).
//
// Design on CDNA4. For the chunk records, one 64-lane wave is one workgroup and
// owns one chunk of one query token; the fused dispatch gives a token one
// workgroup whose waves sweep its chunks. Per chunk:
//   * lane c reads slot c's id; a ballot gives the chunk's valid mask;
//   * the 64 cells' K and V rows are read once for all heads: MFMA tiles put the
//     heads (up to 16) on one tile dimension and the cells on the other;
//   * gathers are shaped for the texture unit, whose cost grows with the number
//     of distinct rows each group of four lanes touches: K rows are copied into
//     LDS with direct-to-LDS loads of 16 bytes per lane, eight lanes per row,
//     and read back in MFMA operand order; V rows are read four full rows per
//     instruction straight into the PV operand registers; a records wave reads
//     its q operands straight from memory (a token's 3 KB of q stay in L2 for
//     all its chunks), the fused workgroup copies q into LDS once for its waves;
//   * the K tile and the q rows are XOR-swizzled in 16-byte granules so that
//     the operand reads hit distinct LDS banks;
//   * QK: v_mfma_f32_16x16x32_f16 with A = K rows (16 cells x 32 dims of one
//     scale group, int8 converted exactly to fp16) and B = q (32 dims x 16
//     heads), giving one fp32 partial per scale group that is then weighted by
//     the cell's group scale, as the pages build the score from partials;
//   * the chunk max and denominator are lane-local folds plus two cross-row
//     exchanges, because the score tile already holds one head per lane column;
//     the exchanges are gfx950's row-swap permutes, which stay in the VALU;
//   * PV: v_mfma_f32_16x16x32_f16 with A = p (heads x 32 cells) straight from
//     the score tile's registers, and B = V rows dequantised to fp16 (the fused
//     kernel swaps the two, so that each lane accumulates its own head's dims). Both sides
//     are split into fp16 high and low parts and contracted as
//     hi*hi + hi*lo + lo*hi, so the products carry about 22 bits:
//       - vq * vsc has at most 18 significant bits, so V = V_hi + V_lo exactly,
//         with V_lo formed by one fp16 fma. When a chunk's largest V scale
//         reaches 2^9 (so vq * vsc could leave fp16 range), the codes are
//         converted as vq * 2^-k (exact, and free: the byte goes under a
//         smaller fp16 exponent), which brings every |V| below 65024, and 2^k
//         is taken back out of the fp32 result; the scales are never rounded;
//       - p = P_hi + P_lo to within 2^-22 relative;
//     a single fp16 rounding of p and of v would cost up to 2^-12 |v| per
//     term, which is too coarse when a chunk holds a few cells whose values
//     nearly cancel;
//   * int8 bytes become fp16 exactly through a byte permute under a 1024.0
//     exponent and one packed subtraction, all visible to the compiler.
// Record waves are ordered by chunk first (all tokens of chunk 0, then chunk
// 1, ...) and each XCD walks a contiguous range of them, so the cells one XCD
// gathers stay within a narrow band of the cache, served from its L2. A record
// is written in whole 1 KB runs, nontemporal when the call's records are too
// large to stay cached until the merge, so that they do not evict that band.
#include "qsa_internal.h"
#include "qsa_device.h"

namespace qsa {
namespace {

using namespace dev;

constexpr int kWaves = kAttnWaves;         // waves of a fused workgroup over many chunks in a large call
constexpr int kWavesMax = 8;               // over few chunks (one wave each), or many chunks in a small call

// LDS layout: one wave region per wave, then (fused workgroup only) the q rows
constexpr int kKTileBytes = kChunk * kD;                 // 8 KB of K rows per wave
constexpr int kWaveBytes = kKTileBytes + kChunk * 8      // K tile, K scales (fp16 x 4)
                           + kChunk * 8 + kChunk * 4     // V scales (group-major), cell ids
                           + kChunk * 4;                 // score penalties
// (gated calls only) then the token's fp32 gate rows
constexpr int attn_lds_bytes(int nw, int H, bool gated) { return nw * kWaveBytes + H * kD * 2 + (gated ? H * kD * 4 : 0); }

typedef __attribute__((address_space(3))) void lds_void;

// cache-policy operand of the buffer store builtins: the nontemporal bit
constexpr int kCachePolicyNT = 2;

// K tile: row r (a cell of the chunk) holds 8 granules of 16 bytes; logical
// granule lg sits at physical granule lg ^ ((r >> 1) & 7). Rows of equal parity
// then spread over all eight granule positions, so the sixteen rows read by one
// MFMA operand load fall on distinct banks.
__device__ inline int ktile_offset(int row, int lg) { return row * kD + ((lg ^ ((row >> 1) & 7)) << 4); }

// q rows: head h holds 16 granules; logical granule lg sits at lg ^ (h & 15).
__device__ inline int qrow_offset(int h, int lg) { return h * (kD * 2) + ((lg ^ (h & 15)) << 4); }

// ---- per-wave LDS regions ----------------------------------------------------

struct WaveLds {
    uint8_t *ktile;      // [64 rows][128 B], swizzled granules
    uint2 *ksc;          // [64] cells x 4 fp16 K scales
    uint16_t *vsc;       // [4 groups][64 cells] fp16 V scales
    int32_t *id;         // [64] cell ids (0 for empty slots)
    float *pen;          // [64] added to the scaled score: -0 for a valid slot, -inf for an empty one
};

__device__ inline WaveLds wave_lds(uint8_t *lds, int w)
{
    uint8_t *base = lds + w * kWaveBytes;
    return WaveLds{base, (uint2 *)(base + kKTileBytes), (uint16_t *)(base + kKTileBytes + kChunk * 8),
                   (int32_t *)(base + kKTileBytes + kChunk * 16), (float *)(base + kKTileBytes + kChunk * 20)};
}

// The token's q rows (H x 256 B) into LDS: 16-byte granules, head h's logical
// granule lg at lg ^ (h & 15). Waves 0..nw-1 share the copy, 1 KB per load.
__device__ inline void copy_q_rows(const AttnArgs &a, uint8_t *qrows, int t, int w, int nw, int lane)
{
    for (int g0 = 64 * w; g0 < 16 * a.H; g0 += 64 * nw) {
        const int gi = g0 + lane;                // destination granule
        const int h = gi >> 4, phys = gi & 15;
        if (h < a.H) {
            const int lg = phys ^ (h & 15);
            const _Float16 *src = a.q + ((int64_t)t * a.H + h) * kD + 8 * lg;
            __builtin_amdgcn_global_load_lds((const void *)src, (lds_void *)(qrows + 16 * g0), 16, 0, 0);
        }
    }
}

// The token's fp32 gate rows (H x 512 B, in memory order) into LDS, 1 KB per
// load, shared by waves 0..nw-1. Issued once the q rows have landed, so they
// complete under the first chunk's gathers instead of at the end.
__device__ inline void copy_gate_rows(const AttnArgs &a, uint8_t *grows, int t, int w, int nw, int lane)
{
    for (int g0 = 64 * w; g0 < 32 * a.H; g0 += 64 * nw) {
        const int gi = g0 + lane;                // destination granule: head gi / 32, dims 4 (gi % 32) ..
        if (gi < 32 * a.H) {
            const float *src = a.gate + (int64_t)t * a.H * kD + 4 * gi;
            __builtin_amdgcn_global_load_lds((const void *)src, (lds_void *)(grows + 16 * g0), 16, 0, 0);
        }
    }
}

// q operand of QK: head c16, dims 32g + 8j .. +7 (zero for padding heads)
__device__ inline void q_operand(const AttnArgs &a, const uint8_t *qrows, int j, int c16, half8 (&qop)[4])
{
#pragma unroll
    for (int g = 0; g < 4; ++g)
        qop[g] = c16 < a.H ? *(const half8 *)(qrows + qrow_offset(c16, 4 * g + j)) : (half8)(_Float16)0.0f;
}

// Chunk k of token t: read the ids, publish them, and issue every gather of the
// chunk (K rows into the wave's LDS tile, V rows and scales into registers).
// Returns the ballot of valid slots; nothing is issued for an empty chunk.
// Slot `lane` of chunk k of token t: its cell id, -1 or out of range for an
// empty slot.
__device__ inline int32_t slot_id(const AttnArgs &a, int t, int k, int lane)
{
    const int64_t slot = (int64_t)k * kChunk + lane;
    if (a.ids)
        return a.ids[(int64_t)t * a.ids_stride + slot];
    return slot <= (int64_t)a.pos0 + t ? (int32_t)slot : -1;
}

__device__ inline uint64_t issue_chunk(const AttnArgs &a, const WaveLds &L, int32_t id, int lane, int j, int c16,
                                       uint2 &ks, uint2 &vs, uint2 (&vraw)[2][8])
{
    const bool valid = (uint32_t)id < (uint32_t)a.n_cells;
    const int32_t sid = valid ? id : 0;
    const uint64_t mask = __ballot(valid);

    L.id[lane] = sid;
    L.pen[lane] = valid ? -0.0f : -INFINITY;
    wave_sync_lds();
    ks = make_uint2(0u, 0u);
    vs = make_uint2(0u, 0u);
    if (mask != 0) {
        if (valid) {
            ks = *(const uint2 *)(a.ksc + (int64_t)sid * 4);
            vs = *(const uint2 *)(a.vsc + (int64_t)sid * 4);
        }
        // K rows into the tile: instruction s writes granules 64s .. 64s+63,
        // i.e. rows 8s .. 8s+7, eight lanes per row. All eight row ids are
        // read first: an LDS read placed after a direct-to-LDS copy waits for
        // it (the compiler cannot tell that they touch different LDS), which
        // would put an LDS round trip between consecutive copies.
        uint32_t koff[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int row = 8 * s + (lane >> 3);
            const int lg = (lane & 7) ^ ((row >> 1) & 7);
            koff[s] = (uint32_t)L.id[row] * kD + 16 * lg;   // n_cells * 128 < 2^32
        }
#pragma unroll
        for (int s = 0; s < 8; ++s)
            __builtin_amdgcn_global_load_lds((const void *)(a.kq + koff[s]), (lds_void *)(L.ktile + 1024 * s), 16, 0, 0);
        // V: slot s of k-step ks is cell 32ks + 16(s/4) + 4j + s%4 -- the cells
        // whose scores this lane holds -- and the lane reads dims 8*c16 .. +7
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int cell = 32 * ks2 + 16 * (s >> 2) + 4 * j + (s & 3);
                vraw[ks2][s] = *(const uint2 *)(a.vq + ((uint32_t)L.id[cell] * kD + 8 * c16));
            }
    }
    return mask;
}

// The two halves of issue_chunk, for a wave that issues the next chunk's
// reads while it still computes the current one. issue_k publishes the ids and
// penalties, reads the scales and copies the K rows into the tile (the tile
// must no longer be read); issue_v reads the V rows of the ids issue_k
// published into the PV operand registers (which must no longer be read).
__device__ inline uint64_t issue_k(const AttnArgs &a, const WaveLds &L, int32_t id, int lane, uint2 &ks, uint2 &vs)
{
    const bool valid = (uint32_t)id < (uint32_t)a.n_cells;
    const int32_t sid = valid ? id : 0;
    const uint64_t mask = __ballot(valid);
    L.id[lane] = sid;
    L.pen[lane] = valid ? -0.0f : -INFINITY;
    wave_sync_lds();
    ks = make_uint2(0u, 0u);
    vs = make_uint2(0u, 0u);
    if (mask != 0) {
        if (valid) {
            ks = *(const uint2 *)(a.ksc + (int64_t)sid * 4);
            vs = *(const uint2 *)(a.vsc + (int64_t)sid * 4);
        }
        uint32_t koff[8];                        // all ids first, as in issue_chunk
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int row = 8 * s + (lane >> 3);
            const int lg = (lane & 7) ^ ((row >> 1) & 7);
            koff[s] = (uint32_t)L.id[row] * kD + 16 * lg;
        }
#pragma unroll
        for (int s = 0; s < 8; ++s)
            __builtin_amdgcn_global_load_lds((const void *)(a.kq + koff[s]), (lds_void *)(L.ktile + 1024 * s), 16, 0, 0);
    }
    return mask;
}

__device__ inline void issue_v(const AttnArgs &a, const WaveLds &L, uint64_t mask, int j, int c16, uint2 (&vraw)[2][8])
{
    if (mask != 0) {
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int cell = 32 * ks2 + 16 * (s >> 2) + 4 * j + (s & 3);
                vraw[ks2][s] = *(const uint2 *)(a.vq + ((uint32_t)L.id[cell] * kD + 8 * c16));
            }
    }
}

// Publish the chunk's scales to LDS. When vq * vsc could leave fp16 range (the
// chunk's largest V scale reaches 2^9), the V codes are converted as
// vq * 2^-k, k = e - 23 (e the largest biased V-scale exponent, so k <= 7),
// and the exact factor 2^k must be put back on the result. Returns k (0 when
// no factor is needed), uniform over the wave.
__device__ inline int stage_scales(const WaveLds &L, int lane, uint2 ks, uint2 vs)
{
    const uint32_t ev = max(max((vs.x >> 10) & 31u, (vs.x >> 26) & 31u),
                            max((vs.y >> 10) & 31u, (vs.y >> 26) & 31u));
    uint32_t e = 0;                 // largest biased exponent in the chunk, bit by bit
#pragma unroll
    for (int bit = 4; bit >= 0; --bit) {
        const uint32_t c = e | (1u << bit);
        if (__ballot(ev >= c) != 0)
            e = c;
    }
    L.ksc[lane] = ks;
    L.vsc[0 * kChunk + lane] = (uint16_t)(vs.x & 0xffffu);
    L.vsc[1 * kChunk + lane] = (uint16_t)(vs.x >> 16);
    L.vsc[2 * kChunk + lane] = (uint16_t)(vs.y & 0xffffu);
    L.vsc[3 * kChunk + lane] = (uint16_t)(vs.y >> 16);
    wave_sync_lds();
    // |vq| <= 127 and vsc < 2^(e - 14): no overflow below vsc = 2^9; above,
    // |vq * 2^-k * vsc| < 127 * 2^9 = 65024
    return e >= 24 ? (int)e - 23 : 0;
}

// 2^k as a float, for 0 <= k <= 7
__device__ inline float pow2f(int k) { return __int_as_float((127 + k) << 23); }

// -0, from an argument the compiler cannot see through (n_cells >= 0). The
// first product of each score is an fma with it, which reads the fp16 scale
// directly (x + -0 = x for every x, so it is the product's value), where a
// constant -0 would be folded back into a multiply.
__device__ inline float opaque_neg_zero(const AttnArgs &a)
{
    return __int_as_float((int)(0x80000000u | (uint32_t)(a.n_cells >> 31)));
}

// Scaled scores of the chunk, kscale times the dot products: the softmax scale
// (the records kernel, whose maxima are written), or the softmax scale times
// log2(e) (the fused kernel, which keeps scores in log2 units so that
// p = exp2(S - max) needs no multiply). S[b][r] is cell 16b + 4j + r, head
// c16. The slot's penalty is the addend of the scaling fma: + -0 leaves the product as
// it is (signed zeros included), + -inf makes an empty slot's score -inf (its
// product is finite: the slot reads row 0 with zero scales).
__device__ inline void chunk_scores(float kscale, float nz, const WaveLds &L, const half8 (&qop)[4], int j, int c16,
                                    float (&S)[4][4])
{
    const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        // A operand: cell 16b + c16, dims 32g + 8j .. +7 = bytes 16(2g + j/2) + 8(j&1)
        floatx4 acc[4];
        const int row = 16 * b + c16;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint2 kr = *(const uint2 *)(L.ktile + ktile_offset(row, 2 * g + (j >> 1)) + 8 * (j & 1));
            acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(i8x8_to_half8(kr), qop[g], zero, 0, 0, 0);
        }
        const float4 p4 = *(const float4 *)(L.pen + 16 * b + 4 * j);   // cells 16b + 4j .. +3
        const float pen[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int cell = 16 * b + 4 * j + r;
            const uint2 kb = L.ksc[cell];
            float dot = __builtin_fmaf(acc[0][r], half_bits_to_float(kb.x & 0xffffu), nz);
            dot = __builtin_fmaf(acc[1][r], half_bits_to_float(kb.x >> 16), dot);
            dot = __builtin_fmaf(acc[2][r], half_bits_to_float(kb.y & 0xffffu), dot);
            dot = __builtin_fmaf(acc[3][r], half_bits_to_float(kb.y >> 16), dot);
            S[b][r] = __builtin_fmaf(kscale, dot, pen[r]);
        }
    }
}

// Max over the chunk's cells for head c16 (the same value in all four rows j).
__device__ inline float chunk_max(const float (&S)[4][4])
{
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            mx = fmaxf(mx, S[b][r]);
    return xor32_max(xor16_max(mx));
}

// p = exp(S - ref) for head c16, and their sum over the chunk; with kLog2Units
// the scores are in log2 units and p = exp2(S - ref).
template <bool kLog2Units>
__device__ inline float chunk_probs(const float (&S)[4][4], float ref, float (&P)[4][4])
{
    float lsum = 0.0f;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            P[b][r] = __builtin_amdgcn_exp2f(kLog2Units ? S[b][r] - ref : (S[b][r] - ref) * kLog2e);  // exp(0) = 1 exactly
            lsum += P[b][r];
        }
    return xor32_sum(xor16_sum(lsum));
}

// O[tt] += p V over the chunk: O[tt][r] is head 4j + r, dim 8*c16 + tt, or
// with kByHead (the operands' roles swapped, so that the MFMA produces O^T) head
// c16, dim 8*(4j + r) + tt: every value a lane holds then belongs to its own
// head c16. The V
// codes are converted times 2^-k_renorm (see stage_scales); V_hi is
// the fp16 product with the scale and V_lo its exact residual from one fp16
// fma (the product has at most 18 significant bits; when it is scaled by 2^-k
// its lowest bits may fall below the fp16 grid, and V_lo then rounds by at
// most 2^-25, i.e. 2^(k - 25) <= 2^-18 of the unscaled value).
template <bool kByHead>
__device__ inline void pv_accumulate(const float (&P)[4][4], const uint2 (&vraw)[2][8], const WaveLds &L, int j,
                                     int c16, int k_renorm, floatx4 (&O)[8])
{
    // the two conversion words are wave-uniform; stating that they live in
    // scalar registers keeps the scheduler from holding more vector values
    // live in the records kernel (129 VGPRs, three waves per SIMD, without
    // it; 128 and four with it)
    I8Scale cv = i8_scale(k_renorm);
    asm volatile("" : "+s"(cv.xr), "+s"(cv.bias));
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
        // A operand: p of slots s = cells 32ks + 16(s/4) + 4j + s%4, as hi + lo
        float pv[8];
#pragma unroll
        for (int s = 0; s < 8; ++s)
            pv[s] = P[2 * ks2 + (s >> 2)][s & 3];
        half8 pa_hi, pa_lo;
        split_half8(pv, pa_hi, pa_lo);
        // V scales of the slot pairs (s, s+1): adjacent cells, one dword each
        half2v sc[4];
#pragma unroll
        for (int sp = 0; sp < 4; ++sp) {
            const int cell = 32 * ks2 + 16 * (sp >> 1) + 4 * j + 2 * (sp & 1);
            sc[sp] = __builtin_bit_cast(half2v, *(const uint32_t *)&L.vsc[(c16 >> 2) * kChunk + cell]);
        }
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
            uint32_t vh[4], vl[4];
#pragma unroll
            for (int sp = 0; sp < 4; ++sp) {
                const uint2 x = vraw[ks2][2 * sp], y = vraw[ks2][2 * sp + 1];
                const uint32_t xs = tt < 4 ? x.x : x.y, ys = tt < 4 ? y.x : y.y;
                const half2v vi = __builtin_bit_cast(half2v, cvt2_sel(tt & 3, xs, ys, cv));
                const half2v hi = vi * sc[sp];                              // round to nearest
                const half2v lo = __builtin_elementwise_fma(vi, sc[sp], -hi); // residual, one rounding
                vh[sp] = __builtin_bit_cast(uint32_t, hi);
                vl[sp] = __builtin_bit_cast(uint32_t, lo);
            }
            const half8 vb_hi = __builtin_bit_cast(half8, make_uint4(vh[0], vh[1], vh[2], vh[3]));
            const half8 vb_lo = __builtin_bit_cast(half8, make_uint4(vl[0], vl[1], vl[2], vl[3]));
            if constexpr (kByHead) {
                O[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vb_hi, pa_hi, O[tt], 0, 0, 0);
                O[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vb_lo, pa_hi, O[tt], 0, 0, 0);
                O[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vb_hi, pa_lo, O[tt], 0, 0, 0);
            } else {
                O[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa_hi, vb_hi, O[tt], 0, 0, 0);
                O[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa_hi, vb_lo, O[tt], 0, 0, 0);
                O[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa_lo, vb_hi, O[tt], 0, 0, 0);
            }
        }
    }
}

// ---- chunk records (qsa_attn) ---------------------------------------------

__global__ __launch_bounds__(64) void attn_kernel(AttnArgs a)
{
    __shared__ __align__(16) uint8_t lds[kWaveBytes];

    const int lane = threadIdx.x;
    const int j = lane >> 4;        // 16-lane row of the wave
    const int c16 = lane & 15;      // column inside a 16-wide MFMA tile

    // one wave per (chunk, token), chunk-major; each XCD (workgroup id mod 8)
    // walks a contiguous range of them
    const int lb = (blockIdx.x & 7) * a.blocks_per_xcd + (blockIdx.x >> 3);
    if (lb >= a.n_blocks)
        return;
    // a wave still issuing its reads (q, ids, K copies, V rows) goes before
    // the waves of its SIMD that are computing, so that its requests leave
    // early; it drops back once they are all out
    __builtin_amdgcn_s_setprio(2);
    const int k = lb / a.T;
    const int t = lb - k * a.T;
    const WaveLds L = wave_lds(lds, 0);

    // q operand straight from memory: head c16, dims 32g + 8j .. +7; a padding
    // head (c16 >= H) repeats head H-1, and its results are never written
    half8 qop[4];
    {
        const _Float16 *qr = a.q + ((int64_t)t * a.H + min(c16, a.H - 1)) * kD + 8 * j;
#pragma unroll
        for (int g = 0; g < 4; ++g)
            qop[g] = *(const half8 *)(qr + 32 * g);
    }
    uint2 ks = make_uint2(0u, 0u), vs = make_uint2(0u, 0u);
    uint2 vraw[2][8];
    const uint64_t mask = issue_chunk(a, L, slot_id(a, t, k, lane), lane, j, c16, ks, vs, vraw);
    __builtin_amdgcn_s_setprio(0);
    const int64_t rec = ((int64_t)t * a.C + k) * a.H;
    if (mask == 0) {                 // empty chunk: (-inf, +0), o left alone
        if (lane < a.H) {
            a.m[rec + lane] = -INFINITY;
            a.l[rec + lane] = 0.0f;
        }
        return;
    }
    __builtin_amdgcn_s_waitcnt(0);   // the K tile copy has landed
    wave_sync_lds();

    const int kr = stage_scales(L, lane, ks, vs);
    float S[4][4];
    chunk_scores(a.scale, opaque_neg_zero(a), L, qop, j, c16, S);
    const float mx = chunk_max(S);
    float P[4][4];
    const float lsum = chunk_probs<false>(S, mx, P);
    floatx4 O[8];
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
        O[tt] = (floatx4){0.f, 0.f, 0.f, 0.f};
    pv_accumulate<false>(P, vraw, L, j, c16, kr, O);

    // ---- write the chunk record ----------------------------------------------
    if (kr != 0) {                  // take the V codes' power of two back out, exactly
        const float down = pow2f(kr);
#pragma unroll
        for (int tt = 0; tt < 8; ++tt)
            O[tt] *= down;
    }
    // The record leaves in whole 1 KB runs: its H head rows (512 B each, in
    // memory order) are laid out in the K tile, free since the scores, and
    // each store instruction then writes 1 KB of consecutive bytes (the MFMA
    // layout would have each instruction fill half of each of 16 lines). The
    // stores go through a buffer resource over the record (raw 32-bit
    // elements: DATA_FORMAT 32 in the descriptor's last word, no stride, no
    // swizzle), which also drops the second half of the last run when H is odd.
    float *st = (float *)L.ktile;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int head = 4 * j + r;
        if (head < a.H) {
            float *row = st + head * kD + 8 * c16;
            *(float4 *)row = make_float4(O[0][r], O[1][r], O[2][r], O[3][r]);
            *(float4 *)(row + 4) = make_float4(O[4][r], O[5][r], O[6][r], O[7][r]);
        }
    }
    wave_sync_lds();
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(a.o + rec * kD, 0, a.H * kD * (int)sizeof(float), 0x00020000);
    const int runs = (a.H + 1) / 2;
    if (a.nt_records) {              // uniform
        for (int i = 0; i < runs; ++i)
            __builtin_amdgcn_raw_buffer_store_b128(*(const floatx4 *)(st + 4 * (64 * i + lane)), rs,
                                                   16 * (64 * i + lane), 0, kCachePolicyNT);
    } else {
        for (int i = 0; i < runs; ++i)
            __builtin_amdgcn_raw_buffer_store_b128(*(const floatx4 *)(st + 4 * (64 * i + lane)), rs,
                                                   16 * (64 * i + lane), 0, 0);
    }
    if (j == 0 && c16 < a.H) {
        a.m[rec + c16] = mx;
        a.l[rec + c16] = lsum;
    }
}

// ---- attention with the merge in the same dispatch (qsa_attn_merge) --------
//
// One workgroup per token, nw = C waves for up to 8 chunks, else 4; wave w
// takes chunks w, w + nw, ... so every workgroup sweeps the chunks in the
// same order. A wave keeps a
// running max M, denominator L and output O per head: a chunk with max m moves
// M to max(M, m), its probabilities are taken against the new M and the old
// (L, O) are rescaled by exp(M_old - M_new) -- the combination of chunk records
// relative to the largest maximum, accumulated as it goes. The waves' (M, L, O)
// are then combined the same way through LDS and divided once. The gated
// entry point then multiplies each value by sigmoid(g) of its fp32 gate before
// the fp16 rounding and may write the exact per-16 sums of the written values
// ("round 5 track b: cached residual norms and fused mtp attention", section
// "preflight / ownership": the fused kernel keeps the sigmoid gate and the
// per-16 sums).

template <bool kPipelined>
__global__ __launch_bounds__(64 * kWavesMax) void attn_merge_kernel(AttnArgs a)
{
    extern __shared__ __align__(16) uint8_t lds[];

    const int lane0 = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;

    const int t = (blockIdx.x & 7) * a.blocks_per_xcd + (blockIdx.x >> 3);
    if (t >= a.T)
        return;                     // uniform over the workgroup

    const WaveLds L = wave_lds(lds, w);
    uint8_t *qrows = lds + nw * kWaveBytes;
    uint8_t *grows = qrows + a.H * kD * 2;       // gated calls only
    copy_q_rows(a, qrows, t, w, nw, lane0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (a.gate)                                  // uniform
        copy_gate_rows(a, grows, t, w, nw, lane0);

    float Mrun = -INFINITY, Lrun = 0.0f;         // head c16
    floatx4 O[8];                                // head c16, dims 8*(4j + r) + tt
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
        O[tt] = (floatx4){0.f, 0.f, 0.f, 0.f};

    if constexpr (kPipelined) {
        // waves that walk several chunks issue the next chunk's reads while
        // they compute the current one: its ids, scales and K rows as soon as
        // the scores have been taken from the K tile, its V rows once the
        // products have read the current ones. The arithmetic is the one below.
        uint2 ks = make_uint2(0u, 0u), vs = make_uint2(0u, 0u);
        uint2 vraw[2][8];
        uint64_t mask = 0;
        if (w < a.C) {
            int lane = lane0;
            asm volatile("" : "+v"(lane));
            mask = issue_k(a, L, slot_id(a, t, w, lane), lane, ks, vs);
            issue_v(a, L, mask, lane >> 4, lane & 15, vraw);
        }
        int32_t id_next = slot_id(a, t, min(w + nw, a.C - 1), lane0);
        for (int k = w; k < a.C; k += nw) {
            int lane = lane0;
            asm volatile("" : "+v"(lane));
            const int j = lane >> 4, c16 = lane & 15;
            __builtin_amdgcn_s_waitcnt(0);       // this chunk's tile, rows and scales; the next chunk's ids
            wave_sync_lds();
            const bool more = k + nw < a.C;      // uniform
            const bool live = mask != 0;         // uniform: an empty chunk adds nothing
            float P[4][4];
            float alpha = 1.0f;
            int kr = 0;
            if (live) {
                kr = stage_scales(L, lane, ks, vs);
                half8 qop[4];
                q_operand(a, qrows, j, c16, qop);
                float S[4][4];
                chunk_scores(a.scale * kLog2e, opaque_neg_zero(a), L, qop, j, c16, S);
                const float Mnew = fmaxf(Mrun, chunk_max(S));
                alpha = __builtin_amdgcn_exp2f(Mrun - Mnew);   // 0 for the first chunk
                Lrun = fmaf(alpha, Lrun, chunk_probs<true>(S, Mnew, P));
                Mrun = Mnew;
            }
            uint64_t mask_n = 0;
            if (more)
                mask_n = issue_k(a, L, id_next, lane, ks, vs);
            if (live) {
                if (__ballot(alpha != 1.0f) != 0) {     // uniform
#pragma unroll
                    for (int tt = 0; tt < 8; ++tt)
                        O[tt] *= alpha;
                }
                if (kr != 0) {
                    const float down = pow2f(kr);
#pragma unroll
                    for (int b = 0; b < 4; ++b)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            P[b][r] *= down;
                }
                pv_accumulate<true>(P, vraw, L, j, c16, kr, O);
            }
            if (more) {
                issue_v(a, L, mask_n, j, c16, vraw);
                id_next = slot_id(a, t, min(k + 2 * nw, a.C - 1), lane);
            }
            mask = mask_n;
            wave_sync_lds();
        }
    } else {
        // each chunk's slot ids are read one chunk ahead (the last chunk re-reads
        // its own), so a chunk's gathers start without a round trip for its ids
        int32_t id_next = slot_id(a, t, min(w, a.C - 1), lane0);
        for (int k = w; k < a.C; k += nw) {
            // lane-derived offsets are rebuilt every chunk (cheap VALU) rather than
            // hoisted out of the loop, where they would pin registers throughout
            int lane = lane0;
            asm volatile("" : "+v"(lane));
            const int j = lane >> 4, c16 = lane & 15;
            uint2 ks, vs;
            uint2 vraw[2][8];
            const uint64_t mask = issue_chunk(a, L, id_next, lane, j, c16, ks, vs, vraw);
            __builtin_amdgcn_s_waitcnt(0);           // the K tile copy has landed
            wave_sync_lds();
            id_next = slot_id(a, t, min(k + nw, a.C - 1), lane);   // in flight during this chunk
            if (mask == 0)
                continue;                            // uniform: an empty chunk adds nothing
            const int kr = stage_scales(L, lane, ks, vs);
            half8 qop[4];
            q_operand(a, qrows, j, c16, qop);
            float S[4][4];
            chunk_scores(a.scale * kLog2e, opaque_neg_zero(a), L, qop, j, c16, S);
            const float Mnew = fmaxf(Mrun, chunk_max(S));
            const float alpha = __builtin_amdgcn_exp2f(Mrun - Mnew);   // 0 for the first chunk
            float P[4][4];
            Lrun = fmaf(alpha, Lrun, chunk_probs<true>(S, Mnew, P));
            Mrun = Mnew;
            // rescale O: every value this lane holds is of its own head c16; a
            // chunk that moves no head's running max (alpha = 1 in every lane)
            // leaves O as it is
            if (__ballot(alpha != 1.0f) != 0) {     // uniform
#pragma unroll
                for (int tt = 0; tt < 8; ++tt)
                    O[tt] *= alpha;
            }
            if (kr != 0) {              // the chunk's V codes carry 2^-k: put 2^k on p
                const float down = pow2f(kr);
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        P[b][r] *= down;
            }
            pv_accumulate<true>(P, vraw, L, j, c16, kr, O);
            wave_sync_lds();                         // the tile is rewritten by the next chunk
        }
    }

    // ---- combine the waves: (M, L) and O through LDS, then divide once ---
    __builtin_amdgcn_s_waitcnt(0);               // this wave's gate copies have landed
    const int j = lane0 >> 4, c16 = lane0 & 15;
    float *sM = (float *)L.ksc;                  // 16 floats
    float *sL = sM + 16;                         // 16 floats
    float *sO = (float *)L.ktile;                // [16 heads][128 dims], rows rotated (below)
    if (j == 0) {
        sM[c16] = Mrun;
        sL[c16] = Lrun;
    }
    // head h's row holds its 32 granules of 4 dims rotated by h (granule g at
    // (g + h) % 32), so the sixteen lanes of a row, one head each, write
    // sixteen different bank groups
#pragma unroll
    for (int r = 0; r < 4; ++r) {               // head c16, dims 8(4j + r) .. +7
        float *row = sO + c16 * kD;
        const int g0 = 2 * (4 * j + r);
        *(float4 *)(row + 4 * ((g0 + c16) & 31)) = make_float4(O[0][r], O[1][r], O[2][r], O[3][r]);
        *(float4 *)(row + 4 * ((g0 + 1 + c16) & 31)) = make_float4(O[4][r], O[5][r], O[6][r], O[7][r]);
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < a.H * (kD / 4); idx += blockDim.x) {
        // H * 32 items: the four lanes of one 16-dim block (d4 = 4b .. 4b+3)
        // are consecutive threads of one wave and run the loop together
        const int h = idx / (kD / 4), d4 = idx - h * (kD / 4);
        float M = -INFINITY;
        for (int v = 0; v < nw; ++v)
            M = fmaxf(M, ((const float *)wave_lds(lds, v).ksc)[h]);
        float4 y = make_float4(0.f, 0.f, 0.f, 0.f);   // +0 when no slot of the row was valid
        if (M != -INFINITY) {
            float Ls = 0.0f;
            float4 Os = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int v = 0; v < nw; ++v) {
                const WaveLds Lv = wave_lds(lds, v);
                const float mv = ((const float *)Lv.ksc)[h];
                if (mv == -INFINITY)
                    continue;
                const float wv = __builtin_amdgcn_exp2f(mv - M);
                Ls = fmaf(wv, ((const float *)Lv.ksc)[16 + h], Ls);
                const float4 ov = *(const float4 *)((const float *)Lv.ktile + h * kD + 4 * ((d4 + h) & 31));
                Os.x = fmaf(wv, ov.x, Os.x);
                Os.y = fmaf(wv, ov.y, Os.y);
                Os.z = fmaf(wv, ov.z, Os.z);
                Os.w = fmaf(wv, ov.w, Os.w);
            }
            y = make_float4(Os.x / Ls, Os.y / Ls, Os.z / Ls, Os.w / Ls);
        }
        const int64_t orow = ((int64_t)t * a.H + h) * kD + 4 * d4;
        if (a.gate) {               // uniform: the gated entry point
            const float4 g = *(const float4 *)(grows + 16 * (h * (kD / 4) + d4));
            y.x *= sigmoid_gate(g.x);
            y.y *= sigmoid_gate(g.y);
            y.z *= sigmoid_gate(g.z);
            y.w *= sigmoid_gate(g.w);
        }
        const uint2 res = pack_half4(y.x, y.y, y.z, y.w);
        *(uint2 *)(a.out + orow) = res;
        if (a.sums) {               // uniform
            const double sb = xor_sum(xor_sum(half4_sum(res), 1), 2);
            if ((d4 & 3) == 0)
                a.sums[((int64_t)t * a.H + h) * (kD / 16) + (d4 >> 2)] = (float)sb;
        }
    }
}

} // namespace

hipError_t launch_attn(const AttnArgs &a, hipStream_t stream)
{
    hipLaunchKernelGGL(attn_kernel, dim3(8 * a.blocks_per_xcd), dim3(64), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_attn_merge(const AttnArgs &a, hipStream_t stream)
{
    // a row of up to kWavesMax chunks (a decode window) gets one wave per
    // chunk, so that its gathers all go out at once. Longer rows take kWaves,
    // except in calls of at most 64 tokens: there the grid is too small to
    // fill the chip at kWaves, and kWavesMax waves per row shorten the
    // serial walk over the chunks (2051 cells at T = 1: 33.8 -> 26.4 us)
    const int nw = a.C <= kWavesMax ? a.C : (a.T <= 64 ? kWavesMax : kWaves);
    dim3 grid(8 * a.blocks_per_xcd), block(64 * nw);
    // rows longer than one chunk per wave take the pipelined walk; a decode
    // window (one chunk per wave) has nothing to overlap
    if (a.C > nw)
        hipLaunchKernelGGL(attn_merge_kernel<true>, grid, block, attn_lds_bytes(nw, a.H, a.gate != nullptr), stream, a);
    else
        hipLaunchKernelGGL(attn_merge_kernel<false>, grid, block, attn_lds_bytes(nw, a.H, a.gate != nullptr), stream, a);
    return hipGetLastError();
}

} // namespace qsa
