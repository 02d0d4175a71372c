// qsa_select.hip -- the ids each query row attends over, chosen from its
// causal scores.
//
// The pages only say that a row's selected ids are unique causal cells ("round
// 11 track b: qsa attention and score", section "boundaries and provenance")
// and never print how they are chosen; this library takes top-K: row t
// (p = pos0 + t) selects the min(K, p + 1) cells c <= p with the largest
// scores[t][c], equal scores (-0 equal to +0) going to the smaller cell, and
// writes them in ascending cell order, padded with -1 to ids_stride -- the id
// rows qsa_attn reads.
//
// Design on CDNA4. One workgroup of 512 threads per row (1024 for rows past
// 16384 cells), at most 64 VGPRs so that two rows share a CU; the row's scores
// become order-preserving 32-bit keys held in registers (thread i holds cells
// i + NT j, so every read is coalesced; the reads go through a buffer resource
// sized to the row's causal cells, so cells past the row read zero without a
// clamp):
//   * the K-th largest key is found with four 8-bit radix passes from the top
//     byte down. The top byte's histogram keeps 32 counters per bin
//     (bin * 32 + lane % 32), so at most two lanes of a wave add to one
//     address, and the copies are then summed; the lower bytes count only the keys left in
//     the chosen bin, into plain 256-bin histograms cleared up front. One wave
//     scans each histogram from the top to pick the digit holding the K-th key;
//   * the result is the exact threshold key tau, the count of keys above it
//     and the number E of keys equal to it that are taken (the first E in
//     cell order);
//   * ids are then written in cell order: ballots turn the strided keys into
//     bit masks of the cells above tau and equal to it, stored in LDS in cell
//     order; each thread then takes 32 consecutive cells of the masks, one
//     scan over the threads gives the counts before them, and every thread
//     writes its selected cells from there -- two barriers for the whole row.
// Cells past the row (c > p) hold key 0, below every score that is not NaN.
// Rows of up to 32768 cells (32 keys per thread).
#include "qsa_internal.h"

#include <algorithm>

namespace qsa {
namespace {

constexpr int kBins = 256;

// LDS layout (the counts of the last phase reuse the histogram)
constexpr int kCopies = 32;                            // counters per bin in the top byte's histogram
constexpr int kLCnt = 0;                               // uint[256 bins][32 copies]; later uint2[KPT][waves]
constexpr int kLTot = kLCnt + kBins * kCopies * 4;     // uint[256] bin totals
constexpr int kLDec = kLTot + kBins * 4;               // uint[2][2]: digit, count above it (by pass parity)
constexpr int kLCnt1 = kLDec + 16;                     // uint[3 passes][256]: single-copy histograms
constexpr int kSelLds = kLCnt1 + 3 * kBins * 4;

// Inclusive prefix sum over the 64 lanes of a wave in six DPP steps: shifts by
// 1, 2, 4 and 8 lanes inside each 16-lane row, then each row adds the totals
// of the rows before it through the row broadcasts of lanes 15 and 31. All in
// the VALU; a shuffle-based scan takes an LDS round trip per step.
__device__ inline uint32_t wave_prefix_sum(uint32_t v)
{
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);   // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);   // row_bcast:15 to rows 1, 3
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);   // row_bcast:31 to rows 2, 3
    return v;
}

// Inclusive suffix sum over the lanes (lane l: lanes l .. 63), from the prefix
// sum and the wave total.
__device__ inline uint32_t wave_suffix_sum(uint32_t v)
{
    const uint32_t pre = wave_prefix_sum(v);
    const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)pre, 63);
    return total - pre + v;
}

// Sum over aligned groups of `parts` lanes (2 or 4) by DPP quad permutes.
__device__ inline uint32_t quad_group_sum(uint32_t v, int parts)
{
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false);    // lane ^ 1
    if (parts == 4)
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false);   // lane ^ 2
    return v;
}

// Order-preserving key: larger score, larger key. Non-negative scores map to
// b | 2^31 (+0 to 2^31); negative ones to 2^32 - b, so -0 (b = 2^31) meets
// +0 at 2^31 and the most negative bit pattern maps to 1, above the key 0
// that cells past the row get.
__device__ inline uint32_t order_key(float f)
{
    const uint32_t b = __float_as_uint(f);
    return (int32_t)b < 0 ? 0u - b : (b | 0x80000000u);
}

// NT threads per row, KPT keys per thread. Eight waves per SIMD (at most 64
// VGPRs) let two 1024-thread rows share a CU, so one row's reads overlap the
// other's histogram passes.
template <int NT, int KPT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(8))) void select_kernel(SelectArgs a)
{
    constexpr int kSelThreads = NT;
    constexpr int kSelWaves = NT / 64;
    static_assert(KPT * kSelWaves * 16 <= kBins * kCopies * 4, "the compaction's masks reuse the histogram");
    static_assert(kSelWaves <= kBins && KPT <= 32, "wave totals reuse the bin totals; one mask bit per key");
    __shared__ __align__(16) uint8_t lds[kSelLds];
    uint32_t *cnt = (uint32_t *)(lds + kLCnt);
    uint32_t *tot = (uint32_t *)(lds + kLTot);
    uint32_t *dec = (uint32_t *)(lds + kLDec);

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int t = blockIdx.x;
    const int n = a.pos0 + t + 1;                       // cells 0 .. p
    int32_t *ids = a.ids + (int64_t)t * a.ids_stride;

    if (n <= a.K) {                                     // every causal cell (uniform per workgroup)
        for (int q = tid; q < a.ids_stride; q += kSelThreads)
            ids[q] = q < n ? q : -1;
        return;
    }

    // the row's causal cells through a buffer resource of n * 4 bytes: a read
    // past cell p returns zero and touches no memory. The whole cell offset
    // goes in the per-lane offset, which the hardware checks against the
    // resource's size (the scalar offset is not part of that check).
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.scores + (int64_t)t * a.row_stride), 0, n * 4, 0x00020000);
    uint32_t key[KPT];
    // the row's reads leave ahead of the other row's passes on this CU
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int j = 0; j < KPT; ++j)
        key[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsrc, (tid + kSelThreads * j) * 4, 0, 0);
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const int lim = n - kSelThreads * j;             // uniform: cell tid + NT j < n iff tid < lim
        key[j] = tid < lim ? order_key(__uint_as_float(key[j])) : 0u;
    }

    // ---- the K-th largest key, one byte at a time ---------------------------
    // The top byte sees every key: its histogram keeps 32 counters per bin so
    // that at most two lanes of a wave add to one address. After it only the keys of
    // the chosen bin remain (a small share for any spread of scores), so the
    // three lower bytes count into plain 256-bin histograms, all cleared up
    // front: two barriers per pass.
    uint32_t *cnt1 = (uint32_t *)(lds + kLCnt1);
    for (int q = tid; q < 3 * kBins; q += kSelThreads)
        cnt1[q] = 0u;
    uint32_t prefix = 0, mask = 0, k_left = (uint32_t)a.K;
    // one wave scans a pass's 256 bin totals from the top for the bin holding
    // the k_left-th largest candidate; every thread then takes its digit
    auto pick = [&](const uint32_t *hist, int pass) {
        const int shift = 24 - 8 * pass;
        if (w == 0) {
            // lane l holds bins 4l .. 4l+3; suffix sums from the top bin down
            uint32_t b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                b[i] = hist[4 * lane + i];
            const uint32_t mine = b[0] + b[1] + b[2] + b[3];
            const uint32_t suf = wave_suffix_sum(mine);  // bins 4l .. 255
            const uint32_t above_lane = suf - mine;      // bins 4l+4 .. 255
            if (above_lane < k_left && suf >= k_left) {
                uint32_t acc = above_lane;
                int digit = 4 * lane + 3;
#pragma unroll
                for (int i = 3; i >= 0; --i) {
                    if (acc + b[i] >= k_left) {
                        digit = 4 * lane + i;
                        break;
                    }
                    acc += b[i];
                }
                dec[2 * (pass & 1)] = (uint32_t)digit;
                dec[2 * (pass & 1) + 1] = acc;           // candidates above the chosen digit
            }
        }
        __syncthreads();
        const uint32_t digit = dec[2 * (pass & 1)], acc = dec[2 * (pass & 1) + 1];
        prefix |= digit << shift;
        mask |= 255u << shift;
        k_left -= acc;
    };

    // the top byte: every key, 32 counters per bin
    for (int q = tid; q < kBins * kCopies / 4; q += kSelThreads)
        ((uint4 *)cnt)[q] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KPT; ++j)
        atomicAdd(&cnt[(key[j] >> 24) * kCopies + (lane & (kCopies - 1))], 1u);
    __syncthreads();
    {   // bin totals: NT / 256 threads per bin, each summing a share of the copies
        constexpr int kParts = NT / kBins;
        const int bin = tid / kParts, part = tid % kParts;
        const uint4 *src = (const uint4 *)(cnt + bin * kCopies + part * (kCopies / kParts));
        uint32_t sum = 0;
#pragma unroll
        for (int i = 0; i < kCopies / 4 / kParts; ++i) {
            const uint4 v = src[i];
            sum += v.x + v.y + v.z + v.w;
        }
        static_assert(kParts == 2 || kParts == 4, "a bin's copies are summed by 2 or 4 lanes");
        sum = quad_group_sum(sum, kParts);
        if (part == 0)
            tot[bin] = sum;
    }
    __syncthreads();
    pick(tot, 0);
    // the lower bytes: only the keys whose higher bytes match the digits so far
#pragma unroll 1
    for (int pass = 1; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        uint32_t *h = cnt1 + (pass - 1) * kBins;
#pragma unroll
        for (int j = 0; j < KPT; ++j)
            if ((key[j] & mask) == prefix)
                atomicAdd(&h[(key[j] >> shift) & 255u], 1u);
        __syncthreads();
        pick(h, pass);
    }
    const uint32_t tau = prefix;                         // the K-th largest key
    const uint32_t take_eq = k_left;                     // keys equal to tau that are taken (in cell order);
                                                         // the other K - take_eq keys lie above tau

    // ---- ids in cell order ----------------------------------------------------
    // A ballot turns the keys of block j (cells NT j .. NT j + NT - 1) held by
    // wave w into the 64-bit masks of cells NT j + 64 w .. +63 above tau and
    // equal to it: mask word (j, w) covers cells 64 (kSelWaves j + w) .. +63,
    // so the words in (j, w) order are the row's masks in cell order. Lane j of
    // each wave gathers block j's words, and one LDS write per wave
    // stores them.
    uint4 *words = (uint4 *)cnt;                         // [KPT * kSelWaves] {gt lo, gt hi, eq lo, eq hi}
    {
        // each ballot's two words go straight into lane j of the collecting
        // registers (v_writelane, lane j an immediate). Selecting them by lane
        // instead left the compiler holding the ballots in scalar registers,
        // 70 of which it spilled into vector lanes.
        uint32_t glo = 0, ghi = 0, elo = 0, ehi = 0;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const uint64_t bg = __ballot(key[j] > tau), be = __ballot(key[j] == tau);
            asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(glo) : "s"((uint32_t)bg), "i"(j));
            asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(ghi) : "s"((uint32_t)(bg >> 32)), "i"(j));
            asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(elo) : "s"((uint32_t)be), "i"(j));
            asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(ehi) : "s"((uint32_t)(be >> 32)), "i"(j));
        }
        if (lane < KPT)
            words[lane * kSelWaves + w] = make_uint4(glo, ghi, elo, ehi);
    }
    __syncthreads();
    // Thread i now takes cells 32 i .. 32 i + 31, half of word i / 2: the counts
    // above and equal to tau before its cells come from one scan over the
    // threads, and its cells are written in order from there.
    constexpr int kCellThreads = KPT * kSelThreads / 32;
    uint32_t gt32 = 0, eq32 = 0;
    if (tid < kCellThreads) {
        const uint4 wd = words[tid >> 1];
        gt32 = (tid & 1) ? wd.y : wd.x;
        eq32 = (tid & 1) ? wd.w : wd.z;
    }
    // counts packed as (above << 16) | equal: each is at most 32768 over the row
    const uint32_t own = ((uint32_t)__popc(gt32) << 16) | (uint32_t)__popc(eq32);
    const uint32_t inc = wave_prefix_sum(own);
    uint32_t *wsum = tot;                                // [kSelWaves] wave totals
    if (lane == 63)
        wsum[w] = inc;
    __syncthreads();
    uint32_t before = inc - own;
    for (int v = 0; v < w; ++v)
        before += wsum[v];
    const uint32_t gt_before = before >> 16, eq_before = before & 0xffffu;
    // the first take_eq cells equal to tau are taken: this thread keeps the
    // lowest of its equal cells while the count before it is short of take_eq
    uint32_t keep = 0, m = eq32;
    for (uint32_t k = eq_before; k < take_eq && m != 0; ++k) {
        keep |= m & (0u - m);
        m &= m - 1;
    }
    uint32_t sel = gt32 | keep;
    uint32_t slot = gt_before + min(eq_before, take_eq);
    while (sel != 0) {
        ids[slot++] = 32 * tid + __builtin_ctz(sel);
        sel &= sel - 1;
    }
    for (int q = a.K + tid; q < a.ids_stride; q += kSelThreads)
        ids[q] = -1;
}

// Rows longer than the registers hold (more than 32768 cells): the same four
// radix passes and the same compaction, but every pass streams the row's
// scores from memory again (the keys are rebuilt on each read), and the ids
// are written one 32768-cell segment at a time, with the counts above and
// equal to the threshold carried from segment to segment.
constexpr int kStreamThreads = 1024;
constexpr int kStreamSeg = 32 * kStreamThreads;       // cells per compaction segment

__global__ __launch_bounds__(kStreamThreads) void select_stream_kernel(SelectArgs a)
{
    constexpr int kSelThreads = kStreamThreads;
    constexpr int kSelWaves = kSelThreads / 64;
    __shared__ __align__(16) uint8_t lds[kSelLds];
    uint32_t *cnt = (uint32_t *)(lds + kLCnt);
    uint32_t *tot = (uint32_t *)(lds + kLTot);
    uint32_t *dec = (uint32_t *)(lds + kLDec);

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int t = blockIdx.x;
    const int n = a.pos0 + t + 1;                       // cells 0 .. p
    int32_t *ids = a.ids + (int64_t)t * a.ids_stride;
    if (n <= a.K) {
        for (int q = tid; q < a.ids_stride; q += kSelThreads)
            ids[q] = q < n ? q : -1;
        return;
    }
    // the row's causal cells; a read past cell p returns zero and touches no
    // memory (the whole offset is in the range-checked per-lane offset)
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.scores + (int64_t)t * a.row_stride), 0, n * 4, 0x00020000);
    auto key_at = [&](int c) -> uint32_t {
        const uint32_t raw = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsrc, c * 4, 0, 0);
        return c < n ? order_key(__uint_as_float(raw)) : 0u;
    };

    uint32_t *cnt1 = (uint32_t *)(lds + kLCnt1);
    for (int q = tid; q < 3 * kBins; q += kSelThreads)
        cnt1[q] = 0u;
    for (int q = tid; q < kBins * kCopies / 4; q += kSelThreads)
        ((uint4 *)cnt)[q] = make_uint4(0u, 0u, 0u, 0u);
    uint32_t prefix = 0, mask = 0, k_left = (uint32_t)a.K;
    __syncthreads();
    for (int c = tid; c < n; c += kSelThreads)
        atomicAdd(&cnt[(key_at(c) >> 24) * kCopies + (lane & (kCopies - 1))], 1u);
    __syncthreads();
    {   // bin totals: four threads per bin, each summing eight of the copies
        constexpr int kParts = kSelThreads / kBins;
        const int bin = tid / kParts, part = tid % kParts;
        const uint4 *src = (const uint4 *)(cnt + bin * kCopies + part * (kCopies / kParts));
        uint32_t sum = 0;
#pragma unroll
        for (int i = 0; i < kCopies / 4 / kParts; ++i) {
            const uint4 v = src[i];
            sum += v.x + v.y + v.z + v.w;
        }
        static_assert(kParts == 2 || kParts == 4, "a bin's copies are summed by 2 or 4 lanes");
        sum = quad_group_sum(sum, kParts);
        if (part == 0)
            tot[bin] = sum;
    }
    __syncthreads();
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        const uint32_t *hist = tot;
        if (pass > 0) {
            uint32_t *h = cnt1 + (pass - 1) * kBins;
            for (int c = tid; c < n; c += kSelThreads) {
                const uint32_t kc = key_at(c);
                if ((kc & mask) == prefix)
                    atomicAdd(&h[(kc >> shift) & 255u], 1u);
            }
            __syncthreads();
            hist = h;
        }
        if (w == 0) {
            uint32_t b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                b[i] = hist[4 * lane + i];
            const uint32_t mine = b[0] + b[1] + b[2] + b[3];
            const uint32_t suf = wave_suffix_sum(mine);
            const uint32_t above_lane = suf - mine;
            if (above_lane < k_left && suf >= k_left) {
                uint32_t acc = above_lane;
                int digit = 4 * lane + 3;
#pragma unroll
                for (int i = 3; i >= 0; --i) {
                    if (acc + b[i] >= k_left) {
                        digit = 4 * lane + i;
                        break;
                    }
                    acc += b[i];
                }
                dec[2 * (pass & 1)] = (uint32_t)digit;
                dec[2 * (pass & 1) + 1] = acc;
            }
        }
        __syncthreads();
        const uint32_t digit = dec[2 * (pass & 1)], acc = dec[2 * (pass & 1) + 1];
        prefix |= digit << shift;
        mask |= 255u << shift;
        k_left -= acc;
    }
    const uint32_t tau = prefix;
    const uint32_t take_eq = k_left;

    // ids segment by segment: ballot masks in cell order, one scan over the
    // threads, counts before the segment carried in (gt_run, eq_run)
    uint4 *words = (uint4 *)cnt;
    uint32_t *wsum = tot;
    uint32_t gt_run = 0, eq_run = 0;
#pragma unroll 1
    for (int seg = 0; seg < n; seg += kStreamSeg) {
        {
            uint32_t glo = 0, ghi = 0, elo = 0, ehi = 0;
#pragma unroll 4
            for (int j = 0; j < 32; ++j) {
                const uint32_t kc = key_at(seg + tid + kSelThreads * j);
                const uint64_t bg = __ballot(kc > tau), be = __ballot(kc == tau);
                const bool mine = lane == j;
                glo = mine ? (uint32_t)bg : glo;
                ghi = mine ? (uint32_t)(bg >> 32) : ghi;
                elo = mine ? (uint32_t)be : elo;
                ehi = mine ? (uint32_t)(be >> 32) : ehi;
            }
            if (lane < 32)
                words[lane * kSelWaves + w] = make_uint4(glo, ghi, elo, ehi);
        }
        __syncthreads();
        const uint4 wd = words[tid >> 1];
        const uint32_t gt32 = (tid & 1) ? wd.y : wd.x, eq32 = (tid & 1) ? wd.w : wd.z;
        const uint32_t own = ((uint32_t)__popc(gt32) << 16) | (uint32_t)__popc(eq32);
        const uint32_t inc = wave_prefix_sum(own);
        if (lane == 63)
            wsum[w] = inc;
        __syncthreads();
        uint32_t before = inc - own, seg_total = 0;
        for (int v = 0; v < kSelWaves; ++v) {
            const uint32_t sv = wsum[v];
            if (v < w)
                before += sv;
            seg_total += sv;
        }
        const uint32_t gt_before = gt_run + (before >> 16), eq_before = eq_run + (before & 0xffffu);
        uint32_t keep = 0, m = eq32;
        for (uint32_t k = eq_before; k < take_eq && m != 0; ++k) {
            keep |= m & (0u - m);
            m &= m - 1;
        }
        uint32_t sel = gt32 | keep;
        uint32_t slot = gt_before + min(eq_before, take_eq);
        while (sel != 0) {
            ids[slot++] = seg + 32 * tid + __builtin_ctz(sel);
            sel &= sel - 1;
        }
        gt_run += seg_total >> 16;
        eq_run += seg_total & 0xffffu;
        __syncthreads();                                 // words and wave totals are rewritten next segment
    }
    for (int q = a.K + tid; q < a.ids_stride; q += kSelThreads)
        ids[q] = -1;
}

template <int NT, int KPT>
hipError_t launch_kpt(const SelectArgs &a, hipStream_t stream)
{
    hipLaunchKernelGGL((select_kernel<NT, KPT>), dim3(a.T), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_rows(const SelectArgs &a, hipStream_t stream)
{
    const int n_max = a.pos0 + a.T;
    if (n_max <= 8 * 512)
        return launch_kpt<512, 8>(a, stream);
    if (n_max <= 16 * 512)
        return launch_kpt<512, 16>(a, stream);
    if (n_max <= 32 * 512)
        return launch_kpt<512, 32>(a, stream);
    return launch_kpt<1024, 32>(a, stream);
}

} // namespace

hipError_t launch_select(const SelectArgs &a, hipStream_t stream)
{
    // rows of up to 32768 cells keep their keys in registers; longer rows
    // (the later rows of a long call) stream their scores
    const int64_t t_split = std::max<int64_t>(0, std::min<int64_t>(a.T, (int64_t)kMaxSelectCells - a.pos0));
    if (t_split > 0) {
        SelectArgs r = a;
        r.T = (int32_t)t_split;
        const hipError_t e = launch_rows(r, stream);
        if (e != hipSuccess || t_split == a.T)
            return e;
    }
    SelectArgs r = a;
    r.scores = a.scores + t_split * a.row_stride;
    r.ids = a.ids + t_split * (int64_t)a.ids_stride;
    r.pos0 = a.pos0 + (int32_t)t_split;
    r.T = a.T - (int32_t)t_split;
    hipLaunchKernelGGL(select_stream_kernel, dim3(r.T), dim3(kStreamThreads), 0, stream, r);
    return hipGetLastError();
}

} // namespace qsa
