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
// 16384 cells);
// the row's scores become order-preserving 32-bit keys held in registers
// (thread i holds cells i + 512 j, so every read is coalesced):
//   * the K-th largest key is found with four 8-bit radix passes from the top
//     byte down. The top byte's histogram keeps 32 counters per bin
//     (bin * 32 + lane % 32), so at most two lanes of a wave add to one
//     address, and the copies are then summed; the lower bytes count only the keys left in
//     the chosen bin, into plain 256-bin histograms cleared up front. One wave
//     scans each histogram from the top to pick the digit holding the K-th key;
//   * the result is the exact threshold key tau, the count of keys above it
//     and the number E of keys equal to it that are taken (the first E in
//     cell order);
//   * ids are then written in cell order: each wave records, for every block
//     j of 512 consecutive cells, how many of its 64 cells lie above tau and
//     how many equal it (ballots); one wave scans those counts in (block,
//     wave) order, and every thread places its cells from the scanned offsets
//     plus its lane prefix -- two barriers for the whole row.
// Cells past the row (c > p) hold key 0, below every score that is not NaN.
// Rows of up to 32768 cells (32 keys per thread).
#include "qsa_internal.h"

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

// Order-preserving key: larger score, larger key; -0 and +0 share one key.
__device__ inline uint32_t order_key(float f)
{
    uint32_t b = __float_as_uint(f);
    if ((b << 1) == 0)
        b = 0;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <int NT, int KPT>      // NT threads per row, KPT keys per thread
__global__ __launch_bounds__(NT) void select_kernel(SelectArgs a)
{
    constexpr int kSelThreads = NT;
    constexpr int kSelWaves = NT / 64;
    static_assert(KPT * kSelWaves * 8 <= kBins * kCopies * 4, "the compaction's counts reuse the histogram");
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

    const float *row = a.scores + (int64_t)t * a.row_stride;
    uint32_t key[KPT];
    // every read is issued (clamped into the row) before any is used, and the
    // empty asm keeps the compiler from moving a read under its c < n test,
    // where each would be waited for on its own; keys replace the raw bits in place
#pragma unroll
    for (int j = 0; j < KPT; ++j)
        key[j] = __float_as_uint(row[min(tid + kSelThreads * j, n - 1)]);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        asm volatile("" : "+v"(key[j]));
        key[j] = tid + kSelThreads * j < n ? order_key(__uint_as_float(key[j])) : 0u;
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
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        const uint32_t *hist;                            // the pass's 256 bin totals
        if (pass == 0) {
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
#pragma unroll
                for (int d = 1; d < kParts; d <<= 1)
                    sum += __shfl_xor(sum, d, 64);
                if (part == 0)
                    tot[bin] = sum;
            }
            __syncthreads();
            hist = tot;
        } else {
            uint32_t *h = cnt1 + (pass - 1) * kBins;
#pragma unroll
            for (int j = 0; j < KPT; ++j)
                if ((key[j] & mask) == prefix)
                    atomicAdd(&h[(key[j] >> shift) & 255u], 1u);
            __syncthreads();
            hist = h;
        }
        if (w == 0) {
            // lane l holds bins 4l .. 4l+3; suffix sums from the top bin down
            uint32_t b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                b[i] = hist[4 * lane + i];
            const uint32_t mine = b[0] + b[1] + b[2] + b[3];
            uint32_t suf = mine;                         // bins 4l .. 255
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const uint32_t o = __shfl_down(suf, d, 64);
                if (lane + d < 64)
                    suf += o;
            }
            const uint32_t above_lane = suf - mine;      // bins 4l+4 .. 255
            // the lane whose bins hold the k_left-th largest candidate
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
    }
    const uint32_t tau = prefix;                         // the K-th largest key
    const uint32_t take_eq = k_left;                     // keys equal to tau that are taken (in cell order);
                                                         // the other K - take_eq keys lie above tau

    // ---- ids in cell order ----------------------------------------------------
    // counts of each (block j, wave) pair: block j is cells NT j .. NT j + NT - 1,
    // wave w holds NT j + 64 w .. +63 of them
    uint2 *pc = (uint2 *)cnt;                            // [KPT][8 waves]
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const uint64_t bg = __ballot(key[j] > tau), be = __ballot(key[j] == tau);
        if (lane == 0)
            pc[j * kSelWaves + w] = make_uint2((uint32_t)__popcll(bg), (uint32_t)__popcll(be));
    }
    __syncthreads();
    if (w == 0) {
        // exclusive scan of the KPT * 8 pairs in (block, wave) order; lane l owns
        // a run of consecutive entries
        constexpr int kEnt = KPT * kSelWaves;
        constexpr int kPer = (kEnt + 63) / 64;
        uint32_t sg = 0, se = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = lane * kPer + i;
            if (e < kEnt) {
                const uint2 v = pc[e];
                sg += v.x;
                se += v.y;
            }
        }
        uint32_t ig = sg, ie = se;                       // inclusive over lanes
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t og = __shfl_up(ig, d, 64), oe = __shfl_up(ie, d, 64);
            if (lane >= d) {
                ig += og;
                ie += oe;
            }
        }
        uint32_t rg = ig - sg, re = ie - se;             // before this lane's run
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = lane * kPer + i;
            if (e < kEnt) {
                const uint2 v = pc[e];
                pc[e] = make_uint2(rg, re);
                rg += v.x;
                re += v.y;
            }
        }
    }
    __syncthreads();
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    // recompute the ballots rather than keep the first loop's (2 x KPT masks
    // would not fit in scalar registers): tau is hidden from the compiler here
    uint32_t tau2 = tau;
    int tid2 = tid;                 // cell indices are rebuilt here, not kept from the reads
    asm volatile("" : "+v"(tau2), "+v"(tid2));
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const bool gt = key[j] > tau2, eq = key[j] == tau2;
        const uint64_t bg = __ballot(gt), be = __ballot(eq);
        const uint2 base = pc[j * kSelWaves + w];
        const uint32_t gt_before = base.x + (uint32_t)__popcll(bg & below);
        const uint32_t eq_before = base.y + (uint32_t)__popcll(be & below);
        if (gt || (eq && eq_before < take_eq))
            ids[gt_before + min(eq_before, take_eq)] = tid2 + kSelThreads * j;
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

} // namespace

hipError_t launch_select(const SelectArgs &a, hipStream_t stream)
{
    const int n_max = a.pos0 + a.T;
    if (n_max <= 8 * 512)
        return launch_kpt<512, 8>(a, stream);
    if (n_max <= 16 * 512)
        return launch_kpt<512, 16>(a, stream);
    if (n_max <= 32 * 512)
        return launch_kpt<512, 32>(a, stream);
    return launch_kpt<1024, 32>(a, stream);          // n_max <= 32768, checked by the caller
}

} // namespace qsa
