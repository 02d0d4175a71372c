// qsa_internal.h -- declarations shared by the kernels and the C-ABI layer of
// libqsa.so. Not installed; the public interface is include/qsa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

constexpr int kD = 128;       // the one head dim the kernels implement
constexpr int kChunk = 64;    // slots per chunk
constexpr int kGroup = 32;    // dims per fp16 scale
constexpr int kMaxHeads = 16; // heads fill the 16-wide MFMA tile dimension
constexpr int kAttnWaves = 4; // waves of a fused attention workgroup (one token) over more than 8 chunks, in calls of more than 64 tokens
constexpr int kMaxCells = 1 << 25; // cache rows addressed with 32-bit byte offsets

struct AttnArgs {
    const _Float16 *q;        // [T][H][D]
    const int8_t *kq;         // [n_cells][D]
    const int8_t *vq;         // [n_cells][D]
    const uint16_t *ksc;      // [n_cells][D/32] fp16 bits
    const uint16_t *vsc;      // [n_cells][D/32] fp16 bits
    const int32_t *ids;       // [T][ids_stride] or nullptr (implicit rows)
    int64_t ids_stride;
    int32_t n_cells, pos0, T, H, C;
    float scale;
    float *o;                 // [T][C][H][D]   chunk records (qsa_attn)
    float *m;                 // [T][C][H]
    float *l;                 // [T][C][H]
    _Float16 *out;            // [T][H][D]      merged output (qsa_attn_merge)
    const float *gate;        // [T][H][D] fp32 sigmoid-gate inputs, or nullptr (ungated)
    float *sums;              // [T][H][D/16] per-16 sums of out, or nullptr
    int32_t n_blocks;         // workgroups that carry work: C x T one-wave records, T fused
    int32_t blocks_per_xcd;   // workgroups each XCD walks through
    int32_t nt_records;       // records kernel: store the chunk records nontemporal
};

// A qsa_attn call whose chunk records take more than this many bytes stores
// them nontemporal. Such records cannot stay in the Infinity Cache (256 MB on
// MI355X) until qsa_merge reads them anyway, and streaming them past L2 and
// the Infinity Cache leaves both to the cache rows the gathers reuse. Smaller
// calls (decode windows, short prompts) keep their records in the caches for
// the merge.
constexpr int64_t kNontemporalRecordBytes = int64_t(128) << 20;

struct MergeArgs {
    const float *o, *m, *l;
    int32_t C, T, H;
    _Float16 *out;            // [T][H][D]
    const float *gate;        // [T][H][D] fp32 sigmoid-gate inputs, or nullptr (ungated)
    float *sums;              // [T][H][D/16] per-16 sums of out, or nullptr
};

struct ScoreArgs {
    const float *q;           // [T][Hs][D]
    const float *k;           // [n_cells][D]
    int32_t n_cells, pos0, T, Hs;
    float scale, dead;
    float *scores;            // [T][row_stride]
    int64_t row_stride;
};

struct QuantArgs {
    const float *k, *v;       // [n_rows][D] fp32
    int8_t *kq, *vq;          // [n_cells_cap][D]
    uint16_t *ksc, *vsc;      // [n_cells_cap][D/32] fp16 bits
    int32_t n_rows, cell0;    // rows land at cells cell0 .. cell0 + n_rows - 1
};

struct SelectArgs {
    const float *scores;      // [T][row_stride]
    int64_t row_stride;
    int32_t pos0, T, K;
    int32_t *ids;             // [T][ids_stride]
    int32_t ids_stride;
};
constexpr int kMaxSelectCells = 1 << 15;   // cells per row the selection kernel holds in registers;
                                            // longer rows (up to kMaxCells) stream their scores

// Part workspace layout: o, then m, then l, each on a 256-byte boundary.
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline void part_layout(int64_t T, int64_t H, int64_t D, int64_t C,
                        size_t *o_off, size_t *m_off, size_t *l_off, size_t *total)
{
    size_t o_bytes = align256(size_t(T) * C * H * D * sizeof(float));
    size_t s_bytes = align256(size_t(T) * C * H * sizeof(float));
    if (o_off) *o_off = 0;
    if (m_off) *m_off = o_bytes;
    if (l_off) *l_off = o_bytes + s_bytes;
    if (total) *total = o_bytes + 2 * s_bytes;
}

hipError_t launch_attn(const AttnArgs &a, hipStream_t stream);
hipError_t launch_attn_merge(const AttnArgs &a, hipStream_t stream);
// implicit rows (ids == nullptr): token blocks share each chunk's cells
hipError_t launch_attn_tile(const AttnArgs &a, hipStream_t stream);
hipError_t launch_attn_merge_tile(const AttnArgs &a, hipStream_t stream);
hipError_t launch_merge(const MergeArgs &a, hipStream_t stream);
// ws: nullptr, or score_ws_bytes(a.T) bytes of device memory for the prepared q operands
hipError_t launch_score(const ScoreArgs &a, void *ws, hipStream_t stream);
inline int64_t score_ws_bytes(int32_t T) { return T <= 0 ? 0 : (((int64_t)T + 63) / 64) * 64 * 512; }
hipError_t launch_quant(const QuantArgs &a, hipStream_t stream);
hipError_t launch_select(const SelectArgs &a, hipStream_t stream);

} // namespace qsa
