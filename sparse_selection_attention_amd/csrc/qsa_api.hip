// qsa_api.hip -- the C ABI of libqsa.so (declared in include/qsa.h).
//
// Every entry point checks its arguments on the host before anything reaches
// the device, so a bad call is rejected with QSA_ERR_ARG or
// QSA_ERR_UNSUPPORTED and enqueues nothing. Kernels are enqueued on the
// caller's stream and the call returns without synchronising.
#include "qsa.h"
#include "qsa_internal.h"

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

namespace {

thread_local char g_err[512] = "";

qsa_status fail(qsa_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

qsa_status ok()
{
    g_err[0] = '\0';
    return QSA_OK;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Per-device answer to "is this a gfx950?": 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

qsa_status check_device()
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(QSA_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(QSA_ERR_UNSUPPORTED, "device index %d out of range", dev);
    int st = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess)
            return fail(QSA_ERR_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_arch_ok[dev].store(st, std::memory_order_relaxed);
        if (st == 2)
            return fail(QSA_ERR_UNSUPPORTED, "device %d is %s, this library is built for gfx950",
                        dev, prop.gcnArchName);
    }
    if (st == 2)
        return fail(QSA_ERR_UNSUPPORTED, "device %d is not a gfx950", dev);
    return QSA_OK;
}

qsa_status launched(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(QSA_ERR_DEVICE, "%s launch: %s", what, hipGetErrorString(e));
    return ok();
}

} // namespace

extern "C" {

size_t qsa_part_bytes(int32_t T, int32_t H, int32_t D, int32_t n_chunks)
{
    if (T < 0 || H < 0 || D < 0 || n_chunks < 0)
        return 0;
    size_t total = 0;
    qsa::part_layout(T, H, D, n_chunks, nullptr, nullptr, nullptr, &total);
    return total;
}

void qsa_part_offsets(int32_t T, int32_t H, int32_t D, int32_t n_chunks,
                      size_t *o_off, size_t *m_off, size_t *l_off)
{
    if (T < 0 || H < 0 || D < 0 || n_chunks < 0) {
        if (o_off) *o_off = 0;
        if (m_off) *m_off = 0;
        if (l_off) *l_off = 0;
        return;
    }
    qsa::part_layout(T, H, D, n_chunks, o_off, m_off, l_off, nullptr);
}

const char *qsa_last_error(void) { return g_err; }

} // extern "C"

namespace {

// Checks shared by qsa_attn and qsa_attn_merge; fills the geometry of `a`.
// Returns QSA_OK with *noop set when T == 0.
qsa_status check_attn(const char *fn, const void *q, const int8_t *kq, const int8_t *vq, const void *ksc,
                      const void *vsc, int32_t n_cells, const int32_t *ids, int32_t ids_stride, int32_t pos0,
                      int32_t T, int32_t H, int32_t D, float scale, qsa::AttnArgs &a, bool *noop)
{
    *noop = false;
    if (T < 0 || pos0 < 0 || n_cells < 0)
        return fail(QSA_ERR_ARG, "%s: negative T (%d), pos0 (%d) or n_cells (%d)", fn, T, pos0, n_cells);
    if (H < 1)
        return fail(QSA_ERR_ARG, "%s: H must be >= 1 (got %d)", fn, H);
    if (H > qsa::kMaxHeads)
        return fail(QSA_ERR_UNSUPPORTED, "%s: at most %d heads (got %d)", fn, qsa::kMaxHeads, H);
    if (D != qsa::kD)
        return fail(QSA_ERR_UNSUPPORTED, "%s: head dim %d not implemented (only %d)", fn, D, qsa::kD);
    if (ids && (ids_stride <= 0 || ids_stride % QSA_CHUNK != 0))
        return fail(QSA_ERR_ARG, "%s: ids_stride must be a positive multiple of %d (got %d)", fn, QSA_CHUNK,
                    ids_stride);
    if ((int64_t)pos0 + T > INT32_MAX)
        return fail(QSA_ERR_ARG, "%s: pos0 + T overflows int32", fn);
    if ((int64_t)n_cells < (int64_t)pos0 + T)
        return fail(QSA_ERR_ARG, "%s: n_cells (%d) < pos0 + T (%lld): the cache must hold every causal cell", fn,
                    n_cells, (long long)pos0 + T);
    if (n_cells > qsa::kMaxCells)
        return fail(QSA_ERR_UNSUPPORTED, "%s: at most %d cached rows (got %d)", fn, qsa::kMaxCells, n_cells);
    if ((int64_t)T * H > INT32_MAX - 64)
        return fail(QSA_ERR_ARG, "%s: T * H too large for one launch", fn);
    if (T == 0) {
        *noop = true;
        return QSA_OK;
    }
    if (!q || !kq || !vq || !ksc || !vsc)
        return fail(QSA_ERR_ARG, "%s: NULL q, kq, vq, ksc or vsc", fn);
    if (!aligned(q, 16) || !aligned(kq, 16) || !aligned(vq, 16) || !aligned(ksc, 8) || !aligned(vsc, 8) ||
        (ids && !aligned(ids, 4)))
        return fail(QSA_ERR_ARG, "%s: misaligned pointer (q, kq, vq: 16 B; ksc, vsc: 8 B; ids: 4 B)", fn);
    const int64_t C = ids ? ids_stride / QSA_CHUNK : ((int64_t)pos0 + T + QSA_CHUNK - 1) / QSA_CHUNK;
    if (C > INT32_MAX)
        return fail(QSA_ERR_ARG, "%s: too many chunks", fn);
    a = qsa::AttnArgs{};
    a.q = static_cast<const _Float16 *>(q);
    a.kq = kq;
    a.vq = vq;
    a.ksc = static_cast<const uint16_t *>(ksc);
    a.vsc = static_cast<const uint16_t *>(vsc);
    a.ids = ids;
    a.ids_stride = ids ? ids_stride : 0;
    a.n_cells = n_cells;
    a.pos0 = pos0;
    a.T = T;
    a.H = H;
    a.C = (int32_t)C;
    a.scale = scale;
    return QSA_OK;
}

} // namespace

extern "C" {

qsa_status qsa_attn(const void *q, const int8_t *kq, const int8_t *vq,
                    const void *ksc, const void *vsc, int32_t n_cells,
                    const int32_t *ids, int32_t ids_stride,
                    int32_t pos0, int32_t T, int32_t H, int32_t D,
                    float scale, void *part, void *stream)
{
    qsa::AttnArgs a;
    bool noop;
    qsa_status st = check_attn("qsa_attn", q, kq, vq, ksc, vsc, n_cells, ids, ids_stride, pos0, T, H, D, scale,
                               a, &noop);
    if (st != QSA_OK)
        return st;
    if (noop)
        return ok();
    if (!part)
        return fail(QSA_ERR_ARG, "qsa_attn: NULL part");
    if (!aligned(part, 256))
        return fail(QSA_ERR_ARG, "qsa_attn: misaligned part (256 B)");
    const int64_t n_blocks = (int64_t)a.C * T;   // one wave per (chunk, token)
    const int64_t per_xcd = (n_blocks + 7) / 8;
    if (per_xcd * 8 > INT32_MAX)
        return fail(QSA_ERR_ARG, "qsa_attn: T * chunks too large for one launch");
    st = check_device();
    if (st != QSA_OK)
        return st;
    size_t o_off, m_off, l_off;
    qsa::part_layout(T, H, D, a.C, &o_off, &m_off, &l_off, nullptr);
    char *pb = static_cast<char *>(part);
    a.o = reinterpret_cast<float *>(pb + o_off);
    a.m = reinterpret_cast<float *>(pb + m_off);
    a.l = reinterpret_cast<float *>(pb + l_off);
    a.n_blocks = (int32_t)n_blocks;
    a.blocks_per_xcd = (int32_t)per_xcd;
    a.nt_records = (int64_t)T * a.C * H * D * (int64_t)sizeof(float) > qsa::kNontemporalRecordBytes;
    if (!ids)   // implicit rows: blocks of (token, head) rows share each chunk's cells
        return launched(qsa::launch_attn_tile(a, static_cast<hipStream_t>(stream)), "qsa_attn");
    return launched(qsa::launch_attn(a, static_cast<hipStream_t>(stream)), "qsa_attn");
}

} // extern "C"

namespace {

qsa_status attn_merge_impl(const char *fn, const void *q, const int8_t *kq, const int8_t *vq, const void *ksc,
                           const void *vsc, int32_t n_cells, const int32_t *ids, int32_t ids_stride, int32_t pos0,
                           int32_t T, int32_t H, int32_t D, float scale, const float *gate, void *out, float *sums16,
                           bool gated, void *stream)
{
    qsa::AttnArgs a;
    bool noop;
    qsa_status st = check_attn(fn, q, kq, vq, ksc, vsc, n_cells, ids, ids_stride, pos0, T, H, D, scale, a, &noop);
    if (st != QSA_OK)
        return st;
    if (noop)
        return ok();
    if (!out)
        return fail(QSA_ERR_ARG, "%s: NULL out", fn);
    if (!aligned(out, 16))
        return fail(QSA_ERR_ARG, "%s: misaligned out (16 B)", fn);
    if (gated && !gate)
        return fail(QSA_ERR_ARG, "%s: NULL gate", fn);
    if ((gate && !aligned(gate, 16)) || (sums16 && !aligned(sums16, 4)))
        return fail(QSA_ERR_ARG, "%s: misaligned gate (16 B) or sums16 (4 B)", fn);
    st = check_device();
    if (st != QSA_OK)
        return st;
    a.out = static_cast<_Float16 *>(out);
    a.gate = gate;
    a.sums = sums16;
    a.n_blocks = T;
    a.blocks_per_xcd = (T + 7) / 8;
    if (!ids)   // implicit rows: blocks of (token, head) rows share each chunk's cells
        return launched(qsa::launch_attn_merge_tile(a, static_cast<hipStream_t>(stream)), fn);
    return launched(qsa::launch_attn_merge(a, static_cast<hipStream_t>(stream)), fn);
}

qsa_status merge_impl(const char *fn, const void *part, int32_t n_chunks, int32_t T, int32_t H, int32_t D,
                      const float *gate, void *out, float *sums16, bool gated, void *stream)
{
    if (T < 0 || n_chunks < 0)
        return fail(QSA_ERR_ARG, "%s: negative T (%d) or n_chunks (%d)", fn, T, n_chunks);
    if (H < 1)
        return fail(QSA_ERR_ARG, "%s: H must be >= 1 (got %d)", fn, H);
    if (H > qsa::kMaxHeads)
        return fail(QSA_ERR_UNSUPPORTED, "%s: at most %d heads (got %d)", fn, qsa::kMaxHeads, H);
    if (D != qsa::kD)
        return fail(QSA_ERR_UNSUPPORTED, "%s: head dim %d not implemented (only %d)", fn, D, qsa::kD);
    if (T == 0)
        return ok();
    if (!part || !out)
        return fail(QSA_ERR_ARG, "%s: NULL part or out", fn);
    if (gated && !gate)
        return fail(QSA_ERR_ARG, "%s: NULL gate", fn);
    if (!aligned(part, 256) || !aligned(out, 16))
        return fail(QSA_ERR_ARG, "%s: misaligned pointer (part: 256 B; out: 16 B)", fn);
    if ((gate && !aligned(gate, 16)) || (sums16 && !aligned(sums16, 4)))
        return fail(QSA_ERR_ARG, "%s: misaligned gate (16 B) or sums16 (4 B)", fn);
    if (((int64_t)T * H + 3) / 4 > INT32_MAX)
        return fail(QSA_ERR_ARG, "%s: T * H too large for one launch", fn);
    qsa_status st = check_device();
    if (st != QSA_OK)
        return st;
    size_t o_off, m_off, l_off;
    qsa::part_layout(T, H, D, n_chunks, &o_off, &m_off, &l_off, nullptr);
    const char *pb = static_cast<const char *>(part);
    qsa::MergeArgs a;
    a.o = reinterpret_cast<const float *>(pb + o_off);
    a.m = reinterpret_cast<const float *>(pb + m_off);
    a.l = reinterpret_cast<const float *>(pb + l_off);
    a.C = n_chunks;
    a.T = T;
    a.H = H;
    a.out = static_cast<_Float16 *>(out);
    a.gate = gate;
    a.sums = sums16;
    return launched(qsa::launch_merge(a, static_cast<hipStream_t>(stream)), fn);
}

} // namespace

extern "C" {

qsa_status qsa_attn_merge(const void *q, const int8_t *kq, const int8_t *vq,
                          const void *ksc, const void *vsc, int32_t n_cells,
                          const int32_t *ids, int32_t ids_stride,
                          int32_t pos0, int32_t T, int32_t H, int32_t D,
                          float scale, void *out, void *stream)
{
    return attn_merge_impl("qsa_attn_merge", q, kq, vq, ksc, vsc, n_cells, ids, ids_stride, pos0, T, H, D, scale,
                           nullptr, out, nullptr, false, stream);
}

qsa_status qsa_attn_merge_gated(const void *q, const int8_t *kq, const int8_t *vq,
                                const void *ksc, const void *vsc, int32_t n_cells,
                                const int32_t *ids, int32_t ids_stride,
                                int32_t pos0, int32_t T, int32_t H, int32_t D,
                                float scale, const float *gate, void *out, float *sums16, void *stream)
{
    return attn_merge_impl("qsa_attn_merge_gated", q, kq, vq, ksc, vsc, n_cells, ids, ids_stride, pos0, T, H, D,
                           scale, gate, out, sums16, true, stream);
}

qsa_status qsa_merge(const void *part, int32_t n_chunks, int32_t T, int32_t H, int32_t D,
                     void *out, void *stream)
{
    return merge_impl("qsa_merge", part, n_chunks, T, H, D, nullptr, out, nullptr, false, stream);
}

qsa_status qsa_merge_gated(const void *part, int32_t n_chunks, int32_t T, int32_t H, int32_t D,
                           const float *gate, void *out, float *sums16, void *stream)
{
    return merge_impl("qsa_merge_gated", part, n_chunks, T, H, D, gate, out, sums16, true, stream);
}

namespace {

qsa_status score_impl(const char *fn, const float *q, const float *k, int32_t n_cells, int32_t pos0, int32_t T,
                      int32_t Hs, int32_t D, float scale, float dead, float *scores, int64_t row_stride,
                      bool with_ws, void *ws, int64_t ws_bytes, void *stream)
{
    if (T < 0 || pos0 < 0 || n_cells < 0)
        return fail(QSA_ERR_ARG, "%s: negative T (%d), pos0 (%d) or n_cells (%d)", fn, T, pos0, n_cells);
    if (Hs < 1)
        return fail(QSA_ERR_ARG, "%s: Hs must be >= 1 (got %d)", fn, Hs);
    if (Hs > qsa::kMaxHeads)
        return fail(QSA_ERR_UNSUPPORTED, "%s: at most %d heads (got %d)", fn, qsa::kMaxHeads, Hs);
    if (D != qsa::kD)
        return fail(QSA_ERR_UNSUPPORTED, "%s: head dim %d not implemented (only %d)", fn, D, qsa::kD);
    if ((int64_t)pos0 + T > INT32_MAX)
        return fail(QSA_ERR_ARG, "%s: pos0 + T overflows int32", fn);
    if ((int64_t)n_cells < (int64_t)pos0 + T)
        return fail(QSA_ERR_ARG, "%s: n_cells (%d) < pos0 + T (%lld)", fn, n_cells, (long long)pos0 + T);
    if (row_stride < (int64_t)pos0 + T)
        return fail(QSA_ERR_ARG, "%s: row_stride (%lld) < pos0 + T (%lld)", fn, (long long)row_stride,
                    (long long)pos0 + T);
    if (((int64_t)T + 63) / 64 > 65535)
        return fail(QSA_ERR_ARG, "%s: T too large for one launch", fn);
    if (T == 0)
        return ok();
    if (!q || !k || !scores)
        return fail(QSA_ERR_ARG, "%s: NULL q, k or scores", fn);
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(scores, 4))
        return fail(QSA_ERR_ARG, "%s: misaligned pointer (q, k: 16 B; scores: 4 B)", fn);
    if (with_ws) {
        if (ws_bytes < qsa::score_ws_bytes(T))
            return fail(QSA_ERR_ARG, "%s: workspace of %lld bytes, %lld needed for %d rows", fn, (long long)ws_bytes,
                        (long long)qsa::score_ws_bytes(T), T);
        if (!ws)
            return fail(QSA_ERR_ARG, "%s: NULL workspace", fn);
        if (!aligned(ws, 16))
            return fail(QSA_ERR_ARG, "%s: misaligned workspace (16 B)", fn);
    }
    qsa_status st = check_device();
    if (st != QSA_OK)
        return st;
    qsa::ScoreArgs a;
    a.q = q;
    a.k = k;
    a.n_cells = n_cells;
    a.pos0 = pos0;
    a.T = T;
    a.Hs = Hs;
    a.scale = scale;
    a.dead = dead;
    a.scores = scores;
    a.row_stride = row_stride;
    return launched(qsa::launch_score(a, with_ws ? ws : nullptr, static_cast<hipStream_t>(stream)), fn);
}

} // namespace

qsa_status qsa_score(const float *q, const float *k, int32_t n_cells, int32_t pos0,
                     int32_t T, int32_t Hs, int32_t D, float scale, float dead,
                     float *scores, int64_t row_stride, void *stream)
{
    return score_impl("qsa_score", q, k, n_cells, pos0, T, Hs, D, scale, dead, scores, row_stride, false, nullptr, 0,
                      stream);
}

int64_t qsa_score_ws_bytes(int32_t T)
{
    return qsa::score_ws_bytes(T);
}

qsa_status qsa_score_ws(const float *q, const float *k, int32_t n_cells, int32_t pos0,
                        int32_t T, int32_t Hs, int32_t D, float scale, float dead,
                        float *scores, int64_t row_stride, void *workspace, int64_t ws_bytes, void *stream)
{
    return score_impl("qsa_score_ws", q, k, n_cells, pos0, T, Hs, D, scale, dead, scores, row_stride, true, workspace,
                      ws_bytes, stream);
}

qsa_status qsa_quant_append(const float *k, const float *v, int32_t n_rows, int32_t D,
                            int8_t *kq, int8_t *vq, void *ksc, void *vsc,
                            int32_t cell0, int32_t n_cells_cap, void *stream)
{
    if (n_rows < 0 || cell0 < 0 || n_cells_cap < 0)
        return fail(QSA_ERR_ARG, "qsa_quant_append: negative n_rows (%d), cell0 (%d) or n_cells_cap (%d)", n_rows,
                    cell0, n_cells_cap);
    if (D != qsa::kD)
        return fail(QSA_ERR_UNSUPPORTED, "qsa_quant_append: head dim %d not implemented (only %d)", D, qsa::kD);
    if ((int64_t)cell0 + n_rows > n_cells_cap)
        return fail(QSA_ERR_ARG, "qsa_quant_append: cells %d .. %lld past the cache capacity %d", cell0,
                    (long long)cell0 + n_rows - 1, n_cells_cap);
    if (n_rows == 0)
        return ok();
    if (!k || !v || !kq || !vq || !ksc || !vsc)
        return fail(QSA_ERR_ARG, "qsa_quant_append: NULL k, v, kq, vq, ksc or vsc");
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(kq, 8) || !aligned(vq, 8) || !aligned(ksc, 8) ||
        !aligned(vsc, 8))
        return fail(QSA_ERR_ARG, "qsa_quant_append: misaligned pointer (k, v: 16 B; kq, vq, ksc, vsc: 8 B)");
    qsa_status st = check_device();
    if (st != QSA_OK)
        return st;
    qsa::QuantArgs a;
    a.k = k;
    a.v = v;
    a.kq = kq;
    a.vq = vq;
    a.ksc = static_cast<uint16_t *>(ksc);
    a.vsc = static_cast<uint16_t *>(vsc);
    a.n_rows = n_rows;
    a.cell0 = cell0;
    return launched(qsa::launch_quant(a, static_cast<hipStream_t>(stream)), "qsa_quant_append");
}

qsa_status qsa_select(const float *scores, int64_t row_stride, int32_t pos0, int32_t T, int32_t K,
                      int32_t *ids, int32_t ids_stride, void *stream)
{
    if (T < 0 || pos0 < 0)
        return fail(QSA_ERR_ARG, "qsa_select: negative T (%d) or pos0 (%d)", T, pos0);
    if (K < 1)
        return fail(QSA_ERR_ARG, "qsa_select: K must be >= 1 (got %d)", K);
    if ((int64_t)pos0 + T > qsa::kMaxCells)
        return fail(QSA_ERR_UNSUPPORTED, "qsa_select: rows of at most %d cells (pos0 + T = %lld)",
                    qsa::kMaxCells, (long long)pos0 + T);
    if (row_stride < (int64_t)pos0 + T)
        return fail(QSA_ERR_ARG, "qsa_select: row_stride (%lld) < pos0 + T (%lld)", (long long)row_stride,
                    (long long)pos0 + T);
    const int64_t longest = (int64_t)pos0 + T < K ? (int64_t)pos0 + T : K;
    if (ids_stride <= 0 || ids_stride % QSA_CHUNK != 0 || ids_stride < longest)
        return fail(QSA_ERR_ARG, "qsa_select: ids_stride (%d) must be a positive multiple of %d holding min(K, pos0 + T) = %lld ids",
                    ids_stride, QSA_CHUNK, (long long)longest);
    if (T == 0)
        return ok();
    if (!scores || !ids)
        return fail(QSA_ERR_ARG, "qsa_select: NULL scores or ids");
    if (!aligned(scores, 4) || !aligned(ids, 4))
        return fail(QSA_ERR_ARG, "qsa_select: misaligned pointer (scores, ids: 4 B)");
    qsa_status st = check_device();
    if (st != QSA_OK)
        return st;
    qsa::SelectArgs a;
    a.scores = scores;
    a.row_stride = row_stride;
    a.pos0 = pos0;
    a.T = T;
    a.K = K;
    a.ids = ids;
    a.ids_stride = ids_stride;
    return launched(qsa::launch_select(a, static_cast<hipStream_t>(stream)), "qsa_select");
}

} // extern "C"

// ---- split path through a static workspace (qsa_split_merge_static) ---------
//
// For callers that cannot allocate: the chunk records go to `scratch`, a
// file-scope device array of QSA_STATIC_PART_BYTES that every GPU holds from
// the library's load until the process ends. Host code never passes the
// array's name to a kernel or a copy (on the host it is only a stand-in): the
// first call on a device, with that device current, asks the runtime for the
// array's device address on that device and keeps it. Nothing in it needs to
// start at zero: qsa_attn writes every record's (m, l) and every non-empty
// record's o, and the merge reads o only for non-empty records.

namespace qsa {
__device__ __align__(256) uint8_t scratch[QSA_STATIC_PART_BYTES];
} // namespace qsa

namespace {

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];    // device address of `scratch` on each device, once known

qsa_status static_workspace(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(QSA_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(QSA_ERR_UNSUPPORTED, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(qsa::scratch));
        if (e != hipSuccess || !p)
            return fail(QSA_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return QSA_OK;
}

} // namespace

extern "C" {

qsa_status qsa_split_merge_static(const void *q, const int8_t *kq, const int8_t *vq,
                                  const void *ksc, const void *vsc, int32_t n_cells,
                                  const int32_t *ids, int32_t ids_stride,
                                  int32_t pos0, int32_t T, int32_t H, int32_t D,
                                  float scale, void *out, void *stream)
{
    const char *fn = "qsa_split_merge_static";
    qsa::AttnArgs a;
    bool noop;
    qsa_status st = check_attn(fn, q, kq, vq, ksc, vsc, n_cells, ids, ids_stride, pos0, T, H, D, scale, a, &noop);
    if (st != QSA_OK)
        return st;
    if (noop)
        return ok();
    if (!out)
        return fail(QSA_ERR_ARG, "%s: NULL out", fn);
    if (!aligned(out, 16))
        return fail(QSA_ERR_ARG, "%s: misaligned out (16 B)", fn);
    size_t o_off, m_off, l_off, total;
    qsa::part_layout(T, H, D, a.C, &o_off, &m_off, &l_off, &total);
    if (total > QSA_STATIC_PART_BYTES)
        return fail(QSA_ERR_ARG, "%s: the chunk records of this call need %zu bytes, more than the static "
                    "workspace's %zu (T * chunks * H <= about %zu records of head dim %d)", fn, total,
                    (size_t)QSA_STATIC_PART_BYTES, (size_t)QSA_STATIC_PART_BYTES / (4 * (qsa::kD + 2)), qsa::kD);
    const int64_t n_blocks = (int64_t)a.C * T;
    const int64_t per_xcd = (n_blocks + 7) / 8;
    st = check_device();
    if (st != QSA_OK)
        return st;
    void *ws = nullptr;
    st = static_workspace(&ws);
    if (st != QSA_OK)
        return st;
    char *pb = static_cast<char *>(ws);
    a.o = reinterpret_cast<float *>(pb + o_off);
    a.m = reinterpret_cast<float *>(pb + m_off);
    a.l = reinterpret_cast<float *>(pb + l_off);
    a.n_blocks = (int32_t)n_blocks;
    a.blocks_per_xcd = (int32_t)per_xcd;
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = launched(ids ? qsa::launch_attn(a, s) : qsa::launch_attn_tile(a, s), fn);
    if (st != QSA_OK)
        return st;
    qsa::MergeArgs mg;
    mg.o = a.o;
    mg.m = a.m;
    mg.l = a.l;
    mg.C = a.C;
    mg.T = T;
    mg.H = H;
    mg.out = static_cast<_Float16 *>(out);
    mg.gate = nullptr;
    mg.sums = nullptr;
    return launched(qsa::launch_merge(mg, s), fn);
}

} // extern "C"
