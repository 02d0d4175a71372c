/*
 * qsa.h -- C ABI of libqsa.so: explicit-selection attention over an int8 K/V
 * cache shared by all query heads, the merge of its chunk records, and causal
 * q.K scores, on AMD Instinct MI355X (gfx950).
 *
 * Every pointer argument is a DEVICE pointer to memory the caller owns. The
 * library allocates nothing, keeps no per-call state (qsa_split_merge_static's
 * static record array aside) and is safe to call from several host threads.
 * Each call validates its arguments on the host, enqueues its kernels on
 * `stream` (a hipStream_t; NULL means the null stream) and returns without
 * synchronising: inputs must stay alive, and outputs must not be read, until
 * the stream has passed the call. A call enqueues kernel launches only (no
 * memset, copy or host wait), so calls made while `stream` is being captured
 * go into the HIP graph, with the pointers and sizes of that call, and every
 * replay repeats them.
 *
 * Status codes:
 *   QSA_OK              success (also for T == 0, which enqueues nothing)
 *   QSA_ERR_ARG         a required pointer is NULL or misaligned, or a size is
 *                       negative or inconsistent; nothing was enqueued
 *   QSA_ERR_UNSUPPORTED a shape the library does not implement (D != 128, more
 *                       than 16 heads, more than 2^25 cached rows) or a device
 *                       that is not gfx950
 *   QSA_ERR_DEVICE      a HIP runtime call failed (message in qsa_last_error)
 *
 * Names follow the pages' notation: q, kq/vq, ksc/vsc, ids with -1 poison,
 * pos0, T and a softmax scale ("round 11 track b: qsa attention and score",
 * section "boundaries and provenance").
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QSA_OK = 0,
    QSA_ERR_ARG = 1,
    QSA_ERR_UNSUPPORTED = 2,
    QSA_ERR_DEVICE = 3
} qsa_status;

/* Symbols of the library; everything else in it is hidden. */
#define QSA_API __attribute__((visibility("default")))

/* Slots of an id row are processed in chunks of this many. */
#define QSA_CHUNK 64
/* Cached rows carry one fp16 scale per this many consecutive dims. */
#define QSA_GROUP 32

/*
 * qsa_attn -- chunk records of explicit-selection attention.
 *
 * Defined by "round 11 track b: qsa attention and score", section
 * "implementation and evaluator" (int8 K/V rows addressed by selected cell
 * ids, one scale per quarter of a row, a last chunk that may be partly filled,
 * empty slots that add nothing, and chunk partials that are stored before they
 * are merged), and by "round 5 track b: cached residual norms and fused mtp
 * attention", section "mtp attention" (chunks of 64 cells, each with its own
 * maximum and denominator; each V value read once per cell and shared by all
 * heads).
 *
 * For each query token t (cache position p = pos0 + t), each chunk k of its id
 * row (slots 64k .. 64k+63) and each head h < H, with the valid slots j of the
 * chunk (0 <= id < n_cells):
 *   k_d = kq[c][d] * ksc[c][d/32],  v_d = vq[c][d] * vsc[c][d/32]
 *   S_j = scale * sum_d q[t][h][d] * k_d
 *   m   = max_j S_j,  p_j = exp(S_j - m),  l = sum_j p_j,  o[d] = sum_j p_j v_d
 * and writes the record (m, l, o) to `part`. A chunk with no valid slot gets
 * m = -inf and l = +0, and its o is not written.
 *
 * q        fp16 [T][H][D], row-major, 16-byte aligned
 * kq, vq   int8 [n_cells][D], 16-byte aligned rows; pos0 + T <= n_cells <= 2^25
 * ksc, vsc fp16 [n_cells][D/32], finite and positive, 8-byte aligned
 * ids      int32 [T][ids_stride], -1 = poison. Any id outside [0, n_cells) is
 *          treated as poison and never dereferenced. ids_stride must be a
 *          positive multiple of 64; the row has C = ids_stride / 64 chunks.
 *          Selected ids are trusted to be causal (id <= p); duplicates count
 *          once per occurrence.
 *          ids == NULL selects implicit rows: slot j holds cell j when j <= p
 *          (else poison), with C = ceil((pos0 + T) / 64); ids_stride is ignored.
 * pos0     cache position of token 0 (>= 0); T query tokens (>= 0);
 *          n_cells >= pos0 + T (the cache holds every causal cell of the
 *          call), else QSA_ERR_ARG
 * H        query heads sharing the one K/V head, 1..16
 * D        head dim; the library implements D == 128 only
 * scale    softmax scale applied to every dot product
 * part     qsa_part_bytes(T, H, D, C) bytes, 256-byte aligned; laid out as
 *          o[T][C][H][D] fp32, then m[T][C][H] fp32, then l[T][C][H] fp32,
 *          each sub-array starting on a 256-byte boundary
 *          (qsa_part_offsets gives the byte offsets).
 */
QSA_API qsa_status qsa_attn(const void *q, const int8_t *kq, const int8_t *vq,
                    const void *ksc, const void *vsc, int32_t n_cells,
                    const int32_t *ids, int32_t ids_stride,
                    int32_t pos0, int32_t T, int32_t H, int32_t D,
                    float scale, void *part, void *stream);

/*
 * qsa_attn_merge -- explicit-selection attention and the merge of its chunk
 * records in one dispatch, with no partial records written to memory.
 *
 * Defined by "round 5 track b: cached residual norms and fused mtp attention",
 * section "mtp attention" (a decode kernel that keeps every chunk's
 * probabilities, maxima and denominators on chip and merges them before it
 * writes the output), applied here to any number of tokens and chunks.
 *
 * out[t][h][d] is the value qsa_attn followed by qsa_merge computes, up to
 * rounding: the chunk records are combined relative to the running largest
 * chunk maximum as they are produced. Arguments are those of qsa_attn, with
 *   out      fp16 [T][H][D], 16-byte aligned, in place of `part`.
 */
QSA_API qsa_status qsa_attn_merge(const void *q, const int8_t *kq, const int8_t *vq,
                          const void *ksc, const void *vsc, int32_t n_cells,
                          const int32_t *ids, int32_t ids_stride,
                          int32_t pos0, int32_t T, int32_t H, int32_t D,
                          float scale, void *out, void *stream);

/*
 * qsa_merge -- max-first merge of chunk records into fp16 output.
 *
 * Defined by "round 5 track b: cached residual norms and fused mtp attention",
 * sections "preflight / ownership" and "mtp attention" (chunk records are
 * combined relative to the largest chunk maximum). For each token t and head
 * h, over chunks with m_k != -inf:
 *   M = max_k m_k,  w_k = exp(m_k - M),  L = sum_k w_k l_k,
 *   out[t][h][d] = fp16_rne( sum_k w_k o_k[d] / L )
 * A (t, h) with no such chunk gets +0 in every dim; so does every row when
 * n_chunks is 0, and then part is not read. Records with m = -inf are
 * skipped and their o is never read.
 *
 * part     records written by qsa_attn with the same T, H, D and n_chunks
 * out      fp16 [T][H][D], 16-byte aligned
 */
QSA_API qsa_status qsa_merge(const void *part, int32_t n_chunks, int32_t T, int32_t H, int32_t D,
                     void *out, void *stream);

/*
 * qsa_merge_gated -- qsa_merge with the sigmoid output gate, and optionally
 * the per-16 sums of the written output.
 *
 * Defined by "round 5 track b: cached residual norms and fused mtp
 * attention", sections "preflight / ownership" (the merge keeps the sigmoid
 * gate and the per-16 sums), "mtp attention" and "actual verification" (gates
 * are fp32 inputs; per-16 sums are compared byte for byte). The pages give
 * neither the gate's shape nor the sums' tree; the readings taken are one
 * fp32 gate per output element and the exact sum of each block of 16 written
 * values:
 *   y     = sum_k w_k o_k[d] / L          (as qsa_merge; +0 for a row with no chunk)
 *   out   = fp16_rne(y / (1 + exp(-gate[t][h][d])))
 *   sums16[t][h][b] = fp32_rne(exact sum_{i<16} out[t][h][16b + i])   (if sums16 != NULL)
 * gate = +inf gives qsa_merge's output, gate = -inf a zero of y's sign, a
 * NaN gate a NaN output. The sums depend on no summation order.
 *
 * gate     fp32 [T][H][D], 16-byte aligned (required)
 * out      fp16 [T][H][D], 16-byte aligned
 * sums16   fp32 [T][H][D/16], 4-byte aligned, or NULL
 * Other arguments and errors are those of qsa_merge; a NULL gate is QSA_ERR_ARG.
 */
QSA_API qsa_status qsa_merge_gated(const void *part, int32_t n_chunks, int32_t T, int32_t H, int32_t D,
                           const float *gate, void *out, float *sums16, void *stream);

/*
 * qsa_attn_merge_gated -- qsa_attn_merge with the sigmoid output gate and the
 * optional per-16 sums, applied as in qsa_merge_gated. This is the pages'
 * fused decode kernel with its gate ("round 5 track b: cached residual norms
 * and fused mtp attention", sections "preflight / ownership" and "mtp
 * attention"). Arguments are those of qsa_attn_merge plus
 *   gate     fp32 [T][H][D], 16-byte aligned (required)
 *   sums16   fp32 [T][H][D/16], 4-byte aligned, or NULL
 */
QSA_API qsa_status qsa_attn_merge_gated(const void *q, const int8_t *kq, const int8_t *vq,
                                const void *ksc, const void *vsc, int32_t n_cells,
                                const int32_t *ids, int32_t ids_stride,
                                int32_t pos0, int32_t T, int32_t H, int32_t D,
                                float scale, const float *gate, void *out, float *sums16, void *stream);

/*
 * qsa_score -- fp32 q.K scores over causal cells with a dead-key tail.
 *
 * Defined by "round 11 track b: qsa attention and score", sections
 * "implementation and evaluator" (causal cells get scores, a single constant
 * marks the cells just past the causal edge, cells after those are not
 * written) and "score: valid negative result" (64-cell tiles, a sum over
 * heads). For row t (p = pos0 + t):
 *   scores[t][c] = scale * sum_{h < Hs} sum_d q[t][h][d] * k[c][d]   for c <= p
 *   scores[t][c] = dead       for p < c < min(64 * ceil((p + 1) / 64), row_stride)
 * and every later cell of the row is left untouched.
 *
 * Precision: each product is formed on the bf16 matrix cores from operands
 * split into two bf16 parts, so a score is within 4.6e-5 * |scale| *
 * sum_d |sum_h q[t][h][d]| * |k[c][d]| of the exact value; infinite operands
 * give infinite scores as in fp32, and operand parts below 2^-126 are lost.
 *
 * q        fp32 [T][Hs][D], 16-byte aligned;  Hs in 1..16
 * k        fp32 [n_cells][D], 16-byte aligned; n_cells >= pos0 + T
 * scores   fp32 [T][row_stride]; row_stride >= pos0 + T; 4-byte aligned.
 *          Fastest when every row starts 64-byte aligned (scores 64-byte
 *          aligned, row_stride a multiple of 16): the stores then bypass the
 *          caches. Other strides go through L2 instead, at about 1.3 times the
 *          time on the long-context workload.
 * D        the library implements D == 128 only
 */
QSA_API qsa_status qsa_score(const float *q, const float *k, int32_t n_cells, int32_t pos0,
                     int32_t T, int32_t Hs, int32_t D, float scale, float dead,
                     float *scores, int64_t row_stride, void *stream);

/*
 * qsa_score_ws_bytes -- bytes of the workspace qsa_score_ws takes for T rows:
 * 512 per row, for T rounded up to a multiple of 64 (0 when T <= 0).
 */
QSA_API int64_t qsa_score_ws_bytes(int32_t T);

/*
 * qsa_score_ws -- qsa_score with the head sum of q taken once per row.
 *
 * Computes what qsa_score computes (same definition, pages and sections as
 * above), to the same bits. qsa_score sums the heads of a 64-row block of q in
 * every workgroup that walks one of the block's column runs (16 such runs at
 * 1984 rows, pos0 = 30000). Here a first pass writes each row's head sum,
 * times scale and split into bf16 parts, to `workspace`, and the walk reads
 * it from there. The library takes that pass only where it pays: where q
 * (T * Hs * D * 4 bytes) is 4 MB or more and the workgroup order it picks has
 * every XCD read all of q. Otherwise the call runs as qsa_score does and
 * leaves the workspace untouched.
 *
 * workspace  device memory of ws_bytes >= qsa_score_ws_bytes(T) bytes,
 *            16-byte aligned, owned by the caller, overlapping neither q, k
 *            nor scores; its contents are overwritten and mean nothing to the
 *            caller afterwards. Calls that share a workspace must be ordered
 *            (one stream, or synchronised).
 * The other arguments, their layouts and the errors are those of qsa_score;
 * a NULL, short or misaligned workspace returns QSA_ERR_ARG before anything
 * is enqueued.
 */
QSA_API qsa_status qsa_score_ws(const float *q, const float *k, int32_t n_cells, int32_t pos0,
                        int32_t T, int32_t Hs, int32_t D, float scale, float dead,
                        float *scores, int64_t row_stride, void *workspace, int64_t ws_bytes,
                        void *stream);

/*
 * qsa_quant_append -- write fp32 K and V rows into the int8 cache with one
 * fp16 scale per 32-element group.
 *
 * The cache format is the one the attention reads ("round 11 track b: qsa
 * attention and score", section "implementation and evaluator": four scale
 * groups per K row); the pages' prep step writes it ("Round 36 Track C ...",
 * section "Summary & Decision") but does not print its rule. The rule taken,
 * for each row i and each 32-element group:
 *   a = max |x|,  s = fp16_rne(a / 127),
 *   code = clamp(rint(x / s), -127, 127), or 0 when s == 0,
 * with both quotients correctly rounded binary32 divisions and rint rounding
 * half to even. Row i of k lands in kq[cell0 + i] and ksc[cell0 + i], row i of
 * v in vq[cell0 + i] and vsc[cell0 + i]; no other cell is written. Inputs are
 * expected finite: a group whose a / 127 exceeds the fp16 range gets an
 * infinite scale and zero codes.
 *
 * k, v          fp32 [n_rows][D], 16-byte aligned (read only)
 * kq, vq        int8 [n_cells_cap][D], 8-byte aligned
 * ksc, vsc      fp16 [n_cells_cap][D/32], 8-byte aligned
 * cell0         first cell written; cell0 + n_rows <= n_cells_cap
 * D             the library implements D == 128 only
 * n_rows == 0 is a no-op. Bad arguments return QSA_ERR_ARG / QSA_ERR_UNSUPPORTED
 * before anything is enqueued.
 */
QSA_API qsa_status qsa_quant_append(const float *k, const float *v, int32_t n_rows, int32_t D,
                            int8_t *kq, int8_t *vq, void *ksc, void *vsc,
                            int32_t cell0, int32_t n_cells_cap, void *stream);

/*
 * qsa_select -- the ids each query row attends over, chosen from its causal
 * scores (the selection step before qsa_attn).
 *
 * The pages say that a row's selected ids are unique causal cells ("round 11
 * track b: qsa attention and score", section "boundaries and provenance") but
 * do not print how they are chosen. The rule taken is top-K: row t
 * (p = pos0 + t) selects the min(K, p + 1) cells c <= p with the largest
 * scores[t][c]; equal scores (-0 and +0 are equal) go to the smaller cell.
 * ids[t] receives them in ascending cell order, then -1 up to ids_stride.
 * Only cells 0 .. p of each score row are read. Scores must not be NaN.
 *
 * scores      fp32 [T][row_stride] (e.g. qsa_score's output); row_stride >= pos0 + T
 * ids         int32 [T][ids_stride]; ids_stride a multiple of 64 holding
 *             min(K, pos0 + T) ids, so the rows feed qsa_attn directly
 * The library supports pos0 + T <= 2^25 (QSA_ERR_UNSUPPORTED beyond); rows of
 * more than 32768 cells read their scores once per radix pass instead of once.
 */
QSA_API qsa_status qsa_select(const float *scores, int64_t row_stride, int32_t pos0, int32_t T, int32_t K,
                      int32_t *ids, int32_t ids_stride, void *stream);

/*
 * qsa_split_merge_static -- qsa_attn followed by qsa_merge, with the chunk
 * records kept in a workspace the library holds instead of one the caller
 * passes.
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the call
 * allocates nothing. The records go to a static device array of
 * QSA_STATIC_PART_BYTES that every GPU the library runs on holds until the
 * process ends. The result is that of qsa_attn + qsa_merge on the same
 * arguments (the same kernels run), written to out (fp16 [T][H][D], 16-byte
 * aligned); the other arguments are those of qsa_attn.
 *
 * Limit: qsa_part_bytes(T, H, D, C) <= QSA_STATIC_PART_BYTES (about 32,000
 * records of head dim 128: e.g. 64 tokens of 33 chunks at 12 heads, or any
 * decode window), else QSA_ERR_ARG with the sizes in qsa_last_error.
 * All calls on one GPU share that GPU's array: calls that overlap on one GPU
 * (from two streams or two host threads without ordering between them) race,
 * and their outputs are undefined. Calls ordered on one stream do not.
 */
#define QSA_STATIC_PART_BYTES (16u << 20)
QSA_API qsa_status qsa_split_merge_static(const void *q, const int8_t *kq, const int8_t *vq,
                                  const void *ksc, const void *vsc, int32_t n_cells,
                                  const int32_t *ids, int32_t ids_stride,
                                  int32_t pos0, int32_t T, int32_t H, int32_t D,
                                  float scale, void *out, void *stream);

/* Bytes of the `part` workspace for T tokens, H heads, head dim D, n_chunks chunks. */
QSA_API size_t qsa_part_bytes(int32_t T, int32_t H, int32_t D, int32_t n_chunks);

/* Byte offsets of the o, m and l sub-arrays inside `part` (any may be NULL). */
QSA_API void qsa_part_offsets(int32_t T, int32_t H, int32_t D, int32_t n_chunks,
                      size_t *o_off, size_t *m_off, size_t *l_off);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
QSA_API const char *qsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
