/*
 * sv.h — C ABI of the speculative-sampling verify library (libsv.so, gfx950).
 *
 * The operation (web pages, cited by title and section):
 *   - deniz.in, "Üç düzeltmeden sonra Qwen3.5 ve Qwen3.6 MTP head, Apple
 *     Silicon'da 1.4 kata ulaştı", section "Örnekleme altında doğrulama
 *     yanlıştı": a greedy row accepts a draft token iff it equals the target
 *     argmax; a sampling row accepts draft token x with probability
 *     min(1, p(x)/q(x)) and, on rejection, draws a replacement from the
 *     clipped and rescaled difference (p - q)+.
 *   - same page, section "Kesme her iki tarafta eşleşmek zorunda": target and
 *     draft distributions get the same temperature / top_k / top_p treatment.
 *   - "MTPLX：让模型用上自己的 MTP 头——Apple Silicon 上的原生投机解码",
 *     section 3.3: the same accept / residual rule, which leaves the output
 *     law equal to plain decoding from the target.
 *   - tinycto.tv, "Spekülatif Kod Çözme (Speculative Decoding)…", section
 *     "1. Temel Çalışma Mekanizması": drafts are tested in order and the first
 *     rejection ends the row; section "Yaygın Yanılgılar": target and draft
 *     share one vocabulary (one V here).
 *   - "Apple Silikon İçin Cihaz Üstü Çıkarımı Optimize Etme", section
 *     "Kelime parçacığı devrini GPU üzerinde tutun": the chosen token stays in
 *     device memory for the next step; this library never copies results to
 *     the host.
 *
 * Readings of points the pages leave open (the oracle uses the same ones):
 *   temperature first, then top_k (ranking by logit descending, token id
 *   ascending), renormalise, then the top_p walk over the renormalised top_k
 *   keeping every token whose preceding mass is < top_p (top_p >= 1: no cut),
 *   renormalise.  top_k <= 0 or >= V disables top_k.  T == 0 is a greedy row.
 *   Accept iff u < a (strict).  The inverse CDF of the final draw walks token
 *   ids in ascending order and returns the first id with u*W < running sum.
 *   Residual mass W <= 0 falls back to p.  When all L drafts are accepted a
 *   bonus token is drawn from the target row at position L.
 */
#ifndef SV_H
#define SV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest top_k served by the in-register top-k path.  Rows with
 * SV_MAX_TOP_K < top_k < V are reported as unsupported (accept length -2). */
#define SV_MAX_TOP_K 64

enum { SV_F32 = 0, SV_BF16 = 1 };

enum {
    SV_OK = 0,
    SV_EINVAL = -1,     /* null required pointer, bad size, dtype or stride   */
    SV_EWORKSPACE = -2, /* workspace missing or smaller than sv_workspace_bytes */
    SV_EHIP = -3,       /* a HIP launch failed; sv_strerror gives the reason   */
    SV_ESCRATCH = -4    /* sv_verify_noalloc: the shape needs more scratch than
                           SV_NOALLOC_SCRATCH_BYTES                            */
};

/* Size of the static device scratch of sv_verify_noalloc (per GPU). */
#define SV_NOALLOC_SCRATCH_BYTES (128ull << 20)

/* Per-row sampler parameters, 16 bytes, one per batch row (device memory).
 * temperature: 0 = greedy, > 0 finite = sampling; anything else is a row
 * error.  top_k: <= 0 or >= V disables.  top_p: > 0; >= 1 disables. */
typedef struct {
    float temperature;
    int32_t top_k;
    float top_p;
    int32_t reserved;
} sv_sampler_params;

/* Host-side descriptor of shapes, layout, stream and scratch. */
typedef struct {
    int32_t batch;     /* B >= 1                                              */
    int32_t max_draft; /* 0 <= K <= 1024 (drafted positions per row); with
                          K = 0 a step only draws one token per row       */
    int32_t vocab;     /* V >= 2, shared by target and draft                  */
    int32_t dtype;     /* SV_F32 or SV_BF16, same for both logits tensors     */
    int64_t target_row_stride; /* elements between consecutive (b, k) rows; 0 => V */
    int64_t draft_row_stride;  /* same for the draft tensor; 0 => V             */
    void* stream;              /* hipStream_t to enqueue on; NULL => default    */
    void* workspace;           /* caller-owned device scratch                   */
    size_t workspace_bytes;    /* >= sv_workspace_bytes(...)                    */
    double* diag; /* optional device [B][K+1][4] fp64, NULL => not written.
                     Slots 0..K-1: (p(x), q(x), a, |u - a|) of each evaluated
                     accept test; slot K: (probability of the drawn token under
                     the final distribution, lower CDF edge, upper CDF edge,
                     margin of u to the nearer edge).  NaN where not evaluated
                     and on greedy rows. */
    int32_t step_mode; /* SV_STEP_AUTO (0): a dense step for small batches
                          (2 B (K+1) <= 1024 rows to stream), position by
                          position otherwise; SV_STEP_POSITIONS (1): always
                          position by position; SV_STEP_DENSE (2): dense
                          (SV_EINVAL when the batch is not small).  The
                          results are the same in every mode. */
    int32_t reserved;  /* 0 */
} sv_config;

enum { SV_STEP_AUTO = 0, SV_STEP_POSITIONS = 1, SV_STEP_DENSE = 2 };

/* Bytes of device workspace sv_verify needs for this shape.  Pure function
 * of its arguments; 0 on invalid arguments. */
size_t sv_workspace_bytes(int32_t batch, int32_t max_draft, int32_t vocab, int32_t dtype);

/*
 * Enqueue one verify step on cfg->stream.  All pointers except cfg are
 * device pointers owned by the caller; inputs must stay alive and unchanged
 * until the stream work completes, outputs must not alias inputs.  The call
 * never synchronises, never reads device memory on the host and keeps no
 * pointer after it returns.  Calls that share a workspace must be ordered on
 * one stream.
 *
 *   target_logits  [B][K+1] rows of V logits (row r at r*target_row_stride)
 *   draft_logits   [B][K]   rows of V logits (row r at r*draft_row_stride);
 *                  may be NULL when K = 0
 *   draft_tokens   [B][K] int32; only the first draft_len[b] are read; may be
 *                  NULL when K = 0
 *   draft_len      [B] int32 in [0, K], or NULL (= K for every row)
 *   sampler_params [B] sv_sampler_params
 *   uniforms       [B][K+1] fp32 in [0, 1): column k is the accept test of
 *                  draft position k, column K the single final draw
 *   out_tokens     [B][K+1] int32: accepted drafts, then the resampled /
 *                  bonus / argmax token, then -1 padding
 *   out_accept_len [B] int32: drafts accepted; -1 for a row with invalid
 *                  data (bad params, draft_len, token id, or a distribution
 *                  with no finite logit), -2 for a row this build does not
 *                  serve (SV_MAX_TOP_K < top_k < V); such rows get tokens -1.
 *
 * Returns SV_OK once the work is enqueued, or a negative SV_E* code (nothing
 * is enqueued then).  Identical inputs give bitwise-identical outputs.
 */
int sv_verify(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
              const int32_t* draft_len, const sv_sampler_params* sampler_params,
              const float* uniforms, int32_t* out_tokens, int32_t* out_accept_len,
              const sv_config* cfg);

/*
 * Same as sv_verify, and additionally records events[i] (hipEvent_t, created
 * by the caller) on cfg->stream just before kernel launch i of the step and
 * events[sv_launch_count(B, K, step_mode)] after the last one, so the caller
 * can time each kernel with hipEventElapsedTime.  n_events must be
 * >= sv_launch_count(B, K, step_mode) + 1.
 * For measuring kernels against the sustainable read rate of the part, the
 * method of "Apple Silikon İçin Cihaz Üstü Çıkarımı Optimize Etme", section
 * "Daha fazla optimizasyonun sınırları".
 */
int sv_verify_profiled(const void* target_logits, const void* draft_logits,
                       const int32_t* draft_tokens, const int32_t* draft_len,
                       const sv_sampler_params* sampler_params, const float* uniforms,
                       int32_t* out_tokens, int32_t* out_accept_len, const sv_config* cfg,
                       void* const* events, int32_t n_events);

/*
 * Tree / multi-candidate verify: draft heads that propose several candidate
 * tokens per position (tinycto.tv "Spekülatif Kod Çözme (Speculative
 * Decoding)…", question "Medusa / Eagle spekülatif taslak mekanizması nedir?";
 * the pages give no checking rule).  Reading: the candidates at a node are
 * drawn independently from the draft distribution q there, and the node's
 * children are tested in ascending node order by recursive rejection, child
 * x against the residual r left by the children rejected before it
 * (r = p at first, r <- (r - q)+ normalised after each rejection, unchanged
 * when that has no mass), accepting with min(1, r(x)/q(x)) (q(x) = 0: accept
 * iff r(x) > 0).  An accepted child becomes the current node; when every
 * child is rejected, or the node has none, the final token is drawn from r
 * by the inverse CDF in ascending token id.  Greedy rows take the first child
 * whose token is the target argmax.  With one child per node this is
 * sv_verify exactly (same arguments, parents[c-1] = c - 1).
 *
 * Node 0 is the committed context; nodes 1..K are candidates.
 *   target_logits  [B][K+1] rows: row v = the target's logits after node v
 *   draft_logits   [B][K] rows: row v = the draft's logits at node v (its
 *                  children were drawn from them); may be NULL when K = 0
 *   node_tokens    [B][K] int32: entry c-1 = candidate token of node c
 *   node_parents   [B][K] int32: entry c-1 = parent of node c, in [0, c)
 *   n_cand         [B] int32 in [0, K]: nodes 1..n_cand[b] are used; NULL = K
 *   sampler_params [B]; the same temperature / top_k / top_p on both sides
 *   uniforms       [B][K+1] fp32 in [0, 1): column c-1 is node c's test,
 *                  column K the final draw
 *   out_tokens     [B][K+1] int32: the accepted path's tokens, then the drawn
 *                  token (the argmax on greedy rows), then -1
 *   out_accept_len [B] int32: length of the accepted path; -1 invalid row
 *                  (as sv_verify, and: a parent outside [0, c), a node deeper
 *                  than max_depth, a node with more than max_children
 *                  children), -2 unsupported top_k
 *   out_path       [B][K+1] int32 or NULL: the accepted nodes, -1 padded
 *   max_depth      0 <= max_depth <= K: levels the call walks
 *   max_children   1 <= max_children <= 64 (K > 0): children per node; a
 *                  full-vocabulary row (top_k off) needs one pass over the
 *                  node's two rows per rejected child beyond the first
 *   cfg            as for sv_verify; diag, if set, is [B][K+1][4] fp64 with
 *                  slot c-1 = (r(x), q(x), a, |u - a|) of node c's test and
 *                  slot K = the final draw, NaN elsewhere.
 * Returns SV_OK once enqueued, SV_EINVAL (also for max_depth / max_children
 * out of range), SV_EWORKSPACE, SV_EHIP.  Ownership, ordering and
 * determinism as for sv_verify.
 */
int sv_verify_tree(const void* target_logits, const void* draft_logits,
                   const int32_t* node_tokens, const int32_t* node_parents,
                   const int32_t* n_cand, const sv_sampler_params* sampler_params,
                   const float* uniforms, int32_t* out_tokens, int32_t* out_accept_len,
                   int32_t* out_path, int32_t max_depth, int32_t max_children,
                   const sv_config* cfg);

/*
 * sv_verify for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, semantics and results as sv_verify, except that cfg->workspace
 * and cfg->workspace_bytes are ignored: the step's scratch lives in a static
 * device array of SV_NOALLOC_SCRATCH_BYTES (128 MiB) that the library holds on
 * every GPU it runs on until the process ends.  The call itself allocates
 * nothing (no hipMalloc, no hipFree; the array's device address is looked up
 * once per device, on the first call there).  The caller still passes every
 * input and output buffer.
 *   Returns SV_ESCRATCH when sv_workspace_bytes(B, K, V, dtype) exceeds
 *   SV_NOALLOC_SCRATCH_BYTES (nothing is enqueued), otherwise as sv_verify.
 *   Every call on one GPU shares that GPU's array, which keeps the last
 *   call's contents: calls that may overlap on one GPU (different streams,
 *   or host threads without ordering) race and must not be made.
 */
int sv_verify_noalloc(const void* target_logits, const void* draft_logits,
                      const int32_t* draft_tokens, const int32_t* draft_len,
                      const sv_sampler_params* sampler_params, const float* uniforms,
                      int32_t* out_tokens, int32_t* out_accept_len, const sv_config* cfg);

/* SV_NOALLOC_SCRATCH_BYTES, as built into the library. */
size_t sv_noalloc_scratch_bytes(void);

/*
 * Draw one token per row from one row of logits, with the temperature,
 * top_k / top_p truncation and inverse-CDF draw of the final draw of
 * sv_verify (it is sv_verify with K = 0: the bonus draw at position 0).
 * Uses: the draft model's own sampling step before a verify, which must
 * apply the same truncation as the target (deniz.in page, section "Kesme her
 * iki tarafta eşleşmek zorunda"), and plain decoding; the drawn ids stay in
 * device memory for the next step ("Apple Silikon İçin Cihaz Üstü Çıkarımı
 * Optimize Etme", section "Kelime parçacığı devrini GPU üzerinde tutun").
 *
 *   logits         [B] rows of V logits (row b at b*cfg->target_row_stride)
 *   sampler_params [B] sv_sampler_params
 *   uniforms       [B] fp32 in [0, 1)
 *   out_tokens     [B] int32: the drawn token (the argmax on greedy rows), -1
 *                  on a row whose status is not 0
 *   out_status     [B] int32 or NULL: 0, -1 invalid row, -2 unsupported top_k
 *   cfg            as for sv_verify; max_draft and draft_row_stride are
 *                  ignored; the workspace must hold
 *                  sv_workspace_bytes(B, 0, V, dtype) bytes; diag, if set, is
 *                  [B][1][4] (slot K = 0 of sv_verify's layout).
 * Same ownership, ordering, error and determinism rules as sv_verify.
 */
int sv_sample(const void* logits, const sv_sampler_params* sampler_params, const float* uniforms,
              int32_t* out_tokens, int32_t* out_status, const sv_config* cfg);

/*
 * Acceptance statistics of one draft position, per row: how often drafts
 * would be kept under the rejection test with matched truncation, under a
 * check that compares two independent draws, and under the rejection test
 * with the draft alone truncated or nothing truncated (deniz.in "Üç
 * düzeltmeden sonra Qwen3.5 ve Qwen3.6 MTP head…", sections "Örnekleme
 * altında doğrulama yanlıştı" and "Kesme her iki tarafta eşleşmek zorunda":
 * the rejection test's acceptance is the overlap of the two distributions).
 * With p, q the target and draft distributions of row b after temperature and
 * the row's top_k / top_p (as sv_verify forms them) and p~, q~ after
 * temperature only:
 *   out[b][0] = sum_i min(p_i, q_i)
 *   out[b][1] = sum_i p_i q_i
 *   out[b][2] = sum_i min(p~_i, q_i)
 *   out[b][3] = sum_i min(p~_i, q~_i)
 * On a greedy row (temperature 0) all four are 1 when the two argmaxes agree
 * and 0 otherwise; on a row with invalid parameters, an unsupported top_k or
 * no finite logit on either side they are NaN.  Sums are fp64 over fp32
 * exp2 terms (relative error about 1e-7).
 *
 *   target_logits  [B] rows of V logits (row b at b*cfg->target_row_stride)
 *   draft_logits   [B] rows of V logits (row b at b*cfg->draft_row_stride)
 *   sampler_params [B] sv_sampler_params
 *   out            [B][4] fp64, device
 *   cfg            batch, vocab, dtype, strides, stream, workspace (at least
 *                  sv_workspace_bytes(B, 1, V, dtype) bytes); max_draft and
 *                  diag are ignored.
 * Same ownership, ordering, error and determinism rules as sv_verify.
 */
int sv_accept_stats(const void* target_logits, const void* draft_logits,
                    const sv_sampler_params* sampler_params, double* out, const sv_config* cfg);

/*
 * Measurement aid, not part of the verify step: stream `bytes` bytes of
 * device memory once with the tiling of the verify step's row pass (16-byte
 * coalesced non-temporal loads, double-buffered tiles split evenly over one
 * resident wave of workgroups) and no work per element beyond a max, which
 * each workgroup folds into *out (device uint32; the caller zeroes it, the
 * value itself means nothing).  Its rate is the sustainable read rate the
 * row pass is measured against, the second denominator next to the HBM
 * peak, after "Apple Silikon İçin Cihaz Üstü Çıkarımı Optimize Etme",
 * section "Daha fazla optimizasyonun sınırları" (judge a kernel against what
 * a trivial read of the same bytes reaches on the part).
 *   data   device pointer, 16-byte aligned; bytes > 0, a multiple of 16
 *   stream hipStream_t, NULL => default stream
 * Returns SV_OK once enqueued, SV_EINVAL on bad arguments, SV_EHIP.
 */
int sv_stream_read(const void* data, size_t bytes, uint32_t* out, void* stream);

/* Number of kernel launches in one sv_verify step of B rows and max_draft K
 * in step mode `step_mode` (0 if B < 1, K is outside [0, 1024] or the mode is
 * not served for the shape), and the name of launch i ("plan", "rowpass",
 * "cut_decide", ...; NULL if out of range).  A dense step has one row pass
 * over every drafted position and one decision launch that walks the
 * positions.  Static strings, host only. */
int32_t sv_launch_count(int32_t batch, int32_t max_draft, int32_t step_mode);
const char* sv_launch_name(int32_t batch, int32_t max_draft, int32_t step_mode, int32_t i);

/* Static description of an error code (the last HIP error for SV_EHIP). */
const char* sv_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* SV_H */
