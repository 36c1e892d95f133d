/*
 * tb.h -- C ABI of libtb, the MI355X (gfx950) decode-time hot path of
 * TokenButler: a learned low-dimensional importance query, produced by a small
 * MLP at a producer layer, is dotted with the consumer layer's cached keys
 * projected into the same space; a fixed budget of the best-scoring tokens,
 * widened by neighbour fetching, is kept on top of an always-kept sink and a
 * local window; decode attention then reads only those tokens' K/V rows.
 * Around that path: the decode-step K/V append with batched key projection,
 * CPU-offload decoding (host-resident cache, HBM buffers) and the predictor's
 * distillation loss.
 *
 * Method source: "TokenButler" technical summary, sections "Core
 * architecture" (query prediction, key-cache projection, scoring),
 * "Inference strategy" (sink / local window / important buffers; batched key
 * projection; prediction interval; neighbour fetching), "Training"
 * (distillation loss) and "Significance" (the full cache is kept, only the
 * most relevant tokens are read).
 *
 * Conventions for every call
 *  - Pointers are DEVICE pointers unless stated, owned by the caller, to
 *    contiguous row-major arrays (innermost index last), 16-byte aligned.
 *    bf16 = bfloat16, fp16 = IEEE binary16, passed as `const void*`.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls only enqueue kernels on it; none synchronizes, none allocates.
 *  - Host-side arguments are validated before anything is enqueued; on any
 *    error the call returns a non-zero tb_status and enqueues nothing.
 *    Device-resident lengths are checked by the kernels where noted.
 *  - The library keeps no mutable global state (the one exception is the
 *    fixed scratch array of tb_sparse_decode_attn_noalloc); calls are
 *    reentrant. Calls that share a workspace must be ordered on one stream
 *    (they race otherwise).
 *  - Workspaces: size them with the matching *_workspace_bytes() query and
 *    zero-fill them once before first use (e.g. torch.zeros). A query
 *    returns 0 for sizes its call rejects (sizes are checked before any
 *    product is formed, so no size wraps around). Every call
 *    that takes a workspace leaves whatever must start at zero (the
 *    attention's arrival counters) at zero again when its kernels complete,
 *    so a workspace can be reused without clearing.
 */
#ifndef TB_H
#define TB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int tb_status;
#define TB_OK 0
#define TB_ERR_INVALID_ARGUMENT 1     /* null/misaligned pointer, bad size  */
#define TB_ERR_UNSUPPORTED_SHAPE 2    /* shape outside the compiled set      */
#define TB_ERR_WORKSPACE_TOO_SMALL 3
#define TB_ERR_HIP 4                  /* a HIP launch failed                 */

/* Neighbour-fetching modes of tb_select (low byte of `mode`). */
#define TB_NF_FILL 0     /* neighbours count against the fixed budget       */
#define TB_NF_DILATE 1   /* neighbours of the top-budget centres added beyond it */
/* Flag of tb_select's `mode`: leave the local window out of idx (the list is
 * sink U important); tb_sparse_decode_attn then adds the window itself from
 * ctx_len, so one selection serves every step of a prediction interval. */
#define TB_SEL_OMIT_WINDOW 0x100
/* mode flag of tb_select / tb_score_select (TB_NF_FILL only): stop before the
 * list is written -- count is written, idx is not; the selection state stays
 * in the workspace for tb_select_attn, which writes idx and attends. */
#define TB_SEL_DEFER_LIST 0x200
/* mode flag of tb_score_select (TB_NF_FILL only), then of the tb_select_attn
 * call that follows it: the selection is split across the two calls. Where
 * it applies (the histogram route of tb_score_select: B * Hq <= 64,
 * 8192 < Lmax <= 131072, radius <= 2, Hq / Hkv <= 4, and, with n =
 * ceil(Lmax / 2048) chunks, ceil(n / 2) + ceil(n / 4) <= ceil(cap / 256)),
 * tb_score_select writes the scores and classifies every token against the
 * histogram bin of the budget's key, and writes neither count nor idx;
 * tb_select_attn then attends the rows already fixed (sink, window, tokens
 * above that bin) from the start, while its threshold workgroups (one per 4
 * chunks of 2048 tokens) find the exact threshold, attend the chosen tokens
 * of the bin and write count and idx as tb_score_select without the flag
 * would. Its out then
 * agrees with tb_sparse_decode_attn over that list to fp32 rounding (other
 * splits: not bit for bit). A workspace whose histograms were not zero before
 * the first call is reported as count -1 and out 0 for the segments it
 * affects (the call leaves them zero, so the next call is exact). Elsewhere
 * the flag acts as TB_SEL_DEFER_LIST. tb_select rejects it. */
#define TB_SEL_DEFER_SELECT 0x400

/* Human-readable text for a status code (static storage). */
const char *tb_status_string(tb_status s);
/* Detail of the last error raised on the calling thread (thread-local). */
const char *tb_last_error_detail(void);
/* Library ABI version: 1. */
int tb_abi_version(void);

/*
 * Query prediction ("Core architecture", query prediction): a lightweight MLP
 * reads the producer layer's hidden state and emits one low-dimensional
 * query per query head (and per slot):
 *     h    = bf16_rne( SiLU( x w1^T ) )        fp32 accumulation
 *     qhat = h w2^T                             fp32 accumulation, fp32 out
 *   x     [B, E]                 bf16
 *   w1    [Eh, E]                bf16  (out x in)
 *   w2    [n_out, Eh]            bf16  (out x in); n_out = n_slots * Hq * dp
 *   qhat  [B, n_out]             fp32  (read as [B, n_slots, Hq, dp])
 * Limits: E % 128 == 0, Eh % 128 == 0, Eh <= 1536, n_out % 16 == 0, 1 <= B <= 64.
 * The workspace holds the split partial sums of x w1^T.
 */
size_t tb_predict_workspace_bytes(int B, int E, int Eh, int n_out);
tb_status tb_predict_queries(const void *x, const void *w1, const void *w2, float *qhat,
                             int B, int E, int Eh, int n_out,
                             void *workspace, size_t ws_bytes, void *stream);

/*
 * tb_predict_queries and tb_project_keys fused: the two steps are independent
 * (the predictor reads the producer layer's state, the projection the consumer
 * layer's newest keys), so the projection runs as extra workgroups of the
 * predictor's first launch; one launch less per decode step. Arguments,
 * limits and results are exactly those of the two calls (same B for both).
 */
tb_status tb_predict_project(const void *x, const void *w1, const void *w2, float *qhat,
                             int B, int E, int Eh, int n_out,
                             void *workspace, size_t ws_bytes,
                             const void *k_cache, const void *wk, void *kp,
                             const int32_t *pos0, int n_tokens,
                             int Hkv, int Lmax, int D, int dp, void *stream);

/*
 * Key-cache projection ("Core architecture", key projection; "Inference
 * strategy", batching: run once per batch of new tokens, not every step):
 *     kp[b, j, t, :] = fp16_rne( k_cache[b, j, t, :] wk[j]^T )   fp32 accumulation
 * for t in [pos0[b], pos0[b] + n_tokens) intersected with [0, Lmax).
 *   k_cache [B, Hkv, Lmax, D]   bf16
 *   wk      [Hkv, dp, D]        bf16  (out x in, one matrix per KV head)
 *   kp      [B, Hkv, Lmax, dp]  fp16  (only the projected rows are written)
 *   pos0    [B]                 int32, device
 * Limits: D in {64, 128}, dp in {16, 32}, n_tokens >= 0.
 */
tb_status tb_project_keys(const void *k_cache, const void *wk, void *kp,
                          const int32_t *pos0, int n_tokens,
                          int B, int Hkv, int Lmax, int D, int dp, void *stream);

/*
 * Decode-step cache append with batched projection ("Inference strategy":
 * the newest token's key and value join the retained cache; "Optimizations":
 * the key projection runs once per batch of n_p new tokens). Per sequence b,
 * with L = ctx_len[b] and P = proj_len[b] read on the device:
 *   if 0 <= P <= L < Lmax: k_new[b, j] and v_new[b, j] are written at
 *   position L of every KV head j; ctx_len[b] becomes L + 1; and when
 *   L + 1 - P >= n_p the keys [P, L + 1) are projected as by tb_project_keys
 *   and proj_len[b] becomes L + 1. Otherwise (a full cache, or lengths out of
 *   range) nothing is written for b.
 *   k_new, v_new [B, Hkv, D]          bf16
 *   k_cache, v_cache [B, Hkv, Lmax, D] bf16, kp [B, Hkv, Lmax, dp] fp16
 *   wk      [Hkv, dp, D]              bf16
 *   ctx_len, proj_len [B]             int32, device, updated in place
 * One workgroup per sequence; meant for n_p up to a few hundred (use
 * tb_project_keys for a whole context). Limits: D in {64, 128}, dp in
 * {16, 32}, n_p >= 1.
 */
tb_status tb_append_kv(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                       void *kp, const void *wk, int32_t *ctx_len, int32_t *proj_len,
                       int B, int Hkv, int Lmax, int D, int dp, int n_p, void *stream);

/*
 * CPU-offload decoding ("Inference strategy": the full cache is retained and
 * attention reads a sink buffer, a circular local window and an important
 * buffer; "Significance": only the selected tokens are accessed). The full
 * K/V cache [B, Hkv, Lmax, D] bf16 lives in pinned host memory (e.g.
 * hipHostMalloc, torch pin_memory) and is read over the host link. Each
 * query head h owns device buffers k_buf, v_buf [B, Hq, buf_rows, D] bf16;
 * attention over them is tb_sparse_decode_attn with Hkv = Hq, Lmax =
 * buf_rows, an identity list over the gathered slots and the implicit
 * window (ctx_len = buf_rows, window = the window size).
 *
 * tb_offload_gather: for every (b, h) and i < count[b, h] (clamped to
 * [0, cap]), the row t = idx[b, h, i] (clamped to [0, Lmax)) of KV head
 * h / (Hq / Hkv) is copied from the host cache to slot s of head h's
 * buffers, s = slot0 + i, or s = slot0 + t mod wrap when wrap > 0 (the
 * circular window); rows whose slot would reach buf_rows are skipped. With
 * wrap > 0, entries whose t mod wrap coincide write the same slot and which
 * of them lands is unspecified; a list of at most wrap consecutive
 * positions (the window) has no such entries.
 * Limits: D in {64, 128}; Hq % Hkv == 0; 0 <= slot0 < buf_rows;
 * slot0 + wrap <= buf_rows. Returns TB_ERR_INVALID_ARGUMENT if the caches
 * are not pinned host memory.
 */
tb_status tb_offload_gather(const void *k_host, const void *v_host, int B, int Hkv, int Lmax,
                            int D, const int32_t *idx, const int32_t *count, int cap, int Hq,
                            void *k_buf, void *v_buf, int buf_rows, int slot0, int wrap,
                            void *stream);

/*
 * tb_offload_append: one decode step of the offloaded cache. Per sequence b
 * with L = ctx_len[b] == proj_len[b] < Lmax (otherwise nothing is written
 * for b): k_new[b, j], v_new[b, j] [B, Hkv, D] are written at position L of
 * the host cache and, when window > 0, into slot buf_rows - window +
 * L mod window of the buffers of every query head of group j; the new key is
 * projected (kp[b, j, L] = fp16(k_new[b, j] wk[j]^T), kp and wk on the
 * device as for tb_project_keys); ctx_len[b] and proj_len[b] become L + 1.
 * Limits: D in {64, 128}, dp in {16, 32}, 0 <= window <= buf_rows.
 */
tb_status tb_offload_append(const void *k_new, const void *v_new, const void *wk, void *k_host,
                            void *v_host, void *kp, int32_t *ctx_len, int32_t *proj_len, int B,
                            int Hkv, int Lmax, int D, int dp, void *k_buf, void *v_buf, int Hq,
                            int buf_rows, int window, void *stream);

/*
 * Distillation loss ("Training": the predictor is trained on the frozen
 * model's masked causal attention distribution, minimizing the cross entropy
 * between the teacher's attention logits and the predictor's logits, with
 * the loss taken at a subset of R query positions so the cost is O(R L)).
 * Per (b, r, query head h), i = pos[b, r] clamped to [0, Lmax - 1], KV head
 * h / (Hq / Hkv), over the causal tokens t <= i:
 *   z_t = scale * q[b, r, h] . k_cache[b, h/g, t]   (teacher logits)
 *   s_t = qhat[b, r, h] . kp[b, h/g, t]             (predictor logits)
 *   loss[b, r, h] = logsumexp_t(s_t) - sum_t softmax(z)_t s_t     (fp32)
 *   q    [B, R, Hq, D]  bf16      qhat [B, R, Hq, dp] fp32
 *   k_cache [B, Hkv, Lmax, D] bf16, kp [B, Hkv, Lmax, dp] fp16
 *   pos  [B, R] int32, device;    loss [B, R, Hq] fp32
 * Limits: D in {64, 128}, dp in {16, 32}, Hq % Hkv == 0, B * Hkv <= 65535.
 * The workspace (zero-filled once) holds per-split partials and arrival
 * counters, which every call leaves at zero.
 */
size_t tb_distill_workspace_bytes(int B, int R, int Hq, int Hkv, int Lmax);
tb_status tb_distill_loss(const void *q, const void *k_cache, const float *qhat, const void *kp,
                          const int32_t *pos, int B, int R, int Hq, int Hkv, int Lmax, int D,
                          int dp, float scale, float *loss, void *workspace, size_t ws_bytes,
                          void *stream);

/*
 * Scoring ("Core architecture", scoring): token importance is the dot product
 * of the predicted query with the projected key; query head h reads KV head
 * h / (Hq / Hkv):
 *     scores[b, h, t] = sum_c qhat[b, slot, h, c] * kp[b, h / g, t, c]   (fp32)
 * for t < proj_len[b] (clamped to Lmax); other positions are not written.
 *   qhat     [B, n_slots, Hq, dp] fp32
 *   kp       [B, Hkv, Lmax, dp]   fp16
 *   proj_len [B]                  int32, device
 *   scores   [B, Hq, Lmax]        fp32
 * Limits: Hq % Hkv == 0, 1 <= Hq / Hkv <= 8, dp in {16, 32}.
 */
tb_status tb_score(const float *qhat, int n_slots, int slot, const void *kp,
                   const int32_t *proj_len, float *scores,
                   int B, int Hq, int Hkv, int Lmax, int dp, void *stream);

/*
 * Selection ("Inference strategy": sink buffer of the first `sink` tokens,
 * circular local window of the most recent `window` tokens, important buffer
 * filled from the predicted scores; "Optimizations": neighbour fetching;
 * "Core architecture": selection under a fixed budget). Per (b, h):
 *   eligible E = [sink, min(ctx_len[b] - window, proj_len[b])) (empty if the
 *     bound is <= sink);
 *   the important buffer takes min(budget, |E|) tokens of E, filled greedily:
 *     visit E in descending score order (IEEE totalOrder, so -0 < +0; equal
 *     scores: lower position first); each visited centre c brings c, c-1,
 *     c+1, ..., c-radius, c+radius (those in E and not yet taken) until the
 *     buffer is full (mode TB_NF_FILL);
 *   with mode TB_NF_DILATE (the other reading of neighbour fetching: the
 *     neighbours come on top of the budget) the min(budget, |E|) first
 *     tokens of E in that order are centres and every position of E within
 *     distance radius of a centre is important;
 *   idx[b, h, 0:count) = sink U window U important, ascending, where
 *     sink = [0, min(sink, L)), window = [max(0, L - window), L), L = ctx_len[b];
 *     with TB_SEL_OMIT_WINDOW in mode the window is left out.
 *   scores  [B, Hq, Lmax] fp32 (any position in [0, Lmax) may be read; only
 *           eligible positions' values are used and must be finite)
 *   ctx_len [B], proj_len [B]  int32, device
 *   idx     [B, Hq, cap]  int32 (slots >= count are left unspecified)
 *   count   [B, Hq]       int32 (-1 when ctx_len or proj_len is outside
 *                                [0, Lmax]; idx is then not written)
 * Limits: cap >= min(Lmax, sink + window + I) with I = budget (TB_NF_FILL)
 * or (2 radius + 1) budget (TB_NF_DILATE), the window left out of the sum
 * with TB_SEL_OMIT_WINDOW; 0 <= radius <= 64; Lmax <= 2^24; sink, window,
 * budget >= 0; mode is TB_NF_FILL or TB_NF_DILATE, optionally ORed with
 * TB_SEL_OMIT_WINDOW.
 */
size_t tb_select_workspace_bytes(int B, int Hq, int Lmax);
tb_status tb_select(const float *scores, const int32_t *ctx_len, const int32_t *proj_len,
                    int B, int Hq, int Lmax, int sink, int window, int budget, int radius,
                    int mode, int32_t *idx, int32_t *count, int cap,
                    void *workspace, size_t ws_bytes, void *stream);

/*
 * Scoring and selection in one call ("Core architecture": scoring, then
 * selection under a fixed budget; "Inference strategy": the three buffers):
 * exactly tb_score(qhat, n_slots, slot, kp, proj_len, scores, ...) followed
 * by tb_select(scores, ctx_len, proj_len, ..., mode, idx, count, cap,
 * workspace, ...) -- the same scores, idx and count. For small problems
 * (radius <= 1 -- 0 in TB_NF_DILATE mode -- and 8 B Hq at most the device's
 * compute-unit count) it takes one launch fewer: the selection's sampled
 * band is computed by extra workgroups of the scoring launch, from the
 * projected keys directly, while the scores stream; otherwise it issues the
 * two calls' launches. Arguments, limits and workspace
 * (tb_select_workspace_bytes) are those of the two calls; scores is still
 * written (the selection reads it).
 */
tb_status tb_score_select(const float *qhat, int n_slots, int slot, const void *kp,
                          const int32_t *ctx_len, const int32_t *proj_len, float *scores,
                          int B, int Hq, int Hkv, int Lmax, int dp, int sink, int window,
                          int budget, int radius, int mode, int32_t *idx, int32_t *count,
                          int cap, void *workspace, size_t ws_bytes, void *stream);

/*
 * The selection's list and the sparse attention over it in one launch
 * ("Inference strategy": the three buffers; "Significance": attention reads
 * only the selected tokens). Called after tb_select or tb_score_select with
 * mode | TB_SEL_DEFER_LIST (or tb_score_select with TB_SEL_DEFER_SELECT, see
 * there) on the same workspace, arguments and stream, with the same mode here: writes idx exactly as the selection without the flag
 * would, and out exactly as tb_sparse_decode_attn(q, k_cache, v_cache, idx,
 * count, cap, NULL, 0, B, Hq, Hkv, Lmax, D, scale, out, attn_workspace, ...)
 * would (bit for bit: the same splits through the same code). Each attention
 * workgroup rebuilds its split's list rows from the selection's bitmap and
 * candidates (one compaction launch fewer); with more than 64 chunks of 2048
 * tokens (Lmax > 131072) it issues the compaction and attention launches
 * instead. attn_workspace is sized by tb_attn_workspace_bytes(B, Hq, cap, 0,
 * D). A selection state from any other call sequence gives unspecified
 * results (every access stays inside the caller's buffers).
 */
tb_status tb_select_attn(const int32_t *ctx_len, const int32_t *proj_len, int B, int Hq, int Hkv,
                         int Lmax, int sink, int window, int budget, int radius, int mode,
                         int32_t *idx, int32_t *count, int cap, void *sel_workspace,
                         size_t sel_ws_bytes, const void *q, const void *k_cache,
                         const void *v_cache, int D, float scale, float *out,
                         void *attn_workspace, size_t attn_ws_bytes, void *stream);

/*
 * The decode step's append and attention in one launch ("Inference strategy":
 * the newest token joins the retained cache and the attention reads the sink,
 * important and local-window rows): the same results, bit for bit, as
 *     tb_append_kv(k_new, v_new, k_cache, v_cache, kp, wk, ctx_len, proj_len,
 *                  B, Hkv, Lmax, D, dp, n_p, stream);
 *     tb_sparse_decode_attn(q, k_cache, v_cache, idx, count, cap, ctx_len,
 *                           window, B, Hq, Hkv, Lmax, D, scale, out,
 *                           workspace, ws_bytes, stream);
 * (arguments as there): the new rows are appended and the pending keys
 * projected, and the attention's window ends at the length the append
 * leaves, so it holds the new token. ctx_len and proj_len are advanced in
 * place within the launch, after every workgroup has read them. workspace is
 * sized by tb_attn_workspace_bytes(B, Hq, cap, window, D) and shared with
 * tb_sparse_decode_attn (zero at rest).
 */
tb_status tb_append_attn(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                         void *kp, const void *wk, int32_t *ctx_len, int32_t *proj_len, int n_p,
                         const void *q, const int32_t *idx, const int32_t *count, int cap,
                         int window, int B, int Hq, int Hkv, int Lmax, int D, int dp, float scale,
                         float *out, void *workspace, size_t ws_bytes, void *stream);

/*
 * Sparse decode attention ("Significance": attend over the retained cache
 * reading only the selected tokens):
 *     out[b, h] = sum_{t in F} softmax_t( scale * q[b,h] . k[b, h/g, t] ) v[b, h/g, t]
 * with F = idx[b, h, 0:count[b, h]], plus, when ctx_len is not NULL and
 * window > 0, the local window [w0, L) with L = ctx_len[b] and
 * w0 = max(L - window, last list entry + 1, 0) ("Inference strategy": the
 * circular buffer of the most recent tokens). Within a prediction interval the
 * list (sink U important, see TB_SEL_OMIT_WINDOW) stays fixed and only
 * ctx_len advances. fp32 softmax and accumulation; out = 0 for an empty F.
 *   q       [B, Hq, D]        bf16
 *   k_cache [B, Hkv, Lmax, D] bf16,  v_cache the same
 *   idx     [B, Hq, cap] int32 ascending, entries in [0, Lmax) (clamped
 *           otherwise); count [B, Hq] int32 (clamped to [0, cap])
 *   ctx_len [B] int32, device, or NULL (ctx_len is clamped to [0, Lmax])
 *   out     [B, Hq, D]        fp32
 * Limits: D in {64, 128}; Hq % Hkv == 0; window >= 0; Lmax * D * 2 < 2^31.
 * The workspace query takes the same window (pass 0 when ctx_len is NULL).
 */
size_t tb_attn_workspace_bytes(int B, int Hq, int cap, int window, int D);
tb_status tb_sparse_decode_attn(const void *q, const void *k_cache, const void *v_cache,
                                const int32_t *idx, const int32_t *count, int cap,
                                const int32_t *ctx_len, int window,
                                int B, int Hq, int Hkv, int Lmax, int D, float scale,
                                float *out, void *workspace, size_t ws_bytes, void *stream);

/*
 * Measurement: bandwidth ceilings of this part, reported beside the HBM peak
 * ("Significance": the method's premise is that reading only the selected
 * tokens relieves the memory-bandwidth bottleneck).
 * tb_probe_stream_read reads `bytes` (a multiple of 16) from src once, in
 * 16-byte loads spread over at most sink_words workgroups (4 per compute
 * unit), and writes one XOR word per workgroup to sink.
 * tb_probe_row_gather requests exactly the K and V rows that
 * tb_sparse_decode_attn(q, k_cache, v_cache, idx, count, cap, NULL, 0, ...)
 * reads (the same workgroups, list splits and order; K and V rows of a split
 * requested together) and writes one XOR word per workgroup to sink, which
 * holds tb_probe_row_gather_sink_words(B, Hq, cap) words; no arithmetic on
 * the rows. Limits as tb_sparse_decode_attn.
 */
tb_status tb_probe_stream_read(const void *src, size_t bytes, uint32_t *sink, int sink_words,
                               void *stream);
size_t tb_probe_row_gather_sink_words(int B, int Hq, int cap);
tb_status tb_probe_row_gather(const void *k_cache, const void *v_cache, const int32_t *idx,
                              const int32_t *count, int cap, int B, int Hq, int Hkv, int Lmax,
                              int D, uint32_t *sink, size_t sink_words, void *stream);

/*
 * tb_sparse_decode_attn for callers that cannot allocate device memory (code
 * under graph capture that must not call hipMalloc, tight serving loops,
 * harnesses that forbid allocation): the same computation, arguments and
 * results as tb_sparse_decode_attn, without the workspace. The split partials
 * and arrival counters live in a fixed 8 MiB device array per GPU, held until
 * the process ends: counters of up to 65536 heads (B * Hq) and at most
 * 8 MiB - 256 KiB of partials, i.e. B * Hq * ceil((cap + window) / 256) *
 * (D + 2) * 4 bytes; larger calls return TB_ERR_UNSUPPORTED_SHAPE and enqueue
 * nothing. Every call on a GPU shares that GPU's array: calls that may
 * overlap on one GPU (several streams, several threads) race and give
 * unspecified results; order them on one stream. The call allocates nothing;
 * on its first use on a device it looks up the array's address (and, outside
 * a graph capture, clears its counters with a small kernel on `stream`).
 */
tb_status tb_sparse_decode_attn_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                        const int32_t *idx, const int32_t *count, int cap,
                                        const int32_t *ctx_len, int window,
                                        int B, int Hq, int Hkv, int Lmax, int D, float scale,
                                        float *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TB_H */
