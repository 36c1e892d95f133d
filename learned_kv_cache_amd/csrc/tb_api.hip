// C ABI entry points of libtb: host-side argument validation, workspace
// layout and kernel dispatch. Nothing here allocates or synchronizes.
#include <stdarg.h>
#include <stdio.h>

#include "tb_common.h"

namespace tb {

static thread_local char g_detail[512] = "";

void set_error(const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof g_detail, fmt, ap);
    va_end(ap);
}

tb_status check_launch(const char *what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_error("%s: %s", what, hipGetErrorString(e));
        return TB_ERR_HIP;
    }
    return TB_OK;
}

// Device address of pinned host memory (false if ptr is not pinned host
// memory the device can reach); the failed query's error is cleared.
bool host_to_device(const void *ptr, const void **dev) {
    void *d = nullptr;
    if (hipHostGetDevicePointer(&d, const_cast<void *>(ptr), 0) != hipSuccess || !d) {
        (void)hipGetLastError();
        return false;
    }
    *dev = d;
    return true;
}

}  // namespace tb

using tb::aligned16;
using tb::aligned4;

extern "C" {

const char *tb_status_string(tb_status s) {
    switch (s) {
        case TB_OK: return "ok";
        case TB_ERR_INVALID_ARGUMENT: return "invalid argument";
        case TB_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
        case TB_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case TB_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

const char *tb_last_error_detail(void) { return tb::g_detail; }

int tb_abi_version(void) { return 1; }

// ---------------------------------------------------------------- predictor
size_t tb_predict_workspace_bytes(int B, int E, int Eh, int n_out) {
    (void)n_out;
    if (B <= 0 || B > 64 || E <= 0 || Eh <= 0 || Eh > 1536 || E % 128 || Eh % 128) return 0;
    return (size_t)tb::predict_nsplit(E, Eh) * B * Eh * sizeof(float);
}

tb_status tb_predict_queries(const void *x, const void *w1, const void *w2, float *qhat, int B,
                             int E, int Eh, int n_out, void *workspace, size_t ws_bytes,
                             void *stream) {
    TB_REQUIRE(x && w1 && w2 && qhat && workspace, TB_ERR_INVALID_ARGUMENT,
               "tb_predict_queries: null pointer");
    TB_REQUIRE(aligned16(x) && aligned16(w1) && aligned16(w2) && aligned16(qhat) &&
                   aligned16(workspace),
               TB_ERR_INVALID_ARGUMENT, "tb_predict_queries: pointers must be 16-byte aligned");
    TB_REQUIRE(B >= 1 && B <= 64 && E > 0 && Eh > 0 && n_out > 0, TB_ERR_INVALID_ARGUMENT,
               "tb_predict_queries: bad sizes B=%d E=%d Eh=%d n_out=%d", B, E, Eh, n_out);
    TB_REQUIRE(E % 128 == 0 && Eh % 128 == 0 && n_out % 16 == 0 && Eh <= 1536,
               TB_ERR_UNSUPPORTED_SHAPE,
               "tb_predict_queries: need E %% 128 == 0, Eh %% 128 == 0, Eh <= 1536, n_out %% 16 == 0");
    const size_t need = tb_predict_workspace_bytes(B, E, Eh, n_out);
    TB_REQUIRE(ws_bytes >= need, TB_ERR_WORKSPACE_TOO_SMALL,
               "tb_predict_queries: workspace %zu < %zu bytes", ws_bytes, need);
    return tb::launch_predict(x, w1, w2, qhat, B, E, Eh, n_out, workspace,
                              tb::predict_nsplit(E, Eh), static_cast<hipStream_t>(stream));
}

tb_status tb_predict_project(const void *x, const void *w1, const void *w2, float *qhat, int B,
                             int E, int Eh, int n_out, void *workspace, size_t ws_bytes,
                             const void *k_cache, const void *wk, void *kp, const int32_t *pos0,
                             int n_tokens, int Hkv, int Lmax, int D, int dp, void *stream) {
    TB_REQUIRE(x && w1 && w2 && qhat && workspace && k_cache && wk && kp && pos0,
               TB_ERR_INVALID_ARGUMENT, "tb_predict_project: null pointer");
    TB_REQUIRE(aligned16(x) && aligned16(w1) && aligned16(w2) && aligned16(qhat) &&
                   aligned16(workspace) && aligned16(k_cache) && aligned16(wk) && aligned16(kp) &&
                   aligned4(pos0),
               TB_ERR_INVALID_ARGUMENT, "tb_predict_project: misaligned pointer");
    TB_REQUIRE(B >= 1 && B <= 64 && E > 0 && Eh > 0 && n_out > 0 && Hkv >= 1 &&
                   Hkv <= 65535 && Lmax >= 1 && n_tokens >= 0,
               TB_ERR_INVALID_ARGUMENT, "tb_predict_project: bad sizes");
    TB_REQUIRE(E % 128 == 0 && Eh % 128 == 0 && n_out % 16 == 0 && Eh <= 1536,
               TB_ERR_UNSUPPORTED_SHAPE,
               "tb_predict_project: need E %% 128 == 0, Eh %% 128 == 0, Eh <= 1536, n_out %% 16 == 0");
    TB_REQUIRE((D == 64 || D == 128) && (dp == 16 || dp == 32), TB_ERR_UNSUPPORTED_SHAPE,
               "tb_predict_project: D must be 64 or 128 and dp 16 or 32");
    const size_t need = tb_predict_workspace_bytes(B, E, Eh, n_out);
    TB_REQUIRE(ws_bytes >= need, TB_ERR_WORKSPACE_TOO_SMALL,
               "tb_predict_project: workspace %zu < %zu bytes", ws_bytes, need);
    return tb::launch_predict_project(x, w1, w2, qhat, B, E, Eh, n_out, workspace,
                                      tb::predict_nsplit(E, Eh), k_cache, wk, kp, pos0, n_tokens,
                                      Hkv, Lmax, D, dp, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------- projection
tb_status tb_project_keys(const void *k_cache, const void *wk, void *kp, const int32_t *pos0,
                          int n_tokens, int B, int Hkv, int Lmax, int D, int dp, void *stream) {
    TB_REQUIRE(k_cache && wk && kp && pos0, TB_ERR_INVALID_ARGUMENT,
               "tb_project_keys: null pointer");
    TB_REQUIRE(aligned16(k_cache) && aligned16(wk) && aligned16(kp) && aligned4(pos0),
               TB_ERR_INVALID_ARGUMENT, "tb_project_keys: misaligned pointer");
    TB_REQUIRE(B >= 1 && B <= 65535 && Hkv >= 1 && Hkv <= 65535 && Lmax >= 1 && n_tokens >= 0,
               TB_ERR_INVALID_ARGUMENT, "tb_project_keys: bad sizes B=%d Hkv=%d Lmax=%d n=%d", B,
               Hkv, Lmax, n_tokens);
    TB_REQUIRE((D == 64 || D == 128) && (dp == 16 || dp == 32), TB_ERR_UNSUPPORTED_SHAPE,
               "tb_project_keys: D must be 64 or 128 and dp 16 or 32 (got %d, %d)", D, dp);
    return tb::launch_project(k_cache, wk, kp, pos0, n_tokens, B, Hkv, Lmax, D, dp,
                              static_cast<hipStream_t>(stream));
}

tb_status tb_append_kv(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                       void *kp, const void *wk, int32_t *ctx_len, int32_t *proj_len, int B,
                       int Hkv, int Lmax, int D, int dp, int n_p, void *stream) {
    TB_REQUIRE(k_new && v_new && k_cache && v_cache && kp && wk && ctx_len && proj_len,
               TB_ERR_INVALID_ARGUMENT, "tb_append_kv: null pointer");
    TB_REQUIRE(aligned16(k_new) && aligned16(v_new) && aligned16(k_cache) && aligned16(v_cache) &&
                   aligned16(kp) && aligned16(wk) && aligned4(ctx_len) && aligned4(proj_len),
               TB_ERR_INVALID_ARGUMENT, "tb_append_kv: misaligned pointer");
    TB_REQUIRE(B >= 1 && B <= 65535 && Hkv >= 1 && Hkv <= 65535 && Lmax >= 1 && n_p >= 1,
               TB_ERR_INVALID_ARGUMENT, "tb_append_kv: bad sizes B=%d Hkv=%d Lmax=%d n_p=%d", B,
               Hkv, Lmax, n_p);
    TB_REQUIRE((D == 64 || D == 128) && (dp == 16 || dp == 32), TB_ERR_UNSUPPORTED_SHAPE,
               "tb_append_kv: D must be 64 or 128 and dp 16 or 32 (got %d, %d)", D, dp);
    return tb::launch_append(k_new, v_new, k_cache, v_cache, kp, wk, ctx_len, proj_len, B, Hkv,
                             Lmax, D, dp, n_p, static_cast<hipStream_t>(stream));
}

tb_status tb_offload_gather(const void *k_host, const void *v_host, int B, int Hkv, int Lmax,
                            int D, const int32_t *idx, const int32_t *count, int cap, int Hq,
                            void *k_buf, void *v_buf, int buf_rows, int slot0, int wrap,
                            void *stream) {
    TB_REQUIRE(k_host && v_host && idx && count && k_buf && v_buf, TB_ERR_INVALID_ARGUMENT,
               "tb_offload_gather: null pointer");
    TB_REQUIRE(aligned16(k_host) && aligned16(v_host) && aligned4(idx) && aligned4(count) &&
                   aligned16(k_buf) && aligned16(v_buf),
               TB_ERR_INVALID_ARGUMENT, "tb_offload_gather: misaligned pointer");
    TB_REQUIRE(B >= 1 && B <= 65535 && Hkv >= 1 && Hq >= 1 && Hq <= 65535 && Lmax >= 1 &&
                   cap >= 1 && buf_rows >= 1 && slot0 >= 0 && slot0 < buf_rows && wrap >= 0 &&
                   slot0 + wrap <= buf_rows,
               TB_ERR_INVALID_ARGUMENT, "tb_offload_gather: bad sizes");
    TB_REQUIRE(Hq % Hkv == 0, TB_ERR_INVALID_ARGUMENT, "tb_offload_gather: Hq %% Hkv != 0");
    TB_REQUIRE(D == 64 || D == 128, TB_ERR_UNSUPPORTED_SHAPE, "tb_offload_gather: D must be 64 or 128");
    const void *kd, *vd;
    TB_REQUIRE(tb::host_to_device(k_host, &kd) && tb::host_to_device(v_host, &vd),
               TB_ERR_INVALID_ARGUMENT, "tb_offload_gather: caches must be pinned host memory");
    return tb::launch_offload_gather(kd, vd, B, Hkv, Lmax, D, idx, count, cap, Hq, k_buf, v_buf,
                                     buf_rows, slot0, wrap, static_cast<hipStream_t>(stream));
}

tb_status tb_offload_append(const void *k_new, const void *v_new, const void *wk, void *k_host,
                            void *v_host, void *kp, int32_t *ctx_len, int32_t *proj_len, int B,
                            int Hkv, int Lmax, int D, int dp, void *k_buf, void *v_buf, int Hq,
                            int buf_rows, int window, void *stream) {
    TB_REQUIRE(k_new && v_new && wk && k_host && v_host && kp && ctx_len && proj_len && k_buf &&
                   v_buf,
               TB_ERR_INVALID_ARGUMENT, "tb_offload_append: null pointer");
    TB_REQUIRE(aligned16(k_new) && aligned16(v_new) && aligned16(wk) && aligned16(k_host) &&
                   aligned16(v_host) && aligned16(kp) && aligned4(ctx_len) && aligned4(proj_len) &&
                   aligned16(k_buf) && aligned16(v_buf),
               TB_ERR_INVALID_ARGUMENT, "tb_offload_append: misaligned pointer");
    TB_REQUIRE(B >= 1 && B <= 65535 && Hkv >= 1 && Hq >= 1 && Lmax >= 1 && buf_rows >= 1 &&
                   window >= 0 && window <= buf_rows,
               TB_ERR_INVALID_ARGUMENT, "tb_offload_append: bad sizes");
    TB_REQUIRE(Hq % Hkv == 0, TB_ERR_INVALID_ARGUMENT, "tb_offload_append: Hq %% Hkv != 0");
    TB_REQUIRE((D == 64 || D == 128) && (dp == 16 || dp == 32), TB_ERR_UNSUPPORTED_SHAPE,
               "tb_offload_append: D must be 64 or 128 and dp 16 or 32");
    const void *kd, *vd;
    TB_REQUIRE(tb::host_to_device(k_host, &kd) && tb::host_to_device(v_host, &vd),
               TB_ERR_INVALID_ARGUMENT, "tb_offload_append: caches must be pinned host memory");
    return tb::launch_offload_append(k_new, v_new, wk, const_cast<void *>(kd),
                                     const_cast<void *>(vd), kp, ctx_len, proj_len, B, Hkv, Lmax,
                                     D, dp, k_buf, v_buf, Hq, buf_rows, window,
                                     static_cast<hipStream_t>(stream));
}

size_t tb_distill_workspace_bytes(int B, int R, int Hq, int Hkv, int Lmax) {
    if (B <= 0 || R <= 0 || Hq <= 0 || Hkv <= 0 || Lmax <= 0 || Hq % Hkv) return 0;
    // the sizes tb_distill_loss accepts (its grid: splits x row groups x B * Hkv)
    if ((long long)B * Hkv > 65535 || (long long)R * Hq > (1LL << 24) || Lmax > (1 << 30) ||
        tb::distill_ngroups(R, Hq / Hkv) > 65535)
        return 0;
    return tb::distill_ws_layout(B, R, Hq, Hkv, Lmax, nullptr, nullptr, nullptr);
}

tb_status tb_distill_loss(const void *q, const void *k_cache, const float *qhat, const void *kp,
                          const int32_t *pos, int B, int R, int Hq, int Hkv, int Lmax, int D,
                          int dp, float scale, float *loss, void *workspace, size_t ws_bytes,
                          void *stream) {
    TB_REQUIRE(q && k_cache && qhat && kp && pos && loss && workspace, TB_ERR_INVALID_ARGUMENT,
               "tb_distill_loss: null pointer");
    TB_REQUIRE(aligned16(q) && aligned16(k_cache) && aligned4(qhat) && aligned16(kp) &&
                   aligned4(pos) && aligned4(loss) && aligned16(workspace),
               TB_ERR_INVALID_ARGUMENT, "tb_distill_loss: misaligned pointer");
    TB_REQUIRE(B >= 1 && R >= 1 && Hq >= 1 && Hkv >= 1 && Lmax >= 1 &&
                   (long long)B * Hkv <= 65535 && (long long)R * Hq <= (1LL << 24),
               TB_ERR_INVALID_ARGUMENT, "tb_distill_loss: bad sizes");
    TB_REQUIRE(Hq % Hkv == 0, TB_ERR_INVALID_ARGUMENT, "tb_distill_loss: Hq %% Hkv != 0");
    TB_REQUIRE((D == 64 || D == 128) && (dp == 16 || dp == 32), TB_ERR_UNSUPPORTED_SHAPE,
               "tb_distill_loss: D must be 64 or 128 and dp 16 or 32");
    TB_REQUIRE(scale == scale, TB_ERR_INVALID_ARGUMENT, "tb_distill_loss: scale is NaN");
    TB_REQUIRE(Lmax <= (1 << 30) && tb::distill_ngroups(R, Hq / Hkv) <= 65535,
               TB_ERR_UNSUPPORTED_SHAPE, "tb_distill_loss: Lmax > 2^30 or more than 65535 row groups");
    const size_t need = tb_distill_workspace_bytes(B, R, Hq, Hkv, Lmax);
    TB_REQUIRE(ws_bytes >= need, TB_ERR_WORKSPACE_TOO_SMALL,
               "tb_distill_loss: workspace %zu < %zu bytes", ws_bytes, need);
    float *part;
    uint32_t *ctr;
    tb::distill_ws_layout(B, R, Hq, Hkv, Lmax, workspace, &part, &ctr);
    return tb::launch_distill(q, k_cache, qhat, kp, pos, B, R, Hq, Hkv, Lmax, D, dp, scale, part,
                              ctr, loss, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------- scoring
tb_status tb_score(const float *qhat, int n_slots, int slot, const void *kp,
                   const int32_t *proj_len, float *scores, int B, int Hq, int Hkv, int Lmax,
                   int dp, void *stream) {
    TB_REQUIRE(qhat && kp && proj_len && scores, TB_ERR_INVALID_ARGUMENT,
               "tb_score: null pointer");
    TB_REQUIRE(aligned4(qhat) && aligned16(kp) && aligned4(proj_len) && aligned4(scores),
               TB_ERR_INVALID_ARGUMENT, "tb_score: misaligned pointer");
    TB_REQUIRE(B >= 1 && B <= 65535 && Hkv >= 1 && Hq >= 1 && Lmax >= 1 && n_slots >= 1 &&
                   slot >= 0 && slot < n_slots,
               TB_ERR_INVALID_ARGUMENT, "tb_score: bad sizes");
    TB_REQUIRE(Hq % Hkv == 0, TB_ERR_INVALID_ARGUMENT, "tb_score: Hq %% Hkv != 0");
    TB_REQUIRE(Hq / Hkv <= 8 && Hkv <= 65535 && (dp == 16 || dp == 32), TB_ERR_UNSUPPORTED_SHAPE,
               "tb_score: need Hq/Hkv <= 8 and dp in {16, 32}");
    return tb::launch_score(qhat, n_slots, slot, kp, proj_len, scores, B, Hq, Hkv, Lmax, dp,
                            static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------- selection
size_t tb_select_workspace_bytes(int B, int Hq, int Lmax) {
    // the sizes the selection calls accept
    if (B <= 0 || Hq <= 0 || Lmax <= 0 || (long long)B * Hq > 65535 || Lmax > (1 << 24)) return 0;
    return tb::select_ws_layout(B, Hq, Lmax, nullptr, nullptr);
}

namespace {

// Checks shared by tb_select and tb_score_select (fn names the caller in the
// error detail); fills ws.
tb_status check_select(const char *fn, const int32_t *ctx_len, const int32_t *proj_len, int B,
                       int Hq, int Lmax, int sink, int window, int budget, int radius, int mode,
                       int32_t *idx, int32_t *count, int cap, void *workspace, size_t ws_bytes,
                       tb::SelectWs *ws) {
    TB_REQUIRE(ctx_len && proj_len && idx && count && workspace, TB_ERR_INVALID_ARGUMENT,
               "%s: null pointer", fn);
    TB_REQUIRE(aligned4(ctx_len) && aligned4(proj_len) && aligned4(idx) && aligned4(count) &&
                   aligned16(workspace),
               TB_ERR_INVALID_ARGUMENT, "%s: misaligned pointer", fn);
    TB_REQUIRE(B >= 1 && Hq >= 1 && (long long)B * Hq <= 65535 && Lmax >= 1,
               TB_ERR_INVALID_ARGUMENT, "%s: bad sizes B=%d Hq=%d Lmax=%d", fn, B, Hq, Lmax);
    TB_REQUIRE(Lmax <= (1 << 24), TB_ERR_UNSUPPORTED_SHAPE, "%s: Lmax > 2^24", fn);
    TB_REQUIRE(sink >= 0 && window >= 0 && budget >= 0 && radius >= 0, TB_ERR_INVALID_ARGUMENT,
               "%s: negative sink/window/budget/radius", fn);
    TB_REQUIRE(radius <= 64, TB_ERR_UNSUPPORTED_SHAPE, "%s: radius > 64", fn);
    TB_REQUIRE((mode & ~(0xff | TB_SEL_OMIT_WINDOW | TB_SEL_DEFER_LIST | TB_SEL_DEFER_SELECT)) == 0,
               TB_ERR_INVALID_ARGUMENT, "%s: unknown mode bits 0x%x", fn, mode);
    TB_REQUIRE((mode & 0xff) == TB_NF_FILL || (mode & 0xff) == TB_NF_DILATE,
               TB_ERR_INVALID_ARGUMENT, "%s: unknown neighbour mode %d", fn, mode & 0xff);
    TB_REQUIRE(!((mode & (TB_SEL_DEFER_LIST | TB_SEL_DEFER_SELECT)) &&
                 (mode & 0xff) == TB_NF_DILATE),
               TB_ERR_INVALID_ARGUMENT, "%s: TB_SEL_DEFER_LIST / TB_SEL_DEFER_SELECT need TB_NF_FILL",
               fn);
    const bool omit = (mode & TB_SEL_OMIT_WINDOW) != 0;
    const bool dilate = (mode & 0xff) == TB_NF_DILATE;
    const long long imp = dilate ? (2LL * radius + 1) * budget : (long long)budget;
    const long long need_cap = (long long)sink + (omit ? 0 : window) + imp;
    const long long min_cap = need_cap < Lmax ? need_cap : Lmax;
    TB_REQUIRE(cap >= 1 && cap >= min_cap, TB_ERR_INVALID_ARGUMENT,
               "%s: cap %d < min(Lmax, sink + important (+ window unless omitted)) = %lld", fn,
               cap, min_cap);
    const size_t need = tb_select_workspace_bytes(B, Hq, Lmax);
    TB_REQUIRE(ws_bytes >= need, TB_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu < %zu bytes", fn,
               ws_bytes, need);
    tb::select_ws_layout(B, Hq, Lmax, workspace, ws);
    return TB_OK;
}

}  // namespace

tb_status tb_select(const float *scores, const int32_t *ctx_len, const int32_t *proj_len, int B,
                    int Hq, int Lmax, int sink, int window, int budget, int radius, int mode,
                    int32_t *idx, int32_t *count, int cap, void *workspace, size_t ws_bytes,
                    void *stream) {
    TB_REQUIRE(scores, TB_ERR_INVALID_ARGUMENT, "tb_select: null pointer");
    TB_REQUIRE(aligned4(scores), TB_ERR_INVALID_ARGUMENT, "tb_select: misaligned pointer");
    TB_REQUIRE((mode & TB_SEL_DEFER_SELECT) == 0, TB_ERR_INVALID_ARGUMENT,
               "tb_select: TB_SEL_DEFER_SELECT is a mode of tb_score_select only");
    tb::SelectWs ws;
    const tb_status e = check_select("tb_select", ctx_len, proj_len, B, Hq, Lmax, sink, window,
                                     budget, radius, mode, idx, count, cap, workspace, ws_bytes,
                                     &ws);
    if (e) return e;
    return tb::launch_select(scores, ctx_len, proj_len, B, Hq, Lmax, sink, window, budget, radius,
                             (mode & 0xff) == TB_NF_DILATE, (mode & TB_SEL_OMIT_WINDOW) != 0, idx,
                             count, cap, ws, static_cast<hipStream_t>(stream),
                             (mode & TB_SEL_DEFER_LIST) != 0);
}

tb_status tb_score_select(const float *qhat, int n_slots, int slot, const void *kp,
                          const int32_t *ctx_len, const int32_t *proj_len, float *scores, int B,
                          int Hq, int Hkv, int Lmax, int dp, int sink, int window, int budget,
                          int radius, int mode, int32_t *idx, int32_t *count, int cap,
                          void *workspace, size_t ws_bytes, void *stream) {
    TB_REQUIRE(qhat && kp && scores, TB_ERR_INVALID_ARGUMENT, "tb_score_select: null pointer");
    TB_REQUIRE(aligned4(qhat) && aligned16(kp) && aligned4(scores), TB_ERR_INVALID_ARGUMENT,
               "tb_score_select: misaligned pointer");
    TB_REQUIRE(Hkv >= 1 && Hkv <= 65535 && n_slots >= 1 && slot >= 0 && slot < n_slots,
               TB_ERR_INVALID_ARGUMENT, "tb_score_select: bad sizes");
    TB_REQUIRE(Hq >= 1 && Hq % Hkv == 0, TB_ERR_INVALID_ARGUMENT,
               "tb_score_select: Hq %% Hkv != 0");
    TB_REQUIRE(Hq / Hkv <= 8 && (dp == 16 || dp == 32), TB_ERR_UNSUPPORTED_SHAPE,
               "tb_score_select: need Hq/Hkv <= 8 and dp in {16, 32}");
    tb::SelectWs ws;
    const tb_status e = check_select("tb_score_select", ctx_len, proj_len, B, Hq, Lmax, sink,
                                     window, budget, radius, mode, idx, count, cap, workspace,
                                     ws_bytes, &ws);
    if (e) return e;
    return tb::launch_score_select(qhat, n_slots, slot, kp, ctx_len, proj_len, scores, B, Hq, Hkv,
                                   Lmax, dp, sink, window, budget, radius,
                                   (mode & 0xff) == TB_NF_DILATE,
                                   (mode & TB_SEL_OMIT_WINDOW) != 0, idx, count, cap, ws,
                                   static_cast<hipStream_t>(stream),
                                   (mode & TB_SEL_DEFER_LIST) != 0,
                                   (mode & TB_SEL_DEFER_SELECT) != 0);
}

tb_status tb_select_attn(const int32_t *ctx_len, const int32_t *proj_len, int B, int Hq, int Hkv,
                         int Lmax, int sink, int window, int budget, int radius, int mode,
                         int32_t *idx, int32_t *count, int cap, void *sel_workspace,
                         size_t sel_ws_bytes, const void *q, const void *k_cache,
                         const void *v_cache, int D, float scale, float *out,
                         void *attn_workspace, size_t attn_ws_bytes, void *stream) {
    TB_REQUIRE(q && k_cache && v_cache && out && attn_workspace, TB_ERR_INVALID_ARGUMENT,
               "tb_select_attn: null pointer");
    TB_REQUIRE(aligned16(q) && aligned16(k_cache) && aligned16(v_cache) && aligned4(out) &&
                   aligned16(attn_workspace),
               TB_ERR_INVALID_ARGUMENT, "tb_select_attn: misaligned pointer");
    TB_REQUIRE(Hkv >= 1 && Hq % Hkv == 0 && Hq / Hkv <= 65535, TB_ERR_INVALID_ARGUMENT,
               "tb_select_attn: Hq %% Hkv != 0");
    TB_REQUIRE(D == 64 || D == 128, TB_ERR_UNSUPPORTED_SHAPE, "tb_select_attn: D must be 64 or 128");
    TB_REQUIRE((long long)Lmax * D * 2 <= 0x7fffffffLL, TB_ERR_UNSUPPORTED_SHAPE,
               "tb_select_attn: one head's cache must be below 2 GiB (Lmax * D * 2)");
    TB_REQUIRE(scale == scale, TB_ERR_INVALID_ARGUMENT, "tb_select_attn: scale is NaN");
    TB_REQUIRE((mode & (TB_SEL_DEFER_LIST | TB_SEL_DEFER_SELECT)) != 0, TB_ERR_INVALID_ARGUMENT,
               "tb_select_attn: mode must carry TB_SEL_DEFER_LIST or TB_SEL_DEFER_SELECT, as the "
               "selection it follows");
    tb::SelectWs ws;
    const tb_status e = check_select("tb_select_attn", ctx_len, proj_len, B, Hq, Lmax, sink, window,
                                     budget, radius, mode, idx, count, cap, sel_workspace,
                                     sel_ws_bytes, &ws);
    if (e) return e;
    const size_t need = tb_attn_workspace_bytes(B, Hq, cap, 0, D);
    TB_REQUIRE(need > 0, TB_ERR_UNSUPPORTED_SHAPE, "tb_select_attn: B * Hq * splits beyond INT_MAX");
    TB_REQUIRE(attn_ws_bytes >= need, TB_ERR_WORKSPACE_TOO_SMALL,
               "tb_select_attn: attention workspace %zu < %zu bytes", attn_ws_bytes, need);
    float *part;
    uint32_t *ctr;
    tb::attn_ws_layout(B, Hq, cap, D, attn_workspace, &part, &ctr);
    if ((mode & TB_SEL_DEFER_SELECT) &&
        tb::defer_select_fits(B, Hq, Hkv, Lmax, radius,
                              (mode & TB_SEL_OMIT_WINDOW) ? 0 : window, cap, ws))
        return tb::launch_hist_attn(ctx_len, proj_len, B, Hq, Hkv, Lmax, sink, window, budget,
                                    radius, (mode & TB_SEL_OMIT_WINDOW) != 0, idx, count, cap, ws,
                                    q, k_cache, v_cache, D, scale, out, part, ctr,
                                    static_cast<hipStream_t>(stream));
    return tb::launch_select_attn(ctx_len, proj_len, B, Hq, Hkv, Lmax, sink, window, budget,
                                  (mode & TB_SEL_OMIT_WINDOW) != 0, idx, count, cap, ws, q,
                                  k_cache, v_cache, D, scale, out, part, ctr,
                                  static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------- attention
size_t tb_attn_workspace_bytes(int B, int Hq, int cap, int window, int D) {
    if (B <= 0 || Hq <= 0 || cap <= 0 || window < 0 || (D != 64 && D != 128)) return 0;
    // the sizes the attention calls accept: cap + window and the grid
    // (B * Hq * splits workgroups, rounded up to 8) within INT_MAX
    const long long rows = (long long)cap + window;
    if (rows > 0x7fffffffLL || (long long)B * Hq > 0x7fffffffLL) return 0;
    const long long items = (long long)B * Hq * tb::attn_nsplit((int)rows);
    if (items > 0x7fffffffLL - 7) return 0;
    return tb::attn_ws_layout(B, Hq, (int)rows, D, nullptr, nullptr, nullptr);
}

tb_status tb_sparse_decode_attn(const void *q, const void *k_cache, const void *v_cache,
                                const int32_t *idx, const int32_t *count, int cap,
                                const int32_t *ctx_len, int window, int B, int Hq, int Hkv,
                                int Lmax, int D, float scale, float *out, void *workspace,
                                size_t ws_bytes, void *stream) {
    TB_REQUIRE(q && k_cache && v_cache && idx && count && out && workspace,
               TB_ERR_INVALID_ARGUMENT, "tb_sparse_decode_attn: null pointer");
    TB_REQUIRE(aligned16(q) && aligned16(k_cache) && aligned16(v_cache) && aligned4(idx) &&
                   aligned4(count) && aligned4(out) && aligned16(workspace) && aligned4(ctx_len),
               TB_ERR_INVALID_ARGUMENT, "tb_sparse_decode_attn: misaligned pointer");
    TB_REQUIRE(B >= 1 && Hq >= 1 && Hkv >= 1 && Lmax >= 1 && cap >= 1 && window >= 0,
               TB_ERR_INVALID_ARGUMENT, "tb_sparse_decode_attn: bad sizes");
    TB_REQUIRE(Hq % Hkv == 0, TB_ERR_INVALID_ARGUMENT, "tb_sparse_decode_attn: Hq %% Hkv != 0");
    TB_REQUIRE(D == 64 || D == 128, TB_ERR_UNSUPPORTED_SHAPE,
               "tb_sparse_decode_attn: D must be 64 or 128");
    TB_REQUIRE((long long)Lmax * D * 2 <= 0x7fffffffLL, TB_ERR_UNSUPPORTED_SHAPE,
               "tb_sparse_decode_attn: one head's cache must be below 2 GiB (Lmax * D * 2)");
    TB_REQUIRE(scale == scale, TB_ERR_INVALID_ARGUMENT, "tb_sparse_decode_attn: scale is NaN");
    const int win = ctx_len ? window : 0;
    const size_t need = tb_attn_workspace_bytes(B, Hq, cap, win, D);
    TB_REQUIRE(need > 0, TB_ERR_UNSUPPORTED_SHAPE,
               "tb_sparse_decode_attn: cap + window or B * Hq * splits beyond INT_MAX");
    TB_REQUIRE(ws_bytes >= need, TB_ERR_WORKSPACE_TOO_SMALL,
               "tb_sparse_decode_attn: workspace %zu < %zu bytes", ws_bytes, need);
    float *part;
    uint32_t *ctr;
    tb::attn_ws_layout(B, Hq, cap + win, D, workspace, &part, &ctr);
    return tb::launch_attn(q, k_cache, v_cache, idx, count, cap, ctx_len, win, B, Hq, Hkv, Lmax,
                           D, scale, out, part, ctr, static_cast<hipStream_t>(stream));
}

tb_status tb_append_attn(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                         void *kp, const void *wk, int32_t *ctx_len, int32_t *proj_len, int n_p,
                         const void *q, const int32_t *idx, const int32_t *count, int cap,
                         int window, int B, int Hq, int Hkv, int Lmax, int D, int dp, float scale,
                         float *out, void *workspace, size_t ws_bytes, void *stream) {
    TB_REQUIRE(k_new && v_new && k_cache && v_cache && kp && wk && ctx_len && proj_len && q &&
                   idx && count && out && workspace,
               TB_ERR_INVALID_ARGUMENT, "tb_append_attn: null pointer");
    TB_REQUIRE(aligned16(k_new) && aligned16(v_new) && aligned16(k_cache) && aligned16(v_cache) &&
                   aligned16(kp) && aligned16(wk) && aligned4(ctx_len) && aligned4(proj_len) &&
                   aligned16(q) && aligned4(idx) && aligned4(count) && aligned4(out) &&
                   aligned16(workspace),
               TB_ERR_INVALID_ARGUMENT, "tb_append_attn: misaligned pointer");
    TB_REQUIRE(B >= 1 && B <= 65535 && Hq >= 1 && Hkv >= 1 && Hkv <= 65535 && Lmax >= 1 &&
                   cap >= 1 && window >= 0 && n_p >= 1,
               TB_ERR_INVALID_ARGUMENT, "tb_append_attn: bad sizes");
    TB_REQUIRE(Hq % Hkv == 0, TB_ERR_INVALID_ARGUMENT, "tb_append_attn: Hq %% Hkv != 0");
    TB_REQUIRE((D == 64 || D == 128) && (dp == 16 || dp == 32), TB_ERR_UNSUPPORTED_SHAPE,
               "tb_append_attn: D must be 64 or 128 and dp 16 or 32 (got %d, %d)", D, dp);
    TB_REQUIRE((long long)Lmax * D * 2 <= 0x7fffffffLL, TB_ERR_UNSUPPORTED_SHAPE,
               "tb_append_attn: one head's cache must be below 2 GiB (Lmax * D * 2)");
    TB_REQUIRE(scale == scale, TB_ERR_INVALID_ARGUMENT, "tb_append_attn: scale is NaN");
    const size_t need = tb_attn_workspace_bytes(B, Hq, cap, window, D);
    TB_REQUIRE(need > 0, TB_ERR_UNSUPPORTED_SHAPE,
               "tb_append_attn: cap + window or B * Hq * splits beyond INT_MAX");
    TB_REQUIRE(ws_bytes >= need, TB_ERR_WORKSPACE_TOO_SMALL,
               "tb_append_attn: workspace %zu < %zu bytes", ws_bytes, need);
    float *part;
    uint32_t *ctr, *bctr;
    tb::attn_ws_layout(B, Hq, cap + window, D, workspace, &part, &ctr, &bctr);
    return tb::launch_append_attn(k_new, v_new, k_cache, v_cache, kp, wk, ctx_len, proj_len, n_p,
                                  q, idx, count, cap, window, B, Hq, Hkv, Lmax, D, dp, scale, out,
                                  part, ctr, bctr, static_cast<hipStream_t>(stream));
}

}  // extern "C"
