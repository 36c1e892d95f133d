// Internal helpers shared by the libtb translation units (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tb.h"

namespace tb {

// ---- error reporting (tb_api.hip) ------------------------------------------
void set_error(const char *fmt, ...);
tb_status check_launch(const char *what);

#define TB_REQUIRE(cond, code, ...)        \
    do {                                    \
        if (!(cond)) {                      \
            ::tb::set_error(__VA_ARGS__);   \
            return (code);                  \
        }                                   \
    } while (0)

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// ---- storage formats -------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// Round-to-nearest-even float -> bfloat16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float f16_lo(uint32_t pair) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(pair & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t pair) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(pair >> 16));
}
// Round-to-nearest-even float -> binary16 bits (hardware conversion).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// ---- cross-lane sums within aligned groups of 4 / 8 / 16 lanes (DPP) --------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// quad_perm [1,0,3,2] = xor 1; [2,3,0,1] = xor 2; row_half_mirror; row_mirror
template <int LANES>
__device__ __forceinline__ float group_sum(float v) {
    v += dpp_f<0xb1>(v);
    v += dpp_f<0x4e>(v);
    if constexpr (LANES >= 8) v += dpp_f<0x141>(v);
    if constexpr (LANES >= 16) v += dpp_f<0x140>(v);
    return v;
}

// IEEE totalOrder key of a finite float: larger key <=> larger in totalOrder
// (so -0 sorts below +0).
__device__ __forceinline__ uint32_t order_key(float s) {
    uint32_t u = __float_as_uint(s);
    return u ^ ((u >> 31) ? 0xffffffffu : 0x80000000u);
}

}  // namespace tb

// ---- launchers (one per translation unit) ------------------------------------
namespace tb {
tb_status launch_predict(const void *x, const void *w1, const void *w2, float *qhat, int B, int E,
                         int Eh, int n_out, void *ws, int nsplit, hipStream_t st);
int predict_nsplit(int E, int Eh);
tb_status launch_predict_project(const void *x, const void *w1, const void *w2, float *qhat,
                                 int B, int E, int Eh, int n_out, void *ws, int nsplit,
                                 const void *kc, const void *wk, void *kp, const int32_t *pos0,
                                 int ntok, int Hkv, int Lmax, int D, int dp, hipStream_t st);
tb_status launch_append(const void *k_new, const void *v_new, void *kc, void *vc, void *kp,
                        const void *wk, int32_t *ctx, int32_t *plen, int B, int Hkv, int Lmax,
                        int D, int dp, int n_p, hipStream_t st);
bool host_to_device(const void *ptr, const void **dev);
int distill_ngroups(int R, int g);
size_t distill_ws_layout(int B, int R, int Hq, int Hkv, int Lmax, void *base, float **part,
                         uint32_t **ctr);
tb_status launch_distill(const void *q, const void *kc, const float *qhat, const void *kp,
                         const int32_t *pos, int B, int R, int Hq, int Hkv, int Lmax, int D,
                         int dp, float scale, float *part, uint32_t *ctr, float *loss,
                         hipStream_t st);
tb_status launch_offload_gather(const void *kh, const void *vh, int B, int Hkv, int Lmax, int D,
                                const int32_t *idx, const int32_t *count, int cap, int Hq,
                                void *kb, void *vb, int buf_rows, int slot0, int wrap,
                                hipStream_t st);
tb_status launch_offload_append(const void *k_new, const void *v_new, const void *wk, void *kh,
                                void *vh, void *kp, int32_t *ctx, int32_t *plen, int B, int Hkv,
                                int Lmax, int D, int dp, void *kb, void *vb, int Hq,
                                int buf_rows, int window, hipStream_t st);
tb_status launch_project(const void *kc, const void *wk, void *kp, const int32_t *pos0, int ntok,
                         int B, int Hkv, int Lmax, int D, int dp, hipStream_t st);
tb_status launch_score(const float *qhat, int n_slots, int slot, const void *kp,
                       const int32_t *plen, float *scores, int B, int Hq, int Hkv, int Lmax,
                       int dp, hipStream_t st);
struct SelectWs {
    uint32_t *bctr;      // [nseg] arrival counters of the band workgroups, zero at rest
    uint32_t *info;      // [nseg][2] band [T_lo, T_hi] of key32 around the budget's key
    uint32_t *ccount;    // [nseg][nchunks] candidates per chunk
    uint32_t *acount;    // [nseg][nchunks] tokens above the band per chunk
    uint32_t *coff;      // [nseg][nchunks] offset of each chunk in the output list
    uint64_t *thr;       // [nseg] threshold key among the candidates (~0: none chosen)
    uint32_t *bitmap;    // [nseg][nwords]
    uint64_t *cand;      // [nseg][Lmax], chunk c owns slots [c * CHUNK, ...)
    uint32_t *samp;      // [nseg][8192] sampled pooled key32
    uint32_t *dbm;       // [nseg][nwords] widened bitmap (dilation mode)
    uint32_t *dcount;    // [nseg][nchunks] widened tokens per chunk (dilation mode)
    uint32_t *hist;      // [2][nseg][4096] the histogram route's two histograms, zero
                         // at rest (null off that route's sizes)
    uint32_t *hinfo;     // [nseg][3] the histogram route's bin B*, tokens above it, in it
    int nwords;
    int nchunks;
};
size_t select_ws_layout(int B, int Hq, int Lmax, void *base, SelectWs *out);
// The histogram route of tb_score_select (select_hist.hip): at most
// kHistMaxSeg segments (b, query head), contexts above kHistMinL tokens
// (below it the sampled band holds every token and is exact) up to 64 chunks
// of 2048 tokens, radius <= 2 (0 in the dilation mode), at most 4 query heads
// per KV head.
constexpr int kHistMinL = 8192;
constexpr int kHistMaxSeg = 64;
bool hist_route_fits(int nseg, int Lmax, int g, int r, bool dilate);
size_t hist_ws_bytes(int B, int Hq, int Lmax);
tb_status launch_score_hist_select(const float *qhat, int n_slots, int slot, const void *kp,
                                   const int32_t *ctx, const int32_t *plen, float *scores, int B,
                                   int Hq, int Hkv, int Lmax, int dp, int S, int W, int K, int r,
                                   bool dilate, bool omit_window, int32_t *count,
                                   const SelectWs &ws, hipStream_t st, bool pass_only = false);
// The split form of tb_score_select + tb_select_attn (TB_SEL_DEFER_SELECT):
// on the histogram route, with chunk-aligned attention splits that fit the
// attention workspace of cap rows; both calls decide it alike.
bool defer_select_fits(int B, int Hq, int Hkv, int Lmax, int r, int win, int cap,
                       const SelectWs &ws);
tb_status launch_hist_attn(const int32_t *ctx, const int32_t *plen, int B, int Hq, int Hkv,
                           int Lmax, int S, int W, int K, int r, bool omit_window, int32_t *idx,
                           int32_t *count, int cap, const SelectWs &ws, const void *q,
                           const void *kc, const void *vc, int D, float scale, float *out,
                           float *part, uint32_t *ctr, hipStream_t st);
tb_status launch_select(const float *scores, const int32_t *ctx, const int32_t *plen, int B,
                        int Hq, int Lmax, int S, int W, int K, int r, bool dilate,
                        bool omit_window, int32_t *idx, int32_t *count, int cap,
                        const SelectWs &ws, hipStream_t st, bool defer_list = false);
tb_status launch_score_select(const float *qhat, int n_slots, int slot, const void *kp,
                              const int32_t *ctx, const int32_t *plen, float *scores, int B,
                              int Hq, int Hkv, int Lmax, int dp, int S, int W, int K, int r,
                              bool dilate, bool omit_window, int32_t *idx, int32_t *count,
                              int cap, const SelectWs &ws, hipStream_t st,
                              bool defer_list = false, bool defer_select = false);
tb_status launch_compact(const int32_t *ctx, const int32_t *plen, int B, int Hq, int Lmax, int S,
                         int W, int K, bool omit_window, int32_t *idx, int cap, const SelectWs &ws,
                         hipStream_t st);
tb_status launch_select_attn(const int32_t *ctx, const int32_t *plen, int B, int Hq, int Hkv,
                             int Lmax, int S, int W, int K, bool omit_window, int32_t *idx,
                             int32_t *count, int cap, const SelectWs &ws, const void *q,
                             const void *kc, const void *vc, int D, float scale, float *out,
                             float *part, uint32_t *ctr, hipStream_t st);
int attn_nsplit(int rows);
size_t attn_ws_layout(int B, int Hq, int rows, int D, void *base, float **part, uint32_t **ctr,
                      uint32_t **bctr = nullptr);
tb_status launch_append_attn(const void *k_new, const void *v_new, void *kc, void *vc, void *kp,
                             const void *wk, int32_t *ctx, int32_t *plen, int n_p, const void *q,
                             const int32_t *idx, const int32_t *count, int cap, int window, int B,
                             int Hq, int Hkv, int Lmax, int D, int dp, float scale, float *out,
                             float *part, uint32_t *ctr, uint32_t *bctr, hipStream_t st);
tb_status launch_attn(const void *q, const void *kc, const void *vc, const int32_t *idx,
                      const int32_t *count, int cap, const int32_t *ctx, int window, int B,
                      int Hq, int Hkv, int Lmax, int D, float scale, float *out, float *part,
                      uint32_t *ctr, hipStream_t st);
}  // namespace tb
