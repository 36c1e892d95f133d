// Scoring: importance = predicted query . projected key, per query head
// ("TokenButler" summary, "Core architecture": scoring).
//
// HBM-streaming GEMV over the fp16 projected-key cache. One lane owns one
// token row (dp halves = 32 or 64 bytes, read as 16-byte loads) and computes
// the dot products of all g query heads that share the row's KV head, so every
// key byte crosses HBM once and the g scores come out as coalesced fp32 rows.
// The g*dp query values are wave-uniform and live in registers.
#include "score_impl.h"

namespace tb {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerThread = 1;
constexpr int kTokPerBlock = kThreads * kRowsPerThread;

template <int G, int DP>
__global__ __launch_bounds__(kThreads) void score_kernel(
    const float *__restrict__ qhat, int q_bstride, int q_off, const uint16_t *__restrict__ kp,
    const int32_t *__restrict__ proj_len, float *__restrict__ scores, int Hq, int Hkv, int Lmax) {
    constexpr int V = DP / 8;  // 16-byte vectors per row
    const int kvh = blockIdx.y, b = blockIdx.z;
    int P = proj_len[b];
    P = P < 0 ? 0 : (P > Lmax ? Lmax : P);
    const int t0 = blockIdx.x * kTokPerBlock + threadIdx.x;
    if (blockIdx.x * kTokPerBlock >= P) return;

    const float *qb = qhat + (size_t)b * q_bstride + q_off + (size_t)kvh * G * DP;
    float q[G][DP];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int c = 0; c < DP; ++c) q[g][c] = qb[g * DP + c];

    const uint4 *kb = reinterpret_cast<const uint4 *>(kp + (size_t)(b * Hkv + kvh) * Lmax * DP);
    float *sb = scores + (size_t)(b * Hq + kvh * G) * Lmax;

    uint4 raw[kRowsPerThread][V];
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
        const int t = t0 + i * kThreads;
        if (t < P) {
#pragma unroll
            for (int v = 0; v < V; ++v) raw[i][v] = kb[(size_t)t * V + v];
        }
    }
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
        const int t = t0 + i * kThreads;
        if (t >= P) continue;
#pragma unroll
        for (int g = 0; g < G; ++g) sb[(size_t)g * Lmax + t] = score_row<DP>(raw[i], q[g]);
    }
}

template <int DP>
tb_status dispatch_g(int g, dim3 grid, hipStream_t st, const float *qhat, int qb, int qo,
                     const uint16_t *kp, const int32_t *pl, float *s, int Hq, int Hkv, int Lmax) {
    switch (g) {
#define TB_G(GG)                                                                              \
    case GG:                                                                                  \
        hipLaunchKernelGGL((score_kernel<GG, DP>), grid, dim3(kThreads), 0, st, qhat, qb, qo, kp, \
                           pl, s, Hq, Hkv, Lmax);                                             \
        break;
        TB_G(1) TB_G(2) TB_G(3) TB_G(4) TB_G(5) TB_G(6) TB_G(7) TB_G(8)
#undef TB_G
        default:
            set_error("tb_score: Hq/Hkv = %d not in [1, 8]", g);
            return TB_ERR_UNSUPPORTED_SHAPE;
    }
    return check_launch("tb_score");
}

}  // namespace

tb_status launch_score(const float *qhat, int n_slots, int slot, const void *kp,
                       const int32_t *plen, float *scores, int B, int Hq, int Hkv, int Lmax,
                       int dp, hipStream_t st) {
    const int g = Hq / Hkv;
    dim3 grid((Lmax + kTokPerBlock - 1) / kTokPerBlock, Hkv, B);
    const int qb = n_slots * Hq * dp, qo = slot * Hq * dp;
    const uint16_t *k = static_cast<const uint16_t *>(kp);
    if (dp == 16) return dispatch_g<16>(g, grid, st, qhat, qb, qo, k, plen, scores, Hq, Hkv, Lmax);
    return dispatch_g<32>(g, grid, st, qhat, qb, qo, k, plen, scores, Hq, Hkv, Lmax);
}

}  // namespace tb
