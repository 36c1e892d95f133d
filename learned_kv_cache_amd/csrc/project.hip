// Key-cache projection into the predictor's low-dimensional space
// ("TokenButler" summary, "Core architecture": key-cache projection by a
// learned matrix; "Inference strategy": done once per batch of new tokens).
//
// kp[t, c] = fp16( sum_i K[t, i] * Wk[c, i] ) for a run of tokens of one
// (sequence, KV head). MFMA 16x16x32 bf16 -> fp32 with A = Wk rows (16
// channels) and B = K rows (16 tokens), so each lane's accumulator holds four
// consecutive channels of one token and is stored as one 8-byte fp16 packet.
// Each lane reads D/4 contiguous elements of its token row (the reduction
// index is permuted identically in A and B, which leaves the sum unchanged),
// so a row is fetched as full 64-byte (D = 128) or 32-byte (D = 64) pieces.
#include "project_impl.h"

namespace tb {
namespace {

// Bulk projection (whole-context prefill): each wave keeps its W_k
// fragments in registers and walks kBulkIter batches of 16 tokens with the
// rows of the next NBUF - 1 batches in flight, so the weights are read once
// per 64 tokens instead of once per 16.
constexpr int kBulkIter = 4;
constexpr int kBulkTokPerWave = kBulkIter * 16;
constexpr int kBulkTokPerBlock = (kProjThreads / 64) * kBulkTokPerWave;
constexpr int kBulkMinTokens = 2048;

template <int D, int DP>
__global__ __launch_bounds__(kProjThreads) void project_bulk_kernel(
    const uint16_t *__restrict__ kc, const uint16_t *__restrict__ wk, uint16_t *__restrict__ kp,
    const int32_t *__restrict__ pos0, int ntok, int Hkv, int Lmax) {
    constexpr int NV = D / 32;
    constexpr int MT = DP / 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, kq = lane >> 4;
    const int kvh = blockIdx.y, b = blockIdx.z;
    const int base = blockIdx.x * kBulkTokPerBlock + wave * kBulkTokPerWave;
    if (base >= ntok) return;
    const int p0 = pos0[b];
    const size_t head = (size_t)(b * Hkv + kvh);
    uint4 w[MT][NV];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const uint4 *wrow = reinterpret_cast<const uint4 *>(
            wk + ((size_t)kvh * DP + mt * 16 + n) * D + kq * (D / 4));
#pragma unroll
        for (int v = 0; v < NV; ++v) w[mt][v] = wrow[v];
    }
    constexpr int NBUF = 3;   // batches in flight per wave
    uint4 kv[NBUF][NV];
    auto load = [&](int it, uint4 (&dst)[NV]) {
        const int run = base + it * 16 + n;
        const int t = p0 + run;
        if (run < ntok && t >= 0 && t < Lmax) {
            const uint4 *row =
                reinterpret_cast<const uint4 *>(kc + (head * Lmax + t) * D + kq * (D / 4));
#pragma unroll
            for (int v = 0; v < NV; ++v) dst[v] = row[v];
        } else {
#pragma unroll
            for (int v = 0; v < NV; ++v) dst[v] = make_uint4(0, 0, 0, 0);
        }
    };
#pragma unroll
    for (int it = 0; it < NBUF - 1; ++it) load(it, kv[it]);
#pragma unroll
    for (int it = 0; it < kBulkIter; ++it) {
        if (base + it * 16 >= ntok) break;
        if (it + NBUF - 1 < kBulkIter) load(it + NBUF - 1, kv[(it + NBUF - 1) % NBUF]);
        const uint4 *cur = kv[it % NBUF];
        const int run = base + it * 16 + n;
        const int t = p0 + run;
        const bool valid = run < ntok && t >= 0 && t < Lmax;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int v = 0; v < NV; ++v)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, w[mt][v]),
                                                              __builtin_bit_cast(bf16x8_t, cur[v]),
                                                              acc, 0, 0, 0);
            // acc[i] = channel mt*16 + 4*kq + i of token t
            if (valid) {
                const uint32_t lo = f32_to_f16_bits(acc[0]) | (f32_to_f16_bits(acc[1]) << 16);
                const uint32_t hi = f32_to_f16_bits(acc[2]) | (f32_to_f16_bits(acc[3]) << 16);
                *reinterpret_cast<uint2 *>(kp + (head * Lmax + t) * DP + mt * 16 + 4 * kq) =
                    make_uint2(lo, hi);
            }
        }
    }
}

template <int D, int DP>
__global__ __launch_bounds__(kProjThreads) void project_kernel(
    const uint16_t *__restrict__ kc, const uint16_t *__restrict__ wk, uint16_t *__restrict__ kp,
    const int32_t *__restrict__ pos0, int ntok, int Hkv, int Lmax) {
    project_block<D, DP>(kc, wk, kp, pos0, ntok, Hkv, Lmax, blockIdx.x, blockIdx.y, blockIdx.z);
}

// Decode-step append with batched projection, one workgroup per sequence
// (append_rows), then the lengths are advanced.
template <int D, int DP>
__global__ __launch_bounds__(kProjThreads) void append_kernel(
    const uint16_t *__restrict__ k_new, const uint16_t *__restrict__ v_new,
    uint16_t *__restrict__ kc, uint16_t *__restrict__ vc, uint16_t *__restrict__ kp,
    const uint16_t *__restrict__ wk, int32_t *__restrict__ ctx, int32_t *__restrict__ plen,
    int Hkv, int Lmax, int n_p) {
    const int b = blockIdx.x;
    const int L = ctx[b], P = plen[b];
    if (!append_applies(L, P, Lmax)) return;
    const bool proj = append_rows<D, DP, kProjThreads>(k_new, v_new, kc, vc, kp, wk, b, L, P, Hkv,
                                                      Lmax, n_p);
    __syncthreads();
    if (threadIdx.x == 0) {
        ctx[b] = L + 1;
        if (proj) plen[b] = L + 1;
    }
}

}  // namespace

tb_status launch_project(const void *kc, const void *wk, void *kp, const int32_t *pos0, int ntok,
                         int B, int Hkv, int Lmax, int D, int dp, hipStream_t st) {
    if (ntok == 0) return TB_OK;
    const bool bulk = ntok >= kBulkMinTokens;
    const int per = bulk ? kBulkTokPerBlock : kProjTokPerBlock;
    dim3 grid((ntok + per - 1) / per, Hkv, B);
    const uint16_t *k = static_cast<const uint16_t *>(kc);
    const uint16_t *w = static_cast<const uint16_t *>(wk);
    uint16_t *o = static_cast<uint16_t *>(kp);
#define TB_P(DD, PP)                                                                        \
    if (D == DD && dp == PP) {                                                              \
        if (bulk)                                                                           \
            hipLaunchKernelGGL((project_bulk_kernel<DD, PP>), grid, dim3(kProjThreads), 0, st, k, \
                               w, o, pos0, ntok, Hkv, Lmax);                                \
        else                                                                                \
            hipLaunchKernelGGL((project_kernel<DD, PP>), grid, dim3(kProjThreads), 0, st, k, w, \
                               o, pos0, ntok, Hkv, Lmax);                                   \
        return check_launch("tb_project_keys");                                             \
    }
    TB_P(128, 32) TB_P(128, 16) TB_P(64, 32) TB_P(64, 16)
#undef TB_P
    set_error("tb_project_keys: unsupported D=%d dp=%d", D, dp);
    return TB_ERR_UNSUPPORTED_SHAPE;
}

tb_status launch_append(const void *k_new, const void *v_new, void *kc, void *vc, void *kp,
                        const void *wk, int32_t *ctx, int32_t *plen, int B, int Hkv, int Lmax,
                        int D, int dp, int n_p, hipStream_t st) {
    const uint16_t *kn = static_cast<const uint16_t *>(k_new);
    const uint16_t *vn = static_cast<const uint16_t *>(v_new);
    uint16_t *k = static_cast<uint16_t *>(kc);
    uint16_t *v = static_cast<uint16_t *>(vc);
    uint16_t *o = static_cast<uint16_t *>(kp);
    const uint16_t *w = static_cast<const uint16_t *>(wk);
#define TB_A(DD, PP)                                                                        \
    if (D == DD && dp == PP) {                                                              \
        hipLaunchKernelGGL((append_kernel<DD, PP>), dim3(B), dim3(kProjThreads), 0, st, kn, vn, k, \
                           v, o, w, ctx, plen, Hkv, Lmax, n_p);                             \
        return check_launch("tb_append_kv");                                                \
    }
    TB_A(128, 32) TB_A(128, 16) TB_A(64, 32) TB_A(64, 16)
#undef TB_A
    set_error("tb_append_kv: unsupported D=%d dp=%d", D, dp);
    return TB_ERR_UNSUPPORTED_SHAPE;
}

}  // namespace tb
