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
#include "tb_common.h"

namespace tb {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kThreads = 256;
constexpr int kTokPerWave = 16;
constexpr int kTokPerBlock = (kThreads / 64) * kTokPerWave;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int D, int DP>
__global__ __launch_bounds__(kThreads) void project_kernel(
    const uint16_t *__restrict__ kc, const uint16_t *__restrict__ wk, uint16_t *__restrict__ kp,
    const int32_t *__restrict__ pos0, int ntok, int Hkv, int Lmax) {
    constexpr int NV = D / 32;   // 16-byte vectors per lane per row (= MFMAs per channel tile)
    constexpr int MT = DP / 16;  // channel tiles
    const int kvh = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, kq = lane >> 4;
    const int p0 = pos0[b];
    const int t = p0 + (blockIdx.x * (kThreads / 64) + wave) * kTokPerWave + n;
    const int run = blockIdx.x * kTokPerBlock + wave * kTokPerWave;
    if (run >= ntok) return;
    const bool valid = t >= 0 && t < Lmax && t < p0 + ntok;

    const size_t head = (size_t)(b * Hkv + kvh);
    uint4 kv[NV];
    if (valid) {
        const uint4 *row = reinterpret_cast<const uint4 *>(kc + (head * Lmax + t) * D + kq * (D / 4));
#pragma unroll
        for (int v = 0; v < NV; ++v) kv[v] = row[v];
    } else {
#pragma unroll
        for (int v = 0; v < NV; ++v) kv[v] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const uint4 *wrow = reinterpret_cast<const uint4 *>(
            wk + ((size_t)kvh * DP + mt * 16 + n) * D + kq * (D / 4));
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < NV; ++v)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wrow[v]), as_bf16x8(kv[v]),
                                                          acc, 0, 0, 0);
        // acc[i] = channel mt*16 + 4*kq + i of token p0 + ... + n
        if (valid) {
            const uint32_t lo = f32_to_f16_bits(acc[0]) | (f32_to_f16_bits(acc[1]) << 16);
            const uint32_t hi = f32_to_f16_bits(acc[2]) | (f32_to_f16_bits(acc[3]) << 16);
            *reinterpret_cast<uint2 *>(kp + (head * Lmax + t) * DP + mt * 16 + 4 * kq) =
                make_uint2(lo, hi);
        }
    }
}

}  // namespace

tb_status launch_project(const void *kc, const void *wk, void *kp, const int32_t *pos0, int ntok,
                         int B, int Hkv, int Lmax, int D, int dp, hipStream_t st) {
    if (ntok == 0) return TB_OK;
    dim3 grid((ntok + kTokPerBlock - 1) / kTokPerBlock, Hkv, B);
    const uint16_t *k = static_cast<const uint16_t *>(kc);
    const uint16_t *w = static_cast<const uint16_t *>(wk);
    uint16_t *o = static_cast<uint16_t *>(kp);
#define TB_P(DD, PP)                                                                        \
    if (D == DD && dp == PP) {                                                              \
        hipLaunchKernelGGL((project_kernel<DD, PP>), grid, dim3(kThreads), 0, st, k, w, o, pos0, \
                           ntok, Hkv, Lmax);                                                \
        return check_launch("tb_project_keys");                                             \
    }
    TB_P(128, 32) TB_P(128, 16) TB_P(64, 32) TB_P(64, 16)
#undef TB_P
    set_error("tb_project_keys: unsupported D=%d dp=%d", D, dp);
    return TB_ERR_UNSUPPORTED_SHAPE;
}

}  // namespace tb
