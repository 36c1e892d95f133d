// Key projection body shared by the projection launch and the fused
// predict + project launch (see project.hip for the method notes).
#pragma once

#include "tb_common.h"

namespace tb {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kProjThreads = 256;
constexpr int kProjTokPerWave = 16;
constexpr int kProjTokPerBlock = (kProjThreads / 64) * kProjTokPerWave;

// Workgroup `blk` of the projection of rows [pos0[b], pos0[b] + ntok) of
// KV head kvh: each wave projects 16 tokens.
template <int D, int DP>
__device__ __forceinline__ void project_block(const uint16_t *__restrict__ kc,
                                              const uint16_t *__restrict__ wk,
                                              uint16_t *__restrict__ kp,
                                              const int32_t *__restrict__ pos0, int ntok, int Hkv,
                                              int Lmax, int blk, int kvh, int b) {
    constexpr int NV = D / 32;   // 16-byte vectors per lane per row (= MFMAs per channel tile)
    constexpr int MT = DP / 16;  // channel tiles
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, kq = lane >> 4;
    const int p0 = pos0[b];
    const int t = p0 + (blk * (kProjThreads / 64) + wave) * kProjTokPerWave + n;
    const int run = blk * kProjTokPerBlock + wave * kProjTokPerWave;
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
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < NV; ++v)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wrow[v]),
                                                          __builtin_bit_cast(bf16x8_t, kv[v]), acc,
                                                          0, 0, 0);
        // acc[i] = channel mt*16 + 4*kq + i of token t
        if (valid) {
            const uint32_t lo = f32_to_f16_bits(acc[0]) | (f32_to_f16_bits(acc[1]) << 16);
            const uint32_t hi = f32_to_f16_bits(acc[2]) | (f32_to_f16_bits(acc[3]) << 16);
            *reinterpret_cast<uint2 *>(kp + (head * Lmax + t) * DP + mt * 16 + 4 * kq) =
                make_uint2(lo, hi);
        }
    }
}

}  // namespace tb
