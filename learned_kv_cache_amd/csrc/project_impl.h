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

// Whether a decode-step append writes anything for a sequence with lengths
// L = ctx_len[b], P = proj_len[b].
__device__ __forceinline__ bool append_applies(int L, int P, int Lmax) {
    return P >= 0 && P <= L && L < Lmax;
}

// Decode-step append with batched projection, by one workgroup of NT
// threads for sequence b (append_applies(L, P, Lmax) holds): the new K/V
// rows go to position L of every KV head; once the pending keys [P, L + 1)
// number n_p, the waves project them (16 tokens of one head per item, the
// new token's row read from k_new rather than from the cache it is written
// to) and the function returns true. The lengths are the caller's.
template <int D, int DP, int NT>
__device__ __forceinline__ bool append_rows(const uint16_t *__restrict__ k_new,
                                            const uint16_t *__restrict__ v_new,
                                            uint16_t *__restrict__ kc, uint16_t *__restrict__ vc,
                                            uint16_t *__restrict__ kp,
                                            const uint16_t *__restrict__ wk, int b, int L, int P,
                                            int Hkv, int Lmax, int n_p) {
    constexpr int NV = D / 32;   // 16-byte pieces per lane per row
    constexpr int MT = DP / 16;
    constexpr int R16 = D / 8;   // 16-byte pieces per row
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < 2 * Hkv * R16; i += NT) {
        const int which = i / (Hkv * R16), r = i % (Hkv * R16);
        const int j = r / R16, v = r % R16;
        const uint4 *src = reinterpret_cast<const uint4 *>((which ? v_new : k_new) +
                                                           ((size_t)b * Hkv + j) * D) + v;
        uint4 *dst = reinterpret_cast<uint4 *>((which ? vc : kc) +
                                               (((size_t)b * Hkv + j) * Lmax + L) * D) + v;
        *dst = *src;
    }
    const int L1 = L + 1;
    const bool proj = L1 - P >= n_p;
    if (proj) {
        const int n = lane & 15, kq = lane >> 4;
        const int nb = (L1 - P + 15) / 16;
        for (int item = wave; item < Hkv * nb; item += NT / 64) {
            const int j = item / nb, blk = item % nb;
            const int t = P + blk * 16 + n;
            const bool valid = t < L1;
            const size_t head = (size_t)b * Hkv + j;
            uint4 kv[NV];
            if (valid) {
                const uint16_t *rowp = t == L ? k_new + head * D : kc + (head * Lmax + t) * D;
                const uint4 *row = reinterpret_cast<const uint4 *>(rowp + kq * (D / 4));
#pragma unroll
                for (int v = 0; v < NV; ++v) kv[v] = row[v];
            } else {
#pragma unroll
                for (int v = 0; v < NV; ++v) kv[v] = make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint4 *wrow = reinterpret_cast<const uint4 *>(
                    wk + ((size_t)j * DP + mt * 16 + n) * D + kq * (D / 4));
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, wrow[v]), __builtin_bit_cast(bf16x8_t, kv[v]),
                        acc, 0, 0, 0);
                if (valid) {
                    const uint32_t lo = f32_to_f16_bits(acc[0]) | (f32_to_f16_bits(acc[1]) << 16);
                    const uint32_t hi = f32_to_f16_bits(acc[2]) | (f32_to_f16_bits(acc[3]) << 16);
                    *reinterpret_cast<uint2 *>(kp + (head * Lmax + t) * DP + mt * 16 + 4 * kq) =
                        make_uint2(lo, hi);
                }
            }
        }
    }
    return proj;
}

}  // namespace tb
