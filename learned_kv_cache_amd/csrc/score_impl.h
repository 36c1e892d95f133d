// Importance score of one projected-key row ("TokenButler" summary, "Core
// architecture": scoring is the dot product of the predicted query with the
// projected key). Shared by the scoring kernel and the selection's band
// sampling, which recomputes scores of sampled positions from the projected
// keys: both must produce the same fp32 bits, so the products are summed in
// one fixed order (channel 0 first, one fused multiply-add per channel).
#pragma once
#include "tb_common.h"

namespace tb {

// raw: the row's DP fp16 values as DP / 8 16-byte vectors; q: DP floats.
template <int DP>
__device__ __forceinline__ float score_row(const uint4 (&raw)[DP / 8], const float *q) {
    float acc = 0.f;
#pragma unroll
    for (int v = 0; v < DP / 8; ++v) {
        const uint32_t w[4] = {raw[v].x, raw[v].y, raw[v].z, raw[v].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc = __builtin_fmaf(f16_lo(w[e]), q[v * 8 + 2 * e], acc);
            acc = __builtin_fmaf(f16_hi(w[e]), q[v * 8 + 2 * e + 1], acc);
        }
    }
    return acc;
}

}  // namespace tb
