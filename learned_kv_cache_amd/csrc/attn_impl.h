// Sparse decode attention over one split of a query head's position list:
// the body shared by the attention launch (positions read from the list) and
// the compaction + attention launch (positions rebuilt from the selection's
// bitmap and candidates). The launch notes are in attn.hip.
#pragma once
#include "tb_common.h"

namespace tb {

constexpr int kAttnThreads = 512;
constexpr int kAttnWaves = kAttnThreads / 64;
constexpr int kAttnCH = 256;  // index-list entries per workgroup
// word 3 of a raw (untyped) buffer resource on gfx9-family parts
constexpr int kRsrcWord3 = 0x00020000;

// Log-sum-exp combine of the (max, sum, o[8]) states held by the lanes of a
// wave that own the same 8 channels (lanes equal modulo LPR): a butterfly over
// the lane bits at and above LPR, after which every lane holds the combined
// state of its channels.
template <int LPR>
__device__ inline void combine_lanes(float &m, float &l, float (&o)[8]) {
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
        const float m2 = __shfl_xor(m, off);
        const float l2 = __shfl_xor(l, off);
        const float M = fmaxf(m, m2);
        const float w1 = exp2f(m - M), w2 = exp2f(m2 - M);
        l = l * w1 + l2 * w2;
#pragma unroll
        for (int c = 0; c < 8; ++c) o[c] = o[c] * w1 + __shfl_xor(o[c], off) * w2;
        m = M;
    }
}

// The workgroup's (max, sum, o) state from its lanes' row-group states: the
// partial of split `split` of head bh is stored and, in the last split of the
// head to arrive, all nsplit partials are merged into out. Returns true in
// that last workgroup, after the merge. poison: the split stores a partial
// (sum -1) that makes the head's output 0 whatever the other splits hold.
template <int D>
__device__ __forceinline__ bool attn_store_merge(float m, float l, float (&acc)[8], int nsplit,
                                                 float *__restrict__ part,
                                                 uint32_t *__restrict__ ctr,
                                                 float *__restrict__ out, int bh, int split,
                                                 bool poison = false) {
    constexpr int LPR = D / 8;               // lanes per row
    constexpr int RPW = 64 / LPR;            // row groups per wave
    __shared__ float sm_o[kAttnWaves][D];
    __shared__ float sm_m[kAttnWaves], sm_l[kAttnWaves];
    __shared__ int sm_last;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rg = lane / LPR, cl = lane % LPR;

    // merge the row groups: within each wave by butterfly, then the waves'
    // states through LDS (wave 0)
    combine_lanes<LPR>(m, l, acc);
    if (rg == 0) {
#pragma unroll
        for (int c = 0; c < 8; ++c) sm_o[wave][cl * 8 + c] = acc[c];
        if (cl == 0) {
            sm_m[wave] = m;
            sm_l[wave] = l;
        }
    }
    __syncthreads();
    float *pp = part + ((size_t)bh * nsplit + split) * (D + 2);
    if (wave == 0) {
        float M = -1e30f;
#pragma unroll
        for (int i = 0; i < kAttnWaves; ++i) M = fmaxf(M, sm_m[i]);
        float Ls = 0.f;
        float O[D / 64];
#pragma unroll
        for (int j = 0; j < D / 64; ++j) O[j] = 0.f;
#pragma unroll
        for (int i = 0; i < kAttnWaves; ++i) {
            const float w = exp2f(sm_m[i] - M);
            Ls += sm_l[i] * w;
#pragma unroll
            for (int j = 0; j < D / 64; ++j) O[j] += sm_o[i][lane + 64 * j] * w;
        }
        if (poison) {
            M = -1e30f;
            Ls = -1.f;
#pragma unroll
            for (int j = 0; j < D / 64; ++j) O[j] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < D / 64; ++j)
            __hip_atomic_store(pp + 2 + lane + 64 * j, O[j], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        if (lane == 0) {
            __hip_atomic_store(pp, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(pp + 1, Ls, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // the partial's stores complete before the arrival is counted
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (lane == 0) {
            const uint32_t prev = __hip_atomic_fetch_add(ctr + bh, 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            sm_last = prev == (uint32_t)(nsplit - 1);
        }
    }
    __syncthreads();
    if (!sm_last) return false;

    // last arrival: thread t folds channel c = t % D of partials q, q + Q,
    // q + 2Q, ... (q = t / D, Q = kAttnThreads / D), KP of them per round
    // trip (every load of a round requested at once), into a running (max,
    // sum, o[c]); threads c < D then fold the Q states through LDS
    constexpr int PW = D + 2;
    constexpr int Q = kAttnThreads / D;
    constexpr int KP = 8;
    static_assert(Q <= kAttnWaves, "one LDS row per state");
    const int ch = threadIdx.x % D, q = threadIdx.x / D;
    const float *base = part + (size_t)bh * nsplit * PW;
    auto ld = [](const float *p) {
        return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    float M = -1e30f, den = 0.f, num = 0.f;
    bool bad = false;   // a poisoned partial (sum -1)
    for (int s0 = 0; s0 < nsplit; s0 += Q * KP) {
        float pm[KP], pl[KP], po[KP];
#pragma unroll
        for (int k = 0; k < KP; ++k) {
            const int sidx = s0 + q + Q * k;
            const bool valid = sidx < nsplit;
            const float *src = base + (size_t)(valid ? sidx : 0) * PW;
            pm[k] = valid ? ld(src) : -1e30f;
            pl[k] = valid ? ld(src + 1) : 0.f;
            po[k] = valid ? ld(src + 2 + ch) : 0.f;
        }
        float Mc = M;
#pragma unroll
        for (int k = 0; k < KP; ++k) {
            Mc = fmaxf(Mc, pm[k]);
            bad |= pl[k] < 0.f;
        }
        const float r = exp2f(M - Mc);
        den *= r;
        num *= r;
#pragma unroll
        for (int k = 0; k < KP; ++k) {
            const float w = exp2f(pm[k] - Mc);
            den += pl[k] * w;
            num += po[k] * w;
        }
        M = Mc;
    }
    // (sm_o, sm_m and sm_l were last read before the barrier above)
    sm_o[q][ch] = num;
    if (ch == 0) {
        sm_m[q] = M;
        sm_l[q] = bad ? -1.f : den;
    }
    __syncthreads();
    if (threadIdx.x < D) {
        float Mt = -1e30f;
#pragma unroll
        for (int w = 0; w < Q; ++w) Mt = fmaxf(Mt, sm_m[w]);
        float dt = 0.f, nt = 0.f;
        bool anybad = false;
#pragma unroll
        for (int w = 0; w < Q; ++w) {
            const float wt = exp2f(sm_m[w] - Mt);
            anybad |= sm_l[w] < 0.f;
            dt += sm_l[w] * wt;
            nt += sm_o[w][threadIdx.x] * wt;
        }
        out[(size_t)bh * D + threadIdx.x] = !anybad && dt > 0.f ? nt / dt : 0.f;
    }
    if (threadIdx.x == 0) __hip_atomic_store(ctr + bh, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

// One workgroup's split of head bh (sequence b, KV head kvh): list rows
// [lo, hi) whose positions, clamped to the cache, are staged in sm_tok[0,
// hi - lo). Forms the split's (max, sum, o) partial and, in the last split of
// the head to arrive, merges all nsplit partials into out (and returns true).
template <int D>
__device__ __forceinline__ bool attn_split(const uint16_t *__restrict__ q,
                                           const uint16_t *__restrict__ kc,
                                           const uint16_t *__restrict__ vc, int Hkv, int Lmax,
                                           float scale_log2, int nsplit,
                                           float *__restrict__ part, uint32_t *__restrict__ ctr,
                                           float *__restrict__ out, int b, int kvh, int bh,
                                           int split, int lo, int hi, const int *sm_tok) {
    constexpr int LPR = D / 8;               // lanes per row
    constexpr int RPW = 64 / LPR;            // row groups per wave
    constexpr int NG = kAttnWaves * RPW;     // row groups per workgroup
    constexpr int STRIDE = NG;               // rows per workgroup pass
    constexpr int RPG = kAttnCH / NG;        // rows per row group

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rg = lane / LPR, cl = lane % LPR;
    const int grp = wave * RPW + rg;

    float qf[8];
    {
        const uint4 qv = *reinterpret_cast<const uint4 *>(q + (size_t)bh * D + cl * 8);
        const uint32_t w[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qf[2 * e] = bf16_lo(w[e]) * scale_log2;
            qf[2 * e + 1] = bf16_hi(w[e]) * scale_log2;
        }
    }
    // buffer resources over this (b, kv head)'s K and V rows: 32-bit row
    // offsets, and the hardware range check returns zeros past the head
    const size_t head_off = (size_t)(b * Hkv + kvh) * Lmax * D;
    const int head_bytes = Lmax * D * 2;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(kc + head_off), (short)0, head_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(vc + head_off), (short)0, head_bytes, kRsrcWord3);
    const int lane_off = cl * 16;

    float m = -1e30f, l = 0.f;
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.f;

    // all K rows of this row group are requested at once; their registers are
    // then reused for the V rows, which are requested as soon as the logits
    // are formed (a 512-thread workgroup then needs few enough registers that
    // four fit on a CU)
    uint4 kv[RPG];
#pragma unroll
    for (int u = 0; u < RPG; ++u) {
        const int t = sm_tok[grp + u * STRIDE];
        kv[u] = (lo + grp + u * STRIDE < hi)
                    ? __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    krs, t * (D * 2) + lane_off, 0, 0))
                    : make_uint4(0, 0, 0, 0);
    }
    float s[RPG];
#pragma unroll
    for (int u = 0; u < RPG; ++u) {
        const uint32_t w[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            d = __builtin_fmaf(bf16_lo(w[e]), qf[2 * e], d);
            d = __builtin_fmaf(bf16_hi(w[e]), qf[2 * e + 1], d);
        }
        s[u] = d;
    }
    // the logits are formed (and the K registers freed) before V is requested
#pragma unroll
    for (int u = 0; u < RPG; ++u) asm volatile("" ::"v"(s[u]));
    asm volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < RPG; ++u) {
        const int t = sm_tok[grp + u * STRIDE];
        kv[u] = (lo + grp + u * STRIDE < hi)
                    ? __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    vrs, t * (D * 2) + lane_off, 0, 0))
                    : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < RPG; ++u) s[u] = group_sum<LPR>(s[u]);
#pragma unroll
    for (int u = 0; u < RPG; ++u)
        if (lo + grp + u * STRIDE < hi) m = fmaxf(m, s[u]);
#pragma unroll
    for (int u = 0; u < RPG; ++u) {
        const float p = (lo + grp + u * STRIDE < hi) ? exp2f(s[u] - m) : 0.f;
        l += p;
        const uint32_t w[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] = __builtin_fmaf(p, bf16_lo(w[e]), acc[2 * e]);
            acc[2 * e + 1] = __builtin_fmaf(p, bf16_hi(w[e]), acc[2 * e + 1]);
        }
    }

    return attn_store_merge<D>(m, l, acc, nsplit, part, ctr, out, bh, split);
}

// The lane's row-group (max, sum, o) state over rows [0, nrows) whose
// positions, clamped to the cache, are staged in sm_tok (nrows <= the
// array's size, a multiple of ROWS): ROWS rows per pass, the state rescaled
// to each pass's new maximum. Rows beyond nrows are not loaded. fresh false:
// the rows extend the state passed in instead of starting a new one.
template <int D, int ROWS = kAttnCH>
__device__ __forceinline__ void attn_rows(const uint16_t *__restrict__ q,
                                          const uint16_t *__restrict__ kc,
                                          const uint16_t *__restrict__ vc, int Hkv, int Lmax,
                                          float scale_log2, int b, int kvh, int bh, int nrows,
                                          const int *sm_tok, float &m, float &l,
                                          float (&acc)[8], bool fresh = true) {
    constexpr int LPR = D / 8;               // lanes per row
    constexpr int RPW = 64 / LPR;            // row groups per wave
    constexpr int NG = kAttnWaves * RPW;     // row groups per workgroup
    constexpr int STRIDE = NG;               // rows per workgroup pass
    constexpr int RPG = ROWS / NG;           // rows per row group and pass
    static_assert(RPG >= 1 && RPG * NG == ROWS, "whole row groups per pass");

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rg = lane / LPR, cl = lane % LPR;
    const int grp = wave * RPW + rg;

    float qf[8];
    {
        const uint4 qv = *reinterpret_cast<const uint4 *>(q + (size_t)bh * D + cl * 8);
        const uint32_t w[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qf[2 * e] = bf16_lo(w[e]) * scale_log2;
            qf[2 * e + 1] = bf16_hi(w[e]) * scale_log2;
        }
    }
    const size_t head_off = (size_t)(b * Hkv + kvh) * Lmax * D;
    const int head_bytes = Lmax * D * 2;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(kc + head_off), (short)0, head_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(vc + head_off), (short)0, head_bytes, kRsrcWord3);
    const int lane_off = cl * 16;

    if (fresh) {
        m = -1e30f;
        l = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = 0.f;
    }
    for (int base = 0; base < nrows; base += ROWS) {
        const int *tok = sm_tok + base;
        const int n = nrows - base;   // rows of this pass: [0, min(n, ROWS))
        uint4 kv[RPG];
#pragma unroll
        for (int u = 0; u < RPG; ++u) {
            const int i = grp + u * STRIDE;
            kv[u] = i < n ? __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                          krs, tok[i] * (D * 2) + lane_off, 0, 0))
                          : make_uint4(0, 0, 0, 0);
        }
        float s[RPG];
#pragma unroll
        for (int u = 0; u < RPG; ++u) {
            const uint32_t w[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                d = __builtin_fmaf(bf16_lo(w[e]), qf[2 * e], d);
                d = __builtin_fmaf(bf16_hi(w[e]), qf[2 * e + 1], d);
            }
            s[u] = d;
        }
        // the logits are formed (and the K registers freed) before V is requested
#pragma unroll
        for (int u = 0; u < RPG; ++u) asm volatile("" ::"v"(s[u]));
        asm volatile("" ::: "memory");
#pragma unroll
        for (int u = 0; u < RPG; ++u) {
            const int i = grp + u * STRIDE;
            kv[u] = i < n ? __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                          vrs, tok[i] * (D * 2) + lane_off, 0, 0))
                          : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < RPG; ++u) s[u] = group_sum<LPR>(s[u]);
        float mt = m;
#pragma unroll
        for (int u = 0; u < RPG; ++u)
            if (grp + u * STRIDE < n) mt = fmaxf(mt, s[u]);
        const float rs = exp2f(m - mt);
        l *= rs;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] *= rs;
        m = mt;
#pragma unroll
        for (int u = 0; u < RPG; ++u) {
            const float p = (grp + u * STRIDE < n) ? exp2f(s[u] - m) : 0.f;
            l += p;
            const uint32_t w[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] = __builtin_fmaf(p, bf16_lo(w[e]), acc[2 * e]);
                acc[2 * e + 1] = __builtin_fmaf(p, bf16_hi(w[e]), acc[2 * e + 1]);
            }
        }
    }
}

}  // namespace tb
