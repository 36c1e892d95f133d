// Helpers of the fixed-budget selection shared by its translation units:
// the eligible region, pooled ranking keys, block / wave scans, the chunk
// and list bookkeeping, and an exact k-th-largest select over 64-bit keys.
// The ranking key of an eligible token t is
//     [ key32(score of c(t)) | 0xFFFFFF - c(t) | 0x7F - |t - c(t)| | t <= c(t) ]
// with c(t) the best centre within the neighbour radius of t (highest score,
// lowest position on ties); descending key order is the greedy fill order of
// neighbour fetching ("TokenButler" summary, "Optimizations").
#pragma once
#include "tb_common.h"

namespace tb {
namespace sel {

constexpr int CHUNK = 2048;          // tokens per classify workgroup
constexpr int MAXR = 64;             // largest neighbour radius
constexpr int GMAX = 64;             // boundary group size ranked directly
// the histogram route: 4096 bins of the 12 high bits of key32 (sign,
// exponent, three mantissa bits), at most 64 chunks per segment
constexpr int HB = 12;
constexpr int HBINS = 1 << HB;
constexpr int HSHIFT = 32 - HB;      // key32 >> HSHIFT = bin
constexpr int MAXC = 64;

struct Region {
    int L, P, e0, e1, need;
    bool bad;
};

__device__ __forceinline__ Region region(const int32_t *ctx, const int32_t *plen, int b, int Lmax,
                                         int S, int W, int K) {
    Region g;
    g.L = ctx[b];
    g.P = plen[b];
    g.bad = g.L < 0 || g.L > Lmax || g.P < 0 || g.P > Lmax;
    g.e0 = S;
    int e1 = g.L - W < g.P ? g.L - W : g.P;
    g.e1 = e1 < S ? S : e1;
    const int nE = g.e1 - g.e0;
    g.need = K < nE ? K : nE;
    return g;
}

// Stage order keys of scores for positions [lo, hi) (clipped to [e0, e1))
// into LDS; slot i holds position lo + i. All loads of a thread are issued
// before any is consumed.
template <int NT>
__device__ __forceinline__ void stage_keys(uint32_t *sk, const float *s, int lo, int hi, int e0,
                                           int e1) {
    constexpr int PER = (CHUNK + 2 * MAXR + NT - 1) / NT;
    float v[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int t = lo + (int)threadIdx.x + k * NT;
        v[k] = (t < hi && t >= e0 && t < e1) ? s[t] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int i = (int)threadIdx.x + k * NT;
        const int t = lo + i;
        if (t < hi) sk[i] = (t >= e0 && t < e1) ? order_key(v[k]) : 0u;
    }
}

// Pooled key of eligible token t (slot base = lo).
__device__ __forceinline__ uint64_t pooled_key(const uint32_t *sk, int lo, int t, int e0, int e1,
                                               int r) {
    const int a = t - r < e0 ? e0 : t - r;
    const int z = t + r >= e1 ? e1 - 1 : t + r;
    uint32_t best = sk[a - lo];
    int c = a;
    for (int u = a + 1; u <= z; ++u) {
        const uint32_t k = sk[u - lo];
        if (k > best) {
            best = k;
            c = u;
        }
    }
    const int d = t < c ? c - t : t - c;
    const uint32_t low = ((uint32_t)(0xffffff - c) << 8) | ((uint32_t)(0x7f - d) << 1) |
                         (uint32_t)(t <= c ? 1 : 0);
    return ((uint64_t)best << 32) | low;
}

__device__ __forceinline__ int key_token(uint64_t key) {
    const uint32_t low = (uint32_t)key;
    const int c = 0xffffff - (int)(low >> 8);
    const int d = 0x7f - (int)((low >> 1) & 0x7f);
    return (low & 1u) ? c - d : c + d;
}

// x of another lane through DPP, or 0 where the control has no source lane
// for this one or the row / bank masks leave it out.
template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_or0(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, BANK_MASK, false);
}

// Inclusive prefix sum over the 64 lanes of a wave (lane order), by DPP:
// within each row of 16 lanes by shifts of 1, 2, 4 and 8 lanes, then the
// last lane of row 0 broadcast into row 1 (and of row 2 into row 3), then
// lane 31 into rows 2 and 3. No LDS traffic.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += dpp_or0<0x111>(x);              // row_shr:1
    x += dpp_or0<0x112>(x);              // row_shr:2
    x += dpp_or0<0x114>(x);              // row_shr:4
    x += dpp_or0<0x118>(x);              // row_shr:8
    x += dpp_or0<0x142, 0xA>(x);         // row_bcast:15 into rows 1 and 3
    x += dpp_or0<0x143, 0xC>(x);         // row_bcast:31 into rows 2 and 3
    return x;
}

// Sum over each row of 16 lanes, in every lane of the row, by DPP.
__device__ __forceinline__ uint32_t row16_sum(uint32_t x) {
    x += dpp_or0<0xB1>(x);               // quad_perm [1, 0, 3, 2]
    x += dpp_or0<0x4E>(x);               // quad_perm [2, 3, 0, 1]
    x += dpp_or0<0x124>(x);              // row_ror:4
    x += dpp_or0<0x128>(x);              // row_ror:8
    return x;
}

// Inclusive prefix sum over the threads of the block (thread order). s_w
// holds NT / 64 slots. Two barriers, and s_w may be reused after return;
// with TRAIL false only the first, and the caller must pass another barrier
// before s_w is written again.
template <int NT, bool TRAIL = true>
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t *s_w, uint32_t *total) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t x = wave_incl_scan(v);
    if (lane == 63) s_w[wave] = x;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t t = s_w[w];
        before += w < wave ? t : 0u;
        tot += t;
    }
    if constexpr (TRAIL) __syncthreads();
    *total = tot;
    return before + x;
}


// Wave-wide: lane l holds the word of tokens [t0, t0 + 32) (t0 ascending with
// the lane) whose first set bit is list row `base` + (set bits of the lanes
// below); each lane stages its own rows that fall in [lo, hi) at sm_tok[row -
// lo]. Every lane takes part in the prefix count.
__device__ __forceinline__ void emit_rows(uint32_t mine, int t0, uint32_t base, int lo, int hi,
                                          int *sm_tok) {
    const uint32_t pop = (uint32_t)__popc(mine);
    uint32_t p = base + wave_incl_scan(pop) - pop;
    if (p + pop <= (uint32_t)lo || p >= (uint32_t)hi) return;
    while (mine) {
        const int bit = __builtin_ctz(mine);
        if (p >= (uint32_t)lo && p < (uint32_t)hi) sm_tok[p - lo] = t0 + bit;
        ++p;
        mine &= mine - 1u;
    }
}

// Pooled key of eligible token t read straight from the scores (global).
__device__ __forceinline__ uint64_t pooled_key_g(const float *s, int t, int e0, int e1, int r) {
    const int a = t - r < e0 ? e0 : t - r;
    const int z = t + r >= e1 ? e1 - 1 : t + r;
    uint32_t best = order_key(s[a]);
    int c = a;
    for (int u = a + 1; u <= z; ++u) {
        const uint32_t k = order_key(s[u]);
        if (k > best) {
            best = k;
            c = u;
        }
    }
    const int d = t < c ? c - t : t - c;
    const uint32_t low = ((uint32_t)(0xffffff - c) << 8) | ((uint32_t)(0x7f - d) << 1) |
                         (uint32_t)(t <= c ? 1 : 0);
    return ((uint64_t)best << 32) | low;
}


// Pooled key of eligible token t with the radius fixed at compile time: the
// 2R + 1 staged keys are read together (slots outside E hold 0, below the key
// of every finite score), and the first maximum in position order is the
// centre -- the same key as pooled_key.
template <int R>
__device__ __forceinline__ uint64_t pooled_key_r(const uint32_t *sk, int lo, int t) {
    uint32_t k[2 * R + 1];
#pragma unroll
    for (int u = 0; u <= 2 * R; ++u) k[u] = sk[t - R + u - lo];
    uint32_t best = 0u;
    int c = t;
#pragma unroll
    for (int u = 0; u <= 2 * R; ++u) {
        if (k[u] > best) {
            best = k[u];
            c = t - R + u;
        }
    }
    const int d = t < c ? c - t : t - c;
    const uint32_t low = ((uint32_t)(0xffffff - c) << 8) | ((uint32_t)(0x7f - d) << 1) |
                         (uint32_t)(t <= c ? 1 : 0);
    return ((uint64_t)best << 32) | low;
}


// Position of the k-th (0-based) set bit of v; requires k < popcount(v).
__device__ __forceinline__ int select_bit(uint32_t v, uint32_t k) {
    int pos = 0;
    uint32_t c = (uint32_t)__popc(v & 0xffffu);
    if (k >= c) { k -= c; pos += 16; v >>= 16; }
    c = (uint32_t)__popc(v & 0xffu);
    if (k >= c) { k -= c; pos += 8; v >>= 8; }
    c = (uint32_t)__popc(v & 0xfu);
    if (k >= c) { k -= c; pos += 4; v >>= 4; }
    c = (uint32_t)__popc(v & 0x3u);
    if (k >= c) { k -= c; pos += 2; v >>= 2; }
    if (k >= (v & 1u)) pos += 1;
    return pos;
}

__device__ __forceinline__ uint32_t bits_below(int n) {
    return n <= 0 ? 0u : (n >= 32 ? 0xffffffffu : ((1u << n) - 1u));
}

// Chunk holding candidate i of the segment (chunk-major order): the last
// chunk c with off[c] <= i; chunk c holds entries [off[c], off[c+1]).
__device__ __forceinline__ int chunk_of(const uint32_t *s_off, int nchunks, uint32_t i) {
    int lo = 0, hi = nchunks - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_off[mid] <= i) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Candidate i of the segment, read from its chunk's slots.
__device__ __forceinline__ uint64_t cand_at(const uint64_t *cl, const uint32_t *s_off, int nchunks,
                                            uint32_t i) {
    const int c = chunk_of(s_off, nchunks, i);
    return cl[(size_t)c * CHUNK + (i - s_off[c])];
}

// How many of the tokens [t0, t1) lie in sink [0, slo) U window [wlo, L)
// (the two ranges may overlap in short contexts).
__device__ __forceinline__ int fixed_in(int t0, int t1, int slo, int wlo, int L) {
    const int e = t1 < L ? t1 : L;
    int n = 0;
    if (t0 < slo) n += (e < slo ? e : slo) - t0;
    int w0 = wlo > slo ? wlo : slo;
    w0 = w0 > t0 ? w0 : t0;
    if (e > w0) n += e - w0;
    return n > 0 ? n : 0;
}

// Scratch of kth_largest for a workgroup of NT threads (NT radix bins).
template <int NT>
struct KthLds {
    uint32_t tile[NT];
    uint64_t grp[GMAX];
    uint32_t w[NT / 64];
    int sel[3];
    uint32_t ng;
    uint64_t thr;
};

// The k-th largest (1 <= k <= count) of distinct 64-bit keys that all carry
// `prefix` on `mask` (every bit at or above `shift`). visit(f) hands each key
// to f exactly once, from any thread; every thread calls it and it may hold
// barriers. grp: how many keys carry the prefix (anything above GMAX when
// unknown). Radix passes of log2(NT) bits (one bin per thread) narrow the
// group to at most GMAX keys, which are ranked directly. sh.tile and sh.ng are zero on entry (cleared by the
// caller before a barrier); each pass clears its bins again as it reads them.
template <int NT, class Visit>
__device__ __forceinline__ uint64_t kth_largest(const Visit &visit, int k, uint64_t prefix,
                                                uint64_t mask, int shift, int grp,
                                                KthLds<NT> &sh) {
    static_assert(NT == 256 || NT == 512 || NT == 1024, "one radix bin per thread");
    constexpr int RBINS = NT;
    constexpr int RBITS = NT == 1024 ? 10 : (NT == 512 ? 9 : 8);
    const int tid = threadIdx.x;
    while (grp > GMAX && shift > 0) {
        const int width = shift < RBITS ? shift : RBITS;
        shift -= width;
        const uint32_t dmask = (1u << width) - 1u;
        // thread t counts digit (RBINS - 1 - t): thread order = descending digit
        visit([&](uint64_t key) {
            if ((key & mask) == prefix)
                atomicAdd(&sh.tile[RBINS - 1 - (int)((key >> shift) & dmask)], 1u);
        });
        __syncthreads();
        const uint32_t c = sh.tile[tid];
        sh.tile[tid] = 0u;   // ordered before the next pass by the scan's barriers
        uint32_t tot;
        // sh.w is written next after the barrier below
        const uint32_t incl = block_incl_scan<NT, false>(c, sh.w, &tot);
        const uint32_t above = incl - c;
        if (c > 0 && above < (uint32_t)k && (uint32_t)k <= incl) {
            sh.sel[0] = RBINS - 1 - tid;
            sh.sel[1] = k - (int)above;
            sh.sel[2] = (int)c;
        }
        __syncthreads();
        prefix |= (uint64_t)sh.sel[0] << shift;
        mask |= (uint64_t)dmask << shift;
        k = sh.sel[1];
        grp = sh.sel[2];
        // sh.sel is written next only after the next pass's barriers
    }
    visit([&](uint64_t key) {
        if ((key & mask) == prefix) {
            const uint32_t slot = atomicAdd(&sh.ng, 1u);
            if (slot < (uint32_t)GMAX) sh.grp[slot] = key;
        }
    });
    __syncthreads();
    const int ng = sh.ng < (uint32_t)GMAX ? (int)sh.ng : GMAX;
    if (tid < 64) {
        // wave 0 ranks the group: lane l holds key l, and every key is read
        // from its lane in turn (register reads, no LDS round trip per key)
        const uint64_t mine = tid < ng ? sh.grp[tid] : 0ull;
        const uint32_t mlo = (uint32_t)mine, mhi = (uint32_t)(mine >> 32);
        int rank = 0;
        for (int j = 0; j < ng; ++j) {
            const uint64_t o =
                ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)mhi, j) << 32) |
                (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)mlo, j);
            rank += o > mine ? 1 : 0;
        }
        if (tid < ng && rank == k - 1) sh.thr = mine;
    }
    __syncthreads();
    return sh.thr;
}

}  // namespace sel
}  // namespace tb
