// Scoring with an exact histogram of the selection keys, and classification
// against the bin that holds the budget's key ("TokenButler" summary, "Core
// architecture": scoring, then selection under a fixed budget;
// "Optimizations": neighbour fetching; "Inference strategy": the sink, window
// and important buffers).
//
// The important buffer of a segment (sequence b, query head h) is the
// min(K, |E|) largest ranking keys of its eligible tokens (select_impl.h).
// Their order is decided first by key32, the totalOrder key of the fp32
// score of the token's centre; the 12 high bits of key32 (sign, exponent,
// three mantissa bits: bins of an eighth of an octave) split the segment
// into 4096 bins.
//
//   score_hist      one 1024-thread workgroup per (b, KV head, 1024 tokens):
//                   the g heads' scores of its tokens (written to `scores`,
//                   the same bits as the scoring kernel), their pooled key32
//                   (the neighbours' scores staged in LDS), a 4096-bin
//                   histogram per head in LDS, added to the segment's
//                   histogram in the workspace with agent-scope atomics
//                   (nonzero bin pairs only, one 64-bit atomic per pair);
//   hist_select     per segment, one 1024-thread workgroup per 4 chunks of
//                   2048 tokens: the bin B* that holds the budget's key from
//                   the histogram, a streaming pass over its tokens (tokens of
//                   higher bins to the bitmap, tokens of B* to their chunk's
//                   candidate slots and a second histogram of their next 12
//                   key bits); the last workgroup of the segment finds the
//                   exact key of the budget's rank inside the sub-bin that
//                   holds it, the chunk offsets and the count, and clears both
//                   histograms for the next call.
// The compaction, the deferred list of tb_select_attn and the dilation mode
// then read the state as they read the sampled-band route's.
#include "score_impl.h"
#include "select_impl.h"

namespace tb {
namespace {

using namespace sel;

constexpr int TS = 1024;               // threads (one token each) of score_hist

template <int G, int DP, int R>
__global__ __launch_bounds__(TS, G <= 4 ? 8 : 4) void score_hist_kernel(
    const float *__restrict__ qhat, int q_bstride, int q_off, const uint16_t *__restrict__ kp,
    const int32_t *__restrict__ ctx, const int32_t *__restrict__ plen,
    float *__restrict__ scores, int Hq, int Hkv, int Lmax, int S, int W, int K, int nxs,
    uint32_t *__restrict__ hist) {
    constexpr int V = DP / 8;   // 16-byte vectors per key row
    __shared__ uint32_t s_h[G * HBINS / 2];    // two 16-bit counters per word
    __shared__ float s_sc[G][TS + 2 * R];      // slot j: position t0 - R + j
    // XCD-aware order when the grid divides into the 8 XCDs (workgroups are
    // dealt to them in turn): a KV head's blocks on one XCD, as the
    // classification pass and the attention launch place that head's work
    const int nbk = gridDim.x, bq = blockIdx.x;
    const int blk = (nbk & 7) == 0 ? (bq & 7) * (nbk >> 3) + (bq >> 3) : bq;
    const int x = blk % nxs, kvh = (blk / nxs) % Hkv, b = blk / (nxs * Hkv);
    const int tid = threadIdx.x;
    const int t0 = x * TS;
    int P = plen[b];
    P = P < 0 ? 0 : (P > Lmax ? Lmax : P);
    if (t0 >= P) return;
    for (int i = tid; i < G * HBINS / 2; i += TS) s_h[i] = 0u;
    const float *qb = qhat + (size_t)b * q_bstride + q_off + (size_t)kvh * G * DP;
    const uint4 *kb = reinterpret_cast<const uint4 *>(kp + (size_t)(b * Hkv + kvh) * Lmax * DP);
    const int t = t0 + tid;
    uint4 raw[V];
    if (t < P) {
#pragma unroll
        for (int v = 0; v < V; ++v) raw[v] = kb[(size_t)t * V + v];
    }
    const Region g = region(ctx, plen, b, Lmax, S, W, K);
    float *sb = scores + (size_t)(b * Hq + kvh * G) * Lmax;
    // one head at a time: its DP query values (wave-uniform) are read just
    // before its dot product
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
        float q[DP];
#pragma unroll
        for (int c = 0; c < DP; ++c) q[c] = qb[gi * DP + c];
        const float sc = t < P ? score_row<DP>(raw, q) : 0.f;
        if (t < P) sb[(size_t)gi * Lmax + t] = sc;
        s_sc[gi][R + tid] = sc;
    }
    // the 2R halo rows on either side of the block's tokens (first wave only)
    const int th = tid < R ? t0 - R + tid : t0 + TS + (tid - R);
    if (R > 0 && tid < 2 * R && th >= 0 && th < P) {
#pragma unroll
        for (int v = 0; v < V; ++v) raw[v] = kb[(size_t)th * V + v];
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            float q[DP];
#pragma unroll
            for (int c = 0; c < DP; ++c) q[c] = qb[gi * DP + c];
            s_sc[gi][tid < R ? tid : TS + tid] = score_row<DP>(raw, q);
        }
    }
    const int nE = g.e1 - g.e0;
    const bool partial = !g.bad && g.need > 0 && g.need < nE;
    if (!partial || t0 + TS <= g.e0 || t0 >= g.e1) return;   // the same for the whole block
    __syncthreads();
    if (t >= g.e0 && t < g.e1) {
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            // key32 of the pooled key: the largest order key within E
            uint32_t key = 0u;
#pragma unroll
            for (int u = -R; u <= R; ++u) {
                const int p = t + u;
                const uint32_t k = order_key(s_sc[gi][R + tid + u]);
                if (p >= g.e0 && p < g.e1 && k > key) key = k;
            }
            const uint32_t bin = key >> HSHIFT;
            atomicAdd(&s_h[gi * (HBINS / 2) + (bin >> 1)], 1u << ((bin & 1u) << 4));
        }
    }
    __syncthreads();
    // bins 2k and 2k + 1 are adjacent 32-bit counters of the workspace: one
    // 64-bit atomic adds both (a segment's count, below 2^25, never carries
    // out of the low word)
    uint64_t *hs = reinterpret_cast<uint64_t *>(hist + (size_t)(b * Hq + kvh * G) * HBINS);
    for (int i = tid; i < G * HBINS / 2; i += TS) {
        const uint32_t w = s_h[i];
        if (w == 0u) continue;
        const uint64_t add = (uint64_t)(w & 0xffffu) | ((uint64_t)(w >> 16) << 32);
        __hip_atomic_fetch_add(hs + i, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

typedef void (*score_hist_fn)(const float *, int, int, const uint16_t *, const int32_t *,
                              const int32_t *, float *, int, int, int, int, int, int, int,
                              uint32_t *);

template <int DP, int R>
score_hist_fn score_hist_pick(int g) {
    switch (g) {
        case 1: return score_hist_kernel<1, DP, R>;
        case 2: return score_hist_kernel<2, DP, R>;
        case 3: return score_hist_kernel<3, DP, R>;
        case 4: return score_hist_kernel<4, DP, R>;
        case 5: return score_hist_kernel<5, DP, R>;
        case 6: return score_hist_kernel<6, DP, R>;
        case 7: return score_hist_kernel<7, DP, R>;
        case 8: return score_hist_kernel<8, DP, R>;
        default: return nullptr;
    }
}

// ---------------------------------------------------------------------------
// hist_select: per segment, one 1024-thread workgroup per CPW chunks classifies
// its tokens against the bin of the budget's key, and the last workgroup of
// the segment to finish (an arrival counter, agent-scope release / acquire)
// resolves the exact threshold inside that bin. Its output is the state the
// sampled-band route leaves for the list: the bitmap of tokens above the bin,
// per chunk the candidates (tokens of the bin, 64-bit ranking keys) and their
// count, the tokens above the bin per chunk, the threshold key, the chunk
// offsets of the list and the count.
//
//  1. Every workgroup reads the segment's histogram (one 16-byte read per
//     thread, bins in descending thread order) and finds the bin B* holding
//     the budget's key: A tokens lie in higher bins, C in B*; the budget's
//     rank inside B* is need1 = need - A.
//  2. Pass: each wave takes a contiguous run of 256-token steps of the
//     workgroup's chunks (lane l holds tokens base + l + 64 j, j < 4: every
//     load row is 256 bytes, every ballot 64 consecutive tokens). A pooled
//     key takes its neighbours from the adjacent lanes and the R positions
//     either side of the step. Tokens of higher bins set their bitmap bit
//     (ballot words); tokens of B* are written to their chunk's candidate
//     slots and counted in a 4096-bin histogram of their next 12 key bits,
//     which is added to the segment's second histogram in the workspace.
//  3. The last workgroup: the second histogram gives the sub-bin holding
//     rank need1; the exact key of that rank among the candidates sharing
//     those 24 high bits is the threshold. Candidates are staged in LDS
//     (read from global when there are more than LDS holds). Both histograms
//     and the arrival counter are left at zero for the next call. Counts that
//     disagree with the histogram (a workspace that was not zero at first
//     use) fall back to an exact selection over the scores that rewrites the
//     bitmap.
constexpr int TSEL = 1024;                 // threads of hist_select
constexpr int NWSEL = TSEL / 64;           // waves
constexpr int SS = 256;                    // tokens per wave step
constexpr int CPW = 4;                     // chunks per workgroup
constexpr int CAPC = 8192;                 // candidates the last workgroup stages in LDS
constexpr int TPC = TSEL / MAXC;           // last workgroup: threads per chunk
constexpr int PFS = 12;                    // candidate slots each of them fetches early
constexpr int NSW = (CPW * CHUNK / SS + NWSEL - 1) / NWSEL;   // steps per wave

// Lane rotations of a wave through DPP (no LDS traffic): lane i takes the
// value of lane i - n (rotr_lanes) or of lane i + n (rotl_lanes), modulo 64.
__device__ __forceinline__ uint32_t rotr_lanes(uint32_t x, int n) {
    for (int i = 0; i < n; ++i) x = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x13C, 0xF, 0xF, false);
    return x;
}
__device__ __forceinline__ uint32_t rotl_lanes(uint32_t x, int n) {
    for (int i = 0; i < n; ++i) x = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x134, 0xF, 0xF, false);
    return x;
}

// One 256-token step of the classification pass, by one wave with every lane
// active: lane l holds the scores of tokens base + l + 64 j in v[j] and, in
// lanes l < R, those of base - R + l (hl) and base + 256 + l (hr); positions
// outside the eligible range [e0, e1) take no part. A token's pooled key
// takes its neighbours from the adjacent lanes. Tokens whose key lies above
// bin bstar set their bits in the words bm (word 0: tokens 32 w0 onward) and
// are counted in *ac; tokens of bin bstar take their chunk's next candidate
// slots (counted in *cc; slots at or beyond lim are not written), their
// 64-bit ranking keys go to cl[slot] and their next 12 key bits to the second
// histogram sub. AGENT: the candidates are stored at agent scope.
template <int R, bool AGENT>
__device__ __forceinline__ void classify_step(int base, const float (&v)[4], float hl, float hr,
                                              int e0, int e1, uint32_t bstar, uint32_t *bm,
                                              int w0, uint32_t *ac, uint32_t *cc, uint32_t *sub,
                                              uint64_t *cl, int lim) {
    const int lane = threadIdx.x & 63;
    auto kof = [&](int p, float x) -> uint32_t {
        return (p >= e0 && p < e1) ? order_key(x) : 0u;
    };
    uint32_t k[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) k[j] = kof(base + lane + 64 * j, v[j]);
    const uint32_t hlk = lane < R ? kof(base - R + lane, hl) : 0u;
    const uint32_t hrk = lane < R ? kof(base + SS + lane, hr) : 0u;
    // keys of the window of token (lane, j): slot R + u is position t + u
    uint32_t wk[4][2 * R + 1];
#pragma unroll
    for (int j = 0; j < 4; ++j) wk[j][R] = k[j];
#pragma unroll
    for (int u = 1; u <= R; ++u) {
        uint32_t rm[4], rp[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            rm[j] = rotr_lanes(k[j], u);
            rp[j] = rotl_lanes(k[j], u);
        }
        const uint32_t hlu = rotl_lanes(hlk, R - u);
        const uint32_t hru = rotl_lanes(hrk, u);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            wk[j][R - u] = lane >= u ? rm[j] : (j > 0 ? rm[j > 0 ? j - 1 : 0] : hlu);
            wk[j][R + u] = lane + u <= 63 ? rp[j] : (j < 3 ? rp[j < 3 ? j + 1 : 3] : hru);
        }
    }
    uint32_t best[4];
    bool sel[4], isc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = base + lane + 64 * j;
        uint32_t bk = 0u;
#pragma unroll
        for (int u = 0; u <= 2 * R; ++u) bk = wk[j][u] > bk ? wk[j][u] : bk;
        best[j] = bk;
        const bool el = t >= e0 && t < e1;
        sel[j] = el && (bk >> HSHIFT) > bstar;
        isc[j] = el && (bk >> HSHIFT) == bstar;
    }
    uint64_t cm[4];
    uint32_t na = 0, ncw = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint64_t m = __ballot(sel[j]);
        if (lane == 0) {
            const int w = ((base + 64 * j) >> 5) - w0;
            bm[w] = (uint32_t)m;
            bm[w + 1] = (uint32_t)(m >> 32);
        }
        na += (uint32_t)__popcll(m);
        cm[j] = __ballot(isc[j]);
        ncw += (uint32_t)__popcll(cm[j]);
    }
    if (lane == 0 && na) atomicAdd(ac, na);
    if (ncw) {
        // candidate (lane, j) takes chunk slot first + (those of rows
        // < j) + (lanes below it in row j); a chunk has CHUNK slots
        uint32_t first = 0;
        if (lane == 0) first = atomicAdd(cc, ncw);
        first = (uint32_t)__builtin_amdgcn_readfirstlane((int)first);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (isc[j]) {
                const int t = base + lane + 64 * j;
                const uint32_t slot =
                    first + (uint32_t)__popcll(cm[j] & ((1ull << lane) - 1ull));
                atomicAdd(&sub[(best[j] >> 8) & (HBINS - 1)], 1u);
                int c = t;
                uint32_t bk = 0u;
#pragma unroll
                for (int u = 0; u <= 2 * R; ++u) {
                    if (wk[j][u] > bk) {
                        bk = wk[j][u];
                        c = t - R + u;
                    }
                }
                const int d = t < c ? c - t : t - c;
                const uint32_t low = ((uint32_t)(0xffffff - c) << 8) |
                                     ((uint32_t)(0x7f - d) << 1) |
                                     (uint32_t)(t <= c ? 1 : 0);
                if (slot < (uint32_t)CHUNK && (int)slot < lim) {
                    if constexpr (AGENT)
                        __hip_atomic_store(cl + slot, ((uint64_t)bk << 32) | low,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    else
                        cl[slot] = ((uint64_t)bk << 32) | low;
                }
            }
            first += (uint32_t)__popcll(cm[j]);
        }
    }
}

struct HistSelLds {
    union {
        struct {
            uint32_t bm[CPW * (CHUNK / 32)];   // the workgroup's bitmap words
            uint32_t sub[HBINS];               // its second histogram
        } p;
        uint64_t cand[CAPC];                   // the last workgroup's candidates
    } u;
    KthLds<TSEL> k;
    uint32_t cc[CPW], ac[CPW];                 // per chunk of the workgroup
    uint32_t m[12];   // B*, A, C, last, sub-bin, above it, in it, candidates, above-bin tokens
    uint32_t ccnt[MAXC], acnt[MAXC], off[MAXC], chosen[MAXC];
};

template <int R>
__global__ __launch_bounds__(TSEL) void hist_select_kernel(
    const float *__restrict__ scores, const int32_t *__restrict__ ctx,
    const int32_t *__restrict__ plen, int Hq, int Lmax, int S, int W, int K, int omit_window,
    uint32_t *__restrict__ hist, uint32_t *__restrict__ sub, uint32_t *__restrict__ arrive,
    int nchunks, uint32_t *__restrict__ ccount, uint32_t *__restrict__ acount,
    uint64_t *__restrict__ cand, uint32_t *__restrict__ bitmap, int nwords,
    uint64_t *__restrict__ thr_out, uint32_t *__restrict__ coff, int32_t *__restrict__ count) {
    static_assert(R >= 0 && R <= 2, "the halo lanes hold radius 2");
    static_assert(TSEL * 4 == HBINS, "four bins per thread");
    static_assert(TPC * MAXC == TSEL && (CHUNK / 32) == 64, "chunk bookkeeping");
    __shared__ __align__(16) HistSelLds sh;
    const int part = blockIdx.x, seg = blockIdx.y, b = seg / Hq;
    const int nparts = gridDim.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c_lo = part * CPW;
    const int c_hi = c_lo + CPW < nchunks ? c_lo + CPW : nchunks;
    uint4 *hs = reinterpret_cast<uint4 *>(hist + (size_t)seg * HBINS);
    uint4 *ss = reinterpret_cast<uint4 *>(sub + (size_t)seg * HBINS);
    const float *sc = scores + (size_t)seg * Lmax;
    uint64_t *cseg = cand + (size_t)seg * Lmax;
    const Region g = region(ctx, plen, b, Lmax, S, W, K);
    const int nE = g.e1 - g.e0;
    const bool partial = !g.bad && g.need > 0 && g.need < nE;
    const int L = g.L;
    const int wlo = omit_window ? L : (L - W > 0 ? L - W : 0);
    const int slo = S < L ? S : L;
    uint4 hv = make_uint4(0u, 0u, 0u, 0u);
    if (partial) hv = hs[HBINS / 4 - 1 - tid];
    // this workgroup's steps of 256 tokens, a contiguous run of at most NSW
    // per wave; their scores are loaded together with the histogram, from
    // addresses clamped into E, unconditionally (values at positions outside
    // E are never used), so no load waits behind another or sits in a branch
    const int e0 = g.e0, e1 = g.e1;
    const int a0 = c_lo * CHUNK;
    const int pend = c_hi * CHUNK < e1 ? c_hi * CHUNK : e1;
    const int nss = partial && pend > a0 ? (pend - a0 + SS - 1) / SS : 0;
    const int qw = nss / NWSEL, rw = nss % NWSEL;
    const int s0 = wave * qw + (wave < rw ? wave : rw);
    const int s1 = s0 + qw + (wave < rw ? 1 : 0);
    auto clampE = [&](int p) { return p < e0 ? e0 : (p >= e1 ? e1 - 1 : p); };
    float v[NSW][4], hl[NSW] = {}, hr[NSW] = {};
    if (partial) {
#pragma unroll
        for (int i = 0; i < NSW; ++i) {
            const int base = a0 + (s0 + i) * SS;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[i][j] = sc[clampE(base + lane + 64 * j)];
            if (R > 0) {
                hl[i] = sc[clampE(base - R + lane)];
                hr[i] = sc[clampE(base + SS + lane)];
            }
        }
    }

    if (!partial) {
        // nothing to rank: every eligible token or none. Each workgroup
        // writes its chunks' words; the first one writes every chunk's
        // offset, the count, and clears both histograms (left untouched by
        // the scoring launch, unless the workspace was not zero at first use)
        const bool all = !g.bad && g.need == nE && nE > 0;
        for (int w = c_lo * 64 + tid; w < c_hi * 64 && w < nwords; w += TSEL) {
            const int t0 = w << 5;
            bitmap[(size_t)seg * nwords + w] =
                all ? (bits_below(g.e1 - t0) & ~bits_below(g.e0 - t0)) : 0u;
        }
        if (part != 0) return;
        hs[HBINS / 4 - 1 - tid] = make_uint4(0u, 0u, 0u, 0u);
        ss[HBINS / 4 - 1 - tid] = make_uint4(0u, 0u, 0u, 0u);
        if (wave == 0) {
            if (g.bad) {
                if (lane == 0) count[seg] = -1;
                return;
            }
            uint32_t v = 0;
            if (lane < nchunks) {
                const int t0 = lane * CHUNK, t1 = t0 + CHUNK;
                const int a = t0 > g.e0 ? t0 : g.e0, z = t1 < g.e1 ? t1 : g.e1;
                v = (uint32_t)((all && z > a ? z - a : 0) + fixed_in(t0, t1, slo, wlo, L));
            }
            const uint32_t incl = wave_incl_scan(v);
            if (lane < nchunks) coff[(size_t)seg * nchunks + lane] = incl - v;
            if (lane == 63) count[seg] = (int32_t)incl;
        }
        return;
    }

    // 1. the bin that holds the budget's key
    for (int i = tid; i < CPW * 64; i += TSEL) sh.u.p.bm[i] = 0u;
    for (int i = tid; i < HBINS; i += TSEL) sh.u.p.sub[i] = 0u;
    if (tid < CPW) {
        sh.cc[tid] = 0u;
        sh.ac[tid] = 0u;
    }
    if (tid < 12) sh.m[tid] = 0u;
    const uint32_t need = (uint32_t)g.need;
    {
        const uint32_t cnt[4] = {hv.w, hv.z, hv.y, hv.x};   // bins 4095 - 4 tid - j
        const uint32_t sum = cnt[0] + cnt[1] + cnt[2] + cnt[3];
        uint32_t tot;
        const uint32_t incl = block_incl_scan<TSEL>(sum, sh.k.w, &tot);
        uint32_t run = incl - sum;
        if (tot >= need && run < need && need <= incl) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (run < need && need <= run + cnt[j]) {
                    sh.m[0] = (uint32_t)(HBINS - 1 - 4 * tid - j);
                    sh.m[1] = run;
                    sh.m[2] = cnt[j];
                }
                run += cnt[j];
            }
        }
        __syncthreads();
    }
    const uint32_t bstar = sh.m[0], A = sh.m[1], C = sh.m[2];
    const bool have_bin = C > 0;   // else the histogram does not hold the budget's rank

    // 2. the pass over this workgroup's chunks
    if (have_bin) {
#pragma unroll
        for (int i = 0; i < NSW; ++i) {
            if (s0 + i >= s1) break;
            const int base = a0 + (s0 + i) * SS;
            const int ci = (base >> 11) - c_lo;   // the step's chunk in the workgroup
            classify_step<R, true>(base, v[i], hl[i], hr[i], e0, e1, bstar, sh.u.p.bm, c_lo * 64,
                                   &sh.ac[ci], &sh.cc[ci], sh.u.p.sub,
                                   cseg + (size_t)(c_lo + ci) * CHUNK, Lmax - (c_lo + ci) * CHUNK);
        }
    }
    __syncthreads();
    // the workgroup's share of the segment's state. What the last workgroup
    // reads (and the bitmap words it may rewrite) is written with agent-scope
    // stores, which bypass the workgroup's non-coherent L2; those complete
    // before the arrival is counted, and the last workgroup reads them with
    // agent-scope loads. (Release / acquire fences instead write back and
    // invalidate the whole L2 of the XCD: measured about 10 us here.)
    for (int w = tid; w < (c_hi - c_lo) * 64; w += TSEL) {
        if (c_lo * 64 + w < nwords)
            __hip_atomic_store(bitmap + (size_t)seg * nwords + c_lo * 64 + w, sh.u.p.bm[w],
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid < c_hi - c_lo) {
        __hip_atomic_store(ccount + (size_t)seg * nchunks + c_lo + tid, sh.cc[tid],
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(acount + (size_t)seg * nchunks + c_lo + tid, sh.ac[tid],
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (have_bin) {
        // adjacent bins as one 64-bit atomic (counts never carry out of 32 bits)
        const uint4 sv = reinterpret_cast<const uint4 *>(sh.u.p.sub)[tid];
        uint64_t *sb = reinterpret_cast<uint64_t *>(sub + (size_t)seg * HBINS + 4 * tid);
        if (sv.x | sv.y)
            __hip_atomic_fetch_add(sb, (uint64_t)sv.x | ((uint64_t)sv.y << 32), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        if (sv.z | sv.w)
            __hip_atomic_fetch_add(sb + 1, (uint64_t)sv.z | ((uint64_t)sv.w << 32),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // arrival: every wave's stores complete before the barrier, then one
    // counter increment per workgroup
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
        const uint32_t old =
            __hip_atomic_fetch_add(arrive + seg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sh.m[3] = old == (uint32_t)(nparts - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (sh.m[3] == 0u) return;
    if (tid == 0) __hip_atomic_store(arrive + seg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // 3. the last workgroup of the segment
    auto ld32 = [](const uint32_t *p) {
        return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    auto ld64 = [](const uint64_t *p) {
        return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    // the second histogram, bins 4095 - 4 tid - j in cnt2[j]
    const uint32_t *sq = sub + (size_t)seg * HBINS + HBINS - 4 * (tid + 1);
    const uint32_t cnt2[4] = {ld32(sq + 3), ld32(sq + 2), ld32(sq + 1), ld32(sq)};
    uint32_t cc_l = 0, ac_l = 0;
    if (tid < nchunks) {
        cc_l = ld32(ccount + (size_t)seg * nchunks + tid);
        ac_l = ld32(acount + (size_t)seg * nchunks + tid);
    }
    // chunk tid / TPC: its candidate slots tid % TPC + TPC u, fetched now
    const int pch = tid / TPC, pln = tid % TPC;
    uint64_t pv[PFS];
#pragma unroll
    for (int u = 0; u < PFS; ++u) {
        const int slot = pln + TPC * u;
        pv[u] = (pch < nchunks && pch * CHUNK + slot < Lmax) ? ld64(cseg + (size_t)pch * CHUNK + slot)
                                                            : 0ull;
    }
    if (tid < nchunks) {
        sh.ccnt[tid] = cc_l < (uint32_t)CHUNK ? cc_l : (uint32_t)CHUNK;
        sh.acnt[tid] = ac_l;
        sh.chosen[tid] = 0u;
    }
    sh.k.tile[tid] = 0u;   // the exact select's state, zero on entry
    if (tid == 0) sh.k.ng = 0u;
    // both histograms back to zero for the next call (the main one was read
    // by every workgroup before it arrived)
    hs[HBINS / 4 - 1 - tid] = make_uint4(0u, 0u, 0u, 0u);
    if (wave == 0) {
        // chunk offsets in the candidate list, and the totals the histogram
        // must agree with
        const uint32_t ccl = lane < nchunks ? (cc_l < (uint32_t)CHUNK ? cc_l : (uint32_t)CHUNK) : 0u;
        const uint32_t inc = wave_incl_scan(ccl);
        if (lane < nchunks) sh.off[lane] = inc - ccl;
        const uint32_t tc = wave_incl_scan(tid < nchunks ? cc_l : 0u);
        const uint32_t ta = wave_incl_scan(tid < nchunks ? ac_l : 0u);
        if (lane == 63) {
            sh.m[7] = tc;
            sh.m[8] = ta;
        }
    }
    const uint32_t sum2 = cnt2[0] + cnt2[1] + cnt2[2] + cnt2[3];
    uint32_t tot2;
    const uint32_t incl2 = block_incl_scan<TSEL>(sum2, sh.k.w, &tot2);
    ss[HBINS / 4 - 1 - tid] = make_uint4(0u, 0u, 0u, 0u);
    const bool exact = have_bin && sh.m[7] == C && sh.m[8] == A && tot2 == C;
    const uint32_t need1 = need - A;
    const bool staged = exact && need1 != C && C <= (uint32_t)CAPC;
    uint64_t thr = ~0ull;   // candidates with key >= thr are chosen
    if (exact && need1 == C) {
        thr = (uint64_t)bstar << (32 + HSHIFT);   // the whole bin
    } else if (exact) {
        uint32_t run = incl2 - sum2;
        if (run < need1 && need1 <= incl2) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (run < need1 && need1 <= run + cnt2[j]) {
                    sh.m[4] = (uint32_t)(HBINS - 1 - 4 * tid - j);
                    sh.m[5] = run;
                    sh.m[6] = cnt2[j];
                }
                run += cnt2[j];
            }
        }
        if (staged && pch < nchunks) {
            // chunk pch's candidates to LDS slots [off[pch], +ccnt[pch])
            const uint32_t o = sh.off[pch], n = sh.ccnt[pch];
#pragma unroll
            for (int u = 0; u < PFS; ++u) {
                const uint32_t slot = (uint32_t)(pln + TPC * u);
                if (slot < n) sh.u.cand[o + slot] = pv[u];
            }
            for (uint32_t slot = pln + TPC * PFS; slot < n && pch * CHUNK + (int)slot < Lmax;
                 slot += TPC)
                sh.u.cand[o + slot] = ld64(cseg + (size_t)pch * CHUNK + slot);
        }
        __syncthreads();
        const uint32_t b2 = sh.m[4];
        const int need2 = (int)(need1 - sh.m[5]);
        const int n2 = (int)sh.m[6];
        const uint64_t prefix = ((uint64_t)bstar << (32 + HSHIFT)) | ((uint64_t)b2 << 40);
        const uint64_t mask = ~0ull << 40;
        if (staged) {
            auto visit = [&](auto f) {
                for (int i = tid; i < (int)C; i += TSEL) f(sh.u.cand[i]);
            };
            thr = kth_largest(visit, need2, prefix, mask, 40, n2, sh.k);
        } else {
            auto visit = [&](auto f) {
                for (int c = 0; c < nchunks; ++c) {
                    const int n = (int)sh.ccnt[c];
                    for (int i = tid; i < n && c * CHUNK + i < Lmax; i += TSEL)
                        f(ld64(cseg + (size_t)c * CHUNK + i));
                }
            };
            thr = kth_largest(visit, need2, prefix, mask, 40, n2, sh.k);
        }
    }
    if (exact) {
        // chosen candidates per chunk: each chunk's threads count their slots
        // (in LDS when staged)
        if (pch < nchunks) {
            const uint32_t n = sh.ccnt[pch];
            uint32_t nch = 0;
            if (need1 == C) {
                nch = pln == 0 ? n : 0u;
            } else if (staged) {
                const uint32_t o = sh.off[pch];
                for (uint32_t slot = pln; slot < n; slot += TPC)
                    nch += sh.u.cand[o + slot] >= thr ? 1u : 0u;
            } else {
#pragma unroll
                for (int u = 0; u < PFS; ++u)
                    nch += ((uint32_t)(pln + TPC * u) < n && pv[u] >= thr) ? 1u : 0u;
                for (uint32_t slot = pln + TPC * PFS; slot < n && pch * CHUNK + (int)slot < Lmax;
                     slot += TPC)
                    nch += ld64(cseg + (size_t)pch * CHUNK + slot) >= thr ? 1u : 0u;
            }
#pragma unroll
            for (int m = TPC / 2; m >= 1; m >>= 1) nch += (uint32_t)__shfl_xor((int)nch, m);
            if (pln == 0) sh.chosen[pch] = nch;
        }
    } else {
        // the counts disagree with the histogram: exact selection over every
        // eligible token, its bitmap written here, no candidates
        uint32_t *sk = reinterpret_cast<uint32_t *>(sh.u.cand);
        const int r = R;
        auto visit_all = [&](auto f) {
            for (int a = g.e0; a < g.e1; a += CHUNK) {
                const int z = a + CHUNK < g.e1 ? a + CHUNK : g.e1;
                __syncthreads();
                stage_keys<TSEL>(sk, sc, a - r, z + r, g.e0, g.e1);
                __syncthreads();
                for (int t = a + tid; t < z; t += TSEL) f(pooled_key(sk, a - r, t, g.e0, g.e1, r));
            }
        };
        const uint64_t kth = kth_largest(visit_all, g.need, 0ull, 0ull, 64, nE, sh.k);
        uint32_t *bm = bitmap + (size_t)seg * nwords;
        for (int c0 = 0; c0 < nchunks * CHUNK; c0 += CHUNK) {
            const int a = c0 > g.e0 ? c0 : g.e0;
            const int z = c0 + CHUNK < g.e1 ? c0 + CHUNK : g.e1;
            __syncthreads();
            if (a < z) stage_keys<TSEL>(sk, sc, a - r, z + r, g.e0, g.e1);
            __syncthreads();
            for (int base = c0 + wave * 64; base < c0 + CHUNK; base += TSEL) {
                const int t = base + lane;
                const bool sel = t >= a && t < z && pooled_key(sk, a - r, t, g.e0, g.e1, r) >= kth;
                const uint64_t m = __ballot(sel);
                if (lane == 0) {
                    const int w = base >> 5;
                    // over the words the other workgroups wrote (agent scope too)
                    if (w < nwords)
                        __hip_atomic_store(bm + w, (uint32_t)m, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    if (w + 1 < nwords)
                        __hip_atomic_store(bm + w + 1, (uint32_t)(m >> 32), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    if (m) atomicAdd(&sh.chosen[c0 / CHUNK], (uint32_t)__popcll(m));
                }
            }
        }
        if (tid < nchunks) sh.acnt[tid] = 0u;   // counted in chosen instead
        thr = ~0ull;
    }
    __syncthreads();
    // chunk offsets of the list and the count
    if (wave == 0) {
        uint32_t v = 0;
        if (lane < nchunks)
            v = sh.acnt[lane] + sh.chosen[lane] +
                (uint32_t)fixed_in(lane * CHUNK, (lane + 1) * CHUNK, slo, wlo, L);
        const uint32_t incl = wave_incl_scan(v);
        if (lane < nchunks) coff[(size_t)seg * nchunks + lane] = incl - v;
        if (lane == 63) {
            count[seg] = (int32_t)incl;
            thr_out[seg] = thr;
        }
    }
}


// ---------------------------------------------------------------------------
// hist_pass: the classification alone, for tb_select_attn to resolve the
// threshold (TB_SEL_DEFER_SELECT). One 512-thread workgroup per (segment,
// chunk), each wave one 256-token step of the chunk: the bin B* from the
// segment's histogram (eight bins per thread), then the pass of hist_select
// over the chunk; the chunk's bitmap words, candidate and above-bin counts,
// its candidates and its part of the second histogram are stored for the
// next launch (plain stores), and the first chunk's workgroup stores B*, A
// and C. No workgroup waits for another; four of them share a CU.
constexpr int TP = 512;                    // threads of hist_pass
constexpr int NWP = TP / 64;               // its waves, one step each
static_assert(NWP * SS == CHUNK && TP * 8 == HBINS, "one step per wave, eight bins per thread");

struct HistPassLds {
    uint32_t bm[CHUNK / 32];   // the chunk's bitmap words
    uint32_t sub[HBINS];       // its second histogram
    uint32_t w[NWP];           // block scan
    uint32_t cc, ac;           // candidates, tokens above B*
    uint32_t m[3];             // B*, A, C
};

template <int R>
__global__ __launch_bounds__(TP) void hist_pass_kernel(
    const float *__restrict__ scores, const int32_t *__restrict__ ctx,
    const int32_t *__restrict__ plen, int Hq, int Lmax, int S, int W, int K, int omit_window,
    uint32_t *__restrict__ hist, uint32_t *__restrict__ sub, int nchunks,
    uint32_t *__restrict__ ccount, uint32_t *__restrict__ acount, uint64_t *__restrict__ cand,
    uint32_t *__restrict__ bitmap, int nwords, uint32_t *__restrict__ coff,
    int32_t *__restrict__ count, uint32_t *__restrict__ hinfo, int n_items) {
    static_assert(R >= 0 && R <= 2, "the halo lanes hold radius 2");
    __shared__ __align__(16) HistPassLds sh;
    // XCD-aware order: the chunks of a segment on one XCD (workgroups are
    // dealt to the 8 XCDs in turn), so its histogram is read from that XCD's
    // L2 after the first miss
    const int nb = gridDim.x, bid = blockIdx.x;
    const int item = (bid & 7) * (nb >> 3) + (bid >> 3);
    if (item >= n_items) return;
    const int c = item % nchunks, seg = item / nchunks, b = seg / Hq;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint4 *hs = reinterpret_cast<uint4 *>(hist + (size_t)seg * HBINS);
    uint4 *ss = reinterpret_cast<uint4 *>(sub + (size_t)seg * HBINS);
    const float *sc = scores + (size_t)seg * Lmax;
    // bins 4095 - 8 tid - j, j < 8 (descending thread order), and this wave's
    // step, requested before the lengths arrive (scores from addresses clamped
    // into the cache; values at positions outside E are never used)
    const uint4 *sq = hs + HBINS / 4 - 2 * (tid + 1);
    const uint4 h0 = sq[1], h1 = sq[0];
    const int base = c * CHUNK + wave * SS;
    auto clampL = [&](int p) { return p < 0 ? 0 : (p >= Lmax ? Lmax - 1 : p); };
    float v[4], hl = 0.f, hr = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = sc[clampL(base + lane + 64 * j)];
    if (R > 0) {
        hl = sc[clampL(base - R + lane)];
        hr = sc[clampL(base + SS + lane)];
    }
    const Region g = region(ctx, plen, b, Lmax, S, W, K);
    const int nE = g.e1 - g.e0;
    const bool partial = !g.bad && g.need > 0 && g.need < nE;
    const int L = g.L;
    const int wlo = omit_window ? L : (L - W > 0 ? L - W : 0);
    const int slo = S < L ? S : L;
    const int e0 = g.e0, e1 = g.e1;
    const bool act = partial && base < e1;

    if (!partial) {
        // every eligible token or none: the chunk's words; the first chunk's
        // workgroup writes every chunk's offset and the count, and clears
        // both histograms (untouched by the scoring launch, unless the
        // workspace was not zero at first use)
        const bool all = !g.bad && g.need == nE && nE > 0;
        const int w = c * (CHUNK / 32) + tid;
        if (tid < CHUNK / 32 && w < nwords) {
            const int t0 = w << 5;
            bitmap[(size_t)seg * nwords + w] =
                all ? (bits_below(g.e1 - t0) & ~bits_below(g.e0 - t0)) : 0u;
        }
        if (c != 0) return;
        for (int i = tid; i < HBINS / 4; i += TP) {
            hs[i] = make_uint4(0u, 0u, 0u, 0u);
            ss[i] = make_uint4(0u, 0u, 0u, 0u);
        }
        if (wave == 0) {
            if (g.bad) {
                if (lane == 0) count[seg] = -1;
                return;
            }
            uint32_t v2 = 0;
            if (lane < nchunks) {
                const int t0 = lane * CHUNK, t1 = t0 + CHUNK;
                const int a = t0 > g.e0 ? t0 : g.e0, z = t1 < g.e1 ? t1 : g.e1;
                v2 = (uint32_t)((all && z > a ? z - a : 0) + fixed_in(t0, t1, slo, wlo, L));
            }
            const uint32_t incl = wave_incl_scan(v2);
            if (lane < nchunks) coff[(size_t)seg * nchunks + lane] = incl - v2;
            if (lane == 63) count[seg] = (int32_t)incl;
        }
        return;
    }

    // 1. the bin that holds the budget's key
    if (tid < CHUNK / 32) sh.bm[tid] = 0u;
    for (int i = tid; i < HBINS / 4; i += TP)
        reinterpret_cast<uint4 *>(sh.sub)[i] = make_uint4(0u, 0u, 0u, 0u);
    if (tid == 0) {
        sh.cc = 0u;
        sh.ac = 0u;
        sh.m[0] = sh.m[1] = sh.m[2] = 0u;
    }
    const uint32_t need = (uint32_t)g.need;
    {
        const uint32_t cnt[8] = {h0.w, h0.z, h0.y, h0.x, h1.w, h1.z, h1.y, h1.x};
        uint32_t sum = 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j) sum += cnt[j];
        uint32_t tot;
        const uint32_t incl = block_incl_scan<TP>(sum, sh.w, &tot);
        uint32_t run = incl - sum;
        if (tot >= need && run < need && need <= incl) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (run < need && need <= run + cnt[j]) {
                    sh.m[0] = (uint32_t)(HBINS - 1 - 8 * tid - j);
                    sh.m[1] = run;
                    sh.m[2] = cnt[j];
                }
                run += cnt[j];
            }
        }
        __syncthreads();
    }
    const uint32_t bstar = sh.m[0], C = sh.m[2];
    const bool have_bin = C > 0;   // else the histogram does not hold the budget's rank
    if (c == 0 && tid == 0) {
        hinfo[(size_t)seg * 3] = bstar;
        hinfo[(size_t)seg * 3 + 1] = sh.m[1];
        hinfo[(size_t)seg * 3 + 2] = C;
    }

    // 2. the pass over the wave's step
    if (have_bin && act)
        classify_step<R, false>(base, v, hl, hr, e0, e1, bstar, sh.bm, c * (CHUNK / 32), &sh.ac,
                                &sh.cc, sh.sub, cand + (size_t)seg * Lmax + (size_t)c * CHUNK,
                                Lmax - c * CHUNK);
    __syncthreads();

    // 3. the chunk's state for the attention launch
    const int w = c * (CHUNK / 32) + tid;
    if (tid < CHUNK / 32 && w < nwords) bitmap[(size_t)seg * nwords + w] = sh.bm[tid];
    if (tid == 0) {
        ccount[(size_t)seg * nchunks + c] = sh.cc;
        acount[(size_t)seg * nchunks + c] = sh.ac;
    }
    if (have_bin) {
        // adjacent bins as one 64-bit atomic (counts never carry out of 32 bits)
        for (int i = tid; i < HBINS / 4; i += TP) {
            const uint4 sv = reinterpret_cast<const uint4 *>(sh.sub)[i];
            uint64_t *sb = reinterpret_cast<uint64_t *>(sub + (size_t)seg * HBINS + 4 * i);
            if (sv.x | sv.y)
                __hip_atomic_fetch_add(sb, (uint64_t)sv.x | ((uint64_t)sv.y << 32),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (sv.z | sv.w)
                __hip_atomic_fetch_add(sb + 1, (uint64_t)sv.z | ((uint64_t)sv.w << 32),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace

bool hist_route_fits(int nseg, int Lmax, int g, int r, bool dilate) {
    const int rk = dilate ? 0 : r;
    const int nchunks = (Lmax + CHUNK - 1) / CHUNK;
    // measured: the histogram's flush atomics grow with the context and the
    // number of scoring workgroups, and a group of more than 4 heads leaves
    // one scoring workgroup per CU; beyond 64 chunks, 4 heads per group or 64
    // segments (8 selection workgroups per segment then queue on the CUs)
    // the sampled band was faster
    return nseg <= kHistMaxSeg && Lmax > kHistMinL && rk <= 2 && nchunks <= MAXC && g <= 4;
}

size_t hist_ws_bytes(int B, int Hq, int Lmax) {
    // the histogram and the second histogram of the selection, per segment
    const int nchunks = (Lmax + CHUNK - 1) / CHUNK;
    const long long nseg = (long long)B * Hq;
    return (nseg <= kHistMaxSeg && Lmax > kHistMinL && nchunks <= MAXC)
               ? 2 * (size_t)nseg * HBINS * sizeof(uint32_t)
               : 0;
}

tb_status launch_score_hist_select(const float *qhat, int n_slots, int slot, const void *kp,
                                   const int32_t *ctx, const int32_t *plen, float *scores, int B,
                                   int Hq, int Hkv, int Lmax, int dp, int S, int W, int K, int r,
                                   bool dilate, bool omit_window, int32_t *count,
                                   const SelectWs &ws, hipStream_t st, bool pass_only) {
    const int rk = dilate ? 0 : r;
    const int g = Hq / Hkv;
    score_hist_fn fn = nullptr;
    if (dp == 16)
        fn = rk == 0 ? score_hist_pick<16, 0>(g) : rk == 1 ? score_hist_pick<16, 1>(g)
                                                           : score_hist_pick<16, 2>(g);
    else
        fn = rk == 0 ? score_hist_pick<32, 0>(g) : rk == 1 ? score_hist_pick<32, 1>(g)
                                                           : score_hist_pick<32, 2>(g);
    if (!fn || !ws.hist || rk > 2 || ws.nchunks > MAXC) {
        set_error("tb_score_select: histogram route unavailable for this shape");
        return TB_ERR_UNSUPPORTED_SHAPE;
    }
    const int nxs = (Lmax + TS - 1) / TS;
    const long long nblk = (long long)nxs * Hkv * B;
    if (nblk > 0x7fffffffLL) {
        set_error("tb_score_select: grid of %lld blocks too large", nblk);
        return TB_ERR_UNSUPPORTED_SHAPE;
    }
    hipLaunchKernelGGL(fn, dim3((unsigned)nblk), dim3(TS), 0, st, qhat, n_slots * Hq * dp,
                       slot * Hq * dp, static_cast<const uint16_t *>(kp), ctx, plen, scores, Hq,
                       Hkv, Lmax, S, W, K, nxs, ws.hist);
    tb_status e = check_launch("tb_score_select(score + histogram)");
    if (e) return e;
    if (pass_only) {
        auto pass = rk == 0 ? hist_pass_kernel<0> : rk == 1 ? hist_pass_kernel<1> : hist_pass_kernel<2>;
        const long long items = (long long)B * Hq * ws.nchunks;   // at most 64 x 64 on this route
        const long long nb = (items + 7) / 8 * 8;
        hipLaunchKernelGGL(pass, dim3((unsigned)nb), dim3(TP), 0, st, scores, ctx, plen, Hq, Lmax,
                           S, W, K, omit_window ? 1 : 0, ws.hist, ws.hist + (size_t)B * Hq * HBINS,
                           ws.nchunks, ws.ccount, ws.acount, ws.cand, ws.bitmap, ws.nwords,
                           ws.coff, count, ws.hinfo, (int)items);
        return check_launch("tb_score_select(classify)");
    }
    auto sel = rk == 0 ? hist_select_kernel<0> : rk == 1 ? hist_select_kernel<1> : hist_select_kernel<2>;
    const int nparts = (ws.nchunks + CPW - 1) / CPW;
    hipLaunchKernelGGL(sel, dim3(nparts, B * Hq), dim3(TSEL), 0, st, scores, ctx, plen, Hq, Lmax,
                       S, W, K, omit_window ? 1 : 0, ws.hist, ws.hist + (size_t)B * Hq * HBINS,
                       ws.bctr, ws.nchunks, ws.ccount, ws.acount, ws.cand, ws.bitmap, ws.nwords,
                       ws.thr, ws.coff, count);
    return check_launch("tb_score_select(select)");
}

}  // namespace tb
