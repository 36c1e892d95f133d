// Fixed-budget selection with neighbour fetching, unioned with the sink and
// the local window ("TokenButler" summary, "Inference strategy": the three
// buffers and the neighbour-fetching optimization; "Core architecture":
// selection under a fixed budget).
//
// The greedy fill (visit centres by descending score; each brings itself and
// its neighbours at distance 1..r, left before right, until the budget is
// full) is computed as a ranking: every eligible token t gets the 64-bit key
//     [ key32(score of c(t)) | 0xFFFFFF - c(t) | 0x7F - |t - c(t)| | t <= c(t) ]
// where c(t) is the best centre within distance r of t (highest score, lowest
// position on ties). The greedy order is exactly descending key order, the
// keys are distinct, and the important buffer is the min(K, |E|) largest keys.
//
// Four launches, all integer work:
//   bounds   eight 1024-thread workgroups per segment sample the pooled key32
//            of every stride-th eligible token, stride = ceil((Lmax - S) /
//            8192) (every token when that is 1); the last to arrive takes
//            sample ranks on either side of the budget's rank, 5 sigma of the
//            sample rank apart, as a band [T_lo, T_hi] that holds the K-th
//            key with overwhelming odds;
//   classify per (segment, 2048-token chunk): tokens above the band go
//            straight into a selection bitmap (wave ballots); tokens in it are
//            gathered in LDS and written to the chunk's own candidate slots;
//   thr      one 1024-thread workgroup per segment: checks that the K-th key
//            lies in the band, gathers the candidates, exact select of the
//            remaining quota among them (10-bit radix passes narrow the group
//            to at most 64 keys, which are ranked directly), then each chunk's
//            offset in the output list. If the band missed (a sample that
//            misrepresents the segment), the workgroup instead selects exactly
//            over every eligible token and writes the list itself;
//   compact  one wave per chunk: bitmap words ORed with the chunk's chosen
//            candidates and the sink / window bits, emitted as ascending
//            positions with coalesced stores.
// For small problems tb_score_select replaces the bounds launch by sampling
// workgroups inside the scoring launch (score_bounds_kernel), which compute
// the scores around their samples from the projected keys themselves.
// With TB_SEL_DEFER_LIST the selection stops after the threshold and
// tb_select_attn does the compaction inside the attention launch
// (compact_attn_kernel, select_attn.hip): each attention workgroup rebuilds
// and writes the list rows it attends.
#include "attn_impl.h"
#include "score_impl.h"
#include "select_impl.h"

namespace tb {
namespace {

using namespace sel;

constexpr int T1 = 256;              // threads of classify
constexpr int NSAMP = 8192;          // sample keys per segment (at most)
constexpr int BG = 8;                // bounds workgroups per segment
constexpr int QB = 12;               // bits per level of the band's histograms
constexpr int QBINS = 1 << QB;
constexpr float MARGIN_SIGMAS = 5.f; // half-width of the band in sample-rank std
constexpr int T3 = 1024;             // threads of the bounds and threshold kernels
constexpr int LDS_CAND = 8192;       // candidates held in LDS by the threshold kernel
constexpr int MAX_CHUNKS = (1 << 24) / CHUNK;   // chunks of the largest Lmax

// Band edges from the n sample keys held PER to a thread (key i * T3 + tid in
// v[i], zero past n): t_hi >= the key of rank ka and t_lo <= the key of rank
// kb (ranks 0-based, descending), each the outer edge of the 24-bit bin that
// holds that key (two 12-bit histogram levels: top bits over all keys, then
// bits 19..8 within each rank's top bin). The band only has to contain the
// budget's key, so bin edges serve as well as the exact order statistics.
// Block-wide, T3 threads; s_h1 holds QBINS and s_h2 2 * QBINS counters, both
// zeroed by the caller before a barrier; s_w holds T3 / 64, s_sel 4.
template <int PER>
__device__ __forceinline__ void band_edges(const uint32_t (&v)[PER], int n, int ka, int kb,
                                           uint32_t *s_h1, uint32_t *s_h2, uint32_t *s_w,
                                           int *s_sel, uint32_t *t_hi, uint32_t *t_lo) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t *s_hist = s_h1;
    // level 1: bins of the top QB bits, bin index = descending digit
#pragma unroll
    for (int i = 0; i < PER; ++i)
        if (i * T3 + tid < n) atomicAdd(&s_hist[QBINS - 1 - (v[i] >> (32 - QB))], 1u);
    __syncthreads();
    {
        constexpr int PB = QBINS / T3;
        uint32_t c[PB], sum = 0;
#pragma unroll
        for (int u = 0; u < PB; ++u) {
            c[u] = s_hist[tid * PB + u];
            sum += c[u];
        }
        uint32_t tot;
        // s_w is written next after the barrier below
        uint32_t run = block_incl_scan<T3, false>(sum, s_w, &tot) - sum;
#pragma unroll
        for (int u = 0; u < PB; ++u) {
            const int d = QBINS - 1 - (tid * PB + u);
            if (c[u] > 0 && run <= (uint32_t)ka && (uint32_t)ka < run + c[u]) {
                s_sel[0] = d;
                s_sel[1] = ka - (int)run;
            }
            if (c[u] > 0 && run <= (uint32_t)kb && (uint32_t)kb < run + c[u]) {
                s_sel[2] = d;
                s_sel[3] = kb - (int)run;
            }
            run += c[u];
        }
    }
    __syncthreads();
    const uint32_t da = (uint32_t)s_sel[0], db = (uint32_t)s_sel[2];
    const int ka2 = s_sel[1], kb2 = s_sel[3];
    // level 2: bits 19..8 of the keys in each rank's top bin (histograms A, B)
    s_hist = s_h2;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const uint32_t key = v[i], top = key >> (32 - QB);
        const int d = QBINS - 1 - (int)((key >> (32 - 2 * QB)) & (QBINS - 1));
        const bool in = i * T3 + tid < n;
        if (in && top == da) atomicAdd(&s_hist[d], 1u);
        if (in && top == db) atomicAdd(&s_hist[QBINS + d], 1u);
    }
    __syncthreads();
    {
        // threads [0, T3/2) scan histogram A, [T3/2, T3) histogram B
        constexpr int PB = 2 * QBINS / T3;
        uint32_t c[PB], sum = 0;
#pragma unroll
        for (int u = 0; u < PB; ++u) {
            c[u] = s_hist[tid * PB + u];
            sum += c[u];
        }
        uint32_t x = sum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane == 63) s_w[wave] = x;
        __syncthreads();
        constexpr int HW = T3 / 128;   // waves per half
        uint32_t run = 0;
        for (int w = wave < HW ? 0 : HW; w < wave; ++w) run += s_w[w];
        run += x - sum;
        const bool A = tid < T3 / 2;
        const int kk = A ? ka2 : kb2;
#pragma unroll
        for (int u = 0; u < PB; ++u) {
            if (c[u] > 0 && run <= (uint32_t)kk && (uint32_t)kk < run + c[u]) {
                s_sel[A ? 0 : 2] = QBINS - 1 - ((tid * PB + u) & (QBINS - 1));
            }
            run += c[u];
        }
    }
    __syncthreads();
    *t_hi = (da << (32 - QB)) | ((uint32_t)s_sel[0] << (32 - 2 * QB)) | ((1u << (32 - 2 * QB)) - 1u);
    *t_lo = (db << (32 - QB)) | ((uint32_t)s_sel[2] << (32 - 2 * QB));
}

// Stores the key of sample j (when j < ns) with an agent-scope store, counts
// the workgroup's arrival at segment seg and, in the last of its BG sampling
// workgroups to arrive, reads the samples back with agent-scope loads, resets
// the arrival counter and writes the band. Every thread of the block calls it.
__device__ __forceinline__ void band_from_samples(int seg, int j, int ns, uint32_t key, int stride,
                                                  const Region &g, uint32_t *__restrict__ samp,
                                                  uint32_t *__restrict__ bctr,
                                                  uint32_t *__restrict__ info) {
    __shared__ uint32_t s_h1[QBINS], s_h2[2 * QBINS];
    __shared__ uint32_t s_w[T3 / 64];
    __shared__ int s_sel[4];
    __shared__ bool s_last;
    uint32_t *sp = samp + (size_t)seg * NSAMP;
    if (j < ns) __hip_atomic_store(sp + j, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // the band's histograms are cleared while the samples are stored and
    // counted (the barrier below orders the clearing before their use)
    for (int i = threadIdx.x; i < QBINS; i += T3) s_h1[i] = 0u;
    for (int i = threadIdx.x; i < 2 * QBINS; i += T3) s_h2[i] = 0u;
    // every wave's sample stores complete before the arrival is counted
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0)
        s_last = __hip_atomic_fetch_add(bctr + seg, 1u, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(BG - 1);
    __syncthreads();
    if (!s_last) return;
    if (threadIdx.x == 0) __hip_atomic_store(bctr + seg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    constexpr int PER = NSAMP / T3;
    uint32_t v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int k = threadIdx.x + i * T3;
        v[i] = k < ns ? __hip_atomic_load(sp + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
    }
    const int nE = g.e1 - g.e0;
    // sample ranks (0-based from the top) on either side of the budget's rank
    int rhi, rlo;
    if (stride == 1) {
        rhi = rlo = g.need - 1;
    } else {
        const float f = (float)g.need / (float)nE;
        const float p = f * (float)ns;
        const int m = (int)ceilf(MARGIN_SIGMAS * sqrtf((float)ns * f * (1.f - f))) + 2;
        rhi = (int)floorf(p) - 1 - m;
        rlo = (int)ceilf(p) - 1 + m;
    }
    uint32_t thi, tlo;
    band_edges(v, ns, rhi < 0 ? 0 : rhi, rlo >= ns ? ns - 1 : rlo, s_h1, s_h2, s_w, s_sel, &thi,
               &tlo);
    if (rhi < 0) thi = 0xffffffffu;   // nothing is surely above the budget's key
    if (rlo >= ns) tlo = 0u;          // every key may be a candidate
    if (threadIdx.x == 0) {
        info[2 * seg] = tlo;
        info[2 * seg + 1] = thi;
    }
}

// The sample grid of a segment depends only on S and Lmax: sample j sits at
// position S + off + j * stride, stride = ceil((Lmax - S) / NSAMP) (every
// position when that is 1), off = stride / 2. ns of them fall inside E.
__device__ __forceinline__ int sample_stride(int Lmax, int S) {
    return Lmax > S + NSAMP ? (Lmax - S + NSAMP - 1) / NSAMP : 1;
}

// Workgroup x of a segment samples j in [x * T3, (x + 1) * T3). R >= 0: the
// radius is R (a thread's neighbour loads are all issued before any is used);
// R < 0: any radius, read token by token.
template <int R>
__global__ __launch_bounds__(T3) void bounds_kernel(const float *__restrict__ scores,
                                                    const int32_t *__restrict__ ctx,
                                                    const int32_t *__restrict__ plen, int Hq,
                                                    int Lmax, int S, int W, int K, int r,
                                                    uint32_t *__restrict__ samp,
                                                    uint32_t *__restrict__ bctr,
                                                    uint32_t *__restrict__ info) {
    static_assert(BG * T3 == NSAMP, "one sample per thread");
    const int seg = blockIdx.y, b = seg / Hq;
    // the scores are loaded before the lengths are known; neighbours outside
    // E are dropped after
    const int stride = sample_stride(Lmax, S);
    const int off = stride / 2;
    const float *sc = scores + (size_t)seg * Lmax;
    const int j = blockIdx.x * T3 + threadIdx.x;
    const int t = S + off + j * stride;
    constexpr int NX = R >= 0 ? 2 * R + 1 : 1;
    float x[NX];
    if constexpr (R >= 0) {
#pragma unroll
        for (int u = 0; u < NX; ++u) {
            int p = t - R + u;
            p = p < S ? S : (p >= Lmax ? Lmax - 1 : p);
            x[u] = t < Lmax ? sc[p] : 0.f;
        }
    }
    const Region g = region(ctx, plen, b, Lmax, S, W, K);
    const int nE = g.e1 - g.e0;
    if (g.bad || g.need == 0 || g.need == nE) return;   // the same for every workgroup of seg
    const int ns = nE > off ? (nE - off + stride - 1) / stride : 0;
    uint32_t key = 0u;
    if (j < ns) {
        if constexpr (R >= 0) {
            // key32 of a pooled key = max order key over [t - R, t + R]
            // within E (t itself is in E)
#pragma unroll
            for (int u = 0; u < NX; ++u) {
                const int p = t - R + u;
                const uint32_t k = order_key(x[u]);
                if (p >= g.e0 && p < g.e1 && k > key) key = k;
            }
        } else {
            key = (uint32_t)(pooled_key_g(sc, t, g.e0, g.e1, r) >> 32);
        }
    }
    band_from_samples(seg, j, ns, key, stride, g, samp, bctr, info);
}

// Scoring and the band's samples in one launch. Blocks [0, nsb), nsb = BG *
// segments, sample: block (seg, x) = (blk / BG, blk % BG) recomputes the
// scores of its sample positions and their neighbours straight from the
// projected keys with score_row (the same bits as the scores written by the
// other blocks) and proceeds as bounds_kernel. Blocks [nsb, ...) score T3
// tokens of one (b, KV head) each, as the scoring kernel does. The sampling
// blocks come first, so they are dispatched first and their band work
// overlaps the scoring stream; block x of every segment lands on the same
// XCD, so the g heads of a KV group read the same key rows through one L2.
// Used for radius <= 1 while the sampling blocks number at most one per CU.
template <int G, int DP, int R>
__global__ __launch_bounds__(T3, 8) void score_bounds_kernel(
    const float *__restrict__ qhat, int q_bstride, int q_off, const uint16_t *__restrict__ kp,
    const int32_t *__restrict__ ctx, const int32_t *__restrict__ plen,
    float *__restrict__ scores, int Hq, int Hkv, int Lmax, int S, int W, int K, int nsb, int nxs,
    uint32_t *__restrict__ samp, uint32_t *__restrict__ bctr, uint32_t *__restrict__ info) {
    static_assert(BG * T3 == NSAMP, "one sample per thread");
    static_assert(R <= 1, "two blocks per CU need at most 64 registers");
    constexpr int V = DP / 8;   // 16-byte vectors per key row
    const int blk = blockIdx.x;
    if (blk >= nsb) {
        const int sbk = blk - nsb;
        const int x = sbk % nxs, kvh = (sbk / nxs) % Hkv, b = sbk / (nxs * Hkv);
        int P = plen[b];
        P = P < 0 ? 0 : (P > Lmax ? Lmax : P);
        if (x * T3 >= P) return;
        const int t = x * T3 + (int)threadIdx.x;
        const float *qb = qhat + (size_t)b * q_bstride + q_off + (size_t)kvh * G * DP;
        float q[G][DP];
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int c = 0; c < DP; ++c) q[gi][c] = qb[gi * DP + c];
        if (t >= P) return;
        const uint4 *kb = reinterpret_cast<const uint4 *>(kp + (size_t)(b * Hkv + kvh) * Lmax * DP);
        uint4 raw[V];
#pragma unroll
        for (int v = 0; v < V; ++v) raw[v] = kb[(size_t)t * V + v];
        float *sb = scores + (size_t)(b * Hq + kvh * G) * Lmax;
#pragma unroll
        for (int gi = 0; gi < G; ++gi) sb[(size_t)gi * Lmax + t] = score_row<DP>(raw, q[gi]);
        return;
    }
    const int seg = blk / BG, b = seg / Hq, h = seg - b * Hq, kvh = h / G;
    const int stride = sample_stride(Lmax, S);
    const int off = stride / 2;
    const int j = (blk % BG) * T3 + (int)threadIdx.x;
    const int t = S + off + j * stride;
    constexpr int NX = 2 * R + 1;
    const uint4 *kb = reinterpret_cast<const uint4 *>(kp + (size_t)(b * Hkv + kvh) * Lmax * DP);
    // the key rows are loaded before the lengths are known; neighbours
    // outside E are dropped after
    uint4 raw[NX][V];
    if (t < Lmax) {
#pragma unroll
        for (int u = 0; u < NX; ++u) {
            int p = t - R + u;
            p = p < S ? S : (p >= Lmax ? Lmax - 1 : p);
#pragma unroll
            for (int v = 0; v < V; ++v) raw[u][v] = kb[(size_t)p * V + v];
        }
    }
    float q[DP];
    const float *qh = qhat + (size_t)b * q_bstride + q_off + (size_t)h * DP;
#pragma unroll
    for (int c = 0; c < DP; ++c) q[c] = qh[c];
    const Region g = region(ctx, plen, b, Lmax, S, W, K);
    const int nE = g.e1 - g.e0;
    if (g.bad || g.need == 0 || g.need == nE) return;   // the same for every workgroup of seg
    const int ns = nE > off ? (nE - off + stride - 1) / stride : 0;
    uint32_t key = 0u;
    if (j < ns) {
#pragma unroll
        for (int u = 0; u < NX; ++u) {
            const int p = t - R + u;
            const uint32_t k = order_key(score_row<DP>(raw[u], q));
            if (p >= g.e0 && p < g.e1 && k > key) key = k;
        }
    }
    band_from_samples(seg, j, ns, key, stride, g, samp, bctr, info);
}

typedef void (*score_bounds_fn)(const float *, int, int, const uint16_t *, const int32_t *,
                                const int32_t *, float *, int, int, int, int, int, int, int, int,
                                uint32_t *, uint32_t *, uint32_t *);

template <int DP, int R>
score_bounds_fn score_bounds_pick(int g) {
    switch (g) {
        case 1: return score_bounds_kernel<1, DP, R>;
        case 2: return score_bounds_kernel<2, DP, R>;
        case 3: return score_bounds_kernel<3, DP, R>;
        case 4: return score_bounds_kernel<4, DP, R>;
        case 5: return score_bounds_kernel<5, DP, R>;
        case 6: return score_bounds_kernel<6, DP, R>;
        case 7: return score_bounds_kernel<7, DP, R>;
        case 8: return score_bounds_kernel<8, DP, R>;
        default: return nullptr;
    }
}

// R >= 0: the radius is R (pooled keys read their neighbours together);
// R < 0: any radius, neighbours read one by one. Each wave handles CHUNK /
// waves tokens and keeps its candidates in its own LDS region, so no slot is
// claimed with an atomic; the regions are written out back to back.
template <int R>
__global__ __launch_bounds__(T1) void classify_kernel(
    const float *__restrict__ scores, const int32_t *__restrict__ ctx,
    const int32_t *__restrict__ plen, int Hq, int Lmax, int S, int W, int K, int r,
    const uint32_t *__restrict__ info, uint32_t *__restrict__ ccount,
    uint32_t *__restrict__ acount, int nchunks, uint64_t *__restrict__ cand,
    uint32_t *__restrict__ bitmap, int nwords) {
    constexpr int NWV = T1 / 64;          // waves
    constexpr int WREG = CHUNK / NWV;     // tokens (and candidate slots) per wave
    __shared__ uint32_t sk[CHUNK + 2 * MAXR];
    __shared__ uint64_t s_cand[CHUNK];
    __shared__ uint32_t s_wc[NWV], s_wa[NWV];
    const int seg = blockIdx.y, b = seg / Hq;
    const int c0 = blockIdx.x * CHUNK;
    const int rr = R >= 0 ? R : r;
    const int lo = c0 - rr;   // LDS slot i holds position lo + i
    // the chunk's scores (with halo) and the band are loaded before the
    // lengths are known; positions outside E are masked when staged
    constexpr int PER = (CHUNK + 2 * MAXR + T1 - 1) / T1;
    const float *sc = scores + (size_t)seg * Lmax;
    float v[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int t = lo + (int)threadIdx.x + k * T1;
        v[k] = (t >= 0 && t < Lmax && t < c0 + CHUNK + rr) ? sc[t] : 0.f;
    }
    const uint32_t tlo = info[2 * seg], thi = info[2 * seg + 1];
    const Region g = region(ctx, plen, b, Lmax, S, W, K);
    uint32_t *bm = bitmap + (size_t)seg * nwords;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nE = g.e1 - g.e0;
    const bool all = !g.bad && g.need == nE && nE > 0;
    const bool partial = !g.bad && g.need > 0 && g.need < nE;
    const int a = c0 > g.e0 ? c0 : g.e0;
    const int z = c0 + CHUNK < g.e1 ? c0 + CHUNK : g.e1;
    const bool touch = partial && a < z;
    if (touch) {
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = (int)threadIdx.x + k * T1;
            const int t = lo + i;
            if (t < c0 + CHUNK + rr) sk[i] = (t >= g.e0 && t < g.e1) ? order_key(v[k]) : 0u;
        }
    }
    __syncthreads();
    // every word of this chunk is written: 64 tokens per wave per step. The
    // keys of all NIT steps are formed first (their LDS reads issued
    // together), then each step's ballots and stores
    constexpr int NIT = CHUNK / T1;
    uint64_t *wcand = s_cand + wave * WREG;
    uint32_t nc_w = 0, na_w = 0;   // this wave's candidates and above-band tokens
    uint64_t keys[NIT];
    bool sels[NIT], iscs[NIT];
    // with the radius fixed, every lane forms its NIT keys from the staged
    // slots (all written when the chunk is touched) in one branch-free loop,
    // so their LDS reads are issued together; tokens outside E drop them
    if constexpr (R >= 0) {
#pragma unroll
        for (int it = 0; it < NIT; ++it) keys[it] = 0;
        if (touch) {
#pragma unroll
            for (int it = 0; it < NIT; ++it)
                keys[it] = pooled_key_r<R>(sk, lo, c0 + wave * 64 + it * T1 + lane);
        }
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int t = c0 + wave * 64 + it * T1 + lane;
        bool sel = false, isc = false;
        uint64_t key = 0;
        if (t >= g.e0 && t < g.e1 && !g.bad) {
            if (all) {
                sel = true;
            } else if (touch) {
                if constexpr (R >= 0) key = keys[it];
                else key = pooled_key(sk, lo, t, g.e0, g.e1, r);
                const uint32_t k32 = (uint32_t)(key >> 32);
                sel = k32 > thi;
                isc = !sel && k32 >= tlo;
            }
        }
        keys[it] = key;
        sels[it] = sel;
        iscs[it] = isc;
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int base = c0 + wave * 64 + it * T1;
        if (base >= nwords * 32) break;
        const uint64_t m = __ballot(sels[it]);
        if (lane == 0) {
            const int w = base >> 5;
            bm[w] = (uint32_t)m;
            if (w + 1 < nwords) bm[w + 1] = (uint32_t)(m >> 32);
        }
        na_w += (uint32_t)__popcll(m);
        const uint64_t cm = __ballot(iscs[it]);
        if (iscs[it]) wcand[nc_w + __popcll(cm & ((1ull << lane) - 1ull))] = keys[it];
        nc_w += (uint32_t)__popcll(cm);
    }
    if (lane == 0) {
        s_wc[wave] = nc_w;
        s_wa[wave] = na_w;
    }
    __syncthreads();
    uint32_t nc = 0, na = 0, before = 0;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
        nc += s_wc[w];
        na += s_wa[w];
        before += w < wave ? s_wc[w] : 0u;
    }
    if (threadIdx.x == 0 && (int)blockIdx.x < nchunks) {
        ccount[(size_t)seg * nchunks + blockIdx.x] = nc;
        acount[(size_t)seg * nchunks + blockIdx.x] = na;
    }
    // the chunk owns candidate slots [c0, c0 + CHUNK) of its segment; each
    // wave writes its region at its offset
    uint64_t *cl = cand + (size_t)seg * Lmax + c0;
    for (uint32_t i = lane; i < nc_w; i += 64)
        if (c0 + (int)(before + i) < Lmax) cl[before + i] = wcand[i];
}

// One workgroup per segment. With A tokens above the band and C candidates
// in it, the band holds the budget's key iff 0 <= need - A <= C; then the
// (need - A)-th largest candidate is the threshold and every chunk's output
// offset (above-band tokens + chosen candidates + sink / window positions in
// the chunk) is scanned. Otherwise the workgroup finds the threshold over
// every eligible token and rewrites the eligible part of the bitmap itself
// (compact then takes no candidates).
__global__ __launch_bounds__(T3) void thr_kernel(
    const float *__restrict__ scores, const int32_t *__restrict__ ctx,
    const int32_t *__restrict__ plen, int Hq, int Lmax, int S, int W, int K, int r,
    int omit_window, const uint32_t *__restrict__ info, const uint32_t *__restrict__ ccount,
    const uint32_t *__restrict__ acount, int nchunks, const uint64_t *__restrict__ cand,
    uint32_t *__restrict__ bitmap, int nwords, uint64_t *__restrict__ thr_out,
    uint32_t *__restrict__ coff, int32_t *__restrict__ count) {
    __shared__ uint64_t s_cand[LDS_CAND];
    __shared__ uint16_t s_cc[LDS_CAND];          // chunk of each LDS candidate
    __shared__ uint32_t s_off[MAX_CHUNKS];
    __shared__ uint32_t s_chosen[MAX_CHUNKS];
    __shared__ KthLds<T3> s_k;
    __shared__ uint32_t s_tot[2];

    const int seg = blockIdx.x, b = seg / Hq;
    const int tid = threadIdx.x;
    constexpr int PC = MAX_CHUNKS / T3;
    // chunk c's counts sit in thread c / PC: with at most 64 PC chunks they
    // all sit in wave 0, whose shuffles then replace the block-wide scans
    const bool small = nchunks <= 64 * PC;
    uint32_t cc[PC], ac[PC];
    // per-chunk counts and the band are loaded before the lengths are known
#pragma unroll
    for (int j = 0; j < PC; ++j) {
        const int c = tid * PC + j;
        cc[j] = c < nchunks ? ccount[(size_t)seg * nchunks + c] : 0u;
        ac[j] = c < nchunks ? acount[(size_t)seg * nchunks + c] : 0u;
    }
    // with at most T3 / 32 chunks, 32 threads per chunk also fetch its first
    // PFC candidate slots now (whatever the counts turn out to be), so that
    // staging the candidates in LDS takes no round trip of its own
    constexpr int PFC = 3;
    const bool pre = nchunks <= T3 / 32;
    const int pch = tid >> 5, pln = tid & 31;
    const uint64_t *cl = cand + (size_t)seg * Lmax;
    uint64_t pv[PFC];
#pragma unroll
    for (int u = 0; u < PFC; ++u) {
        const int slot = pln + 32 * u;
        pv[u] = (pre && pch < nchunks && pch * CHUNK + slot < Lmax)
                    ? cl[(size_t)pch * CHUNK + slot]
                    : 0ull;
    }
    const uint32_t tlo = info[2 * seg], thi = info[2 * seg + 1];
    const Region g = region(ctx, plen, b, Lmax, S, W, K);
    if (g.bad) {
        if (tid == 0) count[seg] = -1;
        return;
    }
    const int nE = g.e1 - g.e0;
    const bool partial = g.need > 0 && g.need < nE;
    const int L = g.L;
    const int wlo = omit_window ? L : (L - W > 0 ? L - W : 0);
    const int slo = S < L ? S : L;
    uint32_t csum = 0, asum = 0;
#pragma unroll
    for (int j = 0; j < PC; ++j) {
        const int c = tid * PC + j;
        if (!partial) cc[j] = 0u;
        if (g.need == 0) ac[j] = 0u;
        csum += cc[j];
        asum += ac[j];
        if (c < nchunks) s_chosen[c] = 0u;
    }
    uint64_t thr = ~0ull;   // candidates with key >= thr are chosen (none by default)
    if (partial) {
        uint32_t nc, above;
        if (small) {
            if (tid < 64) {
                const uint32_t incl = wave_incl_scan(csum);
                uint32_t run = incl - csum;
#pragma unroll
                for (int j = 0; j < PC; ++j) {
                    const int c = tid * PC + j;
                    if (c < nchunks) s_off[c] = run;
                    run += cc[j];
                }
                const uint32_t a_incl = wave_incl_scan(asum);
                if (tid == 63) {
                    s_tot[0] = incl;
                    s_tot[1] = a_incl;
                }
            }
            __syncthreads();
            nc = s_tot[0];
            above = s_tot[1];
        } else {
            uint32_t run = block_incl_scan<T3>(csum, s_k.w, &nc) - csum;
#pragma unroll
            for (int j = 0; j < PC; ++j) {
                const int c = tid * PC + j;
                if (c < nchunks) s_off[c] = run;
                run += cc[j];
            }
            block_incl_scan<T3>(asum, s_k.w, &above);
        }
        const int need1 = g.need - (int)above;
        if (need1 >= 0 && need1 <= (int)nc) {
            if (need1 == (int)nc) {
                thr = 0ull;   // every candidate is chosen
#pragma unroll
                for (int j = 0; j < PC; ++j) {
                    const int c = tid * PC + j;
                    if (c < nchunks) s_chosen[c] = cc[j];
                }
            } else if (need1 > 0) {
                const bool lds = nc <= (uint32_t)LDS_CAND;
                if (lds && pre) {
                    // chunk pch's candidates go to LDS slots [s_off[pch], +n_c)
                    if (pch < nchunks) {
                        const uint32_t o = s_off[pch];
                        const uint32_t n_c = (pch + 1 < nchunks ? s_off[pch + 1] : nc) - o;
#pragma unroll
                        for (int u = 0; u < PFC; ++u) {
                            const uint32_t slot = (uint32_t)(pln + 32 * u);
                            if (slot < n_c) s_cand[o + slot] = pv[u];
                        }
                        for (uint32_t slot = pln + 32 * PFC;
                             slot < n_c && slot < (uint32_t)CHUNK && pch * CHUNK + (int)slot < Lmax;
                             slot += 32)
                            s_cand[o + slot] = cl[(size_t)pch * CHUNK + slot];
                    }
                } else if (lds) {
                    constexpr int PER = LDS_CAND / T3;
                    uint64_t v[PER];
                    int vc[PER];
#pragma unroll
                    for (int j = 0; j < PER; ++j) {
                        const int i = tid + j * T3;
                        vc[j] = 0;
                        v[j] = 0ull;
                        if (i < (int)nc) {
                            vc[j] = chunk_of(s_off, nchunks, (uint32_t)i);
                            v[j] = cl[(size_t)vc[j] * CHUNK + ((uint32_t)i - s_off[vc[j]])];
                        }
                    }
#pragma unroll
                    for (int j = 0; j < PER; ++j) {
                        const int i = tid + j * T3;
                        if (i < (int)nc) {
                            s_cand[i] = v[j];
                            s_cc[i] = (uint16_t)vc[j];
                        }
                    }
                }
                s_k.tile[tid] = 0u;   // the exact select's state, zero on entry
                if (tid == 0) s_k.ng = 0u;
                __syncthreads();
                auto visit_cand = [&](auto f) {
                    for (int i = tid; i < (int)nc; i += T3)
                        f(lds ? s_cand[i] : cand_at(cl, s_off, nchunks, (uint32_t)i));
                };
                // ranked on the keys less the band's lower end: the order is
                // kept (every candidate's key32 lies in [tlo, thi]) and the
                // digits above the band's width are zero, so the radix passes
                // start at that width
                const uint64_t base = (uint64_t)tlo << 32;
                auto visit_off = [&](auto f) { visit_cand([&](uint64_t key) { f(key - base); }); };
                const uint32_t dx = thi - tlo;
                const int shift = 32 + (dx ? 32 - __clz((int)dx) : 0);
                const uint64_t mask = shift >= 64 ? 0ull : (~0ull << shift);
                thr = kth_largest(visit_off, need1, 0ull, mask, shift, (int)nc, s_k) + base;
                if (lds && pre) {
                    // chosen candidates per chunk: each chunk's 32 threads
                    // count the slots they staged and sum over the half wave
                    if (pch < nchunks) {
                        const uint32_t o = s_off[pch];
                        const uint32_t n_c = (pch + 1 < nchunks ? s_off[pch + 1] : nc) - o;
                        uint32_t n = 0;
#pragma unroll
                        for (int u = 0; u < PFC; ++u)
                            n += ((uint32_t)(pln + 32 * u) < n_c && pv[u] >= thr) ? 1u : 0u;
                        for (uint32_t slot = pln + 32 * PFC;
                             slot < n_c && slot < (uint32_t)CHUNK && pch * CHUNK + (int)slot < Lmax;
                             slot += 32)
                            n += s_cand[o + slot] >= thr ? 1u : 0u;
#pragma unroll
                        for (int m = 16; m >= 1; m >>= 1) n += __shfl_xor(n, m);
                        if (pln == 0) s_chosen[pch] = n;
                    }
                }
                // otherwise: candidates are chunk-major, so a wave's lanes form
                // runs of one chunk; each run's first lane adds the run's count
                const int lane = tid & 63;
                for (int i0 = 0; i0 < ((lds && pre) ? 0 : (int)nc); i0 += T3) {
                    const int i = i0 + tid;
                    int c = -1;
                    bool ch = false;
                    if (i < (int)nc) {
                        const uint64_t key = lds ? s_cand[i] : cand_at(cl, s_off, nchunks, i);
                        c = lds ? (int)s_cc[i] : chunk_of(s_off, nchunks, i);
                        ch = key >= thr;
                    }
                    const int prev = __shfl_up(c, 1);
                    const bool head = c >= 0 && (lane == 0 || prev != c);
                    const uint64_t hm = __ballot(head);
                    const uint64_t cm = __ballot(ch);
                    if (head) {
                        const uint64_t later = lane == 63 ? 0ull : (hm >> (lane + 1)) << (lane + 1);
                        const int nxt = later ? __ffsll((long long)later) - 1 : 64;
                        const uint64_t run = (nxt == 64 ? ~0ull : ((1ull << nxt) - 1ull)) &
                                             (~0ull << lane);
                        const int n = __popcll(cm & run);
                        if (n) atomicAdd(&s_chosen[c], (uint32_t)n);
                    }
                }
            }
        } else {
            // the band missed the budget's key: exact selection over every
            // eligible token, pooled keys rebuilt from the scores tile by tile
            const float *sc = scores + (size_t)seg * Lmax;
            uint32_t *sk = reinterpret_cast<uint32_t *>(s_cand);
            auto visit_all = [&](auto f) {
                for (int a = g.e0; a < g.e1; a += CHUNK) {
                    const int z = a + CHUNK < g.e1 ? a + CHUNK : g.e1;
                    __syncthreads();
                    stage_keys<T3>(sk, sc, a - r, z + r, g.e0, g.e1);
                    __syncthreads();
                    for (int t = a + tid; t < z; t += T3) f(pooled_key(sk, a - r, t, g.e0, g.e1, r));
                }
            };
            s_k.tile[tid] = 0u;   // the exact select's state, zero on entry
            if (tid == 0) s_k.ng = 0u;
            __syncthreads();
            const uint64_t kth = kth_largest(visit_all, g.need, 0ull, 0ull, 64, nE, s_k);
            uint32_t *bm = bitmap + (size_t)seg * nwords;
            const int lane = tid & 63, wave = tid >> 6;
            for (int c0 = (g.e0 / CHUNK) * CHUNK; c0 < g.e1; c0 += CHUNK) {
                const int a = c0 > g.e0 ? c0 : g.e0;
                const int z = c0 + CHUNK < g.e1 ? c0 + CHUNK : g.e1;
                __syncthreads();
                stage_keys<T3>(sk, sc, a - r, z + r, g.e0, g.e1);
                __syncthreads();
                for (int base = c0 + wave * 64; base < c0 + CHUNK; base += T3) {
                    const int t = base + lane;
                    const bool sel = t >= a && t < z && pooled_key(sk, a - r, t, g.e0, g.e1, r) >= kth;
                    const uint64_t m = __ballot(sel);
                    if (lane == 0 && base + 64 > a && base < z) {
                        const int w = base >> 5;
                        bm[w] = (uint32_t)m;
                        if (w + 1 < nwords) bm[w + 1] = (uint32_t)(m >> 32);
                        if (m) atomicAdd(&s_chosen[c0 / CHUNK], (uint32_t)__popcll(m));
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < PC; ++j) ac[j] = 0u;   // counted in s_chosen instead
        }
    }
    __syncthreads();
    // chunk offsets of the output list
    uint32_t tot_c[PC];
    uint32_t lsum = 0;
#pragma unroll
    for (int j = 0; j < PC; ++j) {
        const int c = tid * PC + j;
        tot_c[j] = 0u;
        if (c < nchunks)
            tot_c[j] = ac[j] + s_chosen[c] + (uint32_t)fixed_in(c * CHUNK, (c + 1) * CHUNK, slo, wlo, L);
        lsum += tot_c[j];
    }
    if (small) {
        if (tid < 64) {
            const uint32_t incl = wave_incl_scan(lsum);
            uint32_t run = incl - lsum;
#pragma unroll
            for (int j = 0; j < PC; ++j) {
                const int c = tid * PC + j;
                if (c < nchunks) coff[(size_t)seg * nchunks + c] = run;
                run += tot_c[j];
            }
            if (tid == 63) {
                count[seg] = (int32_t)incl;
                thr_out[seg] = thr;
            }
        }
        return;
    }
    uint32_t total;
    uint32_t run = block_incl_scan<T3>(lsum, s_k.w, &total) - lsum;
#pragma unroll
    for (int j = 0; j < PC; ++j) {
        const int c = tid * PC + j;
        if (c < nchunks) coff[(size_t)seg * nchunks + c] = run;
        run += tot_c[j];
    }
    if (tid == 0) {
        count[seg] = (int32_t)total;
        thr_out[seg] = thr;
    }
}

// Wave-wide: lane l holds word l of chunk c (tokens c * CHUNK + 32 l + bit);
// the set bits are written as ascending positions from list slot `base` on,
// 64 at a time (a converged binary search over the words' prefix counts gives
// each lane its word and bit), stopping at cap.
__device__ __forceinline__ void emit_words(uint32_t mine, int c, uint32_t base, int32_t *dst,
                                           int cap) {
    const int lane = threadIdx.x & 63;
    const uint32_t pop = (uint32_t)__popc(mine);
    uint32_t incl = pop;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    const uint32_t first = incl - pop;
    const uint32_t wend = __shfl(incl, 63);
    for (uint32_t s0 = 0; s0 < wend; s0 += 64) {
        const uint32_t sl = s0 + (uint32_t)lane;
        int lo2 = 0;
#pragma unroll
        for (int step = 32; step >= 1; step >>= 1) {
            const uint32_t f = __shfl(first, lo2 + step);
            if (f <= sl) lo2 += step;
        }
        const uint32_t wbits = __shfl(mine, lo2);
        const uint32_t k = sl - __shfl(first, lo2);
        const uint32_t p = base + sl;
        if (sl < wend && p < (uint32_t)cap)
            dst[p] = ((c * (CHUNK / 32) + lo2) << 5) + select_bit(wbits, k);
    }
}

// One wave per (chunk, segment): the chunk's 64 bitmap words, ORed with its
// chosen candidates and the sink / window bits, are emitted as ascending
// positions at the chunk's offset with coalesced stores.
__global__ __launch_bounds__(64) void compact_kernel(
    const int32_t *__restrict__ ctx, const int32_t *__restrict__ plen, int Hq, int Lmax, int S,
    int W, int K, int omit_window, const uint32_t *__restrict__ ccount, int nchunks,
    const uint64_t *__restrict__ cand, const uint32_t *__restrict__ bitmap, int nwords,
    const uint64_t *__restrict__ thr_in, const uint32_t *__restrict__ coff,
    int32_t *__restrict__ idx, int cap) {
    __shared__ uint32_t s_word[64];
    const int c = blockIdx.x, seg = blockIdx.y, b = seg / Hq;
    const int lane = threadIdx.x;
    const int w = c * (CHUNK / 32) + lane;
    const int t0 = w << 5;
    // the chunk's words, offset, candidate count and the threshold are loaded
    // before the lengths are known
    uint32_t bits = w < nwords ? bitmap[(size_t)seg * nwords + w] : 0u;
    const uint32_t base = coff[(size_t)seg * nchunks + c];
    const uint32_t nraw = ccount[(size_t)seg * nchunks + c];
    const uint64_t thr_raw = thr_in[seg];
    // so are the chunk's first 128 candidate slots (used if that many are filled)
    constexpr int PF = 2;
    const uint64_t *cl = cand + (size_t)seg * Lmax + (size_t)c * CHUNK;
    uint64_t pk[PF];
#pragma unroll
    for (int k = 0; k < PF; ++k) {
        const int i = lane + 64 * k;
        pk[k] = c * CHUNK + i < Lmax ? cl[i] : 0ull;
    }
    const Region g = region(ctx, plen, b, Lmax, S, W, K);
    const int L = g.L;
    if (g.bad || c * CHUNK >= L) return;
    const int nE = g.e1 - g.e0;
    const bool partial = g.need > 0 && g.need < nE;
    const int wlo = omit_window ? L : (L - W > 0 ? L - W : 0);
    const int slo = S < L ? S : L;
    if (g.need == 0) bits = 0u;
    uint32_t n = 0;
    uint64_t thr = 0;
    if (partial) {
        thr = thr_raw;
        n = thr == ~0ull ? 0u : (nraw < (uint32_t)CHUNK ? nraw : (uint32_t)CHUNK);
    }
    bits |= bits_below(slo - t0);
    bits |= bits_below(L - t0) & ~bits_below(wlo - t0);
    bits &= bits_below(L - t0);
    s_word[lane] = bits;
    __syncthreads();
    // a candidate's position lies in its chunk after the selection this call
    // follows; anything else (a state left by another call sequence) is
    // ignored rather than written outside the chunk
#pragma unroll
    for (int k = 0; k < PF; ++k) {
        if ((uint32_t)(lane + 64 * k) < n && pk[k] >= thr) {
            const int t = key_token(pk[k]) - c * CHUNK;
            if ((uint32_t)t < (uint32_t)CHUNK) atomicOr(&s_word[t >> 5], 1u << (t & 31));
        }
    }
    for (uint32_t i = lane + 64 * PF; i < n && c * CHUNK + (int)i < Lmax; i += 64) {
        const uint64_t key = cl[i];
        if (key >= thr) {
            const int t = key_token(key) - c * CHUNK;
            if ((uint32_t)t < (uint32_t)CHUNK) atomicOr(&s_word[t >> 5], 1u << (t & 31));
        }
    }
    __syncthreads();
    emit_words(s_word[lane], c, base, idx + (size_t)seg * cap, cap);
}

// Dilation mode, one wave per (chunk, segment): the centres are the top-K
// tokens found with radius 0 (bitmap words and chosen candidates). Lane l
// widens word l of the chunk: it ORs the centre bit stream shifted by every
// distance in [-r, r] (the chunk's words plus HALO words on either side,
// candidates of the neighbouring chunks included), keeps the eligible bits,
// and stores the word and the chunk's count.
constexpr int HALO = (MAXR + 31) / 32;
__global__ __launch_bounds__(64) void dilate_kernel(
    const int32_t *__restrict__ ctx, const int32_t *__restrict__ plen, int Hq, int Lmax, int S,
    int W, int K, int r, const uint32_t *__restrict__ ccount, int nchunks,
    const uint64_t *__restrict__ cand, const uint32_t *__restrict__ bitmap, int nwords,
    const uint64_t *__restrict__ thr_in, uint32_t *__restrict__ dbm,
    uint32_t *__restrict__ dcount) {
    __shared__ uint32_t s_cw[64 + 2 * HALO + 1];
    const int c = blockIdx.x, seg = blockIdx.y, b = seg / Hq;
    const int lane = threadIdx.x;
    const int w0 = c * (CHUNK / 32) - HALO;   // word of s_cw[0]
    const Region g = region(ctx, plen, b, Lmax, S, W, K);
    if (g.bad) return;
    const int nE = g.e1 - g.e0;
    const bool partial = g.need > 0 && g.need < nE;
    const uint64_t thr = partial ? thr_in[seg] : ~0ull;
    for (int j = lane; j < 64 + 2 * HALO + 1; j += 64) {
        const int w = w0 + j;
        s_cw[j] = (g.need > 0 && j < 64 + 2 * HALO && w >= 0 && w < nwords)
                      ? bitmap[(size_t)seg * nwords + w] : 0u;
    }
    __syncthreads();
    if (thr != ~0ull) {
        for (int cc = c - 1; cc <= c + 1; ++cc) {
            if (cc < 0 || cc >= nchunks) continue;
            uint32_t n = ccount[(size_t)seg * nchunks + cc];
            n = n < (uint32_t)CHUNK ? n : (uint32_t)CHUNK;
            const uint64_t *cl = cand + (size_t)seg * Lmax + (size_t)cc * CHUNK;
            for (uint32_t i = lane; i < n && cc * CHUNK + (int)i < Lmax; i += 64) {
                const uint64_t key = cl[i];
                if (key >= thr) {
                    const int t = key_token(key);
                    const int j = (t >> 5) - w0;
                    if (j >= 0 && j < 64 + 2 * HALO) atomicOr(&s_cw[j], 1u << (t & 31));
                }
            }
        }
    }
    __syncthreads();
    const int w = c * (CHUNK / 32) + lane;
    const int t0 = w << 5;
    uint32_t d = 0;
    if (g.need > 0) {
        for (int dd = -r; dd <= r; ++dd) {
            const int p = 32 * (lane + HALO) + dd;   // >= 0 since 32 * HALO >= r
            const int q = p >> 5, o = p & 31;
            d |= o ? (s_cw[q] >> o) | (s_cw[q + 1] << (32 - o)) : s_cw[q];
        }
        d &= bits_below(g.e1 - t0) & ~bits_below(g.e0 - t0);
    }
    if (w < nwords) dbm[(size_t)seg * nwords + w] = d;
    uint32_t n = (uint32_t)__popc(d);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) n += __shfl_xor(n, off);
    if (lane == 0) dcount[(size_t)seg * nchunks + c] = n;
}

// Dilation mode, one wave per (chunk, segment): the chunk's list offset is
// the widened tokens of the earlier chunks plus the sink / window positions
// before it; its widened words ORed with the sink / window bits are emitted.
// The wave of chunk 0 writes the segment's count.
__global__ __launch_bounds__(64) void emit_dilated_kernel(
    const int32_t *__restrict__ ctx, const int32_t *__restrict__ plen, int Hq, int Lmax, int S,
    int W, int K, int omit_window, const uint32_t *__restrict__ dbm, int nwords,
    const uint32_t *__restrict__ dcount, int nchunks, int32_t *__restrict__ idx,
    int32_t *__restrict__ count, int cap) {
    const int c = blockIdx.x, seg = blockIdx.y, b = seg / Hq;
    const int lane = threadIdx.x;
    const Region g = region(ctx, plen, b, Lmax, S, W, K);
    if (g.bad) return;
    const int L = g.L;
    const int wlo = omit_window ? L : (L - W > 0 ? L - W : 0);
    const int slo = S < L ? S : L;
    const uint32_t *dc = dcount + (size_t)seg * nchunks;
    uint32_t before = 0, all = 0;
    for (int j = lane; j < nchunks; j += 64) {
        const uint32_t v = dc[j];
        before += j < c ? v : 0u;
        all += v;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        before += __shfl_xor(before, off);
        all += __shfl_xor(all, off);
    }
    if (c == 0 && lane == 0) count[seg] = (int32_t)(all + (uint32_t)fixed_in(0, L, slo, wlo, L));
    if (c * CHUNK >= L) return;
    const int w = c * (CHUNK / 32) + lane;
    const int t0 = w << 5;
    uint32_t bits = w < nwords ? dbm[(size_t)seg * nwords + w] : 0u;
    bits |= bits_below(slo - t0);
    bits |= bits_below(L - t0) & ~bits_below(wlo - t0);
    bits &= bits_below(L - t0);
    emit_words(bits, c, before + (uint32_t)fixed_in(0, c * CHUNK, slo, wlo, L),
               idx + (size_t)seg * cap, cap);
}
}  // namespace

size_t select_ws_layout(int B, int Hq, int Lmax, void *base, SelectWs *out) {
    const size_t nseg = (size_t)B * Hq;
    const int nwords = (Lmax + 31) / 32 + 1;
    const int nchunks = (Lmax + CHUNK - 1) / CHUNK;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t bctr_b = up(nseg * 4);
    const size_t info_b = up(nseg * 8);
    const size_t hinfo_b = up(nseg * 12);
    const size_t cc_b = up(nseg * (size_t)nchunks * 4);
    const size_t thr_b = up(nseg * 8);
    const size_t bm_b = up(nseg * (size_t)nwords * 4);
    const size_t cand_b = up(nseg * (size_t)Lmax * 8);
    const size_t samp_b = up(nseg * (size_t)NSAMP * 4);
    const size_t dbm_b = bm_b;
    const size_t dc_b = cc_b;
    const size_t hist_b = up(hist_ws_bytes(B, Hq, Lmax));
    if (base && out) {
        char *p = static_cast<char *>(base);
        out->bctr = reinterpret_cast<uint32_t *>(p);
        p += bctr_b;
        out->info = reinterpret_cast<uint32_t *>(p);
        p += info_b;
        out->hinfo = reinterpret_cast<uint32_t *>(p);
        p += hinfo_b;
        out->ccount = reinterpret_cast<uint32_t *>(p);
        p += cc_b;
        out->acount = reinterpret_cast<uint32_t *>(p);
        p += cc_b;
        out->coff = reinterpret_cast<uint32_t *>(p);
        p += cc_b;
        out->thr = reinterpret_cast<uint64_t *>(p);
        p += thr_b;
        out->bitmap = reinterpret_cast<uint32_t *>(p);
        p += bm_b;
        out->cand = reinterpret_cast<uint64_t *>(p);
        p += cand_b;
        out->samp = reinterpret_cast<uint32_t *>(p);
        p += samp_b;
        out->dbm = reinterpret_cast<uint32_t *>(p);
        p += dbm_b;
        out->dcount = reinterpret_cast<uint32_t *>(p);
        p += dc_b;
        out->hist = hist_b ? reinterpret_cast<uint32_t *>(p) : nullptr;
        out->nwords = nwords;
        out->nchunks = nchunks;
    }
    return bctr_b + info_b + hinfo_b + 3 * cc_b + thr_b + bm_b + cand_b + samp_b + dbm_b + dc_b + hist_b;
}

namespace {

tb_status launch_after_thr(const int32_t *ctx, const int32_t *plen, int B, int Hq, int Lmax,
                           int S, int W, int K, int r, bool dilate, bool omit_window,
                           int32_t *idx, int32_t *count, int cap, const SelectWs &ws,
                           hipStream_t st, bool defer_list);
tb_status launch_thr_after(const float *scores, const int32_t *ctx, const int32_t *plen, int B,
                           int Hq, int Lmax, int S, int W, int K, int r, bool dilate,
                           bool omit_window, int32_t *idx, int32_t *count, int cap,
                           const SelectWs &ws, hipStream_t st, bool defer_list);

// classify, threshold, then compaction (or dilation and emission): every
// launch of the selection after the band.
tb_status launch_after_band(const float *scores, const int32_t *ctx, const int32_t *plen, int B,
                            int Hq, int Lmax, int S, int W, int K, int r, bool dilate,
                            bool omit_window, int32_t *idx, int32_t *count, int cap,
                            const SelectWs &ws, hipStream_t st, bool defer_list) {
    const int nseg = B * Hq;
    dim3 grid(ws.nchunks, nseg);
    const int rk = dilate ? 0 : r;
    auto classify = rk == 0 ? classify_kernel<0> : rk == 1 ? classify_kernel<1>
                                             : rk == 2 ? classify_kernel<2> : classify_kernel<-1>;
    hipLaunchKernelGGL(classify, grid, dim3(T1), 0, st, scores, ctx, plen, Hq, Lmax, S, W, K, rk,
                       ws.info, ws.ccount, ws.acount, ws.nchunks, ws.cand, ws.bitmap, ws.nwords);
    const tb_status e = check_launch("tb_select(classify)");
    if (e) return e;
    return launch_thr_after(scores, ctx, plen, B, Hq, Lmax, S, W, K, r, dilate, omit_window, idx,
                            count, cap, ws, st, defer_list);
}

// threshold, then the list.
tb_status launch_thr_after(const float *scores, const int32_t *ctx, const int32_t *plen, int B,
                           int Hq, int Lmax, int S, int W, int K, int r, bool dilate,
                           bool omit_window, int32_t *idx, int32_t *count, int cap,
                           const SelectWs &ws, hipStream_t st, bool defer_list) {
    const int nseg = B * Hq;
    const int rk = dilate ? 0 : r;
    hipLaunchKernelGGL(thr_kernel, dim3(nseg), dim3(T3), 0, st, scores, ctx, plen, Hq, Lmax, S, W,
                       K, rk, omit_window ? 1 : 0, ws.info, ws.ccount, ws.acount, ws.nchunks,
                       ws.cand, ws.bitmap, ws.nwords, ws.thr, ws.coff, count);
    const tb_status e = check_launch("tb_select(threshold)");
    if (e) return e;
    return launch_after_thr(ctx, plen, B, Hq, Lmax, S, W, K, r, dilate, omit_window, idx, count,
                            cap, ws, st, defer_list);
}

// compaction (or dilation and emission) after the threshold: the list.
tb_status launch_after_thr(const int32_t *ctx, const int32_t *plen, int B, int Hq, int Lmax,
                           int S, int W, int K, int r, bool dilate, bool omit_window,
                           int32_t *idx, int32_t *count, int cap, const SelectWs &ws,
                           hipStream_t st, bool defer_list) {
    const int nseg = B * Hq;
    dim3 grid(ws.nchunks, nseg);
    tb_status e;
    if (defer_list) return TB_OK;   // the list is written by tb_select_attn
    if (!dilate) {
        hipLaunchKernelGGL(compact_kernel, grid, dim3(64), 0, st, ctx, plen, Hq, Lmax, S, W, K,
                           omit_window ? 1 : 0, ws.ccount, ws.nchunks, ws.cand, ws.bitmap,
                           ws.nwords, ws.thr, ws.coff, idx, cap);
        return check_launch("tb_select(compact)");
    }
    hipLaunchKernelGGL(dilate_kernel, grid, dim3(64), 0, st, ctx, plen, Hq, Lmax, S, W, K, r,
                       ws.ccount, ws.nchunks, ws.cand, ws.bitmap, ws.nwords, ws.thr, ws.dbm,
                       ws.dcount);
    e = check_launch("tb_select(dilate)");
    if (e) return e;
    hipLaunchKernelGGL(emit_dilated_kernel, grid, dim3(64), 0, st, ctx, plen, Hq, Lmax, S, W, K,
                       omit_window ? 1 : 0, ws.dbm, ws.nwords, ws.dcount, ws.nchunks, idx, count,
                       cap);
    return check_launch("tb_select(emit dilated)");
}

}  // namespace

tb_status launch_select(const float *scores, const int32_t *ctx, const int32_t *plen, int B,
                        int Hq, int Lmax, int S, int W, int K, int r, bool dilate,
                        bool omit_window, int32_t *idx, int32_t *count, int cap,
                        const SelectWs &ws, hipStream_t st, bool defer_list) {
    const int nseg = B * Hq;
    // dilation: the centres are the plain top-K (radius 0), widened afterwards
    const int rk = dilate ? 0 : r;
    auto bounds = rk == 0 ? bounds_kernel<0> : rk == 1 ? bounds_kernel<1>
                                         : rk == 2 ? bounds_kernel<2> : bounds_kernel<-1>;
    hipLaunchKernelGGL(bounds, dim3(BG, nseg), dim3(T3), 0, st, scores, ctx, plen, Hq, Lmax, S, W,
                       K, rk, ws.samp, ws.bctr, ws.info);
    tb_status e = check_launch("tb_select(bounds)");
    if (e) return e;
    return launch_after_band(scores, ctx, plen, B, Hq, Lmax, S, W, K, r, dilate, omit_window, idx,
                             count, cap, ws, st, defer_list);
}

tb_status launch_score_select(const float *qhat, int n_slots, int slot, const void *kp,
                              const int32_t *ctx, const int32_t *plen, float *scores, int B,
                              int Hq, int Hkv, int Lmax, int dp, int S, int W, int K, int r,
                              bool dilate, bool omit_window, int32_t *idx, int32_t *count,
                              int cap, const SelectWs &ws, hipStream_t st, bool defer_list,
                              bool defer_select) {
    if (defer_select && !dilate &&
        defer_select_fits(B, Hq, Hkv, Lmax, r, omit_window ? 0 : W, cap, ws)) {
        // scores, histogram and classification only: tb_select_attn resolves
        // the threshold, writes count and idx, and attends
        return launch_score_hist_select(qhat, n_slots, slot, kp, ctx, plen, scores, B, Hq, Hkv,
                                        Lmax, dp, S, W, K, r, false, omit_window, count, ws, st,
                                        true);
    }
    defer_list = defer_list || defer_select;
    if (hist_route_fits(B * Hq, Lmax, Hq / Hkv, r, dilate) && ws.hist) {
        // scoring with an exact histogram of the pooled keys, then
        // classification against the bin that holds the budget's key
        const tb_status e = launch_score_hist_select(qhat, n_slots, slot, kp, ctx, plen, scores,
                                                     B, Hq, Hkv, Lmax, dp, S, W, K, r, dilate,
                                                     omit_window, count, ws, st);
        if (e) return e;
        return launch_after_thr(ctx, plen, B, Hq, Lmax, S, W, K, r, dilate, omit_window, idx,
                                count, cap, ws, st, defer_list);
    }
    const int rk = dilate ? 0 : r;
    const int g = Hq / Hkv;
    const int nsb = BG * B * Hq;
    // The fused launch saves a launch but its sampling blocks re-read
    // projected-key rows and hold CU slots while they wait on their band; it
    // pays only while they take at most one block slot per CU next to the
    // scoring stream (measured slower with more sampling blocks, and with
    // the 2R + 1 = 5 rows of radius 2, whose registers allow one 1024-thread
    // block per CU).
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        ncu = 0;
    score_bounds_fn fn = nullptr;
    if (nsb <= ncu) {
        if (dp == 16)
            fn = rk == 0 ? score_bounds_pick<16, 0>(g) : rk == 1 ? score_bounds_pick<16, 1>(g) : nullptr;
        else if (dp == 32)
            fn = rk == 0 ? score_bounds_pick<32, 0>(g) : rk == 1 ? score_bounds_pick<32, 1>(g) : nullptr;
    }
    if (!fn) {
        // the scores first, then the selection's own sampling launch
        tb_status e = launch_score(qhat, n_slots, slot, kp, plen, scores, B, Hq, Hkv, Lmax, dp, st);
        if (e) return e;
        return launch_select(scores, ctx, plen, B, Hq, Lmax, S, W, K, r, dilate, omit_window, idx,
                             count, cap, ws, st, defer_list);
    }
    const int nxs = (Lmax + T3 - 1) / T3;
    const long long nblk = (long long)nsb + (long long)nxs * Hkv * B;
    if (nblk > 0x7fffffffLL) {
        set_error("tb_score_select: grid of %lld blocks too large", nblk);
        return TB_ERR_UNSUPPORTED_SHAPE;
    }
    hipLaunchKernelGGL(fn, dim3((unsigned)nblk), dim3(T3), 0, st, qhat, n_slots * Hq * dp,
                       slot * Hq * dp, static_cast<const uint16_t *>(kp), ctx, plen, scores, Hq, Hkv,
                       Lmax, S, W, K, nsb, nxs, ws.samp, ws.bctr, ws.info);
    tb_status e = check_launch("tb_score_select(score + band)");
    if (e) return e;
    return launch_after_band(scores, ctx, plen, B, Hq, Lmax, S, W, K, r, dilate, omit_window, idx,
                             count, cap, ws, st, defer_list);
}

tb_status launch_compact(const int32_t *ctx, const int32_t *plen, int B, int Hq, int Lmax, int S,
                         int W, int K, bool omit_window, int32_t *idx, int cap, const SelectWs &ws,
                         hipStream_t st) {
    hipLaunchKernelGGL(compact_kernel, dim3(ws.nchunks, B * Hq), dim3(64), 0, st, ctx, plen, Hq,
                       Lmax, S, W, K, omit_window ? 1 : 0, ws.ccount, ws.nchunks, ws.cand,
                       ws.bitmap, ws.nwords, ws.thr, ws.coff, idx, cap);
    return check_launch("tb_select(compact)");
}

}  // namespace tb
