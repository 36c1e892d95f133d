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
//                   (nonzero bins only);
//   classify_hist   one 256-thread workgroup per (segment, 2048-token chunk):
//                   scans the segment's histogram from the top for the bin B*
//                   that holds the budget's key; that bin is the band of the
//                   sampled-band route, exact instead of estimated: tokens of
//                   higher bins go to the selection bitmap, tokens of bin B*
//                   are the chunk's candidates (64-bit ranking keys).
// The threshold launch of the sampled-band route then selects exactly among
// the candidates (the band always holds the budget's key here) and clears the
// histogram; the compaction, the deferred list of tb_select_attn and the
// dilation mode follow unchanged.
#include "score_impl.h"
#include "select_impl.h"

namespace tb {
namespace {

using namespace sel;

constexpr int HB = 12;                 // bits of the threshold histogram
constexpr int HBINS = 1 << HB;
constexpr int HSHIFT = 32 - HB;        // key32 >> HSHIFT = bin
constexpr int TS = 1024;               // threads (one token each) of score_hist
constexpr int TC = 256;                // threads of classify_hist
constexpr int MAXC = 64;               // chunks of a segment on this route
constexpr int HPT = HBINS / TC;        // histogram bins per classify thread

template <int G, int DP, int R>
__global__ __launch_bounds__(TS, G <= 4 ? 8 : 4) void score_hist_kernel(
    const float *__restrict__ qhat, int q_bstride, int q_off, const uint16_t *__restrict__ kp,
    const int32_t *__restrict__ ctx, const int32_t *__restrict__ plen,
    float *__restrict__ scores, int Hq, int Hkv, int Lmax, int S, int W, int K, int nxs,
    uint32_t *__restrict__ hist) {
    constexpr int V = DP / 8;   // 16-byte vectors per key row
    __shared__ uint32_t s_h[G * HBINS / 2];    // two 16-bit counters per word
    __shared__ float s_sc[G][TS + 2 * R];      // slot j: position t0 - R + j
    const int blk = blockIdx.x;
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
    uint32_t *hs = hist + (size_t)(b * Hq + kvh * G) * HBINS;
    for (int i = tid; i < G * HBINS / 2; i += TS) {
        const uint32_t w = s_h[i];
        if (w == 0u) continue;
        const int gi = i / (HBINS / 2), bin = 2 * (i % (HBINS / 2));
        uint32_t *dst = hs + (size_t)gi * HBINS + bin;
        if (w & 0xffffu)
            __hip_atomic_fetch_add(dst, w & 0xffffu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (w >> 16)
            __hip_atomic_fetch_add(dst + 1, w >> 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// Per (segment, 2048-token chunk), TC threads: the bin B* that holds the
// budget's key, found by scanning the segment's histogram from the top, is
// the band [B* << 20, (B* << 20) | 0xFFFFF] of the sampled-band route (so the
// threshold launch that follows is that route's): tokens of higher bins go
// to the bitmap, tokens of bin B* are the chunk's candidates. The workgroup
// of chunk 0 writes the band.
template <int R>
__global__ __launch_bounds__(TC) void classify_hist_kernel(
    const float *__restrict__ scores, const int32_t *__restrict__ ctx,
    const int32_t *__restrict__ plen, int Hq, int Lmax, int S, int W, int K,
    const uint32_t *__restrict__ hist, uint32_t *__restrict__ info,
    uint32_t *__restrict__ ccount, uint32_t *__restrict__ acount, int nchunks,
    uint64_t *__restrict__ cand, uint32_t *__restrict__ bitmap, int nwords) {
    static_assert(R <= 2, "the staged halo holds radius 2");
    constexpr int NWV = TC / 64;          // waves
    constexpr int WREG = CHUNK / NWV;     // candidate slots per wave
    constexpr int NIT = CHUNK / TC;       // tokens per thread
    __shared__ uint32_t sk[CHUNK + 2 * 2];
    __shared__ uint64_t s_cand[CHUNK];
    __shared__ uint32_t s_w[NWV], s_wc[NWV], s_wa[NWV];
    __shared__ uint32_t s_band[2];
    const int seg = blockIdx.y, b = seg / Hq, c = blockIdx.x;
    const int c0 = c * CHUNK;
    const int lo = c0 - R;   // LDS slot i holds position lo + i
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // the chunk's scores (with halo) and the segment's histogram are loaded
    // before the lengths are known; positions outside E are masked when staged
    constexpr int PER = (CHUNK + 2 * R + TC - 1) / TC;
    const float *sc = scores + (size_t)seg * Lmax;
    float v[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int p = lo + tid + k * TC;
        v[k] = (p >= 0 && p < Lmax && p < c0 + CHUNK + R) ? sc[p] : 0.f;
    }
    // thread tid holds bins [HBINS - HPT (tid + 1), HBINS - HPT tid): thread
    // order is descending bin order
    const uint4 *hp = reinterpret_cast<const uint4 *>(hist + (size_t)seg * HBINS + HBINS -
                                                      HPT * (tid + 1));
    uint4 hv[HPT / 4];
#pragma unroll
    for (int j = 0; j < HPT / 4; ++j) hv[j] = hp[j];
    const Region g = region(ctx, plen, b, Lmax, S, W, K);
    const int nE = g.e1 - g.e0;
    const bool all = !g.bad && g.need == nE && nE > 0;
    const bool partial = !g.bad && g.need > 0 && g.need < nE;
    const int a = c0 > g.e0 ? c0 : g.e0;
    const int z = c0 + CHUNK < g.e1 ? c0 + CHUNK : g.e1;
    const bool touch = partial && a < z;
    if (touch) {
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = tid + k * TC;
            const int p = lo + i;
            if (p < c0 + CHUNK + R) sk[i] = (p >= g.e0 && p < g.e1) ? order_key(v[k]) : 0u;
        }
    }
    if (partial) {
        uint32_t cnt[HPT];
#pragma unroll
        for (int j = 0; j < HPT / 4; ++j) {
            cnt[4 * j] = hv[j].x;
            cnt[4 * j + 1] = hv[j].y;
            cnt[4 * j + 2] = hv[j].z;
            cnt[4 * j + 3] = hv[j].w;
        }
        uint32_t sum = 0;
#pragma unroll
        for (int j = 0; j < HPT; ++j) sum += cnt[j];
        uint32_t tot;
        // s_w is not written again in this kernel
        const uint32_t incl = block_incl_scan<TC, false>(sum, s_w, &tot);
        uint32_t run = incl - sum;
        const uint32_t need = (uint32_t)g.need;
        if (tot < need) {
            // a histogram that does not hold the budget's rank (a workspace
            // that was not zero at first use): the whole key range is the
            // band, which the threshold launch resolves exactly
            if (tid == 0) {
                s_band[0] = 0u;
                s_band[1] = 0xffffffffu;
            }
        } else if (run < need && need <= incl) {
#pragma unroll
            for (int j = HPT - 1; j >= 0; --j) {
                if (run < need && need <= run + cnt[j]) {
                    const uint32_t bin = (uint32_t)(HBINS - HPT * (tid + 1) + j);
                    s_band[0] = bin << HSHIFT;
                    s_band[1] = (bin << HSHIFT) | ((1u << HSHIFT) - 1u);
                }
                run += cnt[j];
            }
        }
    }
    __syncthreads();
    const uint32_t tlo = s_band[0], thi = s_band[1];
    if (partial && c == 0 && tid == 0) {
        info[2 * seg] = tlo;
        info[2 * seg + 1] = thi;
    }
    uint32_t *bm = bitmap + (size_t)seg * nwords;
    uint64_t *wcand = s_cand + wave * WREG;
    uint32_t nc_w = 0, na_w = 0;
    uint64_t keys[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) keys[it] = 0;
    if (touch) {
#pragma unroll
        for (int it = 0; it < NIT; ++it)
            keys[it] = pooled_key_r<R>(sk, lo, c0 + wave * 64 + it * TC + lane);
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int base = c0 + wave * 64 + it * TC;
        const int p = base + lane;
        bool sel = false, isc = false;
        if (p >= g.e0 && p < g.e1 && !g.bad) {
            if (all) {
                sel = true;
            } else if (touch) {
                const uint32_t k32 = (uint32_t)(keys[it] >> 32);
                sel = k32 > thi;
                isc = !sel && k32 >= tlo;
            }
        }
        if (base >= nwords * 32) break;
        const uint64_t m = __ballot(sel);
        if (lane == 0) {
            const int w = base >> 5;
            bm[w] = (uint32_t)m;
            if (w + 1 < nwords) bm[w + 1] = (uint32_t)(m >> 32);
        }
        na_w += (uint32_t)__popcll(m);
        const uint64_t cm = __ballot(isc);
        if (isc) wcand[nc_w + __popcll(cm & ((1ull << lane) - 1ull))] = keys[it];
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
    if (tid == 0) {
        ccount[(size_t)seg * nchunks + c] = nc;
        acount[(size_t)seg * nchunks + c] = na;
    }
    // the chunk owns candidate slots [c0, c0 + CHUNK) of its segment
    uint64_t *cl = cand + (size_t)seg * Lmax + c0;
    for (uint32_t i = lane; i < nc_w; i += 64)
        if (c0 + (int)(before + i) < Lmax) cl[before + i] = wcand[i];
}

}  // namespace

bool hist_route_fits(int Lmax, int g, int r, bool dilate) {
    const int rk = dilate ? 0 : r;
    const int nchunks = (Lmax + CHUNK - 1) / CHUNK;
    // measured: the histogram's flush atomics grow with the context and a
    // group of more than 4 heads leaves one scoring workgroup per CU; beyond
    // 64 chunks or 4 heads per group the sampled band was faster
    return Lmax > kHistMinL && rk <= 2 && nchunks <= MAXC && g <= 4;
}

size_t hist_ws_bytes(int B, int Hq, int Lmax) {
    const int nchunks = (Lmax + CHUNK - 1) / CHUNK;
    return (Lmax > kHistMinL && nchunks <= MAXC) ? (size_t)B * Hq * HBINS * sizeof(uint32_t) : 0;
}

tb_status launch_score_hist_classify(const float *qhat, int n_slots, int slot, const void *kp,
                                     const int32_t *ctx, const int32_t *plen, float *scores,
                                     int B, int Hq, int Hkv, int Lmax, int dp, int S, int W, int K,
                                     int r, bool dilate, const SelectWs &ws, hipStream_t st) {
    const int rk = dilate ? 0 : r;
    const int g = Hq / Hkv;
    score_hist_fn fn = nullptr;
    if (dp == 16)
        fn = rk == 0 ? score_hist_pick<16, 0>(g) : rk == 1 ? score_hist_pick<16, 1>(g)
                                                           : score_hist_pick<16, 2>(g);
    else
        fn = rk == 0 ? score_hist_pick<32, 0>(g) : rk == 1 ? score_hist_pick<32, 1>(g)
                                                           : score_hist_pick<32, 2>(g);
    if (!fn || !ws.hist || rk > 2) {
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
    auto cls = rk == 0 ? classify_hist_kernel<0> : rk == 1 ? classify_hist_kernel<1>
                                                           : classify_hist_kernel<2>;
    hipLaunchKernelGGL(cls, dim3(ws.nchunks, B * Hq), dim3(TC), 0, st, scores, ctx, plen, Hq, Lmax,
                       S, W, K, ws.hist, ws.info, ws.ccount, ws.acount, ws.nchunks, ws.cand,
                       ws.bitmap, ws.nwords);
    return check_launch("tb_score_select(classify)");
}

}  // namespace tb
