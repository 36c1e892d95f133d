// The threshold, the list and the attention in one launch: tb_select_attn
// after tb_score_select with TB_SEL_DEFER_SELECT on the histogram route
// ("TokenButler" summary, "Core architecture": selection under a fixed
// budget; "Optimizations": neighbour fetching; "Inference strategy":
// attention over the sink, local-window and important buffers).
//
// The scoring call stops after its classification pass (select_hist.hip):
// every eligible token is classified against the bin B* of the budget's key,
// leaving the bitmap of tokens above B*, per chunk of 2048 tokens the
// candidates (tokens of B*, 64-bit ranking keys) and the counts, the second
// histogram of the candidates' next 12 key bits, and B*, A (tokens above it)
// and C (tokens in it). No workgroup of that launch waits for another.
//
// Most of a head's rows are known at that point: the sink, the window and
// the tokens above B*. Here they are attended by rows-known workgroups (two
// chunks each, one round trip for their bitmap words) from the start, while
// threshold workgroups (four chunks each, dispatched first) read, in one
// round trip, the second histogram, every chunk's counts and the first
// candidate slots of every chunk, find the exact key of the budget's rank
// inside B* (the sub-bin holding it, then the few keys of that sub-bin
// ranked directly), count every chunk's chosen candidates (so each knows its
// chunks' list offsets without waiting for any other workgroup; every one of
// them reaches the same threshold), attend the chosen candidates of their
// chunks and write their chunks' list rows (bitmap words, chosen candidates,
// sink and a share of the window, ascending). Both kinds store partials of
// the head; the last to arrive merges them (log-sum-exp) and clears the
// second histogram, and the threshold workgroups clear shares of the first
// one for the next call. Counts that disagree with the histograms (a
// workspace that was not zero at first use) are reported as an invalid
// segment (count -1, out 0: the threshold workgroups' partials are
// poisoned); the next call is exact again.
#include "attn_impl.h"
#include "select_impl.h"

namespace tb {
namespace {

using namespace sel;

constexpr int NT = kAttnThreads;    // threads per workgroup
constexpr int PFC = 10;             // candidate slots per thread read in the first round trip
constexpr int BPT = HBINS / NT;     // second-histogram bins per thread
// window rows per chunk split at most (window <= CHUNK, at least 5 chunks)
constexpr int kMaxWinShare = 512;
// attention rows per pass: 128 keeps the kernel within 64 VGPRs (four
// workgroups per CU) without spilling
constexpr int kRowsPerPass = 128;
static_assert(BPT == 8 && NT / MAXC == 8 && CHUNK % kAttnCH == 0 && NT * 4 == CHUNK,
              "bookkeeping below");

constexpr int KC = 2;                        // chunks per rows-known workgroup
constexpr int TC = 4;                        // chunks per threshold workgroup
constexpr int KW = KC * (CHUNK / 32);        // their words
constexpr int TW = TC * (CHUNK / 32);
constexpr int KB = KW * 32 / NT;             // bits each thread stages
constexpr int TB = TW * 32 / NT;
static_assert(KW <= NT && TW <= NT && TC * 64 <= NT && 32 % KB == 0 && 32 % TB == 0 && KB >= 4 &&
                  TB >= 4,
              "a word (or a run of its bits) per thread");

struct SplitAttnLds {
    KthLds<NT> k;
    uint32_t word[KW > TW ? KW : TW];    // rows-known: the rows' bits; threshold: chosen bits
    uint32_t wrow[KW > TW ? KW : TW];    // attention row of each word's first bit
    uint32_t lword[TW];                  // threshold: the list's bits
    uint32_t lrow[TW];                   // list row of each word's first bit, within its chunk
    uint32_t crow[TC];                   // attention row of each chunk's first chosen row
    uint32_t ccnt[MAXC], acnt[MAXC], chosen[MAXC], off[MAXC];
    uint32_t m[8];
    int tok[KC * (CHUNK + kMaxWinShare)];   // rows to attend
};

// Rows of the bits of word w (whose bit 0 is token tbase, whose first set bit
// is row `first`) to tok[row]: thread t takes bits [NB (t % (32 / NB)), +NB).
template <int NB>
__device__ __forceinline__ void stage_bits(uint32_t w, uint32_t first, int tbase, int *tok) {
    const int lo = (threadIdx.x % (32 / NB)) * NB;
    uint32_t left = (w >> lo) & (NB == 32 ? ~0u : (1u << NB) - 1u);
    uint32_t p = first + (uint32_t)__popc(w & ((1u << lo) - 1u));
    while (left) {
        tok[p++] = tbase + lo + __builtin_ctz(left);
        left &= left - 1u;
    }
}
// The same for the rows [r0, r0 + n) only, to tok[row - r0].
template <int NB>
__device__ __forceinline__ void stage_bits_range(uint32_t w, uint32_t first, int tbase, int *tok,
                                                 uint32_t r0, uint32_t n) {
    const int lo = (threadIdx.x % (32 / NB)) * NB;
    uint32_t left = (w >> lo) & (NB == 32 ? ~0u : (1u << NB) - 1u);
    uint32_t p = first + (uint32_t)__popc(w & ((1u << lo) - 1u));
    while (left) {
        if (p - r0 < n) tok[p - r0] = tbase + lo + __builtin_ctz(left);
        ++p;
        left &= left - 1u;
    }
}

template <int D>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(8))) void split_attn_kernel(
    const int32_t *__restrict__ ctx, const int32_t *__restrict__ plen, int Hq, int Hkv, int Lmax,
    int S, int W, int K, int omit_window, const uint32_t *__restrict__ hinfo,
    uint32_t *__restrict__ hist, int nseg, const uint32_t *__restrict__ ccount,
    const uint32_t *__restrict__ acount, const uint64_t *__restrict__ cand,
    const uint32_t *__restrict__ bitmap, int nwords, int nchunks, int nK, int nT,
    const uint32_t *__restrict__ coff, uint64_t *__restrict__ thr_out,
    int32_t *__restrict__ count, int32_t *__restrict__ idx, int cap,
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, float scale_log2, int n_items, float *__restrict__ part,
    uint32_t *__restrict__ ctr, float *__restrict__ out) {
    __shared__ __align__(16) SplitAttnLds sh;
    const int nb = gridDim.x, bid = blockIdx.x;
    // XCD-aware order: per (b, KV head) the threshold workgroups of its g
    // query heads (dispatched first: their chain is the longer one), then the
    // rows-known ones, on one XCD
    const int item = (bid & 7) * (nb >> 3) + (bid >> 3);
    if (item >= n_items) return;
    const int g = Hq / Hkv;
    const int per = g * (nT + nK);
    const int grp = item / per;
    int r = item % per;
    const bool thr_role = r < g * nT;
    if (!thr_role) r -= g * nT;
    const int hg = r % g, j = r / g;
    const int kvh = grp % Hkv, b = grp / Hkv;
    const int seg = b * Hq + kvh * g + hg;
    const int nsplit = nK + nT;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint4 *hs = reinterpret_cast<uint4 *>(hist + (size_t)seg * HBINS);
    uint4 *ss = reinterpret_cast<uint4 *>(hist + (size_t)(nseg + seg) * HBINS);

    if (!thr_role) {
        // ---- rows known before the threshold: chunks [c0, c1)
        const int c0 = j * KC, c1 = c0 + KC < nchunks ? c0 + KC : nchunks;
        const int wg = c0 * (CHUNK / 32) + tid;   // this thread's word
        uint32_t bits = 0u;
        if (tid < (c1 - c0) * (CHUNK / 32) && wg < nwords) bits = bitmap[(size_t)seg * nwords + wg];
        const Region gr = region(ctx, plen, b, Lmax, S, W, K);
        const int L = gr.L;
        const int wlo = omit_window ? L : (L - W > 0 ? L - W : 0);
        const int slo = S < L ? S : L;
        const int w0 = wlo > slo ? wlo : slo;
        uint32_t wv = 0u;
        if (!gr.bad && tid < KW) {
            // sink rows and tokens above B* (the pass's words), no window-only rows
            const int t0 = wg << 5;
            wv = gr.need == 0 ? 0u : bits;
            wv |= bits_below(slo - t0);
            wv &= bits_below(w0 - t0);
        }
        if (tid < KW) sh.word[tid] = wv;
        uint32_t tot;
        const uint32_t incl = block_incl_scan<NT>(tid < KW ? (uint32_t)__popc(wv) : 0u, sh.k.w, &tot);
        if (tid < KW) sh.wrow[tid] = incl - (uint32_t)__popc(wv);
        // the chunks' shares of the window rows (the list's last rows)
        const int nW = !gr.bad && L > w0 ? L - w0 : 0;
        const int share = (nW + nchunks - 1) / nchunks;
        const int wa = c0 * share < nW ? c0 * share : nW;
        const int wz = c1 * share < nW ? c1 * share : nW;
        __syncthreads();
        {
            const int wi = tid / (32 / KB);
            stage_bits<KB>(sh.word[wi], sh.wrow[wi], (c0 * (CHUNK / 32) + wi) << 5, sh.tok);
        }
        for (int i = tid; i < wz - wa; i += NT) sh.tok[tot + i] = w0 + wa + i;
        __syncthreads();
        const int nrows = (int)tot + (wz - wa);
        float m, l, acc[8];
        attn_rows<D, kRowsPerPass>(q, kc, vc, Hkv, Lmax, scale_log2, b, kvh, seg, nrows, sh.tok, m,
                                   l, acc);
        if (attn_store_merge<D>(m, l, acc, nsplit, part, ctr, out, seg, j))
            for (int i = tid; i < HBINS / 4; i += NT) ss[i] = make_uint4(0u, 0u, 0u, 0u);
        return;
    }

    // ---- threshold workgroup: chunks [c0, c1)
    const int c0 = j * TC, c1 = c0 + TC < nchunks ? c0 + TC : nchunks;
    const uint64_t *cseg = cand + (size_t)seg * Lmax;
    const int lgc = nchunks <= 1 ? 0 : 32 - __clz(nchunks - 1);
    const int tpc = (NT >> lgc) < 64 ? (NT >> lgc) : 64;
    const int pch = tid / tpc, pln = tid % tpc;
    // the first histogram is read by the classification pass only, which has
    // ended: each threshold workgroup clears its share of it for the next call
    for (int i = j + nT * tid; i < HBINS / 4; i += nT * NT) hs[i] = make_uint4(0u, 0u, 0u, 0u);

    // 1. the one round trip, requested before the lengths arrive
    const uint4 *sq = ss + HBINS / 4 - 2 * (tid + 1);
    const uint4 h0 = sq[1], h1 = sq[0];
    const uint32_t bstar = hinfo[(size_t)seg * 3], A = hinfo[(size_t)seg * 3 + 1],
                   C = hinfo[(size_t)seg * 3 + 2];
    uint32_t cc_l = 0u, ac_l = 0u, bits = 0u;
    if (tid < nchunks) {
        cc_l = ccount[(size_t)seg * nchunks + tid];
        ac_l = acount[(size_t)seg * nchunks + tid];
    }
    uint64_t pv[PFC];
#pragma unroll
    for (int jj = 0; jj < PFC; ++jj) {
        const int slot = pln + tpc * jj;
        pv[jj] = pch < nchunks && pch * CHUNK + slot < Lmax ? cseg[(size_t)pch * CHUNK + slot] : 0ull;
    }
    const int wg = c0 * (CHUNK / 32) + tid;
    if (tid < (c1 - c0) * (CHUNK / 32) && wg < nwords) bits = bitmap[(size_t)seg * nwords + wg];
    const Region gr = region(ctx, plen, b, Lmax, S, W, K);
    const int L = gr.L;
    const int nE = gr.e1 - gr.e0;
    const bool partial = !gr.bad && gr.need > 0 && gr.need < nE;
    const int wlo = omit_window ? L : (L - W > 0 ? L - W : 0);
    const int slo = S < L ? S : L;
    const int w0 = wlo > slo ? wlo : slo;

    if (tid < TW) {
        const int t0 = wg << 5;
        uint32_t wv = 0u;
        if (!gr.bad) {
            wv = gr.need == 0 ? 0u : bits;
            wv |= bits_below(slo - t0);
            wv &= bits_below(w0 - t0);
        }
        sh.lword[tid] = wv;
        sh.word[tid] = 0u;
    }
    if (tid < MAXC) {
        sh.chosen[tid] = 0u;
        sh.ccnt[tid] = 0u;
        sh.acnt[tid] = 0u;
    }
    sh.k.tile[tid] = 0u;   // kth_largest's state, zero on entry
    if (tid == 0) {
        sh.k.ng = 0u;
        sh.m[2] = 0u;   // set: the segment's state is inconsistent
    }
    uint64_t thr = ~0ull;

    if (partial) {
        // 2. the threshold
        if (wave == 0) {
            const uint32_t ccl = lane < nchunks ? (cc_l < (uint32_t)CHUNK ? cc_l : (uint32_t)CHUNK)
                                                : 0u;
            sh.ccnt[lane] = ccl;
            sh.acnt[lane] = lane < nchunks ? ac_l : 0u;
            const uint32_t tc = wave_incl_scan(lane < nchunks ? cc_l : 0u);
            const uint32_t ta = wave_incl_scan(lane < nchunks ? ac_l : 0u);
            if (lane == 63) {
                sh.m[0] = tc;
                sh.m[1] = ta;
            }
        }
        const uint32_t cnt2[BPT] = {h0.w, h0.z, h0.y, h0.x, h1.w, h1.z, h1.y, h1.x};
        uint32_t sum2 = 0u;
#pragma unroll
        for (int jj = 0; jj < BPT; ++jj) sum2 += cnt2[jj];
        uint32_t tot2;
        const uint32_t incl2 = block_incl_scan<NT>(sum2, sh.k.w, &tot2);
        const uint32_t need = (uint32_t)gr.need;
        const bool exact = C > 0u && A < need && need <= A + C && sh.m[0] == C && sh.m[1] == A &&
                           tot2 == C;
        const uint32_t need1 = need - A;
        if (exact) {
            if (need1 == C) {
                thr = (uint64_t)bstar << (32 + HSHIFT);   // the whole bin
            } else {
                uint32_t run = incl2 - sum2;
                if (run < need1 && need1 <= incl2) {
#pragma unroll
                    for (int jj = 0; jj < BPT; ++jj) {
                        if (run < need1 && need1 <= run + cnt2[jj]) {
                            sh.m[4] = (uint32_t)(HBINS - 1 - BPT * tid - jj);
                            sh.m[5] = run;
                            sh.m[6] = cnt2[jj];
                        }
                        run += cnt2[jj];
                    }
                }
                __syncthreads();
                const uint32_t b2 = sh.m[4];
                const int need2 = (int)(need1 - sh.m[5]);
                const int n2 = (int)sh.m[6];
                const uint64_t prefix = ((uint64_t)bstar << (32 + HSHIFT)) | ((uint64_t)b2 << 40);
                const uint64_t mask = ~0ull << 40;
                const uint32_t nmine = pch < nchunks ? sh.ccnt[pch] : 0u;
                auto visit = [&](auto f) {
#pragma unroll
                    for (int jj = 0; jj < PFC; ++jj)
                        if ((uint32_t)(pln + tpc * jj) < nmine) f(pv[jj]);
                    for (uint32_t slot = pln + tpc * PFC;
                         slot < nmine && pch * CHUNK + (int)slot < Lmax; slot += tpc)
                        f(cseg[(size_t)pch * CHUNK + slot]);
                };
                thr = kth_largest<NT>(visit, need2, prefix, mask, 40, n2, sh.k);
            }
            // each chunk's chosen candidates; those of this workgroup's chunks
            // into their words
            const uint32_t nmine = pch < nchunks ? sh.ccnt[pch] : 0u;
            const bool mine = pch >= c0 && pch < c1;
            uint32_t nch = 0u;
            auto take = [&](uint64_t key) {
                if (key >= thr) {
                    ++nch;
                    const int t = key_token(key) - pch * CHUNK;
                    // a candidate's position lies in its chunk after the pass
                    // this call follows; anything else is not written
                    if (mine && (uint32_t)t < (uint32_t)CHUNK) {
                        const int tw = t + (pch - c0) * CHUNK;
                        atomicOr(&sh.word[tw >> 5], 1u << (tw & 31));
                    }
                }
            };
#pragma unroll
            for (int jj = 0; jj < PFC; ++jj)
                if ((uint32_t)(pln + tpc * jj) < nmine) take(pv[jj]);
            for (uint32_t slot = pln + tpc * PFC; slot < nmine && pch * CHUNK + (int)slot < Lmax;
                 slot += tpc)
                take(cseg[(size_t)pch * CHUNK + slot]);
            if (tpc >= 16) {
                nch = row16_sum(nch);
                for (int mm = 16; mm < tpc; mm <<= 1) nch += (uint32_t)__shfl_xor((int)nch, mm);
            } else {
                for (int mm = tpc / 2; mm >= 1; mm >>= 1) nch += (uint32_t)__shfl_xor((int)nch, mm);
            }
            if (pln == 0 && pch < nchunks) sh.chosen[pch] = nch;
        } else {
            // the counts disagree with the histograms (a workspace that was
            // not zero at first use): count -1, no list rows, and a poisoned
            // partial (output 0); the histograms are cleared, so the next
            // call is exact again
            if (tid < TW) sh.lword[tid] = 0u;
            if (tid == 0) sh.m[2] = 1u;
        }
    }
    __syncthreads();

    // 3. chunk offsets of the list, the count; per chunk of this workgroup
    // (one wave each) the list row and the attention row of each word
    if (wave == 0) {
        if (partial) {
            uint32_t v = 0u;
            if (lane < nchunks)
                v = sh.acnt[lane] + sh.chosen[lane] +
                    (uint32_t)fixed_in(lane * CHUNK, (lane + 1) * CHUNK, slo, wlo, L);
            const uint32_t incl = wave_incl_scan(v);
            sh.off[lane] = incl - v;
            if (j == 0 && lane == 63) {
                count[seg] = sh.m[2] ? -1 : (int32_t)incl;
                thr_out[seg] = thr;
            }
        } else {
            // all or none: offsets from the pass
            sh.off[lane] = !gr.bad && lane < nchunks ? coff[(size_t)seg * nchunks + lane] : 0u;
        }
    }
    if (wave < c1 - c0) {
        const int wi = wave * 64 + lane;
        const uint32_t cw = sh.word[wi];
        const uint32_t lw = sh.lword[wi] | cw;
        sh.lword[wi] = lw;
        // list rows (low half) and chosen rows (high half) in one scan
        const uint32_t pk = (uint32_t)__popc(lw) | ((uint32_t)__popc(cw) << 16);
        const uint32_t inc = wave_incl_scan(pk) - pk;
        sh.lrow[wi] = inc & 0xffffu;
        sh.wrow[wi] = inc >> 16;
    }
    // chosen rows of each chunk follow those of the chunks before it
    if (tid == 0) {
        uint32_t run = 0u;
        for (int ci = 0; ci < c1 - c0; ++ci) {
            sh.crow[ci] = run;
            run += sh.chosen[c0 + ci];
        }
        sh.m[3] = run;
    }
    __syncthreads();
    const int ncz = (int)sh.m[3];
    // the chosen rows, as many at a time as the row table holds (all of them
    // unless far more than the budget's share fall in these chunks)
    constexpr int TOKCAP = KC * (CHUNK + kMaxWinShare);
    float m, l, acc[8];
    for (int r0 = 0; r0 == 0 || r0 < ncz; r0 += TOKCAP) {
        const int wi = tid / (32 / TB);
        if (wi < (c1 - c0) * 64)
            stage_bits_range<TB>(sh.word[wi], sh.wrow[wi] + sh.crow[wi >> 6],
                                 (c0 * (CHUNK / 32) + wi) << 5, sh.tok, (uint32_t)r0, TOKCAP);
        __syncthreads();
        const int n = ncz - r0 < TOKCAP ? ncz - r0 : TOKCAP;
        attn_rows<D, kRowsPerPass>(q, kc, vc, Hkv, Lmax, scale_log2, b, kvh, seg, n, sh.tok, m, l,
                                   acc, r0 == 0);
        __syncthreads();   // the table is read before it is staged again
    }
    if (attn_store_merge<D>(m, l, acc, nsplit, part, ctr, out, seg, nK + j, sh.m[2] != 0u))
        for (int i = tid; i < HBINS / 4; i += NT) ss[i] = make_uint4(0u, 0u, 0u, 0u);

    // 4. the chunks' rows to the list (nothing in this launch reads them):
    // the words' rows, then each chunk's share of the window rows (the list's
    // last rows, after the sink and the need: all of the region's, or none)
    {
        const int wi = tid / (32 / TB);
        const int ci = wi >> 6;
        if (ci < c1 - c0) {
            const uint32_t w = sh.lword[wi];
            const int lo = (tid % (32 / TB)) * TB;
            uint32_t left = (w >> lo) & (TB == 32 ? ~0u : (1u << TB) - 1u);
            uint32_t p = sh.off[c0 + ci] + sh.lrow[wi] + (uint32_t)__popc(w & ((1u << lo) - 1u));
            const int tb = ((c0 * (CHUNK / 32) + wi) << 5) + lo;
            while (left) {
                if (p < (uint32_t)cap) idx[(size_t)seg * cap + p] = tb + __builtin_ctz(left);
                ++p;
                left &= left - 1u;
            }
        }
    }
    const int nW = !gr.bad && !sh.m[2] && L > w0 ? L - w0 : 0;
    const int share = (nW + nchunks - 1) / nchunks;
    const int wa = c0 * share < nW ? c0 * share : nW;
    const int wz = c1 * share < nW ? c1 * share : nW;
    const uint32_t woff = (uint32_t)(slo + gr.need + wa);
    for (int i = tid; i < wz - wa; i += NT)
        if (woff + (uint32_t)i < (uint32_t)cap) idx[(size_t)seg * cap + woff + i] = w0 + wa + i;
}

}  // namespace

bool defer_select_fits(int B, int Hq, int Hkv, int Lmax, int r, int win, int cap,
                       const SelectWs &ws) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || !ws.hist || cap < 1) return false;
    const int nchunks = (Lmax + CHUNK - 1) / CHUNK;
    // one split per chunk (the attention workspace holds attn_nsplit(cap)
    // partials per head); each takes at most kMaxWinShare window rows
    const int nsplit = (nchunks + KC - 1) / KC + (nchunks + TC - 1) / TC;
    return hist_route_fits(B * Hq, Lmax, Hq / Hkv, r, false) && nchunks <= MAXC &&
           nsplit <= attn_nsplit(cap) && win >= 0 &&
           (win + nchunks - 1) / nchunks <= kMaxWinShare;
}

tb_status launch_hist_attn(const int32_t *ctx, const int32_t *plen, int B, int Hq, int Hkv,
                           int Lmax, int S, int W, int K, int r, bool omit_window, int32_t *idx,
                           int32_t *count, int cap, const SelectWs &ws, const void *q,
                           const void *kc, const void *vc, int D, float scale, float *out,
                           float *part, uint32_t *ctr, hipStream_t st) {
    if (!defer_select_fits(B, Hq, Hkv, Lmax, r, omit_window ? 0 : W, cap, ws)) {
        set_error("tb_select_attn: the deferred selection does not apply to this shape");
        return TB_ERR_UNSUPPORTED_SHAPE;
    }
    const int nK = (ws.nchunks + KC - 1) / KC, nT = (ws.nchunks + TC - 1) / TC;
    const long long items = (long long)B * Hq * (nK + nT);
    const long long nb = (items + 7) / 8 * 8;
    const float scale_log2 = scale * 1.4426950408889634f;
    auto fn = D == 128 ? split_attn_kernel<128> : split_attn_kernel<64>;
    hipLaunchKernelGGL(fn, dim3((unsigned)nb), dim3(NT), 0, st, ctx, plen, Hq, Hkv, Lmax, S, W, K,
                       omit_window ? 1 : 0, ws.hinfo, ws.hist, B * Hq, ws.ccount, ws.acount,
                       ws.cand, ws.bitmap, ws.nwords, ws.nchunks, nK, nT, ws.coff, ws.thr, count,
                       idx, cap, static_cast<const uint16_t *>(q),
                       static_cast<const uint16_t *>(kc), static_cast<const uint16_t *>(vc),
                       scale_log2, (int)items, part, ctr, out);
    return check_launch("tb_select_attn");
}

}  // namespace tb
