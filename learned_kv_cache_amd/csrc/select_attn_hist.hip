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
// Here one workgroup per (b, KV head, chunk, query head in group) -- the
// chunk is its attention split -- reads, in one round trip, the second
// histogram, every chunk's counts, the first candidate slots of every chunk
// and its own chunk's bitmap words. From these it finds the exact key of the
// budget's rank inside B* (the sub-bin holding it, then the few keys of that
// sub-bin ranked directly) and counts every chunk's chosen candidates, so it
// knows the list offset of its chunk without waiting for any other
// workgroup; every workgroup of the segment reaches the same threshold. It
// attends over its chunk's rows (bitmap words, chosen candidates, sink and a
// share of the window, ascending), 128 rows per pass, and writes them to the
// list; the last split of the head to arrive merges the partials and clears
// the second histogram, and every workgroup clears a share of the first one
// for the next call. Counts that disagree with the histograms (a
// workspace that was not zero at first use) are reported as an invalid
// segment (count -1, out 0); the next call is exact again.
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

struct HistAttnLds {
    KthLds<NT> k;
    uint32_t word[CHUNK / 32];      // the chunk's row bits
    uint32_t wrow[CHUNK / 32];      // list row of each word's first bit, within the chunk
    uint32_t ccnt[MAXC], acnt[MAXC], chosen[MAXC], off[MAXC];
    uint32_t m[8];
    int tok[CHUNK + kMaxWinShare];  // the chunk's rows, then its share of the window
};

template <int D>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(8))) void hist_attn_kernel(
    const int32_t *__restrict__ ctx, const int32_t *__restrict__ plen, int Hq, int Hkv, int Lmax,
    int S, int W, int K, int omit_window, const uint32_t *__restrict__ hinfo, uint32_t *__restrict__ hist, int nseg,
    const uint32_t *__restrict__ ccount, const uint32_t *__restrict__ acount,
    const uint64_t *__restrict__ cand, const uint32_t *__restrict__ bitmap, int nwords,
    int nchunks, const uint32_t *__restrict__ coff, uint64_t *__restrict__ thr_out,
    int32_t *__restrict__ count, int32_t *__restrict__ idx, int cap,
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, float scale_log2, int n_items, float *__restrict__ part,
    uint32_t *__restrict__ ctr, float *__restrict__ out) {
    __shared__ __align__(16) HistAttnLds sh;
    const int nb = gridDim.x, bid = blockIdx.x;
    // work items in the attention launch's XCD-aware order: the query heads
    // of a group, then the chunks, of one (b, KV head) on one XCD
    const int item = (bid & 7) * (nb >> 3) + (bid >> 3);
    if (item >= n_items) return;
    const int g = Hq / Hkv;
    const int hg = item % g;
    int rest = item / g;
    const int c = rest % nchunks;
    rest /= nchunks;
    const int kvh = rest % Hkv;
    const int b = rest / Hkv;
    const int seg = b * Hq + kvh * g + hg;   // the selection's segment, the attention's head
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint4 *hs = reinterpret_cast<uint4 *>(hist + (size_t)seg * HBINS);
    uint4 *ss = reinterpret_cast<uint4 *>(hist + (size_t)(nseg + seg) * HBINS);
    const uint64_t *cseg = cand + (size_t)seg * Lmax;
    // candidate bookkeeping: tpc adjacent threads per chunk (512 over the
    // chunk count rounded up to a power of two, at most a wave), thread pln
    // of chunk pch holding slots pln + tpc j
    const int lgc = nchunks <= 1 ? 0 : 32 - __clz(nchunks - 1);
    const int tpc = (NT >> lgc) < 64 ? (NT >> lgc) : 64;
    const int pch = tid / tpc, pln = tid % tpc;

    // 1. the one round trip, requested before the lengths arrive: every
    // address lies in the workspace whatever they are, and what a segment's
    // lengths make unused is ignored below
    // bins 4095 - 8 tid - j, j < 8: descending thread order
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
    for (int j = 0; j < PFC; ++j) {
        const int slot = pln + tpc * j;
        pv[j] = pch < nchunks && pch * CHUNK + slot < Lmax ? cseg[(size_t)pch * CHUNK + slot] : 0ull;
    }
    if (wave == 0) {
        const int w = c * (CHUNK / 32) + lane;
        bits = w < nwords ? bitmap[(size_t)seg * nwords + w] : 0u;
    }
    // the first histogram is read by the classification pass only, which has
    // ended: each workgroup clears its share of it for the next call
    for (int i = c + nchunks * tid; i < HBINS / 4; i += nchunks * NT) hs[i] = make_uint4(0u, 0u, 0u, 0u);
    const Region gr = region(ctx, plen, b, Lmax, S, W, K);
    const int L = gr.L;
    const int nE = gr.e1 - gr.e0;
    const bool partial = !gr.bad && gr.need > 0 && gr.need < nE;
    const int wlo = omit_window ? L : (L - W > 0 ? L - W : 0);
    const int slo = S < L ? S : L;
    // window-only rows [w0, L) (rows below slo are sink rows) are the list's
    // last rows; they are shared out evenly over the segment's chunk splits
    // (the window's own chunk would otherwise hold about twice the rows)
    const int w0 = wlo > slo ? wlo : slo;

    // the chunk's sink rows and its tokens above B* (no window-only rows:
    // the eligible region ends below the window)
    if (wave == 0) {
        const int t0 = (c * (CHUNK / 32) + lane) << 5;
        uint32_t wv = 0u;
        if (!gr.bad) {
            wv = gr.need == 0 ? 0u : bits;
            wv |= bits_below(slo - t0);
            wv &= bits_below(w0 - t0);
        }
        sh.word[lane] = wv;
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
        // 2. the threshold, as the selection's last workgroup finds it
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
        for (int j = 0; j < BPT; ++j) sum2 += cnt2[j];
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
                    for (int j = 0; j < BPT; ++j) {
                        if (run < need1 && need1 <= run + cnt2[j]) {
                            sh.m[4] = (uint32_t)(HBINS - 1 - BPT * tid - j);
                            sh.m[5] = run;
                            sh.m[6] = cnt2[j];
                        }
                        run += cnt2[j];
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
                    for (int j = 0; j < PFC; ++j)
                        if ((uint32_t)(pln + tpc * j) < nmine) f(pv[j]);
                    for (uint32_t slot = pln + tpc * PFC;
                         slot < nmine && pch * CHUNK + (int)slot < Lmax; slot += tpc)
                        f(cseg[(size_t)pch * CHUNK + slot]);
                };
                thr = kth_largest<NT>(visit, need2, prefix, mask, 40, n2, sh.k);
            }
            // each chunk's chosen candidates; this chunk's into its words
            const uint32_t nmine = pch < nchunks ? sh.ccnt[pch] : 0u;
            uint32_t nch = 0u;
            auto take = [&](uint64_t key) {
                if (key >= thr) {
                    ++nch;
                    const int t = key_token(key) - c * CHUNK;
                    // a candidate's position lies in its chunk after the pass
                    // this call follows; anything else is not written
                    if (pch == c && (uint32_t)t < (uint32_t)CHUNK)
                        atomicOr(&sh.word[t >> 5], 1u << (t & 31));
                }
            };
#pragma unroll
            for (int j = 0; j < PFC; ++j)
                if ((uint32_t)(pln + tpc * j) < nmine) take(pv[j]);
            for (uint32_t slot = pln + tpc * PFC; slot < nmine && pch * CHUNK + (int)slot < Lmax;
                 slot += tpc)
                take(cseg[(size_t)pch * CHUNK + slot]);
            // the tpc threads of a chunk are adjacent lanes (rows of 16 lanes
            // summed by DPP)
            if (tpc >= 16) {
                nch = row16_sum(nch);
                for (int mm = 16; mm < tpc; mm <<= 1) nch += (uint32_t)__shfl_xor((int)nch, mm);
            } else {
                for (int mm = tpc / 2; mm >= 1; mm >>= 1) nch += (uint32_t)__shfl_xor((int)nch, mm);
            }
            if (pln == 0 && pch < nchunks) sh.chosen[pch] = nch;
        } else {
            // the counts disagree with the histograms (a workspace that was
            // not zero at first use): the segment is reported as invalid,
            // count -1 and no rows; the histograms are cleared below, so the
            // next call is exact again
            if (wave == 0) sh.word[lane] = 0u;
            if (tid == 0) sh.m[2] = 1u;
        }
    }
    __syncthreads();

    // 3. chunk offsets of the list; the count; the list row of each word's
    // first bit
    if (wave == 0) {
        if (partial) {
            uint32_t v = 0u;
            if (lane < nchunks)
                v = sh.acnt[lane] + sh.chosen[lane] +
                    (uint32_t)fixed_in(lane * CHUNK, (lane + 1) * CHUNK, slo, wlo, L);
            const uint32_t incl = wave_incl_scan(v);
            sh.off[lane] = incl - v;
            if (c == 0 && lane == 63) {
                count[seg] = sh.m[2] ? -1 : (int32_t)incl;
                thr_out[seg] = thr;
            }
        } else {
            // all or none: offsets from the pass
            sh.off[lane] = !gr.bad && lane < nchunks ? coff[(size_t)seg * nchunks + lane] : 0u;
        }
        const uint32_t pop = (uint32_t)__popc(sh.word[lane]);
        const uint32_t incl = wave_incl_scan(pop);
        sh.wrow[lane] = incl - pop;
        if (lane == 63) sh.m[3] = incl;
    }
    __syncthreads();
    // this chunk's share of the window rows: they follow the sink and the
    // important rows (need of them: the budget, all of the region, or none)
    const int nW = !gr.bad && !sh.m[2] && L > w0 ? L - w0 : 0;
    const int share = (nW + nchunks - 1) / nchunks;
    const int ws0 = c * share < nW ? c * share : nW;
    const int nwin = ws0 + share < nW ? share : nW - ws0;
    const int nch = (int)sh.m[3];
    const int nrows = nch + nwin;
    const uint32_t off = sh.off[c];
    const uint32_t woff = (uint32_t)(slo + gr.need + ws0);
    {
        // the chunk's rows, ascending, to the row table: every thread takes
        // four bits of one word (a wave alone would walk up to 32 bits per
        // lane while the CU's other workgroups attend). Every row lies in
        // [0, L), so the table holds the list's values.
        const int wi = tid >> 3, nib = (tid & 7) * 4;
        const uint32_t word = sh.word[wi];
        uint32_t left = (word >> nib) & 15u;
        uint32_t p = sh.wrow[wi] + (uint32_t)__popc(word & ((1u << nib) - 1u));
        const int tb = ((c * (CHUNK / 32) + wi) << 5) + nib;
        while (left) {
            sh.tok[p++] = tb + __builtin_ctz(left);
            left &= left - 1u;
        }
    }
    for (int i = tid; i < nwin; i += NT) sh.tok[nch + i] = w0 + ws0 + i;
    __syncthreads();

    // 4. attention over the chunk's rows; the last split of the head merges
    float m, l, acc[8];
    attn_rows<D, kRowsPerPass>(q, kc, vc, Hkv, Lmax, scale_log2, b, kvh, seg, nrows, sh.tok, m, l,
                               acc);
    if (attn_store_merge<D>(m, l, acc, nchunks, part, ctr, out, seg, c)) {
        // every workgroup of the segment has read the second histogram
        for (int i = tid; i < HBINS / 4; i += NT) ss[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    // the chunk's rows to the list only now: stores issued while the CU's
    // other workgroups stream K/V wait for the memory pipeline (and the
    // partial's stores above wait for every earlier store), and nothing in
    // this launch reads them
    for (int i = tid; i < nrows; i += NT) {
        const uint32_t pos = i < nch ? off + (uint32_t)i : woff + (uint32_t)(i - nch);
        if (pos < (uint32_t)cap) idx[(size_t)seg * cap + pos] = sh.tok[i];
    }
}

}  // namespace

bool defer_select_fits(int B, int Hq, int Hkv, int Lmax, int r, int win, int cap,
                       const SelectWs &ws) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || !ws.hist || cap < 1) return false;
    const int nchunks = (Lmax + CHUNK - 1) / CHUNK;
    // one split per chunk (the attention workspace holds attn_nsplit(cap)
    // partials per head); each takes at most kMaxWinShare window rows
    return hist_route_fits(B * Hq, Lmax, Hq / Hkv, r, false) && nchunks <= MAXC &&
           nchunks <= attn_nsplit(cap) && win >= 0 &&
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
    const long long items = (long long)B * Hq * ws.nchunks;
    const long long nb = (items + 7) / 8 * 8;
    const float scale_log2 = scale * 1.4426950408889634f;
    auto fn = D == 128 ? hist_attn_kernel<128> : hist_attn_kernel<64>;
    hipLaunchKernelGGL(fn, dim3((unsigned)nb), dim3(NT), 0, st, ctx, plen, Hq, Hkv, Lmax, S, W, K,
                       omit_window ? 1 : 0, ws.hinfo, ws.hist, B * Hq, ws.ccount,
                       ws.acount, ws.cand, ws.bitmap, ws.nwords, ws.nchunks, ws.coff, ws.thr,
                       count, idx, cap, static_cast<const uint16_t *>(q),
                       static_cast<const uint16_t *>(kc), static_cast<const uint16_t *>(vc),
                       scale_log2, (int)items, part, ctr, out);
    return check_launch("tb_select_attn");
}

}  // namespace tb
