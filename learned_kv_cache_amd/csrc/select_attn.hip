// The list and the attention in one launch: tb_select_attn after a
// selection with TB_SEL_DEFER_LIST ("TokenButler" summary, "Inference
// strategy": attention over the sink, local-window and important buffers;
// "Significance": only the selected tokens' K/V rows are read). Each
// attention workgroup rebuilds, from the selection's state, the list rows it
// attends, writes them to the list and attends over them.
#include "attn_impl.h"
#include "select_impl.h"

namespace tb {
namespace {

using namespace sel;

// Compaction and attention in one launch (tb_select_attn after a selection
// with TB_SEL_DEFER_LIST; the fill mode, at most 64 chunks). Work items and
// their order are those of the attention launch (b, KV head, split, query
// head in group; XCD-aware). The workgroup of a split rebuilds the list rows
// [lo, hi) it attends from the chunks they fall in, exactly as compact_kernel
// emits them (bitmap words, the chunk's chosen candidates, sink and window;
// one wave per chunk), writes those rows to the list and runs the attention
// split on them. Two dependent round trips precede the K/V loads, as in the
// attention launch: the count and chunk offsets, then the chunk's words,
// candidate count and first 128 candidate slots together.
template <int D>
__global__ __launch_bounds__(kAttnThreads) void compact_attn_kernel(
    const int32_t *__restrict__ ctx, const int32_t *__restrict__ plen, int Hq, int Hkv,
    int Lmax, int S, int W, int K, int omit_window, const uint32_t *__restrict__ ccount,
    int nchunks, const uint64_t *__restrict__ cand, const uint32_t *__restrict__ bitmap,
    int nwords, const uint64_t *__restrict__ thr_in, const uint32_t *__restrict__ coff,
    const int32_t *__restrict__ count, int32_t *__restrict__ idx, int cap,
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, float scale_log2, int nsplit, int n_items,
    float *__restrict__ part, uint32_t *__restrict__ ctr, float *__restrict__ out) {
    constexpr int NW = kAttnThreads / 64;
    constexpr int PF = 2;   // candidate slots per lane fetched with the words
    __shared__ int sm_tok[kAttnCH];
    __shared__ uint32_t s_word[NW][64];
    __shared__ uint32_t s_off[64];
    __shared__ int s_c[2];
    const int nb = gridDim.x;
    const int bid = blockIdx.x;
    const int item = (bid & 7) * (nb >> 3) + (bid >> 3);
    if (item >= n_items) return;
    const int g = Hq / Hkv;
    const int hg = item % g;
    int rest = item / g;
    const int split = rest % nsplit;
    rest /= nsplit;
    const int kvh = rest % Hkv;
    const int b = rest / Hkv;
    const int bh = b * Hq + kvh * g + hg;   // also the selection's segment
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

    // first round trip: count, chunk offsets, threshold, lengths
    int n = count[bh];
    const uint32_t off_l =
        (wave == 0 && lane < nchunks) ? coff[(size_t)bh * nchunks + lane] : 0xffffffffu;
    const uint64_t thr_raw = thr_in[bh];
    const Region gr = region(ctx, plen, b, Lmax, S, W, K);
    n = n < 0 ? 0 : (n > cap ? cap : n);
    const int lo = split * kAttnCH;
    const int hi = (lo + kAttnCH < n) ? lo + kAttnCH : n;
    if (wave == 0) {
        // chunks c0..c1 hold rows [lo, hi): offsets are non-decreasing, so
        // the chunks starting at or before lo (before hi) form a prefix
        const uint64_t m0 = __ballot(lane < nchunks && off_l <= (uint32_t)lo);
        const uint64_t m1 = __ballot(lane < nchunks && off_l < (uint32_t)hi);
        if (lane < nchunks) s_off[lane] = off_l;
        if (lane == 0) {
            s_c[0] = m0 ? 63 - __clzll((long long)m0) : 0;
            s_c[1] = m1 ? 63 - __clzll((long long)m1) : 0;
        }
    }
    for (int i = threadIdx.x; i < kAttnCH; i += kAttnThreads) sm_tok[i] = 0;
    __syncthreads();
    if (lo < hi) {
        const int c0 = s_c[0], c1 = s_c[1];
        const int L = gr.L;
        const int nE = gr.e1 - gr.e0;
        const bool partial = gr.need > 0 && gr.need < nE;
        const int wlo = omit_window ? L : (L - W > 0 ? L - W : 0);
        const int slo = S < L ? S : L;
        for (int cb = c0; cb <= c1; cb += NW) {   // the same trip count in every wave
            const int c = cb + wave;
            const bool act = c <= c1 && c * CHUNK < L;
            const int w = c * (CHUNK / 32) + lane;
            const int t0 = w << 5;
            const uint64_t *cl = cand + (size_t)bh * Lmax + (size_t)c * CHUNK;
            // second round trip: the chunk's words, candidate count and
            // first candidate slots, issued together
            uint32_t bits = (act && w < nwords) ? bitmap[(size_t)bh * nwords + w] : 0u;
            uint32_t nraw = act ? ccount[(size_t)bh * nchunks + c] : 0u;
            nraw = nraw < (uint32_t)CHUNK ? nraw : (uint32_t)CHUNK;
            uint64_t pk[PF];
#pragma unroll
            for (int k = 0; k < PF; ++k) {
                const int i = lane + 64 * k;
                pk[k] = (act && c * CHUNK + i < Lmax) ? cl[i] : 0ull;
            }
            uint32_t nc = 0u;
            uint64_t thr = 0;
            if (act) {
                if (gr.need == 0) bits = 0u;
                if (partial) {
                    thr = thr_raw;
                    nc = thr == ~0ull ? 0u : nraw;
                }
                bits |= bits_below(slo - t0);
                bits |= bits_below(L - t0) & ~bits_below(wlo - t0);
                bits &= bits_below(L - t0);
            }
            s_word[wave][lane] = bits;
            __syncthreads();
#pragma unroll
            // a candidate's position lies in its chunk after the selection
            // this call follows; anything else (a state left by another call
            // sequence) is ignored rather than written outside the chunk
            for (int k = 0; k < PF; ++k) {
                if ((uint32_t)(lane + 64 * k) < nc && pk[k] >= thr) {
                    const int t = key_token(pk[k]) - c * CHUNK;
                    if ((uint32_t)t < (uint32_t)CHUNK) atomicOr(&s_word[wave][t >> 5], 1u << (t & 31));
                }
            }
            for (uint32_t i = lane + 64 * PF; i < nc && c * CHUNK + (int)i < Lmax; i += 64) {
                const uint64_t key = cl[i];
                if (key >= thr) {
                    const int t = key_token(key) - c * CHUNK;
                    if ((uint32_t)t < (uint32_t)CHUNK) atomicOr(&s_word[wave][t >> 5], 1u << (t & 31));
                }
            }
            __syncthreads();
            if (act)
                emit_rows(s_word[wave][lane], (c * (CHUNK / 32) + lane) << 5, s_off[c], lo, hi,
                          sm_tok);
            __syncthreads();
        }
        // the rows to the list (coalesced), then clamped to the cache as the
        // attention launch stages them
        for (int i = threadIdx.x; i < hi - lo; i += kAttnThreads) {
            const int t = sm_tok[i];
            idx[(size_t)bh * cap + lo + i] = t;
            sm_tok[i] = t < 0 ? 0 : (t >= Lmax ? Lmax - 1 : t);
        }
        __syncthreads();
    }
    attn_split<D>(q, kc, vc, Hkv, Lmax, scale_log2, nsplit, part, ctr, out, b, kvh, bh, split, lo,
                  hi, sm_tok);
}


}  // namespace

tb_status launch_select_attn(const int32_t *ctx, const int32_t *plen, int B, int Hq, int Hkv,
                             int Lmax, int S, int W, int K, bool omit_window, int32_t *idx,
                             int32_t *count, int cap, const SelectWs &ws, const void *q,
                             const void *kc, const void *vc, int D, float scale, float *out,
                             float *part, uint32_t *ctr, hipStream_t st) {
    if (ws.nchunks > 64) {
        // too many chunks for one wave's offsets: compaction, then attention
        const tb_status e =
            launch_compact(ctx, plen, B, Hq, Lmax, S, W, K, omit_window, idx, cap, ws, st);
        if (e) return e;
        return launch_attn(q, kc, vc, idx, count, cap, nullptr, 0, B, Hq, Hkv, Lmax, D, scale, out,
                           part, ctr, st);
    }
    const int nsplit = attn_nsplit(cap);
    const long long items = (long long)B * Hq * nsplit;
    const long long nb = (items + 7) / 8 * 8;
    if (nb > 0x7fffffff) {
        set_error("tb_select_attn: grid too large");
        return TB_ERR_UNSUPPORTED_SHAPE;
    }
    const float scale_log2 = scale * 1.4426950408889634f;
    const uint16_t *qq = static_cast<const uint16_t *>(q);
    const uint16_t *kk = static_cast<const uint16_t *>(kc);
    const uint16_t *vv = static_cast<const uint16_t *>(vc);
    auto fn = D == 128 ? compact_attn_kernel<128> : compact_attn_kernel<64>;
    hipLaunchKernelGGL(fn, dim3((unsigned)nb), dim3(kAttnThreads), 0, st, ctx, plen, Hq, Hkv, Lmax,
                       S, W, K, omit_window ? 1 : 0, ws.ccount, ws.nchunks, ws.cand, ws.bitmap,
                       ws.nwords, ws.thr, ws.coff, count, idx, cap, qq, kk, vv, scale_log2, nsplit,
                       (int)items, part, ctr, out);
    return check_launch("tb_select_attn");
}

}  // namespace tb
