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
// Three launches, all integer work:
//   hist     per (segment, 4096-token chunk): pooled keys from LDS-staged
//            scores; 4096-bin LDS histogram of the top 12 key bits, merged
//            into a per-segment global histogram with atomics;
//   classify same grid: find the boundary bin; tokens above it go straight
//            into a selection bitmap (wave ballots), tokens in it are appended
//            to a per-segment candidate list (wave-aggregated atomics);
//   finalize one 1024-thread workgroup per segment: exact radix select of the
//            remaining quota among the candidates (LDS when they fit), then
//            OR sink / window / chosen candidates into 32768-token bitmap
//            tiles and compact them with a block prefix sum into the
//            ascending index list. It also returns the histogram and the
//            candidate counter to zero for the next call.
#include "tb_common.h"

namespace tb {
namespace {

constexpr int HBITS = 12;
constexpr int NBINS = 1 << HBITS;
constexpr int CHUNK = 4096;          // tokens per hist/classify workgroup
constexpr int T1 = 256;              // threads of hist/classify
constexpr int MAXR = 64;
constexpr int T3 = 1024;             // threads of finalize
constexpr int TILE_WORDS = T3;       // bitmap words per compaction tile
constexpr int LDS_CAND = 8192;       // candidates held in LDS by finalize
constexpr int RBITS = 11;            // radix digit of the exact select
constexpr int RBINS = 1 << RBITS;

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
// into LDS; slot i holds position lo + i.
__device__ __forceinline__ void stage_keys(uint32_t *sk, const float *s, int lo, int hi, int e0,
                                           int e1) {
    for (int i = threadIdx.x; i < hi - lo; i += blockDim.x) {
        const int t = lo + i;
        sk[i] = (t >= e0 && t < e1) ? order_key(s[t]) : 0u;
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

// Boundary of the top `need` among a 4096-bin histogram (bin 4095 highest):
// bin B1 with above(B1) < need <= above(B1) + hist[B1]; returns need1 =
// need - above(B1). Block-wide; result in *bin / *need1 (LDS).
template <int NT>
__device__ void find_boundary(const uint32_t *hist, int need, int *s_bin, int *s_need,
                              uint32_t *s_scan) {
    constexpr int PER = NBINS / NT;
    const int tid = threadIdx.x;
    uint32_t local[PER];
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        local[i] = hist[tid * PER + i];
        sum += local[i];
    }
    // inclusive suffix sum over threads: s_scan[tid] = sum of threads >= tid
    s_scan[tid] = sum;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
        const uint32_t v = tid + off < NT ? s_scan[tid + off] : 0u;
        __syncthreads();
        s_scan[tid] += v;
        __syncthreads();
    }
    const uint32_t above = tid + 1 < NT ? s_scan[tid + 1] : 0u;
    if (above < (uint32_t)need && (uint32_t)need <= s_scan[tid]) {
        uint32_t acc = above;
        for (int i = PER - 1; i >= 0; --i) {
            if (acc + local[i] >= (uint32_t)need) {
                *s_bin = tid * PER + i;
                *s_need = need - (int)acc;
                break;
            }
            acc += local[i];
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(T1) void hist_kernel(const float *__restrict__ scores,
                                                  const int32_t *__restrict__ ctx,
                                                  const int32_t *__restrict__ plen, int Hq,
                                                  int Lmax, int S, int W, int K, int r,
                                                  uint32_t *__restrict__ ghist) {
    __shared__ uint32_t sk[CHUNK + 2 * MAXR];
    __shared__ uint32_t lh[NBINS];
    const int seg = blockIdx.y, b = seg / Hq;
    const Region g = region(ctx, plen, b, Lmax, S, W, K);
    if (g.bad || g.need == 0 || g.need == g.e1 - g.e0) return;
    const int c0 = blockIdx.x * CHUNK;
    const int a = c0 > g.e0 ? c0 : g.e0;
    const int z = c0 + CHUNK < g.e1 ? c0 + CHUNK : g.e1;
    if (a >= z) return;
    const int lo = a - r, hi = z + r;
    const float *s = scores + (size_t)seg * Lmax;
    stage_keys(sk, s, lo, hi, g.e0, g.e1);
    for (int i = threadIdx.x; i < NBINS; i += T1) lh[i] = 0u;
    __syncthreads();
    for (int t = a + threadIdx.x; t < z; t += T1) {
        const uint64_t k = pooled_key(sk, lo, t, g.e0, g.e1, r);
        atomicAdd(&lh[(uint32_t)(k >> (64 - HBITS))], 1u);
    }
    __syncthreads();
    uint32_t *gh = ghist + (size_t)seg * NBINS;
    for (int i = threadIdx.x; i < NBINS; i += T1)
        if (lh[i]) atomicAdd(&gh[i], lh[i]);
}

__global__ __launch_bounds__(T1) void classify_kernel(
    const float *__restrict__ scores, const int32_t *__restrict__ ctx,
    const int32_t *__restrict__ plen, int Hq, int Lmax, int S, int W, int K, int r,
    const uint32_t *__restrict__ ghist, uint32_t *__restrict__ ncand,
    uint64_t *__restrict__ cand, uint32_t *__restrict__ bitmap, int nwords) {
    __shared__ uint32_t sk[CHUNK + 2 * MAXR];
    __shared__ uint32_t s_scan[T1];
    __shared__ int s_bin, s_need;
    const int seg = blockIdx.y, b = seg / Hq;
    const Region g = region(ctx, plen, b, Lmax, S, W, K);
    const int c0 = blockIdx.x * CHUNK;
    uint32_t *bm = bitmap + (size_t)seg * nwords;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nE = g.e1 - g.e0;
    const bool all = !g.bad && g.need == nE && nE > 0;
    const bool partial = !g.bad && g.need > 0 && g.need < nE;
    const int a = c0 > g.e0 ? c0 : g.e0;
    const int z = c0 + CHUNK < g.e1 ? c0 + CHUNK : g.e1;
    const bool touch = partial && a < z;
    int B1 = NBINS;
    const int lo = a - r, hi = z + r;
    if (touch) {
        s_bin = NBINS;
        s_need = 0;
        find_boundary<T1>(ghist + (size_t)seg * NBINS, g.need, &s_bin, &s_need, s_scan);
        B1 = s_bin;
        stage_keys(sk, scores + (size_t)seg * Lmax, lo, hi, g.e0, g.e1);
        __syncthreads();
    }
    uint64_t *cl = cand + (size_t)seg * Lmax;
    // every word of this chunk is written: 64 tokens per wave per step
    for (int base = c0 + wave * 64; base < c0 + CHUNK; base += T1) {
        if (base >= nwords * 32) break;
        const int t = base + lane;
        bool sel = false, isc = false;
        uint64_t key = 0;
        if (t >= g.e0 && t < g.e1 && !g.bad) {
            if (all) {
                sel = true;
            } else if (touch) {
                key = pooled_key(sk, lo, t, g.e0, g.e1, r);
                const int bin = (int)(key >> (64 - HBITS));
                sel = bin > B1;
                isc = bin == B1;
            }
        }
        const uint64_t m = __ballot(sel);
        if (lane == 0) {
            const int w = base >> 5;
            bm[w] = (uint32_t)m;
            if (w + 1 < nwords) bm[w + 1] = (uint32_t)(m >> 32);
        }
        const uint64_t cm = __ballot(isc);
        if (cm) {
            uint32_t off = 0;
            if (lane == 0) off = atomicAdd(&ncand[seg], (uint32_t)__popcll(cm));
            off = __shfl(off, 0);
            if (isc) {
                const uint32_t rank = __popcll(cm & ((1ull << lane) - 1ull));
                if (off + rank < (uint32_t)Lmax) cl[off + rank] = key;
            }
        }
    }
}

__device__ __forceinline__ uint32_t block_excl_scan_1024(uint32_t v, uint32_t *s_w,
                                                         uint32_t *total) {
    // wave-level inclusive scan, then across the 16 waves
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_w[wave] = x;
    __syncthreads();
    if (threadIdx.x < 16) {
        uint32_t w = s_w[threadIdx.x];
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            const uint32_t y = __shfl_up(w, off, 16);
            if (threadIdx.x >= off) w += y;
        }
        s_w[16 + threadIdx.x] = w;
    }
    __syncthreads();
    const uint32_t before = wave ? s_w[16 + wave - 1] : 0u;
    *total = s_w[31];
    return before + x - v;
}

__global__ __launch_bounds__(T3) void finalize_kernel(
    const int32_t *__restrict__ ctx, const int32_t *__restrict__ plen, int Hq, int Lmax, int S,
    int W, int K, int omit_window, uint32_t *__restrict__ ghist, uint32_t *__restrict__ ncand,
    const uint64_t *__restrict__ cand, const uint32_t *__restrict__ bitmap, int nwords,
    int32_t *__restrict__ idx, int32_t *__restrict__ count, int cap) {
    __shared__ uint64_t s_cand[LDS_CAND];
    __shared__ uint32_t s_hist[RBINS];
    __shared__ uint32_t s_tile[TILE_WORDS];
    __shared__ uint32_t s_scan[T3];
    __shared__ uint32_t s_w[32];
    __shared__ int s_bin, s_need;
    __shared__ uint64_t s_thr;
    __shared__ int s_found;

    const int seg = blockIdx.x, b = seg / Hq;
    const int tid = threadIdx.x;
    const Region g = region(ctx, plen, b, Lmax, S, W, K);
    if (g.bad) {
        if (tid == 0) count[seg] = -1;
        return;
    }
    const int nE = g.e1 - g.e0;
    const bool partial = g.need > 0 && g.need < nE;
    int nc = 0;
    uint64_t thr = 0;  // candidates with key >= thr are chosen
    const uint64_t *cl = cand + (size_t)seg * Lmax;
    if (partial) {
        s_bin = NBINS;
        s_need = 0;
        find_boundary<T3>(ghist + (size_t)seg * NBINS, g.need, &s_bin, &s_need, s_scan);
        const int need1 = s_need;
        nc = (int)ncand[seg];
        nc = nc < 0 ? 0 : (nc > Lmax ? Lmax : nc);
        const bool lds = nc <= LDS_CAND;
        if (lds)
            for (int i = tid; i < nc; i += T3) s_cand[i] = cl[i];
        __syncthreads();
        if (need1 < nc) {
            // exact select of the need1-th largest key among the candidates
            uint64_t prefix = (uint64_t)s_bin << (64 - HBITS);
            uint64_t mask = (uint64_t)(NBINS - 1) << (64 - HBITS);
            int k = need1;
            int shift = 64 - HBITS;
            bool done = false;
            while (!done && shift > 0) {
                const int width = shift < RBITS ? shift : RBITS;
                shift -= width;
                const uint32_t dmask = (1u << width) - 1u;
                for (int i = tid; i < RBINS; i += T3) s_hist[i] = 0u;
                __syncthreads();
                for (int i = tid; i < nc; i += T3) {
                    const uint64_t key = lds ? s_cand[i] : cl[i];
                    if ((key & mask) == prefix) atomicAdd(&s_hist[(key >> shift) & dmask], 1u);
                }
                __syncthreads();
                if (tid == 0) {
                    uint32_t acc = 0;
                    for (int d = (int)dmask; d >= 0; --d) {
                        if (acc + s_hist[d] >= (uint32_t)k) {
                            s_bin = d;
                            s_need = k - (int)acc;
                            s_found = (int)s_hist[d];
                            break;
                        }
                        acc += s_hist[d];
                    }
                }
                __syncthreads();
                prefix |= (uint64_t)s_bin << shift;
                mask |= (uint64_t)dmask << shift;
                k = s_need;
                if (s_found == 1 && shift > 0) {
                    // a single key carries this prefix: it is the threshold
                    for (int i = tid; i < nc; i += T3) {
                        const uint64_t key = lds ? s_cand[i] : cl[i];
                        if ((key & mask) == prefix) s_thr = key;
                    }
                    __syncthreads();
                    prefix = s_thr;
                    done = true;
                }
                __syncthreads();
            }
            thr = prefix;
        }
        // leave the workspace zero-filled for the next call
        for (int i = tid; i < NBINS; i += T3) ghist[(size_t)seg * NBINS + i] = 0u;
        if (tid == 0) ncand[seg] = 0u;
    }

    // compaction of sink | window | above-boundary bits | chosen candidates
    const int L = g.L;
    const int nw = (L + 31) >> 5;
    const uint32_t *bm = bitmap + (size_t)seg * nwords;
    int32_t *dst = idx + (size_t)seg * cap;
    const bool lds = nc <= LDS_CAND;
    const int wlo = omit_window ? L : (L - W > 0 ? L - W : 0);
    const int slo = S < L ? S : L;
    uint32_t running = 0;
    for (int w0 = 0; w0 < nw; w0 += TILE_WORDS) {
        const int w = w0 + tid;
        uint32_t bits = 0;
        if (w < nw) {
            bits = (g.need > 0) ? bm[w] : 0u;
            const int t0 = w << 5;
            // sink [0, slo) and window [wlo, L) bits of this word
            for (int j = 0; j < 32; ++j) {
                const int t = t0 + j;
                if (t < L && (t < slo || t >= wlo)) bits |= 1u << j;
            }
            if (t0 + 32 > L) bits &= (L - t0 >= 32) ? ~0u : ((1u << (L - t0)) - 1u);
        }
        s_tile[tid] = bits;
        __syncthreads();
        if (partial) {
            const int tlo = w0 << 5, thi = (w0 + TILE_WORDS) << 5;
            for (int i = tid; i < nc; i += T3) {
                const uint64_t key = lds ? s_cand[i] : cl[i];
                if (key >= thr) {
                    const int t = key_token(key);
                    if (t >= tlo && t < thi) atomicOr(&s_tile[(t - tlo) >> 5], 1u << (t & 31));
                }
            }
            __syncthreads();
        }
        const uint32_t mine = s_tile[tid];
        uint32_t total;
        const uint32_t off = block_excl_scan_1024((uint32_t)__popc(mine), s_w, &total);
        uint32_t pos = running + off;
        uint32_t v = mine;
        while (v) {
            const int j = __ffs(v) - 1;
            v &= v - 1;
            if (pos < (uint32_t)cap) dst[pos] = ((w0 + tid) << 5) + j;
            ++pos;
        }
        running += total;
        __syncthreads();
    }
    if (tid == 0) count[seg] = (int32_t)running;
}

}  // namespace

size_t select_ws_layout(int B, int Hq, int Lmax, void *base, SelectWs *out) {
    const size_t nseg = (size_t)B * Hq;
    const int nwords = (Lmax + 31) / 32 + 1;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t hist_b = up(nseg * NBINS * 4);
    const size_t nc_b = up(nseg * 4);
    const size_t bm_b = up(nseg * (size_t)nwords * 4);
    const size_t cand_b = up(nseg * (size_t)Lmax * 8);
    if (base && out) {
        char *p = static_cast<char *>(base);
        out->hist = reinterpret_cast<uint32_t *>(p);
        out->ncand = reinterpret_cast<uint32_t *>(p + hist_b);
        out->bitmap = reinterpret_cast<uint32_t *>(p + hist_b + nc_b);
        out->cand = reinterpret_cast<uint64_t *>(p + hist_b + nc_b + bm_b);
        out->nwords = nwords;
    }
    return hist_b + nc_b + bm_b + cand_b;
}

tb_status launch_select(const float *scores, const int32_t *ctx, const int32_t *plen, int B,
                        int Hq, int Lmax, int S, int W, int K, int r, bool omit_window,
                        int32_t *idx, int32_t *count, int cap, const SelectWs &ws,
                        hipStream_t st) {
    const int nseg = B * Hq;
    dim3 grid((Lmax + CHUNK - 1) / CHUNK, nseg);
    hipLaunchKernelGGL(hist_kernel, grid, dim3(T1), 0, st, scores, ctx, plen, Hq, Lmax, S, W, K,
                       r, ws.hist);
    tb_status e = check_launch("tb_select(hist)");
    if (e) return e;
    hipLaunchKernelGGL(classify_kernel, grid, dim3(T1), 0, st, scores, ctx, plen, Hq, Lmax, S, W,
                       K, r, ws.hist, ws.ncand, ws.cand, ws.bitmap, ws.nwords);
    e = check_launch("tb_select(classify)");
    if (e) return e;
    hipLaunchKernelGGL(finalize_kernel, dim3(nseg), dim3(T3), 0, st, ctx, plen, Hq, Lmax, S, W, K,
                       omit_window ? 1 : 0, ws.hist, ws.ncand, ws.cand, ws.bitmap, ws.nwords, idx, count, cap);
    return check_launch("tb_select(finalize)");
}

}  // namespace tb
