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
// Five launches, all integer work:
//   hist     per (segment, 2048-token chunk): pooled keys from LDS-staged
//            scores; 4096-bin LDS histogram of the top 12 key bits (runs of
//            equal bins in neighbouring lanes are added once), merged into a
//            per-segment global histogram with atomics;
//   boundary one workgroup per segment finds the boundary bin once and
//            returns the histogram to zero;
//   classify same grid: tokens above the boundary bin go straight into a
//            selection bitmap (wave ballots); tokens in it are gathered in LDS
//            and written to the chunk's own slots of the candidate list;
//   thr      one 1024-thread workgroup per segment: gathers the chunks'
//            candidates, exact select of the remaining quota among them (10-bit
//            radix passes narrow the boundary group to at most 64 keys, which
//            are ranked directly), then each chunk's offset in the output list;
//   compact  one wave per chunk: bitmap words ORed with the chunk's chosen
//            candidates and the sink / window bits, emitted as ascending
//            positions with coalesced stores.
#include "tb_common.h"

namespace tb {
namespace {

constexpr int HBITS = 12;
constexpr int NBINS = 1 << HBITS;
constexpr int CHUNK = 2048;          // tokens per hist/classify workgroup
constexpr int T1 = 256;              // threads of hist/classify
constexpr int MAXR = 64;
constexpr int T3 = 1024;             // threads of finalize
constexpr int LDS_CAND = 8192;       // candidates held in LDS by finalize
constexpr int RBITS = 10;            // radix digit of the exact select
constexpr int RBINS = 1 << RBITS;
constexpr int GMAX = 64;             // boundary group size ranked directly
constexpr int MAX_CHUNKS = (1 << 24) / CHUNK;   // chunks of the largest Lmax

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

// Inclusive prefix sum over the threads of the block (thread order). s_w
// holds NT / 64 slots. Two barriers; s_w may be reused after return.
template <int NT>
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t *s_w, uint32_t *total) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_w[wave] = x;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t t = s_w[w];
        before += w < wave ? t : 0u;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return before + x;
}

// Boundary of the top `need` among a 4096-bin histogram (bin 4095 highest):
// bin B1 with above(B1) < need <= above(B1) + hist[B1]; need1 = need -
// above(B1). Thread t owns the t-th group of PER bins counted from the top.
// Block-wide; the result lands in *s_bin / *s_need (LDS, left unchanged when
// the histogram holds fewer than `need` entries).
template <int NT>
struct HistSlice {
    static constexpr int PER = NBINS / NT;
    uint32_t v[PER];
    // thread t owns the t-th group of PER bins counted from the top
    __device__ __forceinline__ void load(const uint32_t *hist) {
        const int top = NBINS - ((int)threadIdx.x + 1) * PER;
#pragma unroll
        for (int i = 0; i < PER; ++i) v[i] = hist[top + i];
    }
};

template <int NT>
__device__ void find_boundary(const HistSlice<NT> &hs, int need, int *s_bin, int *s_need,
                              uint32_t *s_w) {
    constexpr int PER = HistSlice<NT>::PER;
    const int top = NBINS - ((int)threadIdx.x + 1) * PER;
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) sum += hs.v[i];
    uint32_t total;
    const uint32_t incl = block_incl_scan<NT>(sum, s_w, &total);
    const uint32_t above = incl - sum;
    if (above < (uint32_t)need && (uint32_t)need <= incl) {
        uint32_t acc = above;
#pragma unroll
        for (int i = PER - 1; i >= 0; --i) {
            if (acc + hs.v[i] >= (uint32_t)need) {
                *s_bin = top + i;
                *s_need = need - (int)acc;
                break;
            }
            acc += hs.v[i];
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
    stage_keys<T1>(sk, s, lo, hi, g.e0, g.e1);
    for (int i = threadIdx.x; i < NBINS; i += T1) lh[i] = 0u;
    __syncthreads();
    const int lane = threadIdx.x & 63;
    for (int base = a + (int)(threadIdx.x & ~63); base < z; base += T1) {
        const int t = base + lane;
        const bool valid = t < z;
        const uint32_t bin = valid ? (uint32_t)(pooled_key(sk, lo, t, g.e0, g.e1, r) >> (64 - HBITS))
                                   : 0xffffffffu;
        // valid lanes are a prefix of the wave; add each run of equal bins once
        const uint32_t prev = __shfl_up(bin, 1);
        const bool start = valid && (lane == 0 || prev != bin);
        const uint64_t edges = __ballot(start || !valid);
        if (start) {
            const uint64_t after = lane == 63 ? 0ull : edges & (~0ull << (lane + 1));
            const int end = after ? __ffsll((long long)after) - 1 : 64;
            atomicAdd(&lh[bin], (uint32_t)(end - lane));
        }
    }
    __syncthreads();
    uint32_t *gh = ghist + (size_t)seg * NBINS;
    for (int i = threadIdx.x; i < NBINS; i += T1)
        if (lh[i]) atomicAdd(&gh[i], lh[i]);
}

// One workgroup per segment: the boundary bin of the complete histogram
// (written to info), then the histogram is returned to zero for the next call.
__global__ __launch_bounds__(T1) void boundary_kernel(const int32_t *__restrict__ ctx,
                                                      const int32_t *__restrict__ plen, int Hq,
                                                      int Lmax, int S, int W, int K,
                                                      uint32_t *__restrict__ ghist,
                                                      int32_t *__restrict__ info) {
    __shared__ uint32_t s_w[T1 / 64];
    __shared__ int s_bin, s_need;
    const int seg = blockIdx.x, b = seg / Hq;
    const Region g = region(ctx, plen, b, Lmax, S, W, K);
    if (g.bad || g.need == 0 || g.need == g.e1 - g.e0) return;
    uint32_t *gh = ghist + (size_t)seg * NBINS;
    HistSlice<T1> hs;
    hs.load(gh);
    if (threadIdx.x == 0) {
        s_bin = NBINS;
        s_need = 0;
    }
    find_boundary<T1>(hs, g.need, &s_bin, &s_need, s_w);
    if (threadIdx.x == 0) {
        info[2 * seg] = s_bin;
        info[2 * seg + 1] = s_need;
    }
    const int top = NBINS - ((int)threadIdx.x + 1) * HistSlice<T1>::PER;
#pragma unroll
    for (int i = 0; i < HistSlice<T1>::PER; ++i) gh[top + i] = 0u;
}

__global__ __launch_bounds__(T1) void classify_kernel(
    const float *__restrict__ scores, const int32_t *__restrict__ ctx,
    const int32_t *__restrict__ plen, int Hq, int Lmax, int S, int W, int K, int r,
    const int32_t *__restrict__ info, uint32_t *__restrict__ ccount,
    uint32_t *__restrict__ acount, int nchunks, uint64_t *__restrict__ cand,
    uint32_t *__restrict__ bitmap, int nwords) {
    __shared__ uint32_t sk[CHUNK + 2 * MAXR];
    __shared__ uint64_t s_cand[CHUNK];
    __shared__ uint32_t s_nc, s_na;
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
    const int lo = a - r, hi = z + r;
    int B1 = NBINS;
    if (threadIdx.x == 0) {
        s_nc = 0;
        s_na = 0;
    }
    if (touch) {
        B1 = info[2 * seg];
        stage_keys<T1>(sk, scores + (size_t)seg * Lmax, lo, hi, g.e0, g.e1);
    }
    __syncthreads();
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
            if (m) atomicAdd(&s_na, (uint32_t)__popcll(m));
        }
        const uint64_t cm = __ballot(isc);
        if (cm) {
            uint32_t off = 0;
            if (lane == 0) off = atomicAdd(&s_nc, (uint32_t)__popcll(cm));
            off = __shfl(off, 0);
            if (isc) s_cand[off + __popcll(cm & ((1ull << lane) - 1ull))] = key;
        }
    }
    __syncthreads();
    const uint32_t nc = s_nc;
    if (threadIdx.x == 0 && (int)blockIdx.x < nchunks) {
        ccount[(size_t)seg * nchunks + blockIdx.x] = nc;
        acount[(size_t)seg * nchunks + blockIdx.x] = s_na;
    }
    // the chunk owns candidate slots [c0, c0 + CHUNK) of its segment
    uint64_t *cl = cand + (size_t)seg * Lmax + c0;
    for (uint32_t i = threadIdx.x; i < nc; i += T1)
        if (c0 + (int)i < Lmax) cl[i] = s_cand[i];
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

// One workgroup per segment: gather the chunks' candidates, find the exact
// threshold key among them, then every chunk's output offset (above-boundary
// tokens + chosen candidates + sink / window positions in the chunk, scanned).
__global__ __launch_bounds__(T3) void thr_kernel(
    const int32_t *__restrict__ ctx, const int32_t *__restrict__ plen, int Hq, int Lmax, int S,
    int W, int K, int omit_window, const int32_t *__restrict__ info,
    const uint32_t *__restrict__ ccount, const uint32_t *__restrict__ acount, int nchunks,
    const uint64_t *__restrict__ cand, uint64_t *__restrict__ thr_out,
    uint32_t *__restrict__ coff, int32_t *__restrict__ count) {
    __shared__ uint64_t s_cand[LDS_CAND];
    __shared__ uint16_t s_cc[LDS_CAND];          // chunk of each LDS candidate
    __shared__ uint32_t s_off[MAX_CHUNKS];
    __shared__ uint32_t s_chosen[MAX_CHUNKS];
    __shared__ uint32_t s_tile[RBINS];
    __shared__ uint64_t s_grp[GMAX];
    __shared__ uint32_t s_w[T3 / 64];
    __shared__ int s_bin, s_need, s_cnt;
    __shared__ uint32_t s_ng;
    __shared__ uint64_t s_thr;

    const int seg = blockIdx.x, b = seg / Hq;
    const int tid = threadIdx.x;
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
    constexpr int PC = MAX_CHUNKS / T3;
    uint32_t cc[PC], ac[PC];
    uint32_t csum = 0;
#pragma unroll
    for (int j = 0; j < PC; ++j) {
        const int c = tid * PC + j;
        const bool in = c < nchunks && g.need > 0;
        cc[j] = in && partial ? ccount[(size_t)seg * nchunks + c] : 0u;
        ac[j] = in ? acount[(size_t)seg * nchunks + c] : 0u;
        csum += cc[j];
        if (c < nchunks) s_chosen[c] = 0u;
    }
    int nc = 0;
    uint64_t thr = ~0ull;   // candidates with key >= thr are chosen (none by default)
    const uint64_t *cl = cand + (size_t)seg * Lmax;
    bool lds = true;
    if (partial) {
        int k = info[2 * seg + 1];
        const int B1 = info[2 * seg];
        uint32_t total;
        uint32_t run = block_incl_scan<T3>(csum, s_w, &total) - csum;
#pragma unroll
        for (int j = 0; j < PC; ++j) {
            const int c = tid * PC + j;
            if (c < nchunks) s_off[c] = run;
            run += cc[j];
        }
        nc = (int)total;
        lds = nc <= LDS_CAND;
        __syncthreads();
        if (lds) {
            constexpr int PER = LDS_CAND / T3;
            uint64_t v[PER];
            int vc[PER];
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                const int i = tid + j * T3;
                vc[j] = 0;
                v[j] = 0ull;
                if (i < nc) {
                    vc[j] = chunk_of(s_off, nchunks, (uint32_t)i);
                    v[j] = cl[(size_t)vc[j] * CHUNK + ((uint32_t)i - s_off[vc[j]])];
                }
            }
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                const int i = tid + j * T3;
                if (i < nc) {
                    s_cand[i] = v[j];
                    s_cc[i] = (uint16_t)vc[j];
                }
            }
            __syncthreads();
        }
        if (k >= nc) {
            thr = 0ull;   // every candidate is chosen
        } else {
            // the k-th largest key (all keys are distinct) among the candidates
            uint64_t prefix = (uint64_t)B1 << (64 - HBITS);
            uint64_t mask = (uint64_t)(NBINS - 1) << (64 - HBITS);
            int grp = nc;
            int shift = 64 - HBITS;
            while (grp > GMAX && shift > 0) {
                const int width = shift < RBITS ? shift : RBITS;
                shift -= width;
                const uint32_t dmask = (1u << width) - 1u;
                // thread t counts digit (RBINS - 1 - t): thread order = descending digit
                s_tile[tid] = 0u;
                __syncthreads();
                for (int i = tid; i < nc; i += T3) {
                    const uint64_t key = lds ? s_cand[i] : cand_at(cl, s_off, nchunks, i);
                    if ((key & mask) == prefix)
                        atomicAdd(&s_tile[RBINS - 1 - (int)((key >> shift) & dmask)], 1u);
                }
                __syncthreads();
                const uint32_t c = s_tile[tid];
                uint32_t tot;
                const uint32_t incl = block_incl_scan<T3>(c, s_w, &tot);
                const uint32_t above = incl - c;
                if (c > 0 && above < (uint32_t)k && (uint32_t)k <= incl) {
                    s_bin = RBINS - 1 - tid;
                    s_need = k - (int)above;
                    s_cnt = (int)c;
                }
                __syncthreads();
                prefix |= (uint64_t)s_bin << shift;
                mask |= (uint64_t)dmask << shift;
                k = s_need;
                grp = s_cnt;
                __syncthreads();
            }
            // rank the (at most GMAX) keys that carry the prefix
            if (tid == 0) s_ng = 0;
            __syncthreads();
            for (int i = tid; i < nc; i += T3) {
                const uint64_t key = lds ? s_cand[i] : cand_at(cl, s_off, nchunks, i);
                if ((key & mask) == prefix) {
                    const uint32_t slot = atomicAdd(&s_ng, 1u);
                    if (slot < (uint32_t)GMAX) s_grp[slot] = key;
                }
            }
            __syncthreads();
            const int ng = s_ng < (uint32_t)GMAX ? (int)s_ng : GMAX;
            if (tid < ng) {
                const uint64_t mine = s_grp[tid];
                int rank = 0;
                for (int j = 0; j < ng; ++j) rank += s_grp[j] > mine ? 1 : 0;
                if (rank == k - 1) s_thr = mine;
            }
            __syncthreads();
            thr = s_thr;
        }
        // chosen candidates per chunk
        for (int i = tid; i < nc; i += T3) {
            const uint64_t key = lds ? s_cand[i] : cand_at(cl, s_off, nchunks, i);
            if (key >= thr)
                atomicAdd(&s_chosen[lds ? (int)s_cc[i] : chunk_of(s_off, nchunks, i)], 1u);
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
    uint32_t total;
    uint32_t run = block_incl_scan<T3>(lsum, s_w, &total) - lsum;
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
    const Region g = region(ctx, plen, b, Lmax, S, W, K);
    const int L = g.L;
    if (g.bad || c * CHUNK >= L) return;
    const int nE = g.e1 - g.e0;
    const bool partial = g.need > 0 && g.need < nE;
    const int w = c * (CHUNK / 32) + lane;
    const int t0 = w << 5;
    const int wlo = omit_window ? L : (L - W > 0 ? L - W : 0);
    const int slo = S < L ? S : L;
    uint32_t bits = (g.need > 0 && w < nwords) ? bitmap[(size_t)seg * nwords + w] : 0u;
    const uint32_t base = coff[(size_t)seg * nchunks + c];
    uint32_t n = 0;
    uint64_t thr = 0;
    if (partial) {
        n = ccount[(size_t)seg * nchunks + c];
        thr = thr_in[seg];
    }
    bits |= bits_below(slo - t0);
    bits |= bits_below(L - t0) & ~bits_below(wlo - t0);
    bits &= bits_below(L - t0);
    s_word[lane] = bits;
    __syncthreads();
    const uint64_t *cl = cand + (size_t)seg * Lmax + (size_t)c * CHUNK;
    for (uint32_t i = lane; i < n; i += 64) {
        const uint64_t key = cl[i];
        if (key >= thr) {
            const int t = key_token(key) - c * CHUNK;
            atomicOr(&s_word[t >> 5], 1u << (t & 31));
        }
    }
    __syncthreads();
    const uint32_t mine = s_word[lane];
    const uint32_t pop = (uint32_t)__popc(mine);
    uint32_t incl = pop;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    const uint32_t first = incl - pop;
    const uint32_t wend = __shfl(incl, 63);
    int32_t *dst = idx + (size_t)seg * cap;
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

}  // namespace

size_t select_ws_layout(int B, int Hq, int Lmax, void *base, SelectWs *out) {
    const size_t nseg = (size_t)B * Hq;
    const int nwords = (Lmax + 31) / 32 + 1;
    const int nchunks = (Lmax + CHUNK - 1) / CHUNK;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t hist_b = up(nseg * NBINS * 4);
    const size_t info_b = up(nseg * 8);
    const size_t cc_b = up(nseg * (size_t)nchunks * 4);
    const size_t thr_b = up(nseg * 8);
    const size_t bm_b = up(nseg * (size_t)nwords * 4);
    const size_t cand_b = up(nseg * (size_t)Lmax * 8);
    if (base && out) {
        char *p = static_cast<char *>(base);
        out->hist = reinterpret_cast<uint32_t *>(p);
        p += hist_b;
        out->info = reinterpret_cast<int32_t *>(p);
        p += info_b;
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
        out->nwords = nwords;
        out->nchunks = nchunks;
    }
    return hist_b + info_b + 3 * cc_b + thr_b + bm_b + cand_b;
}

tb_status launch_select(const float *scores, const int32_t *ctx, const int32_t *plen, int B,
                        int Hq, int Lmax, int S, int W, int K, int r, bool omit_window,
                        int32_t *idx, int32_t *count, int cap, const SelectWs &ws,
                        hipStream_t st) {
    const int nseg = B * Hq;
    dim3 grid(ws.nchunks, nseg);
    hipLaunchKernelGGL(hist_kernel, grid, dim3(T1), 0, st, scores, ctx, plen, Hq, Lmax, S, W, K,
                       r, ws.hist);
    tb_status e = check_launch("tb_select(hist)");
    if (e) return e;
    hipLaunchKernelGGL(boundary_kernel, dim3(nseg), dim3(T1), 0, st, ctx, plen, Hq, Lmax, S, W, K,
                       ws.hist, ws.info);
    e = check_launch("tb_select(boundary)");
    if (e) return e;
    hipLaunchKernelGGL(classify_kernel, grid, dim3(T1), 0, st, scores, ctx, plen, Hq, Lmax, S, W,
                       K, r, ws.info, ws.ccount, ws.acount, ws.nchunks, ws.cand, ws.bitmap,
                       ws.nwords);
    e = check_launch("tb_select(classify)");
    if (e) return e;
    hipLaunchKernelGGL(thr_kernel, dim3(nseg), dim3(T3), 0, st, ctx, plen, Hq, Lmax, S, W, K,
                       omit_window ? 1 : 0, ws.info, ws.ccount, ws.acount, ws.nchunks, ws.cand,
                       ws.thr, ws.coff, count);
    e = check_launch("tb_select(threshold)");
    if (e) return e;
    hipLaunchKernelGGL(compact_kernel, grid, dim3(64), 0, st, ctx, plen, Hq, Lmax, S, W, K,
                       omit_window ? 1 : 0, ws.ccount, ws.nchunks, ws.cand, ws.bitmap, ws.nwords,
                       ws.thr, ws.coff, idx, cap);
    return check_launch("tb_select(compact)");
}

}  // namespace tb
