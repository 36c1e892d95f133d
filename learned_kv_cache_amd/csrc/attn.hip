// Sparse decode attention over the selected positions of the retained KV
// cache ("TokenButler" summary, "Significance": keep the whole cache, read
// only the most relevant tokens).
//
// Split-K gather: a 512-thread workgroup owns CH consecutive entries of one
// query head's ascending index list, staged in LDS. D/8 lanes share one K/V
// row (16 bytes = 8 channels per lane), so a wave gathers 64/(D/8) rows per
// 16-byte load; each lane group requests all of its K rows at once, then all
// of its V rows once the logits are formed. Logits are reduced with DPP, the
// softmax is fp32 base-2 in registers, the row groups' states are combined by
// a lane butterfly and then across waves, and the workgroup writes one partial
// (max, sum, o[D]). The last workgroup of a head to arrive merges the partials
// by log-sum-exp into the fp32 output, with the same butterfly.
//
// Cross-workgroup handoff without device-scope fences (on this chip a fence at
// agent scope writes back, and on acquire invalidates, the XCD's whole L2):
// wave 0 alone writes the partial with agent-scope atomic stores (coherent
// across XCDs by themselves), waits for them to complete, then increments an
// agent-scope arrival counter; the workgroup that sees the last arrival reads
// every partial with agent-scope atomic loads and resets the counter.
//
// Launch order is XCD-aware: dispatch sends workgroup i to XCD i % 8, and the
// block index is decoded so that each XCD receives a contiguous run of work
// items ordered (b, kv head, split, query head in group). The g query heads of
// one KV group that read the same part of the cache run next to each other on
// the same XCD and share its L2.
#include "attn_impl.h"
#include "project_impl.h"

namespace tb {
namespace {

constexpr int kThreads = kAttnThreads;
constexpr int CH = kAttnCH;

template <int D>
__global__ __launch_bounds__(kThreads) void attn_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ count, int cap, const int32_t *__restrict__ ctx, int window,
    int Hq, int Hkv, int Lmax, float scale_log2,
    int nsplit, int n_items, float *__restrict__ part, uint32_t *__restrict__ ctr,
    float *__restrict__ out) {
    __shared__ int sm_tok[CH];

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
    const int h = kvh * g + hg;
    const int bh = b * Hq + h;

    int n = count[bh];
    n = n < 0 ? 0 : (n > cap ? cap : n);
    const int32_t *ib = idx + (size_t)bh * cap;
    // rows [0, n) come from the list, rows [n, n + nwin) are the window
    int nwin = 0, wstart = 0;
    if (ctx != nullptr && window > 0) {
        int Lb = ctx[b];
        Lb = Lb < 0 ? 0 : (Lb > Lmax ? Lmax : Lb);
        const int last = n > 0 ? ib[n - 1] : -1;
        wstart = Lb - window > last + 1 ? Lb - window : last + 1;
        wstart = wstart < 0 ? 0 : wstart;
        nwin = Lb > wstart ? Lb - wstart : 0;
    }
    const int total = n + nwin;
    const int lo = split * CH;
    const int hi = (lo + CH < total) ? lo + CH : total;
    // this workgroup's positions, clamped to the cache
    for (int i = threadIdx.x; i < CH; i += kThreads) {
        const int r = lo + i;
        int t = r < hi ? (r < n ? ib[r] : wstart + (r - n)) : 0;
        sm_tok[i] = t < 0 ? 0 : (t >= Lmax ? Lmax - 1 : t);
    }
    __syncthreads();

    attn_split<D>(q, kc, vc, Hkv, Lmax, scale_log2, nsplit, part, ctr, out, b, kvh, bh, split, lo,
                  hi, sm_tok);
}

// The last of sequence b's Hq head merges and its append block to arrive
// advances the lengths in place (every workgroup of the launch has read them
// by then) and clears the counter for the next call.
__device__ __forceinline__ void arrive_lengths(uint32_t *bctr, int32_t *ctx, int32_t *plen, int b,
                                               int Hq, int L, int P, int Lmax, int n_p) {
    const uint32_t prev =
        __hip_atomic_fetch_add(bctr + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev != (uint32_t)Hq) return;
    if (append_applies(L, P, Lmax)) {
        ctx[b] = L + 1;
        if (L + 1 - P >= n_p) plen[b] = L + 1;
    }
    __hip_atomic_store(bctr + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The decode step's append and attention in one launch (tb_append_attn).
// The first nbA blocks (B rounded up to 8) append sequence b's new K/V rows
// and project its pending keys as tb_append_kv does (append_rows); the others
// are attn_kernel's work items over the lengths the append leaves (L + 1
// where it applies). The workgroup whose split holds position L, the
// window's last row, writes the new rows of its KV head to the cache itself
// (the bytes the append block writes) and waits for its stores before its
// rows are read, so no workgroup waits for another.
template <int D, int DP>
__global__ __launch_bounds__(kThreads) void append_attn_kernel(
    const uint16_t *__restrict__ k_new, const uint16_t *__restrict__ v_new,
    uint16_t *__restrict__ kc, uint16_t *__restrict__ vc, uint16_t *__restrict__ kp,
    const uint16_t *__restrict__ wk, int32_t *__restrict__ ctx, int32_t *__restrict__ plen,
    int n_p, const uint16_t *__restrict__ q, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ count, int cap, int window, int B, int Hq, int Hkv, int Lmax,
    float scale_log2, int nsplit, int n_items, int nbA, float *__restrict__ part,
    uint32_t *__restrict__ ctr, uint32_t *__restrict__ bctr, float *__restrict__ out) {
    __shared__ int sm_tok[CH];
    const int bid = blockIdx.x;
    if (bid < nbA) {
        const int b = bid;
        if (b >= B) return;
        const int L = ctx[b], P = plen[b];
        if (append_applies(L, P, Lmax))
            append_rows<D, DP, kThreads>(k_new, v_new, kc, vc, kp, wk, b, L, P, Hkv, Lmax, n_p);
        if (threadIdx.x == 0) arrive_lengths(bctr, ctx, plen, b, Hq, L, P, Lmax, n_p);
        return;
    }
    const int nb = gridDim.x - nbA, lb = bid - nbA;
    const int item = (lb & 7) * (nb >> 3) + (lb >> 3);
    if (item >= n_items) return;
    const int g = Hq / Hkv;
    const int hg = item % g;
    int rest = item / g;
    const int split = rest % nsplit;
    rest /= nsplit;
    const int kvh = rest % Hkv;
    const int b = rest / Hkv;
    const int h = kvh * g + hg;
    const int bh = b * Hq + h;

    int n = count[bh];
    n = n < 0 ? 0 : (n > cap ? cap : n);
    const int32_t *ib = idx + (size_t)bh * cap;
    const int L = ctx[b], P = plen[b];
    const bool app = append_applies(L, P, Lmax);
    // rows [0, n) come from the list, rows [n, n + nwin) are the window,
    // which ends at the length the append leaves
    int nwin = 0, wstart = 0;
    if (window > 0) {
        int Lb = app ? L + 1 : L;
        Lb = Lb < 0 ? 0 : (Lb > Lmax ? Lmax : Lb);
        const int last = n > 0 ? ib[n - 1] : -1;
        wstart = Lb - window > last + 1 ? Lb - window : last + 1;
        wstart = wstart < 0 ? 0 : wstart;
        nwin = Lb > wstart ? Lb - wstart : 0;
    }
    const int total = n + nwin;
    const int lo = split * CH;
    const int hi = (lo + CH < total) ? lo + CH : total;
    const bool mine = app && nwin > 0 && n + (L - wstart) >= lo && n + (L - wstart) < hi;
    if (mine) {
        // position L is this split's: its new K and V rows to the cache,
        // complete (waited for below, after the list reads) before any of
        // the split's rows is read
        constexpr int R16 = D / 8;
        const size_t head = (size_t)b * Hkv + kvh;
        for (int i = threadIdx.x; i < 2 * R16; i += kThreads) {
            const int which = i / R16, v = i % R16;
            reinterpret_cast<uint4 *>((which ? vc : kc) + (head * Lmax + L) * D)[v] =
                reinterpret_cast<const uint4 *>((which ? v_new : k_new) + head * D)[v];
        }
    }
    for (int i = threadIdx.x; i < CH; i += kThreads) {
        const int r = lo + i;
        int t = r < hi ? (r < n ? ib[r] : wstart + (r - n)) : 0;
        sm_tok[i] = t < 0 ? 0 : (t >= Lmax ? Lmax - 1 : t);
    }
    if (mine) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    if (attn_split<D>(q, kc, vc, Hkv, Lmax, scale_log2, nsplit, part, ctr, out, b, kvh, bh, split,
                      lo, hi, sm_tok) &&
        threadIdx.x == 0)
        arrive_lengths(bctr, ctx, plen, b, Hq, L, P, Lmax, n_p);
}

}  // namespace

int attn_nsplit(int rows) {
    const long long n = ((long long)rows + CH - 1) / CH;
    return n > 0 ? (int)n : 1;
}

size_t attn_ws_layout(int B, int Hq, int rows, int D, void *base, float **part, uint32_t **ctr,
                      uint32_t **bctr) {
    const size_t nbh = (size_t)B * Hq;
    size_t part_bytes = nbh * attn_nsplit(rows) * (D + 2) * sizeof(float);
    part_bytes = (part_bytes + 255) & ~(size_t)255;
    const size_t b_bytes = ((size_t)B * sizeof(uint32_t) + 255) & ~(size_t)255;
    if (base) {
        *part = static_cast<float *>(base);
        if (bctr) *bctr = reinterpret_cast<uint32_t *>(static_cast<char *>(base) + part_bytes);
        *ctr = reinterpret_cast<uint32_t *>(static_cast<char *>(base) + part_bytes + b_bytes);
    }
    return part_bytes + b_bytes + nbh * sizeof(uint32_t);
}

tb_status launch_attn(const void *q, const void *kc, const void *vc, const int32_t *idx,
                      const int32_t *count, int cap, const int32_t *ctx, int window, int B,
                      int Hq, int Hkv, int Lmax, int D, float scale, float *out, float *part,
                      uint32_t *ctr, hipStream_t st) {
    if (ctx == nullptr) window = 0;
    const int nsplit = attn_nsplit(cap + window);
    const long long items = (long long)B * Hq * nsplit;
    const long long nb = (items + 7) / 8 * 8;
    if (nb > 0x7fffffff) {
        set_error("tb_sparse_decode_attn: grid too large");
        return TB_ERR_UNSUPPORTED_SHAPE;
    }
    const float scale_log2 = scale * 1.4426950408889634f;
    const uint16_t *qq = static_cast<const uint16_t *>(q);
    const uint16_t *kk = static_cast<const uint16_t *>(kc);
    const uint16_t *vv = static_cast<const uint16_t *>(vc);
    if (D == 128)
        hipLaunchKernelGGL(attn_kernel<128>, dim3((unsigned)nb), dim3(kThreads), 0, st, qq, kk, vv,
                           idx, count, cap, ctx, window, Hq, Hkv, Lmax, scale_log2, nsplit,
                           (int)items, part, ctr, out);
    else
        hipLaunchKernelGGL(attn_kernel<64>, dim3((unsigned)nb), dim3(kThreads), 0, st, qq, kk, vv,
                           idx, count, cap, ctx, window, Hq, Hkv, Lmax, scale_log2, nsplit,
                           (int)items, part, ctr, out);
    return check_launch("tb_sparse_decode_attn");
}

tb_status launch_append_attn(const void *k_new, const void *v_new, void *kc, void *vc, void *kp,
                             const void *wk, int32_t *ctx, int32_t *plen, int n_p, const void *q,
                             const int32_t *idx, const int32_t *count, int cap, int window, int B,
                             int Hq, int Hkv, int Lmax, int D, int dp, float scale, float *out,
                             float *part, uint32_t *ctr, uint32_t *bctr, hipStream_t st) {
    const int nsplit = attn_nsplit(cap + window);
    const long long items = (long long)B * Hq * nsplit;
    const int nbA = (B + 7) / 8 * 8;
    const long long nb = nbA + (items + 7) / 8 * 8;
    if (nb > 0x7fffffff) {
        set_error("tb_append_attn: grid too large");
        return TB_ERR_UNSUPPORTED_SHAPE;
    }
    const float scale_log2 = scale * 1.4426950408889634f;
    const uint16_t *kn = static_cast<const uint16_t *>(k_new);
    const uint16_t *vn = static_cast<const uint16_t *>(v_new);
    uint16_t *kk = static_cast<uint16_t *>(kc);
    uint16_t *vv = static_cast<uint16_t *>(vc);
    uint16_t *kpp = static_cast<uint16_t *>(kp);
    const uint16_t *w = static_cast<const uint16_t *>(wk);
    const uint16_t *qq = static_cast<const uint16_t *>(q);
#define TB_AA(DD, PP)                                                                         \
    if (D == DD && dp == PP) {                                                                \
        hipLaunchKernelGGL((append_attn_kernel<DD, PP>), dim3((unsigned)nb), dim3(kThreads), 0,  \
                           st, kn, vn, kk, vv, kpp, w, ctx, plen, n_p, qq, idx, count, cap,      \
                           window, B, Hq, Hkv, Lmax, scale_log2, nsplit, (int)items, nbA, part,  \
                           ctr, bctr, out);                                                    \
        return check_launch("tb_append_attn");                                                \
    }
    TB_AA(128, 32) TB_AA(128, 16) TB_AA(64, 32) TB_AA(64, 16)
#undef TB_AA
    set_error("tb_append_attn: unsupported D=%d dp=%d", D, dp);
    return TB_ERR_UNSUPPORTED_SHAPE;
}

}  // namespace tb
