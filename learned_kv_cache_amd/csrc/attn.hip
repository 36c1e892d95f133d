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

}  // namespace

int attn_nsplit(int rows) {
    const long long n = ((long long)rows + CH - 1) / CH;
    return n > 0 ? (int)n : 1;
}

size_t attn_ws_layout(int B, int Hq, int rows, int D, void *base, float **part, uint32_t **ctr) {
    const size_t nbh = (size_t)B * Hq;
    size_t part_bytes = nbh * attn_nsplit(rows) * (D + 2) * sizeof(float);
    part_bytes = (part_bytes + 255) & ~(size_t)255;
    if (base) {
        *part = static_cast<float *>(base);
        *ctr = reinterpret_cast<uint32_t *>(static_cast<char *>(base) + part_bytes);
    }
    return part_bytes + nbh * sizeof(uint32_t);
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

}  // namespace tb
