// Sparse decode attention over the selected positions of the retained KV
// cache ("TokenButler" summary, "Significance": keep the whole cache, read
// only the most relevant tokens).
//
// Split-K gather: a workgroup owns CH consecutive entries of one query head's
// ascending index list. D/8 lanes share one K/V row (16 bytes = 8 channels per
// lane), so a wave gathers 64/(D/8) rows per 16-byte load and keeps U rows of
// K and V in flight per lane. Logits are reduced with DPP, the softmax runs
// online in registers (base-2, fp32), and the workgroup writes one partial
// (max, sum, o[D]). A second, small launch merges each head's partials by
// log-sum-exp into the fp32 output; the kernel boundary is the only
// synchronization between workgroups (no device-scope fences, which on this
// chip would write back and invalidate the XCD's L2).
//
// Launch order is XCD-aware: dispatch sends workgroup i to XCD i % 8, and the
// block index is decoded so that each XCD receives a contiguous run of work
// items ordered (b, kv head, split, query head in group). The g query heads of
// one KV group that read the same part of the cache run next to each other on
// the same XCD and share its L2.
#include "tb_common.h"

namespace tb {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int CH = 256;  // index-list entries per workgroup
constexpr int U = 4;     // rows in flight per row group per iteration

template <int D>
__global__ __launch_bounds__(kThreads) void attn_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ count, int cap, const int32_t *__restrict__ ctx, int window,
    int Hq, int Hkv, int Lmax, float scale_log2,
    int nsplit, int n_items, float *__restrict__ part) {
    constexpr int LPR = D / 8;          // lanes per row
    constexpr int RPW = 64 / LPR;       // row groups per wave
    constexpr int NG = kWaves * RPW;    // row groups per workgroup
    constexpr int STRIDE = NG;          // rows per workgroup pass

    __shared__ float sm_o[NG][D];
    __shared__ float sm_m[NG], sm_l[NG];
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

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rg = lane / LPR, cl = lane % LPR;
    const int grp = wave * RPW + rg;

    float qf[8];
    {
        const uint4 qv = *reinterpret_cast<const uint4 *>(q + (size_t)bh * D + cl * 8);
        const uint32_t w[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qf[2 * e] = bf16_lo(w[e]) * scale_log2;
            qf[2 * e + 1] = bf16_hi(w[e]) * scale_log2;
        }
    }
    const size_t head_off = (size_t)(b * Hkv + kvh) * Lmax * D + cl * 8;
    const uint16_t *kbase = kc + head_off;
    const uint16_t *vbase = vc + head_off;

    float m = -1e30f, l = 0.f;
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.f;

    for (int r0 = lo + grp; r0 < hi; r0 += STRIDE * U) {
        int tk[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = r0 + u * STRIDE;
            ok[u] = r < hi;
            tk[u] = sm_tok[ok[u] ? r - lo : 0];
        }
        uint4 kr[U], vr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (ok[u]) {
                kr[u] = *reinterpret_cast<const uint4 *>(kbase + (size_t)tk[u] * D);
                vr[u] = *reinterpret_cast<const uint4 *>(vbase + (size_t)tk[u] * D);
            } else {
                kr[u] = make_uint4(0, 0, 0, 0);
                vr[u] = make_uint4(0, 0, 0, 0);
            }
        }
        float s[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t w[4] = {kr[u].x, kr[u].y, kr[u].z, kr[u].w};
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                d = __builtin_fmaf(bf16_lo(w[e]), qf[2 * e], d);
                d = __builtin_fmaf(bf16_hi(w[e]), qf[2 * e + 1], d);
            }
            s[u] = group_sum<LPR>(d);
        }
        float mx = m;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (ok[u]) mx = fmaxf(mx, s[u]);
        const float alpha = exp2f(m - mx);
        float p[U];
        float psum = 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            p[u] = ok[u] ? exp2f(s[u] - mx) : 0.f;
            psum += p[u];
        }
        l = l * alpha + psum;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] *= alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t w[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] = __builtin_fmaf(p[u], bf16_lo(w[e]), acc[2 * e]);
                acc[2 * e + 1] = __builtin_fmaf(p[u], bf16_hi(w[e]), acc[2 * e + 1]);
            }
        }
        m = mx;
    }

    // merge the row groups of this workgroup into one partial
#pragma unroll
    for (int c = 0; c < 8; ++c) sm_o[grp][cl * 8 + c] = acc[c];
    if (cl == 0) {
        sm_m[grp] = m;
        sm_l[grp] = l;
    }
    __syncthreads();
    float *pp = part + ((size_t)bh * nsplit + split) * (D + 2);
    if (threadIdx.x < D) {
        float M = -1e30f;
#pragma unroll
        for (int i = 0; i < NG; ++i) M = fmaxf(M, sm_m[i]);
        float Ls = 0.f, O = 0.f;
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            const float w = exp2f(sm_m[i] - M);
            Ls += sm_l[i] * w;
            O += sm_o[i][threadIdx.x] * w;
        }
        pp[2 + threadIdx.x] = O;
        if (threadIdx.x == 0) {
            pp[0] = M;
            pp[1] = Ls;
        }
    }
}

// One workgroup per (b, h): log-sum-exp merge of the split partials. Up to
// 32 partials at a time are staged in LDS with independent loads, and the
// running (max, sum, numerator) is rescaled from one stage to the next.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float *__restrict__ part,
                                                           int nsplit, float *__restrict__ out) {
    constexpr int CS = 32;
    constexpr int PW = D + 2;
    __shared__ float sm[CS * PW];
    const int bh = blockIdx.x;
    const float *base = part + (size_t)bh * nsplit * PW;
    constexpr int PER = (CS * PW + 255) / 256;
    float M = -1e30f, den = 0.f, num = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += CS) {
        const int ns = nsplit - s0 < CS ? nsplit - s0 : CS;
        const float *src = base + (size_t)s0 * PW;
        float v[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = threadIdx.x + k * 256;
            v[k] = i < ns * PW ? src[i] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = threadIdx.x + k * 256;
            if (i < ns * PW) sm[i] = v[k];
        }
        __syncthreads();
        float Mc = M;
        for (int s = 0; s < ns; ++s) Mc = fmaxf(Mc, sm[s * PW]);
        const float r = exp2f(M - Mc);
        den *= r;
        num *= r;
        for (int s = 0; s < ns; ++s) {
            const float w = exp2f(sm[s * PW] - Mc);
            den += sm[s * PW + 1] * w;
            if (threadIdx.x < D) num += sm[s * PW + 2 + threadIdx.x] * w;
        }
        M = Mc;
    }
    if (threadIdx.x < D) out[(size_t)bh * D + threadIdx.x] = den > 0.f ? num / den : 0.f;
}

}  // namespace

int attn_nsplit(int rows) { return (rows + CH - 1) / CH > 0 ? (rows + CH - 1) / CH : 1; }

size_t attn_ws_layout(int B, int Hq, int rows, int D, void *base, float **part) {
    const size_t nbh = (size_t)B * Hq;
    size_t part_bytes = nbh * attn_nsplit(rows) * (D + 2) * sizeof(float);
    part_bytes = (part_bytes + 255) & ~(size_t)255;
    if (base) *part = static_cast<float *>(base);
    return part_bytes;
}

tb_status launch_attn(const void *q, const void *kc, const void *vc, const int32_t *idx,
                      const int32_t *count, int cap, const int32_t *ctx, int window, int B,
                      int Hq, int Hkv, int Lmax, int D, float scale, float *out, float *part,
                      hipStream_t st) {
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
                           (int)items, part);
    else
        hipLaunchKernelGGL(attn_kernel<64>, dim3((unsigned)nb), dim3(kThreads), 0, st, qq, kk, vv,
                           idx, count, cap, ctx, window, Hq, Hkv, Lmax, scale_log2, nsplit,
                           (int)items, part);
    tb_status e = check_launch("tb_sparse_decode_attn(split)");
    if (e) return e;
    if (D == 128)
        hipLaunchKernelGGL(attn_combine_kernel<128>, dim3(B * Hq), dim3(256), 0, st, part, nsplit,
                           out);
    else
        hipLaunchKernelGGL(attn_combine_kernel<64>, dim3(B * Hq), dim3(256), 0, st, part, nsplit,
                           out);
    return check_launch("tb_sparse_decode_attn(combine)");
}

}  // namespace tb
