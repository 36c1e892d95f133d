// CPU-offload decoding ("TokenButler" summary, "Inference strategy": the
// full cache is retained while a sink buffer, a circular local window and an
// important buffer are what attention reads; "Significance": only the
// selected tokens are accessed, which pays off most when the cache lives in
// host memory).
//
// The full K/V cache lives in pinned host memory, read by the kernels over
// the host link. Each query head has a device buffer of buf_rows rows:
// slots [0, cap) hold the head's sink + important rows, gathered once per
// prediction interval; the last `window` slots hold the circular window
// (token t in slot buf_rows - window + t mod window). Attention then runs on
// the device buffers with an identity list and the implicit window.
#include "tb_common.h"

namespace tb {
namespace {

constexpr int kGThreads = 256;
constexpr int kGRowsPerBlock = 64;

// Gather: grid (ceil(cap / 64), Hq, B). A row of D bf16 is D / 8 pieces of
// 16 bytes; the workgroup's 64 rows x pieces are spread over its threads, and
// every thread issues all of its host loads (K and V) before any store.
template <int D>
__global__ __launch_bounds__(kGThreads) void gather_kernel(
    const uint4 *__restrict__ kh, const uint4 *__restrict__ vh, int Hkv, int Lmax,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ count, int cap, int Hq,
    uint4 *__restrict__ kb, uint4 *__restrict__ vb, int buf_rows, int slot0, int wrap) {
    constexpr int P = D / 8;                               // pieces per row
    constexpr int PER = kGRowsPerBlock * P / kGThreads;    // pieces per thread
    const int h = blockIdx.y, b = blockIdx.z;
    const int g = Hq / Hkv;
    int n = count[b * Hq + h];
    n = n < 0 ? 0 : (n > cap ? cap : n);
    const int r0 = blockIdx.x * kGRowsPerBlock;
    if (r0 >= n) return;
    const int32_t *il = idx + ((size_t)b * Hq + h) * cap;
    const size_t hsrc = ((size_t)b * Hkv + h / g) * Lmax;
    const size_t hdst = ((size_t)b * Hq + h) * buf_rows;
    uint4 kv[PER], vv[PER];
    int slot[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int e = threadIdx.x + k * kGThreads;
        const int i = r0 + e / P, p = e % P;
        slot[k] = -1;
        if (i < n) {
            int t = il[i];
            t = t < 0 ? 0 : (t >= Lmax ? Lmax - 1 : t);
            const int s = slot0 + (wrap > 0 ? t % wrap : i);
            if (s < buf_rows) {
                slot[k] = s;
                kv[k] = kh[(hsrc + t) * P + p];
                vv[k] = vh[(hsrc + t) * P + p];
            }
        }
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        if (slot[k] < 0) continue;
        const int p = (threadIdx.x + k * kGThreads) % P;
        kb[(hdst + slot[k]) * P + p] = kv[k];
        vb[(hdst + slot[k]) * P + p] = vv[k];
    }
}

// Append, one workgroup per sequence: with L = ctx_len[b] = proj_len[b] <
// Lmax, the new K/V rows go to position L of the host cache and to the
// window slot of every query head of their group; the new key is projected
// into kp (fp32 dot products of the bf16 row with W_k, one thread per
// (KV head, channel)); the lengths advance.
template <int D>
__global__ __launch_bounds__(kGThreads) void offload_append_kernel(
    const uint4 *__restrict__ k_new, const uint4 *__restrict__ v_new,
    const uint16_t *__restrict__ wk, uint4 *__restrict__ kh, uint4 *__restrict__ vh,
    uint16_t *__restrict__ kp, int32_t *__restrict__ ctx, int32_t *__restrict__ plen, int Hkv,
    int Lmax, int dp, uint4 *__restrict__ kb, uint4 *__restrict__ vb, int Hq, int buf_rows,
    int window) {
    constexpr int P = D / 8;
    const int b = blockIdx.x;
    const int L = ctx[b], Pl = plen[b];
    if (!(Pl == L && L >= 0 && L < Lmax)) return;
    const int g = Hq / Hkv;
    for (int e = threadIdx.x; e < Hkv * P; e += kGThreads) {
        const int j = e / P, p = e % P;
        const uint4 kr = k_new[((size_t)b * Hkv + j) * P + p];
        const uint4 vr = v_new[((size_t)b * Hkv + j) * P + p];
        const size_t src = (((size_t)b * Hkv + j) * Lmax + L) * P + p;
        kh[src] = kr;
        vh[src] = vr;
        if (window > 0) {
            const int s = buf_rows - window + L % window;
            for (int h = j * g; h < (j + 1) * g; ++h) {
                const size_t dst = (((size_t)b * Hq + h) * buf_rows + s) * P + p;
                kb[dst] = kr;
                vb[dst] = vr;
            }
        }
    }
    const uint16_t *kn = reinterpret_cast<const uint16_t *>(k_new);
    for (int e = threadIdx.x; e < Hkv * dp; e += kGThreads) {
        const int j = e / dp, c = e % dp;
        const uint16_t *row = kn + ((size_t)b * Hkv + j) * D;
        const uint16_t *w = wk + ((size_t)j * dp + c) * D;
        float acc = 0.f;
        for (int i = 0; i < D; i += 2) {
            const uint32_t a = *reinterpret_cast<const uint32_t *>(row + i);
            const uint32_t m = *reinterpret_cast<const uint32_t *>(w + i);
            acc = __builtin_fmaf(bf16_lo(a), bf16_lo(m), acc);
            acc = __builtin_fmaf(bf16_hi(a), bf16_hi(m), acc);
        }
        kp[(((size_t)b * Hkv + j) * Lmax + L) * dp + c] = (uint16_t)f32_to_f16_bits(acc);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        ctx[b] = L + 1;
        plen[b] = L + 1;
    }
}

}  // namespace

tb_status launch_offload_gather(const void *kh, const void *vh, int B, int Hkv, int Lmax, int D,
                                const int32_t *idx, const int32_t *count, int cap, int Hq,
                                void *kb, void *vb, int buf_rows, int slot0, int wrap,
                                hipStream_t st) {
    dim3 grid((cap + kGRowsPerBlock - 1) / kGRowsPerBlock, Hq, B);
    const uint4 *k = static_cast<const uint4 *>(kh);
    const uint4 *v = static_cast<const uint4 *>(vh);
    uint4 *ko = static_cast<uint4 *>(kb);
    uint4 *vo = static_cast<uint4 *>(vb);
    if (D == 128)
        hipLaunchKernelGGL(gather_kernel<128>, grid, dim3(kGThreads), 0, st, k, v, Hkv, Lmax, idx,
                           count, cap, Hq, ko, vo, buf_rows, slot0, wrap);
    else
        hipLaunchKernelGGL(gather_kernel<64>, grid, dim3(kGThreads), 0, st, k, v, Hkv, Lmax, idx,
                           count, cap, Hq, ko, vo, buf_rows, slot0, wrap);
    return check_launch("tb_offload_gather");
}

tb_status launch_offload_append(const void *k_new, const void *v_new, const void *wk, void *kh,
                                void *vh, void *kp, int32_t *ctx, int32_t *plen, int B, int Hkv,
                                int Lmax, int D, int dp, void *kb, void *vb, int Hq,
                                int buf_rows, int window, hipStream_t st) {
    const uint4 *kn = static_cast<const uint4 *>(k_new);
    const uint4 *vn = static_cast<const uint4 *>(v_new);
    const uint16_t *w = static_cast<const uint16_t *>(wk);
    uint16_t *o = static_cast<uint16_t *>(kp);
    if (D == 128)
        hipLaunchKernelGGL(offload_append_kernel<128>, dim3(B), dim3(kGThreads), 0, st, kn, vn, w,
                           static_cast<uint4 *>(kh), static_cast<uint4 *>(vh), o, ctx, plen, Hkv,
                           Lmax, dp, static_cast<uint4 *>(kb), static_cast<uint4 *>(vb), Hq,
                           buf_rows, window);
    else
        hipLaunchKernelGGL(offload_append_kernel<64>, dim3(B), dim3(kGThreads), 0, st, kn, vn, w,
                           static_cast<uint4 *>(kh), static_cast<uint4 *>(vh), o, ctx, plen, Hkv,
                           Lmax, dp, static_cast<uint4 *>(kb), static_cast<uint4 *>(vb), Hq,
                           buf_rows, window);
    return check_launch("tb_offload_append");
}

}  // namespace tb
