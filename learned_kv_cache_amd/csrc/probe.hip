// Bandwidth ceilings measured on the part itself, reported beside the HBM
// peak by the benchmark: a plain streaming read, and a gather of exactly the
// K/V rows a sparse decode attention reads ("TokenButler" summary,
// "Significance": only the selected tokens' rows are read), in the attention
// launch's shape but without its arithmetic. Each kernel folds what it reads
// into one word per workgroup so that no load can be dropped.
#include "attn_impl.h"

namespace tb {
namespace {

constexpr int kReadThreads = 512;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint4 *__restrict__ src,
                                                                   size_t n16,
                                                                   uint32_t *__restrict__ sink) {
    // each thread keeps four 16-byte loads in flight per iteration
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * kReadThreads;
    size_t i = (size_t)blockIdx.x * kReadThreads + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
               d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const uint4 a = src[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    __shared__ uint32_t s[kReadThreads / 64];
    for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
    if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int w = 0; w < kReadThreads / 64; ++w) t ^= s[w];
        sink[blockIdx.x] = t;
    }
}

// The attention launch's work items and order (XCD-aware; kAttnCH list
// entries of one query head per workgroup, D / 8 lanes per row); every lane
// requests its K and V rows together and XORs them.
template <int D>
__global__ __launch_bounds__(kAttnThreads) void row_gather_kernel(
    const uint16_t *__restrict__ kc, const uint16_t *__restrict__ vc,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ count, int cap, int Hq, int Hkv,
    int Lmax, int nsplit, int n_items, uint32_t *__restrict__ sink) {
    constexpr int LPR = D / 8;
    constexpr int RPW = 64 / LPR;
    constexpr int NG = kAttnWaves * RPW;
    constexpr int RPG = kAttnCH / NG;
    __shared__ int sm_tok[kAttnCH];
    __shared__ uint32_t s[kAttnWaves];
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
    const int bh = b * Hq + kvh * g + hg;
    int n = count[bh];
    n = n < 0 ? 0 : (n > cap ? cap : n);
    const int lo = split * kAttnCH;
    const int hi = lo + kAttnCH < n ? lo + kAttnCH : n;
    for (int i = threadIdx.x; i < kAttnCH; i += kAttnThreads) {
        int t = lo + i < hi ? idx[(size_t)bh * cap + lo + i] : 0;
        sm_tok[i] = t < 0 ? 0 : (t >= Lmax ? Lmax - 1 : t);
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rg = lane / LPR, cl = lane % LPR;
    const int grp = wave * RPW + rg;
    const size_t head_off = (size_t)(b * Hkv + kvh) * Lmax * D;
    const int head_bytes = Lmax * D * 2;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(kc + head_off), (short)0, head_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(vc + head_off), (short)0, head_bytes, kRsrcWord3);
    uint4 kk[RPG], vv[RPG];
#pragma unroll
    for (int u = 0; u < RPG; ++u) {
        const int t = sm_tok[grp + u * NG];
        const bool ok = lo + grp + u * NG < hi;
        kk[u] = ok ? __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   krs, t * (D * 2) + cl * 16, 0, 0))
                   : make_uint4(0, 0, 0, 0);
        vv[u] = ok ? __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   vrs, t * (D * 2) + cl * 16, 0, 0))
                   : make_uint4(0, 0, 0, 0);
    }
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < RPG; ++u)
        acc ^= kk[u].x ^ kk[u].y ^ kk[u].z ^ kk[u].w ^ vv[u].x ^ vv[u].y ^ vv[u].z ^ vv[u].w;
    for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
    if (lane == 0) s[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int w = 0; w < kAttnWaves; ++w) t ^= s[w];
        sink[bid] = t;
    }
}

}  // namespace
}  // namespace tb

extern "C" {

tb_status tb_probe_stream_read(const void *src, size_t bytes, uint32_t *sink, int sink_words,
                               void *stream) {
    TB_REQUIRE(src && sink, TB_ERR_INVALID_ARGUMENT, "tb_probe_stream_read: null pointer");
    TB_REQUIRE(tb::aligned16(src) && tb::aligned4(sink), TB_ERR_INVALID_ARGUMENT,
               "tb_probe_stream_read: misaligned pointer");
    TB_REQUIRE(bytes >= 16 && bytes % 16 == 0 && sink_words >= 1, TB_ERR_INVALID_ARGUMENT,
               "tb_probe_stream_read: bytes must be a positive multiple of 16");
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        ncu <= 0)
        ncu = 256;
    int blocks = 4 * ncu;
    blocks = blocks < sink_words ? blocks : sink_words;
    hipLaunchKernelGGL(tb::stream_read_kernel, dim3(blocks), dim3(tb::kReadThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4 *>(src),
                       bytes / 16, sink);
    return tb::check_launch("tb_probe_stream_read");
}

size_t tb_probe_row_gather_sink_words(int B, int Hq, int cap) {
    if (B <= 0 || Hq <= 0 || cap <= 0 || (long long)B * Hq > 0x7fffffffLL) return 0;
    const long long items = (long long)B * Hq * tb::attn_nsplit(cap);
    return items > 0x7fffffffLL - 7 ? 0 : (size_t)((items + 7) / 8 * 8);
}

tb_status tb_probe_row_gather(const void *k_cache, const void *v_cache, const int32_t *idx,
                              const int32_t *count, int cap, int B, int Hq, int Hkv, int Lmax,
                              int D, uint32_t *sink, size_t sink_words, void *stream) {
    TB_REQUIRE(k_cache && v_cache && idx && count && sink, TB_ERR_INVALID_ARGUMENT,
               "tb_probe_row_gather: null pointer");
    TB_REQUIRE(tb::aligned16(k_cache) && tb::aligned16(v_cache) && tb::aligned4(idx) &&
                   tb::aligned4(count) && tb::aligned4(sink),
               TB_ERR_INVALID_ARGUMENT, "tb_probe_row_gather: misaligned pointer");
    TB_REQUIRE(B >= 1 && Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0 && Lmax >= 1 && cap >= 1,
               TB_ERR_INVALID_ARGUMENT, "tb_probe_row_gather: bad sizes");
    TB_REQUIRE(D == 64 || D == 128, TB_ERR_UNSUPPORTED_SHAPE,
               "tb_probe_row_gather: D must be 64 or 128");
    TB_REQUIRE((long long)Lmax * D * 2 <= 0x7fffffffLL, TB_ERR_UNSUPPORTED_SHAPE,
               "tb_probe_row_gather: one head's cache must be below 2 GiB");
    const size_t nb = tb_probe_row_gather_sink_words(B, Hq, cap);
    TB_REQUIRE(nb > 0, TB_ERR_UNSUPPORTED_SHAPE, "tb_probe_row_gather: grid beyond INT_MAX");
    TB_REQUIRE(sink_words >= nb, TB_ERR_WORKSPACE_TOO_SMALL,
               "tb_probe_row_gather: sink holds %zu words, needs %zu", sink_words, nb);
    const int nsplit = tb::attn_nsplit(cap);
    const int items = B * Hq * nsplit;
    const uint16_t *kk = static_cast<const uint16_t *>(k_cache);
    const uint16_t *vv = static_cast<const uint16_t *>(v_cache);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (D == 128)
        hipLaunchKernelGGL(tb::row_gather_kernel<128>, dim3((unsigned)nb), dim3(tb::kAttnThreads),
                           0, st, kk, vv, idx, count, cap, Hq, Hkv, Lmax, nsplit, items, sink);
    else
        hipLaunchKernelGGL(tb::row_gather_kernel<64>, dim3((unsigned)nb), dim3(tb::kAttnThreads),
                           0, st, kk, vv, idx, count, cap, Hq, Hkv, Lmax, nsplit, items, sink);
    return tb::check_launch("tb_probe_row_gather");
}

}  // extern "C"
