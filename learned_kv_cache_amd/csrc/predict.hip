// Query prediction: a two-layer MLP with SiLU on the producer layer's hidden
// state ("TokenButler" summary, "Core architecture": query prediction).
//
//   h    = bf16_rne(SiLU(x w1^T))      mlp1: split over the reduction (E)
//   qhat = h w2^T                      mlp2: each workgroup first builds h
//                                      (sum of the mlp1 partials, SiLU, bf16)
//                                      for its batch tile in LDS
//
// Both are MFMA 16x16x32 bf16 GEMMs with the weight rows as the A operand
// (16 output features per tile) and the batch as the B operand (up to 16
// sequences per tile), so the weights -- the only large operand -- stream from
// HBM in 64-byte runs per lane. The reduction index is permuted identically
// in A and B so that each lane reads 32 contiguous elements per 128-element
// block; the result is the same sum. The four waves of a workgroup take
// interleaved 128-element blocks and are reduced through LDS.
#include "project_impl.h"

namespace tb {
namespace {

typedef bf16x8_t bf16x8;
typedef f32x4_t f32x4;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int BLK = 128;
constexpr int kMaxSplit = 16;
constexpr int kMaxBlkPerWave = 3;   // Eh <= 1536 = 3 blocks per wave

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Reduce the four waves' 16x16 tiles; thread tid gets (row tid/16, col tid%16).
__device__ __forceinline__ float reduce_waves(const f32x4 &acc, float (*red)[64][4]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][lane][i] = acc[i];
    __syncthreads();
    const int row = threadIdx.x >> 4, col = threadIdx.x & 15;
    const int src_lane = (row >> 2) * 16 + col, src_i = row & 3;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += red[w][src_lane][src_i];
    return s;
}

__device__ __forceinline__ void mlp1_block(const uint16_t *__restrict__ x,
                                           const uint16_t *__restrict__ w1,
                                           float *__restrict__ part, int B, int E, int Eh, int bps,
                                           int jt, int sp, int bt, float (*red)[64][4]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, kq = lane >> 4;
    const int nblk = E / BLK;
    const int blk0 = sp * bps;
    const int blk1 = blk0 + bps < nblk ? blk0 + bps : nblk;
    const int bb = bt * 16 + n;
    const uint16_t *arow = w1 + (size_t)(jt * 16 + n) * E + kq * 32;
    const uint16_t *brow = x + (size_t)bb * E + kq * 32;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int blk = blk0 + wave; blk < blk1; blk += kWaves) {
        const uint4 *a = reinterpret_cast<const uint4 *>(arow + blk * BLK);
        uint4 av[4], bv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) av[v] = a[v];
        if (bb < B) {
            const uint4 *bp = reinterpret_cast<const uint4 *>(brow + blk * BLK);
#pragma unroll
            for (int v = 0; v < 4; ++v) bv[v] = bp[v];
        } else {
#pragma unroll
            for (int v = 0; v < 4; ++v) bv[v] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[v]), as_bf16x8(bv[v]), acc,
                                                          0, 0, 0);
    }
    const float s = reduce_waves(acc, red);
    const int j = jt * 16 + (threadIdx.x >> 4);
    const int ob = bt * 16 + (threadIdx.x & 15);
    if (ob < B) part[((size_t)sp * B + ob) * Eh + j] = s;
}

__global__ __launch_bounds__(kThreads) void mlp1_kernel(const uint16_t *__restrict__ x,
                                                        const uint16_t *__restrict__ w1,
                                                        float *__restrict__ part, int B, int E,
                                                        int Eh, int bps) {
    __shared__ float red[kWaves][64][4];
    mlp1_block(x, w1, part, B, E, Eh, bps, blockIdx.x, blockIdx.y, blockIdx.z, red);
}

// mlp1 and an independent key projection in one launch: the first n1
// workgroups are mlp1 tiles, the rest projection workgroups.
template <int D, int DP>
__global__ __launch_bounds__(kThreads) void mlp1_project_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w1, float *__restrict__ part,
    int B, int E, int Eh, int bps, int nsplit, int n1, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ wk, uint16_t *__restrict__ kp, const int32_t *__restrict__ pos0,
    int ntok, int Hkv, int Lmax, int nproj) {
    __shared__ float red[kWaves][64][4];
    const int bid = blockIdx.x;
    if (bid < n1) {
        const int jt = bid % (Eh / 16);
        const int rest = bid / (Eh / 16);
        mlp1_block(x, w1, part, B, E, Eh, bps, jt, rest % nsplit, rest / nsplit, red);
    } else {
        const int q = bid - n1;
        const int blk = q % nproj;
        const int rest = q / nproj;
        project_block<D, DP>(kc, wk, kp, pos0, ntok, Hkv, Lmax, blk, rest % Hkv, rest / Hkv);
    }
}

__device__ __forceinline__ uint32_t silu_bf16(float z) {
    return f32_to_bf16_rne(z / (1.f + expf(-z)));
}

// h for the batch tile is built once per workgroup in LDS: the mlp1 split
// partials are summed in a fixed order, passed through SiLU and rounded to
// bf16; the MFMA B operand is then read from LDS.
__global__ __launch_bounds__(kThreads) void mlp2_kernel(const float *__restrict__ part,
                                                        const uint16_t *__restrict__ w2,
                                                        float *__restrict__ qhat, int B, int Eh,
                                                        int n_out, int nsplit) {
    __shared__ float red[kWaves][64][4];
    extern __shared__ uint16_t s_h[];   // [16][Eh]
    const int nt = blockIdx.x, bt = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, kq = lane >> 4;
    const int nb = B - bt * 16 < 16 ? B - bt * 16 : 16;
    const int nblk = Eh / BLK;
    // the thread's first partials are requested before the wave's W2 tiles,
    // so building h waits for the partials only (loads complete in order)
    const int q4 = Eh / 4;
    const size_t sstride = (size_t)B * Eh;
    float4 f[kMaxSplit];
    const int it0 = threadIdx.x;
    if (it0 < nb * q4) {
        const int bl = it0 / q4, j = (it0 - bl * q4) * 4;
        const float *p0 = part + (size_t)(bt * 16 + bl) * Eh + j;
#pragma unroll
        for (int sp = 0; sp < kMaxSplit; ++sp)
            f[sp] = sp < nsplit ? *reinterpret_cast<const float4 *>(p0 + sp * sstride)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const uint16_t *arow = w2 + (size_t)(nt * 16 + n) * Eh + kq * 32;
    uint4 av[kMaxBlkPerWave][4];
#pragma unroll
    for (int i = 0; i < kMaxBlkPerWave; ++i) {
        const int blk = wave + i * kWaves;
        if (blk < nblk) {
            const uint4 *a = reinterpret_cast<const uint4 *>(arow + blk * BLK);
#pragma unroll
            for (int v = 0; v < 4; ++v) av[i][v] = a[v];
        }
    }
    // rows of the tile beyond B are zero
    for (int i = threadIdx.x; i < (16 - nb) * Eh; i += kThreads) s_h[nb * Eh + i] = 0;
    for (int it = it0; it < nb * q4; it += kThreads) {
        const int bl = it / q4, j = (it - bl * q4) * 4;
        const float *p0 = part + (size_t)(bt * 16 + bl) * Eh + j;
        if (it != it0) {
#pragma unroll
            for (int sp = 0; sp < kMaxSplit; ++sp)
                f[sp] = sp < nsplit ? *reinterpret_cast<const float4 *>(p0 + sp * sstride)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int sp = 0; sp < kMaxSplit; ++sp) {
            z.x += f[sp].x;
            z.y += f[sp].y;
            z.z += f[sp].z;
            z.w += f[sp].w;
        }
        uint2 hv;
        hv.x = silu_bf16(z.x) | (silu_bf16(z.y) << 16);
        hv.y = silu_bf16(z.z) | (silu_bf16(z.w) << 16);
        *reinterpret_cast<uint2 *>(s_h + bl * Eh + j) = hv;
    }
    __syncthreads();
    const uint4 *hrow = reinterpret_cast<const uint4 *>(s_h + n * Eh + kq * 32);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kMaxBlkPerWave; ++i) {
        const int blk = wave + i * kWaves;
        if (blk < nblk) {
            uint4 bv[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) bv[v] = hrow[blk * (BLK / 8) + v];
#pragma unroll
            for (int v = 0; v < 4; ++v)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[i][v]),
                                                              as_bf16x8(bv[v]), acc, 0, 0, 0);
        }
    }
    const float s = reduce_waves(acc, red);
    const int o = nt * 16 + (threadIdx.x >> 4);
    const int ob = bt * 16 + (threadIdx.x & 15);
    if (ob < B) qhat[(size_t)ob * n_out + o] = s;
}

}  // namespace

int predict_nsplit(int E, int Eh) {
    const int nblk = E / BLK;
    const int tiles = Eh / 16 > 0 ? Eh / 16 : 1;
    int ns = (512 + tiles - 1) / tiles;
    if (ns > nblk) ns = nblk;
    if (ns > kMaxSplit) ns = kMaxSplit;
    if (ns < 1) ns = 1;
    const int bps = (nblk + ns - 1) / ns;
    return (nblk + bps - 1) / bps;  // no empty split
}

tb_status launch_predict(const void *x, const void *w1, const void *w2, float *qhat, int B, int E,
                         int Eh, int n_out, void *ws, int nsplit, hipStream_t st) {
    const int nblk = E / BLK;
    const int bps = (nblk + nsplit - 1) / nsplit;
    float *part = static_cast<float *>(ws);
    const int bt = (B + 15) / 16;
    hipLaunchKernelGGL(mlp1_kernel, dim3(Eh / 16, nsplit, bt), dim3(kThreads), 0, st,
                       static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(w1), part,
                       B, E, Eh, bps);
    tb_status e = check_launch("tb_predict_queries(mlp1)");
    if (e) return e;
    hipLaunchKernelGGL(mlp2_kernel, dim3(n_out / 16, 1, bt), dim3(kThreads),
                       (size_t)16 * Eh * sizeof(uint16_t), st, part,
                       static_cast<const uint16_t *>(w2), qhat, B, Eh, n_out, nsplit);
    return check_launch("tb_predict_queries(mlp2)");
}

tb_status launch_predict_project(const void *x, const void *w1, const void *w2, float *qhat,
                                 int B, int E, int Eh, int n_out, void *ws, int nsplit,
                                 const void *kc, const void *wk, void *kp, const int32_t *pos0,
                                 int ntok, int Hkv, int Lmax, int D, int dp, hipStream_t st) {
    if (ntok == 0)
        return launch_predict(x, w1, w2, qhat, B, E, Eh, n_out, ws, nsplit, st);
    const int nblk = E / BLK;
    const int bps = (nblk + nsplit - 1) / nsplit;
    float *part = static_cast<float *>(ws);
    const int bt = (B + 15) / 16;
    const int n1 = (Eh / 16) * nsplit * bt;
    const int nproj = (ntok + kProjTokPerBlock - 1) / kProjTokPerBlock;
    const long long nb = (long long)n1 + (long long)nproj * Hkv * B;
    if (nb > 0x7fffffffLL) {
        set_error("tb_predict_project: grid too large");
        return TB_ERR_UNSUPPORTED_SHAPE;
    }
    const uint16_t *xx = static_cast<const uint16_t *>(x);
    const uint16_t *ww1 = static_cast<const uint16_t *>(w1);
    const uint16_t *k = static_cast<const uint16_t *>(kc);
    const uint16_t *w = static_cast<const uint16_t *>(wk);
    uint16_t *o = static_cast<uint16_t *>(kp);
    bool launched = false;
#define TB_PP(DD, PP)                                                                          \
    if (!launched && D == DD && dp == PP) {                                                    \
        hipLaunchKernelGGL((mlp1_project_kernel<DD, PP>), dim3((unsigned)nb), dim3(kThreads), 0, \
                           st, xx, ww1, part, B, E, Eh, bps, nsplit, n1, k, w, o, pos0, ntok,  \
                           Hkv, Lmax, nproj);                                                  \
        launched = true;                                                                       \
    }
    TB_PP(128, 32) TB_PP(128, 16) TB_PP(64, 32) TB_PP(64, 16)
#undef TB_PP
    if (!launched) {
        set_error("tb_predict_project: unsupported D=%d dp=%d", D, dp);
        return TB_ERR_UNSUPPORTED_SHAPE;
    }
    tb_status e = check_launch("tb_predict_project(mlp1+project)");
    if (e) return e;
    hipLaunchKernelGGL(mlp2_kernel, dim3(n_out / 16, 1, bt), dim3(kThreads),
                       (size_t)16 * Eh * sizeof(uint16_t), st, part,
                       static_cast<const uint16_t *>(w2), qhat, B, Eh, n_out, nsplit);
    return check_launch("tb_predict_project(mlp2)");
}

}  // namespace tb
