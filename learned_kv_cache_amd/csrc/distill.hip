// Distillation loss ("TokenButler" summary, "Training": the predictor learns
// from the frozen model's masked causal attention distribution by the cross
// entropy between the teacher's attention logits and its own logits, at a
// subset of R query positions, so the cost is O(R L)).
//
// Per (b, r, query head h), i = pos[b, r], KV head h / g, tokens t <= i:
//   z_t = scale q . k_t (bf16 x bf16 MFMA, fp32 accumulation),
//   s_t = qhat . kp_t   (qhat split into fp16 hi + lo parts, two fp16 MFMAs
//                        against the fp16 keys: every product is exact in
//                        fp32 and hi + lo carries qhat to 2^-22 relative),
//   loss = logsumexp(s) - sum_t softmax(z)_t s_t.
// A workgroup takes the g * R rows of one (b, KV head) in groups of 256
// (8 waves x 2 tiles of 16 rows) and a 1024-token split of the cache; K and
// K' rows are staged in LDS 64 tokens at a time for all 8 waves, the next
// 64 loaded into registers while the current ones are multiplied. Each lane
// keeps online-softmax states (teacher max / sum / weighted student sum,
// student max / sum) for its 8 (row, token-column) pairs in base 2; they are
// merged across the 16 token columns at the end, written as the split's
// partial, and the last workgroup of the row group to arrive merges the
// splits and writes the loss.
#include "tb_common.h"

namespace tb {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kDThreads = 512;
constexpr int kDWaves = kDThreads / 64;
constexpr int kDRows = kDWaves * 32;   // rows per workgroup
constexpr int kDSplit = 1024;          // tokens per workgroup
constexpr int kDPart = 5;              // floats per (row, split) partial
constexpr float kNeg = -1e30f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ void merge3(float &m, float &z, float &a, float m2, float z2, float a2) {
    const float mm = fmaxf(m, m2);
    const float e1 = exp2f(m - mm), e2 = exp2f(m2 - mm);
    z = z * e1 + z2 * e2;
    a = a * e1 + a2 * e2;
    m = mm;
}

__device__ __forceinline__ void merge2(float &m, float &z, float m2, float z2) {
    const float mm = fmaxf(m, m2);
    z = z * exp2f(m - mm) + z2 * exp2f(m2 - mm);
    m = mm;
}

// Add one logit x (base 2) to a running (max m, sum z[, weighted sum a]),
// branch-free, with one exp2: of the old maximum and x, the larger takes the
// factor 2^0 = 1 and the other 2^-|x - m|, so the running sums are rescaled
// when x is the new maximum and take the term 2^(x - m) otherwise (the same
// roundings as forming both factors; no contraction, so a + e w rounds the
// product first). exp2 is the hardware instruction: its argument is <= 0 and
// results below 2^-126 (flushed) are negligible against the sum, which
// always holds a term of 1.
__device__ __forceinline__ void add3(float &m, float &z, float &a, float x, float w) {
#pragma clang fp contract(off)
    const float e = __builtin_amdgcn_exp2f(-fabsf(x - m));
    const bool up = x > m;
    const float ew = e * w;
    z = up ? __builtin_fmaf(z, e, 1.f) : z + e;
    a = up ? __builtin_fmaf(a, e, w) : a + ew;
    m = fmaxf(m, x);
}

__device__ __forceinline__ void add2(float &m, float &z, float x) {
#pragma clang fp contract(off)
    const float e = __builtin_amdgcn_exp2f(-fabsf(x - m));
    z = x > m ? __builtin_fmaf(z, e, 1.f) : z + e;
    m = fmaxf(m, x);
}

template <int D, int DP>
__global__ __launch_bounds__(kDThreads) void distill_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc, const float *__restrict__ qhat,
    const uint16_t *__restrict__ kp, const int32_t *__restrict__ pos, int R, int Hq, int Hkv,
    int Lmax, float scale_log2, int nsplit, int ngroups, float *__restrict__ part,
    uint32_t *__restrict__ ctr, float *__restrict__ loss) {
    constexpr int NV = D / 32;     // bf16 MFMA k-steps
    constexpr int KP = D / 8;      // 16-byte pieces per K row
    constexpr int KPP = DP / 8;    // 16-byte pieces per K' row
    constexpr int SB = 64;                           // tokens staged per step
    constexpr int NK = (SB * KP + kDThreads - 1) / kDThreads;   // K pieces per thread
    __shared__ uint4 s_k[SB * KP];
    __shared__ uint4 s_kp[SB * KPP];
    __shared__ int s_pmax;
    __shared__ bool s_last;
    const int split = blockIdx.x, grp = blockIdx.y, bkv = blockIdx.z;
    const int b = bkv / Hkv, kvh = bkv % Hkv, g = Hq / Hkv;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, kq = lane >> 4;
    const int nrows = R * g;
    const size_t head = (size_t)b * Hkv + kvh;

    // A operands: rows grp*kDRows + wave*32 + rt*16 + n
    static_assert(DP == 16 || DP == 32, "d' of 16 or 32");
    uint4 qa[2][NV];
    f16x8_t qhi[2], qlo[2];   // qhat[row][8 kq .. 8 kq + 8) as fp16 hi + lo
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int row = grp * kDRows + wave * 32 + rt * 16 + n;
        if (row < nrows) {
            const int r = row / g, h = kvh * g + row % g;
            const size_t qi = ((size_t)b * R + r) * Hq + h;
            const uint4 *qr = reinterpret_cast<const uint4 *>(q + qi * D + kq * (D / 4));
#pragma unroll
            for (int v = 0; v < NV; ++v) qa[rt][v] = qr[v];
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const float x = 8 * kq + s < DP ? qhat[qi * DP + 8 * kq + s] : 0.f;
                const _Float16 hi = (_Float16)x;
                qhi[rt][s] = hi;
                qlo[rt][s] = (_Float16)(x - (float)hi);
            }
        } else {
#pragma unroll
            for (int v = 0; v < NV; ++v) qa[rt][v] = make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                qhi[rt][s] = (_Float16)0.f;
                qlo[rt][s] = (_Float16)0.f;
            }
        }
    }
    // output rows of this lane: grp*kDRows + wave*32 + rt*16 + 4*kq + i
    int po[2][4];
    if (threadIdx.x == 0) s_pmax = -1;
    __syncthreads();
    int pm = -1;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = grp * kDRows + wave * 32 + rt * 16 + 4 * kq + i;
            int p = -1;
            if (row < nrows) {
                p = pos[(size_t)b * R + row / g];
                p = p < 0 ? 0 : (p > Lmax - 1 ? Lmax - 1 : p);
            }
            po[rt][i] = p;
            pm = p > pm ? p : pm;
        }
    atomicMax(&s_pmax, pm);
    __syncthreads();
    const int t_end = min((split + 1) * kDSplit, s_pmax + 1);

    float mz[2][4], zz[2][4], az[2][4], ms[2][4], zs[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            mz[rt][i] = kNeg;
            zz[rt][i] = 0.f;
            az[rt][i] = 0.f;
            ms[rt][i] = kNeg;
            zs[rt][i] = 0.f;
        }

    // the next stage's rows are loaded into registers while the current
    // stage is multiplied out of LDS
    uint4 nk[NK], nkp = make_uint4(0, 0, 0, 0);
    auto fetch = [&](int t0) {
#pragma unroll
        for (int j = 0; j < NK; ++j) {
            const int e = threadIdx.x + j * kDThreads;
            const int tok = t0 + e / KP;
            nk[j] = (e < SB * KP && tok < Lmax)
                        ? reinterpret_cast<const uint4 *>(kc)[(head * Lmax + tok) * KP + e % KP]
                        : make_uint4(0, 0, 0, 0);
        }
        if (threadIdx.x < SB * KPP) {
            const int tok = t0 + threadIdx.x / KPP;
            nkp = tok < Lmax ? reinterpret_cast<const uint4 *>(kp)[(head * Lmax + tok) * KPP +
                                                                   threadIdx.x % KPP]
                             : make_uint4(0, 0, 0, 0);
        }
    };
    const int t_begin = split * kDSplit;
    if (t_begin < t_end) fetch(t_begin);
    for (int t0 = t_begin; t0 < t_end; t0 += SB) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NK; ++j) {
            const int e = threadIdx.x + j * kDThreads;
            if (e < SB * KP) s_k[e] = nk[j];
        }
        if (threadIdx.x < SB * KPP) s_kp[threadIdx.x] = nkp;
        __syncthreads();
        if (t0 + SB < t_end) fetch(t0 + SB);
        const int nsub = (t_end - t0 + 15) / 16 < SB / 16 ? (t_end - t0 + 15) / 16 : SB / 16;
        for (int sb = 0; sb < nsub; ++sb) {
            uint4 kb[NV];
#pragma unroll
            for (int v = 0; v < NV; ++v) kb[v] = s_k[(sb * 16 + n) * KP + kq * (D / 32) + v];
            // K' operand: channels [8 kq, 8 kq + 8) of token n (zero past d')
            uint4 kf = make_uint4(0, 0, 0, 0);
            if (8 * kq < DP) kf = s_kp[(sb * 16 + n) * KPP + kq];
            const int t = t0 + sb * 16 + n;
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                f32x4_t acz = {0.f, 0.f, 0.f, 0.f}, acs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    acz = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, qa[rt][v]), __builtin_bit_cast(bf16x8_t, kb[v]),
                        acz, 0, 0, 0);
                const f16x8_t kh = __builtin_bit_cast(f16x8_t, kf);
                acs = __builtin_amdgcn_mfma_f32_16x16x32_f16(qhi[rt], kh, acs, 0, 0, 0);
                acs = __builtin_amdgcn_mfma_f32_16x16x32_f16(qlo[rt], kh, acs, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (t > po[rt][i]) continue;
                    const float z2 = acz[i] * scale_log2;
                    const float sv = acs[i];
                    add3(mz[rt][i], zz[rt][i], az[rt][i], z2, sv);
                    add2(ms[rt][i], zs[rt][i], sv * kLog2e);
                }
            }
        }
    }
    // merge the 16 token columns (lanes with the same kq)
#pragma unroll
    for (int off = 1; off < 16; off <<= 1)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float m2 = __shfl_xor(mz[rt][i], off), z2 = __shfl_xor(zz[rt][i], off);
                const float a2 = __shfl_xor(az[rt][i], off);
                const float n2 = __shfl_xor(ms[rt][i], off), s2 = __shfl_xor(zs[rt][i], off);
                merge3(mz[rt][i], zz[rt][i], az[rt][i], m2, z2, a2);
                merge2(ms[rt][i], zs[rt][i], n2, s2);
            }
    float *pg = part + ((size_t)bkv * ngroups + grp) * kDRows * nsplit * kDPart;
    if (n == 0) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rl = wave * 32 + rt * 16 + 4 * kq + i;
                float *pp = pg + ((size_t)rl * nsplit + split) * kDPart;
                __hip_atomic_store(pp + 0, mz[rt][i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(pp + 1, zz[rt][i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(pp + 2, az[rt][i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(pp + 3, ms[rt][i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(pp + 4, zs[rt][i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
    }
    // every wave's partial stores complete before the arrival is counted
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    uint32_t *c = ctr + (size_t)bkv * ngroups + grp;
    if (threadIdx.x == 0)
        s_last = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 (uint32_t)(nsplit - 1);
    __syncthreads();
    if (!s_last) return;
    if (threadIdx.x == 0) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x >= kDRows) return;
    const int row = grp * kDRows + threadIdx.x;
    if (row >= nrows) return;
    float m = kNeg, zt = 0.f, at = 0.f, mss = kNeg, zss = 0.f;
    const float *pr = pg + (size_t)threadIdx.x * nsplit * kDPart;
    for (int sp = 0; sp < nsplit; ++sp) {
        const float *pp = pr + (size_t)sp * kDPart;
        const float m2 = __hip_atomic_load(pp + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float z2 = __hip_atomic_load(pp + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float a2 = __hip_atomic_load(pp + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float n2 = __hip_atomic_load(pp + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float s2 = __hip_atomic_load(pp + 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        merge3(m, zt, at, m2, z2, a2);
        merge2(mss, zss, n2, s2);
    }
    const int r = row / g, h = kvh * g + row % g;
    loss[((size_t)b * R + r) * Hq + h] = (mss + log2f(zss)) * kLn2 - at / zt;
}

}  // namespace

int distill_nsplit(int Lmax) { return (int)(((long long)Lmax + kDSplit - 1) / kDSplit); }
int distill_ngroups(int R, int g) { return (int)(((long long)R * g + kDRows - 1) / kDRows); }

size_t distill_ws_layout(int B, int R, int Hq, int Hkv, int Lmax, void *base, float **part,
                         uint32_t **ctr) {
    const size_t nbkv = (size_t)B * Hkv;
    const int ng = distill_ngroups(R, Hq / Hkv);
    size_t part_bytes = nbkv * ng * kDRows * distill_nsplit(Lmax) * kDPart * sizeof(float);
    part_bytes = (part_bytes + 255) & ~(size_t)255;
    if (base) {
        *part = static_cast<float *>(base);
        *ctr = reinterpret_cast<uint32_t *>(static_cast<char *>(base) + part_bytes);
    }
    return part_bytes + ((nbkv * ng * sizeof(uint32_t) + 255) & ~(size_t)255);
}

tb_status launch_distill(const void *q, const void *kc, const float *qhat, const void *kp,
                         const int32_t *pos, int B, int R, int Hq, int Hkv, int Lmax, int D,
                         int dp, float scale, float *part, uint32_t *ctr, float *loss,
                         hipStream_t st) {
    const int nsplit = distill_nsplit(Lmax), ng = distill_ngroups(R, Hq / Hkv);
    dim3 grid(nsplit, ng, B * Hkv);
    const float sl2 = scale * kLog2e;
    const uint16_t *qq = static_cast<const uint16_t *>(q);
    const uint16_t *k = static_cast<const uint16_t *>(kc);
    const uint16_t *p = static_cast<const uint16_t *>(kp);
#define TB_D(DD, PP)                                                                          \
    if (D == DD && dp == PP) {                                                                \
        hipLaunchKernelGGL((distill_kernel<DD, PP>), grid, dim3(kDThreads), 0, st, qq, k, qhat, p, \
                           pos, R, Hq, Hkv, Lmax, sl2, nsplit, ng, part, ctr, loss);          \
        return check_launch("tb_distill_loss");                                               \
    }
    TB_D(128, 32) TB_D(128, 16) TB_D(64, 32) TB_D(64, 16)
#undef TB_D
    set_error("tb_distill_loss: unsupported D=%d dp=%d", D, dp);
    return TB_ERR_UNSUPPORTED_SHAPE;
}

}  // namespace tb
