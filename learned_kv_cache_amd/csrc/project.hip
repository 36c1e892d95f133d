// Key-cache projection into the predictor's low-dimensional space
// ("TokenButler" summary, "Core architecture": key-cache projection by a
// learned matrix; "Inference strategy": done once per batch of new tokens).
//
// kp[t, c] = fp16( sum_i K[t, i] * Wk[c, i] ) for a run of tokens of one
// (sequence, KV head). MFMA 16x16x32 bf16 -> fp32 with A = Wk rows (16
// channels) and B = K rows (16 tokens), so each lane's accumulator holds four
// consecutive channels of one token and is stored as one 8-byte fp16 packet.
// Each lane reads D/4 contiguous elements of its token row (the reduction
// index is permuted identically in A and B, which leaves the sum unchanged),
// so a row is fetched as full 64-byte (D = 128) or 32-byte (D = 64) pieces.
#include "project_impl.h"

namespace tb {
namespace {

template <int D, int DP>
__global__ __launch_bounds__(kProjThreads) void project_kernel(
    const uint16_t *__restrict__ kc, const uint16_t *__restrict__ wk, uint16_t *__restrict__ kp,
    const int32_t *__restrict__ pos0, int ntok, int Hkv, int Lmax) {
    project_block<D, DP>(kc, wk, kp, pos0, ntok, Hkv, Lmax, blockIdx.x, blockIdx.y, blockIdx.z);
}

}  // namespace

tb_status launch_project(const void *kc, const void *wk, void *kp, const int32_t *pos0, int ntok,
                         int B, int Hkv, int Lmax, int D, int dp, hipStream_t st) {
    if (ntok == 0) return TB_OK;
    dim3 grid((ntok + kProjTokPerBlock - 1) / kProjTokPerBlock, Hkv, B);
    const uint16_t *k = static_cast<const uint16_t *>(kc);
    const uint16_t *w = static_cast<const uint16_t *>(wk);
    uint16_t *o = static_cast<uint16_t *>(kp);
#define TB_P(DD, PP)                                                                        \
    if (D == DD && dp == PP) {                                                              \
        hipLaunchKernelGGL((project_kernel<DD, PP>), grid, dim3(kProjThreads), 0, st, k, w, o, pos0, \
                           ntok, Hkv, Lmax);                                                \
        return check_launch("tb_project_keys");                                             \
    }
    TB_P(128, 32) TB_P(128, 16) TB_P(64, 32) TB_P(64, 16)
#undef TB_P
    set_error("tb_project_keys: unsupported D=%d dp=%d", D, dp);
    return TB_ERR_UNSUPPORTED_SHAPE;
}

}  // namespace tb
