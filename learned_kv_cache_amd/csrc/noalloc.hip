// tb_sparse_decode_attn without a workspace argument, for callers that cannot
// allocate device memory (code under graph capture that must not call
// hipMalloc, tight serving loops, harnesses that forbid allocation). The
// split partials and arrival counters that tb_sparse_decode_attn keeps in the
// caller's workspace live here in one file-scope device array per GPU, of a
// fixed size; the kernels are the same and take the array's device address
// as they take the workspace.
//
// The array's name is a host-side stand-in in host code, not a device
// address: its address on each device is fetched once with
// hipGetSymbolAddress (the device current) and only that address is passed
// to kernels.
#include <mutex>

#include "tb_common.h"

namespace tb {

// Layout of the array: the per-head arrival counters at a fixed place (so a
// call of any shape finds them where the previous call, of any other shape,
// left them at zero), then the split partials.
constexpr size_t kScratchBytes = (size_t)8 << 20;   // 8 MiB per GPU
constexpr size_t kCtrBytes = (size_t)256 << 10;     // counters of up to 65536 heads
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

struct DevScratch {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
    bool cleared = false;
};
DevScratch g_dev[kMaxDevices];
std::mutex g_clear_mu;

__global__ void clear_words(uint32_t *p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
        p[i] = 0u;
}

}  // namespace
}  // namespace tb

extern "C" tb_status tb_sparse_decode_attn_noalloc(const void *q, const void *k_cache,
                                                   const void *v_cache, const int32_t *idx,
                                                   const int32_t *count, int cap,
                                                   const int32_t *ctx_len, int window, int B,
                                                   int Hq, int Hkv, int Lmax, int D, float scale,
                                                   float *out, void *stream) {
    using namespace tb;
    TB_REQUIRE(q && k_cache && v_cache && idx && count && out, TB_ERR_INVALID_ARGUMENT,
               "tb_sparse_decode_attn_noalloc: null pointer");
    TB_REQUIRE(aligned16(q) && aligned16(k_cache) && aligned16(v_cache) && aligned4(idx) &&
                   aligned4(count) && aligned4(out) && aligned4(ctx_len),
               TB_ERR_INVALID_ARGUMENT, "tb_sparse_decode_attn_noalloc: misaligned pointer");
    TB_REQUIRE(B >= 1 && Hq >= 1 && Hkv >= 1 && Lmax >= 1 && cap >= 1 && window >= 0,
               TB_ERR_INVALID_ARGUMENT, "tb_sparse_decode_attn_noalloc: bad sizes");
    TB_REQUIRE(Hq % Hkv == 0, TB_ERR_INVALID_ARGUMENT,
               "tb_sparse_decode_attn_noalloc: Hq %% Hkv != 0");
    TB_REQUIRE(D == 64 || D == 128, TB_ERR_UNSUPPORTED_SHAPE,
               "tb_sparse_decode_attn_noalloc: D must be 64 or 128");
    TB_REQUIRE((long long)Lmax * D * 2 <= 0x7fffffffLL, TB_ERR_UNSUPPORTED_SHAPE,
               "tb_sparse_decode_attn_noalloc: one head's cache must be below 2 GiB");
    TB_REQUIRE(scale == scale, TB_ERR_INVALID_ARGUMENT,
               "tb_sparse_decode_attn_noalloc: scale is NaN");
    const int win = ctx_len ? window : 0;
    const long long heads = (long long)B * Hq;
    const long long rows = (long long)cap + win;
    TB_REQUIRE(heads <= (long long)(kCtrBytes / 4) && rows <= 0x7fffffffLL, TB_ERR_UNSUPPORTED_SHAPE,
               "tb_sparse_decode_attn_noalloc: %lld heads (at most %zu) or cap + window beyond "
               "INT_MAX (use tb_sparse_decode_attn with a workspace)",
               heads, kCtrBytes / 4);
    const long long part_bytes = heads * attn_nsplit((int)rows) * (D + 2) * (long long)sizeof(float);
    TB_REQUIRE(part_bytes <= (long long)(kScratchBytes - kCtrBytes), TB_ERR_UNSUPPORTED_SHAPE,
               "tb_sparse_decode_attn_noalloc: needs %lld bytes of partials for %lld heads; the "
               "fixed scratch holds %zu bytes (use tb_sparse_decode_attn with a workspace)",
               part_bytes, heads, kScratchBytes - kCtrBytes);
    int dev = 0;
    const hipError_t he = hipGetDevice(&dev);
    TB_REQUIRE(he == hipSuccess, TB_ERR_HIP, "tb_sparse_decode_attn_noalloc: hipGetDevice: %s",
               hipGetErrorString(he));
    TB_REQUIRE(dev >= 0 && dev < kMaxDevices, TB_ERR_UNSUPPORTED_SHAPE,
               "tb_sparse_decode_attn_noalloc: device %d beyond the %d supported", dev,
               kMaxDevices);
    DevScratch &ds = g_dev[dev];
    // once per device, with that device current: the array's address on it
    std::call_once(ds.once, [&ds]() {
        ds.err = hipGetSymbolAddress(&ds.ptr, HIP_SYMBOL(scratch));
    });
    TB_REQUIRE(ds.err == hipSuccess && ds.ptr != nullptr, TB_ERR_HIP,
               "tb_sparse_decode_attn_noalloc: hipGetSymbolAddress: %s",
               hipGetErrorString(ds.err));
    const hipStream_t st = static_cast<hipStream_t>(stream);
    uint32_t *ctr = static_cast<uint32_t *>(ds.ptr);
    float *part = reinterpret_cast<float *>(static_cast<unsigned char *>(ds.ptr) + kCtrBytes);
    {
        // The counters are zero when the code object loads, and every call
        // leaves the counters it used at zero. The first call on a device
        // issued outside a graph capture also clears them with a kernel on
        // its stream, ahead of its own launch.
        std::lock_guard<std::mutex> lk(g_clear_mu);
        if (!ds.cleared) {
            hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
            const hipError_t ce = hipStreamIsCapturing(st, &cs);
            TB_REQUIRE(ce == hipSuccess, TB_ERR_HIP,
                       "tb_sparse_decode_attn_noalloc: hipStreamIsCapturing: %s",
                       hipGetErrorString(ce));
            if (cs == hipStreamCaptureStatusNone) {
                hipLaunchKernelGGL(clear_words, dim3(64), dim3(256), 0, st, ctr,
                                   (int)(kCtrBytes / 4));
                const tb_status e = check_launch("tb_sparse_decode_attn_noalloc(clear)");
                if (e) return e;
                ds.cleared = true;
            }
        }
    }
    return launch_attn(q, k_cache, v_cache, idx, count, cap, ctx_len, win, B, Hq, Hkv, Lmax, D,
                       scale, out, part, ctr, st);
}
