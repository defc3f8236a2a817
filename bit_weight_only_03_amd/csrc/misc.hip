// misc.hip -- status strings, the dispatch probe string and the read-only
// HBM bandwidth probe.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>

#include "common.h"

using namespace w4k;

namespace {

constexpr int kProbeBlocks = 4096;
constexpr int kProbeThreads = 256;

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];   // 0 = not queried yet

thread_local char g_last_variant[160] = "none";
thread_local char g_last_error[96] = "none";

// Streams `n16` 16-byte words with non-temporal loads and folds them with
// XOR so nothing is elided.  Workgroup b reads its own contiguous share
// [b c, (b + 1) c), c = ceil(n16 / gridDim.x), eight loads in flight per
// thread.  On MI355X (2 GiB read) that order streams at 7.1-7.2 TB/s, while
// a grid-stride order (each pass of the grid over one contiguous window)
// streams at 6.3-6.4 TB/s: the probe measures the better of the two.
__global__ __launch_bounds__(kProbeThreads) void bw_probe_kernel(const u32x4_t* __restrict__ buf,
                                                                 size_t n16, float* __restrict__ sink) {
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t b0 = blockIdx.x * per;
    const size_t e = b0 + per < n16 ? b0 + per : n16;   // <= b0 for workgroups past the end
    const size_t stride = blockDim.x;
    size_t i = b0 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 7 * stride < e; i += 8 * stride) {
        u32x4_t v[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) v[r] = load_nt(buf + i + r * stride);
#pragma unroll
        for (int r = 0; r < 8; ++r) acc ^= v[r][0] ^ v[r][1] ^ v[r][2] ^ v[r][3];
    }
    for (; i < e; i += stride) {
        const u32x4_t v = load_nt(buf + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    __shared__ uint32_t red[kProbeThreads];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t a = 0;
        for (int t = 0; t < kProbeThreads; ++t) a ^= red[t];
        sink[blockIdx.x] = (float)(a & 0xffffu);
    }
}

}  // namespace

namespace w4h {

int cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int n = g_cu_count[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    hipDeviceProp_t prop;
    n = (hipGetDeviceProperties(&prop, dev) == hipSuccess && prop.multiProcessorCount > 0)
            ? prop.multiProcessorCount
            : 256;
    g_cu_count[dev].store(n, std::memory_order_relaxed);   // every racer stores the same value
    return n;
}

const Overrides& overrides() {
    static Overrides o;
    static std::once_flag once;
    std::call_once(once, [] {
        auto geti = [](const char* name, int& v) {
            if (const char* e = getenv(name)) v = atoi(e);
        };
        geti("W4A16_WAVES", o.w4_waves);
        geti("W4A16_SPLIT", o.w4_split);
        geti("W4A16_TPW", o.w4_tpw);
        geti("W4A16_GEMM_MIN_M", o.w4_gemm_min_m);
        geti("W4A16_PX", o.w4_px);
        geti("W4A16_VALU", o.w4_valu);
        geti("W4A16_BAL", o.w4_bal);
        geti("W4A16_GEMM_TN", o.gemm_tn);
        geti("W4A16_GEMM_SPLIT", o.gemm_split);
        geti("W16A16_KSPLIT", o.w16_ksplit);
        geti("W16A16_DOT", o.w16_dot);
        geti("W16A16_BAL", o.w16_bal);
        geti("W16A16_SPLIT", o.w16_split);
        if (const char* e = getenv("W2T_STAGED_LDS_MAX")) o.w2t_staged_lds_max = atoll(e);
    });
    return o;
}

void set_last_variant(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_variant, sizeof g_last_variant, fmt, ap);
    va_end(ap);
}
void set_last_error(const char* what) { snprintf(g_last_error, sizeof g_last_error, "%s", what); }
}  // namespace w4h

extern "C" const char* w4a16_last_variant(void) { return g_last_variant; }

extern "C" const char* w4a16_last_error(void) { return g_last_error; }

extern "C" const char* w4a16_status_string(int status) {
    switch (status) {
        case W4A16_OK: return "ok";
        case W4A16_ERR_NULL: return "a required pointer is NULL";
        case W4A16_ERR_SHAPE: return "M, N, K or group outside the supported contract";
        case W4A16_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
        case W4A16_ERR_DTYPE: return "unknown or disallowed dtype";
        case W4A16_ERR_WORKSPACE: return "workspace smaller than the size query reports";
        case W4A16_ERR_UNSUPPORTED: return "valid request not implemented by this library";
        case W4A16_ERR_HIP: return "HIP runtime error at launch";
        default: return "unknown status";
    }
}

extern "C" int w4a16_bw_probe_sink_floats(void) { return kProbeBlocks; }

extern "C" int w4a16_bw_probe(const void* buf, size_t bytes, float* sink, w4a16_stream_t stream) {
    if (!buf || !sink) return W4A16_ERR_NULL;
    if (bytes == 0 || bytes % 16) return W4A16_ERR_SHAPE;
    if (!w4h::aligned16(buf) || !w4h::aligned16(sink)) return W4A16_ERR_ALIGN;
    w4h::begin_launches();
    hipLaunchKernelGGL(bw_probe_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0,
                       (hipStream_t)stream, (const u32x4_t*)buf, bytes / 16, sink);
    w4h::set_last_variant("bw_probe blocks=%d threads=%d", kProbeBlocks, kProbeThreads);
    return w4h::launch_status();
}
