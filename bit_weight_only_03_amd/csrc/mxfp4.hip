// mxfp4.hip -- load-time conversion between the canonical MXFP4 storage and
// the gfx950 device layout, and an fp32 dequantization through the device
// layout for parity checks.
//
// MXFP4 is the weight format the Z100 vLLM port article's closing section
// names next: 4-bit floating-point (E2M1) elements that share one block-level
// scale, as defined by the OCP Microscaling (MX) specification it cites --
// blocks of 32 elements along K, an E8M0 scale 2^(E - 127) per block.
//
// Canonical (the boundary's input): qweight uint8 [N][K/2], element k of row
// n in byte k/2, low nibble for even k; scales uint8 [N][K/32].
//
// Device layout, per 16-column tile t and 128-k unit u (the 4-bit GEMV's):
//   qweight: [T][U][64 lanes][4 dwords]; lane l = c + 16 kc (column
//            n = 16 t + c), dword j holds the 8 codes k = 128 u + 32 j + 8 kc
//            + e, e = 0..7, code e in bits 4e..4e+3.  This is exactly the
//            canonical dword 16 u + 4 j + kc of row n, so the pack is a pure
//            gather.  Dword j is the B operand of the unit's MFMA step j,
//            and step j covers one whole MX block.
//   scales:  [T][U][16 columns] dwords; byte j of dword (t, u, c) is the E8M0
//            code of block 4 u + j of column n.  One 4-byte load per lane and
//            unit brings the scales of its four steps.
// Padding (columns past N, blocks past K) holds code 0 (element 0, scale
// 2^-127), so padded products are exactly 0.
#include "common.h"

using namespace w4k;

namespace {

__global__ void mx_pack_q_kernel(const uint32_t* __restrict__ canon, uint32_t* __restrict__ dev,
                                 int N, int K, size_t total_dwords) {
    const int U = pad_k(K) / kUnitK;
    const int KW = K / 8;   // canonical dwords per row
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total_dwords;
         i += (size_t)gridDim.x * blockDim.x) {
        const int j = (int)(i & 3);
        const int l = (int)((i >> 2) & 63);
        const size_t tu = i >> 8;   // t * U + u
        const int u = (int)(tu % U), t = (int)(tu / U);
        const int n = t * kTileN + (l & 15);
        const int kw = 16 * u + 4 * j + (l >> 4);
        dev[i] = (n < N && kw < KW) ? canon[(size_t)n * KW + kw] : 0u;
    }
}

__global__ void mx_unpack_q_kernel(const uint32_t* __restrict__ dev, uint32_t* __restrict__ canon,
                                   int N, int K) {
    const int U = pad_k(K) / kUnitK;
    const int KW = K / 8;
    const size_t total = (size_t)N * KW;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total;
         i += (size_t)gridDim.x * blockDim.x) {
        const int n = (int)(i / KW), kw = (int)(i % KW);
        const int t = n / kTileN, c = n % kTileN;
        const int u = kw / 16, j = (kw % 16) / 4, kc = kw % 4;
        canon[i] = dev[(((size_t)t * U + u) * kLanes + (kc * 16 + c)) * 4 + j];
    }
}

// scales [N][K/32] bytes -> [T][U][16] dwords.
__global__ void mx_pack_s_kernel(const uint8_t* __restrict__ canon, uint32_t* __restrict__ dev, int N,
                                 int K, size_t total_dwords) {
    const int U = pad_k(K) / kUnitK;
    const int KB = K / 32;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total_dwords;
         i += (size_t)gridDim.x * blockDim.x) {
        const int c = (int)(i & 15);
        const size_t tu = i >> 4;
        const int u = (int)(tu % U), t = (int)(tu / U);
        const int n = t * kTileN + c;
        uint32_t d = 0;
        if (n < N) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int b = 4 * u + j;
                if (b < KB) d |= (uint32_t)canon[(size_t)n * KB + b] << (8 * j);
            }
        }
        dev[i] = d;
    }
}

__global__ void mx_unpack_s_kernel(const uint8_t* __restrict__ dev, uint8_t* __restrict__ canon, int N,
                                   int K) {
    const int U = pad_k(K) / kUnitK;
    const int KB = K / 32;
    const size_t total = (size_t)N * KB;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total;
         i += (size_t)gridDim.x * blockDim.x) {
        const int n = (int)(i / KB), b = (int)(i % KB);
        const int t = n / kTileN, c = n % kTileN;
        canon[i] = dev[(((size_t)t * U + b / 4) * kTileN + c) * 4 + (b % 4)];
    }
}

// w[n][k] = element * 2^(E - 127) in fp32, [N][K], read through the device
// layout with the GEMV's own element conversion: one thread per 8 elements.
__global__ void mx_dequant_kernel(const uint32_t* __restrict__ qdev, const uint32_t* __restrict__ sdev,
                                  float* __restrict__ w, int N, int K) {
    const int U = pad_k(K) / kUnitK;
    const int KW = K / 8;
    const size_t total = (size_t)N * KW;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total;
         i += (size_t)gridDim.x * blockDim.x) {
        const int n = (int)(i / KW), kw = (int)(i % KW);
        const int t = n / kTileN, c = n % kTileN;
        const int u = kw / 16, j = (kw % 16) / 4, kc = kw % 4;
        const uint32_t d = qdev[(((size_t)t * U + u) * kLanes + (kc * 16 + c)) * 4 + j];
        const uint32_t e = (sdev[((size_t)t * U + u) * kTileN + c] >> (8 * j)) & 255u;
        const float sf = e8m0_to_f32(e);
        const half8_t v = fp4x8_to_f16(d, 1.0f);
        float* out = w + (size_t)n * K + 8 * kw;
#pragma unroll
        for (int q = 0; q < 8; ++q) out[q] = (float)v[q] * sf;
    }
}

inline unsigned grid_for(size_t work, unsigned block) {
    size_t g = (work + block - 1) / block;
    if (g > 65536u * 4) g = 65536u * 4;
    if (g == 0) g = 1;
    return (unsigned)g;
}

}  // namespace

extern "C" int mxfp4_packed_sizes(int N, int K, size_t* q_bytes, size_t* s_bytes) {
    if (!q_bytes || !s_bytes) return W4A16_ERR_NULL;
    if (int rc = w4h::check_mx_shape(N, K)) return rc;
    const size_t Np = pad_n(N), Kp = pad_k(K);
    *q_bytes = Np * Kp / 2;
    *s_bytes = Np * Kp / 32;
    return W4A16_OK;
}

extern "C" int mxfp4_pack(const uint8_t* qweight_canon, const uint8_t* scales_canon, void* qweight,
                          void* scales, int N, int K, w4a16_stream_t stream) {
    if (!qweight_canon || !scales_canon || !qweight || !scales) return W4A16_ERR_NULL;
    if (int rc = w4h::check_mx_shape(N, K)) return rc;
    if (!w4h::aligned16(qweight_canon) || !w4h::aligned16(qweight) || !w4h::aligned16(scales))
        return W4A16_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    const size_t qd = (size_t)pad_n(N) * pad_k(K) / 8;
    const size_t sd = (size_t)pad_n(N) * (pad_k(K) / kUnitK);
    w4h::begin_launches();
    hipLaunchKernelGGL(mx_pack_q_kernel, dim3(grid_for(qd, 256)), dim3(256), 0, s,
                       (const uint32_t*)qweight_canon, (uint32_t*)qweight, N, K, qd);
    hipLaunchKernelGGL(mx_pack_s_kernel, dim3(grid_for(sd, 256)), dim3(256), 0, s, scales_canon,
                       (uint32_t*)scales, N, K, sd);
    return w4h::launch_status();
}

extern "C" int mxfp4_unpack(const void* qweight, const void* scales, uint8_t* qweight_canon,
                            uint8_t* scales_canon, int N, int K, w4a16_stream_t stream) {
    if (!qweight_canon || !scales_canon || !qweight || !scales) return W4A16_ERR_NULL;
    if (int rc = w4h::check_mx_shape(N, K)) return rc;
    if (!w4h::aligned16(qweight_canon) || !w4h::aligned16(qweight) || !w4h::aligned16(scales))
        return W4A16_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    const size_t qc = (size_t)N * (K / 8), sc = (size_t)N * (K / 32);
    w4h::begin_launches();
    hipLaunchKernelGGL(mx_unpack_q_kernel, dim3(grid_for(qc, 256)), dim3(256), 0, s,
                       (const uint32_t*)qweight, (uint32_t*)qweight_canon, N, K);
    hipLaunchKernelGGL(mx_unpack_s_kernel, dim3(grid_for(sc, 256)), dim3(256), 0, s,
                       (const uint8_t*)scales, scales_canon, N, K);
    return w4h::launch_status();
}

extern "C" int mxfp4_dequant(const void* qweight, const void* scales, float* w, int N, int K,
                             w4a16_stream_t stream) {
    if (!qweight || !scales || !w) return W4A16_ERR_NULL;
    if (int rc = w4h::check_mx_shape(N, K)) return rc;
    if (!w4h::aligned16(qweight) || !w4h::aligned16(scales) || !w4h::aligned16(w))
        return W4A16_ERR_ALIGN;
    const size_t total = (size_t)N * (K / 8);
    w4h::begin_launches();
    hipLaunchKernelGGL(mx_dequant_kernel, dim3(grid_for(total, 256)), dim3(256), 0,
                       (hipStream_t)stream, (const uint32_t*)qweight, (const uint32_t*)scales, w, N,
                       K);
    return w4h::launch_status();
}
