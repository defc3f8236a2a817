// w4_pack.hip -- load-time conversion between the canonical 4-bit storage and
// the gfx950 interleaved device layout (see common.h), plus an fp32
// dequantization of the device layout for parity checks.
//
// The Z100 vLLM port article (forum.sourcefind.cn, section 四) moved its
// INT4 repack from many small per-K launches to one 2-D kernel and did the
// [N,K/8] int32 transpose at nibble level instead of through a full int32
// temporary.  Here the canonical layout is already [N][K/8] words and every
// device dword is one canonical word with its nibbles permuted, so the repack
// is one gather-permute-store per 32-bit word and needs no temporary at all.
#include "common.h"

using namespace w4k;

namespace {

// Device nibble position p holds element e = nibble_elem(p) = {0,2,4,6,1,3,5,7}[p];
// elem_pos is the inverse permutation {0,4,1,5,2,6,3,7}.
__host__ __device__ constexpr int nibble_elem(int p) { return 2 * (p & 3) + (p >> 2); }
__host__ __device__ constexpr int elem_pos(int e) { return (e >> 1) + 4 * (e & 1); }

__global__ void w4_pack_q_kernel(const uint32_t* __restrict__ canon, uint32_t* __restrict__ dev,
                                 int N, int K, size_t total_dwords) {
    const int U = pad_k(K) / kUnitK;
    const int KW = K / 8;  // canonical words per column
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total_dwords;
         i += (size_t)gridDim.x * blockDim.x) {
        const int j = (int)(i & 3);
        const int l = (int)((i >> 2) & 63);
        const size_t tu = i >> 8;  // t * U + u
        const int u = (int)(tu % U);
        const int t = (int)(tu / U);
        const int n = t * kTileN + (l & 15);
        const int kw = 16 * u + 4 * j + (l >> 4);
        uint32_t word = 0;
        if (n < N && kw < KW) word = canon[(size_t)n * KW + kw];
        uint32_t out = 0;
#pragma unroll
        for (int p = 0; p < 8; ++p) out |= ((word >> (4 * nibble_elem(p))) & 15u) << (4 * p);
        dev[i] = out;
    }
}

__global__ void w4_unpack_q_kernel(const uint32_t* __restrict__ dev, uint32_t* __restrict__ canon,
                                   int N, int K) {
    const int U = pad_k(K) / kUnitK;
    const int KW = K / 8;
    const size_t total = (size_t)N * KW;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total;
         i += (size_t)gridDim.x * blockDim.x) {
        const int n = (int)(i / KW);
        const int kw = (int)(i % KW);
        const int t = n / kTileN, c = n % kTileN;
        const int u = kw / 16, j = (kw % 16) / 4, kc = kw % 4;
        const uint32_t d = dev[(((size_t)t * U + u) * kLanes + (kc * 16 + c)) * 4 + j];
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) word |= ((d >> (4 * elem_pos(e))) & 15u) << (4 * e);
        canon[i] = word;
    }
}

// Scales [G][N] -> [Np/16][Gp][16]; zeros [G][N/8] words -> [Np/16][Gp][2] words.
__global__ void w4_pack_sz_kernel(const uint16_t* __restrict__ s_canon,
                                  const uint32_t* __restrict__ z_canon, uint16_t* __restrict__ s_dev,
                                  uint32_t* __restrict__ z_dev, int N, int K, int group) {
    const int G = K / group, Gp = pad_k(K) / group, T = pad_n(N) / kTileN;
    const int NZ = N / 8;
    const size_t total = (size_t)T * Gp * 16;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total;
         i += (size_t)gridDim.x * blockDim.x) {
        const int c = (int)(i & 15);
        const size_t tg = i >> 4;
        const int g = (int)(tg % Gp), t = (int)(tg / Gp);
        const int n = t * kTileN + c;
        s_dev[i] = (n < N && g < G) ? s_canon[(size_t)g * N + n] : (uint16_t)0;
        if (c < 2) {
            const int w = 2 * t + c;
            z_dev[tg * 2 + c] = (g < G && w < NZ) ? z_canon[(size_t)g * NZ + w] : 0u;
        }
    }
}

__global__ void w4_unpack_sz_kernel(const uint16_t* __restrict__ s_dev,
                                    const uint32_t* __restrict__ z_dev, uint16_t* __restrict__ s_canon,
                                    uint32_t* __restrict__ z_canon, int N, int K, int group) {
    const int G = K / group, Gp = pad_k(K) / group;
    const int NZ = N / 8;
    const size_t total = (size_t)G * N;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total;
         i += (size_t)gridDim.x * blockDim.x) {
        const int g = (int)(i / N), n = (int)(i % N);
        const int t = n / kTileN, c = n % kTileN;
        s_canon[i] = s_dev[((size_t)t * Gp + g) * 16 + c];
        if (n % 8 == 0) z_canon[(size_t)g * NZ + n / 8] = z_dev[((size_t)t * Gp + g) * 2 + c / 8];
    }
}

// w[k][n] = (q - z) * s in fp32, read through the device layout.
__global__ void w4_dequant_kernel(const uint32_t* __restrict__ qdev, const uint16_t* __restrict__ sdev,
                                  const uint32_t* __restrict__ zdev, float* __restrict__ w, int N,
                                  int K, int group) {
    const int U = pad_k(K) / kUnitK, Gp = pad_k(K) / group;
    const size_t total = (size_t)K * N;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total;
         i += (size_t)gridDim.x * blockDim.x) {
        const int k = (int)(i / N), n = (int)(i % N);
        const int t = n / kTileN, c = n % kTileN;
        const int u = k / kUnitK, j = (k % kUnitK) / 32, kc = (k % 32) / 8, e = k % 8;
        const uint32_t d = qdev[(((size_t)t * U + u) * kLanes + (kc * 16 + c)) * 4 + j];
        const int q = (int)((d >> (4 * elem_pos(e))) & 15u);
        const int g = k / group;
        const size_t tg = (size_t)t * Gp + g;
        const int z = (int)((zdev[tg * 2 + c / 8] >> (4 * (c % 8))) & 15u);
        const float s = f16_bits_to_f32(sdev[tg * 16 + c]);
        w[i] = (float)(q - z) * s;
    }
}

inline unsigned grid_for(size_t work, unsigned block) {
    size_t g = (work + block - 1) / block;
    if (g > 65536u * 4) g = 65536u * 4;
    if (g == 0) g = 1;
    return (unsigned)g;
}

}  // namespace

extern "C" int w4a16_packed_sizes(int N, int K, int group, size_t* q_bytes, size_t* s_bytes,
                                  size_t* z_bytes) {
    if (!q_bytes || !s_bytes || !z_bytes) return W4A16_ERR_NULL;
    int rc = w4h::check_w4_shape(N, K, group);
    if (rc) return rc;
    const size_t Np = pad_n(N), Kp = pad_k(K), Gp = Kp / group;
    *q_bytes = Np * Kp / 2;
    *s_bytes = Np * Gp * 2;
    *z_bytes = Np * Gp / 2;
    return W4A16_OK;
}

extern "C" int w4a16_pack(const int32_t* qweight_canon, const uint16_t* scales_canon,
                          const int32_t* zeros_canon, void* qweight, void* scales, void* zeros,
                          int N, int K, int group, w4a16_stream_t stream) {
    if (!qweight_canon || !scales_canon || !zeros_canon || !qweight || !scales || !zeros)
        return W4A16_ERR_NULL;
    int rc = w4h::check_w4_shape(N, K, group);
    if (rc) return rc;
    if (!w4h::aligned16(qweight_canon) || !w4h::aligned16(scales_canon) ||
        !w4h::aligned16(zeros_canon) || !w4h::aligned16(qweight) || !w4h::aligned16(scales) ||
        !w4h::aligned16(zeros))
        return W4A16_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    const size_t qd = (size_t)pad_n(N) * pad_k(K) / 8;
    w4h::begin_launches();
    hipLaunchKernelGGL(w4_pack_q_kernel, dim3(grid_for(qd, 256)), dim3(256), 0, s,
                       (const uint32_t*)qweight_canon, (uint32_t*)qweight, N, K, qd);
    const size_t sd = (size_t)pad_n(N) * (pad_k(K) / group);
    hipLaunchKernelGGL(w4_pack_sz_kernel, dim3(grid_for(sd, 256)), dim3(256), 0, s, scales_canon,
                       (const uint32_t*)zeros_canon, (uint16_t*)scales, (uint32_t*)zeros, N, K,
                       group);
    return w4h::launch_status();
}

extern "C" int w4a16_unpack(const void* qweight, const void* scales, const void* zeros,
                            int32_t* qweight_canon, uint16_t* scales_canon, int32_t* zeros_canon,
                            int N, int K, int group, w4a16_stream_t stream) {
    if (!qweight_canon || !scales_canon || !zeros_canon || !qweight || !scales || !zeros)
        return W4A16_ERR_NULL;
    int rc = w4h::check_w4_shape(N, K, group);
    if (rc) return rc;
    if (!w4h::aligned16(qweight_canon) || !w4h::aligned16(scales_canon) ||
        !w4h::aligned16(zeros_canon) || !w4h::aligned16(qweight) || !w4h::aligned16(scales) ||
        !w4h::aligned16(zeros))
        return W4A16_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    const size_t qc = (size_t)N * (K / 8);
    w4h::begin_launches();
    hipLaunchKernelGGL(w4_unpack_q_kernel, dim3(grid_for(qc, 256)), dim3(256), 0, s,
                       (const uint32_t*)qweight, (uint32_t*)qweight_canon, N, K);
    const size_t sc = (size_t)N * (K / group);
    hipLaunchKernelGGL(w4_unpack_sz_kernel, dim3(grid_for(sc, 256)), dim3(256), 0, s,
                       (const uint16_t*)scales, (const uint32_t*)zeros, scales_canon,
                       (uint32_t*)zeros_canon, N, K, group);
    return w4h::launch_status();
}

extern "C" int w4a16_dequant(const void* qweight, const void* scales, const void* zeros, float* w,
                             int N, int K, int group, w4a16_stream_t stream) {
    if (!qweight || !scales || !zeros || !w) return W4A16_ERR_NULL;
    int rc = w4h::check_w4_shape(N, K, group);
    if (rc) return rc;
    if (!w4h::aligned16(qweight) || !w4h::aligned16(scales) || !w4h::aligned16(zeros) ||
        !w4h::aligned16(w))
        return W4A16_ERR_ALIGN;
    const size_t total = (size_t)K * N;
    w4h::begin_launches();
    hipLaunchKernelGGL(w4_dequant_kernel, dim3(grid_for(total, 256)), dim3(256), 0,
                       (hipStream_t)stream, (const uint32_t*)qweight, (const uint16_t*)scales,
                       (const uint32_t*)zeros, w, N, K, group);
    return w4h::launch_status();
}
