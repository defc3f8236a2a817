// w2t.hip -- ternary 2-bit variant: w = (c - 1) * s, c in {0, 1, 2}, one fp16
// scale per group of k ("NINFER 三元引擎性能调优", markdownregistry page,
// sections 五/六: the ternary engine's small-T linear path, where decode
// arithmetic, not memory, was the 22% gap to the bandwidth ceiling).
//
// Device layout (tiles of 16 columns, units of 256 k):
//   qweight_dev uint32 [Np/16][Kp/256][64 lanes][4 dwords]
//   lane l: column 16t + (l & 15), k-block kc = l >> 4.
//   Dword d of lane l in unit u carries the two 32-k steps j = 2d + h (h = 0, 1);
//   step j covers k = 256u + 32j + 8kc + e, e = 0..7.  Two-bit field p of the
//   dword (bits 2p, 2p+1) holds step h = (p >> 2) & 1, element
//   e = 2(p & 3) + (p >> 3), so masks 0x00030003 << 2i applied to the dword
//   (and to the dword >> 8) give the element pairs of both steps.
//   scales_dev uint16 [Np/16][Kp/group][16]
// Padding holds code 1 (weight 0) and scale +0.
//
// Dequantization: for fp16 activations each pair is (1024 + f*c) in fp16
// (f = 1, 4, 16, 64, 256 by bit position) and one packed fma by 1/f with
// -(1024/f + 1) gives c - 1 exactly; for bf16 activations the pairs are
// 128 + c and a second MFMA against the constant -129 removes the bias.
#include "common.h"

using namespace w4k;

namespace {

constexpr int kMaxWaves = 8;
constexpr int kMaxRows = 16;

__host__ __device__ constexpr int field_step(int p) { return (p >> 2) & 1; }
__host__ __device__ constexpr int field_elem(int p) { return 2 * (p & 3) + (p >> 3); }
__host__ __device__ constexpr int elem_field(int h, int e) { return (e & 1) * 8 + h * 4 + (e >> 1); }

__global__ void w2_pack_q_kernel(const uint32_t* __restrict__ canon, uint32_t* __restrict__ dev,
                                 int N, int K, size_t total) {
    const int U = pad_k2(K) / kUnitK2;
    const int KW = K / 16;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total;
         i += (size_t)gridDim.x * blockDim.x) {
        const int d = (int)(i & 3);
        const int l = (int)((i >> 2) & 63);
        const size_t tu = i >> 8;
        const int u = (int)(tu % U), t = (int)(tu / U);
        const int n = t * kTileN + (l & 15), kc = l >> 4;
        uint32_t out = 0;
#pragma unroll
        for (int p = 0; p < 16; ++p) {
            const int k = u * kUnitK2 + 32 * (2 * d + field_step(p)) + 8 * kc + field_elem(p);
            uint32_t code = 1u;  // padding: weight 0
            if (n < N && k < K) code = (canon[(size_t)n * KW + k / 16] >> (2 * (k % 16))) & 3u;
            out |= code << (2 * p);
        }
        dev[i] = out;
    }
}

__global__ void w2_unpack_q_kernel(const uint32_t* __restrict__ dev, uint32_t* __restrict__ canon,
                                   int N, int K) {
    const int U = pad_k2(K) / kUnitK2;
    const int KW = K / 16;
    const size_t total = (size_t)N * KW;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total;
         i += (size_t)gridDim.x * blockDim.x) {
        const int n = (int)(i / KW), kw = (int)(i % KW);
        const int t = n / kTileN, c = n % kTileN;
        uint32_t word = 0;
        for (int f = 0; f < 16; ++f) {
            const int k = 16 * kw + f;
            const int u = k / kUnitK2, j = (k % kUnitK2) / 32, kc = (k % 32) / 8, e = k % 8;
            const uint32_t dv = dev[(((size_t)t * U + u) * kLanes + (kc * 16 + c)) * 4 + j / 2];
            word |= ((dv >> (2 * elem_field(j & 1, e))) & 3u) << (2 * f);
        }
        canon[i] = word;
    }
}

__global__ void w2_pack_s_kernel(const uint16_t* __restrict__ s_canon, uint16_t* __restrict__ s_dev,
                                 int N, int K, int group) {
    const int G = K / group, Gp = pad_k2(K) / group, T = pad_n(N) / kTileN;
    const size_t total = (size_t)T * Gp * 16;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total;
         i += (size_t)gridDim.x * blockDim.x) {
        const int c = (int)(i & 15);
        const size_t tg = i >> 4;
        const int g = (int)(tg % Gp), t = (int)(tg / Gp);
        const int n = t * kTileN + c;
        s_dev[i] = (n < N && g < G) ? s_canon[(size_t)g * N + n] : (uint16_t)0;
    }
}

__global__ void w2_unpack_s_kernel(const uint16_t* __restrict__ s_dev, uint16_t* __restrict__ s_canon,
                                   int N, int K, int group) {
    const int G = K / group, Gp = pad_k2(K) / group;
    const size_t total = (size_t)G * N;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total;
         i += (size_t)gridDim.x * blockDim.x) {
        const int g = (int)(i / N), n = (int)(i % N);
        s_canon[i] = s_dev[((size_t)(n / kTileN) * Gp + g) * 16 + n % kTileN];
    }
}

__global__ void w2_dequant_kernel(const uint32_t* __restrict__ qdev, const uint16_t* __restrict__ sdev,
                                  float* __restrict__ w, int N, int K, int group) {
    const int U = pad_k2(K) / kUnitK2, Gp = pad_k2(K) / group;
    const size_t total = (size_t)K * N;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total;
         i += (size_t)gridDim.x * blockDim.x) {
        const int k = (int)(i / N), n = (int)(i % N);
        const int t = n / kTileN, c = n % kTileN;
        const int u = k / kUnitK2, j = (k % kUnitK2) / 32, kc = (k % 32) / 8, e = k % 8;
        const uint32_t dv = qdev[(((size_t)t * U + u) * kLanes + (kc * 16 + c)) * 4 + j / 2];
        const int code = (int)((dv >> (2 * elem_field(j & 1, e))) & 3u);
        const float s = f16_bits_to_f32(sdev[((size_t)t * Gp + k / group) * 16 + c]);
        w[i] = (float)(code - 1) * s;
    }
}

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return bitcast<half2_t>(v); }
__device__ __forceinline__ uint32_t as_u(half2_t v) { return bitcast<uint32_t>(v); }

// The two B operands (c - 1 in fp16, exact) of one dword: steps 2d and 2d + 1.
__device__ __forceinline__ void dequant_w2_f16(uint32_t d, half8_t& b0, half8_t& b1) {
    const uint32_t M = 0x64006400u;  // fp16 1024.0
    const uint32_t t = d >> 8;
    const half2_t q0 = as_h2((d & 0x00030003u) | M);  // 1024 + c
    const half2_t q1 = as_h2((d & 0x000C000Cu) | M);  // 1024 + 4c
    const half2_t q2 = as_h2((d & 0x00300030u) | M);  // 1024 + 16c
    const half2_t q3 = as_h2((d & 0x00C000C0u) | M);  // 1024 + 64c
    const half2_t q4 = as_h2((d & 0x03000300u) | M);  // 1024 + 256c
    const half2_t q5 = as_h2((t & 0x000C000Cu) | M);  // 1024 + 4c
    const half2_t q6 = as_h2((t & 0x00300030u) | M);  // 1024 + 16c
    const half2_t q7 = as_h2((t & 0x00C000C0u) | M);  // 1024 + 64c
    const half2_t n1025 = as_h2(0xE401E401u);
    const half2_t r4 = as_h2(0x34003400u), n257 = as_h2(0xDC04DC04u);
    const half2_t r16 = as_h2(0x2C002C00u), n65 = as_h2(0xD410D410u);
    const half2_t r64 = as_h2(0x24002400u), n17 = as_h2(0xCC40CC40u);
    const half2_t r256 = as_h2(0x1C001C00u), n5 = as_h2(0xC500C500u);
    const u32x4_t v0 = {as_u(q0 + n1025), as_u(__builtin_elementwise_fma(q1, r4, n257)),
                        as_u(__builtin_elementwise_fma(q2, r16, n65)),
                        as_u(__builtin_elementwise_fma(q3, r64, n17))};
    const u32x4_t v1 = {as_u(__builtin_elementwise_fma(q4, r256, n5)),
                        as_u(__builtin_elementwise_fma(q5, r4, n257)),
                        as_u(__builtin_elementwise_fma(q6, r16, n65)),
                        as_u(__builtin_elementwise_fma(q7, r64, n17))};
    b0 = bitcast<half8_t>(v0);
    b1 = bitcast<half8_t>(v1);
}

// The two B operands (128 + c in bf16, exact) of one dword.
__device__ __forceinline__ void biased_w2_bf16(uint32_t d, bf16x8_t& b0, bf16x8_t& b1) {
    const uint32_t M = 0x43004300u;  // bf16 128.0
    const u32x4_t v0 = {(d & 0x00030003u) | M, ((d >> 2) & 0x00030003u) | M,
                        ((d >> 4) & 0x00030003u) | M, ((d >> 6) & 0x00030003u) | M};
    const u32x4_t v1 = {((d >> 8) & 0x00030003u) | M, ((d >> 10) & 0x00030003u) | M,
                        ((d >> 12) & 0x00030003u) | M, ((d >> 14) & 0x00030003u) | M};
    b0 = bitcast<bf16x8_t>(v0);
    b1 = bitcast<bf16x8_t>(v1);
}

template <int NG>
struct Slot2 {
    u32x4_t w;
    uint32_t s[NG];
};

// SPG = group / 32 steps per group; a unit has 8 steps (256 k).
template <bool BF16, int SPG, int D>
__global__ __launch_bounds__(512) void w2t_gemv_kernel(const uint16_t* __restrict__ x,
                                                       const u32x4_t* __restrict__ qdev,
                                                       const uint16_t* __restrict__ sdev,
                                                       void* __restrict__ out, int out_dtype, int M,
                                                       int N, int K, int S) {
    static_assert(D % 2 == 0, "x double buffer alternates with the ring index");
    constexpr int NG = SPG >= 8 ? 1 : 8 / SPG;   // groups per unit
    constexpr int SPU = SPG >= 8 ? 8 : SPG;      // steps per group inside one unit
    __shared__ float red[kMaxWaves][kMaxRows][kTileN];

    const int lane = threadIdx.x & 63, nw = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int t = blockIdx.x, split = blockIdx.y;
    const int U = (K + kUnitK2 - 1) / kUnitK2;
    const int Gp = U * kUnitK2 / (SPG * 32);
    const int su0 = (int)((long long)split * U / S);
    const int su1 = (int)((long long)(split + 1) * U / S);
    const int u0 = su0 + wave * (su1 - su0) / nw;
    const int u1 = su0 + (wave + 1) * (su1 - su0) / nw;
    const int c = lane & 15, kc = lane >> 4;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(qdev + (size_t)t * U * kLanes, (uint32_t)U * 1024u);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(sdev + (size_t)t * Gp * kTileN, (uint32_t)Gp * 32u);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
    const uint32_t wlane = (uint32_t)lane * 16u;
    const uint32_t slane = (uint32_t)c * 2u;
    const int xm = c < M ? c : M - 1;   // rows >= M feed output rows that are never stored
    const uint32_t xlane = ((uint32_t)xm * (uint32_t)K + 8u * (uint32_t)kc) * 2u;

    auto load_slot = [&](int u, Slot2<NG>& r) {
        r.w = bitcast<u32x4_t>(__builtin_amdgcn_raw_buffer_load_b128(rw, wlane, u * 1024, kAuxNT));
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
            r.s[gi] = __builtin_amdgcn_raw_buffer_load_b16(rs, slane, ((u * 8) / SPG + gi) * 32, 0);
    };
    auto load_x = [&](int u, u32x4_t (&xa)[8]) {
        const uint32_t off = xlane + (uint32_t)u * (kUnitK2 * 2);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            xa[j] = bitcast<u32x4_t>(__builtin_amdgcn_raw_buffer_load_b128(rx, off + 64u * j, 0, 0));
    };
    auto apply = [&](float4_t& acc, float4_t& total, uint32_t sbits) {
        const float sf = f16_bits_to_f32((uint16_t)sbits);
#pragma unroll
        for (int r = 0; r < 4; ++r) total[r] = __builtin_fmaf(sf, acc[r], total[r]);
        acc = float4_t{0.f, 0.f, 0.f, 0.f};
    };

    float4_t total = {0.f, 0.f, 0.f, 0.f};
    Slot2<NG> ring[D];
    u32x4_t xb[2][8];
#pragma unroll
    for (int i = 0; i < D; ++i)
        if (u0 + i < u1) load_slot(u0 + i, ring[i]);
    if (u0 < u1) load_x(u0, xb[0]);

    for (int ub = u0; ub < u1; ub += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            const int u = ub + i;
            if (u < u1) {
                u32x4_t (&xcur)[8] = xb[i & 1];
                if (u + 1 < u1) load_x(u + 1, xb[(i + 1) & 1]);
                Slot2<NG>& sl = ring[i];
                float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < 8; st += 2) {
                    const uint32_t dw = sl.w[st / 2];
                    if constexpr (!BF16) {
                        half8_t b0, b1;
                        dequant_w2_f16(dw, b0, b1);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<half8_t>(xcur[st]), b0,
                                                                     acc, 0, 0, 0);
                        if ((st + 1) % SPU == 0) apply(acc, total, sl.s[st / SPU]);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<half8_t>(xcur[st + 1]),
                                                                     b1, acc, 0, 0, 0);
                    } else {
                        bf16x8_t b0, b1;
                        biased_w2_bf16(dw, b0, b1);
                        const bf16x8_t bias = bitcast<bf16x8_t>(
                            u32x4_t{0xC301C301u, 0xC301C301u, 0xC301C301u, 0xC301C301u});  // -129
                        const bf16x8_t a0 = bitcast<bf16x8_t>(xcur[st]);
                        const bf16x8_t a1 = bitcast<bf16x8_t>(xcur[st + 1]);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bias, acc, 0, 0, 0);
                        if ((st + 1) % SPU == 0) apply(acc, total, sl.s[st / SPU]);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bias, acc, 0, 0, 0);
                    }
                    if ((st + 2) % SPU == 0) apply(acc, total, sl.s[(st + 1) / SPU]);
                }
                if (u + D < u1) load_slot(u + D, sl);
            }
        }
    }

    const int rb = 4 * kc;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        if (rb + r < M) red[wave][rb + r][c] = total[r];
    __syncthreads();
    for (int idx = threadIdx.x; idx < M * kTileN; idx += blockDim.x) {
        const int mm = idx >> 4, cc = idx & 15;
        float v = 0.f;
        for (int w = 0; w < nw; ++w) v += red[w][mm][cc];
        const int n = t * kTileN + cc;
        if (n < N) {
            const size_t o = (size_t)split * M * N + (size_t)mm * N + n;
            if (out_dtype == W4A16_F32)
                ((float*)out)[o] = v;
            else if (out_dtype == W4A16_F16)
                ((_Float16*)out)[o] = (_Float16)v;
            else
                ((uint16_t*)out)[o] = f32_to_bf16_bits(v);
        }
    }
}

__global__ void w2_merge_kernel(const float* __restrict__ ws, void* __restrict__ y, int out_dtype,
                                int MN, int S) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= MN) return;
    float v = 0.f;
    for (int s = 0; s < S; ++s) v += ws[(size_t)s * MN + i];
    if (out_dtype == W4A16_F32)
        ((float*)y)[i] = v;
    else if (out_dtype == W4A16_F16)
        ((_Float16*)y)[i] = (_Float16)v;
    else
        ((uint16_t*)y)[i] = f32_to_bf16_bits(v);
}

struct Plan2 {
    int waves, split, depth;
};

Plan2 make_plan2(int N, int K) {
    const int U = (K + kUnitK2 - 1) / kUnitK2;
    const int T = pad_n(N) / kTileN;
    Plan2 p;
    p.waves = (U + 1) / 2;  // about two 256-k units per wave
    if (p.waves > kMaxWaves) p.waves = kMaxWaves;
    if (p.waves < 1) p.waves = 1;
    p.split = 1;
    if (T < 256) {
        int s = (512 + T - 1) / T;
        int smax = U / (2 * p.waves);
        if (smax < 1) smax = 1;
        p.split = s < smax ? s : smax;
    }
    p.depth = 4;
    return p;
}

typedef void (*w2_kernel_t)(const uint16_t*, const u32x4_t*, const uint16_t*, void*, int, int, int,
                            int, int);

template <bool BF16>
w2_kernel_t pick2(int group) {
    switch (group) {
        case 32: return w2t_gemv_kernel<BF16, 1, 4>;
        case 64: return w2t_gemv_kernel<BF16, 2, 4>;
        case 128: return w2t_gemv_kernel<BF16, 4, 4>;
        default: return w2t_gemv_kernel<BF16, 8, 4>;
    }
}

inline unsigned grid_for(size_t work, unsigned block) {
    size_t g = (work + block - 1) / block;
    if (g > 65536u * 4) g = 65536u * 4;
    if (g == 0) g = 1;
    return (unsigned)g;
}

}  // namespace

extern "C" int w2t_packed_sizes(int N, int K, int group, size_t* q_bytes, size_t* s_bytes) {
    if (!q_bytes || !s_bytes) return W4A16_ERR_NULL;
    int rc = w4h::check_w2_shape(N, K, group);
    if (rc) return rc;
    const size_t Np = pad_n(N), Kp = pad_k2(K);
    *q_bytes = Np * Kp / 4;
    *s_bytes = Np * (Kp / group) * 2;
    return W4A16_OK;
}

extern "C" int w2t_pack(const int32_t* codes_canon, const uint16_t* scales_canon, void* qweight,
                        void* scales, int N, int K, int group, w4a16_stream_t stream) {
    if (!codes_canon || !scales_canon || !qweight || !scales) return W4A16_ERR_NULL;
    int rc = w4h::check_w2_shape(N, K, group);
    if (rc) return rc;
    if (!w4h::aligned16(codes_canon) || !w4h::aligned16(scales_canon) || !w4h::aligned16(qweight) ||
        !w4h::aligned16(scales))
        return W4A16_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    const size_t qd = (size_t)pad_n(N) * pad_k2(K) / 16;
    w4h::begin_launches();
    hipLaunchKernelGGL(w2_pack_q_kernel, dim3(grid_for(qd, 256)), dim3(256), 0, s,
                       (const uint32_t*)codes_canon, (uint32_t*)qweight, N, K, qd);
    const size_t sd = (size_t)pad_n(N) * (pad_k2(K) / group);
    hipLaunchKernelGGL(w2_pack_s_kernel, dim3(grid_for(sd, 256)), dim3(256), 0, s, scales_canon,
                       (uint16_t*)scales, N, K, group);
    return w4h::launch_status();
}

extern "C" int w2t_unpack(const void* qweight, const void* scales, int32_t* codes_canon,
                          uint16_t* scales_canon, int N, int K, int group, w4a16_stream_t stream) {
    if (!codes_canon || !scales_canon || !qweight || !scales) return W4A16_ERR_NULL;
    int rc = w4h::check_w2_shape(N, K, group);
    if (rc) return rc;
    if (!w4h::aligned16(codes_canon) || !w4h::aligned16(scales_canon) || !w4h::aligned16(qweight) ||
        !w4h::aligned16(scales))
        return W4A16_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    const size_t qc = (size_t)N * (K / 16);
    w4h::begin_launches();
    hipLaunchKernelGGL(w2_unpack_q_kernel, dim3(grid_for(qc, 256)), dim3(256), 0, s,
                       (const uint32_t*)qweight, (uint32_t*)codes_canon, N, K);
    const size_t sc = (size_t)N * (K / group);
    hipLaunchKernelGGL(w2_unpack_s_kernel, dim3(grid_for(sc, 256)), dim3(256), 0, s,
                       (const uint16_t*)scales, scales_canon, N, K, group);
    return w4h::launch_status();
}

extern "C" int w2t_dequant(const void* qweight, const void* scales, float* w, int N, int K, int group,
                           w4a16_stream_t stream) {
    if (!qweight || !scales || !w) return W4A16_ERR_NULL;
    int rc = w4h::check_w2_shape(N, K, group);
    if (rc) return rc;
    if (!w4h::aligned16(qweight) || !w4h::aligned16(scales) || !w4h::aligned16(w))
        return W4A16_ERR_ALIGN;
    const size_t total = (size_t)K * N;
    w4h::begin_launches();
    hipLaunchKernelGGL(w2_dequant_kernel, dim3(grid_for(total, 256)), dim3(256), 0,
                       (hipStream_t)stream, (const uint32_t*)qweight, (const uint16_t*)scales, w, N,
                       K, group);
    return w4h::launch_status();
}

extern "C" int w2t_workspace_bytes(int M, int N, int K, int group, size_t* bytes) {
    if (!bytes) return W4A16_ERR_NULL;
    if (M < 1 || M > kMaxRows) return W4A16_ERR_SHAPE;
    int rc = w4h::check_w2_shape(N, K, group);
    if (rc) return rc;
    const Plan2 p = make_plan2(N, K);
    *bytes = p.split > 1 ? (size_t)p.split * M * N * sizeof(float) : 0;
    return W4A16_OK;
}

extern "C" int w2t_gemv(const void* x, int x_dtype, const void* qweight, const void* scales, void* y,
                        int y_dtype, int M, int N, int K, int group, void* workspace,
                        size_t workspace_bytes, w4a16_stream_t stream) {
    if (!x || !qweight || !scales || !y) return W4A16_ERR_NULL;
    if (x_dtype != W4A16_F16 && x_dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    if (y_dtype != W4A16_F32 && y_dtype != W4A16_F16 && y_dtype != W4A16_BF16)
        return W4A16_ERR_DTYPE;
    if (M < 1 || M > kMaxRows) return W4A16_ERR_SHAPE;
    int rc = w4h::check_w2_shape(N, K, group);
    if (rc) return rc;
    if (!w4h::aligned16(x) || !w4h::aligned16(qweight) || !w4h::aligned16(scales) ||
        !w4h::aligned16(y))
        return W4A16_ERR_ALIGN;
    const Plan2 p = make_plan2(N, K);
    const size_t need = p.split > 1 ? (size_t)p.split * M * N * sizeof(float) : 0;
    if (need) {
        if (!workspace) return W4A16_ERR_NULL;
        if (workspace_bytes < need) return W4A16_ERR_WORKSPACE;
        if (!w4h::aligned16(workspace)) return W4A16_ERR_ALIGN;
    }
    hipStream_t st = (hipStream_t)stream;
    const int T = pad_n(N) / kTileN;
    const bool bf16 = x_dtype == W4A16_BF16;
    w2_kernel_t k = bf16 ? pick2<true>(group) : pick2<false>(group);
    void* out = p.split > 1 ? workspace : y;
    const int odt = p.split > 1 ? W4A16_F32 : y_dtype;
    w4h::begin_launches();
    hipLaunchKernelGGL(k, dim3(T, p.split), dim3(64 * p.waves), 0, st, (const uint16_t*)x,
                       (const u32x4_t*)qweight, (const uint16_t*)scales, out, odt, M, N, K, p.split);
    if (p.split > 1) {
        const int MN = M * N;
        hipLaunchKernelGGL(w2_merge_kernel, dim3((MN + 255) / 256), dim3(256), 0, st,
                           (const float*)workspace, y, y_dtype, MN, p.split);
    }
    w4h::set_last_variant("w2t_mfma16 %s g%d tiles=%d waves=%d split=%d depth=%d",
                          bf16 ? "bf16" : "f16", group, T, p.waves, p.split, p.depth);
    return w4h::launch_status();
}
