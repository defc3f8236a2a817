// w2t.hip -- ternary 2-bit variant: w = (c - 1) * s, c in {0, 1, 2}, one fp16
// scale per group of k ("NINFER 三元引擎性能调优", markdownregistry page,
// sections 五/六: the ternary engine's small-T linear path, where decode
// arithmetic, not memory, was the 22% gap to the bandwidth ceiling).
//
// Device layout (tiles of 16 columns, units of 256 k):
//   qweight_dev uint32 [Np/16][Kp/256][64 lanes][4 dwords]
//   lane l: column 16t + (l & 15), k-block kc = l >> 4.
//   Dword d of lane l in unit u carries the two 32-k steps j = 2d + h (h = 0, 1);
//   step j covers k = 256u + 32j + 8kc + e, e = 0..7.  The weight w = c - 1
//   of (h, e) is two bits: "nonzero" at bit 4e + 1 - h and "negative" at bit
//   4e + 3 - h.  So d & 0xAAAAAAAA (step h = 0) and (d << 1) & 0xAAAAAAAA
//   (step h = 1) hold, per nibble e, the FP4 E2M1 code of w itself -- sign
//   bit and the low exponent bit, 1.0 or 0 -- and gfx950's
//   v_cvt_scalef32_pk_{f16,bf16}_fp4 turns each byte into the element pair
//   (2i, 2i + 1) of the MFMA B operand: -1, 0, +1 exactly, no bias term.
//   scales_dev uint16 [Np/16][Kp/group][16]
// Padding holds zero bits (weight 0) and scale +0.
#include <stdlib.h>

#include <mutex>

#include "common.h"

using namespace w4k;

namespace {

constexpr int kMaxRows = 16;
constexpr int kWaves2 = 8;       // waves per workgroup of the staged ternary kernel
constexpr int kMaxXLoads2 = 16;  // x load instructions per wave: M * 32 UPW <= 64 * 16

// Bits of the weight of step h (0, 1), element e (0..7) in its device dword.
__host__ __device__ constexpr int nz_bit(int h, int e) { return 4 * e + 1 - h; }
__host__ __device__ constexpr int neg_bit(int h, int e) { return 4 * e + 3 - h; }
// Canonical code c (0, 1, 2 = weight -1, 0, +1) <-> the device bit pair.
__host__ __device__ inline uint32_t w2_bits(uint32_t c, int h, int e) {
    return (uint32_t)(c != 1u) << nz_bit(h, e) | (uint32_t)(c == 0u) << neg_bit(h, e);
}
__host__ __device__ inline uint32_t w2_code(uint32_t dv, int h, int e) {
    return ((dv >> nz_bit(h, e)) & 1u) ? (((dv >> neg_bit(h, e)) & 1u) ? 0u : 2u) : 1u;
}

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
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int k = u * kUnitK2 + 32 * (2 * d + h) + 8 * kc + e;
                uint32_t code = 1u;  // padding: weight 0
                if (n < N && k < K) code = (canon[(size_t)n * KW + k / 16] >> (2 * (k % 16))) & 3u;
                out |= w2_bits(code, h, e);
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
            word |= w2_code(dv, j & 1, e) << (2 * f);
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
        const int code = (int)w2_code(dv, j & 1, e);
        const float s = f16_bits_to_f32(sdev[((size_t)t * Gp + k / group) * 16 + c]);
        w[i] = (float)(code - 1) * s;
    }
}


// The two B operands (the weights -1, 0, +1, exact) of one device dword:
// steps 2d (nibbles of d & 0xAAAAAAAA) and 2d + 1 (of (d << 1) & 0xAAAAAAAA).
template <bool BF16>
__device__ __forceinline__ void w2_operands(uint32_t d, u32x4_t& b0, u32x4_t& b1) {
    const uint32_t lo = d & 0xAAAAAAAAu, hi = (d << 1) & 0xAAAAAAAAu;
    if constexpr (BF16) {
        b0 = bitcast<u32x4_t>(fp4x8_to_bf16(lo, 1.0f));
        b1 = bitcast<u32x4_t>(fp4x8_to_bf16(hi, 1.0f));
    } else {
        b0 = bitcast<u32x4_t>(fp4x8_to_f16(lo, 1.0f));
        b1 = bitcast<u32x4_t>(fp4x8_to_f16(hi, 1.0f));
    }
}

// One ring slot: a unit's 16 weight bytes for this lane plus the scales of
// the groups the unit covers.
template <int NG>
struct Slot2 {
    u32x4_t w;
    uint32_t s[NG];
};

// Launch description shared by host and kernel.
struct W2Launch {
    int M, N, K;
    int U;        // 256-k units per column (K rounded up)
    int S;        // K slices: workgroups (t, s) cover units [s*U/S, (s+1)*U/S) of tile t
    int out_dtype;
};

// Register-ring depth by group size (more groups per unit = more scale words
// per slot).  At g >= 128, 4 slots rather than 6: the ternary down shape (K =
// 17408, N = 5120, 9-unit chains) went from 10.52-10.54 to 10.30-10.32 us at
// M = 1 (graphs of 16 distinct matrices), the other shapes within noise; 3
// slots measured no better.
template <int SPG>
constexpr int max_slots2() { return SPG >= 4 ? 4 : (SPG == 2 ? 5 : 3); }

// Eight waves per SIMD (at most 64 VGPRs) where the chain is short enough.
template <int SPG, int UPW>
constexpr int min_waves2() { return SPG >= 4 && UPW <= 4 ? 8 : 1; }

// The ternary GEMV has the same structure as the 4-bit one: one workgroup per
// (16-column tile, K slice), W waves splitting the slice's 256-k units into
// contiguous ranges of at most UPW units; each wave stages its own x range in
// its own LDS region (straight into LDS), issues the weight and scale loads of its units up front
// (or D of them and one refill per consumed slot, straight-line), and
// dequantizes and multiplies each unit as its slot arrives; the waves then add
// their partial sums through LDS in wave order.
//
// A wave's missing units load as zeros (code 0 and scale +0): the group sums
// they feed are multiplied by a zero scale and add exactly 0, so the
// arithmetic runs unconditionally and each wait covers one slot.
//
// TPW > 1 (layers of many tiles): the workgroup takes TPW consecutive tiles
// and each wave's chain runs unit-major over them, position q = unit q / TPW
// of tile q % TPW, so the workgroup stages x once for all of them (the
// 4-bit kernel's three-tile workgroups, for the same reason).
template <bool BF16, int SPG, int UPW, int TPW = 1>
__global__ __launch_bounds__(512, (TPW > 1 ? 4 : min_waves2<SPG, UPW>())) void w2t_gemv_kernel(
    int M_, int N_, int K_, int U_, int S_,
    const uint16_t* __restrict__ x, const u32x4_t* __restrict__ qdev,
    const uint16_t* __restrict__ sdev, void* __restrict__ out, W2Launch a_in) {
    // The fields a wave needs first arrive as leading scalars (with the
    // pointers: nine arguments, 14 dwords), which the build compiles as
    // preloaded into SGPRs at wave launch; out_dtype stays in the struct.
    const W2Launch a{M_, N_, K_, U_, S_, a_in.out_dtype};
    constexpr int NG = SPG >= 8 ? 1 : 8 / SPG;   // groups per unit
    constexpr int SPU = SPG >= 8 ? 8 : SPG;      // 32-k steps per group inside one unit
    static_assert(TPW >= 1 && TPW <= 3, "one to three tiles per workgroup");
    constexpr int L = UPW * TPW;                 // chain positions
    constexpr int D = L < max_slots2<SPG>() ? L : max_slots2<SPG>();
    // Unconditional arithmetic where the register budget allows (see below).
    constexpr bool kUncond = SPG >= 4 || UPW <= 2;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int M = a.M, K = a.K, U = a.U;
    constexpr int W = kWaves2;                                         // waves per workgroup
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int t0 = blockIdx.x * TPW, split = blockIdx.y;
    const int T = (a.N + kTileN - 1) >> 4;                           // 16-column tiles
    const int nt = T - t0 < TPW ? T - t0 : TPW;                      // tiles of this workgroup
    // Unsplit launches take the slice without a runtime division (it sits
    // between a wave's start and its first load).
    int r0 = 0, r1 = U;
    if (a.S != 1) {
        r0 = split * U / a.S;
        r1 = (split + 1) * U / a.S;
    }
    const int w0 = r0 + wave * (r1 - r0) / W, w1 = r0 + (wave + 1) * (r1 - r0) / W;
    const int nu = w1 - w0;                                           // units of this wave
    const int Gp = U * kUnitK2 / (SPG * 32);
    const int c = lane & 15, kc = lane >> 4;

    // LDS: the slice's x, M x (r1 - r0) units of 512 bytes, split into one
    // region per wave: wave w's [M][nu units] at M * 512 * (w0 - r0) bytes,
    // rows nu * 512 bytes apart, so a workgroup takes exactly M x K-slice x
    // 2 bytes.  Inside each unit of row m, the 16-byte chunk p sits at
    // position p ^ (m % 4): rows a multiple of 256 bytes apart would
    // otherwise share LDS banks (rows m and m + 4 still share one: a
    // two-way conflict at M = 5..8), and the 32-k step keeps one offset
    // for every lane.  Once its products are done, a wave with units reuses
    // its own region for its partial sums (M x 16 floats <= M x 512 bytes).
    const int xrow_bytes = nu * (kUnitK2 * 2);
    uint8_t* const xsb = smem + (size_t)M * (kUnitK2 * 2) * (w0 - r0);

    // 1) x range -> this wave's LDS region, straight from memory into LDS in
    //    one round trip (the 4-bit kernel's scheme: lane l of load i fills
    //    position 64 i + l of the region with the chunk the swizzle puts
    //    there; chunks past K zeroed).  These are the wave's first memory
    //    accesses; where its arithmetic is unconditional it waits for them
    //    after issuing its weight ring, so the round trips overlap.
    {
        const int cpr = nu * (kUnitK2 / 8);          // chunks of a row
        const int xch = M * cpr;
        const uint32_t xbytes = (uint32_t)M * (uint32_t)K * 2u;
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, xbytes);
        // ci -> (row, position): one row needs no division (a division sits
        // on the way to the wave's first load).
        auto stage = [&](auto row_of) {
#pragma unroll
            for (int i = 0; i < kMaxXLoads2; ++i) {
                if (i * 64 < xch) {                    // wave-uniform (false for a wave without units)
                    const int ci = i * 64 + lane;
                    const int m = row_of(ci), pc = ci - m * cpr;
                    const int lc = pc ^ (m & 3);       // same unit and step as pc
                    const int kg = w0 * kUnitK2 + lc * 8;
                    if (m < M) {
                        if (kg < K)
                            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                                rx, (__attribute__((address_space(3))) void*)(xsb + i * 1024), 16,
                                (uint32_t)(m * K + kg) * 2u, 0, 0, 0);
                        else
                            *(u32x4_t*)(xsb + (uint32_t)ci * 16u) = u32x4_t{0u, 0u, 0u, 0u};
                    }
                }
            }
        };
        if (M == 1)
            stage([](int) { return 0; });
        else
            stage([&](int ci) { return ci / cpr; });
        if constexpr (!kUncond) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2) Weight and scale loads of this wave's units.
    // The workgroup's nt tiles are contiguous in both arrays.
    const uint32_t wend = (uint32_t)nt * U * 1024u, send = (uint32_t)nt * Gp * 32u;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(qdev + (size_t)t0 * U * kLanes, wend);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(sdev + (size_t)t0 * Gp * kTileN, send);
    const uint32_t wlane = (uint32_t)lane * 16u;
    const uint32_t slane = (uint32_t)c * 2u;

    auto load_slot = [&](int q, Slot2<NG>& r) {   // unit w0 + q / TPW of tile t0 + q % TPW
        const int i = q / TPW, j = q % TPW;
        const bool valid = i < nu && j < nt;
        const int u = w0 + i;
        r.w = bitcast<u32x4_t>(__builtin_amdgcn_raw_buffer_load_b128(
            rw, valid ? wlane + (uint32_t)(j * U + u) * 1024u : wend, 0, kAuxNT));
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
            r.s[gi] = __builtin_amdgcn_raw_buffer_load_b16(
                rs, valid ? slane + (uint32_t)(j * Gp + u * NG + gi) * 32u : send, 0, 0);
    };

    Slot2<NG> ring[D];
#pragma unroll
    for (int i = 0; i < D; ++i) {
        load_slot(i, ring[i]);
        __builtin_amdgcn_sched_barrier(0);   // slots issue in ring order
    }
    // Loads complete in issue order: with at most the ring's D * (1 + NG)
    // loads outstanding, the x loads issued before them have landed -- as
    // long as every ring load is issued here, which holds only where the
    // arithmetic is unconditional (as in the 4-bit kernel).
    if constexpr (kUncond) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(D * (1 + NG)) : "memory");
    __builtin_amdgcn_sched_barrier(0);

    // 3) Dequantize and multiply, unit by unit, two 32-k steps per dword.
    const bool xrow = c < M;                                    // lane supplies x row c
    // Step st of unit i: chunk 4 st + kc of row c, at position 4 st + (kc ^ c % 4).
    const uint8_t* xlane = xsb + (uint32_t)(c * xrow_bytes) + 16u * (uint32_t)(kc ^ (c & 3));
    float4_t total[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) total[j] = float4_t{0.f, 0.f, 0.f, 0.f};
    u32x4_t xa[2] = {};
#pragma unroll
    for (int q = 0; q < L; ++q) {
        const int i = q / TPW, tj = q % TPW;
        Slot2<NG>& sl = ring[q % D];
        if (kUncond || (i < nu && tj < nt)) {
            float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dd = 0; dd < 4; ++dd) {
                if (i < nu && xrow) {
                    xa[0] = *(const u32x4_t*)(xlane + (uint32_t)i * (kUnitK2 * 2) + 128 * dd);
                    xa[1] = *(const u32x4_t*)(xlane + (uint32_t)i * (kUnitK2 * 2) + 128 * dd + 64);
                }
                // The dword's two steps as B operands.
                u32x4_t bw[2];
                w2_operands<BF16>(sl.w[dd], bw[0], bw[1]);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int st = 2 * dd + h;
                    if constexpr (!BF16) {
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            bitcast<half8_t>(xa[h]), bitcast<half8_t>(bw[h]), acc, 0, 0, 0);
                    } else {
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            bitcast<bf16x8_t>(xa[h]), bitcast<bf16x8_t>(bw[h]), acc, 0, 0, 0);
                    }
                    if ((st + 1) % SPU == 0) {    // group complete: scale once, in fp32
                        const float sf = f16_bits_to_f32((uint16_t)sl.s[st / SPU]);
                        total[tj][0] = __builtin_fmaf(sf, acc[0], total[tj][0]);
                        total[tj][1] = __builtin_fmaf(sf, acc[1], total[tj][1]);
                        total[tj][2] = __builtin_fmaf(sf, acc[2], total[tj][2]);
                        total[tj][3] = __builtin_fmaf(sf, acc[3], total[tj][3]);
                        acc = float4_t{0.f, 0.f, 0.f, 0.f};
                    }
                }
            }
        }
        if (q + D < L) {                   // fixed refill schedule: position q + D into this slot
            __builtin_amdgcn_sched_barrier(0);
            load_slot(q + D, sl);
        }
        __builtin_amdgcn_sched_barrier(0);   // units in order: each waits for its own slot only
    }

    // 4) Wave partials [TPW][M][16] -> the start of each wave's own x region
    //    (TPW M 64 <= M 512 bytes; its last x reads were consumed above, and
    //    a wave's LDS accesses complete in order), then TPW x M x 16 threads
    //    add them in wave order.  A wave without units has no region; its
    //    partial is exactly +0, and skipping it leaves the sum unchanged (the
    //    sum starts at +0 and so is never -0).
    float* const red = (float*)xsb;
    if (nu > 0) {
#pragma unroll
        for (int j = 0; j < TPW; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * kc + r;
                if (m < M) red[(j * M + m) * kTileN + c] = total[j][r];
            }
    }
    __syncthreads();
    const int sl = r1 - r0;
    for (int idx = threadIdx.x; idx < TPW * M * kTileN; idx += blockDim.x) {
        // idx = (tj M + m) 16 + cc, which is also this output's float in a
        // wave's partials (no division by M on this path: tj found by
        // comparison, TPW <= 3).
        const int cc = idx & 15, tm = idx >> 4;
        int tj = 0;
        if constexpr (TPW > 1) tj = (tm >= M) + (tm >= 2 * M);
        const int m = tm - tj * M;
        const int po = idx;
        // All partials are read before the first add, then added in wave order.
        float v = 0.f;
        if (W == kWaves2) {
            float pw[kWaves2];
#pragma unroll
            for (int w = 0; w < kWaves2; ++w) {
                const int b = w * sl / kWaves2, e = (w + 1) * sl / kWaves2;
                pw[w] = e > b ? ((const float*)(smem + (size_t)M * (kUnitK2 * 2) * b))[po] : 0.f;
            }
#pragma unroll
            for (int w = 0; w < kWaves2; ++w)
                if ((w + 1) * sl / kWaves2 > w * sl / kWaves2) v += pw[w];
        } else {
            for (int w = 0; w < W; ++w) {
                const int b = w * sl / W, e = (w + 1) * sl / W;
                if (e > b) v += ((const float*)(smem + (size_t)M * (kUnitK2 * 2) * b))[po];
            }
        }
        const int n = (t0 + tj) * kTileN + cc;
        if (tj < nt && n < a.N) {
            const size_t o = (size_t)split * M * a.N + (size_t)m * a.N + n;
            if (a.out_dtype == W4A16_F32)
                ((float*)out)[o] = v;
            else if (a.out_dtype == W4A16_F16)
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

// ------------------------------------------------- direct-x variant (larger M)
//
// The staged kernel above keeps M x (K slice) x 2 bytes of x in LDS per
// workgroup, and past 8 rows its slices get too short to keep each wave's
// ring busy.  This variant reads each unit's x fragment for the lane's row
// straight from L2 into registers, double-buffered one unit ahead, and keeps
// a four-deep weight ring; it needs no LDS for x.

constexpr int kMaxWavesX = 8;

template <int NG>
struct SlotX {
    u32x4_t w;
    uint32_t s[NG];
};

// SPG = group / 32 steps per group; a unit has 8 steps (256 k).
template <bool BF16, int SPG, int D>
__global__ __launch_bounds__(512) void w2t_gemv_direct_kernel(int M, int N, int K, int S, int nw,
                                                       const uint16_t* __restrict__ x,
                                                       const u32x4_t* __restrict__ qdev,
                                                       const uint16_t* __restrict__ sdev,
                                                       void* __restrict__ out, int out_dtype) {
    static_assert(D % 2 == 0, "x double buffer alternates with the ring index");
    constexpr int NG = SPG >= 8 ? 1 : 8 / SPG;   // groups per unit
    constexpr int SPU = SPG >= 8 ? 8 : SPG;      // steps per group inside one unit
    __shared__ float red[kMaxWavesX][kMaxRows][kTileN];

    const int lane = threadIdx.x & 63;   // nw: waves per workgroup (an argument, preloaded)
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

    auto load_slot = [&](int u, SlotX<NG>& r) {
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
    SlotX<NG> ring[D];
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
                SlotX<NG>& sl = ring[i];
                float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < 8; st += 2) {
                    u32x4_t b0, b1;
                    w2_operands<BF16>(sl.w[st / 2], b0, b1);
                    if constexpr (!BF16) {
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<half8_t>(xcur[st]),
                                                                     bitcast<half8_t>(b0), acc, 0, 0, 0);
                        if ((st + 1) % SPU == 0) apply(acc, total, sl.s[st / SPU]);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<half8_t>(xcur[st + 1]),
                                                                     bitcast<half8_t>(b1), acc, 0, 0, 0);
                    } else {
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8_t>(xcur[st]),
                                                                      bitcast<bf16x8_t>(b0), acc, 0, 0, 0);
                        if ((st + 1) % SPU == 0) apply(acc, total, sl.s[st / SPU]);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8_t>(xcur[st + 1]),
                                                                      bitcast<bf16x8_t>(b1), acc, 0, 0, 0);
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

struct PlanX {
    int waves, split, depth;
};

PlanX make_planx(int N, int K) {
    const int U = (K + kUnitK2 - 1) / kUnitK2;
    const int T = pad_n(N) / kTileN;
    PlanX p;
    p.waves = (U + 1) / 2;  // about two 256-k units per wave
    if (p.waves > kMaxWavesX) p.waves = kMaxWavesX;
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

typedef void (*w2x_kernel_t)(int, int, int, int, int, const uint16_t*, const u32x4_t*,
                             const uint16_t*, void*, int);

template <bool BF16>
w2x_kernel_t pickx(int group) {
    switch (group) {
        case 32: return w2t_gemv_direct_kernel<BF16, 1, 4>;
        case 64: return w2t_gemv_direct_kernel<BF16, 2, 4>;
        case 128: return w2t_gemv_direct_kernel<BF16, 4, 4>;
        default: return w2t_gemv_direct_kernel<BF16, 8, 4>;
    }
}


// ------------------------------------------------------------------ dispatch


constexpr size_t kLdsPerCu2 = 160 * 1024;      // gfx950
constexpr int kUpwSet2[] = {1, 2, 3, 4, 5, 6, 8, 9, 12, 17};

struct Plan2 {
    W2Launch l;
    int waves, upw, tiles, tpw;
    size_t lds;
};

int pick_upw2(int need) {
    for (int u : kUpwSet2)
        if (u >= need) return u;
    return 0;
}

// Same rules as the 4-bit planner: slices only when the compiled ranges or
// LDS require them, or when the tile count leaves CUs idle and each wave
// keeps at least two units per slice.
Plan2 make_plan2(int M, int N, int K, int cus) {
    Plan2 p;
    const int U = (K + kUnitK2 - 1) / kUnitK2;
    const int T = pad_n(N) / kTileN;
    const int W = kWaves2;
    // The workgroup's x is exactly M x (its slice's units) x 512 bytes (the
    // partial sums reuse it); slices differ by at most one unit.
    auto fits = [&](int S, int& upw, size_t& lds) {
        const int RU = (U + S - 1) / S;
        const int w = W < RU ? W : RU;
        upw = pick_upw2((RU + w - 1) / w);
        if (!upw || M * upw > 32) return false;
        lds = (size_t)M * RU * kUnitK2 * 2;
        return lds <= kLdsPerCu2;
    };
    int S = 1, upw = 0;
    size_t lds = 0;
    while (S < U && !fits(S, upw, lds)) S *= 2;
    while ((long long)T * S < cus && U / (2 * S) >= 2 * W && fits(2 * S, upw, lds)) S *= 2;
    // A workgroup with more than half a CU's LDS runs alone on its CU: more
    // slices while each wave keeps at least two units.
    while (lds > kLdsPerCu2 / 2 && U / (2 * S) >= 2 * W && fits(2 * S, upw, lds)) S *= 2;
    if (!fits(S, upw, lds)) upw = 0;
    p.l = W2Launch{M, N, K, U, S, W4A16_F32};
    p.waves = W;
    p.upw = upw;
    p.tiles = T;
    p.lds = lds;
    // Three tiles per workgroup when there are many more tiles than the GPU
    // holds at once (where compiled: the caller checks tpw3_compiled).
    p.tpw = S == 1 && upw >= 1 && upw <= 4 && T >= 6 * cus ? 3 : 1;
    return p;
}

typedef void (*w2_kernel_t)(int, int, int, int, int, const uint16_t*, const u32x4_t*,
                            const uint16_t*, void*, W2Launch);

template <bool BF16, int SPG>
w2_kernel_t pick_upw2_kernel(int upw) {
    switch (upw) {
        case 1: return w2t_gemv_kernel<BF16, SPG, 1>;
        case 2: return w2t_gemv_kernel<BF16, SPG, 2>;
        case 3: return w2t_gemv_kernel<BF16, SPG, 3>;
        case 4: return w2t_gemv_kernel<BF16, SPG, 4>;
        case 5: return w2t_gemv_kernel<BF16, SPG, 5>;
        case 6: return w2t_gemv_kernel<BF16, SPG, 6>;
        case 8: return w2t_gemv_kernel<BF16, SPG, 8>;
        case 9: return w2t_gemv_kernel<BF16, SPG, 9>;
        case 12: return w2t_gemv_kernel<BF16, SPG, 12>;
        default: return w2t_gemv_kernel<BF16, SPG, 17>;
    }
}

template <bool BF16>
w2_kernel_t pick2_group(int group, int upw) {
    switch (group) {
        case 32: return pick_upw2_kernel<BF16, 1>(upw);
        case 64: return pick_upw2_kernel<BF16, 2>(upw);
        case 128: return pick_upw2_kernel<BF16, 4>(upw);
        default: return pick_upw2_kernel<BF16, 8>(upw);
    }
}

w2_kernel_t pick2(bool bf16, int group, int upw) {
    return bf16 ? pick2_group<true>(group, upw) : pick2_group<false>(group, upw);
}

// Three-tile kernels, compiled where the chain keeps its ring loads in
// straight-line code (the x wait's condition, checked on the compiled code by
// a host-side test) and within 128 VGPRs: g = 64 at 3 or 4 units per wave
// (at 1 or 2 the compiler sinks ring loads into branches), g = 128 at 1 to 3
// (4 spills), g = 256 at 1 to 4.
bool tpw3_compiled(int group, int upw) {
    if (group == 64) return upw == 3 || upw == 4;
    if (group == 128) return upw >= 1 && upw <= 3;
    return group == 256 && upw >= 1 && upw <= 4;
}
template <bool BF16>
w2_kernel_t pick2_tpw3_bf(int group, int upw) {
    if (group == 64) return upw == 3 ? w2t_gemv_kernel<BF16, 2, 3, 3> : w2t_gemv_kernel<BF16, 2, 4, 3>;
    if (group == 128)
        return upw == 1 ? w2t_gemv_kernel<BF16, 4, 1, 3>
             : upw == 2 ? w2t_gemv_kernel<BF16, 4, 2, 3>
                        : w2t_gemv_kernel<BF16, 4, 3, 3>;
    return upw == 1 ? w2t_gemv_kernel<BF16, 8, 1, 3>
         : upw == 2 ? w2t_gemv_kernel<BF16, 8, 2, 3>
         : upw == 3 ? w2t_gemv_kernel<BF16, 8, 3, 3>
                    : w2t_gemv_kernel<BF16, 8, 4, 3>;
}
w2_kernel_t pick2_tpw3(bool bf16, int group, int upw) {   // tpw3_compiled(group, upw) only
    return bf16 ? pick2_tpw3_bf<true>(group, upw) : pick2_tpw3_bf<false>(group, upw);
}

// The staged kernel (split or not) up to 8 rows when its workgroup needs at
// most half a CU's LDS (two or more workgroups per CU), the direct-x kernel
// otherwise.  Measured, us per call, staged / direct-x:
//   K 5120 N 7168    M = 1: 5.2 / 6.9    M = 8: 7.7 / 9.3    M = 12: 14.0 / 10.9
//   K 5120 N 34816   M = 1: 15.1 / 22.4  M = 8: 28.0 / 33.3  M = 16: 52.7 / 45.9
//   K 17408 N 5120   M = 4: 14.1 / 19.2  M = 8: 19.0 / 24.2  M = 16: 31.7 / 35.5
// (above 8 rows a wave keeps at most two units per slice).
constexpr size_t kStagedLdsMax = kLdsPerCu2 / 2;
constexpr int kStagedMaxRows = 8;

size_t staged_lds_max() {
    // Override for A/B measurement only (read once per process: common.h).
    const long long n = w4h::overrides().w2t_staged_lds_max;
    return n > 0 ? (size_t)n : kStagedLdsMax;
}

bool use_staged(const Plan2& p) {
    return p.upw && p.l.M <= kStagedMaxRows && p.lds <= staged_lds_max();
}

// Allow every ternary GEMV kernel the whole LDS of a CU, once per process.
void allow_full_lds2() {
    static std::once_flag once;
    std::call_once(once, [] {
        for (int bf = 0; bf < 2; ++bf)
            for (int g : {32, 64, 128, 256}) {
                for (int u : kUpwSet2)
                    (void)hipFuncSetAttribute((const void*)pick2(bf, g, u),
                                              hipFuncAttributeMaxDynamicSharedMemorySize,
                                              (int)kLdsPerCu2);
                for (int u = 1; u <= 4; ++u)
                    if (tpw3_compiled(g, u))
                        (void)hipFuncSetAttribute((const void*)pick2_tpw3(bf, g, u),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize,
                                                  (int)kLdsPerCu2);
            }
        (void)hipGetLastError();
    });
}

inline unsigned grid_for(size_t work, unsigned block) {
    size_t g = (work + block - 1) / block;
    if (g > 65536u * 4) g = 65536u * 4;
    if (g == 0) g = 1;
    return (unsigned)g;
}

}  // namespace

namespace {

int launch_direct(const void* x, int x_dtype, const void* qweight, const void* scales, void* y,
                  int y_dtype, int M, int N, int K, int group, void* workspace,
                  size_t workspace_bytes, w4a16_stream_t stream) {
    const PlanX p = make_planx(N, K);
    const size_t need = w4h::ws_bytes(p.split > 1 ? (size_t)p.split * M * N * sizeof(float) : 0);
    if (need) {
        if (!workspace) return W4A16_ERR_NULL;
        if (workspace_bytes < need) return W4A16_ERR_WORKSPACE;
        if (!w4h::aligned16(workspace)) return W4A16_ERR_ALIGN;
    }
    hipStream_t st = (hipStream_t)stream;
    const int T = pad_n(N) / kTileN;
    const bool bf16 = x_dtype == W4A16_BF16;
    w2x_kernel_t k = bf16 ? pickx<true>(group) : pickx<false>(group);
    void* out = p.split > 1 ? w4h::ws_part(workspace) : y;
    const int odt = p.split > 1 ? W4A16_F32 : y_dtype;
    w4h::begin_launches();
    hipLaunchKernelGGL(k, dim3(T, p.split), dim3(64 * p.waves), 0, st, M, N, K, p.split, p.waves,
                       (const uint16_t*)x, (const u32x4_t*)qweight, (const uint16_t*)scales, out, odt);
    if (p.split > 1) {
        const int MN = M * N;
        hipLaunchKernelGGL(w2_merge_kernel, dim3((MN + 255) / 256), dim3(256), 0, st,
                           (const float*)w4h::ws_part(workspace), y, y_dtype, MN, p.split);
    }
    w4h::set_last_variant("w2t_mfma16 %s g%d kernel=w2t_gemv_direct_kernel<%s, %d, 4> tiles=%d "
                          "slices=%d waves=%d",
                          bf16 ? "bf16" : "f16", group, bf16 ? "true" : "false", group / 32, T,
                          p.split, p.waves);
    return w4h::launch_status();
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
    if (M < 1 || M > kMaxRows || !w4h::x_fits(M, K)) return W4A16_ERR_SHAPE;
    int rc = w4h::check_w2_shape(N, K, group);
    if (rc) return rc;
    const Plan2 p = make_plan2(M, N, K, w4h::cu_count());
    if (use_staged(p)) {
        *bytes = w4h::ws_bytes(p.l.S > 1 ? (size_t)p.l.S * M * N * sizeof(float) : 0);
    } else {
        const PlanX px = make_planx(N, K);
        *bytes = w4h::ws_bytes(px.split > 1 ? (size_t)px.split * M * N * sizeof(float) : 0);
    }
    return W4A16_OK;
}

extern "C" int w2t_gemv(const void* x, int x_dtype, const void* qweight, const void* scales, void* y,
                        int y_dtype, int M, int N, int K, int group, void* workspace,
                        size_t workspace_bytes, w4a16_stream_t stream) {
    if (!x || !qweight || !scales || !y) return W4A16_ERR_NULL;
    if (x_dtype != W4A16_F16 && x_dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    if (y_dtype != W4A16_F32 && y_dtype != W4A16_F16 && y_dtype != W4A16_BF16)
        return W4A16_ERR_DTYPE;
    if (M < 1 || M > kMaxRows || !w4h::x_fits(M, K)) return W4A16_ERR_SHAPE;
    int rc = w4h::check_w2_shape(N, K, group);
    if (rc) return rc;
    if (!w4h::aligned16(x) || !w4h::aligned16(qweight) || !w4h::aligned16(scales) ||
        !w4h::aligned16(y))
        return W4A16_ERR_ALIGN;
    Plan2 p = make_plan2(M, N, K, w4h::cu_count());
    if (!use_staged(p)) return launch_direct(x, x_dtype, qweight, scales, y, y_dtype, M, N, K, group,
                                             workspace, workspace_bytes, stream);
    const size_t need = w4h::ws_bytes(p.l.S > 1 ? (size_t)p.l.S * M * N * sizeof(float) : 0);
    if (need) {
        if (!workspace) return W4A16_ERR_NULL;
        if (workspace_bytes < need) return W4A16_ERR_WORKSPACE;
        if (!w4h::aligned16(workspace)) return W4A16_ERR_ALIGN;
    }
    allow_full_lds2();
    hipStream_t st = (hipStream_t)stream;
    const bool bf16 = x_dtype == W4A16_BF16;
    if (p.tpw > 1 && !tpw3_compiled(group, p.upw)) p.tpw = 1;
    w2_kernel_t k = p.tpw > 1 ? pick2_tpw3(bf16, group, p.upw) : pick2(bf16, group, p.upw);
    void* out = p.l.S > 1 ? w4h::ws_part(workspace) : y;
    p.l.out_dtype = p.l.S > 1 ? W4A16_F32 : y_dtype;
    w4h::begin_launches();
    hipLaunchKernelGGL(k, dim3((p.tiles + p.tpw - 1) / p.tpw, p.l.S), dim3(64 * p.waves), p.lds, st,
                       p.l.M, p.l.N, p.l.K, p.l.U, p.l.S, (const uint16_t*)x,
                       (const u32x4_t*)qweight, (const uint16_t*)scales, out, p.l);
    if (p.l.S > 1) {
        const int MN = M * N;
        hipLaunchKernelGGL(w2_merge_kernel, dim3((MN + 255) / 256), dim3(256), 0, st,
                           (const float*)w4h::ws_part(workspace), y, y_dtype, MN, p.l.S);
    }
    if (p.tpw > 1)
        w4h::set_last_variant("w2t_mfma16 %s g%d kernel=w2t_gemv_kernel<%s, %d, %d, %d> tiles=%d slices=%d "
                              "waves=%d upw=%d tpw=%d lds=%zu",
                              bf16 ? "bf16" : "f16", group, bf16 ? "true" : "false", group / 32, p.upw,
                              p.tpw, p.tiles, p.l.S, p.waves, p.upw, p.tpw, p.lds);
    else
        w4h::set_last_variant("w2t_mfma16 %s g%d kernel=w2t_gemv_kernel<%s, %d, %d> tiles=%d slices=%d "
                              "waves=%d upw=%d lds=%zu",
                              bf16 ? "bf16" : "f16", group, bf16 ? "true" : "false", group / 32, p.upw,
                              p.tiles, p.l.S, p.waves, p.upw, p.lds);
    return w4h::launch_status();
}
