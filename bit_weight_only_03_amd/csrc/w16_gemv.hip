// w16_gemv.hip -- the W16A16 small-M linear layer on gfx950:
// y[M,N] = x[M,K] . w[N,K]^T with fp16 or bf16 weights of the same type as
// x, in the layer's own [N][K] layout (no packing), for M = 1..64.
//
// The Z100 article (section 六) measures this layer next to the W4A16 one:
// large K, a few rows, FP16/BF16 weights read straight from memory.  The
// weights are four times the bytes of the 4-bit path, so the kernel is the
// same stream without the dequantization: each wave owns one 16-column tile
// over its workgroup's K slice, the workgroup streams x through LDS one
// 128-k unit at a time (double-buffered, shared by its waves), and every
// 16-byte chunk a lane loads is directly the MFMA B operand.  Layers of a
// few hundred tiles (up to 16 rows and 8 units per wave) take GEMV-shaped
// kernels instead: one tile per workgroup, its waves splitting K, so they
// fill the GPU without K slices and a merge launch.  Up to 4 rows that is a
// VALU dot-product kernel whose loads read whole lines, above it an MFMA
// kernel in the layout below.
//
// Layout of one unit for one tile: lane l serves column n = 16 t + l % 16;
// its j-th 16-byte load (j = 0..3) is w[n][128 u + 32 j + 8 (l / 16) .. + 8],
// which is also what the 32-k MFMA step j expects from that lane.  One load
// instruction of a wave thus reads 64 contiguous bytes of each of its 16
// rows, and two consecutive instructions fill a 128-byte line.  Giving each
// lane its own contiguous 64 bytes instead (four 16-byte pieces 64 bytes
// apart per row and instruction) ran at 2.2-2.7 TB/s against 3.4-4.4 TB/s.
// The loads take the default cache policy: the two instructions that share
// a line then meet in the vector L1, and the non-temporal hint measured
// 5-25% slower.
#include <stdlib.h>

#include <mutex>

#include "common.h"

using namespace w4k;

namespace {

constexpr int kW16Waves = 4;            // waves per workgroup, one tile each
constexpr int kW16Ring = 2;             // units of weight loads in flight per wave (4: no gain, 92 VGPRs)
constexpr int kW16XStride = kUnitK + 8; // halves per staged x row (+16 B spreads rows over banks)
constexpr int kW16MaxRows = 64;
constexpr int kW16MaxSplit = 16;

struct W16Launch {
    int M, N, K;
    int U;   // 128-k units (K rounded up)
    int S;   // K slices
    int T;   // 16-column tiles
    int out_dtype;
};

// Every kernel here takes the launch fields a wave needs first as seven
// leading scalars (the last, G_, the launch's workgroups along x, which the
// even-share kernel divides its rows by) ahead of its three pointers (ten
// arguments, 13 dwords),
// which the build compiles as preloaded into SGPRs at wave launch, so no
// wave starts with a scalar load of its arguments; out_dtype, used only by
// the stores, stays in the struct.
__device__ __forceinline__ W16Launch lead_launch(int M, int N, int K, int U, int S, int T,
                                                 const W16Launch& rest) {
    return W16Launch{M, N, K, U, S, T, rest.out_dtype};
}

// One workgroup per (4 tiles, K slice); per unit of the slice: x of the unit
// staged in LDS buffer u % 2 by all threads (zeros past K and in rows >= M,
// whose outputs are never stored), every wave multiplies its tile's unit
// (loaded kW16Ring units earlier) while the x of unit u + 2 loads into one
// of two register sets, then stores the x of unit u + 1 (loaded one unit
// earlier, before unit u + 1's weights, so the store does not wait for
// them) into the other buffer; one barrier per unit.  Units past the
// slice and rows past N load as zeros, so the loop body is uniform.
template <bool BF16, int RB>
__global__ __launch_bounds__(256) void w16_gemv_kernel(int M_, int N_, int K_, int U_, int S_, int T_, int G_,
        const uint16_t* __restrict__ x,
                                                       const uint16_t* __restrict__ w, void* out,
                                                       W16Launch a_in) {
    const W16Launch a = lead_launch(M_, N_, K_, U_, S_, T_, a_in);
    constexpr int ROWS = 16 * RB;
    constexpr int XCH = ROWS * (kUnitK / 8);   // 16-byte chunks of one staged unit
    constexpr int XPT = XCH / 256;             // chunks per thread (= RB)
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][ROWS][kW16XStride];

    const int M = a.M, N = a.N, K = a.K, U = a.U, T = a.T;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15, kc = lane >> 4;
    const int split = blockIdx.y;
    const int r0 = split * U / a.S, r1 = (split + 1) * U / a.S;
    const int nu = r1 - r0;
    const int t = blockIdx.x * kW16Waves + wave;                         // this wave's tile
    const int rows = t >= T ? 0 : (N - 16 * t < 16 ? N - 16 * t : 16);  // its columns inside N

    // The tile's rows of w as one resource: lane offset 2 c K + 16 kc, unit
    // offset 256 u, step offset 64 j.  A row past N or a unit past the slice reads zeros; the
    // tail of a ragged last unit reads the next row, which meets zero x.
    const uint32_t wend = (uint32_t)rows * (uint32_t)K * 2u;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w + (size_t)16 * t * K, wend);
    const uint32_t xend = (uint32_t)M * (uint32_t)K * 2u;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, xend);
    const uint32_t wlane = (uint32_t)c * (uint32_t)K * 2u + 16u * kc;

    auto load_unit = [&](int i, u32x4_t (&r)[4]) {
        const uint32_t off = i < nu ? wlane + (uint32_t)(r0 + i) * (kUnitK * 2) : wend;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            r[j] = bitcast<u32x4_t>(__builtin_amdgcn_raw_buffer_load_b128(rw, off + 64u * j, 0, 0));
    };

    u32x4_t xr[2][XPT];
    auto load_x = [&](int i, int slot) {
        const int kb = (r0 + i) * kUnitK;
#pragma unroll
        for (int p = 0; p < XPT; ++p) {
            // Branch-free: a chunk outside x (row >= M, k >= K, or a unit past
            // the slice) takes an offset past the resource and reads zeros.
            // A load under a branch would make the compiler's wait at the
            // loop head cover every load in flight, draining the weight ring.
            const int ch = threadIdx.x + 256 * p;   // < XCH: XCH = 256 RB
            const int m = ch >> 4, k = kb + 8 * (ch & 15);
            const bool in = m < M && k < K && i < nu;
            xr[slot][p] = bitcast<u32x4_t>(__builtin_amdgcn_raw_buffer_load_b128(
                rx, in ? (uint32_t)(m * K + k) * 2u : xend, 0, 0));
        }
    };
    auto store_x = [&](int b, int slot) {
#pragma unroll
        for (int p = 0; p < XPT; ++p) {
            const int ch = threadIdx.x + 256 * p;
            *(u32x4_t*)&xs[b][ch >> 4][8 * (ch & 15)] = xr[slot][p];
        }
    };

    float4_t acc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb] = float4_t{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](const u32x4_t (&r)[4], int b) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const u32x4_t av = *(const u32x4_t*)&xs[b][16 * rb + c][32 * j + 8 * kc];
                if constexpr (BF16)
                    acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        bitcast<bf16x8_t>(av), bitcast<bf16x8_t>(r[j]), acc[rb], 0, 0, 0);
                else
                    acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        bitcast<half8_t>(av), bitcast<half8_t>(r[j]), acc[rb], 0, 0, 0);
            }
        }
    };

    u32x4_t ring[kW16Ring][4];
    load_x(0, 0);
#pragma unroll
    for (int d = 0; d < kW16Ring; ++d) load_unit(d, ring[d]);
    load_x(1, 1);
    store_x(0, 0);
    __syncthreads();
    for (int i = 0; i < nu; i += kW16Ring) {
#pragma unroll
        for (int d = 0; d < kW16Ring; ++d) {
            load_x(i + d + 2, d & 1);           // slot (i + d) % 2: x of unit i + d is in LDS
            compute(ring[d], d & 1);            // unit i + d sits in buffer (i + d) % 2
            load_unit(i + d + kW16Ring, ring[d]);
            store_x((d + 1) & 1, (d + 1) & 1);  // x of unit i + d + 1, loaded one unit ago
            __syncthreads();
        }
    }

    // Lane l holds rows 16 rb + 4 (l / 16) + q of column l % 16.
    const int n = 16 * t + c;
    if (c >= rows) return;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int m = 16 * rb + 4 * kc + q;
            if (m >= M) continue;
            const size_t o = (size_t)m * N + n;
            if (a.S > 1)
                ((float*)out)[(size_t)split * M * N + o] = acc[rb][q];
            else
                store_out(out, a.out_dtype, o, acc[rb][q]);
        }
}

// Layers with few tiles, up to 16 rows: the GEMV kernel's shape instead.
// One workgroup of 8 waves per 16-column tile, the waves splitting the K
// units, so a layer of a few hundred tiles fills the GPU without K slices and
// their merge launch.  Each wave
//   1. stages its own units of x (all M rows) in LDS straight from memory
//      (the 4-bit GEMV's scheme: exact per-wave regions [M][nu units of 256
//      bytes], 16-byte chunk p of a unit in row m at position p ^ (m % 4);
//      chunks past K zeroed);
//   2. streams its units' weights, four 16-byte loads per lane and unit
//      (the coalesced per-step layout above), kW16KRing units ahead;
//   3. multiplies unit by unit: x rows from LDS as A, the weight chunks as B.
// The waves' partial sums go through LDS (each wave's own x region) and are
// added in wave order.  A wave past the units of a short K has no region and
// adds nothing (its partial would be +0, and the sum starts at +0).
constexpr int kW16KWaves = 8;
constexpr size_t kW16KLdsMax = 80 * 1024;   // half of a CU's 160 KB
// Units of weight loads in flight per wave.  Four (92 VGPRs against 58)
// measured 7-15% slower on every shape.
constexpr int kW16KRing = 2;
// Units per wave it takes at most: the down shape (K = 17408, 17 units per
// wave) ran 44.2 us against 36.7 us for the tiled kernel in 16 K slices.
constexpr int kW16KMaxUnits = 8;
constexpr int kW16KMaxXLoads = 16;   // x load instructions per wave: M * 16 * units <= 64 * 16

template <bool BF16>
__global__ __launch_bounds__(512) void w16_ksplit_kernel(int M_, int N_, int K_, int U_, int S_, int T_, int G_,
        const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ w, void* out,
                                                         W16Launch a_in) {
    const W16Launch a = lead_launch(M_, N_, K_, U_, S_, T_, a_in);
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int M = a.M, N = a.N, K = a.K, U = a.U;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15, kc = lane >> 4;
    const int t = blockIdx.x;
    const int w0 = wave * U / kW16KWaves, w1 = (wave + 1) * U / kW16KWaves;
    const int nu = w1 - w0;
    const int rows = N - 16 * t < 16 ? N - 16 * t : 16;
    constexpr int kUnitBytes = kUnitK * 2;                  // one row of one unit of x
    uint8_t* const xsb = smem + (size_t)M * kUnitBytes * w0;
    const int rowb = nu * kUnitBytes;

    // 1) x units of this wave -> LDS (lane l of load i fills position 64 i + l).
    {
        const int cpr = nu * (kUnitK / 8);
        const int xch = M * cpr;
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
#pragma unroll
        for (int i = 0; i < kW16KMaxXLoads; ++i) {
            if (i * 64 < xch) {                      // wave-uniform (false without units)
                const int ci = i * 64 + lane;
                const int m = ci / cpr, pc = ci % cpr;
                const int kg = w0 * kUnitK + (pc ^ (m & 3)) * 8;
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
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2) The tile's rows as one resource (rows past N read zeros; the tail of
    //    a ragged last unit reads the next row, which meets zero x).
    const uint32_t wend = (uint32_t)rows * (uint32_t)K * 2u;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w + (size_t)16 * t * K, wend);
    const uint32_t wlane = (uint32_t)c * (uint32_t)K * 2u + 16u * kc;
    auto load_unit = [&](int i, u32x4_t (&r)[4]) {
        const uint32_t off = i < nu ? wlane + (uint32_t)(w0 + i) * kUnitBytes : wend;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            r[j] = bitcast<u32x4_t>(__builtin_amdgcn_raw_buffer_load_b128(rw, off + 64u * j, 0, 0));
    };
    constexpr int R = kW16KRing;
    u32x4_t ring[R][4];
#pragma unroll
    for (int d = 0; d < R; ++d) {
        load_unit(d, ring[d]);
        __builtin_amdgcn_sched_barrier(0);
    }
    // Loads complete in issue order: with the ring's 4 R loads outstanding
    // the x loads issued before them have landed in LDS.  This needs the
    // ring loads issued here, before the wait: the loop below runs at least
    // once for every wave, so no use of them sits in a conditional block the
    // compiler could sink them into (a host-side test checks the assembly).
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * R) : "memory");
    __builtin_amdgcn_sched_barrier(0);

    // 3) Products.  Step j of unit i: chunk 4 j + kc of row c, at position
    //    4 j + (kc ^ c % 4).  Units past the range load zero weights and keep
    //    the last x fragments, so they add exactly 0.
    const bool xrow = c < M;
    const uint8_t* xl = xsb + (uint32_t)(c * rowb) + 16u * (uint32_t)(kc ^ (c & 3));
    float4_t acc = {0.f, 0.f, 0.f, 0.f};
    u32x4_t xa[4] = {};
    const int upw = (U + kW16KWaves - 1) / kW16KWaves;   // >= 1, the same for every wave
    int i = 0;
    do {
#pragma unroll
        for (int d = 0; d < R; ++d) {
            if (xrow && i + d < nu) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    xa[j] = *(const u32x4_t*)(xl + (uint32_t)(i + d) * kUnitBytes + 64 * j);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (BF16)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8_t>(xa[j]),
                                                                  bitcast<bf16x8_t>(ring[d][j]), acc,
                                                                  0, 0, 0);
                else
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<half8_t>(xa[j]),
                                                                 bitcast<half8_t>(ring[d][j]), acc,
                                                                 0, 0, 0);
            }
            load_unit(i + d + R, ring[d]);
        }
        i += R;
    } while (i < upw);

    // 4) Partials -> the wave's own x region, then the wave-order sum.
    if (nu > 0) {
        float* const red = (float*)xsb;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 4 * kc + r;
            if (m < M) red[m * kTileN + c] = acc[r];
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < M * kTileN; idx += blockDim.x) {
        const int m = idx >> 4, cc = idx & 15;
        float pw[kW16KWaves];
#pragma unroll
        for (int wv = 0; wv < kW16KWaves; ++wv) {
            const int b = wv * U / kW16KWaves, e = (wv + 1) * U / kW16KWaves;
            pw[wv] = e > b ? ((const float*)(smem + (size_t)M * kUnitBytes * b))[m * kTileN + cc] : 0.f;
        }
        float v = 0.f;
#pragma unroll
        for (int wv = 0; wv < kW16KWaves; ++wv)
            if ((wv + 1) * U / kW16KWaves > wv * U / kW16KWaves) v += pw[wv];
        const int n = 16 * t + cc;
        if (n < N) store_out(out, a.out_dtype, (size_t)m * N + n, v);
    }
}

// Layers of up to 4 rows: dot products on the VALU, which frees the weight
// loads from the MFMA operand layout.  One workgroup of 4 waves per
// 16-column tile, the waves splitting its 128-k units as in the K-split
// kernel, x staged the same way (per-wave regions [M][nu units of 256 bytes],
// loaded straight into LDS, no swizzle: every lane of a read takes the same
// row).  Per unit, lane l makes four 16-byte loads j = 0..3 at row
// 16 t + 4 j + l / 16 and bytes 16 (l % 16) of the unit's 256 in that row:
// each load instruction reads four rows of 256 contiguous bytes (whole
// 128-byte lines), with the non-temporal policy.  A read-only copy of this
// pattern streamed gate_up (N = 34816, K = 5120) in 52.9 us against 60.0 us
// for the MFMA layout (16 rows of 64 bytes per instruction, default policy),
// o_proj in 11.7 against 14.3 us.  Against the K-split kernel (bench graphs,
// fp16, us per call at M = 1 / 2 / 4 / 8): qkv 14.3 / 14.5 / 15.8 / 20.2
// against 16.1 / 16.0 / 16.5 / 17.7, o_proj 13.0 / 13.3 / 14.6 / 18.4 against
// 15.1 / 15.2 / 15.7 / 16.7, gate_up 56.8 / 56.9 / 59.6 / 82 against
// 64.6 / 64.1 / 66.0 / 74.2: at 8 rows the 128 v_dot2 per unit and wave
// outweigh the better stream, so it stops at 4 rows.  (Those figures are
// for 8 waves per tile.)  On the down shape (136 units, 320 tiles on 256
// CUs) it took 35.3 / 36.4 us at M = 1 / 2 against 35.1 / 35.2 for the
// tiled kernel in 16 slices, so it keeps to the K-split kernel's 64 units.
// Four waves per tile (10 units each on these shapes) against eight: qkv
// 13.8 against 14.3 us, o_proj 12.3 against 13.0, gate_up even at M = 1
// (M = 4: o_proj 13.9 against 14.6); two waves: o_proj 11.8 but qkv 13.9,
// gate_up 58.9, and every shape 1.3-10 us slower at M = 4; 3 or 4 units
// in flight per wave instead of 2: 0.2-0.6 us slower.
// Each lane keeps, per row of its loads and row of x, an fp32 sum over its
// 8-k chunks (v_dot2: two exact fp16 or bf16 products added in fp32); at
// the end the 16 lanes of a row are added in a fixed butterfly, then the
// waves in wave order through LDS.
constexpr int kW16DWaves = 4;
constexpr int kW16DRing = 2;
constexpr int kW16DMaxRows = 4;
constexpr int kW16DMaxUnits = 16;       // units per wave
constexpr int kW16DMaxXLoads = 16;      // x load instructions per wave: M * 16 * units <= 64 * 16

template <bool BF16, int MR>
__global__ __launch_bounds__(64 * kW16DWaves) void w16_dot_kernel(int M_, int N_, int K_, int U_, int S_, int T_, int G_,
        const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ w, void* out,
                                                      W16Launch a_in) {
    const W16Launch a = lead_launch(M_, N_, K_, U_, S_, T_, a_in);
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int M = a.M, N = a.N, K = a.K, U = a.U;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kc = lane & 15, r = lane >> 4;
    const int t = blockIdx.x;
    const int w0 = wave * U / kW16DWaves, w1 = (wave + 1) * U / kW16DWaves;
    const int nu = w1 - w0;
    const int rows = N - 16 * t < 16 ? N - 16 * t : 16;
    constexpr int kUnitBytes = kUnitK * 2;                  // one row of one unit of x
    uint8_t* const xsb = smem + (size_t)M * kUnitBytes * w0;

    // 1) x units of this wave -> LDS: 16-byte chunk i of row m's range at
    //    (m nu 16 + i) 16 bytes (lane l of load p fills chunk 64 p + l).
    {
        const int cpr = nu * (kUnitK / 8);
        const int xch = M * cpr;
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
#pragma unroll
        for (int p = 0; p < kW16DMaxXLoads; ++p) {
            if (p * 64 < xch) {                      // wave-uniform (false without units)
                const int ci = p * 64 + lane;
                const int m = ci / cpr, pc = ci % cpr;
                const int kg = w0 * kUnitK + pc * 8;
                if (m < M) {
                    if (kg < K)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            rx, (__attribute__((address_space(3))) void*)(xsb + p * 1024), 16,
                            (uint32_t)(m * K + kg) * 2u, 0, 0, 0);
                    else
                        *(u32x4_t*)(xsb + (uint32_t)ci * 16u) = u32x4_t{0u, 0u, 0u, 0u};
                }
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2) The tile's rows as one resource.  Rows past N read zeros; the tail of
    //    a ragged last unit reads the start of the next row, which meets zero x.
    const uint32_t wend = (uint32_t)rows * (uint32_t)K * 2u;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w + (size_t)16 * t * K, wend);
    const uint32_t wlane = (uint32_t)r * (uint32_t)K * 2u + 16u * kc;
    const uint32_t four_rows = 4u * (uint32_t)K * 2u;
    auto load_unit = [&](int i, u32x4_t (&q)[4]) {
        const uint32_t off = i < nu ? wlane + (uint32_t)(w0 + i) * kUnitBytes : wend;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            q[j] = bitcast<u32x4_t>(
                __builtin_amdgcn_raw_buffer_load_b128(rw, off + four_rows * j, 0, kAuxNT));
    };
    constexpr int R = kW16DRing;
    u32x4_t ring[R][4];
#pragma unroll
    for (int d = 0; d < R; ++d) {
        load_unit(d, ring[d]);
        __builtin_amdgcn_sched_barrier(0);
    }
    // Loads complete in issue order: with the ring's 4 R loads outstanding
    // the x loads issued before them have landed in LDS (the loop below runs
    // at least once for every wave, so the ring loads are not sunk into a
    // branch; a host-side test checks the assembly).
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * R) : "memory");
    __builtin_amdgcn_sched_barrier(0);

    // 3) Products.  Units past the range load zero weights and skip the x
    //    read, so they add exactly 0 (x is finite).
    float acc[4][MR];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[j][m] = 0.f;
    const uint8_t* const xl = xsb + 16u * kc;
    const int upw = (U + kW16DWaves - 1) / kW16DWaves;   // >= 1, the same for every wave
    int i = 0;
    do {
#pragma unroll
        for (int d = 0; d < R; ++d) {
            if (i + d < nu) {
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    if (m < M) {
                        const u32x4_t xv =
                            *(const u32x4_t*)(xl + (uint32_t)((m * nu + i + d) * kUnitBytes));
#pragma unroll
                        for (int j = 0; j < 4; ++j)
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                if constexpr (BF16)
                                    acc[j][m] = __builtin_amdgcn_fdot2_f32_bf16(
                                        bitcast<bf16x2_t>(ring[d][j][e]), bitcast<bf16x2_t>(xv[e]),
                                        acc[j][m], false);
                                else
                                    acc[j][m] = __builtin_amdgcn_fdot2(
                                        bitcast<half2_t>(ring[d][j][e]), bitcast<half2_t>(xv[e]),
                                        acc[j][m], false);
                            }
                    }
                }
            }
            load_unit(i + d + R, ring[d]);
        }
        i += R;
    } while (i < upw);

    // 4) The 16 lanes of each row (fixed butterfly; lane 16 r keeps the sum),
    //    then per wave [M][16] partials in the wave's own x region (its last
    //    reads of it came before, in program order), then the wave-order sum.
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            float v = acc[j][m];
            v += __shfl_xor(v, 8);
            v += __shfl_xor(v, 4);
            v += __shfl_xor(v, 2);
            v += __shfl_xor(v, 1);
            acc[j][m] = v;
        }
    if (nu > 0 && kc == 0) {
        float* const red = (float*)xsb;
#pragma unroll
        for (int m = 0; m < MR; ++m)
            if (m < M)
#pragma unroll
                for (int j = 0; j < 4; ++j) red[m * kTileN + 4 * j + r] = acc[j][m];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < M * kTileN; idx += blockDim.x) {
        const int m = idx >> 4, cc = idx & 15;
        float v = 0.f;
#pragma unroll
        for (int wv = 0; wv < kW16DWaves; ++wv) {
            const int b = wv * U / kW16DWaves, e = (wv + 1) * U / kW16DWaves;
            if (e > b) v += ((const float*)(smem + (size_t)M * kUnitBytes * b))[m * kTileN + cc];
        }
        if (cc < rows) store_out(out, a.out_dtype, (size_t)m * N + 16 * t + cc, v);
    }
}

// The same dot products with one even share of the rows per workgroup, one
// workgroup per CU, for long-K layers whose 16-column tiles do not spread
// evenly over the CUs (the down shape's 320 tiles on 256 CUs leave 64 CUs
// with two) at up to 2 rows.  Workgroup c owns row groups [c G4 / C, (c + 1) G4 / C) of the
// G4 = ceil(N / 4) groups of 4 rows; an item is one group's 256 bytes per
// row of one 128-k unit, one 16-byte load per lane (lane l: row l / 16,
// bytes 16 (l % 16)), and its 16 waves take contiguous item ranges in
// group-major order, D items in flight.  x is staged whole, once per
// workgroup ([M][U units of 256 bytes], zeros past K).  A wave adds the
// items of one group in order and, where its range leaves the group, sums
// the 16 lanes of each row (a fixed butterfly) into its slot for that
// group; the slots of the waves that share a group are added in wave order.
// Measured (bench graphs, fp16, us per call at M = 1 / 2 / 4, against the
// kernel each shape takes otherwise): down 32.3-32.5 / 33.8-34.3 / 38.9-39.4
// against 34.8-35.4 / 35.4-35.7 / 36.6-36.8 (tiled, 16 slices); o_proj
// 13.2-13.4 / 13.8-14.0 / 15.5-15.8 against 13.0 / 13.3 / 14.6, qkv 16.7 /
// 17.2-17.4 / 19.6 against 14.4 / 14.6 / 16.1 (one tile per workgroup).
// Only long K at up to 2 rows gains, so only they take it.
constexpr int kW16BWaves = 16;
constexpr int kW16BMaxRows = 2;
constexpr int kW16BMinUnits = 65;               // K > 8192
constexpr int kW16BRing = 8;
constexpr size_t kW16BLdsMax = 144 * 1024;      // x and the slots, one workgroup per CU
constexpr int kW16BMaxXLoads = 9;               // x load instructions per thread (144 KB / 16 KB)

template <bool BF16, int MR>
__global__ __launch_bounds__(1024) void w16_dot_bal_kernel(int M_, int N_, int K_, int U_, int S_, int T_, int G_,
        const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ w,
                                                           void* out, W16Launch a_in) {
    const W16Launch a = lead_launch(M_, N_, K_, U_, S_, T_, a_in);
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int M = a.M, N = a.N, K = a.K, U = a.U;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kc = lane & 15, r = lane >> 4;
    const int G4 = (N + 3) >> 2;
    const int g0 = (int)((long long)blockIdx.x * G4 / G_);
    const int g1 = (int)((long long)(blockIdx.x + 1) * G4 / G_);
    const int ng = g1 - g0;
    if (ng == 0) return;                              // the whole workgroup
    constexpr int kUnitBytes = kUnitK * 2;
    const int I = ng * U;                             // items of the workgroup
    const int a0 = wave * I / kW16BWaves, a1 = (wave + 1) * I / kW16BWaves;
    const int n = a1 - a0;
    float* const slots = (float*)(smem + (size_t)M * U * kUnitBytes);   // [ng][waves][M][4]

    // 1) x -> LDS, chunk ci (16 bytes) of the [M][U * 16] chunk grid at ci * 16.
    {
        const int cpr = U * (kUnitK / 8);
        const int xch = M * cpr;
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
#pragma unroll
        for (int p = 0; p < kW16BMaxXLoads; ++p) {
            if (p * 1024 + wave * 64 < xch) {        // wave-uniform
                const int ci = p * 1024 + (int)threadIdx.x;
                const int m = ci / cpr, kg = (ci % cpr) * 8;
                if (ci < xch) {
                    if (kg < K)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            rx, (__attribute__((address_space(3))) void*)(smem + (size_t)(p * 1024 + wave * 64) * 16), 16,
                            (uint32_t)(m * K + kg) * 2u, 0, 0, 0);
                    else
                        *(u32x4_t*)(smem + (size_t)ci * 16) = u32x4_t{0u, 0u, 0u, 0u};
                }
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2) The workgroup's rows as one resource (rows past N read zeros; the
    //    tail of a ragged last unit reads the next row, which meets zero x).
    const int rows = (4 * g1 < N ? 4 * g1 : N) - 4 * g0;
    const uint32_t wend = (uint32_t)rows * (uint32_t)K * 2u;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w + (size_t)4 * g0 * K, wend);
    const uint32_t row_bytes = (uint32_t)K * 2u;
    const uint32_t wlane = (uint32_t)r * row_bytes + 16u * kc;
    int gl = a0 / U, ul = a0 % U;                     // the next item to load
    auto load_item = [&](bool valid) {
        // Straight-line code (the ring's loads must reach the x wait below
        // without a branch): an item past the range sets the offset's top
        // bit, beyond the resource, so it reads zeros; the counters advance
        // with selects.
        const uint32_t off = (wlane + (uint32_t)gl * 4u * row_bytes + (uint32_t)ul * kUnitBytes) |
                             (valid ? 0u : 0x80000000u);
        const bool wrap = valid && ul + 1 == U;
        ul = wrap ? 0 : ul + (valid ? 1 : 0);
        gl += wrap ? 1 : 0;
        return bitcast<u32x4_t>(__builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, kAuxNT));
    };
    constexpr int D = kW16BRing;
    u32x4_t ring[D];
#pragma unroll
    for (int d = 0; d < D; ++d) ring[d] = load_item(d < n);
    __builtin_amdgcn_sched_barrier(0);
    // Loads complete in issue order: with the D ring loads outstanding the
    // x loads this thread issued before them have landed; the barrier then
    // covers every thread's.
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(D) : "memory");
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();

    // 3) Products, item by item.
    float acc[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[m] = 0.f;
    int gc = a0 / U, uc = a0 % U;                     // the item being added
    const uint8_t* const xl = smem + 16u * kc;
    auto flush = [&]() {
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            float v = acc[m];
            v += __shfl_xor(v, 8);
            v += __shfl_xor(v, 4);
            v += __shfl_xor(v, 2);
            v += __shfl_xor(v, 1);
            if (m < M && kc == 0) slots[((gc * kW16BWaves + wave) * M + m) * 4 + r] = v;
            acc[m] = 0.f;
        }
    };
    for (int i = 0; i < n; i += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (i + d < n) {
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    if (m < M) {
                        const u32x4_t xv =
                            *(const u32x4_t*)(xl + (uint32_t)((m * U + uc) * kUnitBytes));
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if constexpr (BF16)
                                acc[m] = __builtin_amdgcn_fdot2_f32_bf16(
                                    bitcast<bf16x2_t>(ring[d][e]), bitcast<bf16x2_t>(xv[e]), acc[m], false);
                            else
                                acc[m] = __builtin_amdgcn_fdot2(
                                    bitcast<half2_t>(ring[d][e]), bitcast<half2_t>(xv[e]), acc[m], false);
                        }
                    }
                }
                if (++uc == U || i + d + 1 == n) {
                    flush();
                    if (uc == U) { uc = 0; ++gc; }
                }
            }
            ring[d] = load_item(i + d + D < n);
        }
    }

    // 4) Per row and row of x, the slots of the waves whose ranges meet its
    //    group, in wave order.
    __syncthreads();
    for (int idx = threadIdx.x; idx < M * 4 * ng; idx += blockDim.x) {
        const int m = idx / (4 * ng), rl = idx - m * 4 * ng;
        const int g = rl >> 2, rr = rl & 3;
        float v = 0.f;
#pragma unroll
        for (int wv = 0; wv < kW16BWaves; ++wv) {
            const int b = wv * I / kW16BWaves, e = (wv + 1) * I / kW16BWaves;
            if (b < (g + 1) * U && e > g * U) v += slots[((g * kW16BWaves + wv) * M + m) * 4 + rr];
        }
        const int row = 4 * (g0 + g) + rr;
        if (row < N) store_out(out, a.out_dtype, (size_t)m * N + row, v);
    }
}

template <bool BF16>
const void* pick_w16_dot_bal(int M) {
    if (M <= 1) return (const void*)w16_dot_bal_kernel<BF16, 1>;
    return (const void*)w16_dot_bal_kernel<BF16, 2>;
}

template <bool BF16>
const void* pick_w16_dot(int M) {
    if (M <= 1) return (const void*)w16_dot_kernel<BF16, 1>;
    if (M <= 2) return (const void*)w16_dot_kernel<BF16, 2>;
    return (const void*)w16_dot_kernel<BF16, 4>;
}

typedef void (*w16_kernel_t)(int, int, int, int, int, int, int, const uint16_t*, const uint16_t*,
                             void*, W16Launch);

template <bool BF16>
w16_kernel_t pick_w16_rb(int rb) {
    switch (rb) {
        case 1: return w16_gemv_kernel<BF16, 1>;
        case 2: return w16_gemv_kernel<BF16, 2>;
        case 3: return w16_gemv_kernel<BF16, 3>;
        default: return w16_gemv_kernel<BF16, 4>;
    }
}


struct W16Plan {
    int rb, split;
    long long workgroups;
    bool bal;       // the VALU dot-product kernel, one even row share per CU
    bool dot;       // the VALU dot-product kernel (one tile per workgroup)
    bool ksplit;    // the K-split kernel (one tile per workgroup)
    size_t lds;     // their dynamic LDS bytes
};

// K slices double while each keeps at least six units (4 KB of weights per
// wave per unit) and the grid stays under eight workgroups per CU.  The
// merge of M x N fp32 partials per slice is small next to the 2 N K weight
// bytes, and the extra workgroups are what keeps enough loads in flight:
// gate_up (N = 34816, K = 5120) took 80 us unsplit, 67 us in four slices.
W16Plan w16_plan(int M, int N, int K) {
    W16Plan p;
    const int U = (K + kUnitK - 1) / kUnitK;
    const int T = pad_n(N) / kTileN;
    // The K-split kernel up to 16 rows, when a wave's x fits its 16 load
    // instructions and the workgroup's x half a CU's LDS (two per CU).
    const int upw = (U + kW16KWaves - 1) / kW16KWaves;
    p.lds = (size_t)M * U * kUnitK * 2;
    p.ksplit = M <= 16 && upw <= kW16KMaxUnits && M * upw <= 64 && p.lds <= kW16KLdsMax;
    // Override for A/B measurement only: 0 turns the K-split kernel off.
    if (w4h::overrides().w16_ksplit == 0) p.ksplit = false;
    // The dot-product kernel up to 4 rows, under the same limits (x load
    // instructions per wave: M * 16 * units / 64).
    const int upw_d = (U + kW16DWaves - 1) / kW16DWaves;
    p.dot = M <= kW16DMaxRows && upw_d <= kW16DMaxUnits && M * upw_d * 16 <= 64 * kW16DMaxXLoads &&
            p.lds <= kW16KLdsMax;
    if (w4h::overrides().w16_dot == 0) p.dot = false;
    if (p.dot) p.ksplit = false;
    // The even row shares up to 2 rows, for layers of between one and two
    // tiles per CU and more than 64 units (the down shape: 320 tiles on 256
    // CUs, K = 17408), when x and the slots fit a CU's LDS.
    const int C = w4h::cu_count();
    const long long gmax = ((long long)(N + 3) / 4 + C - 1) / C;
    const size_t bal_lds = (size_t)M * U * kUnitK * 2 + (size_t)gmax * kW16BWaves * M * 4 * sizeof(float);
    const bool bal_fits = M <= kW16BMaxRows && bal_lds <= kW16BLdsMax && gmax * 4 * K * 2 < (1LL << 31);
    p.bal = bal_fits && T > C && T < 2 * C && U >= kW16BMinUnits;
    if (const int o = w4h::overrides().w16_bal; o == 0 || (o == 1 && bal_fits)) p.bal = o == 1;
    if (p.bal) {
        p.dot = p.ksplit = false;
        p.lds = bal_lds;
    }
    p.rb = (M + 15) / 16;
    p.workgroups = (T + kW16Waves - 1) / kW16Waves;
    p.split = 1;
    while (p.workgroups * p.split < 8LL * w4h::cu_count() && U / (2 * p.split) >= 6 &&
           p.split < kW16MaxSplit)
        p.split *= 2;
    if (const int s = w4h::overrides().w16_split; s >= 1 && s <= U && s <= kW16MaxSplit) p.split = s;
    return p;
}

int check_w16(int M, int N, int K) {
    if (M < 1 || M > kW16MaxRows || N < 8 || N % 8 || K < 8 || K % 8) return W4A16_ERR_SHAPE;
    if ((long long)M * K * 2 > 0xffffffffLL || 16LL * K * 2 > 0xffffffffLL) return W4A16_ERR_SHAPE;
    return W4A16_OK;
}

size_t w16_workspace(const W16Plan& p, int M, int N) {
    return w4h::ws_bytes(!p.bal && !p.dot && !p.ksplit && p.split > 1 ? (size_t)p.split * M * N * sizeof(float) : 0);
}

void allow_w16_lds() {
    static std::once_flag once;
    std::call_once(once, [] {
        for (const void* k : {(const void*)w16_ksplit_kernel<false>,
                              (const void*)w16_ksplit_kernel<true>,
                              pick_w16_dot<false>(1), pick_w16_dot<false>(2),
                              pick_w16_dot<false>(4), pick_w16_dot<true>(1),
                              pick_w16_dot<true>(2), pick_w16_dot<true>(4)})
            (void)hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kW16KLdsMax);
        for (const void* k : {pick_w16_dot_bal<false>(1), pick_w16_dot_bal<false>(2),
                              pick_w16_dot_bal<true>(1), pick_w16_dot_bal<true>(2)})
            (void)hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kW16BLdsMax);
        (void)hipGetLastError();
    });
}

}  // namespace

extern "C" int w16a16_workspace_bytes(int M, int N, int K, size_t* bytes) {
    if (!bytes) return W4A16_ERR_NULL;
    if (int rc = check_w16(M, N, K)) return rc;
    *bytes = w16_workspace(w16_plan(M, N, K), M, N);
    return W4A16_OK;
}

extern "C" int w16a16_gemv(const void* x, const void* w, int dtype, void* y, int y_dtype, int M,
                           int N, int K, void* workspace, size_t workspace_bytes,
                           w4a16_stream_t stream) {
    if (!x || !w || !y) return W4A16_ERR_NULL;
    if (dtype != W4A16_F16 && dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    if (y_dtype != W4A16_F32 && y_dtype != W4A16_F16 && y_dtype != W4A16_BF16)
        return W4A16_ERR_DTYPE;
    if (int rc = check_w16(M, N, K)) return rc;
    if (!w4h::aligned16(x) || !w4h::aligned16(w) || !w4h::aligned16(y)) return W4A16_ERR_ALIGN;
    const W16Plan p = w16_plan(M, N, K);
    const size_t need = w16_workspace(p, M, N);
    if (need) {
        if (!workspace) return W4A16_ERR_NULL;
        if (workspace_bytes < need) return W4A16_ERR_WORKSPACE;
        if (!w4h::aligned16(workspace)) return W4A16_ERR_ALIGN;
    }
    const bool bf16 = dtype == W4A16_BF16;
    const int U = (K + kUnitK - 1) / kUnitK;
    const int T = pad_n(N) / kTileN;
    W16Launch l{M, N, K, U, p.split, T, y_dtype};
    hipStream_t st = (hipStream_t)stream;
    if (p.bal) {
        allow_w16_lds();
        w4h::begin_launches();
        const void* k = bf16 ? pick_w16_dot_bal<true>(M) : pick_w16_dot_bal<false>(M);
        const int mr = M <= 1 ? 1 : 2;
        const int C = w4h::cu_count();
        hipLaunchKernelGGL((w16_kernel_t)k, dim3(C), dim3(64 * kW16BWaves), p.lds, st, l.M, l.N, l.K,
                           l.U, l.S, l.T, C, (const uint16_t*)x, (const uint16_t*)w, y, l);
        w4h::set_last_variant("w16_dotbal %s kernel=w16_dot_bal_kernel<%s, %d> workgroups=%d slices=1 lds=%zu",
                              bf16 ? "bf16" : "f16", bf16 ? "true" : "false", mr, C, p.lds);
        return w4h::launch_status();
    }
    if (p.dot) {
        allow_w16_lds();
        w4h::begin_launches();
        const void* k = bf16 ? pick_w16_dot<true>(M) : pick_w16_dot<false>(M);
        const int mr = M <= 1 ? 1 : M <= 2 ? 2 : 4;
        hipLaunchKernelGGL((w16_kernel_t)k, dim3(T), dim3(64 * kW16DWaves), p.lds, st, l.M, l.N, l.K,
                           l.U, l.S, l.T, T, (const uint16_t*)x, (const uint16_t*)w, y, l);
        w4h::set_last_variant("w16_dot %s kernel=w16_dot_kernel<%s, %d> tiles=%d slices=1 lds=%zu",
                              bf16 ? "bf16" : "f16", bf16 ? "true" : "false", mr, T, p.lds);
        return w4h::launch_status();
    }
    if (p.ksplit) {
        allow_w16_lds();
        w4h::begin_launches();
        hipLaunchKernelGGL(bf16 ? w16_ksplit_kernel<true> : w16_ksplit_kernel<false>, dim3(T),
                           dim3(64 * kW16KWaves), p.lds, st, l.M, l.N, l.K, l.U, l.S, l.T, T,
                           (const uint16_t*)x, (const uint16_t*)w, y, l);
        w4h::set_last_variant("w16_mfma16 %s kernel=w16_ksplit_kernel<%s> tiles=%d slices=1 lds=%zu",
                              bf16 ? "bf16" : "f16", bf16 ? "true" : "false", T, p.lds);
        return w4h::launch_status();
    }
    w4h::begin_launches();
    hipLaunchKernelGGL(bf16 ? pick_w16_rb<true>(p.rb) : pick_w16_rb<false>(p.rb),
                       dim3((unsigned)p.workgroups, p.split), dim3(64 * kW16Waves), 0, st,
                       l.M, l.N, l.K, l.U, l.S, l.T, (int)p.workgroups, (const uint16_t*)x,
                       (const uint16_t*)w, p.split > 1 ? w4h::ws_part(workspace) : y, l);
    if (p.split > 1) w4h::launch_merge(w4h::ws_part(workspace), y, y_dtype, nullptr, W4A16_F32, M, N, p.split, st);
    w4h::set_last_variant("w16_mfma16 %s kernel=w16_gemv_kernel<%s, %d> tiles=%d slices=%d "
                          "workgroups=%lld",
                          bf16 ? "bf16" : "f16", bf16 ? "true" : "false", p.rb, T, p.split,
                          p.workgroups);
    return w4h::launch_status();
}
