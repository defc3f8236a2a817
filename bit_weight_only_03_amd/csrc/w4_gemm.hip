// w4_gemm.hip -- the M-tiled path of y[M,N] = x[M,K] . ((q - z) * s)[K,N] on
// gfx950, for up to 64 activation rows (several tokens of a batch or several
// speculative drafts at once).
//
// The GEMV kernel gives each wave a range of K and stages that range of x
// per wave, so its LDS holds M x K halves per workgroup: fine for a few rows,
// impossible at M = 64 (655 KB for K = 5120).  Here the roles turn around.
// Each wave owns TN 16-column tiles over the workgroup's whole K range, and
// the workgroup streams x through LDS one 128-k unit at a time, shared by all
// its waves (double-buffered: the next unit is loaded while the current one
// is multiplied, one barrier per unit).  Every weight is still read from HBM
// once and dequantized once per call (the Z100 article, section 五: dequantize
// once, use for every row), then multiplied with up to four 16-row blocks of
// x: one v_mfma_f32_16x16x32 per row block and 32-k step.  The crossover
// against the GEMV kernel (which dispatches which rows) is measured, not
// assumed (NINFER ternary tuning page, sections 五 and 七: the small-T ladder
// rungs were placed by measurement).
//
// Weights, scales and zero points use the device layout of w4_pack and the
// same register dequantization as the GEMV (common.h).  Partials of a K split
// go to the caller's workspace [S][M][N] and are added in slice order by the
// GEMV file's merge kernel.
#include <stdlib.h>

#include "common.h"

using namespace w4k;

namespace {

constexpr int kGemmWaves = 4;             // waves per workgroup
// Units of weight loads in flight per wave (even: the x register sets and
// LDS buffers alternate with the ring position).  Four, or a guard that
// skips the tail units of the last ring turn, measured slower (gate_up at
// M = 64: 57 us with two, 70 us with four, 61 us guarded; with x loaded two
// units ahead, four again lost: 71 us against 61 us).
constexpr int kRing = 2;
constexpr int kXStride = kUnitK + 8;      // halves per staged x row (+16 B spreads rows over banks)

struct GemmLaunch {
    int M, N, K;
    int U;   // 128-k units per column (K rounded up)
    int S;   // K slices
    int T;   // 16-column tiles
    int out_dtype;
    const void* res;   // residual added to y (unsplit calls), or null
    int res_dtype;
};

// A unit's loads for one tile: 16 weight bytes per lane, plus the scale and
// zero-point words of the groups the unit touches.
template <int NG>
struct GSlot {
    u32x4_t w;
    uint32_t s[NG];
    uint32_t z[NG];
};
// MXFP4: 16 weight bytes plus the dword of the unit's four E8M0 codes.
struct GSlotMx {
    u32x4_t w;
    uint32_t s;
};
template <int NG, bool MX>
struct GSlotSel {
    using type = GSlot<NG>;
};
template <int NG>
struct GSlotSel<NG, true> {
    using type = GSlotMx;
};

// One workgroup per (4 x TN tiles, K slice).  Wave w owns tiles
// [t0 + w TN, t0 + (w + 1) TN).  Per 128-k unit u of the slice:
//   - all threads have staged x[0:M, u's 128 k] in LDS buffer u % 2 (zeros
//     past K and in rows >= M, whose outputs are never stored);
//   - every wave multiplies its tiles' unit u, whose loads were issued kRing
//     units earlier (a ring of kRing units per tile), while the x of unit
//     u+2 is loading into one of two register sets; then it stores the x of
//     unit u+1 (loaded one unit earlier) into the other LDS buffer and the
//     workgroup meets at a barrier.  Loading x two units ahead keeps that
//     store's wait off the weight loads: loads complete in issue order, and
//     x of unit u+1 went out before the weights of unit u+1, so the store
//     waits for nothing issued after unit u's weights.
// Units past the slice (and tiles past N) load as zeros -- q = z = 0, s = +0 --
// and add exactly 0 against the finite x, so the loop body is uniform.
// MX = true takes MXFP4 weights (mxfp4.hip's layout, instantiated with
// SPG = 4): no zero points, each unit's four block scales folded into the
// element conversion or applied step by step (mx_unit in common.h).
template <bool BF16, int SPG, int RB, int TN, bool MX = false>
__global__ __launch_bounds__(256) void w4_gemm_kernel(int M_, int N_, int K_, int U_, int S_, int T_,
                                                      const uint16_t* __restrict__ x,
                                                      const u32x4_t* __restrict__ qdev,
                                                      const uint16_t* __restrict__ sdev,
                                                      const uint32_t* __restrict__ zdev,
                                                      void* out, GemmLaunch a_in) {
    // The fields a wave needs first arrive as leading scalars (with the four
    // input pointers: ten arguments, 14 dwords), which the build compiles as
    // preloaded into SGPRs at wave launch; the rest stays in the struct.
    GemmLaunch a = a_in;
    a.M = M_;
    a.N = N_;
    a.K = K_;
    a.U = U_;
    a.S = S_;
    a.T = T_;
    constexpr int NG = SPG >= 4 ? 1 : 4 / SPG;    // groups per unit
    constexpr int SPU = SPG >= 4 ? 4 : SPG;       // 32-k steps per group inside one unit
    constexpr int ROWS = 16 * RB;
    constexpr int XCH = ROWS * (kUnitK / 8);      // 16-byte chunks of one staged unit
    constexpr int XPT = XCH / 256;                // chunks per thread (= RB)
    using SlotT = typename GSlotSel<NG, MX>::type;
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][ROWS][kXStride];

    const int M = a.M, N = a.N, K = a.K, U = a.U, T = a.T;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int c = lane & 15, kc = lane >> 4;
    const int split = blockIdx.y;
    int r0 = 0, r1 = U;                                                   // the slice's units
    if (a.S != 1) {   // (no division on the way to an unsplit launch's first load)
        r0 = split * U / a.S;
        r1 = (split + 1) * U / a.S;
    }
    const int nu = r1 - r0;
    const int tw = (blockIdx.x * kGemmWaves + wave) * TN;                // the wave's first tile
    const int nt = T - tw < 0 ? 0 : (T - tw < TN ? T - tw : TN);         // its tiles inside N
    const int Gp = U * kUnitK / (SPG * 32);

    // Buffer resources over the wave's tiles; a missing unit or tile takes an
    // offset at the resource's end, so each of its lanes reads zeros.
    // MXFP4: scales are [T][U][16] dwords and there are no zero points.
    const uint32_t wend = (uint32_t)nt * U * 1024u,
                   send = MX ? (uint32_t)nt * U * 64u : (uint32_t)nt * Gp * 32u,
                   zend = MX ? 0u : (uint32_t)nt * Gp * 8u;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(qdev + (size_t)tw * U * kLanes, wend);
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(MX ? (const void*)((const uint8_t*)sdev + (size_t)tw * U * 64u)
                     : (const void*)(sdev + (size_t)tw * Gp * kTileN),
                  send);
    const __amdgpu_buffer_rsrc_t rz =
        make_rsrc(MX ? (const void*)qdev : (const void*)(zdev + (size_t)tw * Gp * 2), zend);
    const uint32_t xend = (uint32_t)M * (uint32_t)K * 2u;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, xend);
    const uint32_t wlane = (uint32_t)lane * 16u, slane = (uint32_t)c * 2u,
                   zlane = (uint32_t)(c >> 3) * 4u;

    auto load_unit = [&](int i, SlotT (&r)[TN]) {   // unit r0 + i of every tile
        const int u = r0 + i;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const bool valid = i < nu && j < nt;
            r[j].w = bitcast<u32x4_t>(__builtin_amdgcn_raw_buffer_load_b128(
                rw, valid ? wlane + (uint32_t)(j * U + u) * 1024u : wend, 0, kAuxNT));
            if constexpr (MX) {
                r[j].s = __builtin_amdgcn_raw_buffer_load_b32(
                    rs, valid ? (uint32_t)c * 4u + (uint32_t)(j * U + u) * 64u : send, 0, 0);
            } else {
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    const int g = j * Gp + (u * 4) / SPG + gi;
                    r[j].s[gi] = __builtin_amdgcn_raw_buffer_load_b16(
                        rs, valid ? slane + (uint32_t)g * 32u : send, 0, 0);
                    r[j].z[gi] = __builtin_amdgcn_raw_buffer_load_b32(
                        rz, valid ? zlane + (uint32_t)g * 8u : zend, 0, 0);
                }
            }
        }
    };

    // x of unit r0 + i: chunk ch = row ch / 16, k offset 8 (ch % 16).
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
    // bf16 x with 4-bit weights is stored as fp16 (exact over fp16's range,
    // common.h), so the products take the exact fp16 q - z.
    auto store_x = [&](int b, int slot) {
#pragma unroll
        for (int p = 0; p < XPT; ++p) {
            const int ch = threadIdx.x + 256 * p;
            if constexpr (BF16 && !MX)
                *(u32x4_t*)&xs[b][ch >> 4][8 * (ch & 15)] = bf16x8_to_f16x8(xr[slot][p]);
            else
                *(u32x4_t*)&xs[b][ch >> 4][8 * (ch & 15)] = xr[slot][p];
        }
    };

    const int zshift = 4 * (c & 7);
    const uint32_t magic = opaque_v(0x64006400u);   // fp16 1024.0 pairs
    float4_t total[TN][RB];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) total[j][rb] = float4_t{0.f, 0.f, 0.f, 0.f};

    // MXFP4: per unit, every step's elements convert once per tile and serve
    // the RB row blocks; the steps chain with the scales folded in, or (for a
    // wave with any wide unit) each step's sums take their own scale.
    auto compute_mx = [&](const auto& r, int b) {   // generic: compiled for MX only
        MxUnit mu[TN];
        bool wide = false;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            mu[j] = mx_unit(r[j].s);
            wide = wide || mu[j].wide;
        }
        auto bop = [&](int j, int st, float sc) {
            if constexpr (BF16)
                return bitcast<u32x4_t>(fp4x8_to_bf16(r[j].w[st], sc));
            else
                return bitcast<u32x4_t>(fp4x8_to_f16(r[j].w[st], sc));
        };
        auto mfma = [&](const u32x4_t& av, const u32x4_t& bq, float4_t acc) {
            if constexpr (BF16)
                return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8_t>(av),
                                                               bitcast<bf16x8_t>(bq), acc, 0, 0, 0);
            else
                return __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<half8_t>(av),
                                                              bitcast<half8_t>(bq), acc, 0, 0, 0);
        };
        if (__builtin_amdgcn_ballot_w64(wide) == 0) {
            float4_t acc[TN][RB];
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) acc[j][rb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                u32x4_t av[RB];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    av[rb] = *(const u32x4_t*)&xs[b][16 * rb + c][32 * st + 8 * kc];
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const u32x4_t bq = bop(j, st, mx_fold_scale(mu[j].e[st], mu[j].emax));
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) acc[j][rb] = mfma(av[rb], bq, acc[j][rb]);
                }
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const float sf = mx_unit_scale(mu[j].emax);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        total[j][rb][q] = __builtin_fmaf(sf, acc[j][rb][q], total[j][rb][q]);
            }
        } else {
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                u32x4_t av[RB];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    av[rb] = *(const u32x4_t*)&xs[b][16 * rb + c][32 * st + 8 * kc];
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const u32x4_t bq = bop(j, st, 1.0f);
                    const float sf = e8m0_to_f32(mu[j].e[st]);
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
                        const float4_t acc = mfma(av[rb], bq, float4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            total[j][rb][q] = __builtin_fmaf(sf, acc[q], total[j][rb][q]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);   // one step's sums live at a time
            }
        }
    };

    auto compute = [&](const SlotT (&r)[TN], int b) {
        if constexpr (MX) {
            compute_mx(r, b);
            return;
        } else {
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            float4_t acc[TN][RB];
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) acc[j][rb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int js = 0; js < SPU; ++js) {
                const int st = gi * SPU + js;   // 32-k step inside the unit
                u32x4_t av[RB];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    av[rb] = *(const u32x4_t*)&xs[b][16 * rb + c][32 * st + 8 * kc];
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const uint32_t zq = (r[j].z[gi] >> zshift) & 15u;
                    uint32_t nz1024 = 0xE400u + zq;          // fp16 -(1024 + z)
                    nz1024 |= nz1024 << 16;
                    uint32_t nz64 = 0xD400u + (zq << 4);     // fp16 -(64 + z)
                    nz64 |= nz64 << 16;
                    const half8_t bq = dequant_f16(r[j].w[st], magic, nz1024, nz64);
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
                        acc[j][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            bitcast<half8_t>(av[rb]), bq, acc[j][rb], 0, 0, 0);
                }
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const float sf = f16_bits_to_f32((uint16_t)r[j].s[gi]);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        total[j][rb][q] = __builtin_fmaf(sf, acc[j][rb][q], total[j][rb][q]);
            }
        }
        }
    };

    // Prologue: loads of the first kRing units, x of unit 0 staged.
    SlotT ring[kRing][TN];
    load_x(0, 0);
#pragma unroll
    for (int d = 0; d < kRing; ++d) load_unit(d, ring[d]);
    load_x(1, 1);
    store_x(0, 0);
    __syncthreads();
    for (int i = 0; i < nu; i += kRing) {
#pragma unroll
        for (int d = 0; d < kRing; ++d) {
            load_x(i + d + 2, d & 1);           // slot (i + d) % 2: x of unit i + d is in LDS
            compute(ring[d], d & 1);            // unit i + d sits in buffer (i + d) % 2
            load_unit(i + d + kRing, ring[d]);
            store_x((d + 1) & 1, (d + 1) & 1);  // x of unit i + d + 1, loaded one unit ago
            __syncthreads();
        }
    }

    // Lane l holds rows 16 rb + 4 (l / 16) + q of column l % 16 of each tile.
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int n = (tw + j) * kTileN + c;
        if (j >= nt || n >= N) continue;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = 16 * rb + 4 * kc + q;
                if (m >= M) continue;
                const size_t o = (size_t)m * N + n;
                if (a.S > 1)
                    ((float*)out)[(size_t)split * M * N + o] = total[j][rb][q];
                else
                    store_out(out, a.out_dtype, o, add_residual(total[j][rb][q], a.res, a.res_dtype, o));
            }
    }
}

typedef void (*gemm_kernel_t)(int, int, int, int, int, int, const uint16_t*, const u32x4_t*,
                              const uint16_t*, const uint32_t*, void*, GemmLaunch);

template <bool BF16, int SPG, int TN, bool MX = false>
gemm_kernel_t pick_rb(int rb) {
    switch (rb) {
        case 1: return w4_gemm_kernel<BF16, SPG, 1, TN, MX>;
        case 2: return w4_gemm_kernel<BF16, SPG, 2, TN, MX>;
        case 3: return w4_gemm_kernel<BF16, SPG, 3, TN, MX>;
        default: return w4_gemm_kernel<BF16, SPG, 4, TN, MX>;
    }
}

template <bool BF16, int SPG>
gemm_kernel_t pick_tn(int rb, int tn) {
    return tn == 1 ? pick_rb<BF16, SPG, 1>(rb) : pick_rb<BF16, SPG, 2>(rb);
}

// MXFP4 (register plan of g = 128).
gemm_kernel_t pick_gemm_mx(bool bf16, int rb, int tn) {
    if (bf16) return tn == 1 ? pick_rb<true, 4, 1, true>(rb) : pick_rb<true, 4, 2, true>(rb);
    return tn == 1 ? pick_rb<false, 4, 1, true>(rb) : pick_rb<false, 4, 2, true>(rb);
}

gemm_kernel_t pick_gemm(bool bf16, int group, int rb, int tn) {
    switch (group) {
        case 32: return bf16 ? pick_tn<true, 1>(rb, tn) : pick_tn<false, 1>(rb, tn);
        case 64: return bf16 ? pick_tn<true, 2>(rb, tn) : pick_tn<false, 2>(rb, tn);
        case 128: return bf16 ? pick_tn<true, 4>(rb, tn) : pick_tn<false, 4>(rb, tn);
        default: return bf16 ? pick_tn<true, 8>(rb, tn) : pick_tn<false, 8>(rb, tn);
    }
}

}  // namespace

namespace w4h {

// Plan of the M-tiled path for one shape: row blocks, tiles per wave, K
// slices (so that the grid gives every CU at least two workgroups while each
// slice keeps at least eight units).
GemmPlan gemm_plan(int M, int N, int K, int group, int cus) {
    (void)group;   // every group size has the same unit and register plan
    GemmPlan p;
    const int U = (K + kUnitK - 1) / kUnitK;
    const int T = pad_n(N) / kTileN;
    p.rb = (M + 15) / 16;
    // One tile per wave: the two-tile build needs 212 VGPRs (two waves per
    // SIMD) and measured slower (gate_up at M = 64: 64.9 us against 57.6 us).
    p.tn = 1;
    if (const int t = overrides().gemm_tn; t == 1 || t == 2) p.tn = t;
    const long long cols = (T + kGemmWaves * p.tn - 1) / (kGemmWaves * p.tn);
    p.split = 1;
    while (cols * p.split < 2LL * cus && U / (2 * p.split) >= 8 && p.split < kMaxSplitGemm) p.split *= 2;
    if (const int s = overrides().gemm_split; s >= 1 && s <= U && s <= kMaxSplitGemm) p.split = s;
    p.workgroups = cols;
    return p;
}

int gemm_launch(const GemmPlan& p, const void* x, bool bf16, const void* qweight, const void* scales,
                const void* zeros, void* y, int y_dtype, const void* res, int res_dtype, int M, int N,
                int K, int group, void* workspace, hipStream_t st, bool mx) {
    const int U = (K + kUnitK - 1) / kUnitK;
    const int T = pad_n(N) / kTileN;
    GemmLaunch l{M, N, K, U, p.split, T, y_dtype, res, res_dtype};
    gemm_kernel_t k = mx ? pick_gemm_mx(bf16, p.rb, p.tn) : pick_gemm(bf16, group, p.rb, p.tn);
    hipLaunchKernelGGL(k, dim3((unsigned)p.workgroups, p.split), dim3(64 * kGemmWaves), 0, st,
                       l.M, l.N, l.K, l.U, l.S, l.T, (const uint16_t*)x, (const u32x4_t*)qweight, (const uint16_t*)scales,
                       (const uint32_t*)zeros, p.split > 1 ? workspace : y, l);
    return W4A16_OK;
}

}  // namespace w4h
