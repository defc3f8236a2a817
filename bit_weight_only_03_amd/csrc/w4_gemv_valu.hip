// w4_gemv_valu.hip -- an MFMA-free form of the 4-bit GEMV, kept to measure
// the choice of matrix cores for the dot products against plain vector ALU
// work (per-lane FMA/dot products with a cross-lane reduction, the form of the
// pages' own GEMVs: Ninfer V100 article, section 十; Z100 vLLM port article,
// sections 四 and 六, which found the M = 8 FP16 GEMV bound by its VALU).  It
// is not the default path: the planner override W4A16_VALU=1 selects it for
// up to 8 rows, for A/B runs only.
//
// Same device layout, work split and x staging as the GEMV of w4_gemv.hip:
// one workgroup per (16-column tile, K slice), 8 waves splitting the slice's
// 128-k units, each wave's x range staged in its own LDS region.  Per unit a
// lane dequantizes its 16 weight bytes (column l % 16, k-block l / 16) into
// four exact fp16 (q - z) pairs per dword with the same and-or / packed-add
// sequence, then forms v_dot2_f32_f16 products against each row's x pairs
// (read from LDS, the four k-blocks broadcast to their 16 lanes) into fp32;
// each group's sum takes its scale once.  At the end the four k-block lanes of
// a column are added with two cross-lane exchanges and the waves through LDS,
// in a fixed order.
#include "common.h"

using namespace w4k;

namespace {

constexpr int kVWaves = 8;

struct ValuLaunch {
    int M, N, K;
    int U;    // 128-k units per column
    int S;    // K slices
    int T;    // 16-column tiles
    int out_dtype;
};

template <int NG>
struct VSlot {
    u32x4_t w;
    uint32_t s[NG];
    uint32_t z[NG];
};

// MR: rows compiled for (M <= MR).
template <bool BF16, int SPG, int UPW, int MR>
__global__ __launch_bounds__(512) void w4_gemv_valu_kernel(const uint16_t* __restrict__ x,
                                                           const u32x4_t* __restrict__ qdev,
                                                           const uint16_t* __restrict__ sdev,
                                                           const uint32_t* __restrict__ zdev, void* out,
                                                           ValuLaunch a) {
    constexpr int NG = SPG >= 4 ? 1 : 4 / SPG;   // groups per unit
    constexpr int SPU = SPG >= 4 ? 4 : SPG;      // 32-k steps per group inside a unit
    constexpr int D = UPW < 8 ? UPW : 8;         // ring slots
    constexpr int LPS = 1 + 2 * NG;              // loads per slot
    constexpr int CPR = UPW * (kUnitK / 8);      // 16-byte chunks of a staged row
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int M = a.M, K = a.K, U = a.U;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = blockIdx.x, split = blockIdx.y;
    const int r0 = split * U / a.S, r1 = (split + 1) * U / a.S;
    const int w0 = r0 + wave * (r1 - r0) / kVWaves, w1 = r0 + (wave + 1) * (r1 - r0) / kVWaves;
    const int nu = w1 - w0;
    const int Gp = U * kUnitK / (SPG * 32);
    const int c = lane & 15, kc = lane >> 4;

    // 1) This wave's x range, [M][CPR chunks] row-major in its LDS region,
    //    straight from memory; chunks past K or past the wave's units are
    //    zeroed (the units past its range have zero weights and must meet
    //    finite x).
    uint8_t* const xsb = smem + (size_t)wave * M * CPR * 16;
    const uint32_t xbytes = (uint32_t)M * (uint32_t)K * 2u;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, xbytes);
    const int live = nu * (kUnitK / 8);
    for (int i = 0; i * 64 < M * CPR; ++i) {   // wave-uniform trip count
        const int ci = i * 64 + lane;
        const int m = ci / CPR, pc = ci % CPR;
        const int kg = w0 * kUnitK + pc * 8;
        if (m < M) {
            if (pc < live && kg < K)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rx, (__attribute__((address_space(3))) void*)(xsb + i * 1024), 16,
                    (uint32_t)(m * K + kg) * 2u, 0, 0, 0);
            else
                *(u32x4_t*)(xsb + (uint32_t)ci * 16u) = u32x4_t{0u, 0u, 0u, 0u};
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (BF16) {   // rewritten as fp16, as in the MFMA GEMV (exact over fp16's range)
        for (int i = 0; i * 64 < M * CPR; ++i) {
            const int ci = i * 64 + lane;
            if (ci / CPR < M && ci % CPR < live) {
                u32x4_t* const p = (u32x4_t*)(xsb + (uint32_t)ci * 16u);
                *p = bf16x8_to_f16x8(*p);
            }
        }
    }

    // 2) Weight ring: straight-line, units past the wave's range read zeros.
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(qdev + (size_t)t * U * kLanes, (uint32_t)U * 1024u);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(sdev + (size_t)t * Gp * kTileN, (uint32_t)Gp * 32u);
    const __amdgpu_buffer_rsrc_t rz = make_rsrc(zdev + (size_t)t * Gp * 2, (uint32_t)Gp * 8u);
    const __amdgpu_buffer_rsrc_t rw0 = make_rsrc(qdev, 0), rs0 = make_rsrc(sdev, 0), rz0 = make_rsrc(zdev, 0);
    const uint32_t wlane = (uint32_t)lane * 16u, slane = (uint32_t)c * 2u, zlane = (uint32_t)(c >> 3) * 4u;
    auto load_slot = [&](int i, VSlot<NG>& r) {
        const bool valid = i < nu;
        const int u = w0 + i;
        r.w = bitcast<u32x4_t>(__builtin_amdgcn_raw_buffer_load_b128(valid ? rw : rw0, wlane,
                                                                     (uint32_t)u * 1024u, kAuxNT));
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            const int g = (u * 4) / SPG + gi;
            r.s[gi] = __builtin_amdgcn_raw_buffer_load_b16(valid ? rs : rs0, slane, (uint32_t)g * 32u, 0);
            r.z[gi] = __builtin_amdgcn_raw_buffer_load_b32(valid ? rz : rz0, zlane, (uint32_t)g * 8u, 0);
        }
    };
    VSlot<NG> ring[D];
#pragma unroll
    for (int i = 0; i < D; ++i) {
        load_slot(i, ring[i]);
        __builtin_amdgcn_sched_barrier(0);
    }

    // 3) Dequantize and take dot products, unit by unit.
    const int zshift = 4 * (c & 7);
    const uint32_t magic = opaque_v(0x64006400u);   // fp16 1024.0 pairs
    float total[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) total[m] = 0.f;
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
        VSlot<NG>& sl = ring[i % D];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            const uint32_t zq = (sl.z[gi] >> zshift) & 15u;
            uint32_t nz1024 = 0xE400u + zq;          // fp16 -(1024 + z)
            nz1024 |= nz1024 << 16;
            uint32_t nz64 = 0xD400u + (zq << 4);     // fp16 -(64 + z)
            nz64 |= nz64 << 16;
            float acc[MR];
#pragma unroll
            for (int m = 0; m < MR; ++m) acc[m] = 0.f;
#pragma unroll
            for (int js = 0; js < SPU; ++js) {
                const int j = gi * SPU + js;
                const u32x4_t b = bitcast<u32x4_t>(dequant_f16(sl.w[j], magic, nz1024, nz64));
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    if (m < M) {   // wave-uniform
                        const u32x4_t xv = *(const u32x4_t*)(xsb + (uint32_t)(m * CPR + i * 16 + 4 * j + kc) * 16u);
#pragma unroll
                        for (int p = 0; p < 4; ++p)
                            acc[m] = __builtin_amdgcn_fdot2(as_h2(xv[p]), as_h2(b[p]), acc[m], false);
                    }
                }
            }
            const float sf = f16_bits_to_f32((uint16_t)sl.s[gi]);
#pragma unroll
            for (int m = 0; m < MR; ++m) total[m] = __builtin_fmaf(sf, acc[m], total[m]);
        }
        if (i + D < UPW) {
            __builtin_amdgcn_sched_barrier(0);
            load_slot(i + D, sl);
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // 4) The four k-block lanes of a column (l, l ^ 16, l ^ 32, l ^ 48), then
    //    the waves through LDS in wave order.
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        total[m] += __shfl_xor(total[m], 16);
        total[m] += __shfl_xor(total[m], 32);
    }
    float* const red = (float*)smem;   // [W][M][16], after every wave is done with x
    __syncthreads();
    if (kc == 0) {
#pragma unroll
        for (int m = 0; m < MR; ++m)
            if (m < M) red[(wave * M + m) * kTileN + c] = total[m];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < M * kTileN; idx += blockDim.x) {
        const int m = idx >> 4, cc = idx & 15;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kVWaves; ++w) v += red[(w * M + m) * kTileN + cc];
        const int n = t * kTileN + cc;
        if (n < a.N) {
            const size_t o = (size_t)m * a.N + n;
            if (a.S > 1)
                ((float*)out)[(size_t)split * M * a.N + o] = v;
            else
                store_out(out, a.out_dtype, o, v);
        }
    }
}

typedef void (*valu_kernel_t)(const uint16_t*, const u32x4_t*, const uint16_t*, const uint32_t*, void*,
                              ValuLaunch);

template <bool BF16, int SPG, int MR>
valu_kernel_t pick_valu_upw(int upw) {
    switch (upw) {
        case 1: return w4_gemv_valu_kernel<BF16, SPG, 1, MR>;
        case 2: return w4_gemv_valu_kernel<BF16, SPG, 2, MR>;
        case 3: return w4_gemv_valu_kernel<BF16, SPG, 3, MR>;
        case 4: return w4_gemv_valu_kernel<BF16, SPG, 4, MR>;
        case 5: return w4_gemv_valu_kernel<BF16, SPG, 5, MR>;
        case 6: return w4_gemv_valu_kernel<BF16, SPG, 6, MR>;
        case 8: return w4_gemv_valu_kernel<BF16, SPG, 8, MR>;
        case 9: return w4_gemv_valu_kernel<BF16, SPG, 9, MR>;
        case 12: return w4_gemv_valu_kernel<BF16, SPG, 12, MR>;
        case 17: return w4_gemv_valu_kernel<BF16, SPG, 17, MR>;
        default: return nullptr;
    }
}

valu_kernel_t pick_valu(bool bf16, int group, int upw, int M) {
    if (group != 64 && group != 128) return nullptr;
    if (M == 1)
        return group == 128 ? (bf16 ? pick_valu_upw<true, 4, 1>(upw) : pick_valu_upw<false, 4, 1>(upw))
                            : (bf16 ? pick_valu_upw<true, 2, 1>(upw) : pick_valu_upw<false, 2, 1>(upw));
    return group == 128 ? (bf16 ? pick_valu_upw<true, 4, 8>(upw) : pick_valu_upw<false, 4, 8>(upw))
                        : (bf16 ? pick_valu_upw<true, 2, 8>(upw) : pick_valu_upw<false, 2, 8>(upw));
}

}  // namespace

namespace w4h {

// Launches the MFMA-free GEMV for a plan of w4_gemv.hip's GEMV planner (one
// tile per workgroup, 8 waves, whole-range x staging of upw units per wave,
// S K slices whose fp32 partials go to `out`).  Returns W4A16_ERR_UNSUPPORTED
// for shapes outside its instantiations (group 64 or 128, M <= 8).
int valu_launch(const void* x, bool bf16, const void* qweight, const void* scales, const void* zeros,
                void* out, int out_dtype, int M, int N, int K, int group, int upw, int S, size_t lds,
                hipStream_t st) {
    if (M > 8) return W4A16_ERR_UNSUPPORTED;
    valu_kernel_t k = pick_valu(bf16, group, upw, M);
    if (!k) return W4A16_ERR_UNSUPPORTED;
    static bool once = [] {
        for (int bf = 0; bf < 2; ++bf)
            for (int g : {64, 128})
                for (int u : {1, 2, 3, 4, 5, 6, 8, 9, 12, 17})
                    for (int m : {1, 8})
                        (void)hipFuncSetAttribute((const void*)pick_valu(bf, g, u, m),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        (void)hipGetLastError();
        return true;
    }();
    (void)once;
    const int U = (K + kUnitK - 1) / kUnitK, T = pad_n(N) / kTileN;
    ValuLaunch l{M, N, K, U, S, T, out_dtype};
    hipLaunchKernelGGL(k, dim3(T, S), dim3(64 * kVWaves), lds, st, (const uint16_t*)x,
                       (const u32x4_t*)qweight, (const uint16_t*)scales, (const uint32_t*)zeros, out, l);
    return W4A16_OK;
}

}  // namespace w4h
