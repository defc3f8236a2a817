// w4_gemv.hip -- y[M,N] = x[M,K] . ((q - z) * s)[K,N] on gfx950, M = 1..16.
//
// The layer is bound by HBM bandwidth: every call streams all packed weights
// once (Ninfer V100 article, haowenji.com, section 三), so the kernel is built
// around that stream and keeps the per-weight ALU work small (the ternary
// tuning page, section 六, found decode arithmetic to be the whole gap to the
// bandwidth ceiling; the Z100 vLLM article, section 五, lost 27% to zero-point
// unpacking).
//
// Work decomposition.  One workgroup owns one 16-column tile (and, when the
// tile count is too small to fill the GPU, one of S slices of K); its waves
// split the tile's 128-k units evenly.  Per unit every lane issues one
// non-temporal 16-byte load (1 KiB per wave, fully coalesced), so a wave
// keeps D units in flight in a register ring (software pipelining of the
// weight stream: Ninfer V100 article, section 十四, issue several loads
// before computing).
//
// Dequantization in registers.  A dword of 8 nibbles becomes four fp16 pairs
// with one AND-OR against the magic exponent of 1024 (the "place the integer
// in a 16-bit float's mantissa and subtract a constant" trick of the Ninfer
// V100 article, section 十), then one packed add of -(1024 + z) (or a packed
// fma by 1/16 and -(64 + z) for the nibbles in the high half of a byte), which
// gives q - z exactly.  For bf16 activations the pairs are 128 + q and the
// zero point enters through a second MFMA against the constant operand
// -(128 + z), which also keeps every product exact.
//
// Products.  The dequantized pairs are the B operand of v_mfma_f32_16x16x32
// (lane l supplies column l % 16 and the k-block l / 16) and the x rows are
// the A operand (lane l supplies row l % 16), so one instruction covers 16
// columns x 32 k for up to 16 rows: the weights are streamed once for every
// row (Z100 article, section 五), and M = 1..16 all cost the same VALU work.
// The fp32 accumulator of each group is scaled by s once per group and added
// to the running total (fp32 throughout).
//
// Reduction.  The waves of a workgroup combine their partial sums through LDS
// in a fixed order; with a K split the slices write fp32 partials to the
// caller's workspace and a second kernel adds them in slice order.  No atomics
// anywhere, so results are bitwise reproducible (Ninfer V100 article, section
// 十四: add in a fixed order so both sides agree bit for bit; the qengine
// article: keep split partials in fp32).
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>

#include "common.h"

using namespace w4k;

namespace {

constexpr int kMaxWaves = 8;     // waves per workgroup (launch bound 512 threads)
constexpr int kMaxRows = 16;     // rows per MFMA

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return bitcast<half2_t>(v); }
__device__ __forceinline__ uint32_t as_u(half2_t v) { return bitcast<uint32_t>(v); }

// (a & mask) | (b & ~mask) in one v_bfi_b32.  The magic exponents below never
// overlap the nibble masks, so bfi(mask, d, magic) = (d & mask) | magic.
__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t a, uint32_t b) {
    uint32_t r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(mask), "v"(a), "v"(b));
    return r;
}

// B operand (8 fp16 = q - z, exact) for the 8 weights of one device dword.
__device__ __forceinline__ half8_t dequant_f16(uint32_t d, uint32_t magic, uint32_t nz1024,
                                               uint32_t nz64) {
    const half2_t sixteenth = as_h2(0x2C002C00u);  // fp16 1/16
    const uint32_t t = d >> 8;
    const uint32_t p0 = bfi(0x000F000Fu, d, magic);  // 1024 + q   (elements 0, 1)
    const uint32_t p1 = bfi(0x00F000F0u, d, magic);  // 1024 + 16q (elements 2, 3)
    const uint32_t p2 = bfi(0x000F000Fu, t, magic);  // 1024 + q   (elements 4, 5)
    const uint32_t p3 = bfi(0x00F000F0u, t, magic);  // 1024 + 16q (elements 6, 7)
    const half2_t w0 = as_h2(p0) + as_h2(nz1024);
    const half2_t w1 = __builtin_elementwise_fma(as_h2(p1), sixteenth, as_h2(nz64));
    const half2_t w2 = as_h2(p2) + as_h2(nz1024);
    const half2_t w3 = __builtin_elementwise_fma(as_h2(p3), sixteenth, as_h2(nz64));
    u32x4_t v = {as_u(w0), as_u(w1), as_u(w2), as_u(w3)};
    return bitcast<half8_t>(v);
}

// B operand (8 bf16 = 128 + q, exact) for the 8 weights of one device dword.
__device__ __forceinline__ bf16x8_t biased_bf16(uint32_t d, uint32_t magic) {
    u32x4_t v = {bfi(0x000F000Fu, d, magic), bfi(0x000F000Fu, d >> 4, magic),
                 bfi(0x000F000Fu, d >> 8, magic), bfi(0x000F000Fu, d >> 12, magic)};
    return bitcast<bf16x8_t>(v);
}

// One ring slot: a unit's 16 weight bytes for this lane plus the scale and
// zero-point words of the groups it touches.
template <int NG>
struct Slot {
    u32x4_t w;
    uint32_t s[NG];
    uint32_t z[NG];
};

// Steps (32-k slices) per group SPG = group / 32; NG = groups touched per unit.
template <bool BF16, int SPG, int D>
__global__ __launch_bounds__(512) void w4_gemv_kernel(
    const uint16_t* __restrict__ x, const u32x4_t* __restrict__ qdev,
    const uint16_t* __restrict__ sdev, const uint32_t* __restrict__ zdev, void* __restrict__ out,
    int out_dtype, int M, int N, int K, int S) {
    static_assert(D % 2 == 0, "x double buffer alternates with the ring index");
    constexpr int NG = SPG >= 4 ? 1 : 4 / SPG;          // groups per unit
    constexpr int SPU = SPG >= 4 ? 4 : SPG;             // steps per group inside one unit
    __shared__ float red[kMaxWaves][kMaxRows][kTileN];

    const int lane = threadIdx.x & 63, nw = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int t = blockIdx.x, split = blockIdx.y;
    const int U = (K + kUnitK - 1) / kUnitK;
    const int Gp = U * kUnitK / (SPG * 32);
    const int su0 = (int)((long long)split * U / S);
    const int su1 = (int)((long long)(split + 1) * U / S);
    const int u0 = su0 + wave * (su1 - su0) / nw;
    const int u1 = su0 + (wave + 1) * (su1 - su0) / nw;
    const int c = lane & 15, kc = lane >> 4;
    // Per-workgroup buffer resources.  The weights, scales and zero points of
    // tile t are contiguous; x is addressed as a whole so that the padded k
    // tail reads either the next row (finite values times weights that are
    // exactly 0) or, past the end of x, zeros from the range check.
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(qdev + (size_t)t * U * kLanes, (uint32_t)U * 1024u);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(sdev + (size_t)t * Gp * kTileN, (uint32_t)Gp * 32u);
    const __amdgpu_buffer_rsrc_t rz = make_rsrc(zdev + (size_t)t * Gp * 2, (uint32_t)Gp * 8u);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
    const uint32_t wlane = (uint32_t)lane * 16u;
    const uint32_t slane = (uint32_t)c * 2u;
    const uint32_t zlane = (uint32_t)(c >> 3) * 4u;
    // Lane l supplies x row l % 16 to the A operand.  Rows >= M only feed
    // output rows that are never stored, so those lanes re-read row M - 1.
    const int xm = c < M ? c : M - 1;
    const uint32_t xlane = ((uint32_t)xm * (uint32_t)K + 8u * (uint32_t)kc) * 2u;
    const int zshift = 4 * (c & 7);
    const uint32_t magic = BF16 ? 0x43004300u : 0x64006400u;   // 128.0 / 1024.0 pairs

    auto load_slot = [&](int u, Slot<NG>& r) {
        r.w = bitcast<u32x4_t>(__builtin_amdgcn_raw_buffer_load_b128(rw, wlane, u * 1024, kAuxNT));
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            const int g = (u * 4) / SPG + gi;
            r.s[gi] = __builtin_amdgcn_raw_buffer_load_b16(rs, slane, g * 32, 0);
            r.z[gi] = __builtin_amdgcn_raw_buffer_load_b32(rz, zlane, g * 8, 0);
        }
    };
    auto load_x = [&](int u, u32x4_t (&xa)[4]) {
        const uint32_t off = xlane + (uint32_t)u * (kUnitK * 2);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            xa[j] = bitcast<u32x4_t>(__builtin_amdgcn_raw_buffer_load_b128(rx, off + 64u * j, 0, 0));
    };

    float4_t total = {0.f, 0.f, 0.f, 0.f};
    Slot<NG> ring[D];
    u32x4_t xb[2][4];
#pragma unroll
    for (int i = 0; i < D; ++i)
        if (u0 + i < u1) load_slot(u0 + i, ring[i]);
    if (u0 < u1) load_x(u0, xb[0]);

    for (int ub = u0; ub < u1; ub += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            const int u = ub + i;
            if (u < u1) {
                u32x4_t (&xcur)[4] = xb[i & 1];
                if (u + 1 < u1) load_x(u + 1, xb[(i + 1) & 1]);
                Slot<NG>& sl = ring[i];
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    const uint32_t zq = (sl.z[gi] >> zshift) & 15u;
                    float4_t acc = {0.f, 0.f, 0.f, 0.f};
                    if constexpr (!BF16) {
                        uint32_t nz1024 = 0xE400u + zq;          // fp16 -(1024 + z)
                        nz1024 |= nz1024 << 16;
                        uint32_t nz64 = 0xD400u + (zq << 4);     // fp16 -(64 + z)
                        nz64 |= nz64 << 16;
#pragma unroll
                        for (int js = 0; js < SPU; ++js) {
                            const int j = gi * SPU + js;
                            const half8_t b = dequant_f16(sl.w[j], magic, nz1024, nz64);
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                bitcast<half8_t>(xcur[j]), b, acc, 0, 0, 0);
                        }
                    } else {
                        uint32_t nb = 0xC300u + zq;              // bf16 -(128 + z)
                        nb |= nb << 16;
                        const bf16x8_t bias = bitcast<bf16x8_t>(u32x4_t{nb, nb, nb, nb});
#pragma unroll
                        for (int js = 0; js < SPU; ++js) {
                            const int j = gi * SPU + js;
                            const bf16x8_t a = bitcast<bf16x8_t>(xcur[j]);
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                a, biased_bf16(sl.w[j], magic), acc, 0, 0, 0);
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bias, acc, 0, 0, 0);
                        }
                    }
                    const float sf = f16_bits_to_f32((uint16_t)sl.s[gi]);
                    total[0] = __builtin_fmaf(sf, acc[0], total[0]);
                    total[1] = __builtin_fmaf(sf, acc[1], total[1]);
                    total[2] = __builtin_fmaf(sf, acc[2], total[2]);
                    total[3] = __builtin_fmaf(sf, acc[3], total[3]);
                }
                // Refill the slot just consumed with the unit D ahead.
                if (u + D < u1) load_slot(u + D, sl);
            }
        }
    }

    // Lane l holds rows 4*(l/16) + r of column l % 16.
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

// y = sum over slices of the fp32 partials, in slice order.
__global__ void splitk_merge_kernel(const float* __restrict__ ws, void* __restrict__ y,
                                    int out_dtype, int MN, int S) {
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

// ------------------------------------------------------------------ dispatch

struct Plan {
    int waves;   // waves per workgroup
    int split;   // K slices (grid.y)
    int depth;   // weight ring depth
};

struct Tuning {
    int waves = 0, split = 0, depth = 0;  // 0 = automatic
};

const Tuning& tuning() {
    // Overrides for A/B measurement only, read once per process (decode-path
    // choices are frozen: NINFER tuning page, section 七).
    static Tuning t;
    static std::once_flag once;
    std::call_once(once, [] {
        if (const char* e = getenv("W4A16_WAVES")) t.waves = atoi(e);
        if (const char* e = getenv("W4A16_SPLIT")) t.split = atoi(e);
        if (const char* e = getenv("W4A16_DEPTH")) t.depth = atoi(e);
    });
    return t;
}

Plan make_plan(int M, int N, int K, int unit_k) {
    (void)M;
    const int U = (K + unit_k - 1) / unit_k;
    const int T = pad_n(N) / kTileN;
    Plan p;
    // About four units per wave, at most eight waves per workgroup.
    p.waves = (U + 3) / 4;
    if (p.waves > kMaxWaves) p.waves = kMaxWaves;
    if (p.waves < 1) p.waves = 1;
    // Split K across workgroups only when the tiles alone cannot give every
    // CU a workgroup (narrow N: one GPU's share of a column-split layer), and
    // keep at least two units per wave (a split with too little k per slice
    // loses: NINFER tuning page, section 五, item 21).
    p.split = 1;
    if (T < 256) {
        int s = (512 + T - 1) / T;
        int smax = U / (2 * p.waves);
        if (smax < 1) smax = 1;
        p.split = s < smax ? s : smax;
    }
    p.depth = 8;
    const Tuning& tu = tuning();
    if (tu.waves >= 1 && tu.waves <= kMaxWaves) p.waves = tu.waves;
    if (tu.split >= 1 && tu.split <= U) p.split = tu.split;
    if (tu.depth == 4 || tu.depth == 8) p.depth = tu.depth;
    return p;
}

typedef void (*w4_kernel_t)(const uint16_t*, const u32x4_t*, const uint16_t*, const uint32_t*,
                            void*, int, int, int, int, int);

template <bool BF16, int D>
w4_kernel_t pick_spg(int group) {
    switch (group) {
        case 32: return w4_gemv_kernel<BF16, 1, D>;
        case 64: return w4_gemv_kernel<BF16, 2, D>;
        case 128: return w4_gemv_kernel<BF16, 4, D>;
        default: return w4_gemv_kernel<BF16, 8, D>;
    }
}

w4_kernel_t pick_kernel(bool bf16, int group, int depth) {
    if (bf16) return depth == 4 ? pick_spg<true, 4>(group) : pick_spg<true, 8>(group);
    return depth == 4 ? pick_spg<false, 4>(group) : pick_spg<false, 8>(group);
}

int check_gemv_args(const void* x, int x_dtype, const void* q, const void* s, const void* z,
                    const void* y, int y_dtype, int M, int N, int K, int group) {
    if (!x || !q || !s || !z || !y) return W4A16_ERR_NULL;
    if (x_dtype != W4A16_F16 && x_dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    if (y_dtype != W4A16_F32 && y_dtype != W4A16_F16 && y_dtype != W4A16_BF16)
        return W4A16_ERR_DTYPE;
    if (M < 1 || M > kMaxRows) return W4A16_ERR_SHAPE;
    int rc = w4h::check_w4_shape(N, K, group);
    if (rc) return rc;
    if (!w4h::aligned16(x) || !w4h::aligned16(q) || !w4h::aligned16(s) || !w4h::aligned16(z) ||
        !w4h::aligned16(y))
        return W4A16_ERR_ALIGN;
    return W4A16_OK;
}

}  // namespace

extern "C" int w4a16_workspace_bytes(int M, int N, int K, int group, size_t* bytes) {
    if (!bytes) return W4A16_ERR_NULL;
    if (M < 1 || M > kMaxRows) return W4A16_ERR_SHAPE;
    int rc = w4h::check_w4_shape(N, K, group);
    if (rc) return rc;
    const Plan p = make_plan(M, N, K, kUnitK);
    *bytes = p.split > 1 ? (size_t)p.split * M * N * sizeof(float) : 0;
    return W4A16_OK;
}

extern "C" int w4a16_gemv(const void* x, int x_dtype, const void* qweight, const void* scales,
                          const void* zeros, void* y, int y_dtype, int M, int N, int K, int group,
                          void* workspace, size_t workspace_bytes, w4a16_stream_t stream) {
    int rc = check_gemv_args(x, x_dtype, qweight, scales, zeros, y, y_dtype, M, N, K, group);
    if (rc) return rc;
    const Plan p = make_plan(M, N, K, kUnitK);
    const size_t need = p.split > 1 ? (size_t)p.split * M * N * sizeof(float) : 0;
    if (need) {
        if (!workspace) return W4A16_ERR_NULL;
        if (workspace_bytes < need) return W4A16_ERR_WORKSPACE;
        if (!w4h::aligned16(workspace)) return W4A16_ERR_ALIGN;
    }
    hipStream_t st = (hipStream_t)stream;
    const int T = pad_n(N) / kTileN;
    const bool bf16 = x_dtype == W4A16_BF16;
    w4_kernel_t k = pick_kernel(bf16, group, p.depth);
    void* out = p.split > 1 ? workspace : y;
    const int odt = p.split > 1 ? W4A16_F32 : y_dtype;
    w4h::begin_launches();
    hipLaunchKernelGGL(k, dim3(T, p.split), dim3(64 * p.waves), 0, st, (const uint16_t*)x,
                       (const u32x4_t*)qweight, (const uint16_t*)scales, (const uint32_t*)zeros,
                       out, odt, M, N, K, p.split);
    if (p.split > 1) {
        const int MN = M * N;
        hipLaunchKernelGGL(splitk_merge_kernel, dim3((MN + 255) / 256), dim3(256), 0, st,
                           (const float*)workspace, y, y_dtype, MN, p.split);
    }
    w4h::set_last_variant("w4_mfma16 %s g%d tiles=%d waves=%d split=%d depth=%d",
                          bf16 ? "bf16" : "f16", group, T, p.waves, p.split, p.depth);
    return w4h::launch_status();
}
