// w4_gemv.hip -- y[M,N] = x[M,K] . ((q - z) * s)[K,N] on gfx950: the GEMV
// kernel for M = 1..16, the entry points (w4a16_gemv, w4a16_gemv_add,
// mxfp4_gemv) that route larger M to the M-tiled kernel (w4_gemm.hip), and
// the split-K merge.  The same kernel also runs MXFP4 weights (MX = true:
// E2M1 elements with one E8M0 scale per 32 k, mxfp4.hip's layout).
//
// The layer is bound by HBM bandwidth: every call streams all packed weights
// once (Ninfer V100 article, haowenji.com, section 三), so the kernel is built
// around that stream and keeps the per-weight ALU work small (the ternary
// tuning page, section 六, found decode arithmetic to be the whole gap to the
// bandwidth ceiling; the Z100 vLLM article, section 五, lost 27% to zero-point
// unpacking).
//
// Work decomposition.  One workgroup owns TPW consecutive 16-column tiles
// (TPW = 1 unless there are many more tiles than the GPU holds at once) and,
// when the tile count is too small to fill the GPU, one of S slices of K; its
// waves split the 128-k units evenly, and each wave walks its units for all
// TPW tiles as one chain.  Per unit every lane issues one non-temporal
// 16-byte load (1 KiB per wave, fully coalesced), so a wave keeps D units in
// flight in a register ring (software pipelining of the weight stream: Ninfer
// V100 article, section 十四, issue several loads before computing).
//
// Dequantization in registers.  A dword of 8 nibbles becomes four fp16 pairs
// with one AND-OR against the magic exponent of 1024 (the "place the integer
// in a 16-bit float's mantissa and subtract a constant" trick of the Ninfer
// V100 article, section 十), then one packed add of -(1024 + z) (or a packed
// fma by 1/16 and -(64 + z) for the nibbles in the high half of a byte), which
// gives q - z exactly.  bf16 activations are rewritten as fp16 in LDS right
// after they are staged (exact over fp16's range, common.h), so they meet the
// same exact fp16 q - z: q = z gives exactly 0 for either activation type.
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

constexpr int kMaxWaves = 8;     // waves per workgroup (the kernel's 512-thread launch bound)
// Balanced plan: 8 waves streaming the workgroup's own tile in chains of UPW
// units, and 8 "extra" waves sharing a piece (of at most 4) of a leftover
// tile in chains of bal_extra_cl(UPW) units: a quarter of 8 UPW units over 8
// waves.
constexpr int kBalFull = 8, kBalExtra = 8, kBalMaxPieces = 4;
constexpr int bal_extra_cl(int upw) { return (upw + 3) / 4; }
// Slots in flight per full wave of the balanced plan (4; 3 with per-unit x
// staging).  Measured on down-shaped layers (graphs of 64 distinct matrices,
// us per call at 1 / 4 rows): 9 slots 11.8 / 14.0, 6 slots 11.5 / 13.2, 4
// slots 11.1 / 12.4, 3 slots 11.2 / 12.2, 2 slots 13.1 / 13.4.  A per-wave
// timeline with 9 slots showed why: each of the grid's 2048 full waves put
// 9 units in the memory queues at once, so a wave's first unit arrived
// after about half of that 18 MB burst (4.8 us median), and the waves'
// dequantization work then bunched up behind it.  Fewer slots per wave keep
// enough bytes in flight for the read rate while each unit waits less.
constexpr int bal_full_ring(bool px) { return px ? 3 : 4; }
constexpr int kCounterStride = 32;   // unsigneds between arrival counters (one per 128-byte line)
// Uneven split of three-tile, 5-unit chains (g = 128 or MXFP4, per-unit x
// staging; see the kernel): waves 0 .. kSkewOld - 1 take 6 units, the later
// ones 4.
constexpr int kSkewOld = 4;
constexpr bool skewed_split(int spg, int upw, int tpw, bool px) {
    return px && spg >= 4 && upw == 5 && tpw == 3;
}
constexpr int skew_units(int w) {   // first unit of wave w's region (= units of waves 0 .. w - 1)
    return w < kSkewOld ? 6 * w : 6 * kSkewOld + 4 * (w - kSkewOld);
}
// The balanced plan's full waves split their tile the same way: the first
// four take UPW + 1 units, the later four UPW - 1 (8 UPW in all).  On the
// down-shaped layers (graphs of 32 distinct matrices, us per call, f16 /
// bf16 x): M = 1 11.2-11.3 / 11.2 -> 11.0 / 10.7-10.9, M = 2 11.0-11.2 /
// 11.9-12.5 -> 10.7 / 11.3-11.4, M = 3 11.2-11.3 / 12.4-12.5 -> 10.9-11.3 /
// 12.0-12.2, M = 4 12.0-12.1 / 12.3-12.5 -> 11.7-11.8 / 12.1-12.2; the
// per-wave timeline had shown waves 4-7 ending 0.9 us (M = 1) and 1.5 us
// (M = 4) after waves 0-3.  UPW + 2 and UPW - 2 spilled registers.
template <int UPW>
constexpr int bal_full_units(int w) {   // first unit of full wave w (w = 8: all of them)
    return w < kSkewOld ? (UPW + 1) * w : (UPW + 1) * kSkewOld + (UPW - 1) * (w - kSkewOld);
}
constexpr int kMaxRows = 16;     // rows per MFMA
constexpr int kMaxXLoads = 16;   // x load instructions per wave: M * 16 UPW <= 64 * 16

// One ring slot: a unit's 16 weight bytes for this lane plus the scale and
// zero-point words of the groups it touches.
template <int NG>
struct Slot {
    u32x4_t w;
    uint32_t s[NG];
    uint32_t z[NG];
};

// MXFP4 ring slot: a unit's 16 weight bytes for this lane plus the E8M0 codes
// of the unit's four 32-k blocks of this lane's column (byte j: block j).
struct SlotMx {
    u32x4_t w;
    uint32_t s;
};
template <int NG, bool MX>
struct SlotSel {
    using type = Slot<NG>;
};
template <int NG>
struct SlotSel<NG, true> {
    using type = SlotMx;
};

// Launch description shared by host and kernel.
struct GemvLaunch {
    int M, N, K;
    int U;        // 128-k units per column (K rounded up)
    int S;        // K slices: workgroups (t, s) cover units [s*U/S, (s+1)*U/S) of tile t
    int T;        // 16-column tiles
    int xstride;  // LDS row stride of a wave's staged x, in halves
    int out_dtype;
    const void* res;   // residual added to y (unsplit calls), or null
    int res_dtype;
    // Balanced plan (BAL kernels only): bal_full waves of a workgroup own its
    // whole tile; the others each take a share of one of bal_pieces pieces of
    // a leftover tile (tiles bal_base and up), merged through the workspace.
    int bal_full, bal_pieces, bal_base;
    unsigned* counters;   // arrival counter of leftover tile i at i * kCounterStride, zero between calls
    float* bal_part;      // [leftover tile][piece][M][16] piece partial sums
};

// Slots of the register ring for UPW units per wave: all loads are issued
// up front when they fit, otherwise the first D and a refill per consumed
// slot (the ring never holds more than the VGPR budget allows).
template <int SPG>
constexpr int max_slots() { return SPG >= 4 ? 9 : (SPG == 2 ? 7 : 5); }

// One wave's products: units [w0, w1) of tiles t0 .. t0 + nt - 1 of the
// current K slice into total[], through a chain of CL units per tile (CL =
// UPW except for the balanced plan's extra waves, which run a shorter chain).
// xsb is the wave's LDS region (M rows of UPW units, or PX's per-unit slots).
// BAR = 1 and 2 are the balanced plan's full and extra waves; an extra
// wave's region holds M rows of CL units.  BAR = 4: a wave of an uneven
// split (per-unit staging, one x slot per unit of its CL).  Workgroup barriers order their
// memory traffic so that the extra waves' shares, which are merged across
// workgroups, finish early: the full waves issue their weight loads only
// after every extra wave has issued its own.  With whole-range x staging
// that is the only barrier (each wave's x goes out at its start); with
// per-unit staging a first barrier also waits for every wave to start.
// Measured on down-shaped layers (us per call, graphs of 32 distinct
// matrices, f16 x at 1 / 2 / 3 rows): 11.0-11.5 / 11.1 / 11.3-11.5 with the
// one barrier against 11.5-11.8 / 11.5-11.6 / 11.6 with a second one that
// first had every wave issue its x, and 12.4-12.7 with no barrier.
template <bool BF16, int SPG, int UPW, int TPW, bool MX, bool PX, int CL, int BAR = 0>
__device__ __forceinline__ void w4_wave_chain(const GemvLaunch& a, const uint16_t* __restrict__ x,
                                              const u32x4_t* __restrict__ qdev,
                                              const uint16_t* __restrict__ sdev,
                                              const uint32_t* __restrict__ zdev, uint8_t* const xsb, int t0,
                                              int nt, int w0, int w1, float4_t (&total)[TPW]) {
    constexpr int NG = SPG >= 4 ? 1 : 4 / SPG;          // groups per unit
    constexpr int SPU = SPG >= 4 ? 4 : SPG;             // steps per group inside one unit
    constexpr int L = CL * TPW;                          // units in this wave's chain
    constexpr int DM = BAR == 1 ? bal_full_ring(PX) : TPW > 1 ? 5 : max_slots<SPG>();
    constexpr int D = L < DM ? L : DM;
    constexpr bool kUncond = SPG >= 4 || (SPG == 2 && CL <= 6) || CL <= 2;
    constexpr int LPS = MX ? 2 : 1 + 2 * NG;              // loads per ring slot
    using SlotT = typename SlotSel<NG, MX>::type;
    constexpr bool kCvtX = BF16 && !MX;   // bf16 x taken to fp16 in LDS for the 4-bit products
    // One-tile per-unit chains with bf16 x load each unit's x into registers
    // and store it to LDS converted: one LDS round trip per unit instead of
    // two (an LDS-direct load, then a read, convert and write back).
    // Measured at M = 4 (bf16 x): qkv 6.68-6.78 -> 6.47-6.53 us, o_proj
    // 6.26-6.29 -> 6.06-6.08 us.  Multi-tile chains stay at 128 VGPRs
    // without the room for it.
    constexpr bool kRegX = kCvtX && PX && BAR == 0 && TPW == 1;
    constexpr int XU = BAR == 1 || BAR == 2 ? CL : UPW;   // units per staged row (= xstride / 128 otherwise)
    // PX: x slots in the wave's region.  The balanced plan's waves reuse a
    // ring of D (unit i in slot i % D: its x load goes out with the refill
    // after unit i - D's products, whose fragment reads have completed).
    constexpr int XR = BAR == 4 ? CL : BAR != 0 ? D : UPW;
    const int M = a.M, K = a.K, U = a.U;
    const int lane = threadIdx.x & 63;
    const int nu = w1 - w0;                                           // units of this wave
    const int Gp = U * kUnitK / (SPG * 32);
    const int c = lane & 15, kc = lane >> 4;

    // LDS: wave w's x range, [M][16 UPW chunks of 16 bytes] at byte
    // 2 w M xstride (xstride = 128 UPW halves, no padding).  Inside each
    // 128-k unit of row m, logical chunk p sits at position p ^ (m % 4): the
    // rows are 256-byte multiples apart, so without the XOR the rows' copies
    // of a chunk would share banks; with it, rows 0..3 use four distinct
    // bank groups (rows m and m + 4 share one: a two-way conflict at M = 8).
    // Only the low two bits are swizzled so that the MFMA step j keeps a
    // lane-independent offset (64 j).  Once its products are
    // done, each wave reuses its own region for its partial sums, so a
    // workgroup needs exactly M x K x 2 bytes of LDS (two workgroups per CU
    // up to M = 8 at K = 5120).
    // PX: wave w's region is [UPW units][4 rows][256 bytes] at w UPW 1024
    // bytes, the same chunk swizzle inside each row.
    const uint32_t xbytes = (uint32_t)M * (uint32_t)K * 2u;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, xbytes);

    // 1) x range -> this wave's LDS region, straight from memory into LDS
    //    (no VGPRs, one round trip whatever M is).  Position ci of the region
    //    is row ci / cpr, position ci % cpr of that row; one load instruction
    //    fills 64 consecutive positions (lane l -> position 64 i + l) with the
    //    logical chunk the swizzle puts there.  Chunks past K (a ragged last
    //    unit) are zeroed with ordinary LDS stores.  These are the wave's
    //    first memory accesses; where its arithmetic is unconditional the
    //    wave waits for them only after issuing its weight ring (below), so
    //    the two round trips overlap.
    constexpr int kXL = kMaxXLoads;
    if constexpr (!PX) {
        constexpr int cpr = XU * (kUnitK / 8);       // chunks per staged row
        const int live = nu * (kUnitK / 8);          // positions of a row this wave reads
        const int xch = M * cpr;
#pragma unroll
        for (int i = 0; i < kXL; ++i) {
            if (i * 64 < xch) {                    // wave-uniform
                const int ci = i * 64 + lane;
                const int m = ci / cpr, pc = ci % cpr;
                const int lc = pc ^ (m & 3);   // same unit and step as pc
                const int kg = w0 * kUnitK + lc * 8;
                if (m < M && pc < live) {
                    if (kg < K)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            rx, (__attribute__((address_space(3))) void*)(xsb + i * 1024), 16,
                            (uint32_t)(m * K + kg) * 2u, 0, 0, 0);
                    else
                        *(u32x4_t*)(xsb + (uint32_t)ci * 16u) = u32x4_t{0u, 0u, 0u, 0u};
                }
            }
        }
        if constexpr (!kUncond) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2) Weight / scale / zero-point loads of this wave's units.
    // The workgroup's nt tiles are contiguous in all three arrays.
    // MXFP4: scales are [T][U][16] dwords and there are no zero points.
    const uint32_t wend = (uint32_t)nt * U * 1024u,
                   send = MX ? (uint32_t)nt * U * 64u : (uint32_t)nt * Gp * 32u,
                   zend = MX ? 0u : (uint32_t)nt * Gp * 8u;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(qdev + (size_t)t0 * U * kLanes, wend);
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(MX ? (const void*)((const uint8_t*)sdev + (size_t)t0 * U * 64u)
                     : (const void*)(sdev + (size_t)t0 * Gp * kTileN),
                  send);
    const __amdgpu_buffer_rsrc_t rz =
        make_rsrc(MX ? (const void*)qdev : (const void*)(zdev + (size_t)t0 * Gp * 2), zend);
    // The same resources with no records: every load through them returns
    // zeros.  A missing unit or tile selects these (a wave-uniform choice made
    // on the scalar side), so each load's per-lane offset stays fixed and its
    // unit offset is an SGPR: no vector instruction per load.
    const __amdgpu_buffer_rsrc_t rw0 = make_rsrc(qdev, 0), rs0 = make_rsrc(sdev, 0),
                                 rz0 = make_rsrc(qdev, 0), rx0 = make_rsrc(x, 0);
    const uint32_t wlane = (uint32_t)lane * 16u;
    const uint32_t slane = (uint32_t)c * 2u;
    const uint32_t zlane = (uint32_t)(c >> 3) * 4u;
    // PX: this lane's x chunk of a unit is row lane / 16, position lane % 16;
    // rows past M read past the end of x, i.e. zeros.
    const uint32_t xlane_off = (lane >> 4) < M
                                   ? (uint32_t)((lane >> 4) * K + 8 * ((lane & 15) ^ ((lane >> 4) & 3))) * 2u
                                   : xbytes;

    // Chain position q = unit i (of this wave's range) x tile j, unit-major,
    // so one x fragment serves the workgroup's TPW tiles back to back.
    u32x4_t xreg[kRegX ? XR : 1];
    auto load_slot = [&](int q, SlotT& r) {
        const int i = q / TPW, j = q % TPW;
        const bool valid = i < nu && j < nt;
        const int u = w0 + i;
        if constexpr (PX) {
            if (j == 0) {   // the unit's x: [4 rows][256 bytes] straight into LDS
                if constexpr (kRegX)
                    xreg[i % XR] = bitcast<u32x4_t>(__builtin_amdgcn_raw_buffer_load_b128(
                        i < nu ? rx : rx0, xlane_off, (uint32_t)u * (kUnitK * 2u), 0));
                else
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        i < nu ? rx : rx0, (__attribute__((address_space(3))) void*)(xsb + (i % XR) * 1024), 16,
                        xlane_off, (uint32_t)u * (kUnitK * 2u), 0, 0);
                __builtin_amdgcn_sched_barrier(0);   // before the slot's own loads
            }
        }
        r.w = bitcast<u32x4_t>(__builtin_amdgcn_raw_buffer_load_b128(
            valid ? rw : rw0, wlane, (uint32_t)(j * U + u) * 1024u, kAuxNT));
        if constexpr (MX) {
            r.s = __builtin_amdgcn_raw_buffer_load_b32(valid ? rs : rs0, (uint32_t)c * 4u,
                                                       (uint32_t)(j * U + u) * 64u, 0);
        } else {
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const int g = j * Gp + (u * 4) / SPG + gi;
                r.s[gi] = __builtin_amdgcn_raw_buffer_load_b16(valid ? rs : rs0, slane, (uint32_t)g * 32u, 0);
                r.z[gi] = __builtin_amdgcn_raw_buffer_load_b32(valid ? rz : rz0, zlane, (uint32_t)g * 8u, 0);
            }
        }
    };

    // Balanced plan: no wait before a barrier, so the loads stay in flight.
    if constexpr (BAR == 1) {
        if constexpr (PX) __builtin_amdgcn_s_barrier();   // every wave has started
        __builtin_amdgcn_s_barrier();                     // the extra waves' weight loads are out
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (BAR == 2 && PX) {
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    }
    SlotT ring[D];
#pragma unroll
    for (int i = 0; i < D; ++i) {
        load_slot(i, ring[i]);
        __builtin_amdgcn_sched_barrier(0);   // slots issue in ring order
    }
    if constexpr (BAR == 2) {
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    }
    // Vector memory loads complete in issue order, so once no more than the
    // ring's D * LPS loads are outstanding, every x load issued before
    // them has landed in LDS.  This needs every ring load issued here, after
    // the x loads: the weight loads count as invariant, so the compiler may
    // sink a slot's loads into a conditional block that uses them, and then
    // the wait falls short.  Hence the overlap only where the arithmetic is
    // unconditional (elsewhere the wait above, after the x loads, covers
    // them); a host-side test checks the compiled kernels for this.
    if constexpr (kUncond && !PX) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(D * LPS) : "memory");
    __builtin_amdgcn_sched_barrier(0);
    // bf16 x: each lane rewrites the chunks its own x loads filled as fp16.
    if constexpr (kCvtX && !PX) {
        // Four positions per lane at a time: their LDS reads are all issued
        // before the first conversion waits.
        constexpr int cpr = XU * (kUnitK / 8);       // as in the staging above
        const int live = nu * (kUnitK / 8), xch = M * cpr;
#pragma unroll
        for (int i0 = 0; i0 < kXL; i0 += 4) {
            if (i0 * 64 < xch) {
                u32x4_t v[4];
                bool ok[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int ci = (i0 + k) * 64 + lane;
                    ok[k] = i0 + k < kXL && ci < xch && ci % cpr < live;
                    if (ok[k]) v[k] = *(const u32x4_t*)(xsb + (uint32_t)ci * 16u);
                }
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (ok[k]) *(u32x4_t*)(xsb + (uint32_t)((i0 + k) * 64 + lane) * 16u) = bf16x8_to_f16x8(v[k]);
            }
        }
    }

    // 3) Dequantize and multiply, unit by unit.
    const int zshift = 4 * (c & 7);
    const uint32_t magic = opaque_v(0x64006400u);   // fp16 1024.0 pairs
    const bool xrow = c < M;                                    // lane supplies x row c
    // Step j of unit i: logical chunk 4 j + kc of row c, at position 4 j + (kc ^ c % 4).
    const uint8_t* xlane =
        xsb + (PX ? (uint32_t)(c * 256 + 16 * (kc ^ (c & 3)))
                  : (uint32_t)(c * XU * kUnitK + 8 * (kc ^ (c & 3))) * 2u);
    constexpr uint32_t kXUnit = PX ? 1024u : (uint32_t)kUnitK * 2;   // bytes between units of a row
#pragma unroll
    for (int j = 0; j < TPW; ++j) total[j] = float4_t{0.f, 0.f, 0.f, 0.f};
    u32x4_t xa[4] = {};
#pragma unroll
    for (int q = 0; q < L; ++q) {
        const int i = q / TPW, tj = q % TPW;
        SlotT& sl = ring[q % D];
        if constexpr (kRegX) {
            if (tj == 0) {   // this unit's x, converted, into its LDS slot (the compiler waits for it)
                *(u32x4_t*)(xsb + (uint32_t)(i % XR) * 1024u + (uint32_t)lane * 16u) =
                    bf16x8_to_f16x8(xreg[i % XR]);
            }
        } else if constexpr (PX) {
            if (tj == 0) {
                // Wait for this unit's x: loads complete in issue order, and
                // after it went out came its slot's LPS loads and, for each
                // later slot already issued, LPS loads plus an x load at every
                // TPW-th one.  rem = later slots issued (0 .. D - 1).
                const int rem = (q + D - 1 < L - 1 ? q + D - 1 : L - 1) - q;
#define W4_PX_WAIT(R) \
    case R: asm volatile("s_waitcnt vmcnt(%0)" ::"n"((R + 1) * LPS + R / TPW) : "memory"); break;
                switch (rem) {
                    W4_PX_WAIT(0) W4_PX_WAIT(1) W4_PX_WAIT(2) W4_PX_WAIT(3) W4_PX_WAIT(4)
                    W4_PX_WAIT(5) W4_PX_WAIT(6) W4_PX_WAIT(7) W4_PX_WAIT(8)
                    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                }
#undef W4_PX_WAIT
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (kCvtX) {   // the 16 bytes this lane's x load wrote, as fp16
                    u32x4_t* const p = (u32x4_t*)(xsb + (uint32_t)(i % XR) * 1024u + (uint32_t)lane * 16u);
                    *p = bf16x8_to_f16x8(*p);
                }
            }
        }
        if (tj == 0 && i < nu && xrow) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                xa[j] = *(const u32x4_t*)(xlane + (uint32_t)(PX ? i % XR : i) * kXUnit + 64 * j);
        }
        // Units past this wave's range arrived as zeros (q = z = 0, s = +0) and
        // add exactly 0 with the finite x the lane still holds, so where the
        // register budget allows, the arithmetic runs unconditionally: then no
        // slot's loads get sunk into a conditional block next to their only use
        // (which would make the first unit wait for the whole ring).
        if constexpr (MX) {
            // Scales folded into the conversion where the unit's codes allow
            // it (mx_unit), else step by step.  Units past the range load
            // zeros: codes 0 and scale codes 0 add exactly 0.
            const MxUnit mu = mx_unit(sl.s);
            const uint32_t* e = mu.e;
            const uint32_t emax = mu.emax;
            if (__builtin_amdgcn_ballot_w64(mu.wide) == 0) {
                float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float sj = mx_fold_scale(e[j], emax);
                    if constexpr (!BF16)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            bitcast<half8_t>(xa[j]), fp4x8_to_f16(sl.w[j], sj), acc, 0, 0, 0);
                    else
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            bitcast<bf16x8_t>(xa[j]), fp4x8_to_bf16(sl.w[j], sj), acc, 0, 0, 0);
                }
                const float sf = mx_unit_scale(emax);
                total[tj][0] = __builtin_fmaf(sf, acc[0], total[tj][0]);
                total[tj][1] = __builtin_fmaf(sf, acc[1], total[tj][1]);
                total[tj][2] = __builtin_fmaf(sf, acc[2], total[tj][2]);
                total[tj][3] = __builtin_fmaf(sf, acc[3], total[tj][3]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float4_t acc = {0.f, 0.f, 0.f, 0.f};
                    if constexpr (!BF16)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            bitcast<half8_t>(xa[j]), fp4x8_to_f16(sl.w[j], 1.0f), acc, 0, 0, 0);
                    else
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            bitcast<bf16x8_t>(xa[j]), fp4x8_to_bf16(sl.w[j], 1.0f), acc, 0, 0, 0);
                    const float sf = e8m0_to_f32(e[j]);
                    total[tj][0] = __builtin_fmaf(sf, acc[0], total[tj][0]);
                    total[tj][1] = __builtin_fmaf(sf, acc[1], total[tj][1]);
                    total[tj][2] = __builtin_fmaf(sf, acc[2], total[tj][2]);
                    total[tj][3] = __builtin_fmaf(sf, acc[3], total[tj][3]);
                    __builtin_amdgcn_sched_barrier(0);   // one step's sum live at a time
                }
            }
        } else if (kUncond || (i < nu && tj < nt)) {
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const uint32_t zq = (sl.z[gi] >> zshift) & 15u;
                float4_t acc = {0.f, 0.f, 0.f, 0.f};
                uint32_t nz1024 = 0xE400u + zq;          // fp16 -(1024 + z)
                nz1024 |= nz1024 << 16;
                uint32_t nz64 = 0xD400u + (zq << 4);     // fp16 -(64 + z)
                nz64 |= nz64 << 16;
#pragma unroll
                for (int js = 0; js < SPU; ++js) {
                    const int j = gi * SPU + js;
                    const half8_t b = dequant_f16(sl.w[j], magic, nz1024, nz64);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<half8_t>(xa[j]), b, acc, 0, 0, 0);
                }
                const float sf = f16_bits_to_f32((uint16_t)sl.s[gi]);
                total[tj][0] = __builtin_fmaf(sf, acc[0], total[tj][0]);
                total[tj][1] = __builtin_fmaf(sf, acc[1], total[tj][1]);
                total[tj][2] = __builtin_fmaf(sf, acc[2], total[tj][2]);
                total[tj][3] = __builtin_fmaf(sf, acc[3], total[tj][3]);
                // g = 64 multi-tile chains: left alone, the compiler defers
                // every group's scale FMA to the end of the chain and keeps
                // all the group accumulators live (178 VGPRs for UPW = 5,
                // TPW = 3: one workgroup per CU).  An empty asm statement that
                // claims to change the running total makes each FMA happen
                // here (94 VGPRs, two workgroups per CU).  It emits no
                // instruction.  At g = 128 the same pin measured within noise
                // (gate_up slower, lm_head faster), so it is left out there.
                if constexpr (TPW > 1 && SPG == 2) asm volatile("" : "+v"(total[tj]));
            }
        }
        if (q + D < L) {                   // fixed refill schedule: position q + D into this slot
            __builtin_amdgcn_sched_barrier(0);
            load_slot(q + D, sl);
        }
        __builtin_amdgcn_sched_barrier(0);   // units in order: each waits for its own slot only
    }

}

// One workgroup per (TPW 16-column tiles, K slice); its W waves split the
// slice's 128-k units into contiguous ranges of at most UPW units.  Each wave
//   1. starts staging its own range of x (all M rows, zeros past K) in its
//      own LDS region, loading it straight into LDS -- no other wave's x is
//      on its critical path;
//   2. issues the loads of its chain of TPW x UPW units (16 weight bytes,
//      scale and zero point per lane; unit-major, so one x fragment serves
//      the TPW tiles back to back) -- all of them up front when the chain
//      fits the register ring, otherwise with one refill per consumed slot
//      on a fixed schedule, so the code is straight-line and every wait
//      covers exactly one slot;
//   3. dequantizes and multiplies each unit as its slot arrives;
// then the waves add their partial sums through LDS in wave order and the
// workgroup stores its tiles (or their fp32 slice partials).
//
// A wave whose range is shorter than UPW (or a workgroup with fewer than TPW
// tiles left) gives its missing units an offset past the buffer resource's
// size: such loads return zeros without touching memory, and the units are
// skipped or add exactly zero.
//
// Eight waves per SIMD (at most 64 VGPRs) for the short chains, where the
// register budget allows it without spilling.
template <int SPG, int UPW>
constexpr int min_waves() { return (SPG >= 4 && UPW <= 5) || (SPG == 2 && UPW <= 3) ? 8 : 1; }

// MX = true runs MXFP4 weights (mxfp4.hip's device layout) instead: no zero
// points, one E8M0 scale per 32-k block, which is exactly one MFMA step; the
// scales fold into the element conversion where a unit's codes allow it and
// apply step by step otherwise (mx_unit in common.h).  Its slot (5 VGPRs) is
// the size of a g = 128 slot, so it is instantiated with SPG = 4 for the
// register plan.
// PX = true stages x unit by unit instead (up to 4 rows, K a multiple of
// 128, unconditional arithmetic): each unit's x is one load of [4 rows][256
// bytes] straight into LDS (one-tile chains with bf16 x: into registers,
// stored to LDS converted), issued with the unit's first ring slot, and the
// wave waits for it just before the unit's products.  The first unit then
// waits for its own 1 KB of x and not for the wave's whole range.
// BAL = true runs the balanced plan: one workgroup per CU of 16 waves, 8 of
// which stream the workgroup's own tile while 8 split one piece of a leftover
// tile (see the planner); TPW = 1, whole-range x staging, up to 2 rows.
// One-tile per-unit chains with bf16 x hold each unit's x in registers
// until it is stored converted, so they run under a four-waves-per-SIMD
// bound (their layers put at most two workgroups on a CU).
template <bool BF16, int SPG, int UPW, int TPW, bool MX = false, bool PX = false, bool BAL = false>
__global__ __launch_bounds__(BAL ? 1024 : 512,
                             (TPW > 1 || BAL ? 1 : (BF16 && PX && !MX) ? 4 : min_waves<SPG, UPW>())) void w4_gemv_kernel(
    int M_, int K_, int U_, int T_, int plan0, int plan1,
    const uint16_t* __restrict__ x, const u32x4_t* __restrict__ qdev,
    const uint16_t* __restrict__ sdev, const uint32_t* __restrict__ zdev, void* out,
    GemvLaunch a_in) {
    // The first ten arguments (14 dwords) are everything a wave needs before
    // its first load; this file is compiled to have the hardware preload
    // them into SGPRs at wave launch, so no wave starts with a scalar load
    // of its kernel arguments.  The launch's other fields stay in a_in,
    // loaded where they are used.  plan0 / plan1 are the K slice count and
    // the wave count, or for the balanced plan (one slice, kBalFull +
    // kBalExtra waves) the leftover tiles' piece count and first tile.
    GemvLaunch a = a_in;
    a.M = M_;
    a.K = K_;
    a.U = U_;
    a.T = T_;
    a.xstride = UPW * kUnitK;   // every launch stages rows of exactly UPW units
    if constexpr (BAL) {
        a.S = 1;
        a.bal_full = kBalFull;
        a.bal_pieces = plan0;
        a.bal_base = plan1;
    } else {
        a.S = plan0;
    }
    constexpr int DM = TPW > 1 ? 5 : max_slots<SPG>();
    constexpr bool kUncond = SPG >= 4 || (SPG == 2 && UPW <= 6) || UPW <= 2;
    static_assert(!PX || (kUncond && (UPW * TPW < DM ? UPW * TPW : DM) <= 9),
                  "per-unit x staging needs a straight-line ring");
    static_assert(!BAL || (TPW == 1 && kUncond), "the balanced plan runs one tile");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int M = a.M, U = a.U;
    const int W = BAL ? kBalFull + kBalExtra : plan1;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    int t0 = blockIdx.x * TPW;
    const int split = blockIdx.y;
    int nt = a.T - t0 < TPW ? a.T - t0 : TPW;                         // tiles of this workgroup
    // A wave's share of its slice's units.  Unsplit launches of eight waves
    // (every hot layer) take it without the two runtime divisions, which
    // sit between a wave's start and its first load; the balanced plan (one
    // slice) replaces the shares below.
    static_assert(kMaxWaves == 8, "the unsplit range below divides by 8 with a shift");
    int r0, r1, w0, w1;
    if (BAL || (a.S == 1 && W == kMaxWaves)) {
        r0 = 0;
        r1 = U;
        w0 = (wave * U) >> 3;
        w1 = ((wave + 1) * U) >> 3;
    } else {
        r0 = split * U / a.S;
        r1 = (split + 1) * U / a.S;
        w0 = r0 + wave * (r1 - r0) / W;
        w1 = r0 + (wave + 1) * (r1 - r0) / W;
    }
    // Three-tile chains of 5 units (g = 128, per-unit staging, eight waves):
    // waves 0-3 take 6 units and waves 4-7 take 4.  A wave's first unit
    // arrives in the order the grid issued its ring: every CU's first four
    // waves (the first on each SIMD) before its next four, which on a
    // 27B-class gate_up received theirs 1.5 us later (median 3.8 against
    // 2.3 us) and so ended their equal chains 1.4 us later, while the
    // others waited at the reduction barrier.  Measured (graphs of 64
    // distinct matrices, us per call): gate_up 19.4 -> 18.9 at M = 4 (bf16),
    // 17.6 either way at M = 1; 7 and 3 units, 19.2 and 20.6.  MXFP4 gate_up
    // (16 distinct matrices): 19.6-20.4 -> 19.2-19.6 at M = 1, 19.7-21.6 ->
    // 18.8-20.5 at M = 4.
    // With fewer than eight waves (a shorter K) the first four still take 6
    // units each, which covers the range (6 min(W, 4) + 4 max(W - 4, 0) >=
    // 5 W for W <= 8); the planner sizes the LDS for these regions.
    constexpr bool skew = skewed_split(SPG, UPW, TPW, PX) && !BAL;
    if constexpr (skew) {
        w0 = r0 + skew_units(wave);
        w1 = w0 + (wave < kSkewOld ? UPW + 1 : UPW - 1);
        if (w0 > r1) w0 = r1;
        if (w1 > r1) w1 = r1;
    }
    // Balanced plan: waves 0 .. bal_full - 1 split the workgroup's own tile
    // over K; each later ("extra") wave takes a share of piece blockIdx.x %
    // bal_pieces of leftover tile bal_base + blockIdx.x / bal_pieces.
    const bool extra = BAL && wave >= a.bal_full;
    // Balanced plan LDS: the full waves' x regions (M rows of UPW units
    // each; PX: a ring of kDF units), the extra waves' (M rows of
    // bal_extra_cl(UPW) units; PX: kDE units), the full waves' partial sums
    // [bal_full][M][16], the extra waves' [kBalExtra][M][16], and the extra
    // waves' arrival count.
    constexpr int kDF = UPW < bal_full_ring(PX) ? UPW : bal_full_ring(PX);
    constexpr int kDE = bal_extra_cl(UPW) < max_slots<SPG>() ? bal_extra_cl(UPW) : max_slots<SPG>();
    const size_t xfull = PX ? (size_t)kDF * 1024 : (size_t)M * a.xstride * 2;
    const size_t xext = PX ? (size_t)kDE * 1024 : (size_t)M * bal_extra_cl(UPW) * kUnitK * 2;
    uint8_t* const xextra = smem + (size_t)a.bal_full * xfull;
    float* const fullp = (float*)(xextra + (size_t)kBalExtra * xext);
    float* const extrap = fullp + (size_t)a.bal_full * M * kTileN;
    unsigned* const lcount = (unsigned*)(extrap + (size_t)kBalExtra * M * kTileN);
    if constexpr (BAL) {
        // The count is zeroed before the chains' barriers (nothing else is
        // in flight yet).
        if (threadIdx.x == 0) *lcount = 0u;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        const int WF = a.bal_full;
        if (!extra) {
            // The full waves' 8 x UPW units, the first four taking UPW + 1
            // each and the later four UPW - 1 (see bal_full_units).
            w0 = bal_full_units<UPW>(wave);
            w1 = bal_full_units<UPW>(wave + 1);
        } else {
            const int P = a.bal_pieces, WE = W - WF, pc = blockIdx.x % P, e = wave - WF;
            const int pa = pc * U / P, pb = (pc + 1) * U / P;
            t0 = a.bal_base + blockIdx.x / P;
            w0 = pa + e * (pb - pa) / WE;
            w1 = pa + (e + 1) * (pb - pa) / WE;
        }
        nt = 1;
    }
    // LDS: wave w's x range, [M][16 UPW chunks of 16 bytes] at byte
    // 2 w M xstride; PX: [UPW units][4 rows][256 bytes] at w UPW 1024 bytes
    // (the layouts are described in w4_wave_chain).
    uint8_t* const xsb = extra ? xextra + (size_t)(wave - a.bal_full) * xext
                         : BAL ? smem + (PX ? (size_t)wave * xfull : (size_t)M * 256 * bal_full_units<UPW>(wave))
                               : smem + (skew ? (size_t)skew_units(wave) * 1024
                                         : PX  ? (size_t)wave * UPW * 1024
                                               : (size_t)wave * M * a.xstride * 2);
    const int c = lane & 15, kc = lane >> 4;
    float4_t total[TPW];
    if constexpr (BAL) {
        if (extra)
            w4_wave_chain<BF16, SPG, UPW, TPW, MX, PX, bal_extra_cl(UPW), 2>(a, x, qdev, sdev, zdev, xsb, t0, nt, w0,
                                                                         w1, total);
        else if (wave < kSkewOld)
            w4_wave_chain<BF16, SPG, UPW, TPW, MX, PX, UPW + 1, 1>(a, x, qdev, sdev, zdev, xsb, t0, nt, w0, w1,
                                                                  total);
        else
            w4_wave_chain<BF16, SPG, UPW, TPW, MX, PX, UPW - 1, 1>(a, x, qdev, sdev, zdev, xsb, t0, nt, w0, w1,
                                                                  total);
    } else if constexpr (skew) {
        if (wave < kSkewOld)
            w4_wave_chain<BF16, SPG, UPW, TPW, MX, PX, UPW + 1, 4>(a, x, qdev, sdev, zdev, xsb, t0, nt, w0, w1,
                                                                  total);
        else
            w4_wave_chain<BF16, SPG, UPW, TPW, MX, PX, UPW - 1, 4>(a, x, qdev, sdev, zdev, xsb, t0, nt, w0, w1,
                                                                  total);
    } else {
        w4_wave_chain<BF16, SPG, UPW, TPW, MX, PX, UPW>(a, x, qdev, sdev, zdev, xsb, t0, nt, w0, w1, total);
    }

    // 4) Wave partials (lane l holds rows 4*(l/16) + r of column l % 16) ->
    //    [TPW][M][16] floats at the start of the wave's own x region (TPW M
    //    64 <= M UPW 256 bytes; its last x reads were consumed above, and a
    //    wave's LDS accesses complete in order), then M x 16 threads add
    //    them in wave order and store.  The balanced plan's waves use
    //    partial areas of their own instead.
    float* const red = !BAL ? (float*)xsb
                            : (extra ? extrap + (size_t)(wave - a.bal_full) * M * kTileN
                                     : fullp + (size_t)wave * M * kTileN);
    const float* const red0 = BAL ? fullp : (const float*)smem;
    const size_t rstride = BAL  ? (size_t)M * kTileN
                           : PX ? (size_t)UPW * 1024 / 4
                                : (size_t)M * a.xstride / 2;   // floats between wave partials
    if constexpr (BAL) {
        if (extra) {
            // This wave's share of a leftover tile.  The workgroup's extra
            // waves first add their partial sums through LDS: each writes
            // them to its own partial area and counts itself in; the last to arrive
            // adds the kBalExtra partials in wave order, stores that sum
            // (coherent across the device) as the workgroup's piece of the
            // tile and counts the piece in the tile's arrival counter; the
            // last piece to arrive adds the P pieces in piece order and
            // stores the tile's outputs.  The extra waves' shares are about a
            // quarter of a full wave's units, so all of this runs while the
            // full waves still stream.
            const int P = a.bal_pieces;
            const int lt = t0 - a.bal_base, pc = blockIdx.x % P;
            if (kc == 0) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (r < M) red[r * kTileN + c] = total[0][r];
            }
            unsigned wold = 0;
            if (lane == 0) wold = __hip_atomic_fetch_add(lcount, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
            wold = __builtin_amdgcn_readfirstlane(wold);
            if (wold == kBalExtra - 1) {
                float* const piece = a.bal_part + (size_t)lt * P * M * kTileN;
                if (lane < M * kTileN) {
                    float pw[kBalExtra];
#pragma unroll
                    for (int e = 0; e < kBalExtra; ++e) pw[e] = extrap[e * M * kTileN + lane];
                    float v = 0.f;
#pragma unroll
                    for (int e = 0; e < kBalExtra; ++e) v += pw[e];
                    __hip_atomic_store(piece + (size_t)pc * M * kTileN + lane, v, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
                __builtin_amdgcn_s_waitcnt(0);   // the piece's store is done before it is counted
                unsigned* const counter = a.counters + (size_t)lt * kCounterStride;
                unsigned old = 0;
                if (lane == 0) old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                old = __builtin_amdgcn_readfirstlane(old);
                if (old == (unsigned)(P - 1)) {
                    if (lane < M * kTileN) {
                        // Every piece is loaded before the first add; positions
                        // past P reload the last piece and are not added.
                        float pv[kBalMaxPieces];
#pragma unroll
                        for (int q2 = 0; q2 < kBalMaxPieces; ++q2)
                            pv[q2] = __hip_atomic_load(piece + (size_t)(q2 < P ? q2 : P - 1) * M * kTileN + lane,
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        float v = 0.f;
#pragma unroll
                        for (int q2 = 0; q2 < kBalMaxPieces; ++q2) v = q2 < P ? v + pv[q2] : v;
                        const int m = lane >> 4, n = t0 * kTileN + (lane & 15);
                        if (n < a.N) {
                            const size_t o = (size_t)m * a.N + n;
                            store_out(out, a.out_dtype, o, add_residual(v, a.res, a.res_dtype, o));
                        }
                    }
                    if (lane == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
    }
    if (!extra) {
#pragma unroll
        for (int j = 0; j < TPW; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * kc + r;
                if (m < M) red[(j * M + m) * kTileN + c] = total[j][r];
            }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < TPW * M * kTileN; idx += blockDim.x) {
        const int j = idx / (M * kTileN), rem = idx % (M * kTileN);
        const int m = rem >> 4, cc = rem & 15;
        // All W partials are read before the first add (one LDS round trip),
        // then added in wave order.
        float v = 0.f;
        const int WR = BAL ? a.bal_full : W;   // waves holding this tile's partials
        if (WR == kMaxWaves) {
            float pw[kMaxWaves];
#pragma unroll
            for (int w = 0; w < kMaxWaves; ++w)
                pw[w] = red0[(skew ? (size_t)skew_units(w) * 256 : w * rstride) + (j * M + m) * kTileN + cc];
#pragma unroll
            for (int w = 0; w < kMaxWaves; ++w) v += pw[w];
        } else {
            for (int w = 0; w < WR; ++w)
                v += red0[(skew ? (size_t)skew_units(w) * 256 : w * rstride) + (j * M + m) * kTileN + cc];
        }
        const int n = (t0 + j) * kTileN + cc;
        if (j < nt && n < a.N) {
            const size_t o = (size_t)m * a.N + n;
            if (a.S > 1)   // fp32 slice partials; the merge adds the residual
                ((float*)out)[(size_t)split * M * a.N + o] = v;
            else
                store_out(out, a.out_dtype, o, add_residual(v, a.res, a.res_dtype, o));
        }
    }
}

// y = sum over slices of the fp32 partials, in slice order.  Each thread
// takes four consecutive outputs and issues all S loads before the first add
// (a loop of load-then-add would wait on every slice in turn).
__device__ __forceinline__ void store4(void* y, int out_dtype, int i4, float4_t v) {
    if (out_dtype == W4A16_F32) {
        ((float4_t*)y)[i4] = v;
    } else if (out_dtype == W4A16_F16) {
        typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
        ((half4_t*)y)[i4] = half4_t{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    } else {
        const uint32_t lo = f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
        const uint32_t hi = f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
        ((uint2*)y)[i4] = uint2{lo, hi};
    }
}

__device__ __forceinline__ float4_t add_residual4(float4_t v, const void* r, int r_dtype, int i4) {
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = add_residual(v[q], r, r_dtype, (size_t)4 * i4 + q);
    return v;
}

template <int S>
__global__ void splitk_merge_kernel(const float4_t* __restrict__ ws, void* y, int out_dtype,
                                    int MN4, const void* res, int res_dtype) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= MN4) return;
    float4_t p[S];
#pragma unroll
    for (int s = 0; s < S; ++s) p[s] = ws[(size_t)s * MN4 + i];
    float4_t v = p[0];
#pragma unroll
    for (int s = 1; s < S; ++s) v += p[s];
    store4(y, out_dtype, i, add_residual4(v, res, res_dtype, i));
}

// Any slice count (only reachable through the slice override).
__global__ void splitk_merge_any_kernel(const float4_t* __restrict__ ws, void* y, int out_dtype,
                                        int MN4, const void* res, int res_dtype, int S) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= MN4) return;
    float4_t v = ws[i];
    for (int s = 1; s < S; ++s) v += ws[(size_t)s * MN4 + i];
    store4(y, out_dtype, i, add_residual4(v, res, res_dtype, i));
}

typedef void (*merge_kernel_t)(const float4_t*, void*, int, int, const void*, int);

merge_kernel_t pick_merge(int S) {
    switch (S) {
        case 2: return splitk_merge_kernel<2>;
        case 3: return splitk_merge_kernel<3>;
        case 4: return splitk_merge_kernel<4>;
        case 5: return splitk_merge_kernel<5>;
        case 6: return splitk_merge_kernel<6>;
        case 7: return splitk_merge_kernel<7>;
        case 8: return splitk_merge_kernel<8>;
        case 16: return splitk_merge_kernel<16>;
        default: return nullptr;
    }
}

// ------------------------------------------------------------------ dispatch

// Planner overrides (A/B measurement only), read once per process: common.h.
using w4h::overrides;

constexpr size_t kLdsPerCu = 160 * 1024;      // gfx950
constexpr int kWaves = 8;                     // waves per workgroup (two workgroups per CU)
constexpr int kUpwSet[] = {1, 2, 3, 4, 5, 6, 8, 9, 12, 17};   // compiled units-per-wave

struct Plan {
    GemvLaunch l;
    int waves;
    int upw;
    int tpw;
    bool px;     // x staged unit by unit (PX kernels)
    size_t lds;
    int tiles;
};

// Smallest compiled units-per-wave >= need (0 if none).
int pick_upw(int need) {
    for (int u : kUpwSet)
        if (u >= need) return u;
    return 0;
}

// Instantiations with per-unit x staging: g = 64 and 128 at 3 to 6 units
// per wave with one or three tiles, and g = 128 at 8 units with one tile.
// (With one or two units the compiler moved the lone slot's loads past the
// unit's x wait, which the assembly test caught; short chains keep the
// whole-range staging.)
bool px_compiled(int group, int upw, int tpw) {
    if (group == 128 && upw == 8 && tpw == 1) return true;
    return (group == 64 || group == 128) && upw >= 3 && upw <= 6 && (tpw == 1 || tpw == 3);
}

Plan make_plan(int M, int N, int K, int group, int cus, bool allow_px) {
    // Multi-tile kernels are compiled for g = 64 and 128.  At g = 64, M = 1,
    // they measured 83.8 us on the lm_head shape (N = 152064, K = 5120)
    // against 96.4 us with one tile per workgroup, and 21.2 against 23.5 us
    // on gate_up.
    const bool group_tpw_ok = group == 128 || group == 64;
    Plan p;
    const w4h::Overrides& tu = overrides();
    const int U = (K + kUnitK - 1) / kUnitK;
    const int T = pad_n(N) / kTileN;
    int W = kWaves;
    if (tu.w4_waves >= 1 && tu.w4_waves <= kMaxWaves) W = tu.w4_waves;
    // K slices: a wave's range must fit a compiled UPW, its x range at most
    // 16 chunks per lane (M * UPW <= 64), and the workgroup's x (whose regions the
    // partial sums reuse) the LDS of a CU.
    auto fits = [&](int S, int& upw, size_t& lds, int& xstride) {
        const int RU = (U + S - 1) / S;
        const int w = W < RU ? W : RU;
        upw = pick_upw((RU + w - 1) / w);
        if (!upw || M * upw > 64) return false;
        xstride = upw * kUnitK;      // the kernel swizzles chunks instead of padding rows
        lds = (size_t)W * M * xstride * 2;   // the partial sums reuse the x regions
        return lds <= kLdsPerCu;
    };
    int S = 1, upw = 0, xstride = 0;
    size_t lds = 0;
    while (S < U && !fits(S, upw, lds, xstride)) S *= 2;
    // Narrow N (e.g. one GPU's column share of a layer): more slices so every
    // CU gets a workgroup, as long as each wave keeps at least two units per
    // slice (a split with too little k per slice loses: NINFER tuning page,
    // section 五, item 21).
    while ((long long)T * S < cus && U / (2 * S) >= 2 * W && fits(2 * S, upw, lds, xstride)) S *= 2;
    // A shape whose x range forces a split pays the merge anyway; on a small
    // grid one more halving of the slices (each wave keeping at least four
    // units) spreads the work more evenly: the 27B down shape at M = 4 runs
    // 17.9 us at two slices and 17.0 us at four.
    if (S > 1 && (long long)T * S < 4LL * cus && U / (2 * S) >= 4 * W && fits(2 * S, upw, lds, xstride))
        S *= 2;
    if (tu.w4_split >= 1 && tu.w4_split <= U) S = tu.w4_split;
    if (!fits(S, upw, lds, xstride)) upw = 0;   // an override that cannot run is refused
    p.l = GemvLaunch{M, N, K, U, S, T, xstride, W4A16_F32, nullptr, W4A16_F32};
    p.waves = W;
    p.upw = upw;
    // Several tiles per workgroup when there are many more tiles than the GPU
    // holds at once: each wave then streams a chain of TPW x upw units with a
    // refill ring instead of issuing everything and going idle, and the
    // workgroup stages x once for all its tiles.
    p.tpw = 1;
    if (group_tpw_ok && upw <= 6 && S == 1 && T >= 6 * cus) p.tpw = 3;
    // A one-tile workgroup that needs more than half a CU's LDS runs alone
    // on its CU, and a grid of more tiles than CUs then takes two rounds.
    // Two tiles per workgroup (x staged once for both) make it one round:
    // K = N = 8192 at M = 6 went from 14.0 to 10.5 us, at M = 8 from 13.9 us
    // (the M-tiled kernel) to 11.2 us (g = 64: 15.3 -> 12.2, 14.9 -> 13.0).
    if (group_tpw_ok && p.tpw == 1 && upw == 8 && S == 1 && lds > kLdsPerCu / 2 && T >= 2 * cus)
        p.tpw = 2;
    if (tu.w4_tpw >= 1 && tu.w4_tpw <= 4 && upw <= 6 && group_tpw_ok) p.tpw = tu.w4_tpw;
    // The partial sums of all TPW tiles fit each wave's x region: TPW M 64
    // bytes against M upw 256 (TPW <= 4).
    p.lds = lds;
    // Per-unit x staging up to 4 rows (one [4][256-byte] load per unit) with
    // no ragged unit.  Measured on the 27B-class layers (us, whole-range
    // staging / per-unit): M = 1 qkv 6.33 / 5.96, o_proj 6.15 / 5.76,
    // gate_up 18.1 / 17.6-18.0; M = 4 (bf16) qkv 7.15 / 6.57, o_proj 7.14 /
    // 6.31, gate_up 21.0 / 19.6-19.7, down (4 slices) 15.1 / 13.4.  Down at
    // M = 1 (17 units per wave) keeps the whole-range staging: a quarter-full
    // load per unit ran 15.8 against 14.2 us there.
    p.px = allow_px && M <= 4 && K % kUnitK == 0 && px_compiled(group, upw, p.tpw);
    if (tu.w4_px == 0) p.px = false;   // A/B only
    // (The uneven split of three-tile 5-unit chains needs its regions' units,
    // skew_units(W) >= 5 W.)
    if (p.px) p.lds = (size_t)(skewed_split(group / 32, upw, p.tpw, true) ? skew_units(W) : W * upw) * 1024;
    p.tiles = T;
    return p;
}

typedef void (*w4_kernel_t)(int, int, int, int, int, int, const uint16_t*, const u32x4_t*,
                            const uint16_t*, const uint32_t*, void*, GemvLaunch);

template <bool BF16, int SPG, int TPW>
w4_kernel_t pick_small_upw(int upw) {
    switch (upw) {
        case 1: return w4_gemv_kernel<BF16, SPG, 1, TPW>;
        case 2: return w4_gemv_kernel<BF16, SPG, 2, TPW>;
        case 3: return w4_gemv_kernel<BF16, SPG, 3, TPW>;
        case 4: return w4_gemv_kernel<BF16, SPG, 4, TPW>;
        case 5: return w4_gemv_kernel<BF16, SPG, 5, TPW>;
        default: return w4_gemv_kernel<BF16, SPG, 6, TPW>;
    }
}

template <bool BF16, int SPG, int TPW>
w4_kernel_t pick_px_upw(int upw) {
    switch (upw) {
        case 3: return w4_gemv_kernel<BF16, SPG, 3, TPW, false, true>;
        case 4: return w4_gemv_kernel<BF16, SPG, 4, TPW, false, true>;
        case 5: return w4_gemv_kernel<BF16, SPG, 5, TPW, false, true>;
        default: return w4_gemv_kernel<BF16, SPG, 6, TPW, false, true>;
    }
}

// The per-unit staging kernels (px_compiled says which exist).
template <bool BF16>
w4_kernel_t pick_px(int group, int upw, int tpw) {
    if (group == 128) {
        if (upw == 8) return w4_gemv_kernel<BF16, 4, 8, 1, false, true>;
        return tpw == 3 ? pick_px_upw<BF16, 4, 3>(upw) : pick_px_upw<BF16, 4, 1>(upw);
    }
    return tpw == 3 ? pick_px_upw<BF16, 2, 3>(upw) : pick_px_upw<BF16, 2, 1>(upw);
}

template <bool BF16, int SPG>
w4_kernel_t pick_upw_kernel(int upw, int tpw) {
    if (upw <= 6) {
        if constexpr (SPG == 2 || SPG == 4) {
            if (tpw == 2) return pick_small_upw<BF16, SPG, 2>(upw);
            if (tpw == 3) return pick_small_upw<BF16, SPG, 3>(upw);
            if (tpw == 4) return pick_small_upw<BF16, SPG, 4>(upw);
        }
        return pick_small_upw<BF16, SPG, 1>(upw);
    }
    switch (upw) {
        case 8:
            if constexpr (SPG == 2 || SPG == 4)
                if (tpw == 2) return w4_gemv_kernel<BF16, SPG, 8, 2>;
            return w4_gemv_kernel<BF16, SPG, 8, 1>;
        case 9: return w4_gemv_kernel<BF16, SPG, 9, 1>;
        case 12: return w4_gemv_kernel<BF16, SPG, 12, 1>;
        default: return w4_gemv_kernel<BF16, SPG, 17, 1>;
    }
}

template <bool BF16>
w4_kernel_t pick_group(int group, int upw, int tpw) {
    switch (group) {
        case 32: return pick_upw_kernel<BF16, 1>(upw, tpw);
        case 64: return pick_upw_kernel<BF16, 2>(upw, tpw);
        case 128: return pick_upw_kernel<BF16, 4>(upw, tpw);
        default: return pick_upw_kernel<BF16, 8>(upw, tpw);
    }
}

w4_kernel_t pick_kernel(bool bf16, int group, int upw, int tpw, bool px = false) {
    if (px) return bf16 ? pick_px<true>(group, upw, tpw) : pick_px<false>(group, upw, tpw);
    return bf16 ? pick_group<true>(group, upw, tpw) : pick_group<false>(group, upw, tpw);
}

// MXFP4 kernels (register plan of g = 128, see the kernel).
template <bool BF16, int TPW>
w4_kernel_t pick_mx_small_upw(int upw) {
    switch (upw) {
        case 1: return w4_gemv_kernel<BF16, 4, 1, TPW, true>;
        case 2: return w4_gemv_kernel<BF16, 4, 2, TPW, true>;
        case 3: return w4_gemv_kernel<BF16, 4, 3, TPW, true>;
        case 4: return w4_gemv_kernel<BF16, 4, 4, TPW, true>;
        case 5: return w4_gemv_kernel<BF16, 4, 5, TPW, true>;
        default: return w4_gemv_kernel<BF16, 4, 6, TPW, true>;
    }
}

template <bool BF16>
w4_kernel_t pick_mx_upw(int upw, int tpw) {
    if (upw <= 6) {
        if (tpw == 2) return pick_mx_small_upw<BF16, 2>(upw);
        if (tpw == 3) return pick_mx_small_upw<BF16, 3>(upw);
        if (tpw == 4) return pick_mx_small_upw<BF16, 4>(upw);
        return pick_mx_small_upw<BF16, 1>(upw);
    }
    switch (upw) {
        case 8: return tpw == 2 ? w4_gemv_kernel<BF16, 4, 8, 2, true> : w4_gemv_kernel<BF16, 4, 8, 1, true>;
        case 9: return w4_gemv_kernel<BF16, 4, 9, 1, true>;
        case 12: return w4_gemv_kernel<BF16, 4, 12, 1, true>;
        default: return w4_gemv_kernel<BF16, 4, 17, 1, true>;
    }
}

template <bool BF16, int TPW>
w4_kernel_t pick_mx_px_upw(int upw) {
    switch (upw) {
        case 3: return w4_gemv_kernel<BF16, 4, 3, TPW, true, true>;
        case 4: return w4_gemv_kernel<BF16, 4, 4, TPW, true, true>;
        case 5: return w4_gemv_kernel<BF16, 4, 5, TPW, true, true>;
        default: return w4_gemv_kernel<BF16, 4, 6, TPW, true, true>;
    }
}

// MXFP4 with per-unit x staging (px_compiled(128, upw, tpw) says which).
template <bool BF16>
w4_kernel_t pick_mx_px(int upw, int tpw) {
    if (upw == 8) return w4_gemv_kernel<BF16, 4, 8, 1, true, true>;
    return tpw == 3 ? pick_mx_px_upw<BF16, 3>(upw) : pick_mx_px_upw<BF16, 1>(upw);
}

w4_kernel_t pick_mx_kernel(bool bf16, int upw, int tpw, bool px = false) {
    if (px) return bf16 ? pick_mx_px<true>(upw, tpw) : pick_mx_px<false>(upw, tpw);
    return bf16 ? pick_mx_upw<true>(upw, tpw) : pick_mx_upw<false>(upw, tpw);
}

// Allow every GEMV kernel the whole LDS of a CU, once per process (before any
// graph capture can be in progress for the common case of a warm-up call).
void allow_full_lds() {
    static std::once_flag once;
    std::call_once(once, [] {
        for (int bf = 0; bf < 2; ++bf)
            for (int g : {32, 64, 128, 256})
                for (int u : kUpwSet)
                  for (int tp = 1; tp <= 4; ++tp)
                    (void)hipFuncSetAttribute((const void*)pick_kernel(bf, g, u, tp),
                                              hipFuncAttributeMaxDynamicSharedMemorySize,
                                              (int)kLdsPerCu);
        for (int bf = 0; bf < 2; ++bf)
            for (int g : {64, 128})
                for (int u : kUpwSet)
                    for (int tp = 1; tp <= 4; ++tp)
                        if (px_compiled(g, u, tp))
                            (void)hipFuncSetAttribute((const void*)pick_kernel(bf, g, u, tp, true),
                                                      hipFuncAttributeMaxDynamicSharedMemorySize,
                                                      (int)kLdsPerCu);
        for (int bf = 0; bf < 2; ++bf)
            for (int u : kUpwSet)
                for (int tp = 1; tp <= 4; ++tp)
                    if (px_compiled(128, u, tp))
                        (void)hipFuncSetAttribute((const void*)pick_mx_kernel(bf, u, tp, true),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize,
                                                  (int)kLdsPerCu);
        for (int bf = 0; bf < 2; ++bf)
            for (int u : kUpwSet)
                for (int tp = 1; tp <= 4; ++tp)
                    (void)hipFuncSetAttribute((const void*)pick_mx_kernel(bf, u, tp),
                                              hipFuncAttributeMaxDynamicSharedMemorySize,
                                              (int)kLdsPerCu);
        (void)hipGetLastError();
    });
}

Plan make_plan(int M, int N, int K, int group, int cus, bool allow_px);
Plan valu_plan(int M, int N, int K, int group);

// The balanced plan, for calls of up to 4 rows on layers of C + r tiles (C
// CUs, C a multiple of r) whose K is 8 x 17 units: one workgroup per CU of 8
// "full" waves, which split the workgroup's own tile over K as the GEMV does,
// and 8 "extra" waves, which split one of P = C / r pieces of a leftover
// tile (tile C + b / P, piece b % P).  Every CU then streams the same bytes
// (the 27B down shape: 1.25 tiles each, where one tile per workgroup gives
// 64 CUs two tiles and the rest one).  The extra waves' shares are a quarter
// of a full wave's and their loads are issued first, so their partial sums
// are merged (in LDS within the workgroup, then across the P workgroups
// through an arrival counter per leftover tile, the last arrival adding the
// pieces in a fixed order) while the full waves still stream.  The extra
// waves run a chain of at most bal_extra_cl(UPW) units, a compile-time
// length, so their code stays straight-line.  Instantiated for UPW = 17 (K =
// 17408, the down layer).  At UPW = 5 (K = 5120, o_proj) it measured slower
// than one tile per workgroup (6.25 against 5.67 us per call at M = 1, 7.27
// against 6.67 at M = 4): a 5 us kernel does not hide the merge.

struct BalPlan {
    bool ok = false, px = false;
    int pieces = 0, base = 0, upw = 0;
    size_t lds = 0, ws = 0;
};

BalPlan bal_plan(int M, int N, int K, int group, int cus) {
    BalPlan b;
    if (w4h::overrides().w4_bal == 0) return b;
    const int U = (K + kUnitK - 1) / kUnitK, T = pad_n(N) / kTileN;
    // g = 128 only: at g = 64 a 17-unit chain does not fit the register
    // budget of unconditional arithmetic, which the x wait's overlap needs.
    // The full waves hold all of x, upw units each (an instantiated chain
    // length).  Up to 4 rows (the rows a lane's MFMA sums hold).
    if (M > 4 || group != 128 || K % kUnitK || U % kBalFull) return b;
    const int upw = U / kBalFull;
    if (upw != 17) return b;
    const int r = T - cus;
    if (r <= 0 || r >= cus || cus % r) return b;
    const int P = cus / r;
    if (P > kBalMaxPieces || U / P < kBalExtra) return b;
    const int cle = bal_extra_cl(upw);
    if (((U + P - 1) / P + kBalExtra - 1) / kBalExtra > cle) return b;   // extra waves' chain
    // the full and extra waves' x regions, both partial areas, the extra
    // waves' count.  Where whole-range staging does not fit (4 rows), x is
    // staged unit by unit into rings of each chain's slots (3 and 5).
    const size_t tail = (size_t)(kBalFull + kBalExtra) * M * kTileN * 4 + 16;
    b.lds = (size_t)M * kUnitK * 2 * (kBalFull * upw + kBalExtra * cle) + tail;
    b.px = b.lds > 160 * 1024 || w4h::overrides().w4_px == 1;
    if (b.px) b.lds = (size_t)1024 * (kBalFull * bal_full_ring(true) + kBalExtra * (cle < 9 ? cle : 9)) + tail;
    if (b.lds > 160 * 1024) return b;
    if ((size_t)r * kCounterStride * sizeof(unsigned) > w4h::kWsHead) return b;
    b.ok = true;
    b.pieces = P;
    b.base = cus;
    b.upw = upw;
    b.ws = w4h::ws_bytes((size_t)r * P * M * kTileN * sizeof(float));   // counters, then [tile][piece][M][16]
    return b;
}

// Whether the M-tiled kernel (w4_gemm.hip) takes the call: every M above the
// GEMV's 16, and below that from the measured crossover on.  Measured per
// call on the 27B-class layers (us, GEMV / tiled):
//   qkv      M = 8: 8.6 / 10.2   M = 12: 12.2 / 10.7
//   o_proj   M = 8: 8.3 / 9.9    M = 12: 11.9 / 10.2
//   gate_up  M = 8: 23.5 / 30.0  M = 12: 30.0 / 30.9  M = 16: 80.4 / 31.3
//   down     M = 6: 18.4 / 17.4  M = 8: 26.2 / 17.5
//   K = N = 4096  M = 8: 5.5 / 8.2
// The GEMV falls off once its workgroup needs more than half a CU's LDS (one
// workgroup per CU): its x takes M x K x 2 bytes, 80 KB (exactly half) for
// K = 5120 at M = 8.  So the tiled kernel takes M > 12, and M = 8..12 where the
// GEMV would run one tile per workgroup with more than half the LDS (on wide
// layers the GEMV streams two or three tiles per workgroup and stays ahead:
// K = N = 8192 at M = 8 takes 11.1 us with two, against 13.9 us tiled).
bool use_gemm(int M, int N, int K, int group) {
    const int t = overrides().w4_gemm_min_m;
    if (M > kMaxRows) return true;
    if (t >= 1) return M >= t;
    if (M > 12) return true;
    if (M < 8) return false;
    const Plan p = make_plan(M, N, K, group, w4h::cu_count(), false);
    return p.tpw == 1 && p.lds > kLdsPerCu / 2;
}

size_t gemm_workspace(const w4h::GemmPlan& p, int M, int N) {
    return w4h::ws_bytes(p.split > 1 ? (size_t)p.split * M * N * sizeof(float) : 0);
}

int check_gemv_args(const void* x, int x_dtype, const void* q, const void* s, const void* z,
                    const void* y, int y_dtype, int M, int N, int K, int group) {
    if (!x || !q || !s || !z || !y) return W4A16_ERR_NULL;
    if (x_dtype != W4A16_F16 && x_dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    if (y_dtype != W4A16_F32 && y_dtype != W4A16_F16 && y_dtype != W4A16_BF16)
        return W4A16_ERR_DTYPE;
    if (M < 1 || M > w4h::kMaxRowsGemm || !w4h::x_fits(M, K)) return W4A16_ERR_SHAPE;
    int rc = w4h::check_w4_shape(N, K, group);
    if (rc) return rc;
    if (!w4h::aligned16(x) || !w4h::aligned16(q) || !w4h::aligned16(s) || !w4h::aligned16(z) ||
        !w4h::aligned16(y))
        return W4A16_ERR_ALIGN;
    return W4A16_OK;
}

// The dispatch probe's text for a plan (NINFER tuning page, section 二: every
// dispatch branch names itself): the kernel instantiation and launch shape.
void format_gemv(char* b, size_t n, bool bf16, int group, const Plan& p) {
    snprintf(b, n,
             "w4_mfma16 %s g%d kernel=w4_gemv_kernel<%s, %d, %d, %d%s> tiles=%d slices=%d "
             "waves=%d upw=%d tpw=%d lds=%zu px=%d",
             bf16 ? "bf16" : "f16", group, bf16 ? "true" : "false", group / 32, p.upw, p.tpw,
             p.px ? ", false, true" : "", p.tiles, p.l.S, p.waves, p.upw, p.tpw, p.lds, (int)p.px);
}

void format_gemm(char* b, size_t n, bool bf16, int group, int N, const w4h::GemmPlan& p) {
    snprintf(b, n,
             "w4_gemm16 %s g%d kernel=w4_gemm_kernel<%s, %d, %d, %d> tiles=%d slices=%d "
             "workgroups=%lld",
             bf16 ? "bf16" : "f16", group, bf16 ? "true" : "false", group / 32, p.rb, p.tn,
             pad_n(N) / kTileN, p.split, p.workgroups);
}

// y = the slice-order sum of S fp32 partials [S][M][N] in the workspace.
int launch_gemm(const void* x, int x_dtype, const void* qweight, const void* scales, const void* zeros,
                void* y, int y_dtype, const void* res, int res_dtype, int M, int N, int K, int group,
                void* workspace, size_t workspace_bytes, hipStream_t st) {
    const w4h::GemmPlan p = w4h::gemm_plan(M, N, K, group, w4h::cu_count());
    const size_t need = gemm_workspace(p, M, N);
    if (need) {
        if (!workspace) return W4A16_ERR_NULL;
        if (workspace_bytes < need) return W4A16_ERR_WORKSPACE;
        if (!w4h::aligned16(workspace)) return W4A16_ERR_ALIGN;
    }
    const bool bf16 = x_dtype == W4A16_BF16;
    w4h::begin_launches();
    w4h::gemm_launch(p, x, bf16, qweight, scales, zeros, y, y_dtype, res, res_dtype, M, N, K, group,
                     w4h::ws_part(workspace), st);
    if (p.split > 1) w4h::launch_merge(w4h::ws_part(workspace), y, y_dtype, res, res_dtype, M, N, p.split, st);
    char v[160];
    format_gemm(v, sizeof v, bf16, group, N, p);
    w4h::set_last_variant("%s", v);
    return w4h::launch_status();
}

}  // namespace

namespace w4h {

// y = the slice-order sum of S fp32 partials [S][M][N] in the workspace (+ the
// residual, when there is one).
void launch_merge(const void* workspace, void* y, int y_dtype, const void* res, int res_dtype, int M,
                  int N, int S, hipStream_t st) {
    const int MN4 = M * N / 4;   // N % 8 == 0
    const dim3 grid((MN4 + 255) / 256);
    if (merge_kernel_t mk = pick_merge(S))
        hipLaunchKernelGGL(mk, grid, dim3(256), 0, st, (const float4_t*)workspace, y, y_dtype, MN4,
                           res, res_dtype);
    else
        hipLaunchKernelGGL(splitk_merge_any_kernel, grid, dim3(256), 0, st,
                           (const float4_t*)workspace, y, y_dtype, MN4, res, res_dtype, S);
}

}  // namespace w4h

extern "C" int w4a16_workspace_bytes(int M, int N, int K, int group, size_t* bytes) {
    if (!bytes) return W4A16_ERR_NULL;
    if (M < 1 || M > w4h::kMaxRowsGemm || !w4h::x_fits(M, K)) return W4A16_ERR_SHAPE;
    int rc = w4h::check_w4_shape(N, K, group);
    if (rc) return rc;
    if (overrides().w4_valu == 1 && M <= 8) {
        const Plan p = valu_plan(M, N, K, group);
        *bytes = w4h::ws_bytes(p.l.S > 1 ? (size_t)p.l.S * M * N * sizeof(float) : 0);
        return W4A16_OK;
    }
    if (const BalPlan b = bal_plan(M, N, K, group, w4h::cu_count()); b.ok) {
        *bytes = b.ws;
        return W4A16_OK;
    }
    if (use_gemm(M, N, K, group)) {
        *bytes = gemm_workspace(w4h::gemm_plan(M, N, K, group, w4h::cu_count()), M, N);
        return W4A16_OK;
    }
    const Plan p = make_plan(M, N, K, group, w4h::cu_count(), true);
    *bytes = w4h::ws_bytes(p.l.S > 1 ? (size_t)p.l.S * M * N * sizeof(float) : 0);
    return W4A16_OK;
}

namespace {

// The MFMA-free GEMV (A/B only, W4A16_VALU=1): the GEMV planner's split and
// x staging with one tile per workgroup.
Plan valu_plan(int M, int N, int K, int group) {
    Plan p = make_plan(M, N, K, group, w4h::cu_count(), false);
    p.tpw = 1;
    return p;
}

int launch_valu(const void* x, int x_dtype, const void* qweight, const void* scales, const void* zeros,
                void* y, int y_dtype, int M, int N, int K, int group, void* workspace,
                size_t workspace_bytes, hipStream_t st) {
    const Plan p = valu_plan(M, N, K, group);
    if (!p.upw || p.l.xstride != p.upw * kUnitK) return W4A16_ERR_UNSUPPORTED;
    const size_t need = w4h::ws_bytes(p.l.S > 1 ? (size_t)p.l.S * M * N * sizeof(float) : 0);
    if (need) {
        if (!workspace) return W4A16_ERR_NULL;
        if (workspace_bytes < need) return W4A16_ERR_WORKSPACE;
        if (!w4h::aligned16(workspace)) return W4A16_ERR_ALIGN;
    }
    const bool bf16 = x_dtype == W4A16_BF16;
    w4h::begin_launches();
    int rc = w4h::valu_launch(x, bf16, qweight, scales, zeros, p.l.S > 1 ? w4h::ws_part(workspace) : y,
                              p.l.S > 1 ? W4A16_F32 : y_dtype, M, N, K, group, p.upw, p.l.S, p.lds, st);
    if (rc) return rc;
    if (p.l.S > 1) w4h::launch_merge(w4h::ws_part(workspace), y, y_dtype, nullptr, W4A16_F32, M, N, p.l.S, st);
    w4h::set_last_variant("w4_valu %s g%d kernel=w4_gemv_valu_kernel<%s, %d, %d, %d> tiles=%d slices=%d "
                          "waves=8 upw=%d lds=%zu",
                          bf16 ? "bf16" : "f16", group, bf16 ? "true" : "false", group / 32, p.upw,
                          M == 1 ? 1 : 8, p.tiles, p.l.S, p.upw, p.lds);
    return w4h::launch_status();
}

template <bool BF16, bool MX = false>
w4_kernel_t pick_bal(int upw, bool px) {
    (void)upw;   // 17, the planner's only chain length
    return px ? w4_gemv_kernel<BF16, 4, 17, 1, MX, true, true> : w4_gemv_kernel<BF16, 4, 17, 1, MX, false, true>;
}

void format_bal(char* b, size_t n, bool bf16, bool mx, int group, int N, const BalPlan& bp) {
    if (mx)
        snprintf(b, n,
                 "mxfp4_bal16 %s kernel=w4_gemv_kernel<%s, 4, %d, 1, true, %s, true> tiles=%d "
                 "workgroups=%d waves=%d+%d pieces=%d lds=%zu px=%d",
                 bf16 ? "bf16" : "f16", bf16 ? "true" : "false", bp.upw, bp.px ? "true" : "false",
                 pad_n(N) / kTileN, bp.base, kBalFull, kBalExtra, bp.pieces, bp.lds, (int)bp.px);
    else
        snprintf(b, n,
                 "w4_bal16 %s g%d kernel=w4_gemv_kernel<%s, %d, %d, 1, false, %s, true> tiles=%d "
                 "workgroups=%d waves=%d+%d pieces=%d lds=%zu px=%d",
                 bf16 ? "bf16" : "f16", group, bf16 ? "true" : "false", group / 32, bp.upw,
                 bp.px ? "true" : "false", pad_n(N) / kTileN, bp.base, kBalFull, kBalExtra, bp.pieces, bp.lds,
                 (int)bp.px);
}

// The balanced plan's launch, for 4-bit weights (zeros given) or MXFP4 (mx:
// zeros is null, scales are the E8M0 blocks).
int launch_bal(const BalPlan& bp, const void* x, int x_dtype, const void* qweight, const void* scales,
               const void* zeros, const void* res, int res_dtype, void* y, int y_dtype, int M, int N, int K,
               int group, void* workspace, size_t workspace_bytes, hipStream_t st, bool mx = false) {
    if (!workspace) return W4A16_ERR_NULL;
    if (workspace_bytes < bp.ws) return W4A16_ERR_WORKSPACE;
    if (!w4h::aligned16(workspace)) return W4A16_ERR_ALIGN;
    static std::once_flag once;
    std::call_once(once, [] {
        for (bool px : {false, true})
            for (const void* k : {(const void*)pick_bal<false>(17, px), (const void*)pick_bal<true>(17, px),
                                  (const void*)pick_bal<false, true>(17, px),
                                  (const void*)pick_bal<true, true>(17, px)})
                (void)hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsPerCu);
        (void)hipGetLastError();
    });
    const bool bf16 = x_dtype == W4A16_BF16;
    const int U = (K + kUnitK - 1) / kUnitK, T = pad_n(N) / kTileN;
    GemvLaunch l{M, N, K, U, 1, T, bp.upw * kUnitK, y_dtype, res, res_dtype};
    l.bal_full = kBalFull;
    l.bal_pieces = bp.pieces;
    l.bal_base = bp.base;
    l.counters = (unsigned*)workspace;
    l.bal_part = (float*)w4h::ws_part(workspace);
    w4h::begin_launches();
    const w4_kernel_t k = mx ? (bf16 ? pick_bal<true, true>(bp.upw, bp.px) : pick_bal<false, true>(bp.upw, bp.px))
                             : (bf16 ? pick_bal<true>(bp.upw, bp.px) : pick_bal<false>(bp.upw, bp.px));
    hipLaunchKernelGGL(k, dim3(bp.base), dim3(64 * (kBalFull + kBalExtra)), bp.lds, st, l.M, l.K, l.U, l.T,
                       l.bal_pieces, l.bal_base, (const uint16_t*)x,
                       (const u32x4_t*)qweight, (const uint16_t*)scales, (const uint32_t*)zeros, y, l);
    char v[192];
    format_bal(v, sizeof v, bf16, mx, group, N, bp);
    w4h::set_last_variant("%s", v);
    return w4h::launch_status();
}

int gemv_impl(const void* x, int x_dtype, const void* qweight, const void* scales, const void* zeros,
              const void* res, int res_dtype, void* y, int y_dtype, int M, int N, int K, int group,
              void* workspace, size_t workspace_bytes, w4a16_stream_t stream) {
    int rc = check_gemv_args(x, x_dtype, qweight, scales, zeros, y, y_dtype, M, N, K, group);
    if (rc) return rc;
    if (overrides().w4_valu == 1 && M <= 8 && !res)
        return launch_valu(x, x_dtype, qweight, scales, zeros, y, y_dtype, M, N, K, group, workspace,
                           workspace_bytes, (hipStream_t)stream);
    if (const BalPlan bp = bal_plan(M, N, K, group, w4h::cu_count()); bp.ok)
        return launch_bal(bp, x, x_dtype, qweight, scales, zeros, res, res_dtype, y, y_dtype, M, N, K, group,
                          workspace, workspace_bytes, (hipStream_t)stream);
    if (use_gemm(M, N, K, group))
        return launch_gemm(x, x_dtype, qweight, scales, zeros, y, y_dtype, res, res_dtype, M, N, K,
                           group, workspace, workspace_bytes, (hipStream_t)stream);
    Plan p = make_plan(M, N, K, group, w4h::cu_count(), true);
    // (The kernels stage x rows of exactly upw units: xstride = 128 upw.)
    if (!p.upw || p.l.xstride != p.upw * kUnitK) return W4A16_ERR_UNSUPPORTED;
    const size_t need = w4h::ws_bytes(p.l.S > 1 ? (size_t)p.l.S * M * N * sizeof(float) : 0);
    if (need) {
        if (!workspace) return W4A16_ERR_NULL;
        if (workspace_bytes < need) return W4A16_ERR_WORKSPACE;
        if (!w4h::aligned16(workspace)) return W4A16_ERR_ALIGN;
    }
    allow_full_lds();
    hipStream_t st = (hipStream_t)stream;
    const bool bf16 = x_dtype == W4A16_BF16;
    w4_kernel_t k = pick_kernel(bf16, group, p.upw, p.tpw, p.px);
    void* out = p.l.S > 1 ? w4h::ws_part(workspace) : y;
    p.l.out_dtype = p.l.S > 1 ? W4A16_F32 : y_dtype;
    p.l.res = res;
    p.l.res_dtype = res_dtype;
    w4h::begin_launches();
    hipLaunchKernelGGL(k, dim3((p.tiles + p.tpw - 1) / p.tpw, p.l.S), dim3(64 * p.waves), p.lds, st,
                       p.l.M, p.l.K, p.l.U, p.l.T, p.l.S, p.waves,
                       (const uint16_t*)x,
                       (const u32x4_t*)qweight, (const uint16_t*)scales, (const uint32_t*)zeros,
                       out, p.l);
    if (p.l.S > 1) w4h::launch_merge(w4h::ws_part(workspace), y, y_dtype, res, res_dtype, M, N, p.l.S, st);
    char v[160];
    format_gemv(v, sizeof v, bf16, group, p);
    w4h::set_last_variant("%s", v);
    return w4h::launch_status();
}

}  // namespace

extern "C" int w4a16_plan_variant(int M, int N, int K, int group, int x_dtype, char* text,
                                  size_t text_bytes) {
    if (!text || text_bytes == 0) return W4A16_ERR_NULL;
    if (x_dtype != W4A16_F16 && x_dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    if (M < 1 || M > w4h::kMaxRowsGemm || !w4h::x_fits(M, K)) return W4A16_ERR_SHAPE;
    if (int rc = w4h::check_w4_shape(N, K, group)) return rc;
    const bool bf16 = x_dtype == W4A16_BF16;
    if (const BalPlan bp = bal_plan(M, N, K, group, w4h::cu_count()); bp.ok && overrides().w4_valu != 1) {
        format_bal(text, text_bytes, bf16, false, group, N, bp);
        return W4A16_OK;
    }
    if (use_gemm(M, N, K, group)) {
        format_gemm(text, text_bytes, bf16, group, N, w4h::gemm_plan(M, N, K, group, w4h::cu_count()));
        return W4A16_OK;
    }
    const Plan p = make_plan(M, N, K, group, w4h::cu_count(), true);
    if (!p.upw) return W4A16_ERR_UNSUPPORTED;
    format_gemv(text, text_bytes, bf16, group, p);
    return W4A16_OK;
}

extern "C" int w4a16_gemv(const void* x, int x_dtype, const void* qweight, const void* scales,
                          const void* zeros, void* y, int y_dtype, int M, int N, int K, int group,
                          void* workspace, size_t workspace_bytes, w4a16_stream_t stream) {
    return gemv_impl(x, x_dtype, qweight, scales, zeros, nullptr, W4A16_F32, y, y_dtype, M, N, K, group,
                     workspace, workspace_bytes, stream);
}

extern "C" int w4a16_gemv_add(const void* x, int x_dtype, const void* qweight, const void* scales,
                              const void* zeros, const void* residual, int residual_dtype, void* y,
                              int y_dtype, int M, int N, int K, int group, void* workspace,
                              size_t workspace_bytes, w4a16_stream_t stream) {
    if (!residual) return W4A16_ERR_NULL;
    if (residual_dtype != W4A16_F32 && residual_dtype != W4A16_F16 && residual_dtype != W4A16_BF16)
        return W4A16_ERR_DTYPE;
    if (!w4h::aligned16(residual)) return W4A16_ERR_ALIGN;
    return gemv_impl(x, x_dtype, qweight, scales, zeros, residual, residual_dtype, y, y_dtype, M, N, K,
                     group, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------- no-allocation variant

// The split-K workspace of w4a16_gemv_noalloc: a library-owned device array,
// one copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol):
// the device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kNoAllocScratchBytes = W4A16_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kScratchDevices = 64;
std::once_flag g_scratch_once[kScratchDevices];
void* g_scratch_ptr[kScratchDevices];
hipError_t g_scratch_err[kScratchDevices];

// The device address of `scratch` on the current device, looked up the first
// time this device is used (with that device current) and kept.
int scratch_for_current_device(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) {
        w4h::set_last_error("no usable current HIP device for the static scratch");
        return W4A16_ERR_HIP;
    }
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) {
        w4h::set_last_error(hipGetErrorName(g_scratch_err[dev]));
        return W4A16_ERR_HIP;
    }
    *ptr = g_scratch_ptr[dev];
    return W4A16_OK;
}

}  // namespace

extern "C" int w4a16_gemv_noalloc(const void* x, int x_dtype, const void* qweight, const void* scales,
                                  const void* zeros, void* y, int y_dtype, int M, int N, int K,
                                  int group, w4a16_stream_t stream) {
    // Everything w4a16_gemv checks, then the workspace this shape needs
    // against the static array -- all on the host, before any device work.
    if (int rc = check_gemv_args(x, x_dtype, qweight, scales, zeros, y, y_dtype, M, N, K, group))
        return rc;
    size_t need = 0;
    if (int rc = w4a16_workspace_bytes(M, N, K, group, &need)) return rc;
    if (need > kNoAllocScratchBytes) {
        char msg[96];
        snprintf(msg, sizeof msg, "workspace of %zu bytes exceeds the %zu-byte static scratch", need,
                 kNoAllocScratchBytes);
        w4h::set_last_error(msg);
        return W4A16_ERR_WORKSPACE;
    }
    void* ws = nullptr;
    if (need) {
        if (int rc = scratch_for_current_device(&ws)) return rc;
    }
    return gemv_impl(x, x_dtype, qweight, scales, zeros, nullptr, W4A16_F32, y, y_dtype, M, N, K, group,
                     ws, need ? kNoAllocScratchBytes : 0, stream);
}

// ------------------------------------------------------------------ MXFP4

namespace {

// MXFP4 runs the 4-bit kernels' plans as for g = 128 (same slot size, same
// units, same GEMV / M-tiled crossover): rows 1..64.
constexpr int kMxPlanGroup = 128;

int check_mx_args(const void* x, int x_dtype, const void* q, const void* s, const void* y,
                  int y_dtype, int M, int N, int K) {
    if (!x || !q || !s || !y) return W4A16_ERR_NULL;
    if (x_dtype != W4A16_F16 && x_dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    if (y_dtype != W4A16_F32 && y_dtype != W4A16_F16 && y_dtype != W4A16_BF16)
        return W4A16_ERR_DTYPE;
    if (M < 1 || M > w4h::kMaxRowsGemm || !w4h::x_fits(M, K)) return W4A16_ERR_SHAPE;
    if (int rc = w4h::check_mx_shape(N, K)) return rc;
    if (!w4h::aligned16(x) || !w4h::aligned16(q) || !w4h::aligned16(s) || !w4h::aligned16(y))
        return W4A16_ERR_ALIGN;
    return W4A16_OK;
}

}  // namespace

extern "C" int mxfp4_workspace_bytes(int M, int N, int K, size_t* bytes) {
    if (!bytes) return W4A16_ERR_NULL;
    if (M < 1 || M > w4h::kMaxRowsGemm || !w4h::x_fits(M, K)) return W4A16_ERR_SHAPE;
    if (int rc = w4h::check_mx_shape(N, K)) return rc;
    if (const BalPlan b = bal_plan(M, N, K, kMxPlanGroup, w4h::cu_count()); b.ok) {
        *bytes = b.ws;
        return W4A16_OK;
    }
    if (use_gemm(M, N, K, kMxPlanGroup)) {
        *bytes = gemm_workspace(w4h::gemm_plan(M, N, K, kMxPlanGroup, w4h::cu_count()), M, N);
        return W4A16_OK;
    }
    const Plan p = make_plan(M, N, K, kMxPlanGroup, w4h::cu_count(), true);
    *bytes = w4h::ws_bytes(p.l.S > 1 ? (size_t)p.l.S * M * N * sizeof(float) : 0);
    return W4A16_OK;
}

extern "C" int mxfp4_gemv(const void* x, int x_dtype, const void* qweight, const void* scales, void* y,
                          int y_dtype, int M, int N, int K, void* workspace, size_t workspace_bytes,
                          w4a16_stream_t stream) {
    if (int rc = check_mx_args(x, x_dtype, qweight, scales, y, y_dtype, M, N, K)) return rc;
    if (const BalPlan bp = bal_plan(M, N, K, kMxPlanGroup, w4h::cu_count()); bp.ok)
        return launch_bal(bp, x, x_dtype, qweight, scales, nullptr, nullptr, W4A16_F32, y, y_dtype, M, N, K,
                          kMxPlanGroup, workspace, workspace_bytes, (hipStream_t)stream, true);
    if (use_gemm(M, N, K, kMxPlanGroup)) {
        // Rows past the GEMV's crossover: the M-tiled kernel's MXFP4 mode.
        const w4h::GemmPlan gp = w4h::gemm_plan(M, N, K, kMxPlanGroup, w4h::cu_count());
        const size_t need = gemm_workspace(gp, M, N);
        if (need) {
            if (!workspace) return W4A16_ERR_NULL;
            if (workspace_bytes < need) return W4A16_ERR_WORKSPACE;
            if (!w4h::aligned16(workspace)) return W4A16_ERR_ALIGN;
        }
        const bool bf16 = x_dtype == W4A16_BF16;
        hipStream_t st = (hipStream_t)stream;
        w4h::begin_launches();
        w4h::gemm_launch(gp, x, bf16, qweight, scales, nullptr, y, y_dtype, nullptr, W4A16_F32, M, N, K,
                         kMxPlanGroup, w4h::ws_part(workspace), st, true);
        if (gp.split > 1) w4h::launch_merge(w4h::ws_part(workspace), y, y_dtype, nullptr, W4A16_F32, M, N, gp.split, st);
        w4h::set_last_variant("mxfp4_gemm16 %s kernel=w4_gemm_kernel<%s, 4, %d, %d, true> tiles=%d "
                              "slices=%d workgroups=%lld",
                              bf16 ? "bf16" : "f16", bf16 ? "true" : "false", gp.rb, gp.tn,
                              pad_n(N) / kTileN, gp.split, gp.workgroups);
        return w4h::launch_status();
    }
    Plan p = make_plan(M, N, K, kMxPlanGroup, w4h::cu_count(), true);
    if (!p.upw || p.l.xstride != p.upw * kUnitK) return W4A16_ERR_UNSUPPORTED;
    const size_t need = w4h::ws_bytes(p.l.S > 1 ? (size_t)p.l.S * M * N * sizeof(float) : 0);
    if (need) {
        if (!workspace) return W4A16_ERR_NULL;
        if (workspace_bytes < need) return W4A16_ERR_WORKSPACE;
        if (!w4h::aligned16(workspace)) return W4A16_ERR_ALIGN;
    }
    allow_full_lds();
    hipStream_t st = (hipStream_t)stream;
    const bool bf16 = x_dtype == W4A16_BF16;
    w4_kernel_t k = pick_mx_kernel(bf16, p.upw, p.tpw, p.px);
    void* out = p.l.S > 1 ? w4h::ws_part(workspace) : y;
    p.l.out_dtype = p.l.S > 1 ? W4A16_F32 : y_dtype;
    w4h::begin_launches();
    hipLaunchKernelGGL(k, dim3((p.tiles + p.tpw - 1) / p.tpw, p.l.S), dim3(64 * p.waves), p.lds, st,
                       p.l.M, p.l.K, p.l.U, p.l.T, p.l.S, p.waves,
                       (const uint16_t*)x, (const u32x4_t*)qweight, (const uint16_t*)scales,
                       (const uint32_t*)nullptr, out, p.l);
    if (p.l.S > 1) w4h::launch_merge(w4h::ws_part(workspace), y, y_dtype, nullptr, W4A16_F32, M, N, p.l.S, st);
    w4h::set_last_variant("mxfp4_mfma16 %s kernel=w4_gemv_kernel<%s, 4, %d, %d, true%s> tiles=%d "
                          "slices=%d waves=%d upw=%d tpw=%d lds=%zu px=%d",
                          bf16 ? "bf16" : "f16", bf16 ? "true" : "false", p.upw, p.tpw,
                          p.px ? ", true" : "", p.tiles, p.l.S, p.waves, p.upw, p.tpw, p.lds, (int)p.px);
    return w4h::launch_status();
}
