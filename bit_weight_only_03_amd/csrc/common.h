// common.h -- shared definitions of the gfx950 W4A16 / ternary library:
// device-layout geometry, bit-cast helpers and host-side argument checks.
//
// Device layout of the 4-bit weights ("w4").  Columns are grouped in tiles of
// 16, k in units of 128.  One unit of one tile is 1 KiB: 64 lanes x 16 bytes,
// exactly one 16-byte load per lane of a wave64, so a wave streams a tile with
// fully coalesced dwordx4 loads and every lane dequantizes in registers.
//   qweight_dev uint32 [Np/16][Kp/128][64 lanes][4 dwords]
//   lane l: column n = 16*t + (l & 15), k-block kc = l >> 4
//   dword j of lane l in unit u holds the 8 weights k = 128u + 32j + 8kc + e,
//   e = 0..7, which are exactly the 8 nibbles of canonical word
//   qweight[n][16u + 4j + kc].  Inside the dword, nibble position p
//   (bits 4p..4p+3) holds element e = kNibbleElem[p] = {0,2,4,6,1,3,5,7}[p], so
//   masks 0x000F000F / 0x00F000F0 applied to the word and to the word >> 8 give
//   the element pairs (0,1), (2,3), (4,5), (6,7) in the two 16-bit halves.
//   scales_dev uint16 [Np/16][Gp][16]     (fp16 scale of group g, column c)
//   zeros_dev  uint32 [Np/16][Gp][2]      (nibble c of the 8 bytes = zero of column c)
// with Np = N rounded up to 16, Kp = K rounded up to 128, Gp = Kp / group.
// Padding holds q = 0, z = 0, s = +0, so padded weights are exactly zero.
//
// Device layout of the ternary weights ("w2t"): the same tiles with 256-k units.
//   qweight_dev uint32 [Np/16][Kp/256][64][4]; dword d of lane l in unit u holds
//   16 codes: k = 256u + 32(2d + h) + 8kc + e for h = 0, 1 and e = 0..7, i.e. the
//   16 fields of canonical word codes[n][16u + 4d + 2h... ] -- see w2t.hip.
//   scales_dev uint16 [Np/16][Gp][16], Kp = K rounded up to 256, Gp = Kp / group.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/w4a16.h"

namespace w4k {

constexpr int kTileN = 16;       // columns per tile
constexpr int kUnitK = 128;      // k per 4-bit unit (one 16-byte load per lane)
constexpr int kUnitK2 = 256;     // k per ternary unit
constexpr int kLanes = 64;

__host__ __device__ inline int pad_n(int N) { return (N + 15) & ~15; }
__host__ __device__ inline int pad_k(int K) { return (K + kUnitK - 1) / kUnitK * kUnitK; }
__host__ __device__ inline int pad_k2(int K) { return (K + kUnitK2 - 1) / kUnitK2 * kUnitK2; }

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& v) {
    static_assert(sizeof(To) == sizeof(From), "size mismatch");
    return __builtin_bit_cast(To, v);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
    return (float)bitcast<_Float16>(h);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN kept quiet).
__host__ __device__ inline uint16_t f32_to_bf16_bits(float f) {
    uint32_t b = __builtin_bit_cast(uint32_t, f);
    if ((b & 0x7f800000u) == 0x7f800000u && (b & 0x7fffffu)) return (uint16_t)((b >> 16) | 0x40);
    b += 0x7fffu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

// v + r[o], with r read in its dtype (f32, f16 or bf16); no residual: v.
// The fused residual add of the GEMV epilogues (Ninfer V100 article, section
// 十四: adding the input back inside the matmul's output stage saves a pass
// through memory).
__device__ __forceinline__ float add_residual(float v, const void* r, int r_dtype, size_t o) {
    if (!r) return v;
    if (r_dtype == W4A16_F32) return v + ((const float*)r)[o];
    if (r_dtype == W4A16_F16) return v + (float)((const _Float16*)r)[o];
    return v + __builtin_bit_cast(float, (uint32_t)((const uint16_t*)r)[o] << 16);
}

// y[o] = v in the output dtype (f32, f16, or bf16 rounded to nearest even).
__device__ __forceinline__ void store_out(void* out, int out_dtype, size_t o, float v) {
    if (out_dtype == W4A16_F32)
        ((float*)out)[o] = v;
    else if (out_dtype == W4A16_F16)
        ((_Float16*)out)[o] = (_Float16)v;
    else
        ((uint16_t*)out)[o] = f32_to_bf16_bits(v);
}

// Streamed, read-once loads: non-temporal so the weights do not evict x and
// the scales from the caches.
__device__ __forceinline__ u32x4_t load_nt(const u32x4_t* p) {
    return __builtin_nontemporal_load(p);
}

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return bitcast<half2_t>(v); }
__device__ __forceinline__ uint32_t as_u(half2_t v) { return bitcast<uint32_t>(v); }

// (a & mask) | b, for a b with no bit inside mask (the magic exponents below
// never overlap the nibble masks): one v_and_or_b32 when b is a VGPR value
// the compiler cannot fold, which opaque_v gives the kernels' magic words
// (a folded constant splits it into v_and + v_or).  Plain C on purpose, not an
// inline-asm v_bfi_b32: an MFMA may only read a VGPR two wait states after
// the VALU op that wrote it, and the compiler inserts those only for writes it
// can see -- an asm statement is not one, and a bf16 operand built by asm and
// read by the next-but-one MFMA came out stale.
__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t a, uint32_t b) {
    return (a & mask) | b;
}

// v, held in a VGPR the optimiser treats as unknown (emits no instruction).
__device__ __forceinline__ uint32_t opaque_v(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

// Dequantization in registers, shared by the GEMV and the M-tiled kernel.
// The device dword of a lane holds 8 nibbles; a half pair takes nibbles
// (0, 4), (1, 5), (2, 6), (3, 7), which the pack kernel places at the k
// positions the MFMA B operand expects.
//
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

// bf16 activations for the 4-bit kernels: the staged x is rewritten in place
// as fp16, so the products take the exact fp16 q - z above (gfx950 has no
// packed bf16 add to form q - z in bf16, and a biased bf16 operand with a
// separate zero-point product leaves q = z as a rounding residue instead of
// an exact 0).  One 16-byte chunk, 8 values: bf16 -> fp32 is a shift or a
// mask, fp32 -> fp16 one v_cvt_pk_f16_f32 per pair, round to nearest even.
// Exact for every bf16 value of magnitude in [2^-17, 65280] and for zeros;
// smaller magnitudes land on fp16's 2^-24 subnormal grid (a change below
// 2^-25), and magnitudes of 65536 or more (past fp16's range) become
// infinite -- outside the library's contract for bf16 x.
__device__ __forceinline__ u32x4_t bf16x8_to_f16x8(u32x4_t v) {
    u32x4_t r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float lo = bitcast<float>(v[j] << 16);
        const float hi = bitcast<float>(v[j] & 0xffff0000u);
        r[j] = as_u(half2_t{(_Float16)lo, (_Float16)hi});
    }
    return r;
}

// MXFP4 (OCP MX v1.0: E2M1 elements, one E8M0 scale per 32 elements along K).
// B operand (8 fp16 or bf16 elements) from one device dword of 8 E2M1 codes,
// element e in bits 4e..4e+3: v_cvt_scalef32_pk_{f16,bf16}_fp4 converts the
// two codes of one byte, low nibble first, times the power-of-two scale sc.
// Every E2M1 value (0, +-0.5 .. +-6) times sc is exact in the target type
// while it stays within its range (fp16: 2^-24 grid, below 65504).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ half8_t fp4x8_to_f16(uint32_t d, float sc) {
    const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, sc, 0);
    const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, sc, 1);
    const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, sc, 2);
    const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, sc, 3);
    return bitcast<half8_t>(u32x4_t{as_u(p0), as_u(p1), as_u(p2), as_u(p3)});
}
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16(uint32_t d, float sc) {
    const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 0);
    const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 1);
    const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 2);
    const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 3);
    return bitcast<bf16x8_t>(u32x4_t{bitcast<uint32_t>(p0), bitcast<uint32_t>(p1),
                                     bitcast<uint32_t>(p2), bitcast<uint32_t>(p3)});
}

// E8M0 scale code e (0..254) -> 2^(e - 127), exact in fp32 (2^-127 is a
// subnormal).  Code 255, the NaN encoding, is outside the library's contract.
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
    return __builtin_ldexpf(0x1p-127f, (int)e);
}

// The scales of one 128-k unit of one column: the E8M0 codes e_j of its four
// 32-k blocks (byte j of the unit's scale dword), which are the four MFMA
// steps.  With R = max e_j - 13, step j converts its elements with the scale
// 2^(e_j - R) folded in: exact in fp16 while e_j >= R - 23, i.e. while the
// four codes span at most kMxFoldSpan (every value lands on fp16's 2^-24 grid
// and stays below 6 * 2^13; bf16 has range to spare).  The steps then chain
// in one accumulator and the unit's sum takes 2^(R - 127) once.  A unit with
// a wider span is taken step by step, each step's fp32 sum times its own
// 2^(e_j - 127) -- the MX specification's block dot product.
constexpr uint32_t kMxFoldSpan = 36;
struct MxUnit {
    uint32_t e[4];
    uint32_t emax;
    bool wide;   // the four codes span more than kMxFoldSpan
};
__device__ __forceinline__ MxUnit mx_unit(uint32_t s) {
    MxUnit u;
#pragma unroll
    for (int j = 0; j < 4; ++j) u.e[j] = (s >> (8 * j)) & 255u;
    u.emax = max(max(u.e[0], u.e[1]), max(u.e[2], u.e[3]));
    const uint32_t emin = min(min(u.e[0], u.e[1]), min(u.e[2], u.e[3]));
    u.wide = u.emax - emin > kMxFoldSpan;
    return u;
}
// 2^(e - R) as fp32 bits: exponent field e - emax + 140 (104..140 when folded).
__device__ __forceinline__ float mx_fold_scale(uint32_t e, uint32_t emax) {
    return __builtin_bit_cast(float, (e + 140u - emax) << 23);
}
// 2^(R - 127) = 2^(emax - 140), a subnormal for emax < 14.
__device__ __forceinline__ float mx_unit_scale(uint32_t emax) {
    return __builtin_ldexpf(1.0f, (int)emax - 140);
}

// Raw buffer resources: a wave-uniform 128-bit descriptor (base, byte size)
// lets every load take its lane offset from one VGPR and its unit offset from
// an SGPR, with no per-load 64-bit address arithmetic.  Lanes whose
// VGPR + immediate offset falls outside the byte size read zeros, and a
// descriptor of byte size 0 reads zeros for every lane: the GEMV selects one
// (on the scalar side) for a unit or tile that does not exist.
constexpr int kRsrcFlags = 0x00020000;   // raw (untyped) 32-bit data, gfx9 family
constexpr int kAuxNT = 2;                // non-temporal cache policy

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kRsrcFlags);
}

}  // namespace w4k

// ---------------------------------------------------------------- host side

namespace w4h {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Every workspace begins with kWsHead bytes of arrival counters, zero before
// the workspace's first use and left zero by every call; a call's fp32
// partial sums follow them.  ws_bytes gives the workspace a call needs for
// `partials` bytes of partial sums (0: none at all).
constexpr size_t kWsHead = 64 * 1024;
inline size_t ws_bytes(size_t partials) { return partials ? kWsHead + partials : 0; }
inline void* ws_part(void* ws) { return ws ? (uint8_t*)ws + kWsHead : nullptr; }

inline bool group_ok(int group) {
    return group == 32 || group == 64 || group == 128 || group == 256;
}

// Largest K: keeps every per-workgroup weight, scale and zero-point offset
// (at most three tiles' columns) inside the 32-bit offsets of the kernels'
// buffer resources.
constexpr int kMaxK = 1 << 26;

// x as one buffer resource (M * K * 2 bytes addressed by 32-bit offsets).
inline bool x_fits(int M, int K) { return (long long)M * K * 2 <= 0xffffffffLL; }

// Shape contract of the 4-bit functions (see w4a16.h).
inline int check_w4_shape(int N, int K, int group) {
    if (N < 1 || K < 1 || K > kMaxK || !group_ok(group)) return W4A16_ERR_SHAPE;
    if (N % 8 || K % 8 || K % group) return W4A16_ERR_SHAPE;
    return W4A16_OK;
}

// Shape contract of the MXFP4 functions (see w4a16.h).
inline int check_mx_shape(int N, int K) {
    if (N < 8 || K < 32 || K > kMaxK || N % 8 || K % 32) return W4A16_ERR_SHAPE;
    return W4A16_OK;
}

inline int check_w2_shape(int N, int K, int group) {
    if (N < 1 || K < 1 || K > kMaxK || !group_ok(group)) return W4A16_ERR_SHAPE;
    if (K % 16 || K % group) return W4A16_ERR_SHAPE;
    return W4A16_OK;
}

// Compute units of the current device (256 on MI355X; 256 if the query
// fails), cached per device.  Host only.
int cu_count();

// Planner overrides for A/B measurement, read from the environment once per
// process, at the first planner call; later changes to the environment are
// not seen, so a shape's plan -- and the workspace size it implies -- stays
// the same for the life of the process (NINFER tuning page, section 七:
// decode-path choices stay frozen; section 五: workspace capacity is declared
// up front).  0 (or -1 where 0 is meaningful) means automatic.
struct Overrides {
    int w4_waves = 0;          // W4A16_WAVES: waves per GEMV workgroup
    int w4_split = 0;          // W4A16_SPLIT: GEMV K slices
    int w4_tpw = 0;            // W4A16_TPW: GEMV tiles per workgroup
    int w4_gemm_min_m = 0;     // W4A16_GEMM_MIN_M: rows from which the M-tiled kernel runs
    int w4_px = -1;            // W4A16_PX: 0 turns per-unit x staging off
    int w4_valu = 0;           // W4A16_VALU: 1 runs the MFMA-free GEMV (up to 8 rows)
    int w4_bal = -1;           // W4A16_BAL: 0 turns the balanced GEMV plan off
    int gemm_tn = 0;           // W4A16_GEMM_TN: tiles per wave of the M-tiled kernel
    int gemm_split = 0;        // W4A16_GEMM_SPLIT: K slices of the M-tiled kernel
    int w16_ksplit = -1;       // W16A16_KSPLIT: 0 turns the W16 K-split kernel off
    int w16_dot = -1;          // W16A16_DOT: 0 turns the W16 dot-product kernel off
    int w16_bal = -1;          // W16A16_BAL: 0 / 1 turns the W16 even-share kernel off / on where it fits
    int w16_split = 0;         // W16A16_SPLIT: K slices of the W16 tiled kernel
    long long w2t_staged_lds_max = 0;   // W2T_STAGED_LDS_MAX: LDS limit of the staged ternary kernel
};
const Overrides& overrides();

void set_last_variant(const char* fmt, ...);
void set_last_error(const char* what);

// Launch checking.  begin_launches() clears an error another component may
// have left in HIP's per-thread "last error" slot (it belongs to an earlier
// call, not to this one); launch_status() then reports only what the launches
// of this call raised, and records the HIP error name for w4a16_last_error().
inline void begin_launches() { (void)hipGetLastError(); }

inline int launch_status() {
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) return W4A16_OK;
    set_last_error(hipGetErrorName(e));
    return W4A16_ERR_HIP;
}

// y = the slice-order sum of S fp32 partials [S][M][N] (+ residual); N % 8 == 0.
void launch_merge(const void* workspace, void* y, int y_dtype, const void* res, int res_dtype, int M,
                  int N, int S, hipStream_t st);

// The MFMA-free GEMV (w4_gemv_valu.hip), an A/B alternative selected only by
// the W4A16_VALU override.
int valu_launch(const void* x, bool bf16, const void* qweight, const void* scales, const void* zeros,
                void* out, int out_dtype, int M, int N, int K, int group, int upw, int S, size_t lds,
                hipStream_t st);

// The M-tiled path (w4_gemm.hip) for rows the GEMV does not take.
constexpr int kMaxRowsGemm = 64;
constexpr int kMaxSplitGemm = 16;
struct GemmPlan {
    int rb;                 // 16-row blocks
    int tn;                 // 16-column tiles per wave
    int split;              // K slices
    long long workgroups;   // tile columns of workgroups (grid x)
};
GemmPlan gemm_plan(int M, int N, int K, int group, int cus);
// mx: MXFP4 weights (mxfp4.hip's layout; zeros unused), else 4-bit integers.
int gemm_launch(const GemmPlan& p, const void* x, bool bf16, const void* qweight, const void* scales,
                const void* zeros, void* y, int y_dtype, const void* res, int res_dtype, int M, int N,
                int K, int group, void* workspace, hipStream_t st, bool mx = false);

}  // namespace w4h
