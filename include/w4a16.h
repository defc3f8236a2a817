/*
 * w4a16.h -- C ABI of the MI355X (gfx950) small-M W4A16 / ternary linear layer.
 *
 * The operation.  One decode step's linear layer, y[M,N] = x[M,K] . W[K,N],
 * where M is 1 for a single generated token or a few rows when draft tokens
 * are verified together, so every call re-reads all of W once
 * (Ninfer V100 article, haowenji.com, section 三: decode speed is bounded by
 * memory bandwidth over the bytes read per token, and verifying several
 * draft tokens costs one weight read; Z100 vLLM port article,
 * forum.sourcefind.cn, section 五: stream the weights once for all M rows).
 * W is stored group-wise as 4-bit integers: for the group of `group`
 * consecutive k of column n, w = (q - z) * s with an fp16 scale s and a 4-bit
 * zero point z (Ninfer V100 article, section 十一, "groupwise-int"; Z100
 * article, section 四, unpack INT4, read scale and zero point, restore,
 * multiply-add).  The ternary variant stores w in {-1, 0, +1} times a per-group
 * scale ("NINFER 三元引擎性能调优", sections 五 and 六).  Accumulation is fp32.
 *
 * Canonical storage (the format callers hand in; all little-endian):
 *   qweight_canon int32 [N][K/8]   nibble i (bits 4i..4i+3) of word (n, j) = q[8j+i][n]
 *   scales_canon  fp16  [K/group][N]
 *   zeros_canon   int32 [K/group][N/8]  nibble i of word (g, j) = z[g][8j+i]
 *   codes_canon   int32 [N][K/16]  2-bit field i of word (n, j) = c[16j+i][n],
 *                                  ternary weight = c - 1, c in {0, 1, 2}
 *   x             fp16 or bf16 [M][K], row-major, contiguous (leading dim K)
 *   y             fp32, fp16 or bf16 [M][N], row-major, contiguous (leading dim N)
 *
 * Device layout.  *_pack converts canonical arrays into the library's own
 * interleaved layout once, at load time, before any graph capture (Z100
 * article, section 四: the repacked weights and the output-major scales and
 * zero points must be built after loading, not lazily inside a captured
 * graph).  Its sizes come from *_packed_sizes; its contents are opaque and
 * *_unpack restores the canonical arrays bit for bit.  The device arrays hold
 * exactly the canonical information (4-bit q and z, fp16 s), padded up to
 * whole 16-column by 128-k tiles (256-k for ternary).
 *
 * Conventions for every function:
 *   - Pointers are device pointers unless stated otherwise.  All buffers are
 *     owned by the caller; the library never allocates or frees memory and
 *     keeps no per-call state.
 *   - Device pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     asynchronously; no function synchronizes, so every call can be captured
 *     into a hipGraph.
 *   - Arguments are checked on the host before anything is launched; a
 *     negative w4a16_status is returned and nothing is enqueued.  There is
 *     never a silent fallback: a valid but unsupported request returns
 *     W4A16_ERR_UNSUPPORTED.  A launch failure returns W4A16_ERR_HIP.
 *   - Size-query functions (*_packed_sizes, *_workspace_bytes) do no GPU work.
 *   - Workspaces (sized by the *_workspace_bytes queries; 0 = pass NULL):
 *     the first W4A16_WORKSPACE_HEAD_BYTES of a workspace hold arrival
 *     counters.  Zero them once, when the workspace is allocated
 *     (hipMemset, or a zero-filled allocation); every call leaves them zero
 *     again.  The rest is scratch that a call writes before it reads it.  So
 *     one workspace, zeroed once, may serve any sequence of calls of any
 *     entry point and shape on one stream, graph replays included; calls
 *     that may overlap in time need distinct workspaces.  A head that is not
 *     zero gives wrong results (never a fault or a hang: no kernel waits on
 *     a counter).
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;                       /* hipStream_t is struct ihipStream_t* */
#define W4A16_WORKSPACE_HEAD_BYTES (64u << 10)
typedef struct ihipStream_t* w4a16_stream_t;

typedef enum {
    W4A16_OK = 0,
    W4A16_ERR_NULL = -1,         /* a required pointer is NULL */
    W4A16_ERR_SHAPE = -2,        /* M, N, K or group outside the contract */
    W4A16_ERR_ALIGN = -3,        /* a device pointer is not 16-byte aligned */
    W4A16_ERR_DTYPE = -4,        /* unknown or disallowed dtype */
    W4A16_ERR_WORKSPACE = -5,    /* workspace smaller than *_workspace_bytes */
    W4A16_ERR_UNSUPPORTED = -6,  /* valid request this library does not implement */
    W4A16_ERR_HIP = -7           /* the HIP runtime reported an error at launch */
} w4a16_status;

typedef enum { W4A16_F16 = 0, W4A16_BF16 = 1, W4A16_F32 = 2 } w4a16_dtype;

/* Shape contract shared by the 4-bit functions:
 *   1 <= N, 1 <= K <= 2^26, N % 8 == 0, K % group == 0, K % 8 == 0,
 *   group in {32, 64, 128, 256}; for the GEMV also 1 <= M <= 64 and
 *   M * K * 2 < 2^32 (x is addressed through 32-bit offsets).  The MXFP4 and
 *   ternary functions take the same limits on K and M * K. */

/* Bytes of the device layout for an N x K matrix with the given group, so a
 * caller can allocate the repacked weights once, at load time, before any
 * capture (Z100 article, section 四: repack once after loading; NINFER tuning
 * page, section 五: sizes declared up front).  Host only.  Returns W4A16_OK or
 * W4A16_ERR_SHAPE / W4A16_ERR_NULL. */
int w4a16_packed_sizes(int N, int K, int group, size_t* q_bytes, size_t* s_bytes,
                       size_t* z_bytes);

/* Canonical -> device layout (a pure bit permutation plus zero padding).
 * Reads qweight_canon [N][K/8], scales_canon [K/group][N], zeros_canon
 * [K/group][N/8]; writes the three device arrays of w4a16_packed_sizes bytes
 * (every byte, padding included).  Canonical and device buffers must not
 * overlap. */
int w4a16_pack(const int32_t* qweight_canon, const uint16_t* scales_canon,
               const int32_t* zeros_canon, void* qweight, void* scales, void* zeros, int N,
               int K, int group, w4a16_stream_t stream);

/* Device layout -> canonical, the exact inverse of w4a16_pack: every byte of
 * the canonical arrays comes back as it went in.  A conversion of the weight
 * files must be checkable bit for bit against the original (Ninfer V100
 * article, section 十三: the 452 weight blocks of the split files were
 * compared with the source file bit by bit).  Same arguments, sizes and
 * errors as w4a16_pack, with the roles of the two sides swapped; the
 * buffers must not overlap. */
int w4a16_unpack(const void* qweight, const void* scales, const void* zeros,
                 int32_t* qweight_canon, uint16_t* scales_canon, int32_t* zeros_canon, int N,
                 int K, int group, w4a16_stream_t stream);

/* Workspace bytes w4a16_gemv needs for this shape: 0 when its plan needs
 * none, else the counter head plus fp32 partial sums (a K split, or the
 * balanced plan's pieces of leftover tiles).  Host only; the answer is fixed
 * for the life of the process, so a workspace sized once may be reused
 * inside a captured graph (NINFER tuning page, section 五: declare workspace
 * capacity up front). */
int w4a16_workspace_bytes(int M, int N, int K, int group, size_t* bytes);
/* (The A/B overrides the planners honour are read from the environment once,
 * at the first size query or call of the process; see w4a16_plan_variant.) */

/* y[M,N] = x[M,K] . ((q - z) * s)[K,N] from the packed device layout, for
 * 1 <= M <= 64 (the Z100 article, section 五: the weights are read and
 * dequantized once for every row).  A few rows run a GEMV kernel whose waves
 * split K; larger M (from a crossover measured per layer shape; always above
 * 16) runs an M-tiled kernel whose waves split N and share x through LDS.
 * Layers a little wider than one 16-column tile per CU (C + r tiles on C
 * CUs, r dividing C) with long K run, up to 4 rows, a balanced GEMV whose
 * workgroups also split the r leftover tiles over K and merge those pieces
 * through the workspace.  w4a16_last_variant() names the kernel that ran.
 * x_dtype: W4A16_F16 or W4A16_BF16.  y_dtype: W4A16_F32, W4A16_F16 or
 * W4A16_BF16 (rounded to nearest even from the fp32 result).  q - z is formed
 * exactly before any product (the integer placed in a 16-bit float's mantissa
 * and a constant subtracted: Ninfer V100 article, section 十), so q = z gives
 * exactly 0 and s -> 2s exactly 2y.  bf16 x is taken to fp16 on chip before
 * the products: exact for every magnitude in [2^-17, 65280] and for zeros,
 * rounded to fp16's 2^-24 grid below 2^-17 (a change under 2^-25 per
 * element); magnitudes of 65536 and above are outside the contract (they
 * overflow fp16).  A bf16 x therefore gives bit for bit the result of the
 * fp16 x holding the same values.  Products and sums are fp32; the result is
 * deterministic: the same inputs give the same bits on every call and every
 * graph replay.  workspace may be NULL when
 * w4a16_workspace_bytes reports 0; otherwise it must hold that many bytes,
 * with a zero head (see the conventions above), and is owned by the call
 * while it runs.  x and y must not overlap the weights or each other. */
int w4a16_gemv(const void* x, int x_dtype, const void* qweight, const void* scales,
               const void* zeros, void* y, int y_dtype, int M, int N, int K, int group,
               void* workspace, size_t workspace_bytes, w4a16_stream_t stream);

/* y = x . ((q - z) * s) + residual, with the residual added in the output
 * stage of the same call (Ninfer V100 article, section 十四: adding the input
 * back inside the matmul's output stage saves a pass through memory).  Same
 * arguments, contract and workspace as w4a16_gemv, plus residual [M][N]
 * (row-major, 16-byte aligned) of residual_dtype W4A16_F32, W4A16_F16 or
 * W4A16_BF16, read once per element and added to the fp32 result before the
 * output rounding.  residual may be y itself (y += x . W, in place); it must
 * not overlap y otherwise.  A NULL residual returns W4A16_ERR_NULL. */
int w4a16_gemv_add(const void* x, int x_dtype, const void* qweight, const void* scales,
                   const void* zeros, const void* residual, int residual_dtype, void* y, int y_dtype,
                   int M, int N, int K, int group, void* workspace, size_t workspace_bytes,
                   w4a16_stream_t stream);

/* For callers that cannot allocate device memory -- code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc: w4a16_gemv with the
 * same arguments, kernels and results (bit for bit), except that the split-K
 * workspace is a library-owned static device array of
 * W4A16_NOALLOC_SCRATCH_BYTES per GPU instead of a caller buffer.  The call
 * allocates nothing (no hipMalloc, no library allocation).  Each GPU holds its
 * array from its first use until the process ends; its address is looked up
 * once per device, on the first call that needs it with that device current.
 * The array's counter head starts zeroed (static storage) and every call
 * leaves it zeroed; the rest needs no clearing.  All calls on one GPU share
 * that GPU's array, so calls that overlap in time on one GPU (for example on
 * two streams) race and must be serialized by the caller.  Returns W4A16_ERR_WORKSPACE, before any GPU
 * work, when the shape's workspace (w4a16_workspace_bytes) exceeds the array
 * (w4a16_last_error() then says by how much), and the errors of w4a16_gemv
 * otherwise. */
#define W4A16_NOALLOC_SCRATCH_BYTES (16u << 20)
int w4a16_gemv_noalloc(const void* x, int x_dtype, const void* qweight, const void* scales,
                       const void* zeros, void* y, int y_dtype, int M, int N, int K, int group,
                       w4a16_stream_t stream);

/* Debug / parity: the dequantized matrix w[K][N] = (q - z) * s as fp32 from the
 * packed layout -- the integer restored with its group's zero point and
 * multiplied back by the group's scale (Ninfer V100 article, section 十一,
 * groupwise-int; Z100 article, section 四).  Exact, since |q - z| <= 15 times
 * an fp16 scale fits in fp32.  w is a device buffer of K * N floats, 16-byte
 * aligned, written in full; shape and pointer errors as w4a16_pack. */
int w4a16_dequant(const void* qweight, const void* scales, const void* zeros, float* w, int N,
                  int K, int group, w4a16_stream_t stream);

/* ---- 16-bit weights (W16A16) ----
 * The same small-M layer with unquantized FP16/BF16 weights (the Z100
 * article, section 六, measures it next to W4A16): y[M,N] = x[M,K] . w[N,K]^T,
 * w in the layer's own row-major [N][K] layout (no packing), of the same
 * dtype as x (W4A16_F16 or W4A16_BF16).  Shape: 1 <= M <= 64, N % 8 == 0,
 * K % 8 == 0 (N, K >= 8).  x, w, y 16-byte aligned; y_dtype W4A16_F32,
 * W4A16_F16 or W4A16_BF16.  Products and sums in fp32, deterministic.
 * workspace as for w4a16_gemv (NULL when w16a16_workspace_bytes reports 0;
 * scratch owned by the call). */
int w16a16_workspace_bytes(int M, int N, int K, size_t* bytes);
int w16a16_gemv(const void* x, const void* w, int dtype, void* y, int y_dtype, int M, int N, int K,
                void* workspace, size_t workspace_bytes, w4a16_stream_t stream);

/* ---- MXFP4 weights: w = element * 2^(E - 127) ----
 * The Z100 article's closing section names MXFP4 as the next weight format:
 * 4-bit floating-point elements sharing a block-level scale, as the OCP
 * Microscaling (MX) specification it cites defines them (v1.0 MXFP4): E2M1
 * elements (values 0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6), one E8M0 scale
 * code E per 32 consecutive elements along K, scale 2^(E - 127).
 * Canonical layout (host or device memory as each call states):
 *   qweight_canon uint8 [N][K/2]: element k of row n in byte k/2, low nibble
 *                 for even k (bit 3 sign, bits 2..1 exponent, bit 0 mantissa);
 *   scales_canon  uint8 [N][K/32]: the E8M0 code of block k/32 of row n.
 * Shape contract: N >= 8, N % 8 == 0, K >= 32, K % 32 == 0; for the GEMV
 * also 1 <= M <= 64 (a few rows run the GEMV kernel, more rows the M-tiled
 * kernel, with the crossover of w4a16_gemv at g = 128).  Scale codes 0..254; code 255 (the specification's NaN)
 * is outside the contract (its block's results are unspecified).
 * mxfp4_packed_sizes: device bytes of the packed weights and scales.
 * mxfp4_pack / mxfp4_unpack: canonical <-> device layout, exact inverses;
 *   all pointers are device memory, 16-byte aligned (scales_canon any
 *   alignment), caller-owned; enqueued on stream. */
int mxfp4_packed_sizes(int N, int K, size_t* q_bytes, size_t* s_bytes);
int mxfp4_pack(const uint8_t* qweight_canon, const uint8_t* scales_canon, void* qweight,
               void* scales, int N, int K, w4a16_stream_t stream);
int mxfp4_unpack(const void* qweight, const void* scales, uint8_t* qweight_canon,
                 uint8_t* scales_canon, int N, int K, w4a16_stream_t stream);

/* y[M,N] = x[M,K] . w[N,K]^T from the packed device layout.  Every product
 * is exact and every sum fp32, whatever the scale codes: where the four
 * block scales of a 128-k span of a column lie within 2^36 of each other,
 * they are folded into the exact element conversion (relative to the
 * largest) and the span's fp32 sum takes the remaining power of two; wider
 * spans take the MX specification's block dot product literally, each
 * block's fp32 sum times its own 2^(E - 127).  Deterministic.  Dtypes,
 * alignment, workspace and overlap rules as for w4a16_gemv, whose plans it
 * shares (the balanced plan included, as at g = 128); workspace size from
 * mxfp4_workspace_bytes. */
int mxfp4_workspace_bytes(int M, int N, int K, size_t* bytes);
int mxfp4_gemv(const void* x, int x_dtype, const void* qweight, const void* scales, void* y,
               int y_dtype, int M, int N, int K, void* workspace, size_t workspace_bytes,
               w4a16_stream_t stream);

/* Debug / parity: w[N][K] = element * 2^(E - 127) as fp32 from the packed
 * layout, row-major [N][K].  Exact wherever the value is a finite fp32
 * (scale codes up to 253 for elements up to 6). */
int mxfp4_dequant(const void* qweight, const void* scales, float* w, int N, int K,
                  w4a16_stream_t stream);

/* ---- ternary 2-bit variant: w = (c - 1) * s, one fp16 scale per group ----
 * Weights in {-1, 0, +1} times a per-group scale, streamed at two bits each
 * ("NINFER 三元引擎性能调优", sections 五 and 六: the ternary decode path is
 * bound by the bytes it reads plus its decode arithmetic).  Shape contract:
 * 1 <= N, 1 <= K, K % group == 0, K % 16 == 0, group in {32, 64, 128, 256};
 * for the GEMV also 1 <= M <= 16.  A code of 3 is invalid input: the output
 * for such weights is unspecified (no error is reported; the GPU path does
 * not scan for it).
 * w2t_packed_sizes: device bytes of the packed codes and scales (host only).
 * w2t_pack / w2t_unpack: canonical codes_canon [N][K/16] and scales_canon
 *   [K/group][N] <-> the device layout, exact inverses of each other (as for
 *   w4a16_pack / w4a16_unpack: repacked once after loading, Z100 article,
 *   section 四; checkable bit for bit, Ninfer V100 article, section 十三).
 * w2t_workspace_bytes / w2t_gemv: y[M,N] = x[M,K] . ((c - 1) * s)[K,N], with
 *   the dtypes, alignment, determinism, workspace and overlap rules of
 *   w4a16_gemv.
 * w2t_dequant: debug / parity, w[K][N] = (c - 1) * s as fp32, exact. */
int w2t_packed_sizes(int N, int K, int group, size_t* q_bytes, size_t* s_bytes);
int w2t_pack(const int32_t* codes_canon, const uint16_t* scales_canon, void* qweight,
             void* scales, int N, int K, int group, w4a16_stream_t stream);
int w2t_unpack(const void* qweight, const void* scales, int32_t* codes_canon,
               uint16_t* scales_canon, int N, int K, int group, w4a16_stream_t stream);
int w2t_workspace_bytes(int M, int N, int K, int group, size_t* bytes);
int w2t_gemv(const void* x, int x_dtype, const void* qweight, const void* scales, void* y,
             int y_dtype, int M, int N, int K, int group, void* workspace,
             size_t workspace_bytes, w4a16_stream_t stream);
int w2t_dequant(const void* qweight, const void* scales, float* w, int N, int K, int group,
                w4a16_stream_t stream);

/* ---- measurement and diagnostics ---- */

/* Read-only HBM streaming probe: reads `bytes` (a multiple of 16) from buf
 * with 16-byte loads and writes one fp32 per workgroup into sink so the reads
 * cannot be elided; sink must hold w4a16_bw_probe_sink_floats() floats.  The
 * achievable read bandwidth it measures is the ceiling the GEMV is judged
 * against beside the published peak (the pages each measure their own card's
 * ceiling first: Ninfer V100 article, section 十九; Z100 article, section 四). */
int w4a16_bw_probe(const void* buf, size_t bytes, float* sink, w4a16_stream_t stream);
int w4a16_bw_probe_sink_floats(void);

/* Static text for a status code. */
const char* w4a16_status_string(int status);

/* Name of the kernel variant the most recent gemv call on this host thread
 * chose, with the kernel instantiation and launch shape, e.g.
 * "w4_mfma16 f16 g128 kernel=w4_gemv_kernel<false, 4, 5> tiles=320 slices=1 waves=8 upw=5 lds=10880"
 * (every dispatch branch reports itself: NINFER tuning page, section 二).
 * Host string owned by the library, valid until the next call on the thread. */
const char* w4a16_last_variant(void);

/* The same text for the kernel a w4a16_gemv (or w4a16_gemv_add) call of this
 * shape and x dtype would launch, without launching anything: a host-only
 * query of the frozen dispatch (NINFER tuning page, sections 二 and 七: ask
 * which tier runs, and keep that choice fixed).  Writes a NUL-terminated
 * string of at most text_bytes bytes (truncated if longer) into the host
 * buffer text.  Returns W4A16_OK, or W4A16_ERR_NULL / _DTYPE / _SHAPE /
 * _UNSUPPORTED for the arguments w4a16_gemv would refuse. */
int w4a16_plan_variant(int M, int N, int K, int group, int x_dtype, char* text, size_t text_bytes);

/* HIP error name behind the most recent W4A16_ERR_HIP on this host thread
 * ("none" if there was none).  Static host string. */
const char* w4a16_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
