/*
 * bitdelta.h -- C ABI of the MI355X (gfx950) BitDelta library, libbitdelta.so.
 *
 * BitDelta stores a fine-tuned weight as a shared base plus a 1-bit delta:
 * W_ft ≈ W_base + α·sign(Δ), Δ = W_ft − W_base, α = mean|Δ|.  This library
 * holds the hot path of serving such variants: the compression pass that turns
 * Δ into (packed signs, α), and the fused linear y = x·(W_base + α·sign(Δ))ᵀ
 * whose reconstructed weight lives only in registers and LDS, never in HBM.
 *
 * Source: the post "BitDelta : servir 14 modèles Zen depuis un seul cluster
 * GPU" (hanzo-blog, 2026-02-28; also published in th, zh-Hant and ja-JP).
 * Sections cited by English gloss: "Mathematical foundation" (delta, sign
 * code, scale factor), "Serving architecture" (shared base, per-variant delta
 * cache, router, the fused reconstruct-and-multiply kernel and its
 * conceptual fused_bitdelta_linear listing), "Infrastructure details" (packed
 * storage format, fp32 α per output dimension).
 *
 * Conventions for every entry point
 * ---------------------------------
 * - All data pointers are DEVICE pointers (HIP device memory of the current
 *   device), except the two pointer ARRAYS of bd_linear_grouped, which are
 *   HOST arrays of device pointers.  bf16 values are passed as their 16-bit
 *   patterns (uint16_t).  Arrays are row-major and contiguous.
 * - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *   Every call only enqueues work on `stream` and returns; nothing
 *   synchronises.  Outputs must not alias inputs.
 * - Ownership: the caller owns every buffer, including workspaces.  The
 *   library allocates no device memory and keeps no per-call state.  Calls
 *   are reentrant; concurrent calls on different streams need different
 *   outputs and workspaces.
 * - Errors: argument errors are detected on the host before anything is
 *   enqueued and returned synchronously as a bd_status; nothing is written
 *   then.  A failed kernel launch returns BD_ERR_HIP; bd_last_hip_error()
 *   gives the hipError_t of the calling thread's last such failure.
 *   Faults inside a kernel surface, as with any HIP work, at the next
 *   synchronising call.
 * - Shapes: d_out >= 1, d_in >= 8 and d_in % 8 == 0 (a whole number of sign
 *   bytes per row), M >= 0.  M == 0 is a successful no-op.
 * - Alignment: x, w_base, delta and y must be 16-byte aligned.  signs, alpha,
 *   variant_ids and workspace need only their natural alignment (1, 4, 4, 8).
 */
#ifndef BITDELTA_H
#define BITDELTA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BD_ABI_VERSION 4
#define BD_MAX_VARIANTS 64

typedef enum bd_status {
    BD_OK = 0,
    BD_ERR_NULL = 1,       /* a required pointer is NULL                       */
    BD_ERR_SHAPE = 2,      /* a size violates the shape rules above            */
    BD_ERR_ALIGN = 3,      /* a pointer violates the alignment rules above     */
    BD_ERR_WORKSPACE = 4,  /* workspace smaller than the *_workspace_bytes query */
    BD_ERR_MODE = 5,       /* unknown bd_alpha_mode                            */
    BD_ERR_HIP = 6,        /* a HIP call failed; see bd_last_hip_error()       */
    BD_ERR_DEVICE = 7      /* the current device is not a gfx950 GPU           */
} bd_status;

/*
 * Granularity of α.  "Mathematical foundation" defines one α per matrix
 * (mean |Δ_ij| over all elements); "Infrastructure details" stores one fp32 α
 * per output dimension; the conceptual listing accepts either ([d_out] or a
 * scalar).  Both are supported.
 */
typedef enum bd_alpha_mode {
    BD_ALPHA_PER_MATRIX = 0,  /* alpha has 1 element                      */
    BD_ALPHA_PER_ROW = 1      /* alpha has d_out elements, α_n = mean_k |Δ_nk| */
} bd_alpha_mode;

int32_t bd_abi_version(void);
const char* bd_status_string(bd_status s);
/* hipError_t (as int) of the calling thread's last BD_ERR_HIP, else 0. */
int32_t bd_last_hip_error(void);

/* ---------------------------------------------------------------------------
 * Compression.  "Mathematical foundation": sign(Δ) keeps one bit per element
 * and α = (1/n)·||Δ||_1; "Infrastructure details": signs packed 8 per byte as
 * an int8 tensor (4096x4096 -> 4096x512), α in fp32.
 *
 *   delta  [d_out, d_in] fp32, device, read only.
 *   signs  [d_out, d_in/8] uint8, device, written: bit b of byte j of row n is
 *          1 iff !(delta[n][8j+b] < 0), i.e. bit 1 encodes +1, bit 0 encodes
 *          -1, and +0, -0 (and NaN) encode +1; least significant bit first
 *          along d_in.
 *   alpha  fp32, device, written: [1] (per matrix) or [d_out] (per row); the
 *          mean of |delta| over the matrix or over the row, summed in fp64 in
 *          a fixed order (run-to-run bitwise reproducible), rounded once to
 *          fp32.
 *   workspace  device scratch of at least bd_compress_workspace_bytes(...)
 *          bytes (8-byte aligned); may be NULL when that query returns 0.
 * Returns BD_OK, or BD_ERR_NULL / _SHAPE / _ALIGN / _MODE / _WORKSPACE /
 * _HIP / _DEVICE.
 * ------------------------------------------------------------------------- */
size_t bd_compress_workspace_bytes(int64_t d_out, int64_t d_in, int32_t mode);
bd_status bd_compress(const float* delta, int64_t d_out, int64_t d_in, int32_t mode,
                      uint8_t* signs, float* alpha, void* workspace, size_t workspace_bytes,
                      void* stream);

/* ---------------------------------------------------------------------------
 * Compression from a (fine-tuned, base) pair.  "Mathematical foundation": the
 * delta is the elementwise difference W_ft − W_base; here it is formed in
 * registers (both bf16 weights widened to fp32, subtracted in fp32 with
 * round to nearest even) and never stored, then coded exactly as by
 * bd_compress: the outputs equal bd_compress's on that fp32 Δ.
 *
 *   w_ft, w_base  [d_out, d_in] bf16, device, read only, 16-byte aligned.
 *   signs, alpha  as for bd_compress (bit 1 iff !(Δ < 0), i.e. iff
 *          W_ft >= W_base; equal weights and ±0 pairs encode +1).
 *   workspace  as for bd_compress: at least bd_compress_workspace_bytes(...)
 *          bytes (8-byte aligned); may be NULL when that query returns 0.
 * Returns BD_OK, or BD_ERR_NULL / _SHAPE / _ALIGN / _MODE / _WORKSPACE /
 * _HIP / _DEVICE.
 * ------------------------------------------------------------------------- */
bd_status bd_compress_pair(const uint16_t* w_ft, const uint16_t* w_base, int64_t d_out,
                           int64_t d_in, int32_t mode, uint8_t* signs, float* alpha, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Fused linear.  "Serving architecture": the effective weight
 * W_eff = W_base + α·sign(Δ) is rebuilt inside the kernel from the bf16 base
 * and the sign bits, in registers or LDS, never materialised in HBM, and
 * multiplied in the same pass; the conceptual listing computes
 * F.linear(x, W_eff) for x [batch, seq, d_in] (flatten leading dims to M).
 *
 *   x       [M, d_in] bf16, device.
 *   w_base  [d_out, d_in] bf16, device.
 *   signs   [d_out, d_in/8] uint8, device, layout as written by bd_compress.
 *   alpha   fp32, device, [1] or [d_out] per `mode`.
 *   y       [M, d_out] fp32, device, written.
 * Each W_eff element is the fp32 sum of the bf16 base weight and +α (bit 1)
 * or -α (bit 0), rounded to bf16 (nearest, ties to even); y accumulates
 * x·W_eff products in fp32.  Deterministic: the same inputs give bitwise the
 * same y.  Dispatch by M and shape, all on the same definition: VALU dot
 * products for one token (or a few on small projections, and two or three on
 * large ones with x held in LDS), an MFMA streaming path that keeps x in LDS
 * for up to 16 tokens, MFMA skinny paths up to 64
 * tokens, and an LDS-tiled MFMA path beyond (prefill).  The tiled path
 * addresses a 256-row tile with 32-bit offsets and so takes d_in <= 2^23 - 8;
 * more than 64 tokens on longer rows run through the skinny path 64 tokens
 * at a time (same result, no workspace).
 *   workspace  device scratch of at least bd_linear_workspace_bytes(...)
 *          bytes, 16-byte aligned; may be NULL when that query returns 0.
 *          Two paths use one.  The tiled path (more than 64 tokens): when
 *          the output tiles do not fill whole rounds of 256 workgroups, the
 *          tiles of the last round are split over d_in and their fp32
 *          partial sums live there until they are added (in a fixed order).
 *          The slice path (3..16 tokens on fewer than 4096 rows of at least
 *          2048 weights, where x is large per row): one fp32 M x d_out plane
 *          per 2048-wide slice of d_in, added in slice order.  Its contents
 *          on entry do not matter.  The size depends on M, d_out and d_in
 *          only, not on the device (it may exceed what the kernel a given
 *          device runs needs).
 * ------------------------------------------------------------------------- */
size_t bd_linear_workspace_bytes(int64_t M, int64_t d_out, int64_t d_in);
/* Diagnostic: the name of the kernel instance bd_linear launches for this
 * shape (as it appears in profiler traces); static storage, never NULL, ""
 * for an invalid shape.  Pure host function, touches no device. */
const char* bd_linear_path(int64_t M, int64_t d_out, int64_t d_in);
bd_status bd_linear(const uint16_t* x, const uint16_t* w_base, const uint8_t* signs,
                    const float* alpha, int32_t mode, float* y, int64_t M, int64_t d_out,
                    int64_t d_in, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Fused linear with a bf16 result.  The conceptual listing of "Serving
 * architecture" ends in F.linear on bf16 operands, whose result is bf16:
 * the same computation as bd_linear, with each fp32 result rounded to bf16
 * (nearest, ties to even; NaN stays NaN) as it is stored.  Arguments,
 * dispatch, workspace rule and errors are bd_linear's; y is
 *   y       [M, d_out] bf16 (uint16_t bit patterns), device, written,
 *           16-byte aligned.
 * The rounding happens once, from the kernel's fp32 accumulator; it can
 * differ from rounding the exact sum only where that fp32 value lies within
 * its own rounding error of a bf16 rounding boundary (one bf16 step).
 * ------------------------------------------------------------------------- */
bd_status bd_linear_bf16(const uint16_t* x, const uint16_t* w_base, const uint8_t* signs,
                         const float* alpha, int32_t mode, uint16_t* y, int64_t M, int64_t d_out,
                         int64_t d_in, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Grouped multi-variant linear.  "Serving architecture" diagram: one
 * HBM-resident base shared by every variant, a delta cache with one
 * (α, sign(Δ)) entry per variant, and a router that picks the entry from the
 * request's model id.  One batch mixes tokens of up to BD_MAX_VARIANTS
 * variants: y[m] = x[m]·W_eff(variant_ids[m])ᵀ.
 *
 *   x            [M, d_in] bf16, device.
 *   variant_ids  [M] int32, device; token m uses variant variant_ids[m].
 *                An id outside [0, num_variants) is a precondition
 *                violation: that token's y row is written as NaN and no
 *                memory outside the arguments is read.
 *   w_base       [d_out, d_in] bf16, device, shared by all variants.
 *   signs        HOST array of num_variants DEVICE pointers, each
 *                [d_out, d_in/8] uint8 (separate allocations, as a delta
 *                cache loads and evicts variants independently).
 *   alpha        HOST array of num_variants DEVICE pointers, each fp32 [1] or
 *                [d_out] per `mode` (one mode for all variants).
 *   num_variants 1 .. BD_MAX_VARIANTS.
 *   y            [M, d_out] fp32, device, in the order of x's rows.
 *   workspace    device scratch of at least
 *                bd_linear_grouped_workspace_bytes(M, d_out, d_in,
 *                num_variants) bytes (8-byte aligned): the token-by-variant
 *                bucketing and, when K is split into ranges, the fp32
 *                partial outputs live there.  That size is 0 for
 *                non-positive sizes or an out-of-range variant count.
 * The host pointer arrays are read during the call only.  Each row of y
 * follows the single-variant definition of bd_linear for that token (fp32
 * accumulation; the summation order may differ from bd_linear's).  The
 * result is deterministic for given inputs.
 * ------------------------------------------------------------------------- */
size_t bd_linear_grouped_workspace_bytes(int64_t M, int64_t d_out, int64_t d_in,
                                         int32_t num_variants);
bd_status bd_linear_grouped(const uint16_t* x, const int32_t* variant_ids,
                            const uint16_t* w_base, const uint8_t* const* signs,
                            const float* const* alpha, int32_t mode, int32_t num_variants,
                            float* y, int64_t M, int64_t d_out, int64_t d_in, void* workspace,
                            size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * bd_linear_grouped_plan / bd_linear_grouped_planned
 *
 * The same grouped linear, with its token-by-variant bucketing done once for
 * all the calls of a batch whose ids do not change between them (one decode
 * step runs every projection of every layer over the same requests; the
 * post's router, "Serving architecture", sends each request to its
 * variant once).
 *
 *   bd_linear_grouped_plan_bytes(M, num_variants): the size of the plan, a
 *     prefix of the grouped workspace that depends on M and num_variants
 *     only (0 for M <= 0 or an out-of-range count).
 *   bd_linear_grouped_plan(variant_ids, M, num_variants, workspace, ...):
 *     buckets the ids into the workspace (enqueued on `stream`).  Errors:
 *     BD_ERR_SHAPE, BD_ERR_NULL, BD_ERR_ALIGN, BD_ERR_WORKSPACE (smaller
 *     than the plan), BD_ERR_DEVICE, BD_ERR_HIP.  M == 0 is a no-op.
 *   bd_linear_grouped_planned(...): the arguments and checks of
 *     bd_linear_grouped; skips the bucketing and uses the plan at the start
 *     of `workspace`, which must come from bd_linear_grouped_plan with the
 *     same variant_ids contents, M and num_variants, enqueued earlier in
 *     stream order (the workspace's size rule is bd_linear_grouped's, for
 *     this call's d_out and d_in; calls only read the plan, so any number
 *     of them may follow one plan).  A plan that does not match gives wrong
 *     rows, never an access outside the arguments.  Calls of up to 4
 *     tokens on 4096 or more rows need no bucketing and do not read the
 *     plan (the same result as bd_linear_grouped).
 * ------------------------------------------------------------------------- */
size_t bd_linear_grouped_plan_bytes(int64_t M, int32_t num_variants);
bd_status bd_linear_grouped_plan(const int32_t* variant_ids, int64_t M, int32_t num_variants,
                                 void* workspace, size_t workspace_bytes, void* stream);
bd_status bd_linear_grouped_planned(const uint16_t* x, const int32_t* variant_ids,
                                    const uint16_t* w_base, const uint8_t* const* signs,
                                    const float* const* alpha, int32_t mode, int32_t num_variants,
                                    float* y, int64_t M, int64_t d_out, int64_t d_in, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * bd_linear_grouped_noalloc
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, hosts that forbid allocation): the grouped
 * linear of bd_linear_grouped, with the same arguments except the
 * workspace, and the same result bit for bit.  Its workspace is a fixed
 * array of BD_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, which
 * the GPU holds from the library's first use on it until the process ends;
 * the call allocates nothing (no hipMalloc, no library allocation).
 *
 *   Size limit: shapes whose bd_linear_grouped_workspace_bytes exceeds
 *     BD_NOALLOC_SCRATCH_BYTES (64 MiB: up to 292 tokens on 28672x8192,
 *     511 on 8192x8192 and 8192x28672, 2047 on 1024x8192) are refused with
 *     BD_ERR_WORKSPACE before anything is enqueued.
 *   Sharing: every call on one GPU uses that GPU's array, whose contents
 *     persist from call to call (nothing in it needs to start at zero).
 *     Calls on one stream are ordered; calls that may overlap on one GPU
 *     (other streams, other threads) race on the array and must not be
 *     issued.
 *   Errors: those of bd_linear_grouped (BD_ERR_WORKSPACE meaning the size
 *     limit above), plus BD_ERR_HIP if the array's device address cannot be
 *     obtained.
 * ------------------------------------------------------------------------- */
#define BD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
bd_status bd_linear_grouped_noalloc(const uint16_t* x, const int32_t* variant_ids,
                                    const uint16_t* w_base, const uint8_t* const* signs,
                                    const float* const* alpha, int32_t mode, int32_t num_variants,
                                    float* y, int64_t M, int64_t d_out, int64_t d_in, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BITDELTA_H */
