/*
 * convrot.h - C ABI of the ConvRot-quantized linear forward on MI355X (gfx950).
 *
 * The method (model cards cited by title and section):
 *   [QIE] "Qwen-Image-Edit-2511 - INT4 tensorwise W4A4 (+ConvRot, mixed int8
 *         fallback)", intro and "Speed" table: weights stored as packed signed
 *         INT4, two per byte, rotated offline with a group-256 Hadamard
 *         (ConvRot); the activations are rotated and quantised to INT4 at run time
 *         dynamically inside the kernel; integer MMA with a rank-one rescale.
 *   [REB] "Rebels_w4a8s", "What's inside a file" and "Mixed formats where the
 *         kernel demands it": the W4A8 codebook format (int4 codebook indices,
 *         an fp8 scale per group of 16, a scale per output channel, 16
 *         Lloyd-Max levels), int8 GEMM; layers whose input width is not a
 *         multiple of 256 use int8_tensorwise instead.
 *   [Q3N] "qwen3-4b-nvfp4-convrot", file table and converter flags: ConvRot
 *         INT8, int8 weights with a group-256 Hadamard rotation and one scale
 *         per row.
 *
 * Arithmetic (shared by every entry point, float32 unless stated):
 *   rotation   each contiguous 256-block of K is multiplied by the Sylvester
 *              Hadamard matrix scaled by 1/16: butterflies with strides
 *              1,2,...,128 in that order, (a,b)->(a+b,a-b), then x0.0625.
 *   act quant  per row m: s_x[m] = absmax_k / Q (IEEE division),
 *              code = clamp(rint(v / s_x[m])) with round-half-even;
 *              Q = 7, codes [-8,7] (W4A4); Q = 127, codes [-128,127]
 *              (int8_tensorwise: no rotation; W4A8, ConvRot INT8:
 *              rotated).  s = 0 -> 0.
 *   GEMM       acc[m,n] = sum_k qx[m,k] * qw[n,k], exact int32.
 *   epilogue   y[m,n] = bf16_rne(fl(fl(float(acc) * s_x[m]) * s_w) + bias[n])
 *              with s_w the tensor scale (W4A4, int8_tensorwise),
 *              s_channel[n] (W4A8) or the row scale s_w[n] (ConvRot INT8).
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     allocates no memory and never synchronises.  Its only device state is
 *     the static scratch of cr_linear_w4a4_noalloc (one array per GPU); on
 *     the host it caches, per device id, whether the device is a gfx950 and
 *     which kernels have been given their LDS size (set once, idempotent).
 *   - Work is enqueued on `stream` (NULL = the null stream) in order; results
 *     are valid once the stream reaches that point.
 *   - bf16 tensors are row-major uint16 bit patterns; x is [M,K], W is [N,K]
 *     (y = x W^T), y is [M,N], bias is [N] and may be NULL.
 *   - Pointers must be 16-byte aligned.
 *   - Argument errors are detected before any launch and nothing is enqueued;
 *     cr_last_error() (thread-local) then holds a message.  A launch failure
 *     returns CR_ERR_LAUNCH with the HIP error text.  Nothing aborts or prints.
 *   - Calls are re-entrant; two calls that share a workspace or an output must
 *     be ordered by the caller (same stream or events).
 *   - Packed weight layouts are opaque; sizes come from cr_packed_bytes().
 */
#ifndef CONVROT_H
#define CONVROT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CR_OK = 0,
    CR_ERR_NULL = 1,       /* a required pointer is NULL                        */
    CR_ERR_SHAPE = 2,      /* M < 0, N < 1, K < 1, or a size beyond the limits  */
    CR_ERR_GROUP = 3,      /* K is not a multiple of 256 (rotated formats), or an
                              unsupported rotation group size                   */
    CR_ERR_ALIGN = 4,      /* a pointer is not 16-byte aligned                  */
    CR_ERR_WORKSPACE = 5,  /* workspace smaller than cr_workspace_bytes()       */
    CR_ERR_DEVICE = 6,     /* current device is not gfx950 / no device          */
    CR_ERR_LAUNCH = 7,     /* a kernel launch failed                            */
    CR_ERR_KIND = 8        /* unknown format kind                               */
} cr_status;

/* Format kinds. */
#define CR_W4A4 0    /* ConvRot W4A4: INT4 weights (tensorwise), INT4 activations */
#define CR_INT8TW 1  /* int8_tensorwise: int8 weights (tensorwise), int8 activations */
#define CR_W4A8 2    /* asym W4A8 codebook: 4-bit codebook weights, int8 activations */
#define CR_INT8ROT 3 /* ConvRot INT8 row-scaled: rotated int8 weights (one scale per
                        output row), rotated int8 activations */
#define CR_W4A4_G64 4 /* ConvRot W4A4 with rotation groups of 64 (layout as CR_W4A4) */
#define CR_W4A4_G16 5 /* ConvRot W4A4 with rotation groups of 16 (layout as CR_W4A4) */
#define CR_W4A4_RH 6  /* ConvRot W4A4 with the group-256 regular Hadamard (layout as CR_W4A4) */

/* Limits: 1 <= N, K <= CR_MAX_DIM; 0 <= M <= CR_MAX_DIM. */
#define CR_MAX_DIM (1 << 20)
/* Largest K the rotated activation quantiser accepts (W4A4, W4A8, ConvRot INT8). */
#define CR_MAX_ROT_K 65536
/* Largest K of int8_tensorwise: its codes reach +-127 on both operands, so
 * |acc| <= 16129 K, which int32 holds only up to K = 133144 (CR_ERR_SHAPE
 * beyond this limit). */
#define CR_MAX_INT8_K 131072

/* Bytes of the packed weight of `kind` for an [N,K] weight (0 on bad args). */
size_t cr_packed_bytes(int kind, int N, int K);

/* Bytes of workspace cr_linear_* / cr_dbg_linear_acc need for these sizes
 * (0 on bad args; at least 256 otherwise).  The workspace holds the
 * quantised activations, their scales and split-K partial sums (and, for
 * W4A8 from M = 2048 on, the weight decoded to int8 for that call); its
 * contents need no initialisation and are meaningless after the call. */
size_t cr_workspace_bytes(int kind, int M, int N, int K);

/* ---- W4A4 ConvRot ([QIE] intro; "Speed": one kernel for the rotation, the s4 MMA and the rank-one rescale) */

/* Offline weight preparation: rotate each 256-block of every row of W,
 * s_w = absmax(rotated W) / 7, codes = clamp(rint(v / s_w), -8, 7), written
 * in the packed layout: 4 bits per code (N rounded up to 32 rows) plus one
 * int32 per row that the GEMM's exact integer arithmetic needs.
 *   w_bf16   [N,K] bf16                     (in)
 *   w_packed cr_packed_bytes(CR_W4A4,N,K)   (out)
 *   w_scale  1 float                        (out; also used as scratch)
 * K must be a multiple of 256 (CR_ERR_GROUP otherwise). */
cr_status cr_pack_weight_w4(const void* w_bf16, int N, int K, void* w_packed,
                            float* w_scale, hipStream_t stream);

/* y = W4A4 ConvRot linear of x (rotation, per-row INT4 codes, int32 GEMM
 * against the packed weight, rank-one epilogue, optional bias).
 *   x_bf16 [M,K]; w_packed/w_scale from cr_pack_weight_w4 with the same N,K;
 *   bias_bf16 [N] or NULL; y_bf16 [M,N] (out);
 *   ws / ws_bytes: workspace of at least cr_workspace_bytes(CR_W4A4,M,N,K).
 * M = 0 is a no-op.  K % 256 != 0 -> CR_ERR_GROUP (no silent fallback:
 * such layers use cr_linear_int8tw). */
cr_status cr_linear_w4a4(const void* x_bf16, int M, int K, const void* w_packed,
                         const float* w_scale, int N, const void* bias_bf16,
                         void* y_bf16, void* ws, size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): cr_linear_w4a4
 * with no workspace argument.  Its workspace is a static device array of the
 * library, CR_NOALLOC_SCRATCH_BYTES per GPU (held until the process ends);
 * the call allocates nothing.  Same kernels, same results bit for bit.
 * Shapes whose workspace (cr_workspace_bytes(CR_W4A4, M, N, K)) exceeds the
 * scratch return CR_ERR_WORKSPACE before any launch (e.g. M = 4096, K = 3072
 * fits; a layer that splits K across blocks at large M may not).  All calls
 * on one GPU share that GPU's scratch: two calls that can overlap on one GPU
 * (different streams, no ordering between them) race and give undefined
 * results; calls in one stream are safe. */
#define CR_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
cr_status cr_linear_w4a4_noalloc(const void* x_bf16, int M, int K, const void* w_packed,
                                 const float* w_scale, int N, const void* bias_bf16,
                                 void* y_bf16, hipStream_t stream);

/* ---- W4A4 with smaller rotation groups ([ZIT] "Where Z-Image sits": the
 *      ConvRot group-size sweep 256 / 64 / 16) ------------------------------
 * As cr_pack_weight_w4 / cr_linear_w4a4 with the Hadamard rotation applied
 * to groups of `group` = 256, 64 or 16 consecutive k (normalised by
 * 1/sqrt(group)); any other value -> CR_ERR_GROUP.  K must still be a
 * multiple of 256.  The packed layout and sizes are those of CR_W4A4
 * (cr_packed_bytes / cr_workspace_bytes with CR_W4A4_G64 or CR_W4A4_G16 give
 * the same figures); the generic calls (cr_quantize_activations,
 * cr_gemm_quantized, cr_dbg_*) take the kinds CR_W4A4_G64 / CR_W4A4_G16.
 * A weight must be used with the group it was packed with: nothing in the
 * packed bytes records it. */
cr_status cr_pack_weight_w4_group(const void* w_bf16, int N, int K, int group, void* w_packed,
                                  float* w_scale, hipStream_t stream);

cr_status cr_linear_w4a4_group(const void* x_bf16, int M, int K, int group, const void* w_packed,
                               const float* w_scale, int N, const void* bias_bf16, void* y_bf16,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- W4A4 with the regular Hadamard ([QIE] intro: "regular-Hadamard"
 *      rotation; the construction is this library's reading) -------------
 * As cr_pack_weight_w4 / cr_linear_w4a4 with each 256-block rotated by
 * H = (J - 2I)^(x4) / 16 in place of the Sylvester matrix: J - 2I is the 4x4
 * matrix of ones less twice the identity, the power is the Kronecker power,
 * H is symmetric and orthonormal and every row sums to 1.  Applied as four
 * radix-4 stages over the base-4 digits of k (strides 1, 4, 16, 64), each
 * mapping the group x0..x3 to t - 2 x_k with t = (x0 + x1) + (x2 + x3) in
 * float32, then x 1/16.  Same packed layout and sizes as CR_W4A4; the
 * generic calls take the kind CR_W4A4_RH.  A weight must be used with the
 * rotation it was packed with: nothing in the packed bytes records it. */
cr_status cr_pack_weight_w4_regular(const void* w_bf16, int N, int K, void* w_packed,
                                    float* w_scale, hipStream_t stream);

cr_status cr_linear_w4a4_regular(const void* x_bf16, int M, int K, const void* w_packed,
                                 const float* w_scale, int N, const void* bias_bf16,
                                 void* y_bf16, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- int8_tensorwise ([QIE] intro "stock int8_tensorwise"; [REB] "Mixed
 *      formats": no group constraint) -------------------------------------- */

/* s_w = absmax(W) / 127, codes = clamp(rint(w / s_w), -128, 127); any K. */
cr_status cr_pack_weight_int8tw(const void* w_bf16, int N, int K, void* w_packed,
                                float* w_scale, hipStream_t stream);

/* y = int8_tensorwise linear (no rotation; per-row int8 activations). */
cr_status cr_linear_int8tw(const void* x_bf16, int M, int K, const void* w_packed,
                           const float* w_scale, int N, const void* bias_bf16,
                           void* y_bf16, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- ConvRot INT8, row-scaled ([Q3N] file table: INT8 with group-256
 *      Hadamard rotation and row-wise scaling; converter flags) ------------ */

/* Offline weight preparation: rotate each 256-block of every row of W,
 * s_w[n] = absmax(rotated row n) / 127, codes = clamp(rint(v / s_w[n]),
 * -128, 127), written in the int8 packed layout.
 *   w_bf16   [N,K] bf16                        (in)
 *   w_packed cr_packed_bytes(CR_INT8ROT,N,K)   (out)
 *   w_scale  [N] float, one scale per row      (out)
 * K must be a multiple of 256 (CR_ERR_GROUP otherwise). */
cr_status cr_pack_weight_int8rot(const void* w_bf16, int N, int K, void* w_packed,
                                 float* w_scale, hipStream_t stream);

/* y = ConvRot INT8 linear: x rotated online and quantised per row to int8
 * (absmax/127), exact int32 GEMM against the packed weight, epilogue
 * y[m,n] = bf16(fl(fl(acc * s_x[m]) * w_scale[n]) + bias[n]).
 *   w_packed / w_scale from cr_pack_weight_int8rot with the same N, K;
 *   ws / ws_bytes: workspace of at least cr_workspace_bytes(CR_INT8ROT,M,N,K). */
cr_status cr_linear_int8rot(const void* x_bf16, int M, int K, const void* w_packed,
                            const float* w_scale, int N, const void* bias_bf16,
                            void* y_bf16, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- asym W4A8 codebook ([REB] "What's inside a file", "Why W4A8 instead of
 *      GGUF": int8 GEMM at ~0.56 B/param) -------------------------------- */

/* Re-lay the stored W4A8 tensors for the GEMM and build the decode table
 * T[c][i] = clamp(rint(codebook[i] * e4m3(c)), -127, 127) (NaN codes -> 0).
 *   idx        [N,K/2] uint8, codebook index nibbles, low nibble = even k
 *   s_rel_e4m3 [N,K/16] uint8, OCP E4M3FN scale per group of 16 along K
 *   codebook   16 float
 *   w_packed   cr_packed_bytes(CR_W4A8,N,K) (out)
 * K must be a multiple of 256. */
cr_status cr_pack_weight_w4a8(const void* idx, const void* s_rel_e4m3,
                              const float* codebook, int N, int K, void* w_packed,
                              hipStream_t stream);

/* On-GPU encoder of the W4A8 format ([REB] "What's inside a file": 4-bit
 * codebook indices, an fp8 scale per group of 16 along K, a scale per output
 * channel, 16 Lloyd-Max levels fit to the tensor).  Offline conversion of a
 * bf16 weight [N,K] (K % 256 == 0, N*K <= 2^28):
 *   W~ = each 256-block of each row rotated as in cr_pack_weight_w4;
 *   s_channel[n] = absmax_k |W~[n,k]| / 127;
 *   s_rel[n,g] = E4M3 of min(absmax over the 16-group g of |W~| / s_channel[n],
 *                127), nearest with ties to the even code (0 if s_channel = 0);
 *   u = W~ / fl(e4m3(s_rel) * s_channel), 0 where that product is 0;
 *   codebook: 16-level Lloyd-Max fit of all u, levels starting evenly over
 *     [min u, max u] (float64), each iteration moving every non-empty cell's
 *     level to the exact mean of its samples (sums of rint(u * 2^24) as
 *     integers, one float64 division, times 2^-24), cells bounded by the
 *     midpoints of adjacent levels (a sample on one goes to the lower cell),
 *     levels sorted after each iteration; stops when no level moves or after
 *     `iters` (1..1000) iterations; the codebook is the levels rounded to
 *     float32;
 *   idx[n,k] = the cell of u[n,k] by the float64 midpoints of the float32
 *     codebook.
 * Every quantity is one definite value whatever the launch shape (integer
 * sums are exact), so the output is reproducible bit for bit.
 *   w_bf16     [N,K] bf16 (in)
 *   idx        [N,K/2] uint8 (out), low nibble = even k, as cr_pack_weight_w4a8 takes it
 *   s_rel_e4m3 [N,K/16] uint8 (out)
 *   codebook   16 float (out)
 *   s_channel  [N] float (out)
 *   ws/ws_bytes at least cr_encode_w4a8_workspace_bytes(N,K) (~4 N K bytes). */
size_t cr_encode_w4a8_workspace_bytes(int N, int K);
cr_status cr_encode_w4a8(const void* w_bf16, int N, int K, int iters, void* idx, void* s_rel_e4m3,
                         float* codebook, float* s_channel, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/* y = W4A8 linear: rotated per-row int8 activations (absmax/127) times the
 * decoded int8 weight w8[n,k] = T[s_rel[n,k/16]][idx[n,k]], int32 accumulation,
 * epilogue with s_channel[n] (float [N]) in place of s_w. */
cr_status cr_linear_w4a8(const void* x_bf16, int M, int K, const void* w_packed,
                         const float* s_channel, int N, const void* bias_bf16,
                         void* y_bf16, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- two-phase form of the linears ------------------------------------
 * cr_linear_<kind>(x, ...) == cr_quantize_activations(kind, x, ...) followed
 * by cr_gemm_quantized(kind, ...) on the same workspace and stream; results
 * are bit-identical.  One quantisation may feed GEMMs against several
 * weights with the same K (e.g. the gate and up projections of an MLP,
 * which read the same x); the workspace must then hold the largest
 * cr_workspace_bytes() over the N values sharing it (not necessarily that of
 * the largest N: the split-K partials depend on the tile count), and GEMMs
 * sharing it must run in stream order.  The [QIE] card describes the rotation and quantisation of
 * the activations as part of the same fused kernel as the MMA; here they are
 * two kernels on one stream (rotation + quantisation need the whole row for
 * its scale before any code can be used). */

/* Rotation (the W4A4 kinds, W4A8, ConvRot INT8) and per-row quantisation of
 * x [M,K] into `ws`.
 * ws_bytes >= cr_workspace_bytes(kind, M, 1, K). */
cr_status cr_quantize_activations(int kind, const void* x_bf16, int M, int K, void* ws,
                                  size_t ws_bytes, hipStream_t stream);

/* GEMM + rank-one epilogue from a workspace filled by
 * cr_quantize_activations(kind, x, M, K, ...).  w_scale is the tensor scale
 * (the W4A4 kinds, int8_tensorwise), s_channel [N] (W4A8) or the row scales
 * [N] (ConvRot INT8).
 * ws_bytes >= cr_workspace_bytes(kind, M, N, K). */
cr_status cr_gemm_quantized(int kind, int M, int K, const void* w_packed, const float* w_scale,
                            int N, const void* bias_bf16, void* y_bf16, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* ---- text-encoder MLP block ([Q3N] file table and the "qwen3vl_4b" page:
 *      the decoder blocks' gate_proj, up_proj, down_proj Linears, W4A4
 *      ConvRot; the gated-SiLU form is this library's reading) ------------
 * y = down(h), h = silu(g) * u, g = gate(x), u = up(x): three W4A4 linears
 * (packed with cr_pack_weight_w4, group-256 Sylvester rotation, no biases)
 * and, between them, one kernel that forms h and quantises it for the down
 * projection.  g and u are the bf16 outputs cr_linear_w4a4 gives; h =
 * bf16(float(g / (1 + exp(-g)) * u)) with the quotient and products in
 * float64 (both roundings to nearest even).  x is quantised once for the
 * gate and up GEMMs.  At M <= 8 (see cr_dbg_fused_config) the gate GEMM
 * quantises x inside its own launch and the down GEMM forms and quantises
 * h inside its own: three launches instead of five, same results bit for
 * bit.  All launches go on `stream`, none allocates.
 *   x_bf16 [M,K]; wg, wu: [F,K] packed + tensor scale; wd: [N,F] packed +
 *   tensor scale; y_bf16 [M,N] (out); ws / ws_bytes: at least
 *   cr_mlp_workspace_bytes(M,K,F,N) (g and u live there).
 * K and F must be multiples of 256 (CR_ERR_GROUP otherwise). */
size_t cr_mlp_workspace_bytes(int M, int K, int F, int N);

cr_status cr_mlp_w4a4(const void* x_bf16, int M, int K, const void* wg_packed, const float* wg_scale,
                      const void* wu_packed, const float* wu_scale, int F, const void* wd_packed,
                      const float* wd_scale, int N, void* y_bf16, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/* ---- status ----------------------------------------------------------- */
const char* cr_status_str(cr_status s);
const char* cr_last_error(void);   /* thread-local detail of the last failure */

/* ---- inspection hooks (canonical layouts, for bit-exact checks) ---------- */

/* Activation codes and scales exactly as the linear of `kind` computes them.
 *   codes  [M,K] int8 (W4A4 codes in [-8,7], stored one per byte)
 *   scales [M] float */
cr_status cr_dbg_quant_act(int kind, const void* x_bf16, int M, int K,
                           void* codes, float* scales, hipStream_t stream);

/* Weight codes from a packed weight, canonical row-major [N,K] int8
 * (W4A4: [-8,7]; int8_tensorwise, ConvRot INT8: [-128,127]; W4A8: the
 * decoded int8 w8). */
cr_status cr_dbg_unpack_weight(int kind, const void* w_packed, int N, int K,
                               void* codes, hipStream_t stream);

/* The down projection's input codes [M,K] (one per byte, [-8,7]) and scales
 * [M] of the MLP block, formed from bf16 g, u [M,K] by the same kernel as in
 * cr_mlp_w4a4. */
cr_status cr_dbg_quant_swiglu(const void* g_bf16, const void* u_bf16, int M, int K,
                              void* codes, float* scales, hipStream_t stream);

/* h = silu(g) * u of n bf16 pairs (bf16 out), computed as the MLP block's
 * quantiser computes it. */
cr_status cr_dbg_silu_mul(const void* g_bf16, const void* u_bf16, size_t n, void* h_bf16,
                          hipStream_t stream);

/* E4M3FN codes of n non-negative floats (at most 448), nearest with ties to
 * the even code, as the W4A8 encoder rounds its group scales. */
cr_status cr_dbg_e4m3_encode(const float* v, size_t n, void* codes, hipStream_t stream);

/* Path selection of the fused small-M W4A4 linear.  cr_linear_w4a4, its
 * no-allocation variant, cr_dbg_linear_acc(CR_W4A4) and the gate and down
 * GEMMs of cr_mlp_w4a4 can run as ONE launch each where M <= 128,
 * K <= 16384, N % 4 == 0 and the small-M plan fits one round of blocks: the
 * grid's first blocks rotate and quantise the rows of x, or of h for the
 * down GEMM ([QIE] "Speed": rotation, 4-bit MMA and rescale in one kernel),
 * while the other blocks load their weight tiles; a GEMM block waits, with a
 * bounded number of polls, until every row is in.  Results are bit for bit
 * those of the two-launch path (activation quantiser, then GEMM).
 *   mode: 1 = fused where it applies and M <= 8 (the default: the range
 *         where it is measured faster), 2 = fused wherever it applies,
 *         0 = always two launches; any other value -> CR_ERR_SHAPE.
 *   spin_limit: polls of the bounded wait for later launches (default
 *         4194304, seconds of waiting); < 0 keeps the current value.
 * A GEMM block whose wait runs out writes none of its outputs and counts
 * one timeout (cr_dbg_fused_timeouts); the producers never wait and come
 * first in dispatch order, so this takes a stalled device.  At most 1024
 * fused launches may be in flight at once (a graph holds one of those
 * counter slots for its lifetime).  The setting is process-wide and read at
 * each call; for inspection and timing. */
cr_status cr_dbg_fused_config(int mode, int spin_limit);

/* Number of fused-linear GEMM blocks whose wait ran out since the library
 * was loaded on the current device (reads a device counter; synchronises
 * the device).  count: host pointer, out. */
cr_status cr_dbg_fused_timeouts(uint32_t* count);

/* Large-M GEMM plan override (M > 128), for inspection and timing: later
 * calls use block tiles 256 x bn and K split into `splits` equal slices
 * across blocks, in place of the planner's choice.
 *   bn: 256, 192, 128 or 64 (W4A8's own GEMM keeps 256), 0 = the planner's.
 *   splits: 1..16, 0 = the planner's; a count that does not divide the
 *           layer's 64-k chunks leaves the planner's split for that layer.
 * Any other value -> CR_ERR_SHAPE.  The workspace a call needs follows the
 * plan (cr_workspace_bytes reflects the override), so size it after setting
 * one.  Results do not depend on the plan (exact integer sums).  The setting
 * is process-wide and read at each call. */
cr_status cr_dbg_big_plan(int bn, int splits);

/* Small-M GEMM plan override (M <= 128), for inspection and timing: later
 * calls split K into `splits` slices across blocks (1..16) where that count
 * fits the plan (each wave holds its whole share of the loads in registers;
 * a count that does not fit, or 0, leaves the planner's split).  Any other
 * value -> CR_ERR_SHAPE.  The workspace follows the plan (size it after
 * setting one); results do not depend on it.  Process-wide, read at each
 * call. */
cr_status cr_dbg_small_plan(int splits);

/* The int32 accumulators [M,N] of the linear of `kind` (same kernels as the
 * linear, epilogue replaced by a plain int32 store). */
cr_status cr_dbg_linear_acc(int kind, const void* x_bf16, int M, int K,
                            const void* w_packed, int N, int32_t* acc,
                            void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* CONVROT_H */
