// Internal launch interface of the ConvRot library (host side).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace cr {

// W4A4 rotation selector for the group-256 regular Hadamard (J - 2I)^(x4) / 16,
// J - 2I the 4x4 matrix of ones less twice the identity; the other values
// (256, 64, 16) select the Sylvester Hadamard over groups of that size.
constexpr int kRotRegular = 1;

enum WKind { WK_W4 = 0, WK_I8 = 1, WK_W4A8 = 2, WK_I8R = 3 };

// int8 weights in the int8 tile layout (int8_tensorwise; ConvRot INT8,
// row-scaled) and weights with one scale per output column (W4A8 s_channel;
// ConvRot INT8's row scales).
__host__ __device__ constexpr bool wk_i8w(int wk) { return wk == WK_I8 || wk == WK_I8R; }
__host__ __device__ constexpr bool wk_chan(int wk) { return wk == WK_W4A8 || wk == WK_I8R; }

// Packed-weight geometry.
//   Np = N rounded up to 32 (rows past N are zero), Kp = K rounded up to 64.
//   4-bit tiles (W4 codes, W4A8 indices, W4A4 activations): 1 KiB tiles
//     (32 rows x 64 k), tile (nb, kc) at (nb * Kp/64 + kc) * 1024; row r at
//     r*32; dword d of the 8 bytes at 16h + 8t holds k0 + 0..7,
//     k0 = 64kc + 32t + 16h + 8d, byte b carrying k0 + b and k0 + 4 + b.
//   int8: 2 KiB tiles, row r at r*64, byte 32h + 16t + p holds k = 32t + 16h + p.
//
// W4A4 nibble forms.  CDNA4 has no 4-bit integer MFMA: the codes are
// widened to int8 in registers, one AND per dword, by using two forms of a
// code c in [-8, 7]: in a high nibble as two's complement (the byte masked
// with 0xF0 is the int8 16c), in a low nibble offset-binary (c ^ 8, the byte
// masked with 0x0F is c + 8).  Activations keep k0 + b in the low nibble and
// k0 + 4 + b in the high one, weights the other way round, so every k pairs
// one operand's high form with the other's low form and contributes
// 16 a w + 128 x (x the code in the high form).  Hence
//   sum_k a[m,k] w[n,k] = (acc >> 4) - 8 (ra[m] + cw[n]),
// ra / cw the sums of a row's codes held in high nibbles (activations:
// k % 8 >= 4; weights: k % 8 < 4), int32 vectors next to the codes.
// Bound: |acc| <= 16 * 64 K + 128 * 8 K = 2048 K < 2^31 for K <= 2^20.
//   W4A8 extra: scale codes, 128-byte tiles, row r at r*4, byte 2t + h is the
//     code of group (64kc + 32t + 16h)/16; then the 4 KiB decode table
//     T[c*16 + i] = clamp(rint(codebook[i] * e4m3(c)), -127, 127).
__host__ __device__ inline int round_up(int v, int a) { return (v + a - 1) / a * a; }
__host__ __device__ inline size_t w4_bytes(int N, int K) { return (size_t)round_up(N, 32) * (size_t)K / 2; }
__host__ __device__ inline size_t i8_bytes(int N, int K) { return (size_t)round_up(N, 32) * (size_t)round_up(K, 64); }
// W4A4 packed weight: codes, then cw int32 [Np].
__host__ __device__ inline size_t w4_cw_offset(int N, int K) { return w4_bytes(N, K); }
__host__ __device__ inline size_t w4a4_bytes(int N, int K) { return w4_bytes(N, K) + 4 * (size_t)round_up(N, 32); }
__host__ __device__ inline size_t w4a8_codes_offset(int N, int K) { return w4_bytes(N, K); }
__host__ __device__ inline size_t w4a8_table_offset(int N, int K) {
    return w4_bytes(N, K) + (size_t)round_up(N, 32) * (size_t)K / 16;
}
__host__ __device__ inline size_t w4a8_bytes(int N, int K) { return w4a8_table_offset(N, K) + 4096; }

// Activation quantisation: codes int8 [M, Kp] (row-major, zero for k >= K)
// and scales [M]; with `packed` (W4A4 only) the codes go out 4-bit in the
// 4-bit tile layout with rows = m (round_up(M, 32) rows, rows >= M left
// untouched), in the activation nibble forms, and ra [M] (the sums of the
// codes in high nibbles) beside them.  `group` is the W4A4 rotation: the
// Sylvester Hadamard over groups of 256, 64 or 16, or kRotRegular (1) for the
// group-256 regular Hadamard; the other kinds rotate, if at all, with the
// group-256 Sylvester matrix.
//
// `sync` (nullable): kSyncWords uint32 arrival counters of the split-K GEMMs
// that read this quantisation; the kernel zeroes them (the GEMMs leave them
// zero again), so a workspace needs no initialisation.
constexpr int kSyncWords = 4096;
hipError_t launch_quant_act(int kind, int group, const uint16_t* x, int M, int K, int Kp, int8_t* qx,
                            float* sx, int32_t* ra, bool packed, uint32_t* sync, hipStream_t st);

// W4A4 activations (group-256 Sylvester rotation) of h = silu(g) * u, the
// gated MLP's input to its down projection, from the bf16 gate and up
// outputs g, u [M, K]; outputs as launch_quant_act(WK_W4, 256, ...).
hipError_t launch_quant_swiglu(const uint16_t* g, const uint16_t* u, int M, int K, int8_t* qx, float* sx,
                               int32_t* ra, bool packed, uint32_t* sync, hipStream_t st);

// h = silu(g) * u of n bf16 pairs, as launch_quant_swiglu forms it.
hipError_t launch_silu_mul(const uint16_t* g, const uint16_t* u, size_t n, uint16_t* h, hipStream_t st);

// W4 weight with the rotation `group` (as for launch_quant_act).
hipError_t launch_pack_w4(const uint16_t* w, int N, int K, int group, uint8_t* out, float* scale,
                          hipStream_t st);
hipError_t launch_pack_i8(const uint16_t* w, int N, int K, uint8_t* out, float* scale,
                          hipStream_t st);
// ConvRot INT8 row-scaled: rotated rows, scale[n] = absmax / 127 per row.
hipError_t launch_pack_i8rot(const uint16_t* w, int N, int K, uint8_t* out, float* scale,
                             hipStream_t st);
hipError_t launch_pack_w4a8(const uint8_t* idx, const uint8_t* s_rel, const float* cb, int N,
                            int K, uint8_t* out, hipStream_t st);
// A packed W4A8 weight decoded into the int8 tile layout (i8_bytes(N, K)
// bytes at `out`; K % 256 == 0), for the int8 GEMM with per-column scales.
hipError_t launch_w4a8_expand(const uint8_t* packed, int N, int K, uint8_t* out, hipStream_t st);
hipError_t launch_unpack_weight(int kind, const uint8_t* packed, int N, int K, int8_t* out,
                                hipStream_t st);

// W4A8 encoder (cr_encode.hip): bf16 weight [N, K] (K % 256 == 0) to the
// stored W4A8 tensors (idx [N, K/2], s_rel [N, K/16], codebook [16],
// s_channel [N]), at most `iters` Lloyd-Max iterations; workspace of
// encode_w4a8_workspace(N, K) bytes.
size_t encode_w4a8_workspace(int N, int K);
hipError_t launch_encode_w4a8(const uint16_t* w, int N, int K, int iters, uint8_t* idx, uint8_t* s_rel,
                              float* codebook, float* s_channel, void* ws, hipStream_t st);
// E4M3FN codes (nearest, ties to the even code) of n non-negative floats <= 448.
hipError_t launch_e4m3_encode(const float* v, size_t n, uint8_t* out, hipStream_t st);

struct GemmArgs {
    int kind;              // WKind
    const int8_t* qx;      // [M, Kp]
    const float* sx;       // [M]
    int M, N, K, Kp, Np;
    const uint8_t* wp;     // packed weight
    const float* wscale;   // tensor scale (1 float) or s_channel [N] (W4A8)
    const uint16_t* bias;  // [N] or null
    uint16_t* y;           // [M, N] bf16 (null when acc_out is set)
    int32_t* acc_out;      // [M, N] int32 accumulators instead of y
    int32_t* part;         // split-K partial sums (workspace)
    uint32_t* sync;        // split-K arrival counters (kSyncWords, zero on entry and on exit; workspace)
    const int32_t* ra;     // W4A4: activation high-nibble code sums [M]
    const int32_t* cw;     // W4A4: weight high-nibble code sums [Np]
    // fused small-M W4A4 linear: the bf16 activations, quantised by the
    // GEMM launch's own producer blocks into qx / sx / ra
    const uint16_t* x;
    const uint16_t* xu;    // MLP down projection: x is g, xu is u, the row is silu(g) * u (else NULL)
    int fused_producers;   // producer blocks (the first in the grid)
    int fused_slot;        // its slot of the library's arrival counters
    int spin_limit;        // polls of the bounded wait for the producers
};

// Large-M path plan: block tiles 256 x bn (bn = 256, or 192, 128 or 64 where
// that fills more of the chip), K split into `splits` equal slices of `cps` 64-k chunks
// when the output has too few tiles to fill the chip; the slices' int32
// partial tiles ([splits][tiles][256 x bn] in fragment order) are added by a
// second kernel.
struct BigPlan {
    int splits;
    int cps;
    size_t part_bytes;
    int bn;
};
BigPlan plan_big(int kind, int M, int N, int K);
// Overrides the large-M plan's tile width (256, 192 or 128) and K slices (a
// divisor of the 64-k chunks, at most 16) for later calls; 0 keeps the
// planner's choice (inspection and timing).
void set_big_plan_override(int bn, int splits);

// Small-M path, used for M <= kSmallMaxM: 16-row MFMA tiles, blocks of 8
// waves over 16 * nt weight rows that split their K range between the
// waves and add the waves' sums in LDS; when K is also split across blocks
// (`splits` > 1) a second kernel adds the int32 partial tiles and runs the
// epilogue.  W4A4 activations are stored packed (4-bit) for this path.
constexpr int kSmallMaxM = 128;
struct SmallPlan {
    bool use;
    int mt;        // 16-row activation tiles (1..8)
    int nt;        // 16-row weight tiles per block
    int nblk;      // weight blocks
    int splits;    // K slices across blocks
    int cps;       // 64-k chunks per slice
    int cpw;       // steps per wave (at most; a step is two 64-k chunks for W4A4, one otherwise)
    size_t part_bytes;   // int32 partial tiles, [splits][N/16][mt][64 lanes] x int4
    size_t lds;          // dynamic LDS bytes of the GEMM kernel
};
SmallPlan plan_small(int kind, int M, int N, int K);
// Overrides the small-M plan's K slices across blocks (1..16) for later calls
// where that count fits the plan's register budget; 0 keeps the planner's
// choice (inspection and timing).
void set_small_plan_override(int splits);
hipError_t launch_small(const GemmArgs& a, const SmallPlan& sp, hipStream_t st);

// Fused small-M W4A4 linear (group-256 Sylvester rotation): one launch whose
// first blocks rotate and quantise the rows of a.x (or silu(a.x) * a.xu) into
// a.qx / a.sx / a.ra (and clear a.sync) while the GEMM blocks load their
// weights; a GEMM block waits (bounded by the spin limit's polls) for every
// row before it reads them.  Taken where fused_small_ok() holds; the outputs
// and accumulators are those of the two-kernel linear.
bool fused_small_ok(int kind, int M, int N, int K);
hipError_t launch_small_fused(GemmArgs a, hipStream_t st);
// Polls of the fused linear's bounded wait (default 1 << 22, ~seconds);
// set_fused_spin_limit changes it for later launches (inspection/testing).
void set_fused_spin_limit(int polls);
// GEMM blocks of the fused linear whose wait ran out (device counter; reading it
// synchronises the device).
hipError_t fused_timeouts(uint32_t* count);

// Whether the activations of a linear are stored packed 4-bit (W4A4)
// rather than as int8 [M, Kp].
inline bool act_packed(int kind) { return kind == WK_W4; }
// Bytes of the activation codes in the workspace.
inline size_t act_bytes(int kind, int M, int K) {
    if (act_packed(kind)) return (size_t)round_up(M, 32) * (size_t)K / 2;
    return (size_t)M * (size_t)(wk_i8w(kind) ? round_up(K, 64) : K);
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st);

// Opts `kernel` in to `bytes` of dynamic LDS (beyond the default 64 KiB) on
// the current device, once per device: `done` holds one bit per device id
// (ids past 63 set the attribute on every call).
inline hipError_t opt_in_lds(const void* kernel, int bytes, std::atomic<uint64_t>& done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t)1 << dev : 0;
    if (bit != 0 && (done.load(std::memory_order_relaxed) & bit) != 0) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_relaxed);
    return e;
}

}  // namespace cr
