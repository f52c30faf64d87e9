// Device helpers shared by the ConvRot kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cr_internal.h"

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

namespace cr {

// ---------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Two float32 -> two bf16 (round to nearest even) packed low/high, with
// gfx950's v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2_t f;
    f.x = lo; f.y = hi;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// float32 -> bf16, round to nearest even; NaN -> quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// h = silu(g) * u of two bf16 values: float64 g / (1 + exp(-g)) * u, rounded
// to float32 and then to bf16 (round to nearest even); returned as float.
__device__ __forceinline__ float silu_mul_bf16(float g, float u) {
    const double gd = (double)g;
    const double h = gd / (1.0 + exp(-gd)) * (double)u;
    return __uint_as_float(f32_to_bf16_rne((float)h) << 16);
}

// ---------------------------------------------------------------------------
// Lane exchange v <- v[lane ^ MASK] inside each 32-lane half of the wave.
//   MASK 1, 2 : DPP quad_perm;  MASK 8 : DPP row_ror:8 (a 16-lane row rotated
//   by 8 is lane ^ 8);  MASK 4, 16 : ds_swizzle in bitmask mode (and 0x1F,
//   xor MASK), which never leaves the 32-lane half.
// ---------------------------------------------------------------------------
template <int MASK>
__device__ __forceinline__ float lane_xor(float v) {
    int x = __float_as_int(v);
    int r;
    if constexpr (MASK == 1) {
        r = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    } else if constexpr (MASK == 2) {
        r = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    } else if constexpr (MASK == 4) {
        r = __builtin_amdgcn_ds_swizzle(x, 0x101F);                     // xor 4
    } else if constexpr (MASK == 8) {
        r = __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false);  // row_ror:8
    } else {
        static_assert(MASK == 16, "lane_xor mask");
        r = __builtin_amdgcn_ds_swizzle(x, 0x401F);                     // xor 16
    }
    return __int_as_float(r);
}

// One butterfly stage across lanes: the pair (i, i+h) lives in lanes that
// differ in bit MASK.  The lane holding i computes a+b, the lane holding i+h
// computes a-b, with a the value at i and b the value at i+h.
template <int MASK>
__device__ __forceinline__ void fwht_cross(float (&v)[8], int lane32) {
    const bool upper = (lane32 & MASK) != 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float p = lane_xor<MASK>(v[i]);
        v[i] = upper ? (p - v[i]) : (v[i] + p);
    }
}

// Rotation selector GS: the Sylvester Hadamard over groups of 256, 64 or 16,
// or kRotRegular (cr_internal.h), the group-256 regular Hadamard.

// The rotation's normalisation, 1 / sqrt(group) (a power of two, so exact
// outside the subnormal range).
template <int GS>
__device__ __forceinline__ constexpr float rot_norm() {
    static_assert(GS == 16 || GS == 64 || GS == 256 || GS == kRotRegular, "rotation selector");
    return (GS == 256 || GS == kRotRegular) ? 0.0625f : (GS == 64 ? 0.125f : 0.25f);
}

// One radix-4 stage of the regular rotation on the group a0..a3 (index
// order): a_k <- t - 2 a_k with t = (a0 + a1) + (a2 + a3).
__device__ __forceinline__ void rh4(float& a0, float& a1, float& a2, float& a3) {
    const float t = (a0 + a1) + (a2 + a3);
    a0 = t - 2.0f * a0;
    a1 = t - 2.0f * a1;
    a2 = t - 2.0f * a2;
    a3 = t - 2.0f * a3;
}

// The same stage when the group's four values sit in the lanes that differ
// in lane bits M1 (the low bit of the group index) and M2: the lane pair sum
// with the M1 partner, then t with the M2 partner's pair sum (each lane
// forms the same t: addition is commutative).
template <int M1, int M2>
__device__ __forceinline__ float rh4_cross(float v) {
    const float p = v + lane_xor<M1>(v);
    const float t = p + lane_xor<M2>(p);
    return t - 2.0f * v;
}

// Rotation of a 256-block held by the 32 lanes of a half-wave, lane j
// holding elements 8j..8j+7 in v[0..7], as 256 / GS independent GS-groups:
// strides 1, 2, 4 inside the lane, then 8, 16, ..., GS / 2 across lanes
// (lane bits 0 .. log2(GS / 8) - 1), then x 1/sqrt(GS).  All 32 lanes of
// the half-wave must be active.
template <int GS>
__device__ __forceinline__ void fwht8(float (&v)[8], int lane32) {
    if constexpr (GS == kRotRegular) {
        // strides 1 (inside the lane), 4 (this lane's pair (r, r + 4) and the
        // lane ^ 1 pair (r + 8, r + 12)), 16 (lane bits 1, 2), 64 (bits 3, 4)
        rh4(v[0], v[1], v[2], v[3]);
        rh4(v[4], v[5], v[6], v[7]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float p = v[r] + v[r + 4];
            const float t = p + lane_xor<1>(p);
            v[r] = t - 2.0f * v[r];
            v[r + 4] = t - 2.0f * v[r + 4];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = rh4_cross<2, 4>(v[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = rh4_cross<8, 16>(v[i]) * 0.0625f;
        return;
    }
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if ((i & h) == 0) {
                const float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
        }
    }
    fwht_cross<1>(v, lane32);
    if constexpr (GS >= 64) {
        fwht_cross<2>(v, lane32);
        fwht_cross<4>(v, lane32);
    }
    if constexpr (GS >= 256) {
        fwht_cross<8>(v, lane32);
        fwht_cross<16>(v, lane32);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = v[i] * rot_norm<GS>();
}

// Rotation of a 256-block held by 16 lanes, lane j holding elements
// 16j..16j+15 in v[0..15], as 256 / GS independent GS-groups: strides 1, 2,
// 4, 8 inside the lane, then 16, ..., GS / 2 across lanes (lane bits 0 ..
// log2(GS / 16) - 1), with no final 1/sqrt(GS) (the caller folds it into
// the scale).
//
// Cross-lane stages keep a per-lane sign: a lane holds sigma * (true value)
// with sigma = (-1)^(number of cross stages in which it was the upper lane).
// Before the stage on lane bit b both partners have the same sigma, so with
// own value w and partner value p every lane computes fma(p, c, w), c = +1 in
// the lower lane (sigma (a + b)) and -1 in the upper lane (sigma (b - a) =
// -sigma (a - b)): one instruction per value and stage, and since rounding
// is symmetric the magnitudes are bitwise those of the plain butterflies
// (a zero may carry the other sign, which no later add can tell apart).
// On return sigma = (-1)^popcount(lane & (GS / 16 - 1)).  All 16 lanes of
// each row must be active.
#define CR_FMAC_DPP16(CTRL)                                                                   \
    asm("s_nop 1\n\t"                                                                           \
        "v_fmac_f32_dpp %0, %0, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                    \
        "v_fmac_f32_dpp %1, %1, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                    \
        "v_fmac_f32_dpp %2, %2, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                    \
        "v_fmac_f32_dpp %3, %3, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                    \
        "v_fmac_f32_dpp %4, %4, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                    \
        "v_fmac_f32_dpp %5, %5, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                    \
        "v_fmac_f32_dpp %6, %6, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                    \
        "v_fmac_f32_dpp %7, %7, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                    \
        "v_fmac_f32_dpp %8, %8, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                    \
        "v_fmac_f32_dpp %9, %9, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                    \
        "v_fmac_f32_dpp %10, %10, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                  \
        "v_fmac_f32_dpp %11, %11, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                  \
        "v_fmac_f32_dpp %12, %12, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                  \
        "v_fmac_f32_dpp %13, %13, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                  \
        "v_fmac_f32_dpp %14, %14, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                  \
        "v_fmac_f32_dpp %15, %15, %16 " CTRL " row_mask:0xf bank_mask:0xf"                      \
        : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]),    \
          "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]),            \
          "+v"(v[13]), "+v"(v[14]), "+v"(v[15])                                                  \
        : "v"(c))

// One cross-lane stage: v[i] = v[i] + c * v[i] of lane ^ MASK.  Masks 1, 2
// and 8 are one v_fmac_f32_dpp per value (quad_perm / row_ror:8, all source
// lanes inside the 16-lane row); the leading s_nop gives the two wait states
// a DPP read needs after a VALU write of its source, and inside the block
// each source was written 16 instructions earlier.  Mask 4 goes through
// ds_swizzle.
template <int MASK>
__device__ __forceinline__ void fwht_cross16(float (&v)[16], int lane) {
    const float c = (lane & MASK) ? -1.0f : 1.0f;
    if constexpr (MASK == 1) {
        CR_FMAC_DPP16("quad_perm:[1,0,3,2]");
    } else if constexpr (MASK == 2) {
        CR_FMAC_DPP16("quad_perm:[2,3,0,1]");
    } else if constexpr (MASK == 8) {
        CR_FMAC_DPP16("row_ror:8");
    } else {
        static_assert(MASK == 4, "fwht_cross16 mask");
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = __builtin_fmaf(lane_xor<4>(v[i]), c, v[i]);
    }
}

template <int GS>
__device__ __forceinline__ void fwht16_signed(float (&v)[16], int lane) {
    if constexpr (GS == kRotRegular) {
        // the regular rotation keeps no sign: strides 1 and 4 inside the
        // lane, 16 across lane bits 0, 1 and 64 across lane bits 2, 3
#pragma unroll
        for (int q = 0; q < 4; ++q) rh4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
#pragma unroll
        for (int r = 0; r < 4; ++r) rh4(v[r], v[r + 4], v[r + 8], v[r + 12]);
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = rh4_cross<1, 2>(v[i]);
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = rh4_cross<4, 8>(v[i]);
        return;
    }
#pragma unroll
    for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if ((i & h) == 0) {
                const float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
        }
    }
    if constexpr (GS >= 64) {
        fwht_cross16<1>(v, lane);
        fwht_cross16<2>(v, lane);
    }
    if constexpr (GS >= 256) {
        fwht_cross16<4>(v, lane);
        fwht_cross16<8>(v, lane);
    }
}

// The sign sigma that fwht16_signed<GS> leaves in a lane.
template <int GS>
__device__ __forceinline__ float fwht16_sign(int lane) {
    if constexpr (GS == kRotRegular) return 1.0f;
    else return (__builtin_popcount(lane & (GS / 16 - 1)) & 1) ? -1.0f : 1.0f;
}

// Symmetric code of v with scale s (IEEE division, round half to even).
template <int LO, int HI>
__device__ __forceinline__ int quant_code(float v, float s) {
    if (s == 0.0f) return 0;
    float r = __builtin_rintf(v / s);
    r = fminf(fmaxf(r, (float)LO), (float)HI);
    return (int)r;
}

// ---------------------------------------------------------------------------
// W4A4 fragment producers (mixed nibble forms, see cr_internal.h).
//
// A packed 64-k chunk of one row is 32 bytes; the 16 bytes at 16*h
// (h = lane / 32) hold, for MFMA step t = 0, 1, the dwords (t, d) at 8t + 4d,
// dword (t, d) covering k0 + 0..7, k0 = 32t + 16h + 8d.  Activations: byte b
// has k0 + b (offset-binary) low and k0 + 4 + b (two's complement) high;
// weights the reverse.  One AND per output dword:
//   P & 0x0F0F0F0F = code + 8 of the low nibbles,
//   P & 0xF0F0F0F0 = 16 * code of the high nibbles,
// and {first four k, next four k, ...} come out in natural k order for both
// operands, each k pairing a low form with a high form.
// ---------------------------------------------------------------------------
__device__ __forceinline__ v4i unpack_act4(uint32_t p0, uint32_t p1) {
    v4i r;
    r.x = (int)(p0 & 0x0F0F0F0Fu);
    r.y = (int)(p0 & 0xF0F0F0F0u);
    r.z = (int)(p1 & 0x0F0F0F0Fu);
    r.w = (int)(p1 & 0xF0F0F0F0u);
    return r;
}

__device__ __forceinline__ v4i unpack_wt4(uint32_t p0, uint32_t p1) {
    v4i r;
    r.x = (int)(p0 & 0xF0F0F0F0u);
    r.y = (int)(p0 & 0x0F0F0F0Fu);
    r.z = (int)(p1 & 0xF0F0F0F0u);
    r.w = (int)(p1 & 0x0F0F0F0Fu);
    return r;
}

// Exact W4A4 dot product from the MFMA sum and the two correction terms
// rn = -128 ra[m], cn = -128 cw[n].
__device__ __forceinline__ int w4_exact(int acc, int rn, int cn) {
    // one three-operand add (the compiler otherwise splits it in two)
    int t;
    asm("v_add3_u32 %0, %1, %2, %3" : "=v"(t) : "v"(acc), "v"(rn), "v"(cn));
    return t >> 4;
}

// Four codebook indices (one per byte, 0..15, in `sel`) looked up in a
// 16-byte table row t0..t3: v_perm picks from the low and the high 8 entries
// with the index's low 3 bits, a third v_perm picks between them by bit 3.
__device__ __forceinline__ uint32_t lut16(uint32_t sel, uint32_t t0, uint32_t t1,
                                          uint32_t t2, uint32_t t3) {
    const uint32_t s7 = sel & 0x07070707u;
    const uint32_t lo = __builtin_amdgcn_perm(t1, t0, s7);
    const uint32_t hi = __builtin_amdgcn_perm(t3, t2, s7);
    const uint32_t pick = ((sel >> 1) & 0x04040404u) | 0x03020100u;
    return __builtin_amdgcn_perm(hi, lo, pick);
}

// W4A8: decode the 16 operands of one step from two packed index dwords
// (byte b of the dword of k0..k0+7: k0 + b low, k0 + 4 + b high) and the
// table row of the group's scale code.
__device__ __forceinline__ v4i decode_w4a8(uint32_t p0, uint32_t p1, uint4 trow) {
    v4i r;
    r.x = (int)lut16(p0 & 0x0F0F0F0Fu, trow.x, trow.y, trow.z, trow.w);
    r.y = (int)lut16((p0 >> 4) & 0x0F0F0F0Fu, trow.x, trow.y, trow.z, trow.w);
    r.z = (int)lut16(p1 & 0x0F0F0F0Fu, trow.x, trow.y, trow.z, trow.w);
    r.w = (int)lut16((p1 >> 4) & 0x0F0F0F0Fu, trow.x, trow.y, trow.z, trow.w);
    return r;
}

// Raw buffer resource over [base, base + bytes) (bytes < 2^31): loads with a
// per-lane VGPR offset and a wave-uniform SGPR offset; a lane whose offset is
// past the end reads 0.
typedef int v2i __attribute__((ext_vector_type(2)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ v16i mfma32(v4i a, v4i b, v16i c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// E4M3FN byte -> float (sign, 4-bit exponent with bias 7, 3-bit mantissa,
// exponent 0 subnormal, S.1111.111 NaN).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
    const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
    float v;
    if (e == 15u && m == 7u) return __int_as_float(0x7FC00000);
    if (e == 0u) v = (float)m * 0.001953125f;                 // m/8 * 2^-6 (exact)
    else v = __uint_as_float(((e + 120u) << 23) | (m << 20));  // 2^(e-7) * (1 + m/8)
    return (c & 0x80u) ? -v : v;
}

// ---------------------------------------------------------------------------
// Rows rotated 256-block by 256-block (each block as 256 / GS rotation
// groups of GS).  One block per row; half-wave h handles 256-blocks h,
// h + NHW, ... (at most GPL of them), each lane 8 consecutive values.
// ---------------------------------------------------------------------------
template <int GPL, int GS = 256>
struct RotRow {
    float v[GPL][8];

    // Loads and rotates the row's groups; returns this lane's absmax.
    __device__ __forceinline__ float load_rotate(const uint16_t* __restrict__ row, int G, int hw,
                                                 int nhw, int lane32) {
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < GPL; ++i) {
            const int g = hw + i * nhw;
            if (g < G) {
                const uint4 raw = *reinterpret_cast<const uint4*>(row + (size_t)g * 256 + lane32 * 8);
                v[i][0] = bf16_lo(raw.x); v[i][1] = bf16_hi(raw.x);
                v[i][2] = bf16_lo(raw.y); v[i][3] = bf16_hi(raw.y);
                v[i][4] = bf16_lo(raw.z); v[i][5] = bf16_hi(raw.z);
                v[i][6] = bf16_lo(raw.w); v[i][7] = bf16_hi(raw.w);
                fwht8<GS>(v[i], lane32);
#pragma unroll
                for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[i][j]));
            }
        }
        return amax;
    }
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Max over the block (blockDim.x <= 1024); every thread gets the result.
__device__ __forceinline__ float block_max(float v, float* red) {
    v = wave_max(v);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    const int nw = (blockDim.x + 63) >> 6;
    float r = 0.0f;
    for (int i = 0; i < nw; ++i) r = fmaxf(r, red[i]);
    __syncthreads();
    return r;
}


// Threads of a one-block-per-row rotation kernel for G 256-blocks per row
// (RotRow): up to 16 half-waves, GPL 256-blocks each (a power of two).
inline int rot_threads(int G, int* gpl) {
    int nhw = G < 16 ? G : 16;
    int per = (G + nhw - 1) / nhw;
    int g = 1;
    while (g < per) g <<= 1;
    *gpl = g;
    return round_up(nhw * 32, 64);      // whole waves (half-waves past G idle)
}

// ---------------------------------------------------------------------------
// Activation quantiser pieces (rows rotated and quantised per row)
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) |
           ((uint32_t)(d & 0xFF) << 24);
}

// Max over the `seg` lanes (16, 32 or 64; aligned) of each lane's segment.
__device__ __forceinline__ float seg_max(float a, int seg) {
    a = fmaxf(a, lane_xor<1>(a));
    a = fmaxf(a, lane_xor<2>(a));
    a = fmaxf(a, lane_xor<4>(a));
    a = fmaxf(a, lane_xor<8>(a));
    if (seg >= 32) a = fmaxf(a, lane_xor<16>(a));
    if (seg >= 64) a = fmaxf(a, __shfl_xor(a, 32, 64));
    return a;
}

// Four codes (int, -128..127) -> one dword, first code in the low byte.
__device__ __forceinline__ uint32_t pack4_codes(int a, int b, int c, int d) {
    const uint32_t ab = __builtin_amdgcn_perm((uint32_t)b, (uint32_t)a, 0x0C0C0400u);
    const uint32_t cd = __builtin_amdgcn_perm((uint32_t)d, (uint32_t)c, 0x0C0C0400u);
    return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// The 16 values of x at x + off (16-byte aligned), as float; with GLU, x is
// the gate output g, u the up output, and the values are silu(g) * u
// rounded to bf16 (silu_mul_bf16).
template <bool GLU>
__device__ __forceinline__ void load16(const uint16_t* __restrict__ x, const uint16_t* __restrict__ u, size_t off,
                                       float (&v)[16]) {
    const uint4* src = reinterpret_cast<const uint4*>(x + off);
    const uint4 r0 = src[0], r1 = src[1];
    const uint32_t w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    if constexpr (GLU) {
        const uint4* su = reinterpret_cast<const uint4*>(u + off);
        const uint4 q0 = su[0], q1 = su[1];
        const uint32_t z[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            v[2 * t] = silu_mul_bf16(bf16_lo(w[t]), bf16_lo(z[t]));
            v[2 * t + 1] = silu_mul_bf16(bf16_hi(w[t]), bf16_hi(z[t]));
        }
    } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            v[2 * t] = bf16_lo(w[t]);
            v[2 * t + 1] = bf16_hi(w[t]);
        }
    }
}

// Codes of a lane's 16 rotated values (unscaled, sign-tracked; the scale
// folding and the exact fast path are explained at k_quant_act_rot).
template <int QMAX, int LO, int HI, int GS>
__device__ __forceinline__ void codes16(const float (&v)[16], bool fast, float rinv, float sigma, float s_u,
                                        float s, float (&r)[16]) {
    if (fast) {
        float dmax = 0.0f;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const float q = v[t] * rinv;
            r[t] = __builtin_rintf(q);
            dmax = fmaxf(dmax, fabsf(q - r[t]));
        }
        if (dmax > 0.5f - (float)QMAX * 9.5367431640625e-07f) {   // within QMAX * 2^-20 of a tie
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const float q = __builtin_rintf((sigma * v[t]) / s_u);
                r[t] = fminf(fmaxf(q, (float)LO), (float)HI);
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < 16; ++t) r[t] = (float)quant_code<LO, HI>((sigma * v[t]) * rot_norm<GS>(), s);
    }
}

// W4A4 codes of 16 consecutive k (k0 % 16 == 0) in the activation nibble
// forms: the two dwords of the 4-bit tile layout, byte b of dword d holding
// k0 + 8d + b (low nibble, code ^ 8) and k0 + 8d + 4 + b (high nibble).
__device__ __forceinline__ uint2 pack_act16(const float (&r)[16]) {
    const uint32_t x0 = pack4_codes((int)r[0], (int)r[1], (int)r[2], (int)r[3]);
    const uint32_t x1 = pack4_codes((int)r[4], (int)r[5], (int)r[6], (int)r[7]);
    const uint32_t x2 = pack4_codes((int)r[8], (int)r[9], (int)r[10], (int)r[11]);
    const uint32_t x3 = pack4_codes((int)r[12], (int)r[13], (int)r[14], (int)r[15]);
    uint2 pk;
    pk.x = ((x0 ^ 0x08080808u) & 0x0F0F0F0Fu) | ((x1 << 4) & 0xF0F0F0F0u);
    pk.y = ((x2 ^ 0x08080808u) & 0x0F0F0F0Fu) | ((x3 << 4) & 0xF0F0F0F0u);
    return pk;
}

// Byte offset of the 8 bytes of row m, k0..k0+15 (k0 % 16 == 0) in the 4-bit
// tile layout with rows = m: dwords (t, d = 0, 1) of half h of chunk k0 / 64.
__device__ __forceinline__ size_t act4_offset(int m, int k0, int K) {
    const int kc = k0 >> 6, t = (k0 >> 5) & 1, h = (k0 >> 4) & 1;
    return ((size_t)(m >> 5) * (K >> 6) + kc) * 1024 + (m & 31) * 32 + 16 * h + 8 * t;
}

}  // namespace cr
