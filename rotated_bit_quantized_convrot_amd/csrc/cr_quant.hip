// Activation quantisation and offline weight packing kernels.
//
// Rotation + per-row dynamic quantisation of activations, tensorwise weight
// quantisation and packing ([QIE] model card intro: group-256 Hadamard
// ConvRot; the activations are rotated and quantised to INT4 at run time inside the kernel,
// weights packed signed INT4 two per byte; [REB] "What's inside a file" for
// the W4A8 tensors).
#include "cr_device.h"
#include "cr_internal.h"

namespace cr {

// The split-K arrival counters of the GEMMs that read this quantisation
// start at zero: the first block clears them (the GEMM kernels run after this
// kernel on the same stream).
__device__ __forceinline__ void zero_sync(uint32_t* __restrict__ sync) {
    if (sync != nullptr && blockIdx.x == 0)
        for (int i = threadIdx.x; i < kSyncWords; i += blockDim.x) sync[i] = 0u;
}

// Rotated activations: codes [M, K] int8 (natural order) and scales [M].
//
// Each row is handled by a segment of lanes: 16 lanes per 256-group, each
// lane 16 consecutive values.  seg_log2 >= 0: segments of 2^seg_log2 <= 64
// lanes, 256 / 2^seg_log2 rows per block; seg_log2 < 0: one row per block
// (GPL groups per lane, strided by the block's group count).
//
// Rotation GS: Sylvester groups of 256, 64 or 16 (a 256-block is 256 / GS
// groups), or the group-256 regular Hadamard (GS = kRotRegular).  The
// butterflies run on the unscaled values (sign-tracked, see fwht16_signed);
// the normalisation 2^-e of the rotation is folded into the
// scale.  With amax_u the row's max |value| before the 2^-e, the stored
// scale is s = fl(fl(amax_u 2^-e) / QMAX), and for 2^-100 <= amax_u <= 2^100
// the code fl(v 2^-e / s) equals fl(v / s_u), s_u = fl(amax_u / QMAX):
// scaling by a power of two commutes with rounding away from the subnormal
// range, and values too small for that have code 0 either way.  That quotient is taken as v * fl(1/s_u):
// the product is within QMAX * 2^-22.9 of v / s_u and the correctly rounded
// quotient within half an ulp (< QMAX * 2^-23), so both round to the same
// integer unless v / s_u lies within QMAX * 2^-20 of a half-integer; a lane
// whose 16 products come that close redoes them with the division.  |v/s_u|
// <= QMAX (1 + 2^-23) keeps the fast codes inside [LO, HI].  Rows outside
// the range take the literal path.
//
// PACKED (W4A4): codes in the 4-bit tile layout, activation nibble forms,
// and ra[m] = the sum of the row's codes held in high nibbles (k % 8 >= 4).
// GLU: the row is silu(g) * u of the gate and up outputs x = g and u.
template <int GPL, int QMAX, int LO, int HI, bool PACKED, int GS, bool GLU>
__global__ void __launch_bounds__(1024) k_quant_act_rot(const uint16_t* __restrict__ x, const uint16_t* __restrict__ u,
                                                        int M, int K, int seg_log2, int8_t* __restrict__ qx,
                                                        float* __restrict__ sx, int32_t* __restrict__ ra,
                                                        uint32_t* __restrict__ sync) {
    __shared__ float red[16];
    __shared__ int ired[16];
    zero_sync(sync);
    const int tid = threadIdx.x;
    int m, l, seg;
    if (seg_log2 >= 0) {
        seg = 1 << seg_log2;
        m = blockIdx.x * (blockDim.x >> seg_log2) + (tid >> seg_log2);
        l = tid & (seg - 1);
    } else {
        seg = blockDim.x;
        m = blockIdx.x;
        l = tid;
    }
    const int G = K >> 8, gslot = l >> 4, gstride = seg >> 4, j = l & 15;
    const bool row_ok = m < M;

    float v[GPL][16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
        const int g = gslot + i * gstride;
        if (row_ok && g < G) {
            load16<GLU>(x, u, (size_t)m * K + (size_t)g * 256 + j * 16, v[i]);
            fwht16_signed<GS>(v[i], l);
#pragma unroll
            for (int t = 0; t < 16; ++t) amax = fmaxf(amax, fabsf(v[i][t]));
        }
    }
    amax = seg_max(amax, seg < 64 ? seg : 64);
    if (seg > 64) {                      // one row per block: across waves
        const int wave = tid >> 6, nw = blockDim.x >> 6;
        if ((tid & 63) == 0) red[wave] = amax;
        __syncthreads();
        amax = 0.0f;
        for (int i = 0; i < nw; ++i) amax = fmaxf(amax, red[i]);
    }
    if (!row_ok) return;

    const float s = (amax * rot_norm<GS>()) / (float)QMAX;
    if (l == 0) sx[m] = s;
    const float sigma = fwht16_sign<GS>(l);
    const bool fast = amax >= 0x1p-100f && amax <= 0x1p100f;
    const float s_u = amax / (float)QMAX;
    const float rinv = sigma * (1.0f / s_u);          // undoes the lane's sign too

    int hsum = 0;                                      // PACKED: codes going to high nibbles
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
        const int g = gslot + i * gstride;
        if (g < G) {
            float r[16];
            codes16<QMAX, LO, HI, GS>(v[i], fast, rinv, sigma, s_u, s, r);
            if constexpr (PACKED) {
                const size_t off = act4_offset(m, g * 256 + j * 16, K);
                hsum += (int)(r[4] + r[5] + r[6] + r[7] + r[12] + r[13] + r[14] + r[15]);
                *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(qx) + off) = pack_act16(r);
            } else {
                uint4 o;
                o.x = pack4_codes((int)r[0], (int)r[1], (int)r[2], (int)r[3]);
                o.y = pack4_codes((int)r[4], (int)r[5], (int)r[6], (int)r[7]);
                o.z = pack4_codes((int)r[8], (int)r[9], (int)r[10], (int)r[11]);
                o.w = pack4_codes((int)r[12], (int)r[13], (int)r[14], (int)r[15]);
                *reinterpret_cast<uint4*>(qx + (size_t)m * K + (size_t)g * 256 + j * 16) = o;
            }
        }
    }
    if constexpr (PACKED) {
        // row sum over the segment (and, one row per block, over its waves)
        const int sg = seg < 64 ? seg : 64;
        for (int o = 1; o < sg; o <<= 1) hsum += __shfl_xor(hsum, o, 64);
        if (seg > 64) {
            const int wave = tid >> 6, nw = blockDim.x >> 6;
            if ((tid & 63) == 0) ired[wave] = hsum;
            __syncthreads();
            hsum = 0;
            for (int i = 0; i < nw; ++i) hsum += ired[i];
        }
        if (l == 0) ra[m] = hsum;
    }
}

// Rotated activations, four rows per block: lanes 16r..16r+15 of every wave
// work on row 4 blockIdx.x + r, wave w on groups w, w + nw, ... (GPL at
// most).  PACKED (W4A4): each store instruction writes, for every 64-k chunk
// it touches, the four rows' 32-byte pieces: one whole 128-byte line of the
// 4-bit tile.  Otherwise (the int8 codes of W4A8 and ConvRot INT8, QMAX 127)
// rows of [M, K] int8, 16 bytes per lane.  Same arithmetic as
// k_quant_act_rot.
template <int GPL, int GS, bool GLU, int QMAX = 7, int LO = -8, int HI = 7, bool PACKED = true>
__global__ void __launch_bounds__(1024) k_quant_rows4(const uint16_t* __restrict__ x, const uint16_t* __restrict__ u,
                                                         int M, int K, int8_t* __restrict__ qx, float* __restrict__ sx,
                                                         int32_t* __restrict__ ra, uint32_t* __restrict__ sync) {
    __shared__ float redm[16][4];
    __shared__ int reds[16][4];
    zero_sync(sync);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = tid >> 6, nw = blockDim.x >> 6;
    const int r = lane >> 4, j = lane & 15;
    const int m = blockIdx.x * 4 + r;
    const int G = K >> 8;
    const bool row_ok = m < M;

    float v[GPL][16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
        const int g = wave + i * nw;
        if (row_ok && g < G) {
            load16<GLU>(x, u, (size_t)m * K + (size_t)g * 256 + j * 16, v[i]);
            fwht16_signed<GS>(v[i], j);
#pragma unroll
            for (int t = 0; t < 16; ++t) amax = fmaxf(amax, fabsf(v[i][t]));
        }
    }
    amax = seg_max(amax, 16);
    if (j == 0) redm[wave][r] = amax;
    __syncthreads();
    amax = 0.0f;
    for (int w = 0; w < nw; ++w) amax = fmaxf(amax, redm[w][r]);

    const float s = (amax * rot_norm<GS>()) / (float)QMAX;
    const float sigma = fwht16_sign<GS>(j);
    const bool fast = amax >= 0x1p-100f && amax <= 0x1p100f;
    const float s_u = amax / (float)QMAX;
    const float rinv = sigma * (1.0f / s_u);
    int hsum = 0;
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
        const int g = wave + i * nw;
        if (row_ok && g < G) {
            float c[16];
            codes16<QMAX, LO, HI, GS>(v[i], fast, rinv, sigma, s_u, s, c);
            if constexpr (PACKED) {
                hsum += (int)(c[4] + c[5] + c[6] + c[7] + c[12] + c[13] + c[14] + c[15]);
                *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(qx) + act4_offset(m, g * 256 + j * 16, K)) =
                    pack_act16(c);
            } else {
                uint4 o;
                o.x = pack4_codes((int)c[0], (int)c[1], (int)c[2], (int)c[3]);
                o.y = pack4_codes((int)c[4], (int)c[5], (int)c[6], (int)c[7]);
                o.z = pack4_codes((int)c[8], (int)c[9], (int)c[10], (int)c[11]);
                o.w = pack4_codes((int)c[12], (int)c[13], (int)c[14], (int)c[15]);
                *reinterpret_cast<uint4*>(qx + (size_t)m * K + (size_t)g * 256 + j * 16) = o;
            }
        }
    }
    if constexpr (PACKED) {
        for (int o = 1; o < 16; o <<= 1) hsum += __shfl_xor(hsum, o, 64);
        if (j == 0) reds[wave][r] = hsum;
        __syncthreads();
    }
    if (wave == 0 && j == 0 && row_ok) {
        if constexpr (PACKED) {
            int t = 0;
            for (int w = 0; w < nw; ++w) t += reds[w][r];
            ra[m] = t;
        }
        sx[m] = s;
    }
}

// Unrotated activations (int8_tensorwise): any K; codes [M, Kp] with zeros
// in [K, Kp).  Two passes over the row (the second one hits the cache).
__global__ void __launch_bounds__(256) k_quant_act_plain(const uint16_t* __restrict__ x, int M,
                                                         int K, int Kp, int8_t* __restrict__ qx,
                                                         float* __restrict__ sx, uint32_t* __restrict__ sync) {
    __shared__ float red[16];
    zero_sync(sync);
    const int m = blockIdx.x;
    const uint16_t* row = x + (size_t)m * K;
    int8_t* out = qx + (size_t)m * Kp;
    const bool vec = (K % 8) == 0;
    float amax = 0.0f;
    if (vec) {
        for (int k = threadIdx.x * 8; k < K; k += blockDim.x * 8) {
            const uint4 raw = *reinterpret_cast<const uint4*>(row + k);
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(bf16_lo(raw.x)), fabsf(bf16_hi(raw.x))),
                                     fmaxf(fabsf(bf16_lo(raw.y)), fabsf(bf16_hi(raw.y)))));
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(bf16_lo(raw.z)), fabsf(bf16_hi(raw.z))),
                                     fmaxf(fabsf(bf16_lo(raw.w)), fabsf(bf16_hi(raw.w)))));
        }
    } else {
        for (int k = threadIdx.x; k < K; k += blockDim.x) amax = fmaxf(amax, fabsf(bf16_to_f32(row[k])));
    }
    amax = block_max(amax, red);
    const float s = amax / 127.0f;
    if (threadIdx.x == 0) sx[m] = s;
    if (vec) {
        for (int k = threadIdx.x * 8; k < K; k += blockDim.x * 8) {
            const uint4 raw = *reinterpret_cast<const uint4*>(row + k);
            uint2 o;
            o.x = pack4_i8(quant_code<-128, 127>(bf16_lo(raw.x), s), quant_code<-128, 127>(bf16_hi(raw.x), s),
                           quant_code<-128, 127>(bf16_lo(raw.y), s), quant_code<-128, 127>(bf16_hi(raw.y), s));
            o.y = pack4_i8(quant_code<-128, 127>(bf16_lo(raw.z), s), quant_code<-128, 127>(bf16_hi(raw.z), s),
                           quant_code<-128, 127>(bf16_lo(raw.w), s), quant_code<-128, 127>(bf16_hi(raw.w), s));
            *reinterpret_cast<uint2*>(out + k) = o;
        }
    } else {
        for (int k = threadIdx.x; k < K; k += blockDim.x)
            out[k] = (int8_t)quant_code<-128, 127>(bf16_to_f32(row[k]), s);
    }
    for (int k = K + threadIdx.x; k < Kp; k += blockDim.x) out[k] = 0;
}


// The same for K % 8 == 0 and K <= 8 * CH * blockDim.x, in one pass: each
// thread keeps its CH 8-value chunks (chunk tid + j * blockDim.x) in
// registers between the row maximum and the codes instead of reading the row
// again.  Same arithmetic and outputs as k_quant_act_plain.
template <int CH>
__global__ void __launch_bounds__(256) k_quant_act_plain_reg(const uint16_t* __restrict__ x, int M, int K, int Kp,
                                                             int8_t* __restrict__ qx, float* __restrict__ sx,
                                                             uint32_t* __restrict__ sync) {
    __shared__ float red[16];
    zero_sync(sync);
    const int m = blockIdx.x;
    const uint16_t* row = x + (size_t)m * K;
    int8_t* out = qx + (size_t)m * Kp;
    const int nch = K >> 3;
    uint4 raw[CH];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int c = threadIdx.x + j * blockDim.x;
        raw[j] = c < nch ? reinterpret_cast<const uint4*>(row)[c] : make_uint4(0u, 0u, 0u, 0u);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(bf16_lo(raw[j].x)), fabsf(bf16_hi(raw[j].x))),
                                 fmaxf(fabsf(bf16_lo(raw[j].y)), fabsf(bf16_hi(raw[j].y)))));
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(bf16_lo(raw[j].z)), fabsf(bf16_hi(raw[j].z))),
                                 fmaxf(fabsf(bf16_lo(raw[j].w)), fabsf(bf16_hi(raw[j].w)))));
    }
    amax = block_max(amax, red);
    const float s = amax / 127.0f;
    if (threadIdx.x == 0) sx[m] = s;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int c = threadIdx.x + j * blockDim.x;
        if (c < nch) {
            uint2 o;
            o.x = pack4_i8(quant_code<-128, 127>(bf16_lo(raw[j].x), s), quant_code<-128, 127>(bf16_hi(raw[j].x), s),
                           quant_code<-128, 127>(bf16_lo(raw[j].y), s), quant_code<-128, 127>(bf16_hi(raw[j].y), s));
            o.y = pack4_i8(quant_code<-128, 127>(bf16_lo(raw[j].z), s), quant_code<-128, 127>(bf16_hi(raw[j].z), s),
                           quant_code<-128, 127>(bf16_lo(raw[j].w), s), quant_code<-128, 127>(bf16_hi(raw[j].w), s));
            *reinterpret_cast<uint2*>(out + (size_t)c * 8) = o;
        }
    }
    for (int k = K + threadIdx.x; k < Kp; k += blockDim.x) out[k] = 0;
}

template <int QMAX, int LO, int HI, bool PACKED, int GS = 256, bool GLU = false>
static hipError_t launch_rot(const uint16_t* x, const uint16_t* u, int M, int K, int8_t* qx, float* sx, int32_t* ra,
                             uint32_t* sync, hipStream_t st) {
    const int T = K / 16;              // lanes per row
    if (T <= 64) {
        int lg = 4;
        while ((1 << lg) < T) ++lg;
        const int rows = 256 >> lg;
        k_quant_act_rot<1, QMAX, LO, HI, PACKED, GS, GLU><<<dim3((M + rows - 1) / rows), dim3(256), 0, st>>>(x, u, M, K, lg, qx, sx, ra, sync);
        return hipGetLastError();
    }
    const int G = K >> 8;
    if constexpr (!PACKED) {
        // four rows per block where there are rows enough to fill the chip
        // (the rule of the packed W4A4 activations)
        if (M >= 2048 && G <= 32) {
            int g4 = 1;
            while ((G + g4 - 1) / g4 > 16) g4 <<= 1;
            if (g4 == 1 && G >= 8) g4 = 2;
            const int nw = (G + g4 - 1) / g4;
            const dim3 grid((unsigned)((M + 3) / 4)), block((unsigned)(64 * nw));
            switch (g4) {
                case 1: k_quant_rows4<1, GS, GLU, QMAX, LO, HI, false><<<grid, block, 0, st>>>(x, u, M, K, qx, sx, nullptr, sync); break;
                case 2: k_quant_rows4<2, GS, GLU, QMAX, LO, HI, false><<<grid, block, 0, st>>>(x, u, M, K, qx, sx, nullptr, sync); break;
                default: return hipErrorInvalidValue;
            }
            return hipGetLastError();
        }
    }
    int gpl = 1;
    while ((T + gpl - 1) / gpl > 1024) gpl <<= 1;
    // more groups per lane (fewer waves) while the grid would exceed what the
    // chip holds at once (~8192 waves) and a row keeps at least one whole wave
    // (text-encoder down layer at M=1220: 14.5 -> 11.9 us)
    while (gpl < 4 && (long)M * (round_up((T + gpl - 1) / gpl, 64) / 64) > 8192 && (T + 2 * gpl - 1) / (2 * gpl) >= 64)
        gpl <<= 1;
    const int threads = round_up((T + gpl - 1) / gpl, 64);
    dim3 grid(M), block(threads);
    switch (gpl) {
        case 1: k_quant_act_rot<1, QMAX, LO, HI, PACKED, GS, GLU><<<grid, block, 0, st>>>(x, u, M, K, -1, qx, sx, ra, sync); break;
        case 2: k_quant_act_rot<2, QMAX, LO, HI, PACKED, GS, GLU><<<grid, block, 0, st>>>(x, u, M, K, -1, qx, sx, ra, sync); break;
        case 4: k_quant_act_rot<4, QMAX, LO, HI, PACKED, GS, GLU><<<grid, block, 0, st>>>(x, u, M, K, -1, qx, sx, ra, sync); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// W4A4 activations with rotation GS (GLU: of silu(x) * u).
template <int GS, bool GLU = false>
static hipError_t launch_w4_act(const uint16_t* x, const uint16_t* u, int M, int K, int8_t* qx, float* sx,
                                int32_t* ra, bool packed, uint32_t* sync, hipStream_t st) {
    const int G = K >> 8;
    // four rows per block where there are rows enough to fill the chip
    // with such blocks (at smaller M one row per block keeps more lanes busy;
    // past 32 groups a row's own block has more loads in flight: DiT W2,
    // K = 12288, 36.1 -> 31.8 us)
    if (packed && G <= 32 && M >= 2048) {
        int gpl = 1;
        while ((G + gpl - 1) / gpl > 16) gpl <<= 1;
        // two 256-blocks per lane from K = 2048 up: half as many waves, so
        // the whole grid is resident at once instead of a thin last round
        // (DiT W1: 11.1 -> 9.7 us)
        if (gpl == 1 && G >= 8) gpl = 2;
        const int nw = (G + gpl - 1) / gpl;
        const dim3 grid((unsigned)((M + 3) / 4)), block((unsigned)(64 * nw));
        switch (gpl) {
            case 1: k_quant_rows4<1, GS, GLU><<<grid, block, 0, st>>>(x, u, M, K, qx, sx, ra, sync); break;
            case 2: k_quant_rows4<2, GS, GLU><<<grid, block, 0, st>>>(x, u, M, K, qx, sx, ra, sync); break;
            case 4: k_quant_rows4<4, GS, GLU><<<grid, block, 0, st>>>(x, u, M, K, qx, sx, ra, sync); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    return packed ? launch_rot<7, -8, 7, true, GS, GLU>(x, u, M, K, qx, sx, ra, sync, st)
                  : launch_rot<7, -8, 7, false, GS, GLU>(x, u, M, K, qx, sx, nullptr, sync, st);
}

hipError_t launch_quant_act(int kind, int group, const uint16_t* x, int M, int K, int Kp, int8_t* qx,
                            float* sx, int32_t* ra, bool packed, uint32_t* sync, hipStream_t st) {
    if (kind == WK_W4) {
        if (packed && ra == nullptr) return hipErrorInvalidValue;
        switch (group) {
            case 256: return launch_w4_act<256>(x, nullptr, M, K, qx, sx, ra, packed, sync, st);
            case 64: return launch_w4_act<64>(x, nullptr, M, K, qx, sx, ra, packed, sync, st);
            case 16: return launch_w4_act<16>(x, nullptr, M, K, qx, sx, ra, packed, sync, st);
            case kRotRegular: return launch_w4_act<kRotRegular>(x, nullptr, M, K, qx, sx, ra, packed, sync, st);
            default: return hipErrorInvalidValue;
        }
    }
    // W4A8 and ConvRot INT8: rotated, per-row int8
    if (kind == WK_W4A8 || kind == WK_I8R) return launch_rot<127, -128, 127, false>(x, nullptr, M, K, qx, sx, nullptr, sync, st);
    // two waves per row when four per row would exceed what the chip holds at once
    const int threads = M * 4 > 8192 ? 128 : 256;
    const int ch = (K / 8 + threads - 1) / threads;
    if (K % 8 == 0 && ch >= 1 && ch <= 4) {
        const dim3 grid(M), block(threads);
        switch (ch) {
            case 1: k_quant_act_plain_reg<1><<<grid, block, 0, st>>>(x, M, K, Kp, qx, sx, sync); break;
            case 2: k_quant_act_plain_reg<2><<<grid, block, 0, st>>>(x, M, K, Kp, qx, sx, sync); break;
            case 3: k_quant_act_plain_reg<3><<<grid, block, 0, st>>>(x, M, K, Kp, qx, sx, sync); break;
            default: k_quant_act_plain_reg<4><<<grid, block, 0, st>>>(x, M, K, Kp, qx, sx, sync); break;
        }
        return hipGetLastError();
    }
    k_quant_act_plain<<<dim3(M), dim3(threads), 0, st>>>(x, M, K, Kp, qx, sx, sync);
    return hipGetLastError();
}

// h = silu(g) * u element by element (bf16 in, bf16 out), the values the
// MLP block's quantiser forms (inspection).
__global__ void __launch_bounds__(256) k_silu_mul(const uint16_t* __restrict__ g, const uint16_t* __restrict__ u,
                                                  size_t n, uint16_t* __restrict__ h) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) h[i] = (uint16_t)(__float_as_uint(silu_mul_bf16(bf16_to_f32(g[i]), bf16_to_f32(u[i]))) >> 16);
}

hipError_t launch_silu_mul(const uint16_t* g, const uint16_t* u, size_t n, uint16_t* h, hipStream_t st) {
    if (n == 0) return hipSuccess;
    k_silu_mul<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(g, u, n, h);
    return hipGetLastError();
}

hipError_t launch_quant_swiglu(const uint16_t* g, const uint16_t* u, int M, int K, int8_t* qx, float* sx,
                               int32_t* ra, bool packed, uint32_t* sync, hipStream_t st) {
    if (packed && ra == nullptr) return hipErrorInvalidValue;
    return launch_w4_act<256, true>(g, u, M, K, qx, sx, ra, packed, sync, st);
}

// ---------------------------------------------------------------------------
// Weight packing (offline).  The tensor absmax is accumulated with atomicMax
// on the float bit pattern (valid for non-negative floats) in the scale slot,
// which is then read as the absmax and finally replaced by absmax / Q.
// ---------------------------------------------------------------------------
__global__ void k_set_zero(uint32_t* p) { *p = 0u; }

__global__ void k_finalize_scale(float* p, float q) { p[0] = p[0] / q; }

template <int GPL, int GS>
__global__ void __launch_bounds__(512) k_absmax_rot_rows(const uint16_t* __restrict__ w, int K,
                                                         uint32_t* __restrict__ amax_bits) {
    __shared__ float red[16];
    const int n = blockIdx.x;
    const int hw = threadIdx.x >> 5, nhw = blockDim.x >> 5, lane32 = threadIdx.x & 31;
    RotRow<GPL, GS> r;
    const float a = block_max(r.load_rotate(w + (size_t)n * K, K >> 8, hw, nhw, lane32), red);
    if (threadIdx.x == 0) atomicMax(amax_bits, __float_as_uint(a));
}

// One dword of the W4 layout from 8 codes of k0..k0+7 (k0 % 8 == 0), the
// weight nibble forms: byte b = (code(k0+4+b) ^ 8) | code(k0+b) << 4.
__device__ __forceinline__ uint32_t w4_dword(const int (&q)[8]) {
    uint32_t o = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) o |= ((uint32_t)((q[b + 4] ^ 8) & 0xF) | ((uint32_t)(q[b] & 0xF) << 4)) << (8 * b);
    return o;
}

// Byte offset of the W4 dword holding k0..k0+7 of row n.
__device__ __forceinline__ size_t w4_dword_offset(int n, int k0, int K) {
    const int nb = n >> 5, r = n & 31, kc = k0 >> 6, kk = k0 & 63;
    const int t = kk >> 5, h = (kk >> 4) & 1, d = (kk >> 3) & 1;
    return ((size_t)nb * (K >> 6) + kc) * 1024 + r * 32 + 16 * h + 8 * t + 4 * d;
}

// One block per row (padding rows: zero codes); also cw[n], the sum of the
// row's codes held in high nibbles (k % 8 < 4).
template <int GPL, int GS>
__global__ void __launch_bounds__(512) k_pack_w4(const uint16_t* __restrict__ w, int N, int K,
                                                 const float* __restrict__ amax_slot,
                                                 uint8_t* __restrict__ out) {
    __shared__ int tot;
    const int n = blockIdx.x;
    const int G = K >> 8;
    const int hw = threadIdx.x >> 5, nhw = blockDim.x >> 5, lane32 = threadIdx.x & 31;
    int32_t* cw = reinterpret_cast<int32_t*>(out + w4_cw_offset(N, K));
    if (n >= N) {  // padding rows
        for (int i = 0; i < GPL; ++i) {
            const int g = hw + i * nhw;
            if (g < G) *reinterpret_cast<uint32_t*>(out + w4_dword_offset(n, g * 256 + lane32 * 8, K)) = 0x08080808u;
        }
        if (threadIdx.x == 0) cw[n] = 0;
        return;
    }
    if (threadIdx.x == 0) tot = 0;
    const float s = amax_slot[0] / 7.0f;
    RotRow<GPL, GS> r;
    r.load_rotate(w + (size_t)n * K, G, hw, nhw, lane32);
    int hsum = 0;
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
        const int g = hw + i * nhw;
        if (g < G) {
            int q[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) q[j] = quant_code<-8, 7>(r.v[i][j], s);
            *reinterpret_cast<uint32_t*>(out + w4_dword_offset(n, g * 256 + lane32 * 8, K)) = w4_dword(q);
            hsum += q[0] + q[1] + q[2] + q[3];
        }
    }
    __syncthreads();
    atomicAdd(&tot, hsum);
    __syncthreads();
    if (threadIdx.x == 0) cw[n] = tot;
}

template <int GS>
static hipError_t launch_pack_w4_gs(const uint16_t* w, int N, int K, uint8_t* out, float* scale, hipStream_t st) {
    const int Np = round_up(N, 32);
    int gpl = 1;
    const int threads = rot_threads(K >> 8, &gpl);
    uint32_t* bits = reinterpret_cast<uint32_t*>(scale);
    k_set_zero<<<1, 1, 0, st>>>(bits);
    switch (gpl) {
#define CR_PACK_CASE(G_)                                                                 \
    case G_:                                                                             \
        k_absmax_rot_rows<G_, GS><<<dim3(N), dim3(threads), 0, st>>>(w, K, bits);        \
        k_pack_w4<G_, GS><<<dim3(Np), dim3(threads), 0, st>>>(w, N, K, scale, out);      \
        break;
        CR_PACK_CASE(1) CR_PACK_CASE(2) CR_PACK_CASE(4) CR_PACK_CASE(8) CR_PACK_CASE(16)
#undef CR_PACK_CASE
        default: return hipErrorInvalidValue;
    }
    k_finalize_scale<<<1, 1, 0, st>>>(scale, 7.0f);
    return hipGetLastError();
}

hipError_t launch_pack_w4(const uint16_t* w, int N, int K, int group, uint8_t* out, float* scale,
                          hipStream_t st) {
    switch (group) {
        case 256: return launch_pack_w4_gs<256>(w, N, K, out, scale, st);
        case 64: return launch_pack_w4_gs<64>(w, N, K, out, scale, st);
        case 16: return launch_pack_w4_gs<16>(w, N, K, out, scale, st);
        case kRotRegular: return launch_pack_w4_gs<kRotRegular>(w, N, K, out, scale, st);
        default: return hipErrorInvalidValue;
    }
}

// --- int8_tensorwise ------------------------------------------------------

__global__ void __launch_bounds__(256) k_absmax_plain(const uint16_t* __restrict__ w, size_t count,
                                                      uint32_t* __restrict__ amax_bits) {
    __shared__ float red[16];
    float a = 0.0f;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (size_t)gridDim.x * blockDim.x)
        a = fmaxf(a, fabsf(bf16_to_f32(w[i])));
    a = block_max(a, red);
    if (threadIdx.x == 0) atomicMax(amax_bits, __float_as_uint(a));
}

// One thread per 16-byte segment (row n, 64-chunk kc, half h, step t).
__global__ void __launch_bounds__(256) k_pack_i8(const uint16_t* __restrict__ w, int N, int K,
                                                 int Kp, const float* __restrict__ amax_slot,
                                                 uint8_t* __restrict__ out, size_t nseg) {
    const size_t seg = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (seg >= nseg) return;
    const float s = amax_slot[0] / 127.0f;
    const size_t tile = seg >> 7;            // 128 segments of 16 B per 2 KiB tile
    const int within = (int)(seg & 127);
    const int r = within >> 2, h = (within >> 1) & 1, t = within & 1;
    const int nkc = Kp >> 6;
    const int nb = (int)(tile / nkc), kc = (int)(tile % nkc);
    const int n = nb * 32 + r;
    const int k0 = kc * 64 + 32 * t + 16 * h;
    uint32_t o[4] = {0u, 0u, 0u, 0u};
    if (n < N) {
#pragma unroll
        for (int p = 0; p < 16; ++p) {
            const int k = k0 + p;
            const int q = (k < K) ? quant_code<-128, 127>(bf16_to_f32(w[(size_t)n * K + k]), s) : 0;
            o[p >> 2] |= (uint32_t)(q & 0xFF) << (8 * (p & 3));
        }
    }
    *reinterpret_cast<uint4*>(out + tile * 2048 + r * 64 + 32 * h + 16 * t) = make_uint4(o[0], o[1], o[2], o[3]);
}

hipError_t launch_pack_i8(const uint16_t* w, int N, int K, uint8_t* out, float* scale,
                          hipStream_t st) {
    const int Np = round_up(N, 32), Kp = round_up(K, 64);
    uint32_t* bits = reinterpret_cast<uint32_t*>(scale);
    k_set_zero<<<1, 1, 0, st>>>(bits);
    const size_t count = (size_t)N * K;
    size_t blocks = (count + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    k_absmax_plain<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(w, count, bits);
    const size_t nseg = (size_t)Np * Kp / 16;
    k_pack_i8<<<dim3((unsigned)((nseg + 255) / 256)), dim3(256), 0, st>>>(w, N, K, Kp, scale, out, nseg);
    k_finalize_scale<<<1, 1, 0, st>>>(scale, 127.0f);
    return hipGetLastError();
}

// --- ConvRot INT8, row-scaled ---------------------------------------------

// One block per row n of the padded weight: the row rotated group by group,
// its absmax, scale[n] = absmax / 127 (IEEE division), codes
// clamp(rint(v / scale[n]), -128, 127) in the int8 tile layout (K % 256 == 0,
// so Kp = K).  Padding rows get zero codes.
template <int GPL>
__global__ void __launch_bounds__(512) k_pack_i8rot(const uint16_t* __restrict__ w, int N, int K,
                                                    uint8_t* __restrict__ out, float* __restrict__ scale) {
    __shared__ float red[16];
    const int n = blockIdx.x;
    const int G = K >> 8, nkc = K >> 6;
    const int hw = threadIdx.x >> 5, nhw = blockDim.x >> 5, lane32 = threadIdx.x & 31;
    const int nb = n >> 5, r = n & 31;
    // the 8 codes of k0..k0+7 (k0 % 8 == 0) are 8 consecutive bytes of the tile
    auto dst = [&](int k0) -> uint2* {
        const int kc = k0 >> 6, kk = k0 & 63;
        return reinterpret_cast<uint2*>(out + ((size_t)nb * nkc + kc) * 2048 + r * 64 +
                                        32 * ((kk >> 4) & 1) + 16 * (kk >> 5) + (kk & 15));
    };
    if (n >= N) {                                       // padding rows (whole block)
        for (int i = 0; i < GPL; ++i) {
            const int g = hw + i * nhw;
            if (g < G) *dst(g * 256 + lane32 * 8) = make_uint2(0u, 0u);
        }
        return;
    }
    RotRow<GPL> rr;
    const float amax = block_max(rr.load_rotate(w + (size_t)n * K, G, hw, nhw, lane32), red);
    const float s = amax / 127.0f;
    if (threadIdx.x == 0) scale[n] = s;
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
        const int g = hw + i * nhw;
        if (g < G) {
            int q[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) q[j] = quant_code<-128, 127>(rr.v[i][j], s);
            *dst(g * 256 + lane32 * 8) = make_uint2(pack4_i8(q[0], q[1], q[2], q[3]), pack4_i8(q[4], q[5], q[6], q[7]));
        }
    }
}

hipError_t launch_pack_i8rot(const uint16_t* w, int N, int K, uint8_t* out, float* scale,
                             hipStream_t st) {
    const int Np = round_up(N, 32);
    int gpl = 1;
    const int threads = rot_threads(K >> 8, &gpl);
    switch (gpl) {
#define CR_PACK8R_CASE(G_) \
    case G_: k_pack_i8rot<G_><<<dim3(Np), dim3(threads), 0, st>>>(w, N, K, out, scale); break;
        CR_PACK8R_CASE(1) CR_PACK8R_CASE(2) CR_PACK8R_CASE(4) CR_PACK8R_CASE(8) CR_PACK8R_CASE(16)
#undef CR_PACK8R_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// --- W4A8 -----------------------------------------------------------------

// One thread per W4-layout dword: re-orders the canonical index nibbles
// (low nibble = even k) of k0..k0+7 into the GEMM's nibble order.
__global__ void __launch_bounds__(256) k_pack_w4a8_idx(const uint8_t* __restrict__ idx, int N,
                                                       int K, uint8_t* __restrict__ out,
                                                       size_t ndw) {
    const size_t id = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= ndw) return;
    const size_t tile = id >> 8;
    const int within = (int)(id & 255);
    const int r = within >> 3, rem = within & 7;
    const int h = rem >> 2, t = (rem >> 1) & 1, d = rem & 1;
    const int nkc = K >> 6;
    const int nb = (int)(tile / nkc), kc = (int)(tile % nkc);
    const int n = nb * 32 + r;
    const int k0 = kc * 64 + 32 * t + 16 * h + 8 * d;
    uint32_t o = 0u;
    if (n < N) {
        const uint32_t c = *reinterpret_cast<const uint32_t*>(idx + (size_t)n * (K / 2) + k0 / 2);
        int nib[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) nib[j] = (c >> (4 * j)) & 0xF;   // nibble j = k0 + j
#pragma unroll
        for (int b = 0; b < 4; ++b) o |= ((uint32_t)nib[b] | ((uint32_t)nib[b + 4] << 4)) << (8 * b);
    }
    *reinterpret_cast<uint32_t*>(out + tile * 1024 + r * 32 + 16 * h + 8 * t + 4 * d) = o;
}

// One thread per (row, 64-chunk): the four group codes, natural group order.
__global__ void __launch_bounds__(256) k_pack_w4a8_codes(const uint8_t* __restrict__ s_rel, int N,
                                                         int K, uint8_t* __restrict__ out,
                                                         size_t nitems) {
    const size_t id = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= nitems) return;
    const int nkc = K >> 6;
    const size_t tile = id >> 5;
    const int r = (int)(id & 31);
    const int nb = (int)(tile / nkc), kc = (int)(tile % nkc);
    const int n = nb * 32 + r;
    uint32_t c = 0u;
    if (n < N) c = *reinterpret_cast<const uint32_t*>(s_rel + (size_t)n * (K / 16) + kc * 4);
    *reinterpret_cast<uint32_t*>(out + tile * 128 + r * 4) = c;
}

__global__ void __launch_bounds__(256) k_w4a8_table(const float* __restrict__ cb,
                                                    int8_t* __restrict__ table) {
    const int id = blockIdx.x * blockDim.x + threadIdx.x;   // 4096 entries
    const int c = id >> 4, i = id & 15;
    const float v = cb[i] * e4m3_decode((uint32_t)c);
    int q = 0;
    if (!__builtin_isnan(v)) q = (int)fminf(fmaxf(__builtin_rintf(v), -127.0f), 127.0f);
    table[id] = (int8_t)q;
}

hipError_t launch_pack_w4a8(const uint8_t* idx, const uint8_t* s_rel, const float* cb, int N,
                            int K, uint8_t* out, hipStream_t st) {
    const int Np = round_up(N, 32);
    const size_t ndw = (size_t)Np * K / 8;
    k_pack_w4a8_idx<<<dim3((unsigned)((ndw + 255) / 256)), dim3(256), 0, st>>>(idx, N, K, out, ndw);
    const size_t nitems = (size_t)Np * (K / 64);
    k_pack_w4a8_codes<<<dim3((unsigned)((nitems + 255) / 256)), dim3(256), 0, st>>>(
        s_rel, N, K, out + w4a8_codes_offset(N, K), nitems);
    k_w4a8_table<<<dim3(16), dim3(256), 0, st>>>(cb, reinterpret_cast<int8_t*>(out + w4a8_table_offset(N, K)));
    return hipGetLastError();
}

// --- W4A8 expanded to the int8 tile layout (per call, large M) ------------
// One thread per 16-byte segment (row n, 64-k chunk, half h, step t) of the
// int8 layout: the 16 indices k0 + 0..15 (k0 = 64 kc + 32 t + 16 h) decoded
// with their group's 16-byte table row by decode_w4a8, the decode the W4A8
// GEMM runs in registers, so the values are the same.  The 4 KiB table is
// read straight from memory (it stays in the caches); staging it in LDS per
// block read as many table bytes as the kernel writes (15.7 us at the W4A8
// layer, M = 4096).  Padding rows get zeros.
__global__ void __launch_bounds__(256) k_w4a8_expand(const uint8_t* __restrict__ p, int N, int K, size_t codes_off,
                                                     size_t table_off, uint8_t* __restrict__ out, size_t nseg) {
    const size_t seg = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (seg >= nseg) return;
    const size_t tile = seg >> 7;                 // 128 segments of 16 B per 2 KiB tile
    const int within = (int)(seg & 127);
    const int r = within >> 2, h = (within >> 1) & 1, t = within & 1;
    const int nkc = K >> 6;
    const int n = (int)(tile / nkc) * 32 + r;
    uint4 o = make_uint4(0u, 0u, 0u, 0u);
    if (n < N) {
        const uint2 src = *reinterpret_cast<const uint2*>(p + tile * 1024 + r * 32 + 16 * h + 8 * t);
        const uint32_t code = p[codes_off + tile * 128 + r * 4 + 2 * t + h];
        const uint4 trow = reinterpret_cast<const uint4*>(p + table_off)[code];
        const v4i d = decode_w4a8(src.x, src.y, trow);
        o = make_uint4((uint32_t)d.x, (uint32_t)d.y, (uint32_t)d.z, (uint32_t)d.w);
    }
    *reinterpret_cast<uint4*>(out + tile * 2048 + r * 64 + 32 * h + 16 * t) = o;
}

hipError_t launch_w4a8_expand(const uint8_t* packed, int N, int K, uint8_t* out, hipStream_t st) {
    const size_t nseg = (size_t)round_up(N, 32) * K / 16;
    k_w4a8_expand<<<dim3((unsigned)((nseg + 255) / 256)), dim3(256), 0, st>>>(
        packed, N, K, w4a8_codes_offset(N, K), w4a8_table_offset(N, K), out, nseg);
    return hipGetLastError();
}

// --- canonical weight codes (inspection) ---------------------------------

__global__ void __launch_bounds__(256) k_unpack_weight(int kind, const uint8_t* __restrict__ p, int N,
                                                       int K, int Kp, size_t codes_off,
                                                       size_t table_off, int8_t* __restrict__ out) {
    const size_t id = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= (size_t)N * K) return;
    const int n = (int)(id / K), k = (int)(id % K);
    const int nb = n >> 5, r = n & 31, kc = k >> 6, kk = k & 63;
    const int t = kk >> 5, h = (kk >> 4) & 1, pp = kk & 15;
    const size_t tile = (size_t)nb * (Kp >> 6) + kc;
    int v;
    if (wk_i8w(kind)) {
        v = (int8_t)p[tile * 2048 + r * 64 + 32 * h + 16 * t + pp];
    } else {
        const int d = pp >> 3, b = pp & 3, hi = (pp >> 2) & 1;
        const uint8_t byte = p[tile * 1024 + r * 32 + 16 * h + 8 * t + 4 * d + b];
        if (kind == WK_W4) {          // k0 + b high (two's complement), k0 + 4 + b low (offset)
            v = hi ? (int)(byte & 0xF) - 8 : (int)(int8_t)(byte & 0xF0) >> 4;
        } else {
            const int nib = hi ? (byte >> 4) : (byte & 0xF);
            const uint8_t code = p[codes_off + tile * 128 + r * 4 + 2 * t + h];
            v = (int8_t)p[table_off + (size_t)code * 16 + nib];
        }
    }
    out[id] = (int8_t)v;
}

hipError_t launch_unpack_weight(int kind, const uint8_t* packed, int N, int K, int8_t* out,
                                hipStream_t st) {
    const size_t count = (size_t)N * K;
    const int Kp = round_up(K, 64);
    size_t co = 0, to = 0;
    if (kind == WK_W4A8) { co = w4a8_codes_offset(N, K); to = w4a8_table_offset(N, K); }
    k_unpack_weight<<<dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st>>>(kind, packed, N, K, Kp, co, to, out);
    return hipGetLastError();
}

}  // namespace cr
