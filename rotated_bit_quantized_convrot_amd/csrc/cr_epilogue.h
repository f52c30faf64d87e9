// Epilogue shared by the GEMM kernels: y[m,n] = bf16_rne(fl(fl(float(acc) *
// s_x[m]) * s_w) + bias[n]) (a per-column scale in place of s_w for W4A8 and
// ConvRot INT8), or the
// exact int32 accumulator for the inspection hook.  The functions take the
// MFMA sums; W4A4 sums are turned into the exact dot products here (see the
// nibble forms in cr_internal.h).
#pragma once
#include "cr_device.h"
#include "cr_internal.h"

namespace cr {

// Epilogue operands, copied out of the kernel arguments.
struct Epi {
    const float* wscale;   // tensor scale (1 float) or s_channel [N]
    const uint16_t* bias;  // [N] or null
    uint16_t* y;           // [M, N]
    int32_t* acc_out;      // [M, N] or null
    const int32_t* ra;     // W4A4 correction sums [M] and [Np]
    const int32_t* cw;
    int N;
};

__device__ __forceinline__ Epi make_epi(const GemmArgs& p) {
    Epi e;
    e.wscale = p.wscale; e.bias = p.bias; e.y = p.y; e.acc_out = p.acc_out; e.N = p.N;
    e.ra = p.ra; e.cw = p.cw;
    return e;
}

// W4A4: exact dot products of row m, columns n..n+3 (n % 4 == 0, n < N; the
// cw vector has Np >= n + 4 entries) from the MFMA sums, in place.
template <int WK>
__device__ __forceinline__ void exact4(const Epi& e, int m, int n, int& a0, int& a1, int& a2, int& a3) {
    if constexpr (WK == WK_W4) {
        const int rn = -128 * e.ra[m];
        const int4 c = *reinterpret_cast<const int4*>(e.cw + n);
        a0 = w4_exact(a0, rn, -128 * c.x);
        a1 = w4_exact(a1, rn, -128 * c.y);
        a2 = w4_exact(a2, rn, -128 * c.z);
        a3 = w4_exact(a3, rn, -128 * c.w);
    }
}

// Writes 4 consecutive outputs n..n+3 of row m (n % 4 == 0, n < N) from
// their MFMA sums.  sw0: the tensor scale (unused with per-column scales,
// which are read from wscale[n]).
template <int WK, bool ACC>
__device__ __forceinline__ void store4(const Epi& e, int m, int n, float sxm, float sw0, int a0,
                                       int a1, int a2, int a3) {
    const int N = e.N;
    exact4<WK>(e, m, n, a0, a1, a2, a3);
    const bool full = (N & 3) == 0;          // n + 3 < N then, rows 8-byte aligned
    if constexpr (ACC) {
        int32_t* dst = e.acc_out + (size_t)m * N + n;
        if (full) {
            *reinterpret_cast<int4*>(dst) = make_int4(a0, a1, a2, a3);
        } else {
            dst[0] = a0;
            if (n + 1 < N) dst[1] = a1;
            if (n + 2 < N) dst[2] = a2;
            if (n + 3 < N) dst[3] = a3;
        }
    } else if (full) {
        float sw[4] = {sw0, sw0, sw0, sw0};
        if constexpr (wk_chan(WK)) {
            const float4 c = *reinterpret_cast<const float4*>(e.wscale + n);
            sw[0] = c.x; sw[1] = c.y; sw[2] = c.z; sw[3] = c.w;
        }
        float b[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        const bool has_bias = e.bias != nullptr;
        if (has_bias) {
            const uint2 bb = *reinterpret_cast<const uint2*>(e.bias + n);
            b[0] = bf16_lo(bb.x); b[1] = bf16_hi(bb.x); b[2] = bf16_lo(bb.y); b[3] = bf16_hi(bb.y);
        }
        const int a[4] = {a0, a1, a2, a3};
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[j] = (float)a[j] * sxm;
            v[j] = v[j] * sw[j];
            if (has_bias) v[j] = v[j] + b[j];
        }
        *reinterpret_cast<uint2*>(e.y + (size_t)m * N + n) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    } else {
        const int a[4] = {a0, a1, a2, a3};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int nn = n + j;
            if (nn < N) {
                float v = (float)a[j] * sxm;
                v = v * (wk_chan(WK) ? e.wscale[nn] : sw0);
                if (e.bias != nullptr) v = v + bf16_to_f32(e.bias[nn]);
                e.y[(size_t)m * N + nn] = (uint16_t)f32_to_bf16_rne(v);
            }
        }
    }
}

// Epilogue operands of 4 outputs n..n+3 of row m, fetched ahead of the
// accumulators (full-vector case: N % 4 == 0, m < M, n < N; otherwise
// `full` is false and store4 is used instead).
struct Epi4 {
    float sx, sw[4], b[4];
    int rn, cn[4];         // W4A4: -128 ra[m], -128 cw[n + j]
    bool full;
};

// Loads are unconditional so that nothing waits for them before they are
// used: indices are clamped to valid elements (rows past M read row M - 1,
// columns past N the last ones), and an absent operand (no bias; no weight
// scale, as in the accumulator hook) is read from s_x instead, its value
// unused.  `sx` must be valid.  COHERENT: s_x and ra were written by other
// blocks of the same kernel; they are read at device scope (not from a line
// a cache may hold from before).
template <int WK, bool COHERENT = false>
__device__ __forceinline__ Epi4 epi4_fetch(const Epi& e, const float* sx, int M, int m, int n) {
    Epi4 r;
    const int N = e.N;
    const bool vec = (N & 3) == 0;                           // then N >= 4
    const bool has_w = e.wscale != nullptr;
    r.full = vec && m < M && n < N && has_w;
    const int mc = min(m, M - 1);
    const int nc = vec ? min(n, N - 4) : 0;
    if constexpr (COHERENT) r.sx = __hip_atomic_load(sx + mc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else r.sx = sx[mc];
    const float* wsp = has_w ? e.wscale : sx;
    if constexpr (wk_chan(WK)) {
        const float* sc = wsp + (has_w ? nc : 0);
        r.sw[0] = sc[0];
        r.sw[1] = sc[has_w ? min(1, N - 1 - nc) : 0];
        r.sw[2] = sc[has_w ? min(2, N - 1 - nc) : 0];
        r.sw[3] = sc[has_w ? min(3, N - 1 - nc) : 0];
    } else {
        const float w = wsp[0];
        for (int j = 0; j < 4; ++j) r.sw[j] = w;
    }
    const uint16_t* bp = e.bias != nullptr ? e.bias + nc : reinterpret_cast<const uint16_t*>(sx);
    const uint32_t b01 = (uint32_t)bp[0] | ((uint32_t)bp[e.bias != nullptr ? min(1, N - 1 - nc) : 0] << 16);
    const uint32_t b23 = (uint32_t)bp[e.bias != nullptr ? min(2, N - 1 - nc) : 0] |
                         ((uint32_t)bp[e.bias != nullptr ? min(3, N - 1 - nc) : 0] << 16);
    r.b[0] = bf16_lo(b01); r.b[1] = bf16_hi(b01); r.b[2] = bf16_lo(b23); r.b[3] = bf16_hi(b23);
    // no bias: -0.0, which leaves every sum as it is (x + -0 == x, zeros
    // included), so store4_pre adds without a test
    if (e.bias == nullptr)
        for (int j = 0; j < 4; ++j) r.b[j] = -0.0f;
    if constexpr (WK == WK_W4) {
        if constexpr (COHERENT) r.rn = -128 * __hip_atomic_load(e.ra + mc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else r.rn = -128 * e.ra[mc];
        const int4 c = *reinterpret_cast<const int4*>(e.cw + (vec ? nc : 0));
        r.cn[0] = -128 * c.x; r.cn[1] = -128 * c.y; r.cn[2] = -128 * c.z; r.cn[3] = -128 * c.w;
    }
    return r;
}

// store4 with prefetched operands (r.full must hold): same arithmetic.
template <int WK>
__device__ __forceinline__ void store4_pre(const Epi& e, const Epi4& r, int m, int n, int a0, int a1,
                                           int a2, int a3) {
    int a[4] = {a0, a1, a2, a3};
    if constexpr (WK == WK_W4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = w4_exact(a[j], r.rn, r.cn[j]);
    }
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[j] = (float)a[j] * r.sx;
        v[j] = v[j] * r.sw[j];
        v[j] = v[j] + r.b[j];          // -0.0 without a bias
    }
    *reinterpret_cast<uint2*>(e.y + (size_t)m * e.N + n) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

}  // namespace cr
