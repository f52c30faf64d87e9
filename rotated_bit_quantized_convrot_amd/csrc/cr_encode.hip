// On-GPU W4A8 encoder: a bf16 weight [N, K] to the stored W4A8 tensors
// ([REB] "Rebels_w4a8s", "What's inside a file": 4-bit codebook indices two
// to a byte, an fp8 scale for every 16 weights along K, a scale per output
// row, 16 Lloyd-Max levels fit to the tensor).  Offline conversion, not the
// linear's hot path.
//
// Steps (float32 unless stated; every step has one definite result, so the
// tensors are the same whatever the launch shape):
//   1. rotate each 256-block of every row (the Sylvester matrix / 16, the
//      butterflies of the W4 packer), s_channel[n] = absmax / 127;
//   2. per 16-group: rel = min(gmax / s_channel, 127) (0 when s_channel is 0),
//      s_rel = E4M3 of rel, nearest with ties to the even code;
//      u = W~ / fl(e4m3(s_rel) * s_channel) (0 where that is 0);
//   3. Lloyd-Max on all u: levels start at lo + (j + 1/2) ((hi - lo) / 16) in
//      float64 (lo, hi the min and max of u); an iteration puts each u in the
//      cell of the levels' midpoints (on a midpoint: the lower cell) and moves
//      each non-empty cell's level to fl(float64(S) / float64(n)) 2^-24, S the
//      exact integer sum of rint(u 2^24) over the cell; the levels are then
//      sorted; stop when none moves or after `iters` iterations;
//   4. codebook = the levels rounded to float32; idx = the cell of u by the
//      float64 midpoints of the float32 codebook.
#include <hip/hip_runtime.h>

#include "convrot.h"
#include "cr_device.h"
#include "cr_internal.h"

namespace cr {

namespace {

constexpr int kPassBlocks = 1024;      // blocks of the Lloyd pass (partials per iteration)
constexpr int kPassThreads = 256;

// Workspace of the encoder: u float [N*K], row min / max of u, the Lloyd
// pass partials [kPassBlocks][16] (int64 sums, int64 counts), the levels
// (float64 [16]) and the state (converged flag).
struct EncLayout {
    size_t u, rmin, rmax, psum, pcnt, levels, state, total;
};

size_t a256(size_t v) { return (v + 255) / 256 * 256; }

EncLayout enc_layout(int N, int K) {
    EncLayout l{};
    l.u = 0;
    l.rmin = a256((size_t)N * K * 4);
    l.rmax = l.rmin + a256((size_t)N * 4);
    l.psum = l.rmax + a256((size_t)N * 4);
    l.pcnt = l.psum + a256((size_t)kPassBlocks * 16 * 8);
    l.levels = l.pcnt + a256((size_t)kPassBlocks * 16 * 8);
    l.state = l.levels + 256;
    l.total = l.state + 256;
    return l;
}

// Max over the block of any floats (blockDim.x <= 1024); every thread gets it.
__device__ __forceinline__ float block_max_any(float v, float* red) {
    v = wave_max(v);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    const int nw = (blockDim.x + 63) >> 6;
    float r = -__builtin_inff();
    for (int i = 0; i < nw; ++i) r = fmaxf(r, red[i]);
    __syncthreads();
    return r;
}

// Non-negative finite float (at most 448) -> E4M3FN code, nearest value, ties
// to the even code.  Below 2^-6 the values are the multiples m 2^-9 (m = 8 is
// 2^-6, code 0x08); above, 3 mantissa bits rounded half to even, a carry
// moving to the next exponent.
__device__ __forceinline__ uint32_t e4m3_encode_rne(float v) {
    if (v < 0.015625f) return (uint32_t)__builtin_rintf(v * 512.0f);
    const uint32_t b = __float_as_uint(v);
    const uint32_t e = (b >> 23) - 127u + 7u;         // biased E4M3 exponent (>= 1)
    const uint32_t mant = b & 0x7FFFFFu;
    uint32_t r = mant >> 20;
    const uint32_t rem = mant & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
    return (e << 3) + r;
}

// 1+2. One block per row: rotation, s_channel, s_rel, u and the row's min and
// max of u.  Lane pair (2i, 2i + 1) of a half-wave holds one 16-group.
template <int GPL>
__global__ void __launch_bounds__(512) k_enc_scales(const uint16_t* __restrict__ w, int K, float* __restrict__ s_channel,
                                                    uint8_t* __restrict__ s_rel, float* __restrict__ u,
                                                    float* __restrict__ rmin, float* __restrict__ rmax) {
    __shared__ float red[16];
    const int n = blockIdx.x;
    const int G = K >> 8;
    const int hw = threadIdx.x >> 5, nhw = blockDim.x >> 5, lane32 = threadIdx.x & 31;
    RotRow<GPL> rr;
    const float amax = block_max(rr.load_rotate(w + (size_t)n * K, G, hw, nhw, lane32), red);
    const float sc = amax / 127.0f;
    if (threadIdx.x == 0) s_channel[n] = sc;
    float lo = __builtin_inff(), hi = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
        const int g = hw + i * nhw;
        if (g < G) {                                  // whole half-waves: the pair partner is active
            float lm = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) lm = fmaxf(lm, fabsf(rr.v[i][j]));
            const float gm = fmaxf(lm, __shfl_xor(lm, 1, 64));
            float rel = sc > 0.0f ? gm / sc : 0.0f;
            rel = fminf(rel, 127.0f);
            const uint32_t code = e4m3_encode_rne(rel);
            const int k0 = g * 256 + lane32 * 8;
            if ((lane32 & 1) == 0) s_rel[(size_t)n * (K >> 4) + (k0 >> 4)] = (uint8_t)code;
            const float div = e4m3_decode(code) * sc;
            float q[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                q[j] = div > 0.0f ? rr.v[i][j] / div : 0.0f;
                lo = fminf(lo, q[j]);
                hi = fmaxf(hi, q[j]);
            }
            float4* dst = reinterpret_cast<float4*>(u + (size_t)n * K + k0);
            dst[0] = make_float4(q[0], q[1], q[2], q[3]);
            dst[1] = make_float4(q[4], q[5], q[6], q[7]);
        }
    }
    const float bhi = block_max_any(hi, red);
    const float blo = -block_max_any(-lo, red);
    if (threadIdx.x == 0) {
        rmin[n] = blo;
        rmax[n] = bhi;
    }
}

// 3 (start).  One block: lo, hi over the rows, the starting levels, state.
__global__ void __launch_bounds__(256) k_enc_init(const float* __restrict__ rmin, const float* __restrict__ rmax, int N,
                                                  double* __restrict__ levels, int* __restrict__ state) {
    __shared__ float red[16];
    float lo = __builtin_inff(), hi = -__builtin_inff();
    for (int i = threadIdx.x; i < N; i += blockDim.x) {
        lo = fminf(lo, rmin[i]);
        hi = fmaxf(hi, rmax[i]);
    }
    const float ghi = block_max_any(hi, red);
    const float glo = -block_max_any(-lo, red);
    if (threadIdx.x < 16) {
        const double l = (double)glo, h = (double)ghi;
        const double wd = (h - l) / 16.0;
        levels[threadIdx.x] = l + ((double)threadIdx.x + 0.5) * wd;
    }
    if (threadIdx.x == 0) state[0] = 0;
}

// Cell of x by the 15 midpoints (number of midpoints strictly below x).
__device__ __forceinline__ int cell_of(double x, const double (&t)[15]) {
    int j = 0;
#pragma unroll
    for (int c = 0; c < 15; ++c) j += t[c] < x ? 1 : 0;
    return j;
}

// 3 (pass).  Cell sums of rint(u 2^24) and counts, exact int64, per block.
__global__ void __launch_bounds__(kPassThreads) k_enc_pass(const float* __restrict__ u, size_t n,
                                                           const double* __restrict__ levels,
                                                           const int* __restrict__ state,
                                                           long long* __restrict__ psum, long long* __restrict__ pcnt) {
    if (state[0] != 0) return;                        // converged: nothing moves any more
    __shared__ unsigned long long ssum[16];
    __shared__ unsigned long long scnt[16];
    if (threadIdx.x < 16) {
        ssum[threadIdx.x] = 0ull;
        scnt[threadIdx.x] = 0ull;
    }
    double t[15];
#pragma unroll
    for (int c = 0; c < 15; ++c) t[c] = 0.5 * (levels[c] + levels[c + 1]);
    __syncthreads();
    for (size_t i = (size_t)blockIdx.x * kPassThreads + threadIdx.x; i < n; i += (size_t)gridDim.x * kPassThreads) {
        const float x = u[i];
        const int j = cell_of((double)x, t);
        const long long q = (long long)__builtin_rintf(x * 16777216.0f);
        atomicAdd(&ssum[j], (unsigned long long)q);   // two's complement: the int64 sum
        atomicAdd(&scnt[j], 1ull);
    }
    __syncthreads();
    if (threadIdx.x < 16) {
        psum[(size_t)blockIdx.x * 16 + threadIdx.x] = (long long)ssum[threadIdx.x];
        pcnt[(size_t)blockIdx.x * 16 + threadIdx.x] = (long long)scnt[threadIdx.x];
    }
}

// 3 (update).  One block of 64: the cell means, sorted; converged when no
// level moves.
__global__ void __launch_bounds__(64) k_enc_update(const long long* __restrict__ psum, const long long* __restrict__ pcnt,
                                                   int nblk, double* __restrict__ levels, int* __restrict__ state) {
    if (state[0] != 0) return;
    __shared__ double nl[16];
    const int c = threadIdx.x;
    if (c < 16) {
        long long s = 0, m = 0;
        for (int b = 0; b < nblk; ++b) {
            s += psum[(size_t)b * 16 + c];
            m += pcnt[(size_t)b * 16 + c];
        }
        nl[c] = m > 0 ? (double)s / (double)m * 0x1p-24 : levels[c];
    }
    __syncthreads();
    if (c == 0) {
        double v[16];
        for (int i = 0; i < 16; ++i) v[i] = nl[i];
        for (int i = 1; i < 16; ++i) {                // insertion sort
            const double x = v[i];
            int j = i - 1;
            while (j >= 0 && v[j] > x) {
                v[j + 1] = v[j];
                --j;
            }
            v[j + 1] = x;
        }
        bool same = true;
        for (int i = 0; i < 16; ++i) same = same && (v[i] == levels[i]);
        if (same) state[0] = 1;
        else
            for (int i = 0; i < 16; ++i) levels[i] = v[i];
    }
}

// 4.  The codebook (float32) and the indices, two per byte (low nibble = even k).
__global__ void __launch_bounds__(256) k_enc_idx(const float* __restrict__ u, size_t npairs,
                                                 const double* __restrict__ levels, float* __restrict__ codebook,
                                                 uint8_t* __restrict__ idx) {
    float cb[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) cb[c] = (float)levels[c];
    if (blockIdx.x == 0 && threadIdx.x < 16) codebook[threadIdx.x] = cb[threadIdx.x];
    double t[15];
#pragma unroll
    for (int c = 0; c < 15; ++c) t[c] = 0.5 * ((double)cb[c] + (double)cb[c + 1]);
    for (size_t p = (size_t)blockIdx.x * 256 + threadIdx.x; p < npairs; p += (size_t)gridDim.x * 256) {
        const float2 x = reinterpret_cast<const float2*>(u)[p];
        idx[p] = (uint8_t)(cell_of((double)x.x, t) | (cell_of((double)x.y, t) << 4));
    }
}

__global__ void __launch_bounds__(256) k_e4m3_encode(const float* __restrict__ v, size_t n, uint8_t* __restrict__ out) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) out[i] = (uint8_t)e4m3_encode_rne(v[i]);
}

}  // namespace

size_t encode_w4a8_workspace(int N, int K) { return enc_layout(N, K).total; }

hipError_t launch_encode_w4a8(const uint16_t* w, int N, int K, int iters, uint8_t* idx, uint8_t* s_rel,
                              float* codebook, float* s_channel, void* ws, hipStream_t st) {
    const EncLayout l = enc_layout(N, K);
    char* b = static_cast<char*>(ws);
    float* u = reinterpret_cast<float*>(b + l.u);
    float* rmin = reinterpret_cast<float*>(b + l.rmin);
    float* rmax = reinterpret_cast<float*>(b + l.rmax);
    long long* psum = reinterpret_cast<long long*>(b + l.psum);
    long long* pcnt = reinterpret_cast<long long*>(b + l.pcnt);
    double* levels = reinterpret_cast<double*>(b + l.levels);
    int* state = reinterpret_cast<int*>(b + l.state);
    int gpl = 1;
    const int threads = rot_threads(K >> 8, &gpl);
    switch (gpl) {
#define CR_ENC_CASE(G_) \
    case G_: k_enc_scales<G_><<<dim3(N), dim3(threads), 0, st>>>(w, K, s_channel, s_rel, u, rmin, rmax); break;
        CR_ENC_CASE(1) CR_ENC_CASE(2) CR_ENC_CASE(4) CR_ENC_CASE(8) CR_ENC_CASE(16)
#undef CR_ENC_CASE
        default: return hipErrorInvalidValue;
    }
    k_enc_init<<<1, 256, 0, st>>>(rmin, rmax, N, levels, state);
    const size_t n = (size_t)N * K;
    for (int it = 0; it < iters; ++it) {
        k_enc_pass<<<kPassBlocks, kPassThreads, 0, st>>>(u, n, levels, state, psum, pcnt);
        k_enc_update<<<1, 64, 0, st>>>(psum, pcnt, kPassBlocks, levels, state);
    }
    const size_t npairs = n / 2;
    size_t blocks = (npairs + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    k_enc_idx<<<dim3((unsigned)blocks), 256, 0, st>>>(u, npairs, levels, codebook, idx);
    return hipGetLastError();
}

hipError_t launch_e4m3_encode(const float* v, size_t n, uint8_t* out, hipStream_t st) {
    k_e4m3_encode<<<dim3((unsigned)((n + 255) / 256)), 256, 0, st>>>(v, n, out);
    return hipGetLastError();
}

}  // namespace cr
