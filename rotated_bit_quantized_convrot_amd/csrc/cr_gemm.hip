// Integer GEMM + rank-one epilogue on v_mfma_i32_32x32x32_i8.
//
// acc[m,n] = sum_k qx[m,k] * qw[n,k] (exact int32), then
// y[m,n] = bf16(fl(fl(float(acc) * s_x[m]) * s_w) + bias[n])
// ([QIE] model card, "Speed" table: fused ConvRot + rank-one s4 MMA kernel;
// [REB] "Why W4A8 instead of GGUF": the W4A8 weights stay 4-bit in memory and
// the math is int8).  CDNA4 has no int4 MFMA, so 4-bit weights are widened to
// int8 in registers: W4 codes as 16*code (exact, then acc >> 4), W4A8 indices
// through a per-group 16-entry table row.
//
// MFMA operand roles: the weight fragment is the A operand (32 rows = n) and
// the activation fragment the B operand (32 columns = m).  Lane l supplies,
// for both, row/column l%32 and the 16 k values 16*(l/32)+0..15 of the step;
// the 32x32 int32 result leaves lane l with column m = l%32 and rows
// n = 8*(r/4) + 4*(l/32) + r%4 for accumulator register r.
#include "cr_device.h"
#include "cr_internal.h"

namespace cr {

constexpr int LDA = 80;   // LDS bytes per 64-k activation row (16 B pad: conflict-free b128 reads)

template <int WK> struct WRaw;
template <> struct WRaw<WK_W4> { uint4 a; };
template <> struct WRaw<WK_I8> { uint4 a, b; };
template <> struct WRaw<WK_W4A8> { uint4 a; uint32_t c; };

// Loads this lane's part of weight tile (nb, kc).
template <int WK>
__device__ __forceinline__ void load_wraw(WRaw<WK>& w, const uint8_t* __restrict__ wp,
                                          size_t codes_off, int nb, int nkc, int kc, int lane) {
    const size_t tile = (size_t)nb * nkc + kc;
    const int r = lane & 31, h = lane >> 5;
    if constexpr (WK == WK_W4) {
        w.a = *reinterpret_cast<const uint4*>(wp + tile * 1024 + r * 32 + 16 * h);
    } else if constexpr (WK == WK_I8) {
        const uint8_t* q = wp + tile * 2048 + r * 64 + 32 * h;
        w.a = *reinterpret_cast<const uint4*>(q);
        w.b = *reinterpret_cast<const uint4*>(q + 16);
    } else {
        w.a = *reinterpret_cast<const uint4*>(wp + tile * 1024 + r * 32 + 16 * h);
        w.c = *reinterpret_cast<const uint32_t*>(wp + codes_off + tile * 128 + r * 4);
    }
}

// The int8 A operand of MFMA step t (0 or 1) of a loaded tile.
template <int WK, int T>
__device__ __forceinline__ v4i wfrag(const WRaw<WK>& w, const uint4* __restrict__ stable, int h) {
    if constexpr (WK == WK_W4) {
        return T == 0 ? unpack_w4x16(w.a.x, w.a.y) : unpack_w4x16(w.a.z, w.a.w);
    } else if constexpr (WK == WK_I8) {
        const uint4 v = T == 0 ? w.a : w.b;
        v4i r;
        r.x = (int)v.x; r.y = (int)v.y; r.z = (int)v.z; r.w = (int)v.w;
        return r;
    } else {
        const uint32_t code = (w.c >> (8 * (2 * T + h))) & 0xFFu;
        const uint4 trow = stable[code];
        return T == 0 ? decode_w4a8(w.a.x, w.a.y, trow) : decode_w4a8(w.a.z, w.a.w, trow);
    }
}

// Exact accumulator from the MFMA sum (W4 operands carry a factor 16).
template <int WK>
__device__ __forceinline__ int fix_acc(int v) {
    if constexpr (WK == WK_W4) return v >> 4;
    else return v;
}

// Epilogue operands, copied out of the kernel arguments.
struct Epi {
    const float* wscale;   // tensor scale (1 float) or s_channel [N]
    const uint16_t* bias;  // [N] or null
    uint16_t* y;           // [M, N]
    int32_t* acc_out;      // [M, N] or null
    int N;
};

__device__ __forceinline__ Epi make_epi(const GemmArgs& p) {
    Epi e;
    e.wscale = p.wscale; e.bias = p.bias; e.y = p.y; e.acc_out = p.acc_out; e.N = p.N;
    return e;
}

// Writes 4 consecutive outputs n..n+3 of row m (n % 4 == 0, n < N).
template <int WK, bool ACC>
__device__ __forceinline__ void store4(const Epi& e, int m, int n, float sxm, int a0, int a1,
                                       int a2, int a3) {
    const int N = e.N;
    if constexpr (ACC) {
        int32_t* dst = e.acc_out + (size_t)m * N + n;
        if ((N & 3) == 0) {
            *reinterpret_cast<int4*>(dst) = make_int4(a0, a1, a2, a3);
        } else {
            dst[0] = a0;
            if (n + 1 < N) dst[1] = a1;
            if (n + 2 < N) dst[2] = a2;
            if (n + 3 < N) dst[3] = a3;
        }
    } else {
        const float sw0 = (WK == WK_W4A8) ? 0.0f : e.wscale[0];
        auto one = [&](int a, int nn) -> uint32_t {
            nn = nn < N ? nn : N - 1;
            float v = (float)a * sxm;
            v = v * ((WK == WK_W4A8) ? e.wscale[nn] : sw0);
            if (e.bias != nullptr) v = v + bf16_to_f32(e.bias[nn]);
            return f32_to_bf16_rne(v);
        };
        const uint32_t h0 = one(a0, n), h1 = one(a1, n + 1), h2 = one(a2, n + 2), h3 = one(a3, n + 3);
        uint16_t* dst = e.y + (size_t)m * N + n;
        if ((N & 3) == 0) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
        } else {
            dst[0] = (uint16_t)h0;
            if (n + 1 < N) dst[1] = (uint16_t)h1;
            if (n + 2 < N) dst[2] = (uint16_t)h2;
            if (n + 3 < N) dst[3] = (uint16_t)h3;
        }
    }
}

// ---------------------------------------------------------------------------
// Large-M kernel.  Block tile BM (activations) x BN (weights), 64-k stages.
// Activation tiles go through double-buffered LDS; each wave streams its
// weight tiles straight from global memory into registers (the packed layout
// gives every lane its operand bytes in one 16-byte load) one stage ahead.
// ---------------------------------------------------------------------------
template <int WK, int BM, int BN, int WM, int WN, bool ACC>
__global__ void __launch_bounds__(64 * WM * WN, 2) k_gemm_big(GemmArgs p, int tiles_m, int tiles_n) {
    constexpr int NT = 64 * WM * WN;
    constexpr int FM = BM / WM / 32, FN = BN / WN / 32;
    constexpr int CA = BM * 4 / NT;
    static_assert(CA * NT == BM * 4, "activation tile split");
    __shared__ __attribute__((aligned(16))) int8_t sA[2 * BM * LDA];
    __shared__ uint4 sT[WK == WK_W4A8 ? 256 : 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;

    // Block -> tile: blocks are dealt to the 8 XCDs round-robin; give each XCD
    // a contiguous run of tiles, ordered in bands of 8 tile-rows.
    const int total = tiles_m * tiles_n;
    const int bid = blockIdx.x;
    const int xcd = bid & 7, per = total >> 3, rem = total & 7;
    const int lid = xcd * per + (xcd < rem ? xcd : rem) + (bid >> 3);
    constexpr int GM = 8;
    const int band = lid / (GM * tiles_n);
    const int first_m = band * GM;
    const int gm = min(tiles_m - first_m, GM);
    const int in_band = lid - band * GM * tiles_n;
    const int tm = first_m + in_band % gm;
    const int tn = in_band / gm;
    const int m0 = tm * BM, n0 = tn * BN;

    const int M = p.M, Kp = p.Kp;
    const int nkc = Kp >> 6;
    const int nbmax = (p.Np >> 5) - 1;
    const size_t codes_off = w4a8_codes_offset(p.N, p.K);
    if constexpr (WK == WK_W4A8) {
        const uint4* tg = reinterpret_cast<const uint4*>(p.wp + w4a8_table_offset(p.N, p.K));
        for (int i = tid; i < 256; i += NT) sT[i] = tg[i];
    }

    int nbs[FN];
#pragma unroll
    for (int f = 0; f < FN; ++f) nbs[f] = min((n0 >> 5) + wn * FN + f, nbmax);

    uint4 ra[CA];
    const int8_t* arow[CA];
    int aoff[CA];
#pragma unroll
    for (int c = 0; c < CA; ++c) {
        const int idx = tid + c * NT;
        const int row = idx >> 2, ch = idx & 3;
        const int m = min(m0 + row, M - 1);
        arow[c] = p.qx + (size_t)m * Kp + ch * 16;
        aoff[c] = row * LDA + ch * 16;
    }

    WRaw<WK> wr[FN];
#pragma unroll
    for (int c = 0; c < CA; ++c) ra[c] = *reinterpret_cast<const uint4*>(arow[c]);
#pragma unroll
    for (int f = 0; f < FN; ++f) load_wraw<WK>(wr[f], p.wp, codes_off, nbs[f], nkc, 0, lane);
#pragma unroll
    for (int c = 0; c < CA; ++c) *reinterpret_cast<uint4*>(sA + aoff[c]) = ra[c];

    v16i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][f][r] = 0;
    __syncthreads();

    const int h = lane >> 5;
    const int arow_lds = (wm * FM * 32 + (lane & 31)) * LDA + 16 * h;
    for (int kc = 0; kc < nkc; ++kc) {
        const int cur = kc & 1;
        WRaw<WK> wc[FN];
#pragma unroll
        for (int f = 0; f < FN; ++f) wc[f] = wr[f];
        // Prefetch the next stage (the last iteration re-reads its own
        // stage; that copy is written to the idle buffer and never read).
        const int kn = min(kc + 1, nkc - 1);
#pragma unroll
        for (int c = 0; c < CA; ++c) ra[c] = *reinterpret_cast<const uint4*>(arow[c] + kn * 64);
#pragma unroll
        for (int f = 0; f < FN; ++f) load_wraw<WK>(wr[f], p.wp, codes_off, nbs[f], nkc, kn, lane);
        const int8_t* sa = sA + cur * BM * LDA + arow_lds;
        {
            v4i bf[FN];
#pragma unroll
            for (int f = 0; f < FN; ++f) bf[f] = wfrag<WK, 0>(wc[f], sT, h);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const v4i af = *reinterpret_cast<const v4i*>(sa + i * 32 * LDA);
#pragma unroll
                for (int f = 0; f < FN; ++f) acc[i][f] = mfma32(bf[f], af, acc[i][f]);
            }
        }
        {
            v4i bf[FN];
#pragma unroll
            for (int f = 0; f < FN; ++f) bf[f] = wfrag<WK, 1>(wc[f], sT, h);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const v4i af = *reinterpret_cast<const v4i*>(sa + i * 32 * LDA + 32);
#pragma unroll
                for (int f = 0; f < FN; ++f) acc[i][f] = mfma32(bf[f], af, acc[i][f]);
            }
        }
        {
            int8_t* dst = sA + (cur ^ 1) * BM * LDA;
#pragma unroll
            for (int c = 0; c < CA; ++c) *reinterpret_cast<uint4*>(dst + aoff[c]) = ra[c];
        }
        __syncthreads();
    }

    // Epilogue.
    const Epi epi = make_epi(p);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * FM * 32 + i * 32 + (lane & 31);
        if (m < M) {
            const float sxm = ACC ? 0.0f : p.sx[m];
#pragma unroll
            for (int f = 0; f < FN; ++f) {
                const int nbase = n0 + (wn * FN + f) * 32 + 4 * h;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = nbase + 8 * q;
                    if (n < p.N)
                        store4<WK, ACC>(epi, m, n, sxm, fix_acc<WK>(acc[i][f][4 * q + 0]),
                                        fix_acc<WK>(acc[i][f][4 * q + 1]),
                                        fix_acc<WK>(acc[i][f][4 * q + 2]),
                                        fix_acc<WK>(acc[i][f][4 * q + 3]));
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Small-M kernel (M <= 128).  Block = 4 waves over 128 weight rows (one 32-row
// tile per wave) and one K slice of at most KSLMAX 64-chunks; the slice of the
// activations (all rows) is staged in LDS once and shared by the 4 waves.
// Each wave issues all of its weight loads up front.  With several K slices
// each block stores its int32 partial sums in accumulator-register order
// (fully coalesced) and k_splitk_reduce, the next kernel on the stream, adds
// the slices in order and runs the epilogue: no atomics and no device-scope
// fences (both cost far more than a second launch here).
// ---------------------------------------------------------------------------
constexpr int KSLMAX = 8;

template <int WK, int MF, bool ACC>
__global__ void __launch_bounds__(256) k_gemm_skinny(GemmArgs p, int splits) {
    constexpr int MR = MF * 32;
    constexpr int CAMAX = MR * KSLMAX * 4 / 256;
    __shared__ __attribute__((aligned(16))) int8_t sA[MR * (KSLMAX * 64 + 16)];
    __shared__ uint4 sT[WK == WK_W4A8 ? 256 : 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
    const int bx = blockIdx.x, s = blockIdx.y;
    const int M = p.M, Kp = p.Kp, N = p.N;
    const int nkc = Kp >> 6;
    const int kc0 = (int)((long long)s * nkc / splits);
    const int kc1 = (int)((long long)(s + 1) * nkc / splits);
    const int ksl = kc1 - kc0;
    const int lrow = ksl * 64 + 16;
    const int nb = bx * 4 + wave;
    const bool active = nb < (p.Np >> 5);
    const size_t codes_off = w4a8_codes_offset(p.N, p.K);

    // 1. activation slice -> registers.  Thread chunk idx covers row
    //    idx / (4*KSLMAX), 16-byte column idx % (4*KSLMAX); columns past the
    //    slice re-read (and later re-store) the slice's last column, rows
    //    past M re-read row M-1.  Issued before the weight loads so that the
    //    wait for them does not wait for the weights.
    uint4 ra[CAMAX];
    int aoff[CAMAX];
#pragma unroll
    for (int c = 0; c < CAMAX; ++c) {
        const int idx = tid + c * 256;
        const int row = idx / (4 * KSLMAX);
        const int col = min(idx % (4 * KSLMAX), ksl * 4 - 1);
        const int m = min(row, M - 1);
        ra[c] = *reinterpret_cast<const uint4*>(p.qx + (size_t)m * Kp + (size_t)kc0 * 64 + col * 16);
        aoff[c] = row * lrow + col * 16;
    }
    // 2. all weight loads of this wave (chunks past the slice re-read its
    //    last chunk and are not used; idle waves read tile 0)
    WRaw<WK> wr[KSLMAX];
    const int nbl = active ? nb : 0;
#pragma unroll
    for (int j = 0; j < KSLMAX; ++j) load_wraw<WK>(wr[j], p.wp, codes_off, nbl, nkc, kc0 + min(j, ksl - 1), lane);
    // 3. activations -> LDS (duplicate chunks store identical bytes)
#pragma unroll
    for (int c = 0; c < CAMAX; ++c) *reinterpret_cast<uint4*>(sA + aoff[c]) = ra[c];
    if constexpr (WK == WK_W4A8) {
        const uint4* tg = reinterpret_cast<const uint4*>(p.wp + w4a8_table_offset(p.N, p.K));
        for (int i = tid; i < 256; i += 256) sT[i] = tg[i];
    }
    __syncthreads();

    v16i acc[MF];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0;

    if (active) {
        const int8_t* sa = sA + (lane & 31) * lrow + 16 * h;
#pragma unroll
        for (int j = 0; j < KSLMAX; ++j) {
            if (j < ksl) {
                const v4i b0 = wfrag<WK, 0>(wr[j], sT, h);
                const v4i b1 = wfrag<WK, 1>(wr[j], sT, h);
#pragma unroll
                for (int i = 0; i < MF; ++i) {
                    const v4i a0 = *reinterpret_cast<const v4i*>(sa + i * 32 * lrow + j * 64);
                    const v4i a1 = *reinterpret_cast<const v4i*>(sa + i * 32 * lrow + j * 64 + 32);
                    acc[i] = mfma32(b0, a0, acc[i]);
                    acc[i] = mfma32(b1, a1, acc[i]);
                }
            }
        }
    }

    const Epi epi = make_epi(p);
    if (splits == 1) {
        if (!active) return;
#pragma unroll
        for (int i = 0; i < MF; ++i) {
            const int m = i * 32 + (lane & 31);
            if (m < M) {
                const float sxm = ACC ? 0.0f : p.sx[m];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = nb * 32 + 8 * q + 4 * h;
                    if (n < N)
                        store4<WK, ACC>(epi, m, n, sxm, fix_acc<WK>(acc[i][4 * q]), fix_acc<WK>(acc[i][4 * q + 1]),
                                        fix_acc<WK>(acc[i][4 * q + 2]), fix_acc<WK>(acc[i][4 * q + 3]));
                }
            }
        }
        return;
    }

    // Split K: this slice's raw MFMA sums, in register order.
    if (!active) return;
    int4* dst = reinterpret_cast<int4*>(p.part) + ((((size_t)s * gridDim.x + bx) * 4 + wave) * MF) * 4 * 64 + lane;
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            dst[(i * 4 + q) * 64] = make_int4(acc[i][4 * q], acc[i][4 * q + 1], acc[i][4 * q + 2], acc[i][4 * q + 3]);
}

// Sum of the K slices' partials (in slice order) + epilogue.  One thread per
// (column block, wave, fragment, register quad, lane) of k_gemm_skinny.
template <int WK, int MF, bool ACC>
__global__ void __launch_bounds__(256) k_splitk_reduce(GemmArgs p, int splits, int nblk) {
    const size_t items = (size_t)nblk * 4 * MF * 4 * 64;
    const size_t id = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= items) return;
    const int lane = (int)(id & 63);
    size_t t = id >> 6;
    const int q = (int)(t % 4); t /= 4;
    const int i = (int)(t % MF); t /= MF;
    const int wave = (int)(t % 4);
    const int bx = (int)(t / 4);
    const int nb = bx * 4 + wave;
    if (nb >= (p.Np >> 5)) return;
    const int m = i * 32 + (lane & 31);
    const int n = nb * 32 + 8 * q + 4 * (lane >> 5);
    if (m >= p.M || n >= p.N) return;
    const int4* src = reinterpret_cast<const int4*>(p.part) + id;
    const size_t stride = items;
    int4 a = make_int4(0, 0, 0, 0);
    int k = 0;
    for (; k + 4 <= splits; k += 4) {
        const int4 v0 = src[(k + 0) * stride], v1 = src[(k + 1) * stride];
        const int4 v2 = src[(k + 2) * stride], v3 = src[(k + 3) * stride];
        a.x += v0.x; a.y += v0.y; a.z += v0.z; a.w += v0.w;
        a.x += v1.x; a.y += v1.y; a.z += v1.z; a.w += v1.w;
        a.x += v2.x; a.y += v2.y; a.z += v2.z; a.w += v2.w;
        a.x += v3.x; a.y += v3.y; a.z += v3.z; a.w += v3.w;
    }
    for (; k < splits; ++k) {
        const int4 v = src[k * stride];
        a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
    }
    const Epi epi = make_epi(p);
    const float sxm = ACC ? 0.0f : p.sx[m];
    store4<WK, ACC>(epi, m, n, sxm, fix_acc<WK>(a.x), fix_acc<WK>(a.y), fix_acc<WK>(a.z), fix_acc<WK>(a.w));
}

// ---------------------------------------------------------------------------
// Planning and launch.
// ---------------------------------------------------------------------------
SkinnyPlan plan_skinny(int M, int N, int K) {
    SkinnyPlan sp{};
    sp.use = M > 0 && M <= kSkinnyMaxM;
    if (!sp.use) return sp;
    const int Np = round_up(N, 32), Kp = round_up(K, 64);
    const int nkc = Kp / 64;
    sp.mf = (M + 31) / 32;
    sp.nblk = (Np + 127) / 128;
    sp.splits = (nkc + KSLMAX - 1) / KSLMAX;
    sp.part_bytes = sp.splits > 1 ? (size_t)sp.splits * sp.nblk * 4 * sp.mf * 4 * 64 * 16 : 0;
    return sp;
}

template <int WK, int MF, bool ACC>
static hipError_t launch_skinny_mf(const GemmArgs& a, const SkinnyPlan& sp, hipStream_t st) {
    k_gemm_skinny<WK, MF, ACC><<<dim3(sp.nblk, sp.splits), dim3(256), 0, st>>>(a, sp.splits);
    if (sp.splits > 1) {
        const size_t items = (size_t)sp.nblk * 4 * MF * 4 * 64;
        k_splitk_reduce<WK, MF, ACC><<<dim3((unsigned)((items + 255) / 256)), dim3(256), 0, st>>>(a, sp.splits, sp.nblk);
    }
    return hipGetLastError();
}

template <int WK, bool ACC>
static hipError_t launch_skinny_t(const GemmArgs& a, const SkinnyPlan& sp, hipStream_t st) {
    switch (sp.mf) {
        case 1: return launch_skinny_mf<WK, 1, ACC>(a, sp, st);
        case 2: return launch_skinny_mf<WK, 2, ACC>(a, sp, st);
        case 3: return launch_skinny_mf<WK, 3, ACC>(a, sp, st);
        case 4: return launch_skinny_mf<WK, 4, ACC>(a, sp, st);
        default: return hipErrorInvalidValue;
    }
}

template <int WK, bool ACC>
static hipError_t launch_big_t(const GemmArgs& a, hipStream_t st) {
    constexpr int BM = 256, BN = 128, WM = 2, WN = 2;
    const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
    k_gemm_big<WK, BM, BN, WM, WN, ACC><<<dim3(tiles_m * tiles_n), dim3(64 * WM * WN), 0, st>>>(a, tiles_m, tiles_n);
    return hipGetLastError();
}

template <int WK>
static hipError_t launch_kind(const GemmArgs& a, hipStream_t st) {
    const SkinnyPlan sp = plan_skinny(a.M, a.N, a.K);
    const bool acc = a.acc_out != nullptr;
    if (sp.use) return acc ? launch_skinny_t<WK, true>(a, sp, st) : launch_skinny_t<WK, false>(a, sp, st);
    return acc ? launch_big_t<WK, true>(a, st) : launch_big_t<WK, false>(a, st);
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
    switch (a.kind) {
        case WK_W4: return launch_kind<WK_W4>(a, st);
        case WK_I8: return launch_kind<WK_I8>(a, st);
        case WK_W4A8: return launch_kind<WK_W4A8>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace cr
