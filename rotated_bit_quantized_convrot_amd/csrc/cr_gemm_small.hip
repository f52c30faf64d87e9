// Small-M GEMM path (M <= 128): k_gemm_small and k_small_reduce, their plan
// and launch.  Same arithmetic as the large-M kernel (exact int32
// accumulators, rank-one epilogue).
#include <algorithm>
#include <atomic>
#include <cmath>

#include "cr_device.h"
#include "cr_epilogue.h"
#include "cr_internal.h"

namespace cr {

// ---------------------------------------------------------------------------
// Small-M kernel (M <= 128) on v_mfma_i32_16x16x64_i8.
//
// Operand roles: weights are the A operand (16 rows = n), activations the B
// operand (16 columns = m).  Lane l supplies row/column l % 16 and 16 k
// values; both operands use the same k order, which is all the dot product
// needs.  The result leaves lane l with column m = l % 16 and rows
// n = 4 (l / 16) + r in register r.
//
// int8 layouts: a step is one 64-k chunk, lane group g = l / 16 takes
// k = kb(g) + 0..15 with kb(g) = 32 (g & 1) + 16 (g >> 1): 16 bytes at 16 g
// of the weight row's 64, and at kb(g) of the activation row [M, Kp].
// Packed 4-bit layouts (W4A4 and the W4A8 indices): in a chunk row r holds
// 32 bytes at r * 32, k = 32 t + 16 h + 0..15 in the 8 bytes at 16 h + 8 t.
// W4A4 steps over two chunks c, c + 1 with 16-byte loads: lane group g reads
// the 16 bytes at 16 (g & 1) of chunk c + (g >> 1), and MFMA t of the step
// takes their t-th 8 bytes, i.e. k = 64 (c + (g >> 1)) + 32 t + 16 (g & 1)
// + 0..15 on both operands (the two MFMAs cover the 128 k once).  W4A8 steps
// over one chunk, lane group g reading the 8 bytes at 8 g (k = kb(g) + ..).
//
// Block = 8 waves over NT 16-row weight tiles and a range of 64-k chunks
// (the whole K, or one of `splits` slices); wave w takes a contiguous run of
// the range's steps (run lengths differ by at most one), issues every load
// of its run up front, then runs NT x MT MFMAs per chunk.  The eight waves'
// int32 sums meet in LDS and each wave adds up and finishes a share of the
// NT x MT output tiles: epilogue when the block covers all of K, else an
// int32 partial tile for k_small_reduce.  W4A4 activations arrive packed
// (4-bit tiles, rows = m, activation nibble forms), the others as int8.
// ---------------------------------------------------------------------------
constexpr int SM_W = 8;   // waves per block
constexpr int SM_MAX_SPLITS = 16;   // K slices across blocks, at most

// Cache policy of a buffer access at device scope (the SC1 bit): a store is
// written through to the level every XCD reads, a load does not take a line
// another XCD may have left stale.
constexpr int kDeviceScope = 16;
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Loads of one chunk: NT weight fragments + MT activation fragments.
template <int WK> struct SmW;
template <> struct SmW<WK_W4> { v4i a; };
template <> struct SmW<WK_I8> { v4i a; };
template <> struct SmW<WK_I8R> { v4i a; };
template <> struct SmW<WK_W4A8> { v2i a; int c; };
template <int WK> struct SmA { v4i a; };             // int8 activations; W4A4: two 8-byte pieces

// 64-k chunks per step of a wave's run.
__host__ __device__ constexpr int small_ck(int wk) { return wk == WK_W4 ? 2 : 1; }

// ---------------------------------------------------------------------------
// Fused small-M W4A4 linear ([QIE] "Speed": the rotation, the 4-bit MMA and
// the rank-one rescale in one kernel).  The grid's first
// `fused_producers` blocks rotate and quantise the activation rows - two rows
// per block, 256 threads each, for K <= 4096, one row per block up to
// K = 16384; the row is x or, for the MLP block's down projection,
// silu(g) * u - with the arithmetic of the activation kernels
// (k_quant_act_rot: same butterflies, scale and codes), write the 4-bit codes, scales and
// correction sums with device-scope stores and count the rows on an arrival
// counter.  The GEMM blocks come after them: waves 1..7 issue their weight
// loads at once, wave 0 issues none and polls the counter (bounded), then
// every wave reads the codes at device scope.  Producers never wait and come
// first in dispatch order, so a waiting block never holds back the rows it
// waits for, and the launch needs no co-residency.  The counters are a device
// array of the library (zero when the library loads), one slot per launch
// taken round-robin on the host (at most kFusedSlots launches may be in
// flight at once); the last block of a launch to finish resets its slot.  A
// wait that runs out counts a timeout and leaves that block's outputs
// unwritten.
// ---------------------------------------------------------------------------
constexpr int kFusedSlots = 1024;
__device__ uint32_t fused_state[kFusedSlots][2];    // rows counted, blocks finished
__device__ uint32_t fused_timeout_count;

// Rows per producer block: two (256 threads each) up to K = 4096, else one.
// A lane takes 16 consecutive k of a 256-group and, past K = 8192, the same
// of a second group 32 groups on (K <= 16384).
__host__ __device__ constexpr int fused_rows_per_block(int K) { return K <= 4096 ? 2 : 1; }
constexpr int kFusedMaxK = 16384;

__device__ __forceinline__ void fused_finish(const GemmArgs& p) {
    if (threadIdx.x == 0) {
        uint32_t* st = fused_state[p.fused_slot];
        const uint32_t total = gridDim.x * gridDim.y;
        if (__hip_atomic_fetch_add(&st[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == total - 1) {
            __hip_atomic_store(&st[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&st[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Producer block pb: rows pb * rpb + h, h < rpb.  GLU: the row is
// silu(x) * xu (x the gate output, xu the up output), rounded to bf16 as the
// MLP block's quantiser forms it.
template <bool GLU>
__device__ __forceinline__ void fused_produce(const GemmArgs& p, int pb, float* redf, int* redi) {
    const int K = p.K, M = p.M;
    const int rpb = fused_rows_per_block(K), lpr = 512 / rpb, wpr = lpr >> 6;
    const int tid = threadIdx.x, h = tid / lpr, l = tid - h * lpr, wave = tid >> 6;
    const int m = pb * rpb + h;
    const int G = K >> 8, gslot = l >> 4, gstride = lpr >> 4, j = l & 15;
    float v[2][16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int g = gslot + i * gstride;
        if (m < M && g < G) {
            load16<GLU>(p.x, p.xu, (size_t)m * K + (size_t)g * 256 + j * 16, v[i]);
            fwht16_signed<256>(v[i], l);
#pragma unroll
            for (int t = 0; t < 16; ++t) amax = fmaxf(amax, fabsf(v[i][t]));
        }
    }
    amax = seg_max(amax, 64);
    if ((tid & 63) == 0) redf[wave] = amax;
    // the split-K arrival counters start at zero (device scope: GEMM blocks
    // on every XCD count on them once the rows are in)
    if (pb == 0 && p.sync != nullptr)
        for (int i = tid; i < kSyncWords; i += 512) __hip_atomic_store(p.sync + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    amax = 0.0f;
    for (int i = 0; i < wpr; ++i) amax = fmaxf(amax, redf[h * wpr + i]);
    const float s = (amax * rot_norm<256>()) / 7.0f;
    int hsum = 0;
    const float sigma = fwht16_sign<256>(l);
    const bool fast = amax >= 0x1p-100f && amax <= 0x1p100f;
    const float s_u = amax / 7.0f;
    const float rinv = sigma * (1.0f / s_u);               // undoes the lane's sign too
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int g = gslot + i * gstride;
        if (m < M && g < G) {
            float r[16];
            codes16<7, -8, 7, 256>(v[i], fast, rinv, sigma, s_u, s, r);
            hsum += (int)(r[4] + r[5] + r[6] + r[7] + r[12] + r[13] + r[14] + r[15]);
            const uint2 c = pack_act16(r);
            uint32_t* dst = reinterpret_cast<uint32_t*>(const_cast<int8_t*>(p.qx) + act4_offset(m, g * 256 + j * 16, K));
            __hip_atomic_store(dst, c.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(dst + 1, c.y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    for (int o = 1; o < 64; o <<= 1) hsum += __shfl_xor(hsum, o, 64);
    if ((tid & 63) == 0) redi[wave] = hsum;
    __syncthreads();
    if (l == 0 && m < M) {
        int t = 0;
        for (int i = 0; i < wpr; ++i) t += redi[h * wpr + i];
        __hip_atomic_store(const_cast<float*>(p.sx) + m, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(const_cast<int32_t*>(p.ra) + m, t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // every store of the rows is acknowledged before they are counted
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0 && pb * rpb < M)
        __hip_atomic_fetch_add(&fused_state[p.fused_slot][0], (uint32_t)min(rpb, M - pb * rpb), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
}

template <int WK, int MT, int NT, int CPW, bool FUSED = false>
__global__ void __launch_bounds__(512) k_gemm_small(GemmArgs p, int splits, int cps, int acc_mode) {
    extern __shared__ __attribute__((aligned(16))) int8_t smem[];
    int4* red = reinterpret_cast<int4*>(smem);                         // [SM_W][NT*MT][64]
    const uint4* stab = reinterpret_cast<const uint4*>(smem + SM_W * NT * MT * 1024);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    static_assert(!FUSED || WK == WK_W4, "fused quantisation: W4A4 only");
    int bx = blockIdx.x;                                               // weight block
    if constexpr (FUSED) {
        if ((int)blockIdx.x < p.fused_producers) {
            if (blockIdx.y == 0) {
                float* redf = reinterpret_cast<float*>(smem);
                int* redi = reinterpret_cast<int*>(smem) + 16;
                if (p.xu != nullptr) fused_produce<true>(p, blockIdx.x, redf, redi);
                else fused_produce<false>(p, blockIdx.x, redf, redi);
            }
            fused_finish(p);
            return;
        }
        bx -= p.fused_producers;
    }
    const int kb = 32 * (g & 1) + 16 * (g >> 1);
    const int nkc = p.Kp >> 6;
    const int nt16 = (p.N + 15) >> 4;
    const int s = blockIdx.y;
    const int kc0 = s * cps;
    constexpr int CK = small_ck(WK);
    const int kcs = min(nkc - kc0, cps) / CK;                         // steps of this block (>= 1)
    // this wave's run: steps [b0, b0 + len) from chunk kc0 (fused: wave 0
    // loads nothing, it waits for the producers)
    constexpr int NWL = FUSED ? SM_W - 1 : SM_W;                     // loading waves
    const int wl = FUSED ? wave - 1 : wave;
    const bool loader = wl >= 0;
    const int base = kcs / NWL, extra = kcs % NWL;
    const int len = loader ? base + (wl < extra ? 1 : 0) : 0;
    const int b0 = loader ? wl * base + min(wl, extra) : 0;

    // W4A8 decode table: loaded first, stored to LDS once the rest is in flight
    v4i tabv = v4i{0, 0, 0, 0};
    if constexpr (WK == WK_W4A8)
        tabv = reinterpret_cast<const v4i*>(p.wp + w4a8_table_offset(p.N, p.K))[tid & 255];

    // ---- epilogue operands of the (at most QPW) output tiles this wave
    //      finishes, fetched now so their latency hides behind the loads
    //      (fused: once the producers are done, the scales being theirs)
    constexpr int QPW = (NT * MT + SM_W - 1) / SM_W;
    Epi4 pre[QPW];
    auto prefetch = [&](auto COH) {
        const Epi epi0 = make_epi(p);
#pragma unroll
        for (int k = 0; k < QPW; ++k) {
            const int q = wave + SM_W * k;
            const int nt = bx * NT + q / MT;
            const int m = (q % MT) * 16 + r16, n = nt * 16 + 4 * g;
            pre[k] = epi4_fetch<WK, decltype(COH)::value>(epi0, p.sx, p.M, m, min(n, p.N - 1));
        }
    };
    if constexpr (!FUSED) prefetch(std::false_type{});

    // ---- buffer resources and per-lane offsets.  Weights: the (at most
    // three) 32-row bands the block's tiles live in; tile (band, chunk) is
    // WT bytes, row r of it at r * RB.  Activations: the whole code array.
    constexpr int WT = wk_i8w(WK) ? 2048 : 1024, RB = wk_i8w(WK) ? 64 : 32;
    const int nt_first = min(bx * NT, nt16 - 1);
    const int band0 = nt_first >> 1;
    const int nbands = min((p.Np >> 5) - band0, 3);
    const uint32_t band_bytes = (uint32_t)nkc * WT;
    const auto rs_w = buf_rsrc(p.wp + (size_t)band0 * band_bytes, (uint32_t)nbands * band_bytes);
    uint32_t wvo[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int nt = min(bx * NT + t, nt16 - 1);
        wvo[t] = (uint32_t)((nt >> 1) - band0) * band_bytes + (uint32_t)(((nt & 1) * 16 + r16) * RB) +
                 (uint32_t)(wk_i8w(WK) ? 16 * g : (WK == WK_W4 ? 16 * (g & 1) + (g >> 1) * WT : 8 * g));
    }
    __amdgpu_buffer_rsrc_t rs_c = rs_w;                                 // replaced below for W4A8
    uint32_t cvo[NT];
    if constexpr (WK == WK_W4A8) {
        const uint32_t cband = (uint32_t)nkc * 128;
        rs_c = buf_rsrc(p.wp + w4a8_codes_offset(p.N, p.K) + (size_t)band0 * cband, (uint32_t)nbands * cband);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int nt = min(bx * NT + t, nt16 - 1);
            cvo[t] = (uint32_t)((nt >> 1) - band0) * cband + (uint32_t)(((nt & 1) * 16 + r16) * 4);
        }
    }
    constexpr int AT = WK == WK_W4 ? 1024 : 64;                        // activation bytes per chunk step
    const uint32_t a_bytes = WK == WK_W4 ? (uint32_t)round_up(p.M, 32) * (uint32_t)(p.K / 2)
                                         : (uint32_t)p.M * (uint32_t)p.Kp;
    const auto rs_a = buf_rsrc(p.qx, a_bytes);
    uint32_t avo[MT];
#pragma unroll
    for (int j = 0; j < MT; ++j) {
        const int m = j * 16 + r16;
        if constexpr (WK == WK_W4)
            avo[j] = (uint32_t)((m >> 5) * nkc) * 1024u + (uint32_t)((m & 31) * 32 + 16 * (g & 1) + (g >> 1) * 1024);
        else avo[j] = (uint32_t)min(m, p.M - 1) * (uint32_t)p.Kp + (uint32_t)kb;
    }

    // ---- all loads of the run (slots past the run re-read its last chunk;
    //      a wave with an empty run reads the block's last chunk)
    SmW<WK> wr[CPW][NT];
    SmA<WK> ar[CPW][MT];
    if (loader) {
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const int kc = kc0 + CK * min(b0 + i, kcs - 1);                 // wave-uniform
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if constexpr (wk_i8w(WK) || WK == WK_W4) {
                wr[i][t].a = __builtin_amdgcn_raw_buffer_load_b128(rs_w, wvo[t], kc * WT, 0);
            } else {
                wr[i][t].a = __builtin_amdgcn_raw_buffer_load_b64(rs_w, wvo[t], kc * WT, 0);
                if constexpr (WK == WK_W4A8) wr[i][t].c = __builtin_amdgcn_raw_buffer_load_b32(rs_c, cvo[t], kc * 128, 0);
            }
        }
        if constexpr (!FUSED) {
#pragma unroll
            for (int j = 0; j < MT; ++j) ar[i][j].a = __builtin_amdgcn_raw_buffer_load_b128(rs_a, avo[j], kc * AT, 0);
        }
    }
    }
    // keep every load above this point: all of the run is in flight before
    // the first MFMA waits for its chunk
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (FUSED) {
        // wave 0 (no loads in flight, so each poll returns at once) waits
        // for every row; then all waves read the codes at device scope
        __shared__ int s_ready;
        if (tid == 0) {
            int ready = 0;
            const uint32_t* rows = &fused_state[p.fused_slot][0];
            for (int it = 0; it < p.spin_limit; ++it) {
                if (__hip_atomic_load(rows, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= (uint32_t)p.M) {
                    ready = 1;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            if (!ready) __hip_atomic_fetch_add(&fused_timeout_count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_ready = ready;
        }
        __syncthreads();
        if (!s_ready) {
            fused_finish(p);
            return;
        }
        if (loader) {
#pragma unroll
            for (int i = 0; i < CPW; ++i) {
                const int kc = kc0 + CK * min(b0 + i, kcs - 1);
#pragma unroll
                for (int j = 0; j < MT; ++j)
                    ar[i][j].a = __builtin_amdgcn_raw_buffer_load_b128(rs_a, avo[j], kc * AT, kDeviceScope);
            }
        } else {
#pragma unroll
            for (int i = 0; i < CPW; ++i)
#pragma unroll
                for (int j = 0; j < MT; ++j) ar[i][j].a = v4i{0, 0, 0, 0};
        }
        prefetch(std::true_type{});
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (WK == WK_W4A8) {
        if (tid < 256) const_cast<uint4*>(stab)[tid] = make_uint4((uint32_t)tabv.x, (uint32_t)tabv.y, (uint32_t)tabv.z, (uint32_t)tabv.w);
        __syncthreads();
    }

    v4i acc[NT][MT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < MT; ++j) acc[t][j] = v4i{0, 0, 0, 0};

    // Every slot runs its MFMAs (slots past the run with a zero weight
    // operand), so no load is only used under a branch and none gets sunk
    // behind the wait for another.
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const bool valid = i < len;
        if constexpr (WK == WK_W4) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {                                  // the step's two MFMAs
                v4i b[MT];
#pragma unroll
                for (int j = 0; j < MT; ++j)
                    b[j] = h == 0 ? unpack_act4((uint32_t)ar[i][j].a.x, (uint32_t)ar[i][j].a.y)
                                  : unpack_act4((uint32_t)ar[i][j].a.z, (uint32_t)ar[i][j].a.w);
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    v4i a = h == 0 ? unpack_wt4((uint32_t)wr[i][t].a.x, (uint32_t)wr[i][t].a.y)
                                   : unpack_wt4((uint32_t)wr[i][t].a.z, (uint32_t)wr[i][t].a.w);
                    if (!valid) a = v4i{0, 0, 0, 0};
#pragma unroll
                    for (int j = 0; j < MT; ++j)
                        acc[t][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[j], acc[t][j], 0, 0, 0);
                }
            }
        } else {
            v4i b[MT];
#pragma unroll
            for (int j = 0; j < MT; ++j) b[j] = ar[i][j].a;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                v4i a;
                if constexpr (wk_i8w(WK)) {
                    a = wr[i][t].a;
                } else {
                    const uint32_t code = ((uint32_t)wr[i][t].c >> (8 * (2 * (g & 1) + (g >> 1)))) & 0xFFu;
                    a = decode_w4a8((uint32_t)wr[i][t].a.x, (uint32_t)wr[i][t].a.y, stab[code]);
                }
                if (!valid) a = v4i{0, 0, 0, 0};
#pragma unroll
                for (int j = 0; j < MT; ++j)
                    acc[t][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[j], acc[t][j], 0, 0, 0);
            }
        }
    }

    // ---- the eight waves' sums meet in LDS
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < MT; ++j)
            red[((wave * NT + t) * MT + j) * 64 + lane] = make_int4(acc[t][j].x, acc[t][j].y, acc[t][j].z, acc[t][j].w);
    __syncthreads();

    const Epi epi = make_epi(p);
    const float sw0 = (wk_chan(WK) || acc_mode) ? 0.0f : p.wscale[0];
    // K split across blocks: with arrival counters (in-kernel completion) the
    // last of a weight block's `splits` blocks to arrive adds the others'
    // partial tiles and runs the epilogue; without, k_small_reduce does.
    const bool inkernel = splits > 1 && p.sync != nullptr && (int)gridDim.x - (FUSED ? p.fused_producers : 0) <= kSyncWords;
    // outputs m, n..n+3 from the MFMA sums of output tile k of this wave
    auto finish4 = [&](int k, int m, int n, const int4& sum) {
        if constexpr (FUSED) {
            // the row's scale and correction as prefetched (device scope;
            // N % 4 == 0 on this path, so every tile is a full vector)
            if (acc_mode) {
                int a[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) a[jj] = w4_exact(a[jj], pre[k].rn, pre[k].cn[jj]);
                *reinterpret_cast<int4*>(p.acc_out + (size_t)m * p.N + n) = make_int4(a[0], a[1], a[2], a[3]);
            } else {
                store4_pre<WK>(epi, pre[k], m, n, sum.x, sum.y, sum.z, sum.w);
            }
        } else {
            if (acc_mode)
                store4<WK, true>(epi, m, n, 0.0f, 0.0f, sum.x, sum.y, sum.z, sum.w);
            else if (pre[k].full)
                store4_pre<WK>(epi, pre[k], m, n, sum.x, sum.y, sum.z, sum.w);
            else
                store4<WK, false>(epi, m, n, p.sx[m], sw0, sum.x, sum.y, sum.z, sum.w);
        }
    };
    const size_t slice_i4 = (size_t)nt16 * MT * 64;                    // int4 per K slice
    int4 keep[QPW];
#pragma unroll
    for (int k = 0; k < QPW; ++k) {
        const int q = wave + SM_W * k;
        if (q >= NT * MT) break;
        int4 sum = red[q * 64 + lane];
#pragma unroll
        for (int w = 1; w < SM_W; ++w) {
            const int4 v = red[(w * NT * MT + q) * 64 + lane];
            sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
        }
        keep[k] = sum;
        const int t = q / MT, j = q % MT;
        const int nt = bx * NT + t;
        if (nt >= nt16) continue;
        if (splits > 1) {
            const size_t at = ((size_t)nt * MT + j) * 64 + lane;
            if (inkernel) {
                // device-scope store: written through to where every XCD reads it
                const auto rs = buf_rsrc(reinterpret_cast<int4*>(p.part) + (size_t)s * slice_i4,
                                         (uint32_t)(slice_i4 * 16));
                __builtin_amdgcn_raw_buffer_store_b128(v4u{(uint32_t)sum.x, (uint32_t)sum.y, (uint32_t)sum.z,
                                                           (uint32_t)sum.w},
                                                       rs, (int)(at * 16), 0, kDeviceScope);
            } else {
                reinterpret_cast<int4*>(p.part)[(size_t)s * slice_i4 + at] = sum;
            }
            continue;
        }
        const int m = j * 16 + r16, n = nt * 16 + 4 * g;
        if (m >= p.M || n >= p.N) continue;
        finish4(k, m, n, sum);
    }
    if (!inkernel) {
        if constexpr (FUSED) fused_finish(p);
        return;
    }
    // Every wave's partial stores are acknowledged at device scope before the
    // block counts itself in; the block that brings the count to `splits` is
    // the last, resets the counter for the next GEMM on this workspace and
    // finishes the tiles.
    __shared__ int s_last;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
        s_last = __hip_atomic_fetch_add(&p.sync[bx], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 (uint32_t)(splits - 1);
    __syncthreads();
    if (!s_last) {
        if constexpr (FUSED) fused_finish(p);
        return;
    }
    if (tid == 0) __hip_atomic_store(&p.sync[bx], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // device-scope loads (the other XCDs' stores, not a stale cached copy),
    // all issued before the first is used; the other slices' tiles in a
    // fixed order (integer sums: the order does not change the result)
    const auto rs_part = buf_rsrc(p.part, (uint32_t)(slice_i4 * 16 * splits));
    v4u oth[QPW][SM_MAX_SPLITS];
#pragma unroll
    for (int s2 = 0; s2 < SM_MAX_SPLITS; ++s2) {
#pragma unroll
        for (int k = 0; k < QPW; ++k) {
            const int q = wave + SM_W * k;
            const int nt = bx * NT + q / MT;
            oth[k][s2] = v4u{0u, 0u, 0u, 0u};
            if (s2 < splits && s2 != s && q < NT * MT && nt < nt16) {
                const size_t at = ((size_t)nt * MT + q % MT) * 64 + lane;
                oth[k][s2] = __builtin_amdgcn_raw_buffer_load_b128(rs_part, (int)((s2 * slice_i4 + at) * 16), 0,
                                                                   kDeviceScope);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < QPW; ++k) {
        const int q = wave + SM_W * k;
        if (q >= NT * MT) break;
        const int t = q / MT, j = q % MT;
        const int nt = bx * NT + t;
        if (nt >= nt16) continue;
        int4 sum = keep[k];
#pragma unroll
        for (int s2 = 0; s2 < SM_MAX_SPLITS; ++s2) {
            sum.x += (int)oth[k][s2].x; sum.y += (int)oth[k][s2].y;
            sum.z += (int)oth[k][s2].z; sum.w += (int)oth[k][s2].w;
        }
        const int m = j * 16 + r16, n = nt * 16 + 4 * g;
        if (m >= p.M || n >= p.N) continue;
        finish4(k, m, n, sum);
    }
    if constexpr (FUSED) fused_finish(p);
}

// Sum of the S K slices' partial tiles + epilogue; one thread per (16-row
// weight tile, activation tile, lane).  S is a template parameter so that
// all S loads are issued before the first add.
template <int WK, int S>
__global__ void __launch_bounds__(256) k_small_reduce(GemmArgs p, int mt, int acc_mode) {
    const int nt16 = (p.N + 15) >> 4;
    const size_t items = (size_t)nt16 * mt * 64;
    const size_t id = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= items) return;
    const int lane = (int)(id & 63);
    const size_t q = id >> 6;
    const int j = (int)(q % mt), nt = (int)(q / mt);
    const int m = j * 16 + (lane & 15), n = nt * 16 + 4 * (lane >> 4);
    if (m >= p.M || n >= p.N) return;
    const int4* src = reinterpret_cast<const int4*>(p.part) + id;
    int4 v[S];
#pragma unroll
    for (int k = 0; k < S; ++k) v[k] = src[(size_t)k * items];
    int4 a = v[0];
#pragma unroll
    for (int k = 1; k < S; ++k) {
        a.x += v[k].x; a.y += v[k].y; a.z += v[k].z; a.w += v[k].w;
    }
    const Epi epi = make_epi(p);
    if (acc_mode) {
        store4<WK, true>(epi, m, n, 0.0f, 0.0f, a.x, a.y, a.z, a.w);
    } else {
        const float sw0 = wk_chan(WK) ? 0.0f : p.wscale[0];
        store4<WK, false>(epi, m, n, p.sx[m], sw0, a.x, a.y, a.z, a.w);
    }
}

template <int WK>
static hipError_t launch_small_reduce(const GemmArgs& a, int splits, int mt, int acc_mode, hipStream_t st) {
    const size_t items = (size_t)((a.N + 15) / 16) * mt * 64;
    const dim3 grid((unsigned)((items + 255) / 256)), block(256);
    switch (splits) {
#define CR_RED_CASE(S_) \
    case S_: k_small_reduce<WK, S_><<<grid, block, 0, st>>>(a, mt, acc_mode); break;
        CR_RED_CASE(2) CR_RED_CASE(3) CR_RED_CASE(4) CR_RED_CASE(5) CR_RED_CASE(6) CR_RED_CASE(7)
        CR_RED_CASE(8) CR_RED_CASE(9) CR_RED_CASE(10) CR_RED_CASE(11) CR_RED_CASE(12) CR_RED_CASE(13)
        CR_RED_CASE(14) CR_RED_CASE(15) CR_RED_CASE(16)
#undef CR_RED_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Planning and launch of the small-M path.
// ---------------------------------------------------------------------------
// 16-row weight tiles per block for MT activation tiles (the LDS meeting
// point holds SM_W * NT * MT KiB).
__host__ __device__ constexpr int small_nt(int mt) { return mt <= 5 ? 3 : 2; }
constexpr int SM_CPW_MAX = 8;

// VGPRs of one step's loads; a wave holds at most 128 of them.
__host__ __device__ constexpr int small_regs_per_chunk(int wk, int mt, int nt) {
    return nt * (wk == WK_W4A8 ? 3 : 4) + mt * 4;
}
constexpr int SM_LOAD_REGS = 128;

// Plan override for inspection and timing (cr_dbg_small_plan): K slices
// across blocks; 0 leaves the planner's choice.
static std::atomic<int> g_small_force_splits{0};
void set_small_plan_override(int splits) { g_small_force_splits.store(splits); }

SmallPlan plan_small(int kind, int M, int N, int K) {
    SmallPlan sp{};
    sp.use = M > 0 && M <= kSmallMaxM;
    if (!sp.use) return sp;
    const int Kp = wk_i8w(kind) ? round_up(K, 64) : K;
    const int ck = small_ck(kind);
    const int nkc = Kp / 64;
    const int nsteps = nkc / ck;                 // W4A4: K % 256 == 0, so nkc is even
    const int nt16 = (N + 15) / 16;
    sp.mt = (M + 15) / 16;
    sp.nt = small_nt(sp.mt);
    const int nblk = (nt16 + sp.nt - 1) / sp.nt;
    const int per_chunk = small_regs_per_chunk(kind, sp.mt, sp.nt);
    const double wbytes = kind == WK_W4 ? 0.5 : (wk_i8w(kind) ? 1.0 : 0.5625);
    const double abytes = kind == WK_W4 ? 0.5 : 1.0;
    double best = 1e30;
    const int forced = g_small_force_splits.load();
    for (int pass = forced > 0 ? 0 : 1; pass < 2 && best >= 1e30; ++pass)
    for (int S = 1; S <= nsteps && S <= SM_MAX_SPLITS; ++S) {
        if (pass == 0 && S != forced) continue;  // the forced count, where it fits
        const int sps = (nsteps + S - 1) / S;    // steps per slice
        const int splits = (nsteps + sps - 1) / sps;
        if (splits != S) continue;
        const int cps = sps * ck;
        const int cpw = (sps + SM_W - 1) / SM_W;
        if (cpw > SM_CPW_MAX || cpw * per_chunk > SM_LOAD_REGS) continue;
        // rough cycle model: per block max(L2->CU bytes at 64 B/clk, MFMA
        // issue of 2 waves per SIMD) + latency, rounds of 256 blocks, and
        // the partial round trip + second launch when K is split
        const double blocks = (double)nblk * splits;
        const double rounds = std::ceil(blocks / 256.0);
        const double bytes = (double)cps * 64.0 * (sp.nt * 16 * wbytes + sp.mt * 16 * abytes);
        const double mfma = 2.0 * cpw * ck * sp.nt * sp.mt * 16.0;
        double cost = rounds * (std::max(bytes / 64.0, mfma) + 2000.0);
        // (the last-arriving block finishes the tiles: ~800 cycles for its
        // dependent reads; a second kernel where the counters cannot cover
        // the blocks: ~3000; and ~300 per slice for its partial tile's
        // device-scope store and acknowledgement.  Forced splits at M = 76,
        // cold weights: ConvRot INT8 2560^2 10.1 us with 3 slices against
        // 10.9 with 4 and 11.6 with 2; the down projection, K = 9728, 11.0
        // with 4 against 11.4 with 3)
        if (splits > 1)
            cost += (double)splits * (sp.mt * 16 * N * 8 / 4000.0 + 300.0) + (nblk <= kSyncWords ? 800.0 : 3000.0);
        if (cost < best) {
            best = cost;
            sp.splits = splits;
            sp.cps = cps;
            sp.cpw = cpw;
        }
    }
    if (best >= 1e30) {          // K beyond what the plan covers: no small-M path
        sp.use = false;
        return sp;
    }
    sp.nblk = nblk;
    sp.part_bytes = sp.splits > 1 ? (size_t)sp.splits * nt16 * sp.mt * 64 * 16 : 0;
    sp.lds = (size_t)SM_W * sp.nt * sp.mt * 1024 + (kind == WK_W4A8 ? 4096 : 0);
    return sp;
}

template <int WK, int MT, int CPW>
static hipError_t launch_small_c(const GemmArgs& a, const SmallPlan& sp, hipStream_t st) {
    constexpr int NT = small_nt(MT);
    if constexpr (CPW * small_regs_per_chunk(WK, MT, NT) > SM_LOAD_REGS) {
        return hipErrorInvalidValue;            // never planned
    } else {
    auto kern = &k_gemm_small<WK, MT, NT, CPW>;
    static std::atomic<uint64_t> lds_done;
    {
        const int lds = SM_W * NT * MT * 1024 + (WK == WK_W4A8 ? 4096 : 0);
        hipError_t e = opt_in_lds(reinterpret_cast<const void*>(kern), lds, lds_done);
        if (e != hipSuccess) return e;
    }
    const int acc_mode = a.acc_out != nullptr ? 1 : 0;
    kern<<<dim3(sp.nblk, sp.splits), dim3(64 * SM_W), sp.lds, st>>>(a, sp.splits, sp.cps, acc_mode);
    // the kernel completes split tiles itself when it has the arrival counters
    if (sp.splits > 1 && (a.sync == nullptr || sp.nblk > kSyncWords))
        return launch_small_reduce<WK>(a, sp.splits, MT, acc_mode, st);
    return hipGetLastError();
    }
}

template <int WK, int MT>
static hipError_t launch_small_m(const GemmArgs& a, const SmallPlan& sp, hipStream_t st) {
    switch (sp.cpw) {
        case 1: return launch_small_c<WK, MT, 1>(a, sp, st);
        case 2: return launch_small_c<WK, MT, 2>(a, sp, st);
        case 3: return launch_small_c<WK, MT, 3>(a, sp, st);
        case 4: return launch_small_c<WK, MT, 4>(a, sp, st);
        case 5: return launch_small_c<WK, MT, 5>(a, sp, st);
        case 6: return launch_small_c<WK, MT, 6>(a, sp, st);
        case 7: return launch_small_c<WK, MT, 7>(a, sp, st);
        case 8: return launch_small_c<WK, MT, 8>(a, sp, st);
        default: return hipErrorInvalidValue;
    }
}

template <int WK>
static hipError_t launch_small_t(const GemmArgs& a, const SmallPlan& sp, hipStream_t st) {
    switch (sp.mt) {
        case 1: return launch_small_m<WK, 1>(a, sp, st);
        case 2: return launch_small_m<WK, 2>(a, sp, st);
        case 3: return launch_small_m<WK, 3>(a, sp, st);
        case 4: return launch_small_m<WK, 4>(a, sp, st);
        case 5: return launch_small_m<WK, 5>(a, sp, st);
        case 6: return launch_small_m<WK, 6>(a, sp, st);
        case 7: return launch_small_m<WK, 7>(a, sp, st);
        case 8: return launch_small_m<WK, 8>(a, sp, st);
        default: return hipErrorInvalidValue;
    }
}

// ---- fused small-M W4A4 linear: plan and launch --------------------------
namespace {
std::atomic<uint32_t> g_fused_next{0};      // round-robin slot of the next launch
std::atomic<int> g_spin_limit{1 << 22};      // polls of the bounded wait

// Steps per loading wave of the fused kernel (7 of the 8 waves load).
int fused_cpw(const SmallPlan& sp) { return (sp.cps / small_ck(WK_W4) + SM_W - 2) / (SM_W - 1); }
}  // namespace

bool fused_small_ok(int kind, int M, int N, int K) {
    if (kind != WK_W4 || M < 1 || M > kSmallMaxM || K > kFusedMaxK || (N & 3) != 0) return false;
    const SmallPlan sp = plan_small(kind, M, N, K);
    if (!sp.use || sp.nblk > kSyncWords) return false;
    // producers and GEMM blocks in one round on the 256 CUs (one block per
    // CU): a GEMM block left for a second round would start only after the
    // first round's blocks, which all wait for the producers, are done
    const int producers = (M + fused_rows_per_block(K) - 1) / fused_rows_per_block(K);
    if (producers + sp.nblk * sp.splits > 256) return false;
    const int cpw = fused_cpw(sp);
    return cpw >= 1 && cpw <= 4 && cpw * small_regs_per_chunk(kind, sp.mt, sp.nt) <= SM_LOAD_REGS;
}

void set_fused_spin_limit(int polls) { g_spin_limit.store(polls < 0 ? 0 : polls); }

hipError_t fused_timeouts(uint32_t* count) {
    return hipMemcpyFromSymbol(count, HIP_SYMBOL(fused_timeout_count), sizeof(uint32_t), 0, hipMemcpyDeviceToHost);
}

template <int MT, int CPW>
static hipError_t launch_fused_c(const GemmArgs& a, const SmallPlan& sp, hipStream_t st) {
    constexpr int NT = small_nt(MT);
    if constexpr (CPW * small_regs_per_chunk(WK_W4, MT, NT) > SM_LOAD_REGS) {
        return hipErrorInvalidValue;            // excluded by fused_small_ok
    } else {
    auto kern = &k_gemm_small<WK_W4, MT, NT, CPW, true>;
    static std::atomic<uint64_t> lds_done;
    hipError_t e = opt_in_lds(reinterpret_cast<const void*>(kern), SM_W * NT * MT * 1024, lds_done);
    if (e != hipSuccess) return e;
    const int acc_mode = a.acc_out != nullptr ? 1 : 0;
    kern<<<dim3(a.fused_producers + sp.nblk, sp.splits), dim3(64 * SM_W), sp.lds, st>>>(a, sp.splits, sp.cps, acc_mode);
    return hipGetLastError();
    }
}

template <int MT>
static hipError_t launch_fused_m(const GemmArgs& a, const SmallPlan& sp, int cpw, hipStream_t st) {
    switch (cpw) {
        case 1: return launch_fused_c<MT, 1>(a, sp, st);
        case 2: return launch_fused_c<MT, 2>(a, sp, st);
        case 3: return launch_fused_c<MT, 3>(a, sp, st);
        case 4: return launch_fused_c<MT, 4>(a, sp, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_small_fused(GemmArgs a, hipStream_t st) {
    if (!fused_small_ok(a.kind, a.M, a.N, a.K) || a.x == nullptr || a.sync == nullptr) return hipErrorInvalidValue;
    const SmallPlan sp = plan_small(WK_W4, a.M, a.N, a.K);
    const int rpb = fused_rows_per_block(a.K);
    a.fused_producers = (a.M + rpb - 1) / rpb;
    a.fused_slot = (int)(g_fused_next.fetch_add(1, std::memory_order_relaxed) % kFusedSlots);
    a.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
    const int cpw = fused_cpw(sp);
    switch (sp.mt) {
        case 1: return launch_fused_m<1>(a, sp, cpw, st);
        case 2: return launch_fused_m<2>(a, sp, cpw, st);
        case 3: return launch_fused_m<3>(a, sp, cpw, st);
        case 4: return launch_fused_m<4>(a, sp, cpw, st);
        case 5: return launch_fused_m<5>(a, sp, cpw, st);
        case 6: return launch_fused_m<6>(a, sp, cpw, st);
        case 7: return launch_fused_m<7>(a, sp, cpw, st);
        case 8: return launch_fused_m<8>(a, sp, cpw, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_small(const GemmArgs& a, const SmallPlan& sp, hipStream_t st) {
    switch (a.kind) {
        case WK_W4: return launch_small_t<WK_W4>(a, sp, st);
        case WK_I8: return launch_small_t<WK_I8>(a, sp, st);
        case WK_W4A8: return launch_small_t<WK_W4A8>(a, sp, st);
        case WK_I8R: return launch_small_t<WK_I8R>(a, sp, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace cr
