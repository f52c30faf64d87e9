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
// sw0: the tensor scale (unused for W4A8, which reads s_channel[n]).
template <int WK, bool ACC>
__device__ __forceinline__ void store4(const Epi& e, int m, int n, float sxm, float sw0, int a0,
                                       int a1, int a2, int a3) {
    const int N = e.N;
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
        if constexpr (WK == WK_W4A8) {
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
                v = v * ((WK == WK_W4A8) ? e.wscale[nn] : sw0);
                if (e.bias != nullptr) v = v + bf16_to_f32(e.bias[nn]);
                e.y[(size_t)m * N + nn] = (uint16_t)f32_to_bf16_rne(v);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Large-M kernel.  Block tile 256 activation rows x 256 weight rows, 8 waves
// (2 along m x 4 along n, 128 x 64 each), 64-k stages in a 4-deep LDS ring.
// Stages are filled with direct-to-LDS loads (global_load_lds_dwordx4: lane i
// of a wave writes its 16 bytes at base + 16 i), issued three stages ahead,
// so no registers hold data in flight.  LDS layouts are XOR-swizzled so the
// MFMA operand reads (ds_read_b128, 16 consecutive lanes = 16 rows) hit 16
// distinct 16-byte bank groups:
//   activations / int8 weights: row r (64 B) at r*64, 16-byte chunk c at
//     slot c ^ ((r >> 2) & 3);
//   packed 4-bit weights: 1 KiB tile of 32 rows, row r half h at slot
//     2r + (h ^ ((r >> 3) & 1)).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lds_ptr;

// global_load_lds_dwordx4 issued from inline asm: the compiler does not see
// it as an LDS write, so it inserts no vmcnt(0) before later LDS reads (the
// stage ring makes them independent); completion is tracked with explicit
// wait_vmcnt<> before the barrier that publishes a stage.  The instruction
// has no register result; M0 (the wave's LDS base) is set in the same block.
__device__ __forceinline__ void lds_dma16(const void* g, void* lds_base) {
    const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr)lds_base);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(l), "v"(g) : "m0");
}

// Raw buffer resource over [base, base + bytes): loads past the end return
// zero without touching memory.  Word 3 selects 32-bit untyped data.
__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    v4i r;
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
    r.z = __builtin_amdgcn_readfirstlane((int)bytes);
    r.w = 0x00020000;
    return r;
}

// buffer_load_dwordx4 ... lds: lane i's 16 bytes at offset voff + soff of the
// resource go to LDS address lds + 16 i (same inline-asm reasoning as
// lds_dma16).
__device__ __forceinline__ void buf_lds16(v4i rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 : : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "m0");
}

template <int V> struct IntC { static constexpr int value = V; };

// Workgroup barrier without the memory fence of __syncthreads(): LDS data
// written by this workgroup's direct-to-LDS loads is published by waiting
// for them (wait_vmcnt) before the barrier.  The "memory" clobber keeps the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt vmcnt(N) (N < 64), other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

constexpr int BIG_BM = 256;
constexpr int BIG_WM = 2;   // waves along m in the large-M kernel (wave tile 128 x 64)

// NW waves (2 along m x NW/2 along n; wave tile 128 x 512/NW), block tile
// 256 x 256, NS-stage LDS ring.
template <int WK, int NW, int NS>
struct BigCfg {
    static constexpr int BN = 256;
    static constexpr int TPW = 8 / NW;                                 // 32-row weight tiles loaded per wave
    static constexpr int A_BYTES = BIG_BM * 64;                       // activations per stage
    static constexpr int B_BYTES = WK == WK_I8 ? BN * 64 : BN * 32;
    static constexpr int C_BYTES = WK == WK_W4A8 ? BN * 4 : 0;        // W4A8 scale codes
    static constexpr int STAGE = A_BYTES + B_BYTES + C_BYTES;
    static constexpr int LA = 16 / NW;                                 // activation loads per wave
    // direct-to-LDS loads per wave per stage
    static constexpr int LPS = LA + TPW * (WK == WK_I8 ? 2 : 1) + (WK == WK_W4A8 ? 1 : 0);
    static constexpr size_t LDS = (size_t)NS * STAGE + (WK == WK_W4A8 ? 4096 : 0);
};

template <int WK, int NW, int NS, bool ACC>
__global__ void __launch_bounds__(64 * NW) k_gemm_big(GemmArgs p, int tiles_m, int tiles_n) {
    using C = BigCfg<WK, NW, NS>;
    constexpr int BN = C::BN;
    // WM waves along m, NW/WM along n; wave tile (256/WM) x (256*WM/NW)
    constexpr int WM = BIG_WM, WNW = NW / WM;
    constexpr int WROWS = BIG_BM / WM;
    constexpr int FM = WROWS / 32, FN = 8 / WNW;
    extern __shared__ __attribute__((aligned(16))) int8_t smem[];
    int8_t* ring = smem;
    uint4* sT = reinterpret_cast<uint4*>(smem + NS * C::STAGE);   // W4A8 decode table

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
    const int wm = wave % WM, wn = wave / WM;
    const int h = lane >> 5, l32 = lane & 31;

    const int M = p.M, Kp = p.Kp;
    const int nkc = Kp >> 6;
    const int nbmax = (p.Np >> 5) - 1;
    const size_t codes_off = w4a8_codes_offset(p.N, p.K);
    if constexpr (WK == WK_W4A8) {
        const uint4* tg = reinterpret_cast<const uint4*>(p.wp + w4a8_table_offset(p.N, p.K));
        for (int i = tid; i < 256; i += 64 * NW) sT[i] = tg[i];
        __syncthreads();
    }

    // Persistent blocks: block b handles tiles b, b + G, b + 2G, ...  Blocks
    // are dealt to the 8 XCDs round-robin, so within each round the blocks
    // of one XCD take a contiguous run of tile ids (bands of 8 tile-rows),
    // which keeps the operands they share in that XCD's L2.
    const int total = tiles_m * tiles_n;
    const int G = gridDim.x, bid = blockIdx.x;
    // slot: a permutation of 0..G-1; tile id j*G + slot for round j, so every
    // tile id below `total` belongs to exactly one (block, round)
    const int slot = (G & 7) == 0 ? (bid & 7) * (G >> 3) + (bid >> 3) : bid;
    const int my_tiles = (total - slot + G - 1) / G;
    const int total_stages = my_tiles * nkc;
    auto tile_origin = [&](int j, int& m0, int& n0) {
        int lid = j * G + slot;
        if (lid >= total) lid = total - 1;           // only for the clamped tail re-reads
        constexpr int GM = 8;
        const int band = lid / (GM * tiles_n);
        const int first_m = band * GM;
        const int gm = min(tiles_m - first_m, GM);
        const int in_band = lid - band * GM * tiles_n;
        m0 = (first_m + in_band % gm) * BIG_BM;
        n0 = (in_band / gm) * BN;
    };

    // --- stage loads: buffer loads straight to LDS --------------------------
    // Per tile, one buffer resource per operand starts at the tile's first
    // row; per lane the offset inside a stage is fixed, and the stage's k
    // offset goes in the scalar offset.  Rows past M (activations) and tiles
    // past Np (weights) are outside the resource and load as zero.
    //   activations: rows 16*(LA*wave + j) + lane/4, chunk (lane%4) ^ swizzle
    //   weights: tile n0/32 + wave, this lane's row and half (swizzled)
    constexpr int BSTEP = WK == WK_I8 ? 2048 : 1024;
    uint32_t a_voff[C::LA];
#pragma unroll
    for (int j = 0; j < C::LA; ++j) {
        const int row = 16 * (C::LA * wave + j) + (lane >> 2);
        a_voff[j] = (uint32_t)(row * Kp + (((lane & 3) ^ ((row >> 2) & 3)) * 16));
    }
    uint32_t b_voff[C::TPW][2];
#pragma unroll
    for (int t = 0; t < C::TPW; ++t) {
        const uint32_t tb = (uint32_t)((wave * C::TPW + t) * nkc * BSTEP);
        if constexpr (WK == WK_I8) {
            const int row0 = lane >> 2, row1 = row0 + 16;
            b_voff[t][0] = tb + row0 * 64 + (((lane & 3) ^ ((row0 >> 2) & 3)) * 16);
            b_voff[t][1] = tb + row1 * 64 + (((lane & 3) ^ ((row1 >> 2) & 3)) * 16);
        } else {
            b_voff[t][0] = tb + (lane >> 1) * 32 + (((lane & 1) ^ ((lane >> 4) & 1)) * 16);
            b_voff[t][1] = b_voff[t][0];
        }
    }
    const uint32_t c_voff = (uint32_t)((wave * C::TPW + (lane >> 3)) * nkc * 128 + (lane & 7) * 16);
    const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_ptr)ring;
    v4i rs_a, rs_b, rs_c;
    uint32_t soff_a = 0, soff_b = 0, soff_c = 0;
    int is_tile = 0, is_kc = 0;   // issue cursor
    auto aim = [&](int j) {       // resources of tile j, stage 0
        int m0, n0;
        tile_origin(j, m0, n0);
        rs_a = make_rsrc(p.qx + (size_t)m0 * Kp, (uint32_t)((size_t)(M - m0) * Kp));
        const int nb0 = n0 >> 5;
        const size_t tiles_left = (size_t)(nbmax + 1 - nb0);
        rs_b = make_rsrc(p.wp + (size_t)nb0 * nkc * BSTEP, (uint32_t)(tiles_left * nkc * BSTEP));
        if constexpr (WK == WK_W4A8)
            rs_c = make_rsrc(p.wp + codes_off + (size_t)nb0 * nkc * 128, (uint32_t)(tiles_left * nkc * 128));
        soff_a = 0; soff_b = 0; soff_c = 0;
    };
    aim(0);
    auto issue_stage = [&](auto BUF) {
        constexpr int buf = decltype(BUF)::value;
        const uint32_t st = ring_lds + buf * C::STAGE;
#pragma unroll
        for (int j = 0; j < C::LA; ++j) buf_lds16(rs_a, a_voff[j], soff_a, st + 16 * (C::LA * wave + j) * 64);
        const uint32_t sb = st + C::A_BYTES;
#pragma unroll
        for (int t = 0; t < C::TPW; ++t) {
            const uint32_t dst = sb + (wave * C::TPW + t) * BSTEP;
            buf_lds16(rs_b, b_voff[t][0], soff_b, dst);
            if constexpr (WK == WK_I8) buf_lds16(rs_b, b_voff[t][1], soff_b, dst + 1024);
        }
        if constexpr (WK == WK_W4A8) {
            if (lane < 8 * C::TPW) buf_lds16(rs_c, c_voff, soff_c, st + C::A_BYTES + C::B_BYTES + wave * C::TPW * 128);
        }
        // advance (past the last stage the offsets stay put: the tail
        // re-reads it into a buffer that is never consumed)
        if (++is_kc < nkc) {
            soff_a += 64; soff_b += BSTEP; soff_c += 128;
        } else if (is_tile + 1 < my_tiles) {
            ++is_tile;
            is_kc = 0;
            aim(is_tile);
        } else {
            is_kc = nkc;
        }
    };

    v16i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][f][r] = 0;

    // per-lane LDS read offsets
    const int swz = (l32 >> 2) & 3;                 // activation row swizzle (row % 32 == l32)
    int aoff[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) aoff[t] = (wm * WROWS + l32) * 64 + (((2 * t + h) ^ swz) * 16);
    int boff[FN];
#pragma unroll
    for (int f = 0; f < FN; ++f) {
        const int tile = wn * FN + f;
        if constexpr (WK == WK_I8) boff[f] = tile * 2048 + l32 * 64;
        else boff[f] = tile * 1024 + (2 * l32 + (h ^ ((l32 >> 3) & 1))) * 16;
    }

    // Weight operand bytes of one stage (both MFMA steps) and their decode.
    struct WStage { uint4 a, b; uint32_t codes; };
    auto read_w = [&](const int8_t* st, int f) -> WStage {
        WStage w;
        const int8_t* sb = st + C::A_BYTES;
        if constexpr (WK == WK_I8) {
            w.a = *reinterpret_cast<const uint4*>(sb + boff[f] + (((2 * h + 0) ^ swz) * 16));
            w.b = *reinterpret_cast<const uint4*>(sb + boff[f] + (((2 * h + 1) ^ swz) * 16));
        } else {
            w.a = *reinterpret_cast<const uint4*>(sb + boff[f]);
        }
        if constexpr (WK == WK_W4A8)
            w.codes = *reinterpret_cast<const uint32_t*>(st + C::A_BYTES + C::B_BYTES + (wn * FN + f) * 128 + l32 * 4);
        return w;
    };
    auto wop = [&](const WStage& w, int t) -> v4i {
        if constexpr (WK == WK_I8) {
            const uint4 v = t == 0 ? w.a : w.b;
            v4i r;
            r.x = (int)v.x; r.y = (int)v.y; r.z = (int)v.z; r.w = (int)v.w;
            return r;
        } else if constexpr (WK == WK_W4) {
            return t == 0 ? unpack_w4x16(w.a.x, w.a.y) : unpack_w4x16(w.a.z, w.a.w);
        } else {
            const uint4 tr = sT[(w.codes >> (8 * (2 * t + h))) & 0xFF];
            return t == 0 ? decode_w4a8(w.a.x, w.a.y, tr) : decode_w4a8(w.a.z, w.a.w, tr);
        }
    };
    auto read_a = [&](const int8_t* st, int t, v4i (&af)[FM]) {
#pragma unroll
        for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const v4i*>(st + aoff[t] + i * 32 * 64);
    };

    const Epi epi = make_epi(p);
    const float sw0 = (WK == WK_W4A8 || ACC) ? 0.0f : p.wscale[0];

    // Pipeline over the block's whole stage stream (its tiles back to back):
    // stage s lives in ring buffer s % NS and is loaded NS-1 stages ahead.
    // Inside a stage the fragments of the second MFMA step are read while the
    // first step's MFMAs run, and the next stage's first-step fragments while
    // the second step's MFMAs run; a buffer is refilled only after the
    // barrier that follows the last read of it by every wave.
    static_assert(NS == 4 || NS == 6, "ring depth (even: register sets alternate per stage)");
    // Fragments of one stage: activation operands of both MFMA steps and the
    // weight bytes.  Two sets alternate: while the MFMAs of stage s run from
    // one set, the reads of stage s+1 land in the other.
    struct Frags { v4i a[2][FM]; WStage w[FN]; };
    auto read_frags = [&](const int8_t* st, Frags& F) {
        read_a(st, 0, F.a[0]);
        read_a(st, 1, F.a[1]);
#pragma unroll
        for (int f = 0; f < FN; ++f) F.w[f] = read_w(st, f);
    };
    issue_stage(IntC<0>{});
    issue_stage(IntC<1>{});
    issue_stage(IntC<2>{});
    if constexpr (NS > 4) { issue_stage(IntC<3>{}); issue_stage(IntC<4>{}); }
    wait_vmcnt<(NS - 2) * C::LPS>();
    lds_barrier();
    Frags F0, F1;
    read_frags(ring, F0);

    int cur_tile = 0, kc = 0;
    // One stage in buffer B: publish stage B+1 (and free the buffer of the
    // previous stage), refill it, read the next stage's fragments into the
    // other register set, then run this stage's 16 MFMAs back to back.
    auto step = [&](auto BUF) {
        constexpr int B = decltype(BUF)::value;
        Frags& cur = (B & 1) ? F1 : F0;
        Frags& nxt = (B & 1) ? F0 : F1;
        wait_vmcnt<(NS - 3) * C::LPS>();
        lds_barrier();
        issue_stage(IntC<(B + NS - 1) % NS>{});
        read_frags(ring + ((B + 1) % NS) * C::STAGE, nxt);
        __builtin_amdgcn_sched_barrier(0);   // the next stage's reads go out before the MFMAs
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            v4i bt[FN];
#pragma unroll
            for (int f = 0; f < FN; ++f) bt[f] = wop(cur.w[f], t);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int f = 0; f < FN; ++f) acc[i][f] = mfma32(bt[f], cur.a[t][i], acc[i][f]);
        }

        if (++kc == nkc) {
            // Tile done: epilogue while the next tile's stages are in flight.
            int m0, n0;
            tile_origin(cur_tile, m0, n0);
            const bool full = m0 + BIG_BM <= M && n0 + BN <= p.N && (p.N & 3) == 0;
            if (full && !ACC) {
                // All epilogue operands are loaded up front (one wait), then
                // every output quad is converted and stored without checks.
                float sxv[FM];
#pragma unroll
                for (int i = 0; i < FM; ++i) sxv[i] = p.sx[m0 + wm * WROWS + i * 32 + l32];
#pragma unroll
                for (int f = 0; f < FN; ++f) {
                    uint2 bv[4];
                    float4 cv[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int n = n0 + (wn * FN + f) * 32 + 4 * h + 8 * q;
                        bv[q] = p.bias != nullptr ? *reinterpret_cast<const uint2*>(p.bias + n) : make_uint2(0u, 0u);
                        if constexpr (WK == WK_W4A8) cv[q] = *reinterpret_cast<const float4*>(p.wscale + n);
                        else cv[q] = make_float4(sw0, sw0, sw0, sw0);
                    }
#pragma unroll
                    for (int i = 0; i < FM; ++i) {
                        const int m = m0 + wm * WROWS + i * 32 + l32;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int n = n0 + (wn * FN + f) * 32 + 4 * h + 8 * q;
                            const float c[4] = {cv[q].x, cv[q].y, cv[q].z, cv[q].w};
                            const float b[4] = {bf16_lo(bv[q].x), bf16_hi(bv[q].x), bf16_lo(bv[q].y), bf16_hi(bv[q].y)};
                            float v[4];
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                v[j] = (float)fix_acc<WK>(acc[i][f][4 * q + j]) * sxv[i];
                                v[j] = v[j] * c[j];
                                if (p.bias != nullptr) v[j] = v[j] + b[j];
                            }
                            *reinterpret_cast<uint2*>(p.y + (size_t)m * p.N + n) =
                                make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                        }
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int m = m0 + wm * WROWS + i * 32 + l32;
                    if (m < M) {
                        const float sxm = ACC ? 0.0f : p.sx[m];
#pragma unroll
                        for (int f = 0; f < FN; ++f) {
                            const int nbase = n0 + (wn * FN + f) * 32 + 4 * h;
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const int n = nbase + 8 * q;
                                if (n < p.N)
                                    store4<WK, ACC>(epi, m, n, sxm, sw0, fix_acc<WK>(acc[i][f][4 * q + 0]),
                                                    fix_acc<WK>(acc[i][f][4 * q + 1]),
                                                    fix_acc<WK>(acc[i][f][4 * q + 2]),
                                                    fix_acc<WK>(acc[i][f][4 * q + 3]));
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int f = 0; f < FN; ++f)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][f][r] = 0;
            kc = 0;
            ++cur_tile;
        }
    };
    for (int gs = 0; gs < total_stages; gs += NS) {
        step(IntC<0>{});
        if (gs + 1 >= total_stages) break;
        step(IntC<1>{});
        if (gs + 2 >= total_stages) break;
        step(IntC<2>{});
        if (gs + 3 >= total_stages) break;
        step(IntC<3>{});
        if constexpr (NS > 4) {
            if (gs + 4 >= total_stages) break;
            step(IntC<4 % NS>{});
            if (gs + 5 >= total_stages) break;
            step(IntC<5 % NS>{});
        }
    }
    wait_vmcnt<0>();
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
    const float sw0 = (WK == WK_W4A8 || ACC) ? 0.0f : p.wscale[0];
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
                        store4<WK, ACC>(epi, m, n, sxm, sw0, fix_acc<WK>(acc[i][4 * q]), fix_acc<WK>(acc[i][4 * q + 1]),
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
    const float sw0 = (WK == WK_W4A8 || ACC) ? 0.0f : p.wscale[0];
    const float sxm = ACC ? 0.0f : p.sx[m];
    store4<WK, ACC>(epi, m, n, sxm, sw0, fix_acc<WK>(a.x), fix_acc<WK>(a.y), fix_acc<WK>(a.z), fix_acc<WK>(a.w));
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

// Large-M configuration: 8 waves (block tile 256 x 256), one persistent block
// per CU; ring depth 6 for 4-bit weights (144 KiB of LDS; W4A8 154 KiB with
// its table), 4 for int8 weights (128 KiB).
constexpr int BIG_NW = 8;
template <int WK> constexpr int big_stages() { return WK == WK_I8 ? 4 : 6; }

// Compute units of the current device (cached per device).
static int num_cus() {
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

template <int WK, bool ACC>
static hipError_t launch_big_t(const GemmArgs& a, hipStream_t st) {
    constexpr int NS = big_stages<WK>();
    using C = BigCfg<WK, BIG_NW, NS>;
    const int tiles_m = (a.M + BIG_BM - 1) / BIG_BM, tiles_n = (a.N + C::BN - 1) / C::BN;
    static bool attr_set = false;   // opt in to more than 64 KiB of dynamic LDS (once per process)
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_big<WK, BIG_NW, NS, ACC>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int grid = min(tiles_m * tiles_n, num_cus());
    k_gemm_big<WK, BIG_NW, NS, ACC><<<dim3(grid), dim3(64 * BIG_NW), C::LDS, st>>>(a, tiles_m, tiles_n);
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
