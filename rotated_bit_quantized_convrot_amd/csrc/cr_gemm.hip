// Integer GEMM + rank-one epilogue on v_mfma_i32_32x32x32_i8.
//
// acc[m,n] = sum_k qx[m,k] * qw[n,k] (exact int32), then
// y[m,n] = bf16(fl(fl(float(acc) * s_x[m]) * s_w) + bias[n])
// ([QIE] model card, "Speed" table: one kernel for the rotation, the s4 MMA and the rank-one rescale;
// [REB] "Why W4A8 instead of GGUF": the W4A8 weights stay 4-bit in memory and
// the math is int8).  CDNA4 has no int4 MFMA, so 4-bit codes are widened to
// int8 in registers: W4A4 weights and activations by one AND per dword (two
// nibble forms, exact after the epilogue's integer correction), W4A8 indices
// through a per-group 16-entry table row.
//
// MFMA operand roles: the weight fragment is the A operand (32 rows = n) and
// the activation fragment the B operand (32 columns = m).  Lane l supplies,
// for both, row/column l%32 and the 16 k values 16*(l/32)+0..15 of the step;
// the 32x32 int32 result leaves lane l with column m = l%32 and rows
// n = 8*(r/4) + 4*(l/32) + r%4 for accumulator register r.
#include "cr_device.h"
#include "cr_epilogue.h"
#include "cr_internal.h"

#include <cmath>
#include <type_traits>

namespace cr {

// ---------------------------------------------------------------------------
// Large-M kernel.  Block tile 256 activation rows x 256 weight rows, 8 waves
// (2 along m x 4 along n, 128 x 64 each), 64-k stages in an NS-deep LDS ring.
// Stages are filled with direct-to-LDS buffer loads (lane i of a wave writes
// its 16 bytes at base + 16 i), issued NS - 1 stages ahead, so no registers
// hold data in flight.  When the output has too few tiles to fill the chip,
// the K range of every tile is split into equal slices taken by different
// blocks, which store int32 partial tiles; a second kernel adds them and runs
// the epilogue.  W4A4 activations arrive as 4-bit tiles (rows = m) and go
// through LDS like the weights; both operands are widened by one AND per
// dword (nibble forms in cr_internal.h) and the epilogue corrects the sums.  LDS layouts are XOR-swizzled so the
// MFMA operand reads (ds_read_b128, 16 consecutive lanes = 16 rows) hit 16
// distinct 16-byte bank groups:
//   activations / int8 weights: row r (64 B) at r*64, 16-byte chunk c at
//     slot c ^ ((r >> 2) & 3);
//   packed 4-bit weights: 1 KiB tile of 32 rows, row r half h at slot
//     2r + (h ^ ((r >> 3) & 1)).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lds_ptr;

// Byte count of a buffer resource (32 bits; a block never reaches past 4 GiB
// from the base of its resources).
__host__ __device__ __forceinline__ uint32_t clamp_u32(size_t v) { return v > 0xFFFFFFFFu ? 0xFFFFFFFFu : (uint32_t)v; }

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
// resource go to LDS address lds + 16 i.  Issued from inline asm, the load is
// not seen by the compiler as an LDS write, so it neither inserts waits for it
// before later LDS reads nor orders those reads after it (the stage ring
// makes them independent); completion is tracked with explicit wait_vmcnt<>
// before the barrier that publishes a stage.  The instruction has no register
// result.  The LDS address goes in M0 through an input operand bound to that
// register, so the compiler itself sets M0 and knows its value.
// (The compiler's direct-to-LDS buffer-load builtin gives the same
// instruction, but with it the int8-weight kernels need ~40 more VGPRs and
// spill at 256-wide tiles.)
__device__ __forceinline__ void buf_lds16(v4i rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" : : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds));
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

// Origin of output tile `lid` (0 .. tiles_m * tiles_n - 1) of width bn: tiles
// are taken in bands of 8 tile-rows, column by column inside a band, so that
// consecutive ids share weight columns and activation rows.
__device__ __forceinline__ void big_tile_origin(int lid, int tiles_m, int tiles_n, int bn, int& m0, int& n0) {
    constexpr int GM = 8;
    const int band = lid / (GM * tiles_n);
    const int first_m = band * GM;
    const int gm = min(tiles_m - first_m, GM);
    const int in_band = lid - band * GM * tiles_n;
    m0 = (first_m + in_band % gm) * BIG_BM;
    n0 = (in_band / gm) * bn;
}

// 8 waves, block tile 256 (m) x BN (n), NS-stage LDS ring.  BN = 256: 2
// waves along m x 4 along n, wave tile 128 x 64; BN = 192 (fills the chip
// where 256-wide tiles leave CUs idle): 4 x 2, wave tile 64 x 96; BN = 128
// (layers with few output tiles): 4 x 2, wave tile 64 x 64; BN = 64 (fewer
// still): 4 x 2, wave tile 64 x 32.
template <int WK, int NW, int NS, int BN_>
struct BigCfg {
    static_assert(NW == 8, "8 waves");
    static_assert(BN_ == 256 || BN_ == 192 || BN_ == 128 || BN_ == 64, "block tile width");
    static constexpr int BN = BN_;
    static constexpr int NWT = BN / 32;                                // 32-row weight tiles per stage
    static constexpr int WM = BN == 256 ? 2 : 4;                       // waves along m
    static constexpr int WNW = NW / WM;                                // waves along n
    static constexpr int WROWS = BIG_BM / WM, FM = WROWS / 32, FN = NWT / WNW;
    static constexpr bool PA = WK == WK_W4;                            // 4-bit activation tiles
    static constexpr int BSTEP = wk_i8w(WK) ? 2048 : 1024;             // bytes of a weight tile's stage
    static constexpr int A_BYTES = PA ? BIG_BM * 32 : BIG_BM * 64;    // activations per stage
    static constexpr int B_BYTES = NWT * BSTEP;
    static constexpr int C_BYTES = WK == WK_W4A8 ? NWT * 128 : 0;     // W4A8 scale codes
    static constexpr int STAGE = A_BYTES + B_BYTES + C_BYTES;
    // Direct-to-LDS loads per wave per stage: each wave fills one NW-th of
    // every operand's region, 1 KiB (64 lanes x 16 B) per load, the last one
    // with fewer lanes where its share is not a whole KiB.
    static constexpr int LA = A_BYTES / (NW * 1024);
    static constexpr int WB = B_BYTES / NW, LW = (WB + 1023) / 1024;
    static constexpr int CB = C_BYTES / NW;
    static constexpr int LPS = LA + LW + (WK == WK_W4A8 ? 1 : 0);
    // LDS-staged epilogue: per wave 32 rows of EPI_TR bytes, then its FN * 32
    // columns' bias (fp32), scale (fp32) and (W4A4) weight correction (int32)
    static constexpr int EPI_TR = 80;
    static constexpr int EPI_OPB = FN * 32 * (4 + 4 + (PA ? 4 : 0));
    static constexpr int EPI_BYTES = NW * (32 * EPI_TR + EPI_OPB);
    // W4A4 stages are too small to hold it: its own region after the ring.
    // int8 operands: in the ring buffer of the stage just consumed, or (64-wide
    // tiles, whose stage holds the staging rows only) the rows there and the
    // column operands in a region after the ring.
    static constexpr bool EPI_OPS_IN_RING = !PA && EPI_BYTES <= STAGE;
    static constexpr size_t EPI_OFF = (size_t)NS * STAGE;
    static constexpr size_t LDS = (size_t)NS * STAGE + (WK == WK_W4A8 ? 4096 : 0) +
                                  (PA ? EPI_BYTES : (EPI_OPS_IN_RING ? 0 : NW * EPI_OPB));
    static_assert(A_BYTES % (NW * 1024) == 0 && WB % 16 == 0 && CB % 16 == 0 && CB <= 1024, "load split");
};

// SPLIT: units are K slices whose int32 sums go to partial tiles (splits > 1);
// otherwise every unit is a whole tile and splits == 1.
template <int WK, int NW, int NS, int BN_, bool ACC, bool SPLIT>
__global__ void __launch_bounds__(64 * NW) k_gemm_big(GemmArgs p, int tiles_m, int tiles_n, int splits, int cps) {
    using C = BigCfg<WK, NW, NS, BN_>;
    constexpr int BN = C::BN;
    constexpr int WM = C::WM, WROWS = C::WROWS, FM = C::FM, FN = C::FN;
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

    // Persistent blocks: block b handles work units b, b + G, b + 2G, ...
    // A unit is one K slice (cps 64-k chunks) of one output tile; unit id
    // s * total + tile, so with one slice units are tiles.  Blocks are dealt
    // to the 8 XCDs round-robin, so within each round the blocks of one XCD
    // take a contiguous run of unit ids, which keeps the operands they share
    // in that XCD's L2.
    const int total = tiles_m * tiles_n;
    const int units = total * splits;
    const int G = gridDim.x, bid = blockIdx.x;
    // slot: a permutation of 0..G-1; unit id j*G + slot for round j, so every
    // unit id below `units` belongs to exactly one (block, round)
    const int slot = (G & 7) == 0 ? (bid & 7) * (G >> 3) + (bid >> 3) : bid;
    const int my_tiles = (units - slot + G - 1) / G;
    const int total_stages = my_tiles * cps;
    auto tile_origin = [&](int j, int& m0, int& n0, int& kc0, int& uid) {
        int lid = j * G + slot;
        if (lid >= units) lid = units - 1;           // only for the clamped tail re-reads
        const int sl = SPLIT ? lid / total : 0;
        big_tile_origin(lid - sl * total, tiles_m, tiles_n, BN, m0, n0);
        kc0 = sl * cps;
        uid = lid;
    };

    // --- stage loads: buffer loads straight to LDS --------------------------
    // Per tile, one buffer resource per operand starts at the tile's first
    // row; per lane the offset inside a stage is fixed, and the stage's k
    // offset goes in the scalar offset.  Rows past M (activations) and tiles
    // past Np (weights) are outside the resource and load as zero.
    //   activations: rows 16*(LA*wave + j) + lane/4, chunk (lane%4) ^ swizzle
    //   weights: tile n0/32 + wave, this lane's row and half (swizzled)
    constexpr int BSTEP = C::BSTEP;
    //   4-bit activations: 32-row tile `wave` of the block, like the weights
    static_assert(!C::PA || C::LA == 1, "one 4-bit activation tile per wave");
    constexpr int ASTEP = C::PA ? 1024 : 64;                    // activation bytes per 64-k step
    uint32_t a_voff[C::LA];
#pragma unroll
    for (int j = 0; j < C::LA; ++j) {
        if constexpr (C::PA) {
            a_voff[j] = (uint32_t)(wave * nkc * 1024 + (lane >> 1) * 32 + (((lane & 1) ^ ((lane >> 4) & 1)) * 16));
        } else {
            const int row = 16 * (C::LA * wave + j) + (lane >> 2);
            a_voff[j] = (uint32_t)(row * Kp + (((lane & 3) ^ ((row >> 2) & 3)) * 16));
        }
    }
    // weights / W4A8 codes: LDS byte o of the operand's stage region (this
    // wave's share starts at wave * WB) comes from weight tile o / BSTEP of the
    // block and, inside it, the swizzled position of slot (o % BSTEP) / 16
    uint32_t b_voff[C::LW];
#pragma unroll
    for (int j = 0; j < C::LW; ++j) {
        const int o = wave * C::WB + j * 1024 + lane * 16;
        const int t = o / BSTEP, sl = (o % BSTEP) >> 4;
        int src;
        if constexpr (wk_i8w(WK)) {
            const int r = sl >> 2;
            src = r * 64 + (((sl & 3) ^ ((r >> 2) & 3)) * 16);
        } else {
            const int r = sl >> 1;
            src = r * 32 + (((sl & 1) ^ ((r >> 3) & 1)) * 16);
        }
        b_voff[j] = (uint32_t)(t * nkc * BSTEP + src);
    }
    uint32_t c_voff = 0;
    if constexpr (WK == WK_W4A8) {
        const int o = wave * C::CB + lane * 16;
        c_voff = (uint32_t)((o / 128) * nkc * 128 + (o % 128));
    }
    const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_ptr)ring;
    v4i rs_a, rs_b, rs_c;
    uint32_t soff_a = 0, soff_b = 0, soff_c = 0;
    int is_tile = 0, is_kc = 0;   // issue cursor
    auto aim = [&](int j) {       // resources of unit j's tile, its first stage
        int m0, n0, kc0, uid;
        tile_origin(j, m0, n0, kc0, uid);
        if constexpr (C::PA)
            rs_a = make_rsrc(p.qx + (size_t)(m0 >> 5) * nkc * 1024,
                             clamp_u32((size_t)((round_up(M, 32) - m0) >> 5) * nkc * 1024));
        else
            rs_a = make_rsrc(p.qx + (size_t)m0 * Kp, clamp_u32((size_t)(M - m0) * Kp));
        const int nb0 = n0 >> 5;
        const size_t tiles_left = (size_t)(nbmax + 1 - nb0);
        rs_b = make_rsrc(p.wp + (size_t)nb0 * nkc * BSTEP, clamp_u32(tiles_left * nkc * BSTEP));
        if constexpr (WK == WK_W4A8)
            rs_c = make_rsrc(p.wp + codes_off + (size_t)nb0 * nkc * 128, clamp_u32(tiles_left * nkc * 128));
        soff_a = (uint32_t)kc0 * ASTEP; soff_b = (uint32_t)kc0 * BSTEP; soff_c = (uint32_t)kc0 * 128;
    };
    aim(0);
    auto issue_stage = [&](auto BUF) {
        constexpr int buf = decltype(BUF)::value;
        const uint32_t st = ring_lds + buf * C::STAGE;
#pragma unroll
        for (int j = 0; j < C::LA; ++j)
            buf_lds16(rs_a, a_voff[j], soff_a, st + (C::PA ? wave * 1024 : 16 * (C::LA * wave + j) * 64));
        const uint32_t sb = st + C::A_BYTES + wave * C::WB;
#pragma unroll
        for (int j = 0; j < C::LW; ++j) {
            if (C::WB % 1024 == 0 || j + 1 < C::LW || lane < (C::WB % 1024) / 16)
                buf_lds16(rs_b, b_voff[j], soff_b, sb + j * 1024);
        }
        if constexpr (WK == WK_W4A8) {
            if (lane < C::CB / 16) buf_lds16(rs_c, c_voff, soff_c, st + C::A_BYTES + C::B_BYTES + wave * C::CB);
        }
        // advance (past the last stage the offsets stay put: the tail
        // re-reads it into a buffer that is never consumed)
        if (++is_kc < cps) {
            soff_a += ASTEP; soff_b += BSTEP; soff_c += 128;
        } else if (is_tile + 1 < my_tiles) {
            ++is_tile;
            is_kc = 0;
            aim(is_tile);
        } else {
            is_kc = cps;
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
    // 4-bit activations: 32-row tile wm * FM + i, this lane's row and half
    const int apoff = wm * FM * 1024 + (2 * l32 + (h ^ ((l32 >> 3) & 1))) * 16;
    int boff[FN];
#pragma unroll
    for (int f = 0; f < FN; ++f) {
        const int tile = wn * FN + f;
        if constexpr (wk_i8w(WK)) boff[f] = tile * 2048 + l32 * 64;
        else boff[f] = tile * 1024 + (2 * l32 + (h ^ ((l32 >> 3) & 1))) * 16;
    }

    // Weight operand bytes of one stage (both MFMA steps) and their decode.
    struct WStage { uint4 a, b; uint32_t codes; };
    auto read_w = [&](const int8_t* st, int f) -> WStage {
        WStage w;
        const int8_t* sb = st + C::A_BYTES;
        if constexpr (wk_i8w(WK)) {
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
        if constexpr (wk_i8w(WK)) {
            const uint4 v = t == 0 ? w.a : w.b;
            v4i r;
            r.x = (int)v.x; r.y = (int)v.y; r.z = (int)v.z; r.w = (int)v.w;
            return r;
        } else if constexpr (WK == WK_W4) {
            return t == 0 ? unpack_wt4(w.a.x, w.a.y) : unpack_wt4(w.a.z, w.a.w);
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

    // Pipeline over the block's whole stage stream (its tiles back to back):
    // stage s lives in ring buffer s % NS and is loaded NS-1 stages ahead.
    // Inside a stage the fragments of the second MFMA step are read while the
    // first step's MFMAs run, and the next stage's first-step fragments while
    // the second step's MFMAs run; a buffer is refilled only after the
    // barrier that follows the last read of it by every wave.
    static_assert(NS == 4 || NS == 6, "ring depth (even: register sets alternate per stage)");
    // Fragments of one stage: activation operands of both MFMA steps (int8)
    // or the activation bytes (4-bit), and the weight bytes.  Two sets
    // alternate: while the MFMAs of stage s run from one set, the reads of
    // stage s+1 land in the other.
    struct AI8 { v4i a[2][FM]; };
    struct AP4 { uint4 r[FM]; };
    struct Frags { typename std::conditional<C::PA, AP4, AI8>::type a; WStage w[FN]; };
    auto read_frags = [&](const int8_t* st, Frags& F) {
        if constexpr (C::PA) {
#pragma unroll
            for (int i = 0; i < FM; ++i) F.a.r[i] = *reinterpret_cast<const uint4*>(st + apoff + i * 1024);
        } else {
            read_a(st, 0, F.a.a[0]);
            read_a(st, 1, F.a.a[1]);
        }
#pragma unroll
        for (int f = 0; f < FN; ++f) F.w[f] = read_w(st, f);
    };
    auto aop = [&](const Frags& F, int t, int i) -> v4i {
        if constexpr (C::PA)
            return t == 0 ? unpack_act4(F.a.r[i].x, F.a.r[i].y) : unpack_act4(F.a.r[i].z, F.a.r[i].w);
        else
            return F.a.a[t][i];
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
    // PAIR (rings of 6 or more): stages go in pairs with one barrier; an
    // even step publishes stages B+1 and B+2 and refills the buffers of B-1
    // and B, whose fragments every wave has read before that barrier.  The
    // refills are issued among the step's MFMAs (PAIR: after the first and
    // the second half of them; otherwise the one refill after the first
    // half): issued right after the barrier they held back the first MFMA by
    // ~570 cycles per stage pair (the loads' scalar set-up and issue), with
    // the MFMA pipe idle meanwhile (DiT W1 121.8 -> 116.8 us, W2 115.2 ->
    // 106.5 us; int8_tensorwise K=2688 38.3 -> 36.5 us).
    constexpr bool PAIR = NS >= 6;
    auto step = [&](auto BUF) {
        constexpr int B = decltype(BUF)::value;
        Frags& cur = (B & 1) ? F1 : F0;
        Frags& nxt = (B & 1) ? F0 : F1;
        if constexpr (!PAIR) {
            wait_vmcnt<(NS - 3) * C::LPS>();
            lds_barrier();
        } else if constexpr ((B & 1) == 0) {
            wait_vmcnt<(NS - 4) * C::LPS>();
            lds_barrier();
        }
        constexpr bool ISS = PAIR && (B & 1) == 0;       // this step refills two buffers
        constexpr int NMF = 2 * FM * FN;                  // MFMAs of the step
        constexpr int N1 = NMF / 2, N2 = NMF;             // refills after these many
        // W4A8: the last stage of a tile reads the next stage's fragments
        // after the epilogue instead (fewer registers live across it; the
        // other formats have them to spare and keep the plain schedule).
        constexpr bool DEFER = WK == WK_W4A8;
        // The next stage's fragment reads: before the MFMAs (W4A4), or after
        // the first four of them (int8 operands, twice the bytes per read:
        // W4A8 178.8 -> 173.8 us, int8_tensorwise K=2688 34.5 -> 33.7 us; for
        // W4A4 it measured slower)
        constexpr bool READ_LATE = !C::PA;
        if constexpr (!READ_LATE) {
            if (!DEFER || kc + 1 != cps) read_frags(ring + ((B + 1) % NS) * C::STAGE, nxt);
        }
        __builtin_amdgcn_sched_barrier(0);
        // W4A8: the table decode makes the MFMA block VALU-heavy; a raised
        // priority keeps the other wave of the SIMD from starving it (-2%)
        if constexpr (WK == WK_W4A8) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            v4i bt[FN];
#pragma unroll
            for (int f = 0; f < FN; ++f) bt[f] = wop(cur.w[f], t);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int f = 0; f < FN; ++f) {
                    acc[i][f] = mfma32(bt[f], aop(cur, t, i), acc[i][f]);
                    const int done = (t * FM + i) * FN + f + 1;   // a constant once unrolled
                    if (READ_LATE && done == 4) {
                        __builtin_amdgcn_sched_barrier(0);
                        if (!DEFER || kc + 1 != cps) read_frags(ring + ((B + 1) % NS) * C::STAGE, nxt);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    if ((ISS || !PAIR) && done == N1) {
                        __builtin_amdgcn_sched_barrier(0);
                        issue_stage(IntC<(B + NS - 1) % NS>{});
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    if (ISS && done == N2) {
                        __builtin_amdgcn_sched_barrier(0);
                        issue_stage(IntC<B % NS>{});
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
        }
        if constexpr (WK == WK_W4A8) __builtin_amdgcn_s_setprio(0);

        if (++kc == cps) {
            // Unit done: epilogue while the next unit's stages are in flight.
            // The tensor scale is read here, next to its use: a scalar load
            // left outstanding across the k-loop would turn every wait for
            // LDS reads there into lgkmcnt(0) (scalar loads share that
            // counter and return out of order).
            const float sw0 = (wk_chan(WK) || ACC) ? 0.0f : p.wscale[0];
            int m0, n0, kc0, uid;
            tile_origin(cur_tile, m0, n0, kc0, uid);
            const bool full = m0 + BIG_BM <= M && n0 + BN <= p.N && (p.N & 7) == 0;
            if constexpr (SPLIT) {
                // K slice of a tile: the raw sums go to the unit's partial
                // tile in fragment order, 1 KiB contiguous per store
                int4* dst = reinterpret_cast<int4*>(p.part) + ((size_t)uid * NW + wave) * (FM * FN * 4 * 64) + lane;
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int f = 0; f < FN; ++f)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            dst[((i * FN + f) * 4 + q) * 64] =
                                make_int4(acc[i][f][4 * q], acc[i][f][4 * q + 1], acc[i][f][4 * q + 2], acc[i][f][4 * q + 3]);
            } else if (full && !ACC) {
                // Full tile.  The MFMA layout gives each lane 4 consecutive
                // columns of one row, so direct stores would write 16-byte
                // pieces of 32 rows per instruction.  Instead each wave passes
                // its results through LDS one 32-row x 32-column block at a
                // time (every lane writes its 16 values of the block) and
                // stores 64-byte row segments (4 lanes x 16 bytes per row, 16
                // rows per store); the two blocks of a row's 128-byte line go
                // out back to back.  Rows are padded to 80 bytes; the wave's
                // 64 bias values, scales and (W4A4) weight corrections sit
                // behind them.  Scratch: W4A4 has a region of its own, each
                // wave only touching its part; the int8-weight and W4A8
                // kernels use the ring buffer of this step's stage, which
                // every wave has read (into registers) before the barrier
                // below and which is refilled only after the next step's
                // barrier.  (For the int8-weight kernels this replaced
                // direct stores from registers: int8_tensorwise V/O 47.9 ->
                // 44.2 us, W4A8 at M = 4096 195.9 -> 190.2 us.)
                constexpr int TR = C::EPI_TR, OPB = C::EPI_OPB;
                int8_t* ebase;
                int8_t* obase;
                if constexpr (C::PA) {
                    ebase = ring + C::EPI_OFF;
                    obase = ebase + NW * 32 * TR;
                } else if constexpr (C::EPI_OPS_IN_RING) {
                    ebase = ring + B * C::STAGE;
                    obase = ebase + NW * 32 * TR;
                } else {
                    static_assert(NW * 32 * TR <= C::STAGE, "staging rows fit one stage buffer");
                    ebase = ring + B * C::STAGE;
                    obase = ring + C::EPI_OFF + (WK == WK_W4A8 ? 4096 : 0);
                }
                int8_t* scr = ebase + wave * 32 * TR;
                int8_t* sop = obase + wave * OPB;
                float sxv[FM];
                int rnv[FM];                                  // W4A4: -128 ra[m]
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int m = m0 + wm * WROWS + i * 32 + l32;
                    sxv[i] = p.sx[m];
                    if constexpr (C::PA) rnv[i] = -128 * p.ra[m];
                }
                const int nw0 = n0 + wn * FN * 32;            // the wave's first column
                constexpr int NCW = FN * 32;                  // the wave's columns
                constexpr int OS = NCW * 4, OC = NCW * 8;     // scale and correction offsets in sop
                // bias as float; with no bias -0.0, which leaves every sum as
                // it is (x + -0 == x, zeros included), so the add needs no test
                float bl[(NCW + 63) / 64];
                float cl[(NCW + 63) / 64];
                int cnl[(NCW + 63) / 64];
#pragma unroll
                for (int c = 0; c < (NCW + 63) / 64; ++c) {
                    const int col = min(c * 64 + lane, NCW - 1);
                    bl[c] = p.bias != nullptr ? bf16_lo(p.bias[nw0 + col]) : -0.0f;
                    cl[c] = sw0;
                    if constexpr (wk_chan(WK)) cl[c] = p.wscale[nw0 + col];
                    cnl[c] = 0;
                    if constexpr (C::PA) cnl[c] = -128 * p.cw[nw0 + col];
                }
                if constexpr (!C::PA) lds_barrier();          // stage buffer B is no longer read
#pragma unroll
                for (int c = 0; c < (NCW + 63) / 64; ++c) {
                    if (NCW % 64 == 0 || c * 64 + lane < NCW) {
                        reinterpret_cast<float*>(sop)[c * 64 + lane] = bl[c];
                        reinterpret_cast<float*>(sop + OS)[c * 64 + lane] = cl[c];
                        if constexpr (C::PA) reinterpret_cast<int*>(sop + OC)[c * 64 + lane] = cnl[c];
                    }
                }
                // per-lane bases; every other offset below is a constant
                const int8_t* sbias = sop + 16 * h;           // bias of column 4h (+ 32f + 8q)
                const int8_t* sscale = sop + OS + 16 * h;     // scale of column 4h
                const int8_t* scorr = sop + OC + 16 * h;      // correction of column 4h
                int8_t* swr = scr + l32 * TR + 8 * h;         // this lane's row, its 4 columns
                const int8_t* srd = scr + (lane >> 2) * TR + (lane & 3) * 16;
#pragma unroll
                for (int i = 0; i < FM; ++i) {
#pragma unroll
                    for (int f = 0; f < FN; ++f) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float4 bq = *reinterpret_cast<const float4*>(sbias + 4 * (32 * f + 8 * q));
                            const float4 cq = *reinterpret_cast<const float4*>(sscale + 4 * (32 * f + 8 * q));
                            const float c[4] = {cq.x, cq.y, cq.z, cq.w};
                            const float b[4] = {bq.x, bq.y, bq.z, bq.w};
                            int a[4] = {acc[i][f][4 * q], acc[i][f][4 * q + 1], acc[i][f][4 * q + 2], acc[i][f][4 * q + 3]};
                            if constexpr (C::PA) {
                                const int4 rq = *reinterpret_cast<const int4*>(scorr + 4 * (32 * f + 8 * q));
                                a[0] = w4_exact(a[0], rnv[i], rq.x);
                                a[1] = w4_exact(a[1], rnv[i], rq.y);
                                a[2] = w4_exact(a[2], rnv[i], rq.z);
                                a[3] = w4_exact(a[3], rnv[i], rq.w);
                            }
                            float v[4];
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                v[j] = (float)a[j] * sxv[i];
                                v[j] = v[j] * c[j];
                                v[j] = v[j] + b[j];
                            }
                            *reinterpret_cast<uint2*>(swr + q * 16) =
                                make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                        }
#pragma unroll
                        for (int sg = 0; sg < 2; ++sg) {
                            const int lr = (lane >> 2) + 16 * sg;
                            const uint4 o = *reinterpret_cast<const uint4*>(srd + sg * 16 * TR);
                            const int m = m0 + wm * WROWS + i * 32 + lr;
                            const int n = nw0 + f * 32 + (lane & 3) * 8;
                            *reinterpret_cast<uint4*>(p.y + (size_t)m * p.N + n) = o;
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
                                    store4<WK, ACC>(epi, m, n, sxm, sw0, acc[i][f][4 * q + 0], acc[i][f][4 * q + 1],
                                                    acc[i][f][4 * q + 2], acc[i][f][4 * q + 3]);
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
            if constexpr (DEFER) read_frags(ring + ((B + 1) % NS) * C::STAGE, nxt);
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

// Large-M configuration: 8 waves (block tile 256 x 256), one persistent block
// per CU; ring depth 6 for 4-bit weights (144 KiB of LDS; W4A8 154 KiB with
// its table), 4 for int8 weights (128 KiB).
constexpr int BIG_NW = 8;
template <int WK> constexpr int big_stages() { return wk_i8w(WK) ? 4 : 6; }

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

// Second kernel of a K-split GEMM: adds the `splits` int32 partial tiles of
// every output tile (exact, so the result does not depend on the split) and
// runs the epilogue.  One wavefront per 32 x 32 fragment (tile, wave, i, f)
// of the GEMM kernel, reading the partials in the order they were stored.
template <int WK, bool ACC, int BN>
__global__ void __launch_bounds__(256) k_big_fixup(GemmArgs p, int tiles_m, int tiles_n, int splits) {
    using C = BigCfg<WK, BIG_NW, 4, BN>;            // tile geometry only
    constexpr int NW = BIG_NW, WM = C::WM, WROWS = C::WROWS;
    constexpr int FM = C::FM, FN = C::FN, FRAGS = NW * FM * FN;
    const int lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
    const int item = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
    const int total = tiles_m * tiles_n;
    const int t = item / FRAGS;
    if (t >= total) return;
    const int r = item - t * FRAGS;                  // wave * FM * FN + i * FN + f
    const int wave = r / (FM * FN), fi = r - wave * (FM * FN);
    const int i = fi / FN, f = fi - i * FN;
    int m0, n0;
    big_tile_origin(t, tiles_m, tiles_n, BN, m0, n0);
    const int m = m0 + (wave % WM) * WROWS + i * 32 + l32;
    const int4* src = reinterpret_cast<const int4*>(p.part) + (size_t)t * NW * FM * FN * 4 * 64 + r * 4 * 64 + lane;
    const size_t sstride = (size_t)total * NW * FM * FN * 4 * 64;   // int4 per K slice
    int4 sum[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) sum[q] = make_int4(0, 0, 0, 0);
#pragma unroll 4
    for (int k = 0; k < splits; ++k) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int4 v = src[k * sstride + q * 64];
            sum[q].x += v.x; sum[q].y += v.y; sum[q].z += v.z; sum[q].w += v.w;
        }
    }
    const Epi epi = make_epi(p);
    const int mrow0 = m0 + (wave % WM) * WROWS + i * 32;            // the fragment's first row and column
    const int ncol0 = n0 + ((wave / WM) * FN + f) * 32;
    const int nbase = ncol0 + 4 * h;
    if (!ACC && mrow0 + 32 <= p.M && ncol0 + 32 <= p.N && (p.N & 7) == 0) {
        // Whole fragment: the outputs pass through LDS so that each store
        // writes 64-byte row segments (4 lanes x 16 bytes, 16 rows per
        // store) instead of 16-byte pieces of 32 rows; same arithmetic as
        // store4.  Rows of 64 bytes padded to 80.
        __shared__ __attribute__((aligned(16))) uint8_t stg[4][32 * 80];
        uint8_t* stw = stg[threadIdx.x >> 6];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const Epi4 op = epi4_fetch<WK>(epi, p.sx, p.M, m, nbase + 8 * q);
            int a[4] = {sum[q].x, sum[q].y, sum[q].z, sum[q].w};
            if constexpr (WK == WK_W4) {
#pragma unroll
                for (int j = 0; j < 4; ++j) a[j] = w4_exact(a[j], op.rn, op.cn[j]);
            }
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[j] = (float)a[j] * op.sx;
                v[j] = v[j] * op.sw[j];
                v[j] = v[j] + op.b[j];          // -0.0 without a bias
            }
            *reinterpret_cast<uint2*>(stw + l32 * 80 + 8 * h + 16 * q) =
                make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) {
            const int lr = (lane >> 2) + 16 * sg;
            const uint4 o = *reinterpret_cast<const uint4*>(stw + lr * 80 + (lane & 3) * 16);
            *reinterpret_cast<uint4*>(p.y + (size_t)(mrow0 + lr) * p.N + ncol0 + (lane & 3) * 8) = o;
        }
        return;
    }
    if (m >= p.M) return;
    const float sw0 = (wk_chan(WK) || ACC) ? 0.0f : p.wscale[0];
    const float sxm = ACC ? 0.0f : p.sx[m];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int n = nbase + 8 * q;
        if (n < p.N)
            store4<WK, ACC>(epi, m, n, sxm, sw0, sum[q].x, sum[q].y, sum[q].z, sum[q].w);
    }
}

// Large-M plan: the block tile width and the K slices per tile.  Rough time
// model in microseconds: per 64-k stage of a 256 x 256 tile about 0.8 us for
// 4-bit weights, 1.0 for int8, 1.3 for W4A8, 0.9 of that for a 256 x 192
// tile (three quarters of the work; its 64 x 96 wave tiles read more LDS bytes
// and widen more operands per MFMA, measured ~1.2x the time per op) and 0.55
// for a 256 x 128 tile (half the work on 64 x 64 wave tiles; it lets layers
// with few output tiles fill the chip with fewer K slices: ConvRot INT8 2560^2
// at M = 1220 29.2 -> 25.9 us without a split instead of 4 slices; and it
// fills the last round where 256-wide tiles leave half of it idle: the W4A8
// layer's int8 GEMM, 640 tiles of 256 x 256 against 1280 of 256 x 128,
// 186.5 -> 182.0 us), and 0.41 for a 256 x 64 tile (below);
// rounds of one unit per CU; plus, for a split, the int32 partial tiles
// written and read back at about 4.5 TB/s and a second launch.  Anything
// other than 256-wide whole tiles has to win by 5%.  Slices divide the K
// chunks evenly, at most 16.  W4A8 keeps 256-wide tiles (its LDS has no room
// for the narrower tiles' epilogue scratch).
constexpr int BIG_CUS = 256;
constexpr double BIG_T128 = 0.55;   // a 256 x 128 tile's stage, relative to 256 x 256
// a 256 x 64 tile's stage: 64 x 32 wave tiles, 1.5x the LDS bytes per MFMA
// of 64 x 64; measured with forced plans, ConvRot INT8 2560^2 at M = 1220
// (200 whole tiles against 100 of 256 x 128): 19.8-20.5 us against
// 26.9-27.1 us; slower on every other bench layer
constexpr double BIG_T64 = 0.41;
constexpr int BIG_MAX_SPLITS = 16;

// Plan override for inspection and timing (cr_dbg_big_plan): block tile width
// and K slices; 0 leaves the planner's choice.
static std::atomic<int> g_big_force_bn{0}, g_big_force_splits{0};
void set_big_plan_override(int bn, int splits) {
    g_big_force_bn.store(bn);
    g_big_force_splits.store(splits);
}

BigPlan plan_big(int kind, int M, int N, int K) {
    BigPlan bp{1, 0, 0, 256};
    if (M <= 0 || N <= 0 || K <= 0) return bp;
    const int Kp = wk_i8w(kind) ? round_up(K, 64) : K;
    const int nkc = Kp / 64;
    bp.cps = nkc;
    const double t_stage = kind == WK_W4 ? 0.8 : (wk_i8w(kind) ? 1.0 : 1.3);
    const double tiles_m = (double)((M + BIG_BM - 1) / BIG_BM);
    double best = std::ceil(tiles_m * ((N + 255) / 256) / BIG_CUS) * nkc * t_stage;
    for (int bn : {256, 192, 128, 64}) {
        if (bn != 256 && kind == WK_W4A8) continue;
        const double total = tiles_m * ((N + bn - 1) / bn);
        const double ts = t_stage * (bn == 256 ? 1.0 : (bn == 192 ? 0.9 : (bn == 128 ? BIG_T128 : BIG_T64)));
        for (int S = 1; S <= BIG_MAX_SPLITS && S <= nkc; ++S) {
            if (nkc % S != 0 || (bn == 256 && S == 1)) continue;
            double cost = std::ceil(total * S / BIG_CUS) * (nkc / S) * ts;
            if (S > 1) cost += (2.0 * total * S * BIG_BM * bn * 4.0 + 2.0 * M * N) / 4.5e6 + 4.0;
            if (cost < best * 0.95) {
                best = cost;
                bp.bn = bn;
                bp.splits = S;
                bp.cps = nkc / S;
            }
        }
    }
    const int fbn = g_big_force_bn.load(), fs = g_big_force_splits.load();
    if (fbn > 0 && (kind != WK_W4A8 || fbn == 256)) bp.bn = fbn;
    if (fs > 0 && fs <= nkc && nkc % fs == 0) {
        bp.splits = fs;
        bp.cps = nkc / fs;
    }
    const double total = tiles_m * ((N + bp.bn - 1) / bp.bn);
    bp.part_bytes = bp.splits > 1 ? (size_t)total * bp.splits * BIG_BM * bp.bn * 4 : 0;
    return bp;
}

template <int WK, bool ACC, int BN>
static hipError_t launch_big_bn(const GemmArgs& a, const BigPlan& bp, hipStream_t st) {
    constexpr int NS = big_stages<WK>();
    using C = BigCfg<WK, BIG_NW, NS, BN>;
    const int tiles_m = (a.M + BIG_BM - 1) / BIG_BM, tiles_n = (a.N + BN - 1) / BN;
    if (bp.splits > 1 && a.part == nullptr) return hipErrorInvalidValue;
    // opt in to more than 64 KiB of dynamic LDS (once per device and kernel)
    static std::atomic<uint64_t> lds_done[2];
    const bool split = bp.splits > 1;
    {
        const void* k = split ? reinterpret_cast<const void*>(&k_gemm_big<WK, BIG_NW, NS, BN, ACC, true>)
                              : reinterpret_cast<const void*>(&k_gemm_big<WK, BIG_NW, NS, BN, ACC, false>);
        hipError_t e = opt_in_lds(k, (int)C::LDS, lds_done[split]);
        if (e != hipSuccess) return e;
    }
    const int units = tiles_m * tiles_n * bp.splits;
    const int grid = min(units, num_cus());
    if (!split) {
        k_gemm_big<WK, BIG_NW, NS, BN, ACC, false><<<dim3(grid), dim3(64 * BIG_NW), C::LDS, st>>>(a, tiles_m, tiles_n, 1, bp.cps);
        return hipGetLastError();
    }
    k_gemm_big<WK, BIG_NW, NS, BN, ACC, true><<<dim3(grid), dim3(64 * BIG_NW), C::LDS, st>>>(a, tiles_m, tiles_n, bp.splits, bp.cps);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int FRAGS = BIG_NW * C::FM * C::FN;
    const int items = tiles_m * tiles_n * FRAGS;
    k_big_fixup<WK, ACC, BN><<<dim3((items + 3) / 4), dim3(256), 0, st>>>(a, tiles_m, tiles_n, bp.splits);
    return hipGetLastError();
}

template <int WK, bool ACC>
static hipError_t launch_big_t(const GemmArgs& a, hipStream_t st) {
    const BigPlan bp = plan_big(WK, a.M, a.N, a.K);
    if constexpr (WK != WK_W4A8) {
        if (bp.bn == 192) return launch_big_bn<WK, ACC, 192>(a, bp, st);
        if (bp.bn == 128) return launch_big_bn<WK, ACC, 128>(a, bp, st);
        if (bp.bn == 64) return launch_big_bn<WK, ACC, 64>(a, bp, st);
    }
    if (bp.bn != 256) return hipErrorInvalidValue;
    return launch_big_bn<WK, ACC, 256>(a, bp, st);
}

template <int WK>
static hipError_t launch_kind(const GemmArgs& a, hipStream_t st) {
    const SmallPlan sp = plan_small(WK, a.M, a.N, a.K);
    if (sp.use) return launch_small(a, sp, st);
    return a.acc_out != nullptr ? launch_big_t<WK, true>(a, st) : launch_big_t<WK, false>(a, st);
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
    switch (a.kind) {
        case WK_W4: return launch_kind<WK_W4>(a, st);
        case WK_I8: return launch_kind<WK_I8>(a, st);
        case WK_W4A8: return launch_kind<WK_W4A8>(a, st);
        case WK_I8R: return launch_kind<WK_I8R>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace cr
