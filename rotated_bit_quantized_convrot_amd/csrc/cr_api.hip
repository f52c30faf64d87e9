// C ABI of the ConvRot linear library: argument checks, workspace layout and
// dispatch to the kernels.  Nothing here allocates device memory or
// synchronises.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <atomic>
#include <mutex>

#include "convrot.h"
#include "cr_internal.h"

namespace {

thread_local char g_err[512] = "";

cr_status fail(cr_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

cr_status ok() {
    g_err[0] = '\0';
    return CR_OK;
}

// Per device id: 0 = unknown, 1 = gfx950, 2 = other (set once; calls from
// several host threads may race to set the same value).
std::atomic<int> g_dev_state[64];

cr_status check_device() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0) return fail(CR_ERR_DEVICE, "no HIP device: %s", hipGetErrorString(e));
    if (dev < 64 && g_dev_state[dev].load(std::memory_order_relaxed) == 1) return CR_OK;
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(CR_ERR_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    const bool good = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64) g_dev_state[dev].store(good ? 1 : 2, std::memory_order_relaxed);
    if (!good) return fail(CR_ERR_DEVICE, "device %d is %s, this library is built for gfx950", dev, prop.gcnArchName);
    return CR_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t a256(size_t v) { return (v + 255) / 256 * 256; }

bool rotated(int kind) { return kind != CR_INT8TW; }

cr_status check_kind(int kind) {
    if (kind < CR_W4A4 || kind > CR_W4A4_RH) return fail(CR_ERR_KIND, "unknown kind %d", kind);
    return CR_OK;
}

// Rotation selector of a kind (the W4A4 variants; 256 for the others).
int group_of(int kind) {
    switch (kind) {
        case CR_W4A4_G64: return 64;
        case CR_W4A4_G16: return 16;
        case CR_W4A4_RH: return cr::kRotRegular;
        default: return 256;
    }
}

cr_status check_nk(int kind, int N, int K) {
    if (N < 1 || K < 1 || N > CR_MAX_DIM || K > CR_MAX_DIM)
        return fail(CR_ERR_SHAPE, "bad shape N=%d K=%d (need 1..%d)", N, K, CR_MAX_DIM);
    // int8 codes reach +-127 on both sides, so |acc| <= 16129 K: int32 holds
    // it up to K = 133144; the limit is the power of two below
    if (kind == CR_INT8TW && K > CR_MAX_INT8_K)
        return fail(CR_ERR_SHAPE, "K=%d exceeds %d for int8_tensorwise (int32 accumulator range)", K, CR_MAX_INT8_K);
    if (rotated(kind)) {
        if (K % 256 != 0)
            return fail(CR_ERR_GROUP, "K=%d is not a multiple of the 256-wide rotation group; "
                        "use the int8_tensorwise format for this layer", K);
        if (K > CR_MAX_ROT_K) return fail(CR_ERR_SHAPE, "K=%d exceeds %d for rotated formats", K, CR_MAX_ROT_K);
    }
    return CR_OK;
}

size_t packed_bytes(int kind, int N, int K) {
    switch (kind) {
        case CR_W4A4:
        case CR_W4A4_G64:
        case CR_W4A4_G16:
        case CR_W4A4_RH: return cr::w4a4_bytes(N, K);
        case CR_INT8TW: return cr::i8_bytes(N, K);
        case CR_W4A8: return cr::w4a8_bytes(N, K);
        case CR_INT8ROT: return cr::i8_bytes(N, K);
        default: return 0;
    }
}

int kp_of(int kind, int K) { return kind == CR_INT8TW ? cr::round_up(K, 64) : K; }

int wkind(int kind) {
    switch (kind) {
        case CR_W4A4:
        case CR_W4A4_G64:
        case CR_W4A4_G16:
        case CR_W4A4_RH: return cr::WK_W4;
        case CR_INT8TW: return cr::WK_I8;
        case CR_INT8ROT: return cr::WK_I8R;
        default: return cr::WK_W4A8;
    }
}

// Workspace: [codes][scales M][W4A4: ra M][split-K partials].  Codes are
// int8 [M, Kp], or for W4A4 4-bit tiles (round_up(M, 32) x K/2 bytes).  The
// codes and scales do not depend on N, so one quantisation can feed GEMMs
// against several weights (with the workspace sized for the largest need
// over their N).
struct WsLayout {
    size_t qx, sx, ra, sync, part, wexp, quant_end, total;
};

// W4A8 at large M: the GEMM's per-16-weight table decode is the costly part
// of its inner loop, so the weight is first decoded once into the int8 tile
// layout (in the workspace) and the int8 GEMM with per-column scales runs on
// it; the decoded values and so the accumulators are the same.  Pays off
// from about M = 1300 at the W4A8 layer (K = 3840, N = 10240: 216.7 -> 178.2
// us for the GEMM, ~10 us for the decode pass); taken from M = 2048 on.
bool w4a8_expands(int kind, int M) { return kind == CR_W4A8 && M >= 2048; }

// The GEMM kernels' format for this call.
int gemm_wkind(int kind, int M) { return w4a8_expands(kind, M) ? cr::WK_I8R : wkind(kind); }

WsLayout ws_layout(int kind, int M, int N, int K) {
    WsLayout l{};
    const int wk = wkind(kind), gk = gemm_wkind(kind, M);
    l.qx = 0;
    l.sx = a256(cr::act_bytes(wk, M, K));
    l.ra = l.sx + a256((size_t)M * 4);
    l.sync = l.ra + (cr::act_packed(wk) ? a256((size_t)M * 4) : 0);
    l.part = l.sync + (size_t)cr::kSyncWords * 4;
    l.quant_end = l.part;
    const cr::SmallPlan sp = cr::plan_small(gk, M, N, K);
    l.wexp = l.part + a256(sp.use ? sp.part_bytes : cr::plan_big(gk, M, N, K).part_bytes);
    l.total = l.wexp + (w4a8_expands(kind, M) ? a256(cr::i8_bytes(N, K)) : 0);
    if (l.total < 256) l.total = 256;
    if (l.quant_end < 256) l.quant_end = 256;
    return l;
}

cr_status launch_err(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(CR_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
}

cr_status check_m(int M) {
    if (M < 0 || M > CR_MAX_DIM) return fail(CR_ERR_SHAPE, "bad M=%d", M);
    return CR_OK;
}

// Phase 1: codes and scales of x into the workspace.
cr_status quantize_phase(int kind, const void* x, int M, int K, void* ws, size_t ws_bytes, hipStream_t st) {
    const WsLayout l = ws_layout(kind, M, 1, K);
    if (ws_bytes < l.quant_end)
        return fail(CR_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, l.quant_end);
    char* w = static_cast<char*>(ws);
    hipError_t e = cr::launch_quant_act(wkind(kind), group_of(kind), static_cast<const uint16_t*>(x), M, K,
                                        kp_of(kind, K),
                                        reinterpret_cast<int8_t*>(w + l.qx), reinterpret_cast<float*>(w + l.sx),
                                        reinterpret_cast<int32_t*>(w + l.ra), cr::act_packed(wkind(kind)),
                                        reinterpret_cast<uint32_t*>(w + l.sync), st);
    return launch_err(e, "activation quantisation");
}

// Arguments of the GEMM kernels for a linear whose workspace is at w.
cr::GemmArgs gemm_args(int kind, int M, int K, const void* wp, const float* wscale, int N, const void* bias,
                       void* y, int32_t* acc, char* w, const WsLayout& l) {
    cr::GemmArgs a{};
    a.kind = gemm_wkind(kind, M);
    a.qx = reinterpret_cast<const int8_t*>(w + l.qx);
    a.sx = reinterpret_cast<const float*>(w + l.sx);
    a.M = M; a.N = N; a.K = K; a.Kp = kp_of(kind, K); a.Np = cr::round_up(N, 32);
    a.wp = static_cast<const uint8_t*>(wp);
    a.wscale = wscale;
    a.bias = static_cast<const uint16_t*>(bias);
    a.y = static_cast<uint16_t*>(y);
    a.acc_out = acc;
    a.part = reinterpret_cast<int32_t*>(w + l.part);
    a.sync = reinterpret_cast<uint32_t*>(w + l.sync);
    if (cr::act_packed(a.kind)) {
        a.ra = reinterpret_cast<const int32_t*>(w + l.ra);
        a.cw = reinterpret_cast<const int32_t*>(a.wp + cr::w4_cw_offset(N, K));
    }
    return a;
}

// Phase 2: GEMM + epilogue from the workspace.
cr_status gemm_phase(int kind, int M, int K, const void* wp, const float* wscale, int N, const void* bias,
                     void* y, int32_t* acc, void* ws, size_t ws_bytes, hipStream_t st) {
    const WsLayout l = ws_layout(kind, M, N, K);
    if (ws_bytes < l.total)
        return fail(CR_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, l.total);
    char* w = static_cast<char*>(ws);
    if (w4a8_expands(kind, M)) {
        cr_status s = launch_err(cr::launch_w4a8_expand(static_cast<const uint8_t*>(wp), N, K,
                                                        reinterpret_cast<uint8_t*>(w + l.wexp), st),
                                 "W4A8 weight decode");
        if (s != CR_OK) return s;
        wp = w + l.wexp;
    }
    const cr::GemmArgs a = gemm_args(kind, M, K, wp, wscale, N, bias, y, acc, w, l);
    return launch_err(cr::launch_gemm(a, st), "integer GEMM");
}

// The fused small-M W4A4 linear (rotation and quantisation by the GEMM
// launch's own first blocks): mode 1 takes it where it applies and M <= 8,
// mode 2 wherever it applies, mode 0 never.  Measured by graph replay with
// cold weights (K x N = 3072 x 3072, 2560 x 9728, 9728 x 2560): it saves up
// to 2 us at M = 1 and ties or wins up to M = 8; from M = 12 on its in-launch
// hand-off (producer stores, arrival counter, polls, device-scope code
// loads, all queued behind the weight stream) costs more than the second
// launch does.
constexpr int kFusedAutoMaxM = 8;
std::atomic<int> g_fused_mode{1};
bool use_fused(int kind, int M, int N, int K) {
    const int mode = g_fused_mode.load(std::memory_order_relaxed);
    if (kind != CR_W4A4 || mode == 0 || (mode == 1 && M > kFusedAutoMaxM)) return false;
    return cr::fused_small_ok(cr::WK_W4, M, N, K);
}

// Phases 1 and 2 in one launch (use_fused holds); writes the same workspace
// regions as the two phases.  xu non-NULL: the rows are silu(x) * xu (the MLP
// block's down projection).
cr_status fused_phase(int kind, const void* x, const void* xu, int M, int K, const void* wp, const float* wscale,
                      int N, const void* bias, void* y, int32_t* acc, void* ws, size_t ws_bytes, hipStream_t st) {
    const WsLayout l = ws_layout(kind, M, N, K);
    if (ws_bytes < l.total)
        return fail(CR_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, l.total);
    cr::GemmArgs a = gemm_args(kind, M, K, wp, wscale, N, bias, y, acc, static_cast<char*>(ws), l);
    a.x = static_cast<const uint16_t*>(x);
    a.xu = static_cast<const uint16_t*>(xu);
    return launch_err(cr::launch_small_fused(a, st), "fused W4A4 linear");
}

// Both phases of a linear: one fused launch where it applies, else the
// activation quantiser and the GEMM.
cr_status linear_phases(int kind, const void* x, int M, int K, const void* wp, const float* wscale, int N,
                        const void* bias, void* y, int32_t* acc, void* ws, size_t ws_bytes, hipStream_t st) {
    if (use_fused(kind, M, N, K))
        return fused_phase(kind, x, nullptr, M, K, wp, wscale, N, bias, y, acc, ws, ws_bytes, st);
    cr_status s = quantize_phase(kind, x, M, K, ws, ws_bytes, st);
    if (s != CR_OK) return s;
    return gemm_phase(kind, M, K, wp, wscale, N, bias, y, acc, ws, ws_bytes, st);
}

// Checks shared by the linears and the GEMM phase.
cr_status check_linear_args(int kind, int M, int K, const void* wp, const float* wscale, int N,
                            const void* bias, const void* y, const int32_t* acc, const void* ws) {
    cr_status s;
    if ((s = check_kind(kind)) != CR_OK) return s;
    if ((s = check_m(M)) != CR_OK) return s;
    if ((s = check_nk(kind, N, K)) != CR_OK) return s;
    if (wp == nullptr) return fail(CR_ERR_NULL, "packed weight is NULL");
    if (acc == nullptr && wscale == nullptr) return fail(CR_ERR_NULL, "weight scale is NULL");
    if (!aligned16(wp)) return fail(CR_ERR_ALIGN, "packed weight not 16-byte aligned");
    if (bias != nullptr && !aligned16(bias)) return fail(CR_ERR_ALIGN, "bias not 16-byte aligned");
    if (M == 0) return CR_OK;
    if (ws == nullptr || (acc == nullptr && y == nullptr)) return fail(CR_ERR_NULL, "y or workspace is NULL");
    if (!aligned16(ws) || (y && !aligned16(y)) || (acc && !aligned16(acc)))
        return fail(CR_ERR_ALIGN, "y, accumulator or workspace not 16-byte aligned");
    return CR_OK;
}

// Shared body of the three linears and the accumulator hook.
cr_status run_linear(int kind, const void* x, int M, int K, const void* wp, const float* wscale, int N,
                     const void* bias, void* y, int32_t* acc, void* ws, size_t ws_bytes,
                     hipStream_t st) {
    cr_status s = check_linear_args(kind, M, K, wp, wscale, N, bias, y, acc, ws);
    if (s != CR_OK) return s;
    if (M == 0) return ok();
    if (x == nullptr) return fail(CR_ERR_NULL, "x is NULL");
    if (!aligned16(x)) return fail(CR_ERR_ALIGN, "x not 16-byte aligned");
    const WsLayout l = ws_layout(kind, M, N, K);
    if (ws_bytes < l.total)
        return fail(CR_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, l.total);
    if ((s = check_device()) != CR_OK) return s;
    return linear_phases(kind, x, M, K, wp, wscale, N, bias, y, acc, ws, ws_bytes, st);
}

// ---- static scratch of cr_linear_w4a4_noalloc ----------------------------
// For callers that cannot allocate: the workspace of one W4A4 linear lives in
// this file-scope device array (one copy per GPU, held until the process
// ends).  Host code never passes the array's name to a kernel: its device
// address is looked up once per device with hipGetSymbolAddress and kept.
constexpr size_t kScratchBytes = (size_t)8 << 20;
static_assert(kScratchBytes == CR_NOALLOC_SCRATCH_BYTES, "header and library agree on the scratch size");

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];          // device address of `scratch` per device id, under g_scratch_mu

cr_status scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0) return fail(CR_ERR_DEVICE, "no HIP device: %s", hipGetErrorString(e));
    if (dev >= 64) return fail(CR_ERR_DEVICE, "device id %d beyond the 64 the static scratch table covers", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(CR_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return CR_OK;
}

// Gated MLP block workspace: [x codes + gate/up partials | g | u | h codes +
// down partials], each region at a 256-byte boundary.
struct MlpLayout {
    size_t g, u, b, total;
};

MlpLayout mlp_layout(int M, int K, int F, int N) {
    MlpLayout l{};
    l.g = a256(ws_layout(CR_W4A4, M, F, K).total);
    l.u = l.g + a256((size_t)M * F * 2);
    l.b = l.u + a256((size_t)M * F * 2);
    l.total = l.b + ws_layout(CR_W4A4, M, N, F).total;
    return l;
}

cr_status check_mlp_shape(int M, int K, int F, int N) {
    cr_status s;
    if ((s = check_m(M)) != CR_OK) return s;
    if ((s = check_nk(CR_W4A4, F, K)) != CR_OK) return s;
    return check_nk(CR_W4A4, N, F);
}

}  // namespace

extern "C" {

size_t cr_mlp_workspace_bytes(int M, int K, int F, int N) {
    if (check_mlp_shape(M, K, F, N) != CR_OK) return 0;
    return mlp_layout(M, K, F, N).total;
}

cr_status cr_mlp_w4a4(const void* x_bf16, int M, int K, const void* wg_packed, const float* wg_scale,
                      const void* wu_packed, const float* wu_scale, int F, const void* wd_packed,
                      const float* wd_scale, int N, void* y_bf16, void* ws, size_t ws_bytes, hipStream_t stream) {
    cr_status s;
    if ((s = check_mlp_shape(M, K, F, N)) != CR_OK) return s;
    if (!wg_packed || !wg_scale || !wu_packed || !wu_scale || !wd_packed || !wd_scale)
        return fail(CR_ERR_NULL, "packed weight or scale is NULL");
    if (!aligned16(wg_packed) || !aligned16(wu_packed) || !aligned16(wd_packed))
        return fail(CR_ERR_ALIGN, "packed weight not 16-byte aligned");
    if (M == 0) return ok();
    if (!x_bf16 || !y_bf16 || !ws) return fail(CR_ERR_NULL, "x, y or workspace is NULL");
    if (!aligned16(x_bf16) || !aligned16(y_bf16) || !aligned16(ws))
        return fail(CR_ERR_ALIGN, "x, y or workspace not 16-byte aligned");
    const MlpLayout l = mlp_layout(M, K, F, N);
    if (ws_bytes < l.total) return fail(CR_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, l.total);
    if ((s = check_device()) != CR_OK) return s;
    char* w = static_cast<char*>(ws);
    // x quantised once for the gate and up GEMMs (at small M by the gate
    // GEMM's own launch)
    if ((s = linear_phases(CR_W4A4, x_bf16, M, K, wg_packed, wg_scale, F, nullptr, w + l.g, nullptr, w, l.g,
                           stream)) != CR_OK)
        return s;
    if ((s = gemm_phase(CR_W4A4, M, K, wu_packed, wu_scale, F, nullptr, w + l.u, nullptr, w, l.g, stream)) != CR_OK)
        return s;
    // h = silu(g) * u, rotated and quantised for the down GEMM (at small M
    // by the down GEMM's own launch)
    const WsLayout lb = ws_layout(CR_W4A4, M, N, F);
    char* wb = w + l.b;
    if (use_fused(CR_W4A4, M, N, F))
        return fused_phase(CR_W4A4, w + l.g, w + l.u, M, F, wd_packed, wd_scale, N, nullptr, y_bf16, nullptr, wb,
                           lb.total, stream);
    s = launch_err(cr::launch_quant_swiglu(reinterpret_cast<const uint16_t*>(w + l.g),
                                           reinterpret_cast<const uint16_t*>(w + l.u), M, F,
                                           reinterpret_cast<int8_t*>(wb + lb.qx), reinterpret_cast<float*>(wb + lb.sx),
                                           reinterpret_cast<int32_t*>(wb + lb.ra), true,
                                           reinterpret_cast<uint32_t*>(wb + lb.sync), stream),
                   "MLP activation quantisation");
    if (s != CR_OK) return s;
    return gemm_phase(CR_W4A4, M, F, wd_packed, wd_scale, N, nullptr, y_bf16, nullptr, wb, lb.total, stream);
}

cr_status cr_dbg_silu_mul(const void* g_bf16, const void* u_bf16, size_t n, void* h_bf16, hipStream_t stream) {
    if (n == 0) return ok();
    if (!g_bf16 || !u_bf16 || !h_bf16) return fail(CR_ERR_NULL, "NULL argument");
    if (n > ((size_t)1 << 40)) return fail(CR_ERR_SHAPE, "n=%zu too large", n);
    cr_status s;
    if ((s = check_device()) != CR_OK) return s;
    return launch_err(cr::launch_silu_mul(static_cast<const uint16_t*>(g_bf16), static_cast<const uint16_t*>(u_bf16), n,
                                          static_cast<uint16_t*>(h_bf16), stream),
                      "silu product");
}

cr_status cr_dbg_quant_swiglu(const void* g_bf16, const void* u_bf16, int M, int K, void* codes, float* scales,
                              hipStream_t stream) {
    cr_status s;
    if (M < 0 || M > CR_MAX_DIM) return fail(CR_ERR_SHAPE, "bad M=%d", M);
    if ((s = check_nk(CR_W4A4, 1, K)) != CR_OK) return s;
    if (M == 0) return ok();
    if (!g_bf16 || !u_bf16 || !codes || !scales) return fail(CR_ERR_NULL, "NULL argument");
    if (!aligned16(g_bf16) || !aligned16(u_bf16) || !aligned16(codes))
        return fail(CR_ERR_ALIGN, "pointer not 16-byte aligned");
    if ((s = check_device()) != CR_OK) return s;
    return launch_err(cr::launch_quant_swiglu(static_cast<const uint16_t*>(g_bf16), static_cast<const uint16_t*>(u_bf16),
                                              M, K, static_cast<int8_t*>(codes), scales, nullptr, false, nullptr, stream),
                      "MLP activation quantisation");
}

size_t cr_packed_bytes(int kind, int N, int K) {
    if (check_kind(kind) != CR_OK || check_nk(kind, N, K) != CR_OK) return 0;
    return packed_bytes(kind, N, K);
}

size_t cr_workspace_bytes(int kind, int M, int N, int K) {
    if (check_kind(kind) != CR_OK || check_nk(kind, N, K) != CR_OK || M < 0 || M > CR_MAX_DIM) return 0;
    return ws_layout(kind, M, N, K).total;
}

static cr_status pack_common_checks(int kind, const void* w, int N, int K, void* out, const void* scale) {
    cr_status s;
    if ((s = check_nk(kind, N, K)) != CR_OK) return s;
    if (w == nullptr || out == nullptr || scale == nullptr) return fail(CR_ERR_NULL, "NULL argument");
    if (!aligned16(w) || !aligned16(out)) return fail(CR_ERR_ALIGN, "pointer not 16-byte aligned");
    return check_device();
}

cr_status cr_pack_weight_w4(const void* w_bf16, int N, int K, void* w_packed, float* w_scale,
                            hipStream_t stream) {
    cr_status s = pack_common_checks(CR_W4A4, w_bf16, N, K, w_packed, w_scale);
    if (s != CR_OK) return s;
    return launch_err(cr::launch_pack_w4(static_cast<const uint16_t*>(w_bf16), N, K, 256,
                                         static_cast<uint8_t*>(w_packed), w_scale, stream),
                      "W4 weight packing");
}

static cr_status w4_group_kind(int group, int* kind) {
    switch (group) {
        case 256: *kind = CR_W4A4; return CR_OK;
        case 64: *kind = CR_W4A4_G64; return CR_OK;
        case 16: *kind = CR_W4A4_G16; return CR_OK;
        default: return fail(CR_ERR_GROUP, "rotation group %d is not one of 256, 64, 16", group);
    }
}

cr_status cr_pack_weight_w4_group(const void* w_bf16, int N, int K, int group, void* w_packed, float* w_scale,
                                  hipStream_t stream) {
    int kind = 0;
    cr_status s = w4_group_kind(group, &kind);
    if (s != CR_OK) return s;
    if ((s = pack_common_checks(kind, w_bf16, N, K, w_packed, w_scale)) != CR_OK) return s;
    return launch_err(cr::launch_pack_w4(static_cast<const uint16_t*>(w_bf16), N, K, group,
                                         static_cast<uint8_t*>(w_packed), w_scale, stream),
                      "W4 weight packing");
}

cr_status cr_linear_w4a4_group(const void* x_bf16, int M, int K, int group, const void* w_packed,
                               const float* w_scale, int N, const void* bias_bf16, void* y_bf16, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
    int kind = 0;
    const cr_status s = w4_group_kind(group, &kind);
    if (s != CR_OK) return s;
    return run_linear(kind, x_bf16, M, K, w_packed, w_scale, N, bias_bf16, y_bf16, nullptr, ws, ws_bytes,
                      stream);
}

cr_status cr_pack_weight_w4_regular(const void* w_bf16, int N, int K, void* w_packed, float* w_scale,
                                    hipStream_t stream) {
    cr_status s = pack_common_checks(CR_W4A4_RH, w_bf16, N, K, w_packed, w_scale);
    if (s != CR_OK) return s;
    return launch_err(cr::launch_pack_w4(static_cast<const uint16_t*>(w_bf16), N, K, cr::kRotRegular,
                                         static_cast<uint8_t*>(w_packed), w_scale, stream),
                      "W4 weight packing (regular Hadamard)");
}

cr_status cr_linear_w4a4_regular(const void* x_bf16, int M, int K, const void* w_packed, const float* w_scale,
                                 int N, const void* bias_bf16, void* y_bf16, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
    return run_linear(CR_W4A4_RH, x_bf16, M, K, w_packed, w_scale, N, bias_bf16, y_bf16, nullptr, ws, ws_bytes,
                      stream);
}

cr_status cr_pack_weight_int8tw(const void* w_bf16, int N, int K, void* w_packed, float* w_scale,
                                hipStream_t stream) {
    cr_status s = pack_common_checks(CR_INT8TW, w_bf16, N, K, w_packed, w_scale);
    if (s != CR_OK) return s;
    return launch_err(cr::launch_pack_i8(static_cast<const uint16_t*>(w_bf16), N, K,
                                         static_cast<uint8_t*>(w_packed), w_scale, stream),
                      "int8 weight packing");
}

cr_status cr_pack_weight_w4a8(const void* idx, const void* s_rel_e4m3, const float* codebook, int N,
                              int K, void* w_packed, hipStream_t stream) {
    cr_status s;
    if ((s = check_nk(CR_W4A8, N, K)) != CR_OK) return s;
    if (idx == nullptr || s_rel_e4m3 == nullptr || codebook == nullptr || w_packed == nullptr)
        return fail(CR_ERR_NULL, "NULL argument");
    if (!aligned16(idx) || !aligned16(s_rel_e4m3) || !aligned16(w_packed))
        return fail(CR_ERR_ALIGN, "pointer not 16-byte aligned");
    if ((s = check_device()) != CR_OK) return s;
    return launch_err(cr::launch_pack_w4a8(static_cast<const uint8_t*>(idx),
                                           static_cast<const uint8_t*>(s_rel_e4m3), codebook, N, K,
                                           static_cast<uint8_t*>(w_packed), stream),
                      "W4A8 weight packing");
}

static cr_status check_encode_shape(int N, int K) {
    cr_status s;
    if ((s = check_nk(CR_W4A8, N, K)) != CR_OK) return s;
    if ((size_t)N * (size_t)K > ((size_t)1 << 28))
        return fail(CR_ERR_SHAPE, "N*K = %zu exceeds 2^28 (the exact integer sums of the codebook fit)",
                    (size_t)N * (size_t)K);
    return CR_OK;
}

size_t cr_encode_w4a8_workspace_bytes(int N, int K) {
    if (check_encode_shape(N, K) != CR_OK) return 0;
    return cr::encode_w4a8_workspace(N, K);
}

cr_status cr_encode_w4a8(const void* w_bf16, int N, int K, int iters, void* idx, void* s_rel_e4m3,
                         float* codebook, float* s_channel, void* ws, size_t ws_bytes, hipStream_t stream) {
    cr_status s;
    if ((s = check_encode_shape(N, K)) != CR_OK) return s;
    if (iters < 1 || iters > 1000) return fail(CR_ERR_SHAPE, "iters=%d (need 1..1000)", iters);
    if (!w_bf16 || !idx || !s_rel_e4m3 || !codebook || !s_channel || !ws) return fail(CR_ERR_NULL, "NULL argument");
    if (!aligned16(w_bf16) || !aligned16(ws)) return fail(CR_ERR_ALIGN, "weight or workspace not 16-byte aligned");
    const size_t need = cr::encode_w4a8_workspace(N, K);
    if (ws_bytes < need) return fail(CR_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    if ((s = check_device()) != CR_OK) return s;
    return launch_err(cr::launch_encode_w4a8(static_cast<const uint16_t*>(w_bf16), N, K, iters,
                                             static_cast<uint8_t*>(idx), static_cast<uint8_t*>(s_rel_e4m3), codebook,
                                             s_channel, ws, stream),
                      "W4A8 encoder");
}

cr_status cr_dbg_e4m3_encode(const float* v, size_t n, void* codes, hipStream_t stream) {
    if (n == 0) return ok();
    if (!v || !codes) return fail(CR_ERR_NULL, "NULL argument");
    if (n > ((size_t)1 << 32)) return fail(CR_ERR_SHAPE, "n=%zu too large", n);
    cr_status s;
    if ((s = check_device()) != CR_OK) return s;
    return launch_err(cr::launch_e4m3_encode(v, n, static_cast<uint8_t*>(codes), stream), "e4m3 encode");
}

cr_status cr_pack_weight_int8rot(const void* w_bf16, int N, int K, void* w_packed, float* w_scale,
                                 hipStream_t stream) {
    cr_status s = pack_common_checks(CR_INT8ROT, w_bf16, N, K, w_packed, w_scale);
    if (s != CR_OK) return s;
    return launch_err(cr::launch_pack_i8rot(static_cast<const uint16_t*>(w_bf16), N, K,
                                            static_cast<uint8_t*>(w_packed), w_scale, stream),
                      "ConvRot INT8 weight packing");
}

cr_status cr_linear_int8rot(const void* x_bf16, int M, int K, const void* w_packed, const float* w_scale,
                            int N, const void* bias_bf16, void* y_bf16, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
    return run_linear(CR_INT8ROT, x_bf16, M, K, w_packed, w_scale, N, bias_bf16, y_bf16, nullptr, ws,
                      ws_bytes, stream);
}

cr_status cr_linear_w4a4(const void* x_bf16, int M, int K, const void* w_packed, const float* w_scale,
                         int N, const void* bias_bf16, void* y_bf16, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
    return run_linear(CR_W4A4, x_bf16, M, K, w_packed, w_scale, N, bias_bf16, y_bf16, nullptr, ws,
                      ws_bytes, stream);
}

cr_status cr_linear_w4a4_noalloc(const void* x_bf16, int M, int K, const void* w_packed, const float* w_scale,
                                 int N, const void* bias_bf16, void* y_bf16, hipStream_t stream) {
    // the same checks as cr_linear_w4a4 (the workspace pointer stands in as non-null)
    cr_status s = check_linear_args(CR_W4A4, M, K, w_packed, w_scale, N, bias_bf16, y_bf16, nullptr, w_packed);
    if (s != CR_OK) return s;
    if (M == 0) return ok();
    if (x_bf16 == nullptr) return fail(CR_ERR_NULL, "x is NULL");
    if (!aligned16(x_bf16)) return fail(CR_ERR_ALIGN, "x not 16-byte aligned");
    const size_t need = ws_layout(CR_W4A4, M, N, K).total;
    if (need > kScratchBytes)
        return fail(CR_ERR_WORKSPACE, "M=%d N=%d K=%d needs %zu bytes of workspace; the static scratch of the "
                    "no-allocation entry point holds %zu (use cr_linear_w4a4 with a workspace)",
                    M, N, K, need, kScratchBytes);
    if ((s = check_device()) != CR_OK) return s;
    void* ws = nullptr;
    if ((s = scratch_address(&ws)) != CR_OK) return s;
    return linear_phases(CR_W4A4, x_bf16, M, K, w_packed, w_scale, N, bias_bf16, y_bf16, nullptr, ws, kScratchBytes,
                         stream);
}

cr_status cr_linear_int8tw(const void* x_bf16, int M, int K, const void* w_packed, const float* w_scale,
                           int N, const void* bias_bf16, void* y_bf16, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
    return run_linear(CR_INT8TW, x_bf16, M, K, w_packed, w_scale, N, bias_bf16, y_bf16, nullptr, ws,
                      ws_bytes, stream);
}

cr_status cr_linear_w4a8(const void* x_bf16, int M, int K, const void* w_packed, const float* s_channel,
                         int N, const void* bias_bf16, void* y_bf16, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
    return run_linear(CR_W4A8, x_bf16, M, K, w_packed, s_channel, N, bias_bf16, y_bf16, nullptr, ws,
                      ws_bytes, stream);
}

cr_status cr_quantize_activations(int kind, const void* x_bf16, int M, int K, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
    cr_status s;
    if ((s = check_kind(kind)) != CR_OK) return s;
    if ((s = check_m(M)) != CR_OK) return s;
    if ((s = check_nk(kind, 1, K)) != CR_OK) return s;
    if (M == 0) return ok();
    if (x_bf16 == nullptr || ws == nullptr) return fail(CR_ERR_NULL, "x or workspace is NULL");
    if (!aligned16(x_bf16) || !aligned16(ws)) return fail(CR_ERR_ALIGN, "pointer not 16-byte aligned");
    if ((s = check_device()) != CR_OK) return s;
    return quantize_phase(kind, x_bf16, M, K, ws, ws_bytes, stream);
}

cr_status cr_gemm_quantized(int kind, int M, int K, const void* w_packed, const float* w_scale, int N,
                            const void* bias_bf16, void* y_bf16, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
    cr_status s = check_linear_args(kind, M, K, w_packed, w_scale, N, bias_bf16, y_bf16, nullptr, ws);
    if (s != CR_OK) return s;
    if (M == 0) return ok();
    if ((s = check_device()) != CR_OK) return s;
    return gemm_phase(kind, M, K, w_packed, w_scale, N, bias_bf16, y_bf16, nullptr, ws, ws_bytes, stream);
}

const char* cr_status_str(cr_status s) {
    switch (s) {
        case CR_OK: return "CR_OK";
        case CR_ERR_NULL: return "CR_ERR_NULL";
        case CR_ERR_SHAPE: return "CR_ERR_SHAPE";
        case CR_ERR_GROUP: return "CR_ERR_GROUP";
        case CR_ERR_ALIGN: return "CR_ERR_ALIGN";
        case CR_ERR_WORKSPACE: return "CR_ERR_WORKSPACE";
        case CR_ERR_DEVICE: return "CR_ERR_DEVICE";
        case CR_ERR_LAUNCH: return "CR_ERR_LAUNCH";
        case CR_ERR_KIND: return "CR_ERR_KIND";
        default: return "CR_ERR_UNKNOWN";
    }
}

const char* cr_last_error(void) { return g_err; }

cr_status cr_dbg_quant_act(int kind, const void* x_bf16, int M, int K, void* codes, float* scales,
                           hipStream_t stream) {
    cr_status s;
    if ((s = check_kind(kind)) != CR_OK) return s;
    if (M < 0 || M > CR_MAX_DIM) return fail(CR_ERR_SHAPE, "bad M=%d", M);
    if ((s = check_nk(kind, 1, K)) != CR_OK) return s;
    if (M == 0) return ok();
    if (x_bf16 == nullptr || codes == nullptr || scales == nullptr) return fail(CR_ERR_NULL, "NULL argument");
    if (!aligned16(x_bf16) || !aligned16(codes)) return fail(CR_ERR_ALIGN, "pointer not 16-byte aligned");
    if ((s = check_device()) != CR_OK) return s;
    const int wk = wkind(kind);
    return launch_err(cr::launch_quant_act(wk, group_of(kind), static_cast<const uint16_t*>(x_bf16), M, K, K,
                                           static_cast<int8_t*>(codes), scales, nullptr, false, nullptr, stream),
                      "activation quantisation");
}

cr_status cr_dbg_unpack_weight(int kind, const void* w_packed, int N, int K, void* codes,
                               hipStream_t stream) {
    cr_status s;
    if ((s = check_kind(kind)) != CR_OK) return s;
    if ((s = check_nk(kind, N, K)) != CR_OK) return s;
    if (w_packed == nullptr || codes == nullptr) return fail(CR_ERR_NULL, "NULL argument");
    if (!aligned16(w_packed)) return fail(CR_ERR_ALIGN, "pointer not 16-byte aligned");
    if ((s = check_device()) != CR_OK) return s;
    const int wk = wkind(kind);
    return launch_err(cr::launch_unpack_weight(wk, static_cast<const uint8_t*>(w_packed), N, K,
                                               static_cast<int8_t*>(codes), stream),
                      "weight unpacking");
}

cr_status cr_dbg_linear_acc(int kind, const void* x_bf16, int M, int K, const void* w_packed, int N,
                            int32_t* acc, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (acc == nullptr && M > 0) return fail(CR_ERR_NULL, "accumulator output is NULL");
    return run_linear(kind, x_bf16, M, K, w_packed, nullptr, N, nullptr, nullptr, acc, ws, ws_bytes,
                      stream);
}

cr_status cr_dbg_fused_config(int mode, int spin_limit) {
    if (mode < 0 || mode > 2) return fail(CR_ERR_SHAPE, "mode must be 0, 1 or 2, got %d", mode);
    g_fused_mode.store(mode);
    if (spin_limit >= 0) cr::set_fused_spin_limit(spin_limit);
    return ok();
}

cr_status cr_dbg_big_plan(int bn, int splits) {
    if (bn != 0 && bn != 64 && bn != 128 && bn != 192 && bn != 256)
        return fail(CR_ERR_SHAPE, "bn must be 0, 64, 128, 192 or 256, got %d", bn);
    if (splits < 0 || splits > 16) return fail(CR_ERR_SHAPE, "splits must be 0..16, got %d", splits);
    cr::set_big_plan_override(bn, splits);
    return ok();
}

cr_status cr_dbg_small_plan(int splits) {
    if (splits < 0 || splits > 16) return fail(CR_ERR_SHAPE, "splits must be 0..16, got %d", splits);
    cr::set_small_plan_override(splits);
    return ok();
}

cr_status cr_dbg_fused_timeouts(uint32_t* count) {
    if (count == nullptr) return fail(CR_ERR_NULL, "count is NULL");
    cr_status s;
    if ((s = check_device()) != CR_OK) return s;
    return launch_err(cr::fused_timeouts(count), "reading the fused linear's timeout counter");
}

}  // extern "C"
