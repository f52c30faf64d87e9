// Measurement probes (convrot_probe.h): the matrix-core, cold-read and copy
// ceilings the benchmark reports beside the spec peaks.  No kernel here
// touches the linear's data.
#include <hip/hip_runtime.h>

#include "convrot_probe.h"
#include "cr_device.h"

namespace {

constexpr int kProbeChains = 4;      // independent accumulator chains per wave
constexpr int kReadUnroll = 4;       // 16-byte loads in flight per thread
constexpr int kSinkWords = 4096;     // cr_probe_read's sink size, in uint32

// Every wave runs kProbeChains independent chains of 32x32x32 int8 MFMAs on
// operands derived from its lane id (the values do not matter to the rate).
__global__ void __launch_bounds__(512) k_probe_mfma(int iters, int32_t* sink, uint64_t* stamps) {
    const uint32_t t = threadIdx.x + 512u * blockIdx.x;
    v4i a, b;
    a.x = (int)(t * 0x9E3779B1u); a.y = (int)(t * 0x85EBCA77u); a.z = (int)(t ^ 0xC2B2AE3Du); a.w = (int)(t + 0x27D4EB2Fu);
    b.x = a.w; b.y = a.z ^ 0x5555; b.z = a.y + 7; b.w = a.x ^ 0x1234567;
    v16i acc[kProbeChains];
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = c + r;
    const uint64_t c0 = __builtin_amdgcn_s_memtime(), w0 = __builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < kProbeChains; ++c) acc[c] = cr::mfma32(a, b, acc[c]);
    }
    int s = 0;
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s ^= acc[c][r];
    const uint64_t c1 = __builtin_amdgcn_s_memtime(), w1 = __builtin_amdgcn_s_memrealtime();
    sink[t] = s;
    if (t == 0) {
        stamps[0] = c0; stamps[1] = c1; stamps[2] = w0; stamps[3] = w1;
    }
}

// Grid-stride read of n16 16-byte words, kReadUnroll loads issued per thread
// before any is used; one xor-fold per block goes to sink.
__global__ void __launch_bounds__(256) k_probe_read(const uint4* src, size_t n16, uint32_t* sink) {
    __shared__ uint32_t part[4];
    const size_t stride = (size_t)gridDim.x * 256 * kReadUnroll;
    uint32_t x = 0;
    for (size_t base = (size_t)blockIdx.x * 256 * kReadUnroll + threadIdx.x; base < n16; base += stride) {
        uint4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) {
            const size_t i = base + (size_t)u * 256;
            v[u] = i < n16 ? src[i] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // fold the block's values so the loads stay live
    for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

__global__ void __launch_bounds__(256) k_probe_copy(const uint4* src, uint4* dst, size_t n16) {
    const size_t stride = (size_t)gridDim.x * 256 * kReadUnroll;
    for (size_t base = (size_t)blockIdx.x * 256 * kReadUnroll + threadIdx.x; base < n16; base += stride) {
        uint4 v[kReadUnroll];
        if (base + (size_t)(kReadUnroll - 1) * 256 < n16) {     // all loads issued before any store
#pragma unroll
            for (int u = 0; u < kReadUnroll; ++u) v[u] = src[base + (size_t)u * 256];
#pragma unroll
            for (int u = 0; u < kReadUnroll; ++u) dst[base + (size_t)u * 256] = v[u];
        } else {
            for (int u = 0; u < kReadUnroll; ++u) {
                const size_t i = base + (size_t)u * 256;
                if (i < n16) dst[i] = src[i];
            }
        }
    }
}

// Blocks of a grid-stride probe over n16 words: enough for one pass with
// kReadUnroll loads per thread, at most kSinkWords.
unsigned probe_grid(size_t n16) {
    const size_t per_block = (size_t)256 * kReadUnroll;
    size_t g = (n16 + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > (size_t)kSinkWords) g = kSinkWords;
    return (unsigned)g;
}

cr_status launched() { return hipGetLastError() == hipSuccess ? CR_OK : CR_ERR_LAUNCH; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

cr_status cr_probe_mfma_i8(int blocks, int iters, int32_t* sink, uint64_t* stamps, hipStream_t stream) {
    if (blocks < 1 || blocks > 65535 || iters < 1 || iters > (1 << 24)) return CR_ERR_SHAPE;
    if (sink == nullptr || stamps == nullptr) return CR_ERR_NULL;
    k_probe_mfma<<<dim3(blocks), dim3(512), 0, stream>>>(iters, sink, stamps);
    return launched();
}

cr_status cr_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
    if (bytes == 0 || bytes % 16 != 0 || bytes > ((size_t)1 << 36)) return CR_ERR_SHAPE;
    if (src == nullptr || sink == nullptr) return CR_ERR_NULL;
    if (!aligned16(src)) return CR_ERR_ALIGN;
    const size_t n16 = bytes / 16;
    k_probe_read<<<dim3(probe_grid(n16)), dim3(256), 0, stream>>>(static_cast<const uint4*>(src), n16, sink);
    return launched();
}

cr_status cr_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
    if (bytes == 0 || bytes % 16 != 0 || bytes > ((size_t)1 << 36)) return CR_ERR_SHAPE;
    if (src == nullptr || dst == nullptr) return CR_ERR_NULL;
    if (!aligned16(src) || !aligned16(dst)) return CR_ERR_ALIGN;
    const char* s = static_cast<const char*>(src);
    const char* d = static_cast<const char*>(dst);
    if (s < d + bytes && d < s + bytes) return CR_ERR_SHAPE;
    const size_t n16 = bytes / 16;
    k_probe_copy<<<dim3(probe_grid(n16)), dim3(256), 0, stream>>>(static_cast<const uint4*>(src),
                                                                 static_cast<uint4*>(dst), n16);
    return launched();
}

int cr_probe_wall_clock_khz(void) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
    return khz;
}

}  // extern "C"
