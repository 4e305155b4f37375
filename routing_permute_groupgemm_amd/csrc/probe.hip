// MFMA throughput probe: a measurement aid beside the layer's path.
//
// The GroupGEMMs are priced against the bf16 MFMA peak of the data sheet
// (256 CUs x 4096 flop per clock x 2.4 GHz).  Under sustained MFMA load the
// chip holds a lower clock, and how much lower depends on the operand bits,
// so a bench also reports what back-to-back MFMAs reach on this GPU with the
// caller's operands: every wave keeps four A and four B fragments in
// registers and runs a 4 x 4 block of independent 32x32x16 bf16 MFMAs, the
// accumulator footprint of the GroupGEMM's 128 x 128 wave tile, with no
// memory traffic inside the loop.  The second kernel does the same with
// 16x16x32 bf16 MFMAs (an 8 x 8 block, eight A and eight B fragments), the
// other MFMA shape of the same bf16 rate on paper.
//
// The copy probe does the same for the HBM-bound steps: a streaming copy of
// a large buffer, 16-byte loads and stores, fully coalesced, four loads in
// flight per lane, with or without the non-temporal hint on either side.  The
// best rate it reaches is the practical ceiling of a kernel that reads and
// writes as many bytes as it moves, beside the 8 TB/s of the data sheet.
#include "moe_common.hpp"

namespace moe {

__global__ __launch_bounds__(256) void mfma_probe_kernel(const bf16x8* __restrict__ ops, int iters,
                                                         float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const bf16x8* o = ops + w * 8 * 64 + lane;
    bf16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = o[i * 64];
        b[i] = o[(4 + i) * 64];
    }
    f32x16 acc[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[m][n] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int n = 0; n < 4; ++n)
                acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m], b[n], acc[m][n], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) s += acc[m][n][i];
    out[w * 64 + lane] = s;
}

// The same 128 x 128 accumulator footprint on v_mfma_f32_16x16x32_bf16: fragments
// 0..7 of a wave are A, 8..15 B; lane l holds row / column l%16 and k values
// 8*(l/16) + 0..7 of its fragment.
__global__ __launch_bounds__(256) void mfma16_probe_kernel(const bf16x8* __restrict__ ops, int iters,
                                                           float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const bf16x8* o = ops + w * 16 * 64 + lane;
    bf16x8 a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = o[i * 64];
        b[i] = o[(8 + i) * 64];
    }
    f32x4 acc[8][8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[m][n] = f32x4{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int n = 0; n < 8; ++n)
                acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m], b[n], acc[m][n], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int n = 0; n < 8; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) s += acc[m][n][i];
    out[w * 64 + lane] = s;
}

// A block copies 1024 consecutive 16-byte words per pass (lane t: words t,
// t+256, t+512, t+768), then strides over the grid.  NT bit 0: non-temporal
// loads, bit 1: non-temporal stores.
template <int NT>
__global__ __launch_bounds__(256) void copy_probe_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * 1024;
    for (int64_t base = (int64_t)blockIdx.x * 1024 + threadIdx.x; base < n16; base += stride) {
        u32x4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t i = base + 256 * j;
            if (i < n16) v[j] = (NT & 1) ? __builtin_nontemporal_load(src + i) : src[i];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t i = base + 256 * j;
            if (i < n16) {
                if (NT & 2)
                    __builtin_nontemporal_store(v[j], dst + i);
                else
                    dst[i] = v[j];
            }
        }
    }
}

}  // namespace moe

extern "C" int moe_probe_copy(const void* src, void* dst, int64_t bytes, int nontemporal, int blocks,
                              moe_stream stream) {
    if (bytes < 0 || (bytes & 15) || nontemporal < 0 || nontemporal > 3 || blocks < 0 || blocks > (1 << 20))
        return MOE_EINVAL;
    if (bytes == 0) return MOE_OK;
    if (!src || !dst) return MOE_EINVAL;
    if (moe_host::misaligned(src) || moe_host::misaligned(dst)) return MOE_EALIGN;
    const int64_t n16 = bytes / 16;
    const int64_t need = (n16 + 1023) / 1024;
    const int64_t grid = std::min<int64_t>(need, blocks ? blocks : (int64_t)moe_host::num_cus() * 8);
    const auto* s = (const moe::u32x4*)src;
    auto* d = (moe::u32x4*)dst;
    hipStream_t st = (hipStream_t)stream;
    switch (nontemporal) {
        case 0: moe::copy_probe_kernel<0><<<(int)grid, 256, 0, st>>>(s, d, n16); break;
        case 1: moe::copy_probe_kernel<1><<<(int)grid, 256, 0, st>>>(s, d, n16); break;
        case 2: moe::copy_probe_kernel<2><<<(int)grid, 256, 0, st>>>(s, d, n16); break;
        default: moe::copy_probe_kernel<3><<<(int)grid, 256, 0, st>>>(s, d, n16); break;
    }
    return moe_host::launch_status();
}

extern "C" int moe_probe_mfma(const moe_bf16* operands, int blocks, int iters, float* out, moe_stream stream) {
    if (blocks < 1 || blocks > (1 << 20) || iters < 0 || !operands || !out) return MOE_EINVAL;
    if (moe_host::misaligned(operands) || moe_host::misaligned(out)) return MOE_EALIGN;
    moe::mfma_probe_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>((const moe::bf16x8*)operands, iters, out);
    return moe_host::launch_status();
}

extern "C" int moe_probe_mfma16(const moe_bf16* operands, int blocks, int iters, float* out, moe_stream stream) {
    if (blocks < 1 || blocks > (1 << 20) || iters < 0 || !operands || !out) return MOE_EINVAL;
    if (moe_host::misaligned(operands) || moe_host::misaligned(out)) return MOE_EALIGN;
    moe::mfma16_probe_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>((const moe::bf16x8*)operands, iters, out);
    return moe_host::launch_status();
}
