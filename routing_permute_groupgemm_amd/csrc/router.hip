// Elementwise passes of the router projection and its backward.
//
// UniEP paper, "MoE workflow": the router network gives every token a score
// per expert.  Here that is logits = x . W_r (+ a per-expert bias) on the
// GroupGEMM kernel as one dense group; when the contraction is split into
// chunks for parallelism, each chunk leaves an fp32 partial and the pass
// below adds the partials in chunk order, so the result does not depend on
// scheduling.  The backward takes the score gradient in bf16 (as every other
// activation gradient of the path), which the second pass rounds.
#include "moe_common.hpp"

namespace moe {

// out[i] = part[0][i] + part[1][i] + ... (chunk order) + bias[i % period]
__global__ __launch_bounds__(256) void sum_partials_kernel(const f32x4* __restrict__ part, int S, int64_t n4,
                                                           int64_t stride4, const float* __restrict__ bias,
                                                           int period, f32x4* __restrict__ out) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
        f32x4 acc = __builtin_nontemporal_load(part + i);
        for (int s = 1; s < S; ++s) acc += __builtin_nontemporal_load(part + s * stride4 + i);
        if (bias) acc += *(const f32x4*)(bias + (i * 4) % period);
        out[i] = acc;
    }
}

// 8 fp32 -> 8 bf16 (nearest even) per thread and step
__global__ __launch_bounds__(256) void cast_bf16_kernel(const f32x4* __restrict__ in, int64_t n8,
                                                        u32x4* __restrict__ out) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
        const f32x4 a = __builtin_nontemporal_load(in + 2 * i);
        const f32x4 b = __builtin_nontemporal_load(in + 2 * i + 1);
        out[i] = u32x4{pack_bf2(a[0], a[1]), pack_bf2(a[2], a[3]), pack_bf2(b[0], b[1]), pack_bf2(b[2], b[3])};
    }
}

}  // namespace moe

namespace moe_host {

static int grid_for(int64_t items) {
    const int64_t blocks = (items + 255) / 256;
    return (int)std::min<int64_t>(blocks, (int64_t)num_cus() * 8);
}

int sum_partials(const float* part, int S, int64_t n, int64_t stride, const float* bias, int period, float* out,
                 hipStream_t s) {
    const int64_t n4 = n / 4;
    if (n4 == 0) return MOE_OK;
    moe::sum_partials_kernel<<<grid_for(n4), 256, 0, s>>>((const moe::f32x4*)part, S, n4, stride / 4, bias, period,
                                                          (moe::f32x4*)out);
    return launch_status();
}

int cast_f32_bf16(const float* in, int64_t n, uint16_t* out, hipStream_t s) {
    const int64_t n8 = n / 8;
    if (n8 == 0) return MOE_OK;
    moe::cast_bf16_kernel<<<grid_for(n8), 256, 0, s>>>((const moe::f32x4*)in, n8, (moe::u32x4*)out);
    return launch_status();
}

}  // namespace moe_host
