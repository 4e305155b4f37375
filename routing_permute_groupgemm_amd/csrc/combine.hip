// Gate-weighted combine (forward), combine-gradient (backward) and the
// gate-scaled gather of the output gradient (backward).
//
// UniEP paper, "MoE workflow": expert outputs are weighted by their gating
// scores and aggregated back in token order; "Top-k accumulation
// constraint": a token's K contributions are summed only all together, in
// one fixed order (here k ascending, fp32 from +0, one bf16 rounding), never
// as partial sums; "Relay & Reduce Workers": one warp per token with vector
// loads and no shared memory.  MoonEP page: the dispatch gradient sums each
// token's K dispatched copies, i.e. the same combine without gates.
//
// One wave64 per token, lanes over 16-byte column vectors.  For every
// column vector the K source rows are loaded together (K independent 16-byte
// loads in flight per lane), then accumulated in k order.
#include "moe_common.hpp"

namespace moe {

template <bool GATED, int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const u32x4* __restrict__ y, const int32_t* __restrict__ pos,
                                                      const float* __restrict__ gates, int T, int K, int H,
                                                      u32x4* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int my_pos = lane < K ? pos[t * K + lane] : -1;
    float my_g = 1.0f;
    if (GATED && lane < K) my_g = gates[t * K + lane];
    int rows[KMAX];
    float g[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        rows[k] = k < K ? __shfl(my_pos, k, 64) : -1;
        g[k] = GATED ? __shfl(my_g, k, 64) : 1.0f;
    }
    const int nv = H >> 3;
    u32x4* orow = out + t * nv;
    for (int v = lane; v < nv; v += 64) {
        u32x4 buf[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (rows[k] >= 0) buf[k] = y[(int64_t)rows[k] * nv + v];
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (rows[k] < 0) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float lo = bf_lo(buf[k][i]), hi = bf_hi(buf[k][i]);
                if (GATED) {
                    acc[2 * i] += g[k] * lo;
                    acc[2 * i + 1] += g[k] * hi;
                } else {
                    acc[2 * i] += lo;
                    acc[2 * i + 1] += hi;
                }
            }
        }
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = pack_bf2(acc[2 * i], acc[2 * i + 1]);
        __builtin_nontemporal_store(o, orow + v);
    }
}

// dy_perm[pos[t,k]] = bf16(gate[t,k] * d_out[t]); the d_out row is read once.
template <bool GATED>
__global__ __launch_bounds__(256) void gather_kernel(const u32x4* __restrict__ d_out, const int32_t* __restrict__ pos,
                                                     const float* __restrict__ gates, int T, int K, int H,
                                                     u32x4* __restrict__ dy_perm) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int my_pos = lane < K ? pos[t * K + lane] : -1;
    if (__ballot(my_pos >= 0) == 0ull) return;
    float my_g = 1.0f;
    if (GATED && lane < K) my_g = gates[t * K + lane];
    const int nv = H >> 3;
    const u32x4* src = d_out + t * nv;
    constexpr int U = 4;
    for (int v0 = 0; v0 < nv; v0 += 64 * U) {
        u32x4 buf[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int v = v0 + u * 64 + lane;
            if (v < nv) buf[u] = __builtin_nontemporal_load(src + v);
        }
        for (int k = 0; k < K; ++k) {
            int r = __shfl(my_pos, k, 64);
            float gk = __shfl(my_g, k, 64);
            if (r < 0) continue;
            u32x4* dst = dy_perm + (int64_t)r * nv;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                int v = v0 + u * 64 + lane;
                if (v >= nv) continue;
                u32x4 o;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (GATED)
                        o[i] = pack_bf2(gk * bf_lo(buf[u][i]), gk * bf_hi(buf[u][i]));
                    else
                        o[i] = buf[u][i];
                }
                dst[v] = o;
            }
        }
    }
}

}  // namespace moe

extern "C" int moe_combine(const moe_bf16* y, const int32_t* pos, const float* gates, int T, int K, int H,
                           moe_bf16* out, moe_stream stream) {
    using namespace moe;
    using moe_host::misaligned;
    if (T < 0 || K < 1 || K > 16 || H < 0) return MOE_EINVAL;
    if ((int64_t)T * K >= (1ll << 31)) return MOE_EINVAL;
    if (H % 64 != 0) return MOE_ESHAPE;
    if (T == 0 || H == 0) return MOE_OK;
    if (!y || !pos || !out) return MOE_EINVAL;
    if (misaligned(y) || misaligned(pos) || misaligned(gates) || misaligned(out)) return MOE_EALIGN;
    hipStream_t s = (hipStream_t)stream;
    dim3 grid((T + 3) / 4), block(256);
    const u32x4* yy = (const u32x4*)y;
    u32x4* oo = (u32x4*)out;
    if (gates) {
        if (K <= 8) combine_kernel<true, 8><<<grid, block, 0, s>>>(yy, pos, gates, T, K, H, oo);
        else combine_kernel<true, 16><<<grid, block, 0, s>>>(yy, pos, gates, T, K, H, oo);
    } else {
        if (K <= 8) combine_kernel<false, 8><<<grid, block, 0, s>>>(yy, pos, gates, T, K, H, oo);
        else combine_kernel<false, 16><<<grid, block, 0, s>>>(yy, pos, gates, T, K, H, oo);
    }
    return moe_host::launch_status();
}

extern "C" int moe_gather(const moe_bf16* d_out, const int32_t* pos, const float* gates, int T, int K, int H,
                          moe_bf16* dy_perm, moe_stream stream) {
    using namespace moe;
    using moe_host::misaligned;
    if (T < 0 || K < 1 || K > 16 || H < 0) return MOE_EINVAL;
    if ((int64_t)T * K >= (1ll << 31)) return MOE_EINVAL;
    if (H % 64 != 0) return MOE_ESHAPE;
    if (T == 0 || H == 0) return MOE_OK;
    if (!d_out || !pos || !dy_perm) return MOE_EINVAL;
    if (misaligned(d_out) || misaligned(pos) || misaligned(gates) || misaligned(dy_perm)) return MOE_EALIGN;
    hipStream_t s = (hipStream_t)stream;
    dim3 grid((T + 3) / 4), block(256);
    if (gates)
        gather_kernel<true><<<grid, block, 0, s>>>((const u32x4*)d_out, pos, gates, T, K, H, (u32x4*)dy_perm);
    else
        gather_kernel<false><<<grid, block, 0, s>>>((const u32x4*)d_out, pos, gates, T, K, H, (u32x4*)dy_perm);
    return moe_host::launch_status();
}
