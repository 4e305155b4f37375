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
// One wave64 per token, lanes over 16-byte column vectors.  The token's
// valid rows (pos >= 0) are compacted in k order; a body sized for that count
// then keeps NV x U independent 16-byte loads in flight per lane (NV rows x U
// column vectors, 8 to 16 in all) before accumulating each column vector over
// the rows in k order.  A token with no local row gets zeros.  When the
// output alone is a large share of the 256 MB last-level cache, the rows
// cannot still be cached from the GEMM that wrote them, and they are read
// with non-temporal loads (which cost time when the rows are still cached).
#include "moe_common.hpp"

namespace moe {

template <bool GATED, bool NT, int NV, int U>
__device__ __forceinline__ void combine_rows(const u32x4* __restrict__ y, const int (&rows)[16], const float (&g)[16],
                                             int nv_rows, int nv, int lane, u32x4* __restrict__ orow) {
    for (int v0 = 0; v0 < nv; v0 += 64 * U) {
        u32x4 buf[NV][U];
#pragma unroll
        for (int r = 0; r < NV; ++r) {
            const u32x4* src = y + (int64_t)rows[r] * nv;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = v0 + u * 64 + lane;
                if (r < nv_rows && v < nv) buf[r][u] = NT ? __builtin_nontemporal_load(src + v) : src[v];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * 64 + lane;
            if (v >= nv) continue;
            float acc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
            for (int r = 0; r < NV; ++r) {
                if (r >= nv_rows) continue;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float lo = bf_lo(buf[r][u][i]), hi = bf_hi(buf[r][u][i]);
                    if (GATED) {
                        acc[2 * i] += g[r] * lo;
                        acc[2 * i + 1] += g[r] * hi;
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
}

template <bool GATED, bool NT>
__global__ __launch_bounds__(256) void combine_kernel(const u32x4* __restrict__ y, const int32_t* __restrict__ pos,
                                                      const float* __restrict__ gates, int T, int K, int H,
                                                      u32x4* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t >= T) return;
    const int my_pos = lane < K ? pos[t * K + lane] : -1;
    float my_g = 1.0f;
    if (GATED && lane < K) my_g = gates[t * K + lane];
    // compact the valid k in ascending order (uniform over the wave)
    uint64_t m = __ballot(my_pos >= 0);
    const int nv_rows = __popcll(m);
    int rows[16];
    float g[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        // the same in every lane: read from lane k into scalar registers
        const int k = m ? __builtin_ctzll(m) : 0;
        rows[r] = __builtin_amdgcn_readlane(my_pos, k);
        g[r] = GATED ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_g), k)) : 1.0f;
        m &= m - 1;
    }
    const int nv = H >> 3;
    u32x4* orow = out + t * nv;
    if (nv_rows == 0) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        for (int v = lane; v < nv; v += 64) __builtin_nontemporal_store(z, orow + v);
    } else if (nv_rows == 1) {
        combine_rows<GATED, NT, 1, 8>(y, rows, g, nv_rows, nv, lane, orow);
    } else if (nv_rows <= 2) {
        combine_rows<GATED, NT, 2, 4>(y, rows, g, nv_rows, nv, lane, orow);
    } else if (nv_rows <= 4) {
        combine_rows<GATED, NT, 4, 2>(y, rows, g, nv_rows, nv, lane, orow);
    } else if (nv_rows <= 8) {
        combine_rows<GATED, NT, 8, 2>(y, rows, g, nv_rows, nv, lane, orow);
    } else {
        combine_rows<GATED, NT, 16, 1>(y, rows, g, nv_rows, nv, lane, orow);
    }
}

// dy_perm[pos[t,k]] = bf16(gate[t,k] * d_out[t]), the d_out row read once,
// and with DG the gate gradient dgates[t,k] = <d_out[t], y[pos[t,k]]>: each
// local row's dot product is a per-lane fp32 sum over its column vectors (8
// products each, in order) followed by a fixed butterfly over the lanes.
template <bool GATED, bool DG, int NV, int U>
__device__ __forceinline__ void gather_rows(const u32x4* __restrict__ src, const u32x4* __restrict__ y,
                                            const int (&rows)[16], const float (&g)[16], int nv_rows, int nv,
                                            int lane, u32x4* __restrict__ dy_perm, float (&dot)[16]) {
    for (int v0 = 0; v0 < nv; v0 += 64 * U) {
        u32x4 buf[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * 64 + lane;
            if (v < nv) buf[u] = __builtin_nontemporal_load(src + v);
        }
        u32x4 yb[NV][U];
        if (DG) {
#pragma unroll
            for (int r = 0; r < NV; ++r) {
                const u32x4* yr = y + (int64_t)rows[r] * nv;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int v = v0 + u * 64 + lane;
                    if (r < nv_rows && v < nv) yb[r][u] = yr[v];
                }
            }
        }
#pragma unroll
        for (int r = 0; r < NV; ++r) {
            if (r >= nv_rows) continue;
            u32x4* dst = dy_perm + (int64_t)rows[r] * nv;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = v0 + u * 64 + lane;
                if (v >= nv) continue;
                u32x4 o;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (GATED)
                        o[i] = pack_bf2(g[r] * bf_lo(buf[u][i]), g[r] * bf_hi(buf[u][i]));
                    else
                        o[i] = buf[u][i];
                }
                dst[v] = o;
                if (DG) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        dot[r] += bf_lo(buf[u][i]) * bf_lo(yb[r][u][i]);
                        dot[r] += bf_hi(buf[u][i]) * bf_hi(yb[r][u][i]);
                    }
                }
            }
        }
    }
}

template <bool GATED, bool DG>
__global__ __launch_bounds__(256) void gather_kernel(const u32x4* __restrict__ d_out, const int32_t* __restrict__ pos,
                                                     const float* __restrict__ gates, const u32x4* __restrict__ y,
                                                     int T, int K, int H, u32x4* __restrict__ dy_perm,
                                                     float* __restrict__ dgates) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t >= T) return;
    const int my_pos = lane < K ? pos[t * K + lane] : -1;
    float my_g = 1.0f;
    if (GATED && lane < K) my_g = gates[t * K + lane];
    uint64_t m = __ballot(my_pos >= 0);
    const uint64_t local = m;
    const int nv_rows = __popcll(m);
    int rows[16];
    float g[16], dot[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        // the same in every lane: read from lane k into scalar registers
        const int k = m ? __builtin_ctzll(m) : 0;
        rows[r] = __builtin_amdgcn_readlane(my_pos, k);
        g[r] = GATED ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_g), k)) : 1.0f;
        dot[r] = 0.0f;
        m &= m - 1;
    }
    const int nv = H >> 3;
    const u32x4* src = d_out + t * nv;
    if (nv_rows == 0) {
        // nothing to gather; the gate gradients are 0
    } else if (nv_rows <= 2) {
        gather_rows<GATED, DG, 2, 4>(src, y, rows, g, nv_rows, nv, lane, dy_perm, dot);
    } else if (nv_rows <= 4) {
        gather_rows<GATED, DG, 4, 2>(src, y, rows, g, nv_rows, nv, lane, dy_perm, dot);
    } else if (nv_rows <= 8) {
        gather_rows<GATED, DG, 8, 2>(src, y, rows, g, nv_rows, nv, lane, dy_perm, dot);
    } else {
        gather_rows<GATED, DG, 16, 1>(src, y, rows, g, nv_rows, nv, lane, dy_perm, dot);
    }
    if (DG) {
        // lane k < K holds pair k; a local pair is compacted row popc(local below k)
        const int my_r = __popcll(local & ((1ull << lane) - 1));
        float mine = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if (r >= nv_rows) continue;
            float v = dot[r];
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
            if (my_r == r) mine = v;
        }
        if (lane < K) dgates[t * K + lane] = ((local >> lane) & 1) ? mine : 0.0f;
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
    // an output of 64 MiB or more: a quarter of the last-level cache
    const bool nt = (int64_t)T * H * 2 >= (64ll << 20);
    if (gates) {
        if (nt) combine_kernel<true, true><<<grid, block, 0, s>>>(yy, pos, gates, T, K, H, oo);
        else combine_kernel<true, false><<<grid, block, 0, s>>>(yy, pos, gates, T, K, H, oo);
    } else {
        if (nt) combine_kernel<false, true><<<grid, block, 0, s>>>(yy, pos, gates, T, K, H, oo);
        else combine_kernel<false, false><<<grid, block, 0, s>>>(yy, pos, gates, T, K, H, oo);
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
    const u32x4* d = (const u32x4*)d_out;
    u32x4* o = (u32x4*)dy_perm;
    if (gates)
        gather_kernel<true, false><<<grid, block, 0, s>>>(d, pos, gates, nullptr, T, K, H, o, nullptr);
    else
        gather_kernel<false, false><<<grid, block, 0, s>>>(d, pos, gates, nullptr, T, K, H, o, nullptr);
    return moe_host::launch_status();
}

extern "C" int moe_gather_gate_grad(const moe_bf16* d_out, const int32_t* pos, const float* gates,
                                    const moe_bf16* y, int T, int K, int H, moe_bf16* dy_perm, float* dgates,
                                    moe_stream stream) {
    using namespace moe;
    using moe_host::misaligned;
    if (T < 0 || K < 1 || K > 16 || H < 0) return MOE_EINVAL;
    if ((int64_t)T * K >= (1ll << 31)) return MOE_EINVAL;
    if (H % 64 != 0) return MOE_ESHAPE;
    if (T == 0) return MOE_OK;
    if (!d_out || !pos || !gates || !y || !dy_perm || !dgates) return MOE_EINVAL;
    if (misaligned(d_out) || misaligned(pos) || misaligned(gates) || misaligned(y) || misaligned(dy_perm) ||
        misaligned(dgates))
        return MOE_EALIGN;
    hipStream_t s = (hipStream_t)stream;
    dim3 grid((T + 3) / 4), block(256);
    gather_kernel<true, true><<<grid, block, 0, s>>>((const u32x4*)d_out, pos, gates, (const u32x4*)y, T, K, H,
                                                     (u32x4*)dy_perm, dgates);
    return moe_host::launch_status();
}
