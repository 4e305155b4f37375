// Routing: softmax over router scores and top-k with a total order.
//
// UniEP paper, "MoE workflow": the router gives each token a probability
// distribution over the experts and each token is sent to its top-k.  The
// chosen experts are ordered by (score descending, expert id ascending);
// selecting on the fp32 scores equals selecting on the probabilities
// (softmax is monotonic) and is immune to rounding ties.  The gates are the
// chosen probabilities renormalised over the K choices; the softmax
// normaliser cancels, so g_k = exp(s_k - s_max) / sum_k' exp(s_k' - s_max).
//
// One wave64 per token.  Lane l holds the scores of experts l, l+64, ... as
// order-preserving 32-bit keys.  Each of the K rounds takes the lane's best
// remaining key (the lowest slot wins a tie inside the lane: lowest expert
// id), reduces the lane bests to the wave maximum with DPP row operations
// (no LDS round trips), and, if several lanes hold that score, takes the
// lowest expert id among them; the winner clears its key.  Row loads are
// lane-strided and coalesced.
#include "moe_common.hpp"

namespace moe {

__device__ __forceinline__ uint32_t score_key(float s) {
    if (s == 0.0f) s = 0.0f;  // -0 and +0 compare equal: canonicalise to +0
    uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // > 0 for every non-NaN score
}

__device__ __forceinline__ float key_score(uint32_t u) {
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// max / min over the 64 lanes: butterflies within each row of 16 (quad
// permutes, half-row and row mirrors), then row broadcasts bring every row
// into lane 63.  Lanes without a DPP source take the identity.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false));   // quad [1,0,3,2]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false));   // quad [2,3,0,1]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));  // row_half_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));  // row_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    const int id = -1;  // all ones: the identity of an unsigned min
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0xB1, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x4E, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x141, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x140, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x142, 0xa, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x143, 0xc, 0xf, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E, int K,
                                                    int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ gates) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float* row = logits + t * E;
    uint32_t key[EPL];  // 0 = absent or taken (below every score's key)
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = i * 64 + lane;
        key[i] = e < E ? score_key(__builtin_nontemporal_load(row + e)) : 0u;
    }
    int my_idx = 0;
    float my_score = 0.0f, s_max = 0.0f;
    for (int k = 0; k < K; ++k) {
        // the lane's best remaining key; strict > keeps the lowest slot on a tie
        uint32_t best = key[0];
        int bj = 0;
#pragma unroll
        for (int i = 1; i < EPL; ++i)
            if (key[i] > best) {
                best = key[i];
                bj = i;
            }
        const uint32_t m = wave_max_u32(best);
        const uint64_t tied = __ballot(best == m);
        int e_win;
        if (__popcll(tied) == 1) {
            const int wl = __builtin_ctzll(tied);
            e_win = __builtin_amdgcn_readlane(bj, wl) * 64 + wl;
        } else {
            // several lanes hold this score: the lowest expert id among them
            e_win = (int)wave_min_u32(best == m ? (uint32_t)(bj * 64 + lane) : 0xffffffffu);
        }
        e_win = __builtin_amdgcn_readfirstlane(e_win);
        if (lane == (e_win & 63)) {
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (i == (e_win >> 6)) key[i] = 0u;
        }
        const float s = key_score(m);
        if (k == 0) s_max = s;
        if (lane == k) {
            my_idx = e_win;
            my_score = s;
        }
    }
    // gates: lanes 0..K-1 hold one choice each; the sum runs over k ascending
    float ex = lane < K ? expf(my_score - s_max) : 0.0f;
    float z = 0.0f;
    for (int k = 0; k < K; ++k) z += __shfl(ex, k, 64);
    if (lane < K) {
        topk_idx[t * K + lane] = my_idx;
        gates[t * K + lane] = ex / z;
    }
}

// Router backward: one wave per token.  The gates are the softmax of the
// chosen scores, so with g, dg the token's gates and gate gradients the
// score gradient is g_k * (dg_k - sum_j g_j dg_j) at the chosen experts and 0
// elsewhere.  The sum runs over j ascending.  The K chosen experts and their
// values are wave-uniform: lane k holds choice k, and readlane copies them
// into scalar registers once.  Each lane then writes its experts lane,
// lane + 64, ..., selecting its value among the K choices, so the row is
// written once, coalesced.
template <int KMAX>
__global__ __launch_bounds__(256) void route_backward_kernel(const int32_t* __restrict__ topk_idx,
                                                             const float* __restrict__ gates,
                                                             const float* __restrict__ dgates, int T, int E, int K,
                                                             float* __restrict__ dlogits) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int my_idx = lane < K ? topk_idx[t * K + lane] : -1;
    const float my_g = lane < K ? gates[t * K + lane] : 0.0f;
    const float my_dg = lane < K ? dgates[t * K + lane] : 0.0f;
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (j < K) {
            const float gj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_g), j));
            const float dgj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_dg), j));
            sum += gj * dgj;
        }
    }
    const float my_val = my_g * (my_dg - sum);
    int ik[KMAX];
    float vk[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        ik[k] = k < K ? __builtin_amdgcn_readlane(my_idx, k) : -1;
        vk[k] = k < K ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_val), k)) : 0.0f;
    }
    float* row = dlogits + t * E;
    for (int e0 = 0; e0 < E; e0 += 64) {
        const int e = e0 + lane;
        float v = 0.0f;
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (ik[k] == e) v = vk[k];
        if (e < E) row[e] = v;
    }
}

}  // namespace moe

extern "C" int moe_route(const float* logits, int T, int E, int K, int32_t* topk_idx, float* gates,
                         moe_stream stream) {
    using namespace moe;
    if (T < 0 || E < 1 || E > 512 || K < 1 || K > 16) return MOE_EINVAL;
    if (K > E) return MOE_ESHAPE;
    if ((int64_t)T * K >= (1ll << 31) || (int64_t)T * E >= (1ll << 40)) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!logits || !topk_idx || !gates) return MOE_EINVAL;
    if (moe_host::misaligned(logits) || moe_host::misaligned(topk_idx) || moe_host::misaligned(gates))
        return MOE_EALIGN;
    hipStream_t s = (hipStream_t)stream;
    dim3 grid((T + 3) / 4), block(256);
    int epl = (E + 63) / 64;
    switch (epl) {
        case 1: route_kernel<1><<<grid, block, 0, s>>>(logits, T, E, K, topk_idx, gates); break;
        case 2: route_kernel<2><<<grid, block, 0, s>>>(logits, T, E, K, topk_idx, gates); break;
        case 3: route_kernel<3><<<grid, block, 0, s>>>(logits, T, E, K, topk_idx, gates); break;
        case 4: route_kernel<4><<<grid, block, 0, s>>>(logits, T, E, K, topk_idx, gates); break;
        case 5: route_kernel<5><<<grid, block, 0, s>>>(logits, T, E, K, topk_idx, gates); break;
        case 6: route_kernel<6><<<grid, block, 0, s>>>(logits, T, E, K, topk_idx, gates); break;
        case 7: route_kernel<7><<<grid, block, 0, s>>>(logits, T, E, K, topk_idx, gates); break;
        default: route_kernel<8><<<grid, block, 0, s>>>(logits, T, E, K, topk_idx, gates); break;
    }
    return moe_host::launch_status();
}

extern "C" int moe_route_backward(const int32_t* topk_idx, const float* gates, const float* dgates, int T, int E,
                                  int K, float* dlogits, moe_stream stream) {
    using namespace moe;
    if (T < 0 || E < 1 || E > 512 || K < 1 || K > 16) return MOE_EINVAL;
    if (K > E) return MOE_ESHAPE;
    if ((int64_t)T * K >= (1ll << 31) || (int64_t)T * E >= (1ll << 40)) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!topk_idx || !gates || !dgates || !dlogits) return MOE_EINVAL;
    if (moe_host::misaligned(topk_idx) || moe_host::misaligned(gates) || moe_host::misaligned(dgates) ||
        moe_host::misaligned(dlogits))
        return MOE_EALIGN;
    const dim3 grid((T + 3) / 4), block(256);
    hipStream_t s = (hipStream_t)stream;
    if (K <= 8) route_backward_kernel<8><<<grid, block, 0, s>>>(topk_idx, gates, dgates, T, E, K, dlogits);
    else route_backward_kernel<16><<<grid, block, 0, s>>>(topk_idx, gates, dgates, T, E, K, dlogits);
    return moe_host::launch_status();
}

extern "C" const char* moe_strerror(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_EINVAL: return "invalid argument (NULL pointer or size out of range)";
        case MOE_ESHAPE: return "unsupported shape (H/F not a multiple of 64, K > E, ...)";
        case MOE_EALIGN: return "pointer not 16-byte aligned";
        case MOE_EWORKSPACE: return "workspace missing or too small";
        case MOE_EHIP: return "HIP launch error";
        default: return "unknown status";
    }
}

extern "C" int moe_abi_version(void) { return 1; }

namespace moe_host {
int num_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}
}  // namespace moe_host
