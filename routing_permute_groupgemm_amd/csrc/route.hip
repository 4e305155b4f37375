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
// A wave64 takes one token at a time.  Lane l holds the scores of experts l,
// l+64, ... as order-preserving 32-bit keys (row loads are lane-strided and
// coalesced).  The top K are found by a threshold and a rank count over the
// few candidates above it (route_kernel, below); tokens with too many
// candidates take K rounds of a wave maximum instead: each round takes the
// lane's best remaining key (the lowest slot wins a tie inside the lane:
// lowest expert id), reduces the lane bests to the wave maximum with DPP row
// operations, and, if several lanes hold that score, takes the lowest expert
// id among them; the winner clears its key.
#include "moe_common.hpp"

namespace moe {

typedef __attribute__((ext_vector_type(2))) unsigned long long u64x2;

__device__ __forceinline__ uint32_t score_key(float s) {
    // -0 and +0 compare equal: s + 0 is +0 for both (and s for every other s)
    const uint32_t u = __float_as_uint(s + 0.0f);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);  // negative: ~u; else u | sign; > 0 unless NaN
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

// The K rounds above, for one token whose lane l holds the keys of experts
// l, l + 64, ... (0: absent or taken).  On return lane k < K holds choice k
// (its expert id and score); s_max is the best score.
template <int EPL>
__device__ __forceinline__ void select_rounds(uint32_t (&key)[EPL], int K, int lane, int& my_idx, float& my_score,
                                              float& s_max) {
    my_idx = 0;
    my_score = 0.0f;
    s_max = 0.0f;
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
        const float sc = key_score(m);
        if (k == 0) s_max = sc;
        if (lane == k) {
            my_idx = e_win;
            my_score = sc;
        }
    }
}

// Top-K by a threshold and a rank count.  Split the lanes into G >= K groups
// (8 groups of 8 lanes for K <= 8, 16 of 4 for K <= 16): the G group maxima
// are G distinct experts, so the K-th best key is at least theta, the
// smallest group maximum, and every expert of the top K has a key >= theta.
// Those candidates (about 20 of 256 on the router scores of the layer's
// workloads) are compacted into LDS as 64-bit words key << 32 | ~id, whose
// unsigned order is (score descending, id ascending); lane c then counts the
// candidates above candidate c, which is its rank, and ranks 0..K-1 are the
// choices.  Tokens with more than 64 candidates (ties, or flat scores) take
// the K rounds instead.  Both paths give the same choices.
//
// A wave takes a batch of tb_n consecutive tokens (at most 64 / KP, KP the
// next power of two >= K; fewer when T is small, so that more waves share the
// work), one token at a time with the next row in flight.  The choices
// (expert id and score - s_max) go to LDS, slot KP*token + rank; after the
// batch, lane KP*i + k computes choice k of token i's gate,
// exp(s_k - s_max) / sum_k' exp(s_k' - s_max) with the sum taken over k'
// ascending, and the batch's ids and gates are written with one coalesced
// store each.  FULL: E is a multiple of 64 (no absent lanes).
template <int EPL, bool FULL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E, int K,
                                                    int kp_log2, int tb_n, int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ gates) {
    __shared__ __attribute__((aligned(16))) uint64_t s_cand[4][72];  // 64 candidates and 8 zero words
    __shared__ int s_bid[4][64];    // batch: chosen expert id, slot KP*token + rank
    __shared__ float s_bsc[4][64];  // batch: chosen score - s_max, then exp of it
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar loop control
    const int64_t n_batches = ((int64_t)T + tb_n - 1) / tb_n;
    const int64_t stride = (int64_t)gridDim.x * 4;
    uint64_t* cand = s_cand[wave];
    int* bid = s_bid[wave];
    float* bsc = s_bsc[wave];
    float raw[EPL];
    // branch-free row loads: lanes past E (and rows past T) load a valid
    // address, and their values are discarded
    auto load_row = [&](int64_t tt) {
        const float* row = logits + min(tt, (int64_t)T - 1) * E;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = i * 64 + lane;
            raw[i] = __builtin_nontemporal_load(row + (FULL || e < E ? e : 0));
        }
    };
    int64_t b = (int64_t)blockIdx.x * 4 + wave;
    load_row(b * tb_n);
    for (; b < n_batches; b += stride) {
        const int64_t t0 = b * tb_n;
        const int nt = (int)min((int64_t)tb_n, (int64_t)T - t0);
        for (int ti = 0; ti < nt; ++ti) {
            uint32_t key[EPL];  // 0 = absent (below every score's key)
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const uint32_t kv = score_key(raw[i]);
                key[i] = FULL || i * 64 + lane < E ? kv : 0u;
            }
            // the next row: this batch's next token, or the next batch's first
            load_row(ti + 1 < nt ? t0 + ti + 1 : (b + stride) * tb_n);

            // theta: the smallest of the G group maxima
            uint32_t gmax = key[0];
#pragma unroll
            for (int i = 1; i < EPL; ++i) gmax = max(gmax, key[i]);
            gmax = max(gmax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)gmax, 0xB1, 0xf, 0xf, false));  // quad [1,0,3,2]
            gmax = max(gmax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)gmax, 0x4E, 0xf, 0xf, false));  // quad [2,3,0,1]
            if (K <= 8)
                gmax = max(gmax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)gmax, 0x141, 0xf, 0xf, false));  // half-row
            const uint32_t theta = max(wave_min_u32(gmax), 1u);  // absent keys (0) are never candidates

            uint64_t cm[EPL];
            int n = 0;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                cm[i] = __ballot(key[i] >= theta);
                n += __popcll(cm[i]);
            }
            int my_idx = 0, rank = 64;
            float my_score = 0.0f, s_max;
            if (n <= 64) {
                int off = 0;
#pragma unroll
                for (int i = 0; i < EPL; ++i) {
                    if (key[i] >= theta) {
                        const int pos = off + (int)__builtin_amdgcn_mbcnt_hi(
                                                  (uint32_t)(cm[i] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)cm[i], 0u));
                        *(MOE_LDS uint64_t*)(cand + pos) =
                            ((uint64_t)key[i] << 32) | (uint32_t)~(uint32_t)(i * 64 + lane);
                    }
                    off += __popcll(cm[i]);
                }
                // zeros past the last candidate: they rank below every key, so
                // the count below runs over whole groups of 8 words
                if (lane < 8) *(MOE_LDS uint64_t*)(cand + n + lane) = 0ull;
                asm volatile("" ::: "memory");  // a wave's LDS accesses execute in order
                const uint64_t v = lane < n ? *(const MOE_LDS uint64_t*)(cand + lane) : 0ull;
                int r = 0;
                for (int j0 = 0; j0 < n; j0 += 8) {
                    u64x2 c[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) c[q] = *(const MOE_LDS u64x2*)(cand + j0 + 2 * q);
#pragma unroll
                    for (int q = 0; q < 4; ++q) r += (int)(c[q][0] > v) + (int)(c[q][1] > v);
                }
                if (lane < n) rank = r;
                const int top = __builtin_ctzll(__ballot(rank == 0));
                s_max = key_score((uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), top));
                my_score = key_score((uint32_t)(v >> 32));
                my_idx = (int)~(uint32_t)v;
            } else {
                select_rounds<EPL>(key, K, lane, my_idx, my_score, s_max);
                if (lane < K) rank = lane;
            }
            if (rank < K) {
                *(MOE_LDS int*)(bid + (ti << kp_log2) + rank) = my_idx;
                *(MOE_LDS float*)(bsc + (ti << kp_log2) + rank) = my_score - s_max;
            }
            asm volatile("" ::: "memory");  // this token's candidates are read before the next token's are written
        }
        // the batch's gates: lane KP*i + k holds choice k of token i
        const int ti = lane >> kp_log2, k = lane & ((1 << kp_log2) - 1);
        const bool valid = ti < nt && k < K;
        const float ex = valid ? expf(*(const MOE_LDS float*)(bsc + lane)) : 0.0f;
        asm volatile("" ::: "memory");
        if (valid) *(MOE_LDS float*)(bsc + lane) = ex;
        asm volatile("" ::: "memory");
        float z = 0.0f;
        const int base = lane & ~((1 << kp_log2) - 1);
        for (int j = 0; j < K; ++j) z += *(const MOE_LDS float*)(bsc + base + j);
        if (valid) {
            const int64_t o = (t0 + ti) * K + k;
            topk_idx[o] = *(const MOE_LDS int*)(bid + lane);
            gates[o] = ex / z;
        }
        asm volatile("" ::: "memory");  // the batch's slots are read before the next batch writes them
    }
}

// Router backward.  The gates are the softmax of the chosen scores, so with
// g, dg a token's gates and gate gradients the score gradient is
// g_k * (dg_k - sum_j g_j dg_j) at the chosen experts and 0 elsewhere; the
// sum runs over j ascending (fused multiply-adds from 0).
//
// The output is a dense [T, E] fp32 array that is almost all zeros, so the
// kernel is bound by its writes.  A wave takes a group of 8 tokens at a time
// (4 when K > 8): with KP the next power of two >= K, lane KP*t + k holds
// choice k of token t of the group.  The group's rows, contiguous in dlogits,
// are built in the wave's slice of LDS (zeroed, then one scatter of the
// chosen values; a wave's LDS accesses execute in order) and written with
// 16-byte stores, 1 KiB per instruction.  Waves loop over token groups and
// load the next group's inputs before they write the current one.
// Precondition: a token's K experts are distinct (moe_route's output is).
constexpr int kRbTok = 8;  // rows of a group (K <= 8; K > 8 uses 4)

template <int EMAX>
__global__ __launch_bounds__(256) void route_backward_kernel(const int32_t* __restrict__ topk_idx,
                                                             const float* __restrict__ gates,
                                                             const float* __restrict__ dgates, int T, int E, int K,
                                                             int kp_log2, float* __restrict__ dlogits) {
    __shared__ __attribute__((aligned(16))) float s_rows[4][kRbTok * EMAX];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar loop control
    float* rows = s_rows[wave];
    const int KP = 1 << kp_log2;
    const int tpw = min(kRbTok, 64 >> kp_log2);  // tokens per group
    const int tj = lane >> kp_log2, k = lane & (KP - 1);
    const int64_t n_groups = ((int64_t)T + tpw - 1) / tpw;
    const int64_t stride = (int64_t)gridDim.x * 4;
    auto load = [&](int64_t grp, int& idx, float& g, float& dg) {
        const int64_t t = grp * tpw + tj;
        idx = -1;
        g = dg = 0.0f;
        if (tj < tpw && k < K && t < T) {
            idx = topk_idx[t * K + k];
            g = gates[t * K + k];
            dg = dgates[t * K + k];
        }
    };
    int64_t grp = (int64_t)blockIdx.x * 4 + wave;
    int idx;
    float g, dg;
    load(grp, idx, g, dg);
    for (; grp < n_groups; grp += stride) {
        int n_idx;
        float n_g, n_dg;
        load(grp + stride, n_idx, n_g, n_dg);
        // the token's sum over its choices: lanes of the token read them in turn
        float sum = 0.0f;
        const int base = (tj << kp_log2) & 63;
        for (int j = 0; j < K; ++j) {
            const float gj = __shfl(g, base + j, 64);
            const float dgj = __shfl(dg, base + j, 64);
            sum = __builtin_fmaf(gj, dgj, sum);
        }
        const float val = g * (dg - sum);
        asm volatile("" ::: "memory");  // the previous group's rows are read before they are cleared
        const int64_t t0 = grp * tpw;
        const int nf = (int)min((int64_t)tpw, (int64_t)T - t0) * E;  // floats of the group's rows
        const int nq = (nf + 3) >> 2;
#pragma unroll 4
        for (int q = lane; q < nq; q += 64) *(MOE_LDS f32x4*)(rows + 4 * q) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        asm volatile("" ::: "memory");
        if (idx >= 0 && idx < E) *(MOE_LDS float*)(rows + tj * E + idx) = val;
        asm volatile("" ::: "memory");
        float* dst = dlogits + t0 * E;
        if ((nf & 3) == 0) {
#pragma unroll 4
            for (int q = lane; q < nq; q += 64) *(f32x4*)(dst + 4 * q) = *(const MOE_LDS f32x4*)(rows + 4 * q);
        } else {
            for (int f = lane; f < nf; f += 64) dst[f] = *(const MOE_LDS float*)(rows + f);
        }
        idx = n_idx;
        g = n_g;
        dg = n_dg;
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
    // waves loop over batches of tb tokens: at most 64 / KP (KP: the next power
    // of two >= K), so that a batch's choices fill one wave, and fewer (down to
    // 2) while that leaves under 4 waves per SIMD to run them
    int kp = 1;
    while (kp < K) kp <<= 1;
    int tb = 64 / kp;
    while (tb > 2 && ((int64_t)T + tb - 1) / tb < (int64_t)moe_host::num_cus() * 16) tb >>= 1;
    const int64_t batches = ((int64_t)T + tb - 1) / tb;
    const dim3 grid((unsigned)std::min<int64_t>((batches + 3) / 4, (int64_t)moe_host::num_cus() * 8)), block(256);
    int kp_log2 = 0;
    while ((1 << kp_log2) < K) ++kp_log2;
    const int epl = (E + 63) / 64;
    const bool full = E % 64 == 0;
#define MOE_ROUTE_CASE(N)                                                                                  \
    case N:                                                                                                \
        if (full) route_kernel<N, true><<<grid, block, 0, s>>>(logits, T, E, K, kp_log2, tb, topk_idx, gates); \
        else route_kernel<N, false><<<grid, block, 0, s>>>(logits, T, E, K, kp_log2, tb, topk_idx, gates);     \
        break;
    switch (epl) {
        MOE_ROUTE_CASE(1)
        MOE_ROUTE_CASE(2)
        MOE_ROUTE_CASE(3)
        MOE_ROUTE_CASE(4)
        MOE_ROUTE_CASE(5)
        MOE_ROUTE_CASE(6)
        MOE_ROUTE_CASE(7)
        default: MOE_ROUTE_CASE(8)
    }
#undef MOE_ROUTE_CASE
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
    hipStream_t s = (hipStream_t)stream;
    int kp_log2 = 0;
    while ((1 << kp_log2) < K) ++kp_log2;
    const int tpw = std::min(kRbTok, 64 >> kp_log2);
    const int64_t groups = ((int64_t)T + tpw - 1) / tpw;
    // LDS: 4 waves x 8 rows x EMAX floats per workgroup (32 or 64 KiB)
    const int per_cu = E <= 256 ? 4 : 2;
    const int64_t blocks = std::min<int64_t>((groups + 3) / 4, (int64_t)moe_host::num_cus() * per_cu);
    const dim3 grid((unsigned)blocks), block(256);
    if (E <= 256) route_backward_kernel<256><<<grid, block, 0, s>>>(topk_idx, gates, dgates, T, E, K, kp_log2, dlogits);
    else route_backward_kernel<512><<<grid, block, 0, s>>>(topk_idx, gates, dgates, T, E, K, kp_log2, dlogits);
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
