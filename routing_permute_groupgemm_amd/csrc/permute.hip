// Stable expert-grouped permutation (a counting sort of the T*K routing pairs).
//
// UniEP paper, "MoE workflow": tokens are grouped by destination expert in a
// deterministic order (a stable sort that keeps the source order);
// "Deterministic Token Mapping": a token's destination is the exclusive
// prefix of the per-expert counts plus its stable index inside the expert,
// computed without atomics deciding any order.  Here the flat pair index
// p = t*K + k is the sort's source order; since a token chooses an expert at
// most once, ordering by p inside an expert is ordering by token.
//
// Four launches, none of which reads device data back to the host:
// TB (tokens per block of count and rank) is 64 while blocks x local experts
// fits one 8192-entry pass of the one-block scan: there few blocks would
// leave the GPU idle and each wave's ranking rounds are a latency chain.
// Otherwise it is 256, which keeps the scan short.
//
//  1. count:   per block of TB tokens, an LDS histogram of local experts
//              (integer adds commute, so the result has no order dependence);
//              written expert-major to the workspace: ws[j*nblk + b].
//  2. scan:    one block per expert scans its row of ws in place
//              (exclusive), so ws[j*nblk+b] becomes the rows of expert j owned
//              by the blocks before b, and writes the expert's total to
//              counts[j]; the rank blocks add the experts' offsets (a prefix
//              over counts), and the first of them writes offsets and the
//              overflow status.
//  3. rank:    each block ranks its pairs inside each expert with wave
//              ballots (a match of equal expert ids, then a popcount of the
//              lower lanes) and per-wave running counters in LDS, processed
//              strictly in pair order; writes pos and src.
//  4. copy:    one wave per token reads the token's row once (16-byte
//              loads) and writes it to each of its local destination rows.
// With TB = 64 and at most 256 blocks, step 2 runs inside step 3 instead:
// every rank block reads the whole count matrix (at most 8192 entries) and
// derives its own first rows, which costs less than the one-block launch.
#include <mutex>

#include "moe_common.hpp"

namespace moe {

constexpr int kMaxLocal = 512;

// tokens per block of the count and rank kernels
inline int perm_tb(int64_t T, int e_local) { return (T + 63) / 64 * e_local <= 8192 ? 64 : 256; }

__global__ __launch_bounds__(256) void perm_count_kernel(const int32_t* __restrict__ idx, int T, int K,
                                                         int e_begin, int e_local, int nblk, int tb,
                                                         int32_t* __restrict__ ws) {
    __shared__ int hist[kMaxLocal];
    for (int j = threadIdx.x; j < e_local; j += 256) hist[j] = 0;
    __syncthreads();
    const int64_t p0 = (int64_t)blockIdx.x * tb * K;
    const int64_t p1 = min(p0 + (int64_t)tb * K, (int64_t)T * K);
    for (int64_t p = p0 + threadIdx.x; p < p1; p += 256) {
        int j = idx[p] - e_begin;
        if ((unsigned)j < (unsigned)e_local) atomicAdd(&hist[j], 1);
    }
    __syncthreads();
    for (int j = threadIdx.x; j < e_local; j += 256) ws[(int64_t)j * nblk + blockIdx.x] = hist[j];
}

// Inclusive scan of one value per thread over a 1024-thread block.
__device__ __forceinline__ int block_inclusive_scan_1024(int v, int* sh_wave /*[16]*/) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    if (lane == 63) sh_wave[wave] = v;
    __syncthreads();
    if (wave == 0) {
        int w = lane < 16 ? sh_wave[lane] : 0;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            int o = __shfl_up(w, off, 64);
            if (lane >= off) w += o;
        }
        if (lane < 16) sh_wave[lane] = w;
    }
    __syncthreads();
    int add = wave > 0 ? sh_wave[wave - 1] : 0;
    __syncthreads();
    return v + add;
}

// Step 2 when the rank kernel does not scan: block j scans row j of the
// count matrix (expert j's counts over the token blocks) in place, exclusive,
// and writes the row total to counts[j].  The experts' offsets (a prefix over
// these totals) are then formed by each rank block from counts.
__global__ __launch_bounds__(1024) void perm_rowscan_kernel(int32_t* __restrict__ ws, int nblk,
                                                            int32_t* __restrict__ counts) {
    __shared__ int sh_wave[16];
    __shared__ int sh_carry;
    int32_t* row = ws + (int64_t)blockIdx.x * nblk;
    if (threadIdx.x == 0) sh_carry = 0;
    __syncthreads();
    // chunks of 1024*ITEMS, each thread owns ITEMS consecutive entries
    constexpr int ITEMS = 4;
    for (int base = 0; base < nblk; base += 1024 * ITEMS) {
        int vals[ITEMS];
        int sum = 0;
        const int my0 = base + threadIdx.x * ITEMS;
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            vals[i] = my0 + i < nblk ? row[my0 + i] : 0;
            sum += vals[i];
        }
        const int incl = block_inclusive_scan_1024(sum, sh_wave);
        int run = sh_carry + incl - sum;
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            if (my0 + i < nblk) row[my0 + i] = run;
            run += vals[i];
        }
        __syncthreads();
        if (threadIdx.x == 1023) sh_carry = run;
        __syncthreads();
    }
    if (threadIdx.x == 0) counts[blockIdx.x] = sh_carry;
}

// No pairs to place (no tokens or no local experts): every count and offset is 0.
__global__ void perm_empty_kernel(int e_local, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                  int32_t* __restrict__ status) {
    for (int j = threadIdx.x; j <= e_local; j += blockDim.x) {
        offsets[j] = 0;
        if (j < e_local) counts[j] = 0;
    }
    if (threadIdx.x == 0) status[0] = 0;
}

// Lanes whose key equals this lane's key (keys < 2^nbits; inactive lanes excluded).
__device__ __forceinline__ uint64_t match_key(int key, bool active, int nbits) {
    uint64_t m = __ballot(active);
    for (int b = 0; b < nbits; ++b) {
        bool bit = (key >> b) & 1;
        uint64_t on = __ballot(active && bit);
        m &= bit ? on : ~on;
    }
    return m;
}

// Largest block count for which the rank kernel also does the scan: each of
// its blocks then reads the whole e_local x nblk count matrix (at most 8192
// entries), which stays cheap only while the blocks are few.
constexpr int kFusedScanBlocks = 256;

// KMAX: an upper bound of the rounds of 64 pairs per wave (tb/4 tokens * K pairs).
// Every block derives its own first row per expert: the expert's offset (an
// exclusive scan of the expert totals) plus the counts of the token blocks
// before it.  FUSED: ws holds the raw per-(expert, block) counts and the
// block adds them up itself, and block 0 also writes counts.  Otherwise the
// rows of ws are already scanned per expert and counts holds the totals
// (perm_rowscan_kernel's output).  Block 0 writes offsets and status.
template <int KMAX, bool FUSED>
__global__ __launch_bounds__(256) void perm_rank_kernel(const int32_t* __restrict__ idx, int T, int K,
                                                        int e_begin, int e_local, int nbits, int nblk, int tb,
                                                        const int32_t* __restrict__ ws, int64_t cap_rows,
                                                        int32_t* __restrict__ pos, int32_t* __restrict__ src,
                                                        int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ status) {
    __shared__ int cnt[4][kMaxLocal];
    __shared__ int s_base[kMaxLocal];  // this block's first row per expert
    __shared__ int s_tot[kMaxLocal];
    __shared__ int s_wsum[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int j = lane; j < e_local; j += 64) cnt[wave][j] = 0;
    {
        if constexpr (FUSED) {
            for (int j = threadIdx.x; j < e_local; j += 256) s_base[j] = s_tot[j] = 0;
            __syncthreads();
            // per expert: the total over all blocks and the part before this block
            // (integer adds, so the order of the LDS atomics does not matter)
            const int64_t n = (int64_t)e_local * nblk;
            for (int64_t q = threadIdx.x; q < n; q += 256) {
                const int c = ws[q];
                const int j = (int)(q / nblk), b = (int)(q - (int64_t)j * nblk);
                if (c) {
                    atomicAdd(&s_tot[j], c);
                    if (b < (int)blockIdx.x) atomicAdd(&s_base[j], c);
                }
            }
        } else {
            for (int j = threadIdx.x; j < e_local; j += 256) {
                s_tot[j] = counts[j];
                s_base[j] = ws[(int64_t)j * nblk + blockIdx.x];
            }
        }
        __syncthreads();
        // exclusive scan of the totals over experts: thread i owns experts 2i, 2i+1
        const int j0 = 2 * threadIdx.x;
        const int t0 = j0 < e_local ? s_tot[j0] : 0, t1 = j0 + 1 < e_local ? s_tot[j0 + 1] : 0;
        int v = t0 + t1;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(v, off, 64);
            if (lane >= off) v += o;
        }
        if (lane == 63) s_wsum[wave] = v;
        __syncthreads();
        int before = 0;
        for (int w = 0; w < wave; ++w) before += s_wsum[w];
        const int off0 = before + v - (t0 + t1);
        if (j0 < e_local) s_base[j0] += off0;
        if (j0 + 1 < e_local) s_base[j0 + 1] += off0 + t0;
        if (blockIdx.x == 0) {
            if (j0 < e_local) {
                if (FUSED) counts[j0] = t0;
                offsets[j0] = off0;
            }
            if (j0 + 1 < e_local) {
                if (FUSED) counts[j0 + 1] = t1;
                offsets[j0 + 1] = off0 + t0;
            }
            if (threadIdx.x == 0) {
                const int total = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
                offsets[e_local] = total;
                status[0] = (int64_t)total > cap_rows ? 1 : 0;
            }
        }
    }
    __syncthreads();
    const int64_t npairs = (int64_t)T * K;
    // wave `wave` owns the pairs of tb/4 consecutive tokens, [p0, pend), in
    // rounds of 64 consecutive pairs
    const int64_t per_wave = (int64_t)(tb / 4) * K;
    const int64_t p0 = (int64_t)blockIdx.x * tb * K + wave * per_wave;
    const int64_t pend = min(p0 + per_wave, npairs);
    const int rounds = (int)((per_wave + 63) / 64);
    const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int rk[KMAX], jj[KMAX];
#pragma unroll
    for (int it = 0; it < KMAX; ++it) {
        rk[it] = 0;
        jj[it] = -1;
        if (it < rounds) {
            const int64_t p = p0 + (int64_t)it * 64 + lane;
            int j = p < pend ? idx[p] - e_begin : -1;
            bool local = (unsigned)j < (unsigned)e_local;
            uint64_t m = match_key(local ? j : 0, local, nbits);
            if (local) {
                int before = __popcll(m & lower);
                int base = cnt[wave][j];
                if (before == 0) cnt[wave][j] = base + __popcll(m);
                rk[it] = base + before;
                jj[it] = j;
            }
        }
    }
    __syncthreads();
    // exclusive prefix of the four waves' counts, per expert
    for (int j = threadIdx.x; j < e_local; j += 256) {
        int s = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            int c = cnt[w][j];
            cnt[w][j] = s;
            s += c;
        }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < KMAX; ++it) {
        if (it < rounds) {
            const int64_t p = p0 + (int64_t)it * 64 + lane;
            if (p < pend) {
                int j = jj[it];
                int row = -1;
                if (j >= 0) {
                    const int first = s_base[j];
                    int64_t r = (int64_t)first + cnt[wave][j] + rk[it];
                    if (r < cap_rows) {
                        row = (int)r;
                        src[r] = (int32_t)p;
                    }
                }
                pos[p] = row;
            }
        }
    }
}

// x_perm[pos[t,k]] = x[t]; 16-byte vectors; one wave per token, 4 tokens per block.
template <int UNROLL>
__global__ __launch_bounds__(256) void perm_copy_kernel(const u32x4* __restrict__ x, int T, int K, int H,
                                                        const int32_t* __restrict__ pos,
                                                        u32x4* __restrict__ x_perm) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t >= T) return;
    const int my_pos = lane < K ? pos[t * K + lane] : -1;
    if (__ballot(my_pos >= 0) == 0ull) return;  // no local pair
    const int nv = H >> 3;                        // 16-byte vectors per row
    const u32x4* xr = x + t * nv;
    for (int v0 = 0; v0 < nv; v0 += 64 * UNROLL) {
        u32x4 buf[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            int v = v0 + u * 64 + lane;
            if (v < nv) buf[u] = __builtin_nontemporal_load(xr + v);
        }
        for (int k = 0; k < K; ++k) {
            const int r = __builtin_amdgcn_readlane(my_pos, k);  // uniform: lane k's destination row
            if (r < 0) continue;
            u32x4* dst = x_perm + (int64_t)r * nv;
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                int v = v0 + u * 64 + lane;
                // plain stores: non-temporal ones measured slower here once
                // the GEMM that reads x_perm runs after the copy
                if (v < nv) dst[v] = buf[u];
            }
        }
    }
}

}  // namespace moe

extern "C" size_t moe_permute_workspace_size(int T, int K, int e_local) {
    (void)K;
    if (T < 0 || e_local < 0) return 0;
    const int tb = moe::perm_tb(T, e_local);
    int64_t nblk = (T + tb - 1) / tb;
    int64_t n = nblk * (int64_t)e_local;
    return (size_t)((n * 4 + 255) / 256 * 256 + 256);
}

namespace moe {

// Host-side argument checks of the permutation (shared by both entry points).
static int permute_check(const int32_t* topk_idx, int T, int K, int e_begin, int e_local, const moe_bf16* x, int H,
                         int cap_rows, const int32_t* counts, const int32_t* offsets, const int32_t* pos,
                         const int32_t* src, const moe_bf16* x_perm, const int32_t* status) {
    using moe_host::misaligned;
    if (T < 0 || K < 1 || K > 16 || e_begin < 0 || e_local < 0 || e_local > kMaxLocal || H < 0 ||
        cap_rows < 0)
        return MOE_EINVAL;
    if ((int64_t)T * K >= (1ll << 31) || (int64_t)cap_rows > (int64_t)T * K) return MOE_EINVAL;
    if (H % 64 != 0) return MOE_ESHAPE;
    if (!offsets || !status) return MOE_EINVAL;
    if (e_local > 0 && !counts) return MOE_EINVAL;
    if (T > 0 && (!topk_idx || !pos)) return MOE_EINVAL;
    // x_perm NULL: the index-only permutation (no row copy, x not read)
    if (cap_rows > 0 && !src) return MOE_EINVAL;
    if (x_perm && T > 0 && cap_rows > 0 && H > 0 && !x) return MOE_EINVAL;
    if (misaligned(topk_idx) || misaligned(x) || misaligned(counts) || misaligned(offsets) ||
        misaligned(pos) || misaligned(src) || misaligned(x_perm) || misaligned(status))
        return MOE_EALIGN;
    return MOE_OK;
}

// The launches of the permutation, with the per-(expert, block) count matrix
// in w (every entry of it is written by the count kernel before it is read,
// so w needs no clearing).
static int permute_launch(const int32_t* topk_idx, int T, int K, int e_begin, int e_local, const moe_bf16* x, int H,
                          int cap_rows, int32_t* counts, int32_t* offsets, int32_t* pos, int32_t* src,
                          moe_bf16* x_perm, int32_t* status, int32_t* w, hipStream_t s) {
    const int tb = perm_tb(T, e_local);
    const int nblk = (T + tb - 1) / tb;
    const int rounds = (tb / 4 * K + 63) / 64;
    int nbits = 0;
    while ((1 << nbits) < e_local) ++nbits;
    // few blocks of the small token block: the rank kernel does the scan too
    const bool fused = tb == 64 && nblk > 0 && nblk <= kFusedScanBlocks;
    if (nblk > 0 && e_local > 0)
        perm_count_kernel<<<nblk, 256, 0, s>>>(topk_idx, T, K, e_begin, e_local, nblk, tb, w);
    if (nblk == 0 || e_local == 0) {
        perm_empty_kernel<<<1, 256, 0, s>>>(e_local, counts, offsets, status);
    } else if (!fused) {
        perm_rowscan_kernel<<<e_local, 1024, 0, s>>>(w, nblk, counts);
    }
    if (nblk > 0) {
#define MOE_RANK(KM, FU)                                                                                    \
    perm_rank_kernel<KM, FU><<<nblk, 256, 0, s>>>(topk_idx, T, K, e_begin, e_local, nbits, nblk, tb, w, cap_rows, \
                                                  pos, src, counts, offsets, status)
        if (fused) {
            if (rounds <= 4) MOE_RANK(4, true);
            else if (rounds <= 8) MOE_RANK(8, true);
            else MOE_RANK(16, true);
        } else {
            if (rounds <= 4) MOE_RANK(4, false);
            else if (rounds <= 8) MOE_RANK(8, false);
            else MOE_RANK(16, false);
        }
#undef MOE_RANK
        if (H > 0 && x_perm)
            perm_copy_kernel<4><<<(T + 3) / 4, 256, 0, s>>>((const u32x4*)x, T, K, H, pos, (u32x4*)x_perm);
    }
    return moe_host::launch_status();
}

// Scratch of the allocation-free entry point: the count matrix lives in this
// file-scope device array (one copy per GPU, held until the process ends)
// instead of a caller's workspace.  Host code never passes the array's name
// to a kernel (on the host it is a stand-in, not a device address): it uses
// the address hipGetSymbolAddress returns, fetched once per device.
constexpr size_t kPermuteScratchBytes = MOE_PERMUTE_SCRATCH_BYTES;
static __device__ __align__(256) int32_t scratch[kPermuteScratchBytes / 4];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch`, looked up on the first call on
// that device (with it current) and kept.
static int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_EHIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace moe

extern "C" int moe_permute(const int32_t* topk_idx, int T, int K, int e_begin, int e_local,
                           const moe_bf16* x, int H, int cap_rows, int32_t* counts, int32_t* offsets,
                           int32_t* pos, int32_t* src, moe_bf16* x_perm, int32_t* status, void* ws,
                           size_t ws_bytes, moe_stream stream) {
    using namespace moe;
    const int rc = permute_check(topk_idx, T, K, e_begin, e_local, x, H, cap_rows, counts, offsets, pos, src,
                                 x_perm, status);
    if (rc != MOE_OK) return rc;
    if (moe_host::misaligned(ws)) return MOE_EALIGN;
    const size_t need = moe_permute_workspace_size(T, K, e_local);
    if (!ws || ws_bytes < need) return MOE_EWORKSPACE;
    return permute_launch(topk_idx, T, K, e_begin, e_local, x, H, cap_rows, counts, offsets, pos, src, x_perm,
                          status, (int32_t*)ws, (hipStream_t)stream);
}

extern "C" int moe_permute_noalloc(const int32_t* topk_idx, int T, int K, int e_begin, int e_local,
                                   const moe_bf16* x, int H, int cap_rows, int32_t* counts, int32_t* offsets,
                                   int32_t* pos, int32_t* src, moe_bf16* x_perm, int32_t* status,
                                   moe_stream stream) {
    using namespace moe;
    const int rc = permute_check(topk_idx, T, K, e_begin, e_local, x, H, cap_rows, counts, offsets, pos, src,
                                 x_perm, status);
    if (rc != MOE_OK) return rc;
    if (moe_permute_workspace_size(T, K, e_local) > kPermuteScratchBytes) return MOE_EWORKSPACE;
    void* w = nullptr;
    const int st = scratch_address(&w);
    if (st != MOE_OK) return st;
    return permute_launch(topk_idx, T, K, e_begin, e_local, x, H, cap_rows, counts, offsets, pos, src, x_perm,
                          status, (int32_t*)w, (hipStream_t)stream);
}
