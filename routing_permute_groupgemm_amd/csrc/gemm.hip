// Padding-free grouped GEMMs on bf16 MFMA (gfx950), fp32 accumulation.
//
// UniEP paper: "MoE workflow" (a GroupGEMM projects the permuted tokens,
// SwiGLU follows, a second GroupGEMM projects back; the backward computes
// dgrad GEMMs and, for the weights, a transposed GroupGEMM reducing over the
// token dimension), "Scoreboard-based Synchronization" (a padding-free
// GroupGEMM with dynamic pointer arithmetic over irregular per-expert tiles),
// "Computation Worker" (a 128x256x64 tile; here 128x128x64 for 64-wide
// waves).  The blog restatement of the performance model notes that SwiGLU
// is purely memory-bound, so it is fused into the GEMM epilogue.
//
// One kernel template covers every GEMM of the layer:
//   ROWS schedule  C[r, :] = A[r, :] . B_j for the rows r of expert j
//     A (x_perm, h, dy_perm, dab) is contraction-contiguous ("KC");
//     B is the expert weight, either [Kd][N] (N contiguous, "MN") or [N][Kd]
//     (contraction contiguous, "KC").  Tiles: 128 rows x 128 B-columns; the
//     per-expert row counts stay on the device: every workgroup rebuilds the
//     tile prefix of the experts from `offsets` and finds a tile's expert by
//     binary search over it.
//   WGRAD schedule dW_j = A_j^T . B_j over the rows of expert j, A and B both
//     "MN" (their rows are the contraction).  The contraction over rows is one
//     fixed-order loop per output tile (no split, no atomics); experts are
//     visited longest first.
//
// Data path: global -> LDS by buffer_load ... lds (16 bytes per lane, no
// VGPR staging; loads past the resource bound return zero, which masks
// ragged row tails), two LDS stages; LDS rows are 128 bytes, 16-byte chunks
// XOR-swizzled by row; contraction-contiguous fragments are read with
// ds_read_b128, the others with the transposing ds_read_b64_tr_b16.  The
// MFMA is v_mfma_f32_32x32x16_bf16 with the weight fragment as its first
// operand, so each lane ends with 4 consecutive output columns of one row.
// Workgroups are persistent, and block ids are remapped so each XCD (own L2)
// walks a contiguous run of tiles; tiles are visited in groups of 4 row
// blocks so neighbouring tiles share A rows and B columns.
#include <algorithm>

#include "moe_common.hpp"

namespace moe {

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kGroupM = 4;
constexpr int kMaxGroups = 512;
constexpr int kStageBytes = 32768;  // A 16 KiB + B 16 KiB
constexpr int kLdsBytes = 2 * kStageBytes;

enum : int { LAY_KC = 0, LAY_MN = 1 };
enum : int { EPI_BF16 = 0, EPI_SWIGLU = 1, EPI_SWIGLU_BWD = 2, EPI_F32 = 3 };
enum : int { SCHED_ROWS = 0, SCHED_WGRAD = 1 };

struct GemmParams {
    const uint16_t* a;   // A rows (ROWS) / first operand rows (WGRAD)
    int64_t lda;
    const uint16_t* w0;  // ROWS: expert weight (or gate weight)
    const uint16_t* w1;  // ROWS: up weight (SWIGLU) or second segment (two_seg)
    int64_t w_stride;    // elements per expert matrix
    int ldw;             // row stride of a weight matrix
    int two_seg;         // A has 2*Kd columns; the second half multiplies w1
    const uint16_t* b;   // WGRAD: second operand rows
    int64_t ldb;
    const int32_t* offsets;
    int e_local;
    int64_t cap;
    int N;   // output columns (SWIGLU: F)
    int Kd;  // contraction length per segment (ROWS)
    int M;   // WGRAD output rows
    uint16_t* c;
    int64_t ldc;
    uint16_t* c2;         // SWIGLU: ab_save [rows, 2F]
    const uint16_t* ab;   // SWIGLU_BWD: saved [a | b], row stride 2N
    float* cf;            // WGRAD: fp32 out [e_local, M, N]
};

// 16-byte chunk swizzles of 128-byte LDS rows.
// KC tiles are read 32 rows x 16 B at a time: chunk ^= (row/2)%8 spreads 16
// consecutive rows over all banks.  MN tiles are read as 4-row x 32-byte
// patches (transposing reads): chunk ^= 4*((row/2)%2) puts rows r and r+2 on
// different banks.
__device__ __forceinline__ int swz_kc(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz_mn(int row) { return ((row >> 1) & 1) << 2; }

__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (MOE_LDS void*)lds, 16, voff, 0, 0, 0);
}

// KC fragment: 32 rows starting at rb, k16-step kk; lane holds row rb+l%32, 8 k values.
__device__ __forceinline__ bf16x8 frag_kc(const uint8_t* tile, int rb, int kk, int lane) {
    int row = rb + (lane & 31);
    int ch = (kk * 2 + (lane >> 5)) ^ swz_kc(row);
    u32x4 v = *(const MOE_LDS u32x4*)(tile + row * 128 + (ch << 4));
    return __builtin_bit_cast(bf16x8, v);
}

// MN fragment: 32 columns starting at cb (0..127) of a [64][128] tile stored as
// two [64][64] sub-tiles; lane holds column cb+l%32 and 8 consecutive k.
__device__ __forceinline__ bf16x8 frag_mn(const uint8_t* tile, int cb, int kk, int lane) {
    const int g = lane >> 4, q = lane & 15;
    const int krow = kk * 16 + 8 * (g >> 1) + (q >> 2);
    const int col = (cb & 63) + 16 * (g & 1) + 4 * (q & 3);
    const uint8_t* sub = tile + (cb >> 6) * 8192;
    const int off = ((col >> 3) ^ swz_mn(krow)) * 16 + (col & 7) * 2;
    s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS s16x4*)(sub + krow * 128 + off));
    s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS s16x4*)(sub + (krow + 4) * 128 + off));
    u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    u32x4 v = {l2[0], l2[1], h2[0], h2[1]};
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + __expf(-a)); }

__device__ __forceinline__ int xcd_remap(int b, int G) { return (b & 7) * (G >> 3) + (b >> 3); }

template <int LB, int EPI, int SCHED>
__global__ __launch_bounds__(256) void gg_kernel(GemmParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kLdsBytes];
    __shared__ int s_off[kMaxGroups + 1];    // clamped row offsets
    __shared__ int s_start[kMaxGroups + 1];  // ROWS: first m-tile of each expert; WGRAD: sorted order
    __shared__ int s_wave[4];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int EL = p.e_local;

    // ---- per-workgroup schedule setup (device-resident row counts) ----
    for (int j = tid; j <= EL; j += 256) {
        int64_t o = p.offsets[j];
        s_off[j] = (int)(o < p.cap ? o : p.cap);
    }
    __syncthreads();
    int n_tiles_total;
    int tiles_n;  // tiles along N (ROWS) ; tiles per group (WGRAD)
    int tiles_mw = 0;
    if (SCHED == SCHED_ROWS) {
        tiles_n = EPI == EPI_SWIGLU ? (p.N + 63) / 64 : (p.N + kBN - 1) / kBN;
        // exclusive scan of per-expert m-tile counts, 2 experts per thread
        int j0 = 2 * tid, c0 = 0, c1 = 0;
        if (j0 < EL) c0 = (s_off[j0 + 1] - s_off[j0] + kBM - 1) / kBM;
        if (j0 + 1 < EL) c1 = (s_off[j0 + 2] - s_off[j0 + 1] + kBM - 1) / kBM;
        int v = c0 + c1;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            int t = __shfl_up(v, o, 64);
            if (lane >= o) v += t;
        }
        if (lane == 63) s_wave[wave] = v;
        __syncthreads();
        int add = 0;
        for (int w = 0; w < wave; ++w) add += s_wave[w];
        int excl = add + v - (c0 + c1);
        if (j0 < EL) s_start[j0] = excl;
        if (j0 + 1 < EL) s_start[j0 + 1] = excl + c0;
        if (tid == 255) s_start[EL] = add + v;
        __syncthreads();
        n_tiles_total = s_start[EL] * tiles_n;
    } else {
        tiles_mw = (p.M + kBM - 1) / kBM;
        tiles_n = tiles_mw * ((p.N + kBN - 1) / kBN);
        // order experts by row count, longest first (ties: lower id first)
        for (int j = tid; j < EL; j += 256) {
            int cj = s_off[j + 1] - s_off[j], rank = 0;
            for (int i = 0; i < EL; ++i) {
                int ci = s_off[i + 1] - s_off[i];
                rank += (ci > cj) || (ci == cj && i < j);
            }
            s_start[rank] = j;
        }
        __syncthreads();
        n_tiles_total = EL * tiles_n;
    }

    const int G = gridDim.x;
    for (int tile = xcd_remap(blockIdx.x, G); tile < n_tiles_total; tile += G) {
        // ---- decode the tile ----
        int j, row0 = 0, valid = 0, ni = 0, mi_w = 0, KT;
        if (SCHED == SCHED_ROWS) {
            const int MT = s_start[EL];
            const int grp = tile / (kGroupM * tiles_n);
            const int first = grp * kGroupM;
            const int gsz = min(kGroupM, MT - first);
            const int r = tile - grp * kGroupM * tiles_n;
            const int mi = first + r % gsz;
            ni = r / gsz;
            int lo = 0, hi = EL - 1;  // largest j with s_start[j] <= mi
            while (lo < hi) {
                int mid = (lo + hi + 1) >> 1;
                if (s_start[mid] <= mi) lo = mid;
                else hi = mid - 1;
            }
            j = lo;
            row0 = s_off[j] + (mi - s_start[j]) * kBM;
            valid = min(kBM, s_off[j + 1] - row0);
            KT = (p.two_seg ? 2 * p.Kd : p.Kd) / kBK;
        } else {
            j = s_start[tile / tiles_n];
            const int r = tile % tiles_n;
            mi_w = r % tiles_mw;
            ni = r / tiles_mw;
            row0 = s_off[j];
            valid = s_off[j + 1] - row0;
            KT = (valid + kBK - 1) / kBK;
        }

        // ---- loaders ----
        // A, ROWS (KC): rows row0.. of a, resource bounded by the valid rows.
        __amdgpu_buffer_rsrc_t rsA = make_rsrc(p.a + (int64_t)row0 * p.lda,
                                               SCHED == SCHED_ROWS ? (uint32_t)(valid * p.lda * 2) : 0u);
        auto issue = [&](int kt, int stage) {
            uint8_t* sA = smem + stage * kStageBytes;
            uint8_t* sB = sA + 16384;
            const int k0 = kt * kBK;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int q = wave * 4 + u;  // 1 KiB chunk index 0..15
                const int lrow = q * 8 + (lane >> 3), phys = lane & 7;
                // ---------------- A ----------------
                if (SCHED == SCHED_ROWS) {
                    const int lch = phys ^ swz_kc(lrow);
                    uint32_t voff = (uint32_t)((lrow * p.lda + k0 + lch * 8) * 2);
                    lds_load16(rsA, sA + q * 1024, voff);
                } else {
                    const int krow = lrow & 63, s = lrow >> 6;
                    const int lch = phys ^ swz_mn(krow);
                    const int rows_left = valid - k0;
                    __amdgpu_buffer_rsrc_t r = make_rsrc(p.a + (int64_t)(row0 + k0) * p.lda,
                                                         (uint32_t)(min(kBK, rows_left) * p.lda * 2));
                    const int col = mi_w * kBM + s * 64 + lch * 8;
                    uint32_t voff = col < p.M ? (uint32_t)((krow * p.lda + col) * 2) : kOOB;
                    lds_load16(r, sA + q * 1024, voff);
                }
                // ---------------- B ----------------
                if (SCHED == SCHED_WGRAD) {
                    const int krow = lrow & 63, s = lrow >> 6;
                    const int lch = phys ^ swz_mn(krow);
                    const int rows_left = valid - k0;
                    __amdgpu_buffer_rsrc_t r = make_rsrc(p.b + (int64_t)(row0 + k0) * p.ldb,
                                                         (uint32_t)(min(kBK, rows_left) * p.ldb * 2));
                    const int col = ni * kBN + s * 64 + lch * 8;
                    uint32_t voff = col < p.N ? (uint32_t)((krow * p.ldb + col) * 2) : kOOB;
                    lds_load16(r, sB + q * 1024, voff);
                } else if (LB == LAY_MN) {
                    // weight [Kd][ldw], N contiguous: two [64 k][64 col] sub-tiles
                    const int krow = lrow & 63, s = lrow >> 6;
                    const int lch = phys ^ swz_mn(krow);
                    const uint16_t* w;
                    int col;
                    if (EPI == EPI_SWIGLU) {
                        w = s ? p.w1 : p.w0;
                        col = ni * 64 + lch * 8;
                    } else {
                        w = p.w0;
                        col = ni * kBN + s * 64 + lch * 8;
                    }
                    __amdgpu_buffer_rsrc_t r = make_rsrc(w + (int64_t)j * p.w_stride + (int64_t)k0 * p.ldw,
                                                         (uint32_t)(kBK * p.ldw * 2));
                    uint32_t voff = col < p.N ? (uint32_t)((krow * p.ldw + col) * 2) : kOOB;
                    lds_load16(r, sB + q * 1024, voff);
                } else {
                    // weight [N][Kd], contraction contiguous; second segment from w1
                    const int lch = phys ^ swz_kc(lrow);
                    const bool seg1 = p.two_seg && k0 >= p.Kd;
                    const uint16_t* w = seg1 ? p.w1 : p.w0;
                    const int kk0 = seg1 ? k0 - p.Kd : k0;
                    const int n0 = ni * kBN;
                    __amdgpu_buffer_rsrc_t r = make_rsrc(w + (int64_t)j * p.w_stride + (int64_t)n0 * p.ldw,
                                                         (uint32_t)(min(kBN, p.N - n0) * p.ldw * 2));
                    uint32_t voff = (uint32_t)((lrow * p.ldw + kk0 + lch * 8) * 2);
                    lds_load16(r, sB + q * 1024, voff);
                }
            }
        };

        f32x16 acc[2][2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

        if (KT > 0) issue(0, 0);
        for (int kt = 0; kt < KT; ++kt) {
            const int stage = kt & 1;
            if (kt + 1 < KT) {
                issue(kt + 1, stage ^ 1);
                __builtin_amdgcn_s_waitcnt(0x0F70 | 8);  // vmcnt(8): this stage's 8 loads are done
            } else {
                __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0)
            }
            __syncthreads();
            const uint8_t* sA = smem + stage * kStageBytes;
            const uint8_t* sB = sA + 16384;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                bf16x8 af[2], bfv[2];
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    const int rb = wm * 64 + mt * 32;
                    af[mt] = SCHED == SCHED_ROWS ? frag_kc(sA, rb, kk, lane) : frag_mn(sA, rb, kk, lane);
                }
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const int cb = EPI == EPI_SWIGLU ? nt * 64 + wn * 32 : wn * 64 + nt * 32;
                    bfv[nt] = (SCHED == SCHED_ROWS && LB == LAY_KC) ? frag_kc(sB, cb, kk, lane)
                                                                    : frag_mn(sB, cb, kk, lane);
                }
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
                        acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfv[nt], af[mt], acc[mt][nt], 0, 0, 0);
            }
            __syncthreads();
        }

        // ---- epilogue: lane holds row (l%32) and columns 8*j4 + 4*(l/32) + 0..3 ----
        const int cq = 4 * (lane >> 5);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int mloc = wm * 64 + mt * 32 + (lane & 31);
            if (SCHED == SCHED_WGRAD) {
                const int m = mi_w * kBM + mloc;
                if (m >= p.M) continue;
                float* orow = p.cf + ((int64_t)j * p.M + m) * p.N;
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                    for (int j4 = 0; j4 < 4; ++j4) {
                        const int n = ni * kBN + wn * 64 + nt * 32 + 8 * j4 + cq;
                        if (n < p.N) {
                            f32x4 v = {acc[mt][nt][4 * j4], acc[mt][nt][4 * j4 + 1], acc[mt][nt][4 * j4 + 2],
                                       acc[mt][nt][4 * j4 + 3]};
                            __builtin_nontemporal_store(v, (f32x4*)(orow + n));
                        }
                    }
                continue;
            }
            if (mloc >= valid) continue;
            const int64_t row = row0 + mloc;
            if (EPI == EPI_SWIGLU) {
#pragma unroll
                for (int j4 = 0; j4 < 4; ++j4) {
                    const int hc = ni * 64 + wn * 32 + 8 * j4 + cq;
                    if (hc >= p.N) continue;
                    float hv[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float a = acc[mt][0][4 * j4 + i], b = acc[mt][1][4 * j4 + i];
                        hv[i] = silu_f(a) * b;
                    }
                    u32x2 hw = {pack_bf2(hv[0], hv[1]), pack_bf2(hv[2], hv[3])};
                    *(u32x2*)(p.c + row * p.ldc + hc) = hw;
                    if (p.c2) {
                        u32x2 aw = {pack_bf2(acc[mt][0][4 * j4], acc[mt][0][4 * j4 + 1]),
                                    pack_bf2(acc[mt][0][4 * j4 + 2], acc[mt][0][4 * j4 + 3])};
                        u32x2 bw = {pack_bf2(acc[mt][1][4 * j4], acc[mt][1][4 * j4 + 1]),
                                    pack_bf2(acc[mt][1][4 * j4 + 2], acc[mt][1][4 * j4 + 3])};
                        *(u32x2*)(p.c2 + row * 2 * p.N + hc) = aw;
                        *(u32x2*)(p.c2 + row * 2 * p.N + p.N + hc) = bw;
                    }
                }
            } else {
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                    for (int j4 = 0; j4 < 4; ++j4) {
                        const int n = ni * kBN + wn * 64 + nt * 32 + 8 * j4 + cq;
                        if (n >= p.N) continue;
                        float v[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) v[i] = acc[mt][nt][4 * j4 + i];
                        if (EPI == EPI_BF16) {
                            u32x2 w = {pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
                            *(u32x2*)(p.c + row * p.ldc + n) = w;
                        } else {  // EPI_SWIGLU_BWD: v is dh
                            u32x2 aw = *(const u32x2*)(p.ab + row * 2 * p.N + n);
                            u32x2 bw = *(const u32x2*)(p.ab + row * 2 * p.N + p.N + n);
                            float da[4], db[4];
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                float a = (i & 1) ? bf_hi(aw[i >> 1]) : bf_lo(aw[i >> 1]);
                                float b = (i & 1) ? bf_hi(bw[i >> 1]) : bf_lo(bw[i >> 1]);
                                float s = 1.0f / (1.0f + __expf(-a));
                                da[i] = v[i] * b * s * (1.0f + a * (1.0f - s));
                                db[i] = v[i] * a * s;
                            }
                            u32x2 dw = {pack_bf2(da[0], da[1]), pack_bf2(da[2], da[3])};
                            u32x2 ew = {pack_bf2(db[0], db[1]), pack_bf2(db[2], db[3])};
                            *(u32x2*)(p.c + row * p.ldc + n) = dw;
                            *(u32x2*)(p.c + row * p.ldc + p.N + n) = ew;
                        }
                    }
            }
        }
    }
}

template <int LB, int EPI, int SCHED>
static int launch(const GemmParams& p, int grid, hipStream_t s) {
    gg_kernel<LB, EPI, SCHED><<<grid, 256, 0, s>>>(p);
    return moe_host::launch_status();
}

static int rows_grid(int64_t cap, int e_local, int tiles_n) {
    int64_t upper = ((cap + kBM - 1) / kBM + e_local) * (int64_t)tiles_n;
    int64_t g = std::min<int64_t>(upper, (int64_t)moe_host::num_cus() * 2);
    return (int)((g + 7) / 8 * 8);
}

}  // namespace moe

using moe_host::misaligned;

extern "C" int moe_grouped_gemm_swiglu(const moe_bf16* x_perm, const moe_bf16* w_gate, const moe_bf16* w_up,
                                       const int32_t* offsets, int e_local, int H, int F, int cap_rows,
                                       moe_bf16* h, moe_bf16* ab_save, moe_stream stream) {
    using namespace moe;
    if (e_local < 0 || e_local > kMaxGroups || H < 0 || F < 0 || cap_rows < 0) return MOE_EINVAL;
    if (H % 64 || F % 64) return MOE_ESHAPE;
    if (!offsets) return MOE_EINVAL;
    if (e_local == 0 || cap_rows == 0 || F == 0) return MOE_OK;
    if (!x_perm || !w_gate || !w_up || !h) return MOE_EINVAL;
    if (misaligned(x_perm) || misaligned(w_gate) || misaligned(w_up) || misaligned(offsets) || misaligned(h) ||
        misaligned(ab_save))
        return MOE_EALIGN;
    if ((int64_t)kBM * H * 2 >= (1ll << 31) || (int64_t)kBK * F * 2 >= (1ll << 31)) return MOE_EINVAL;
    GemmParams p{};
    p.a = x_perm;
    p.lda = H;
    p.w0 = w_gate;
    p.w1 = w_up;
    p.w_stride = (int64_t)H * F;
    p.ldw = F;
    p.offsets = offsets;
    p.e_local = e_local;
    p.cap = cap_rows;
    p.N = F;
    p.Kd = H;
    p.c = h;
    p.ldc = F;
    p.c2 = ab_save;
    if (H == 0) return MOE_EINVAL;
    int grid = rows_grid(cap_rows, e_local, F / 64);
    return launch<LAY_MN, EPI_SWIGLU, SCHED_ROWS>(p, grid, (hipStream_t)stream);
}

extern "C" int moe_grouped_gemm(const moe_bf16* a, int lda, const moe_bf16* w0, const moe_bf16* w1, int trans_w,
                                const int32_t* offsets, int e_local, int Kd, int N, int cap_rows, int epilogue,
                                const moe_bf16* ab, moe_bf16* c, int ldc, moe_stream stream) {
    using namespace moe;
    if (e_local < 0 || e_local > kMaxGroups || Kd <= 0 || N < 0 || cap_rows < 0) return MOE_EINVAL;
    if (trans_w != 0 && trans_w != 1) return MOE_EINVAL;
    if (epilogue != MOE_EPI_NONE && epilogue != MOE_EPI_SWIGLU_BWD) return MOE_EINVAL;
    if (Kd % 64 || N % 64) return MOE_ESHAPE;
    if (w1 && !trans_w) return MOE_EINVAL;
    const int acols = w1 ? 2 * Kd : Kd;
    const int ccols = epilogue == MOE_EPI_SWIGLU_BWD ? 2 * N : N;
    if (lda < acols || ldc < ccols || lda % 8 || ldc % 8) return MOE_EINVAL;
    if (!offsets) return MOE_EINVAL;
    if (e_local == 0 || cap_rows == 0 || N == 0) return MOE_OK;
    if (!a || !w0 || !c || (epilogue == MOE_EPI_SWIGLU_BWD && !ab)) return MOE_EINVAL;
    if (misaligned(a) || misaligned(w0) || misaligned(w1) || misaligned(offsets) || misaligned(ab) ||
        misaligned(c))
        return MOE_EALIGN;
    if ((int64_t)kBM * lda * 2 >= (1ll << 31) || (int64_t)kBN * Kd * 2 >= (1ll << 31) ||
        (int64_t)kBK * N * 2 >= (1ll << 31))
        return MOE_EINVAL;
    GemmParams p{};
    p.a = a;
    p.lda = lda;
    p.w0 = w0;
    p.w1 = w1;
    p.w_stride = (int64_t)Kd * N;
    p.ldw = trans_w ? Kd : N;
    p.two_seg = w1 != nullptr;
    p.offsets = offsets;
    p.e_local = e_local;
    p.cap = cap_rows;
    p.N = N;
    p.Kd = Kd;
    p.c = c;
    p.ldc = ldc;
    p.ab = ab;
    int grid = rows_grid(cap_rows, e_local, (N + kBN - 1) / kBN);
    hipStream_t s = (hipStream_t)stream;
    if (trans_w) {
        if (epilogue == MOE_EPI_SWIGLU_BWD) return launch<LAY_KC, EPI_SWIGLU_BWD, SCHED_ROWS>(p, grid, s);
        return launch<LAY_KC, EPI_BF16, SCHED_ROWS>(p, grid, s);
    }
    if (epilogue == MOE_EPI_SWIGLU_BWD) return launch<LAY_MN, EPI_SWIGLU_BWD, SCHED_ROWS>(p, grid, s);
    return launch<LAY_MN, EPI_BF16, SCHED_ROWS>(p, grid, s);
}

extern "C" int moe_wgrad(const moe_bf16* a, int lda, const moe_bf16* b, int ldb, const int32_t* offsets,
                         int e_local, int M, int N, int cap_rows, float* dw, moe_stream stream) {
    using namespace moe;
    if (e_local < 0 || e_local > kMaxGroups || M < 0 || N < 0 || cap_rows < 0) return MOE_EINVAL;
    if (M % 64 || N % 64) return MOE_ESHAPE;
    if (lda < M || ldb < N || lda % 8 || ldb % 8) return MOE_EINVAL;
    if (!offsets) return MOE_EINVAL;
    if (e_local == 0 || M == 0 || N == 0) return MOE_OK;
    if (!dw || (cap_rows > 0 && (!a || !b))) return MOE_EINVAL;
    if (misaligned(a) || misaligned(b) || misaligned(offsets) || misaligned(dw)) return MOE_EALIGN;
    if ((int64_t)kBK * lda * 2 >= (1ll << 31) || (int64_t)kBK * ldb * 2 >= (1ll << 31)) return MOE_EINVAL;
    GemmParams p{};
    p.a = a;
    p.lda = lda;
    p.b = b;
    p.ldb = ldb;
    p.offsets = offsets;
    p.e_local = e_local;
    p.cap = cap_rows;
    p.M = M;
    p.N = N;
    p.cf = dw;
    int64_t total = (int64_t)e_local * ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
    int64_t g = std::min<int64_t>(total, (int64_t)moe_host::num_cus() * 2);
    int grid = (int)((g + 7) / 8 * 8);
    return launch<LAY_MN, EPI_F32, SCHED_WGRAD>(p, grid, (hipStream_t)stream);
}
