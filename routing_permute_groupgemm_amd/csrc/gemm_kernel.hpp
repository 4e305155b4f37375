// Padding-free grouped GEMMs on bf16 MFMA (gfx950), fp32 accumulation.
//
// UniEP paper: "MoE workflow" (a GroupGEMM projects the permuted tokens,
// SwiGLU follows, a second GroupGEMM projects back; the backward computes
// dgrad GEMMs and, for the weights, a transposed GroupGEMM reducing over the
// token dimension), "Scoreboard-based Synchronization" (a padding-free
// GroupGEMM with dynamic pointer arithmetic over irregular per-expert tiles),
// "Computation Worker" (a 128x256x64 tile on Hopper; here 256x256 or 192x256
// blocks of 64-wide waves, BK = 32).  The blog restatement of the
// performance model notes that SwiGLU is purely memory-bound, so it is fused
// into the GEMM epilogue.
//
// One kernel template covers every GEMM of the layer:
//   ROWS schedule  C[r, :] = A[r, :] . B_j for the rows r of expert j
//     A (x_perm, h, dy_perm, dab) is contraction-contiguous ("KC");
//     B is the expert weight, either [Kd][N] (N contiguous, "MN") or [N][Kd]
//     (contraction contiguous, "KC").  The per-expert row counts stay on the
//     device: every workgroup rebuilds the tile prefix of the experts from
//     `offsets` and finds a tile's expert by binary search over it.  The
//     kernel carries a 256-row and a 192-row body and every workgroup picks
//     the same one from the row counts (prefer_alt).
//   WGRAD schedule dW_j = A_j^T . B_j over the rows of expert j, A and B both
//     "MN" (their rows are the contraction).  The contraction over rows is one
//     fixed-order loop per output tile (no split, no atomics); experts are
//     visited longest first.
//
// Zero-copy variant (GATHER, gate/up only): the A rows are read from the
// tokens x[src[r] / K] instead of the permuted copy (MoonEP page, "How
// Redundant Expert Planning Achieves Perfect Balance": zero-copy dispatch);
// each lane's row offsets are set once per tile from indices fetched a tile
// ahead.
//
// Data path: global -> LDS by buffer_load ... lds (16 bytes per lane, no
// VGPR staging; loads past the resource bound return zero, which masks
// ragged row tails) into a four-stage ring that runs on across a workgroup's
// tiles; LDS rows are XOR-swizzled by 16-byte chunk; contraction-contiguous
// fragments are read with ds_read_b128, the others with the transposing
// ds_read_b64_tr_b16.  Inside a stage every MFMA is followed by an LDS read
// of the next k-step's fragments, and the stage's loads are spread among the
// MFMAs.  The MFMA is v_mfma_f32_32x32x16_bf16 with the weight fragment as
// its first operand, so each lane ends with 4 consecutive output columns of
// one row.  Workgroups are persistent, and block ids are remapped so each XCD
// (own L2) walks a contiguous run of tiles.
#pragma once

#include <stdlib.h>

#include <algorithm>
#include <type_traits>

#include "moe_common.hpp"

namespace moe {

constexpr int kGroupM = 4;  // row-tiled GEMMs: m-tiles per group of the tile order
constexpr int kGroupN = 4;  // weight gradient: n-tiles per group of the tile order
constexpr int kMaxGroups = 512;
constexpr int kLdsBudget = 128 * 1024;  // LDS per workgroup for the stage ring
#ifndef MOE_GEMM_MFMA16
#define MOE_GEMM_MFMA16 1  // the down dgrad's 256 x 256 body computes with 16x16x32 MFMAs (0: 32x32x16)
#endif
#ifndef MOE_GEMM_DGRAD_STAGED
#define MOE_GEMM_DGRAD_STAGED 1  // 0: the down dgrad's epilogue loads and stores straight from the MFMA layout
#endif
#ifndef MOE_GEMM_DGRAD_PREFETCH
#define MOE_GEMM_DGRAD_PREFETCH 2  // 16-row blocks of saved (a, b) rows in flight in the staged epilogue
#endif
#ifndef MOE_GEMM_MFMA16_WGRAD
#define MOE_GEMM_MFMA16_WGRAD 0  // 1: the weight gradient's too (measured 5% slower, so off)
#endif

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
    float* cf;            // WGRAD: fp32 out [e_local, M, n_split]: the columns n < n_split
    float* cf2;           // WGRAD: the columns n >= n_split, out [e_local, M, N - n_split] (NULL: n_split = N)
    int n_split;
    const int32_t* src;   // ROWS gather: row r of the tile reads a[src[r] / topk]
    int topk;
    uint32_t topk_rcp;    // floor((2^32 - 1) / topk): src / topk without a divide
    int64_t a_rows;       // ROWS gather: rows of a (bounds every A load)
    // Dense operands, no offsets array: offsets[j] = min(j * row_chunk, dense_rows)
    // (ROWS: one group of all rows; WGRAD: the rows in chunks, one partial each)
    int dense_rows;
    int row_chunk;
    // ROWS: the contraction in ksplit chunks of kchunk elements (a multiple of
    // BK); with EPI_F32, chunk ks writes its partial result at cf + ks*part_stride
    int ksplit;
    int kchunk;
    int64_t part_stride;
    const float* bias;    // ROWS EPI_F32: added to every row, [N]
    int stagger_ticks;    // start delay step of the workgroups (100 MHz ticks; 0: none)
    int stagger_phases;
};

typedef __attribute__((ext_vector_type(4))) int i32x4;

// Buffer descriptor (gfx9 layout: base, stride 0, byte range, format dword);
// loads at or past `bytes` return zero.
// Callers pass wave-uniform values; readfirstlane states that to the compiler
// (a no-op on values it already holds in scalar registers) so the descriptor
// can always live in SGPRs as the buffer instructions require.
__device__ __forceinline__ i32x4 make_srd(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffff));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}

// 16 bytes per lane from global memory straight into LDS at lds + 16*lane.
// Written as inline asm so the compiler does not treat every later LDS read
// as dependent on it (it would wait for all outstanding loads, serialising
// the LDS stages); the kernel waits for it explicitly (vmcnt + barrier).
__device__ __forceinline__ void lds_load16(i32x4 srd, uint32_t lds, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(srd)
                 : "memory");
}

// The same with the non-temporal hint: for data read exactly once (weights of
// experts that fit one row tile), so that it does not displace reused lines.
__device__ __forceinline__ void lds_load16_nt(i32x4 srd, uint32_t lds, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :
                 : "s"(lds), "v"(voff), "s"(srd)
                 : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const MOE_LDS void*)p;
}

// 4 bytes per lane into LDS at lds + 4*lane (same contract as lds_load16).
__device__ __forceinline__ void lds_load4(i32x4 srd, uint32_t lds, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(srd)
                 : "memory");
}

// s_waitcnt vmcnt(n) for a compile-time n (lgkmcnt and expcnt left alone).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// The same wait, also a compiler barrier for memory: LDS written by
// LDS-direct loads is read after it.
template <int N>
__device__ __forceinline__ void wait_vmcnt_mem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// ---- LDS tile layouts -------------------------------------------------------
// KC ("contraction-contiguous"): the tile is [rows][BK] bf16, BK*2 bytes per row,
// 16-byte chunks XOR-swizzled by row so that the 32 rows x 16 B a fragment read
// touches spread over all banks.  MN: the tile is [BK][cols] stored as
// [BK][64] sub-tiles with 128-byte rows, read by the transposing
// ds_read_b64_tr_b16; a 4-row x 32-byte read patch is spread by a 4-chunk XOR.
template <int BK>
struct Lay {
    static constexpr int kRowBytes = BK * 2;          // KC row
    static constexpr int kChunks = BK / 8;            // 16-byte chunks per KC row
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;
    static constexpr int kSubBytes = BK * 128;        // MN sub-tile [BK][64]
    static constexpr int kLoadsPerSub = BK / 8;
    __device__ static __forceinline__ int swz_kc(int row) {
        return BK == 64 ? ((row >> 1) & 7) : ((row >> 2) & 3);
    }
    __device__ static __forceinline__ int swz_mn(int krow) { return ((krow >> 1) & 1) << 2; }

    // lane holds row rb + l%32 and k values 16*kk + 8*(l/32) + 0..7
    __device__ static __forceinline__ bf16x8 frag_kc(const uint8_t* tile, int rb, int kk, int lane) {
        const int row = rb + (lane & 31);
        const int ch = (kk * 2 + (lane >> 5)) ^ swz_kc(row);
        u32x4 v = *(const MOE_LDS u32x4*)(tile + row * kRowBytes + (ch << 4));
        return __builtin_bit_cast(bf16x8, v);
    }
    // lane holds column cb + l%32 and k values 16*kk + 8*(l/32) + 0..7
    __device__ static __forceinline__ bf16x8 frag_mn(const uint8_t* tile, int cb, int kk, int lane) {
        const int g = lane >> 4, q = lane & 15;
        const int krow = kk * 16 + 8 * (g >> 1) + (q >> 2);
        const int col = (cb & 63) + 16 * (g & 1) + 4 * (q & 3);
        const uint8_t* sub = tile + (cb >> 6) * kSubBytes;
        const int off = ((col >> 3) ^ swz_mn(krow)) * 16 + (col & 7) * 2;
        s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS s16x4*)(sub + krow * 128 + off));
        s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS s16x4*)(sub + (krow + 4) * 128 + off));
        u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        u32x4 v = {l2[0], l2[1], h2[0], h2[1]};
        return __builtin_bit_cast(bf16x8, v);
    }
    // Fragments of v_mfma_f32_16x16x32_bf16 (one 32-deep step per stage, BK = 32):
    // lane holds row rb + l%16 and k values 8*(l/16) + 0..7
    __device__ static __forceinline__ bf16x8 frag_kc16(const uint8_t* tile, int rb, int lane) {
        static_assert(BK == 32, "one 32-deep MFMA step per stage");
        const int row = rb + (lane & 15);
        const int ch = (lane >> 4) ^ swz_kc(row);
        u32x4 v = *(const MOE_LDS u32x4*)(tile + row * kRowBytes + (ch << 4));
        return __builtin_bit_cast(bf16x8, v);
    }
    // lane holds column cb + l%16 (cb a multiple of 16) and k values 8*(l/16) + 0..7:
    // each group of 16 lanes reads a 4 k-row x 16 column patch twice (k-rows
    // 8g..8g+3, then 8g+4..8g+7) and the transposing read gives lane q column q
    __device__ static __forceinline__ bf16x8 frag_mn16(const uint8_t* tile, int cb, int lane) {
        static_assert(BK == 32, "one 32-deep MFMA step per stage");
        const int g = lane >> 4, q = lane & 15;
        const int krow = 8 * g + (q >> 2);
        const int col = (cb & 63) + 4 * (q & 3);
        const uint8_t* sub = tile + (cb >> 6) * kSubBytes;
        const int off = ((col >> 3) ^ swz_mn(krow)) * 16 + (col & 7) * 2;
        s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS s16x4*)(sub + krow * 128 + off));
        s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS s16x4*)(sub + (krow + 4) * 128 + off));
        u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        u32x4 v = {l2[0], l2[1], h2[0], h2[1]};
        return __builtin_bit_cast(bf16x8, v);
    }
    // per-lane byte offset of an LDS-direct load into a KC tile: load q fills
    // rows q*kRowsPerLoad + l/kChunks; `v` is q's part of the swizzle period
    __device__ static __forceinline__ uint32_t lane_kc(int lane, int v, int64_t ld) {
        const int r = lane / kChunks, c = lane % kChunks;
        return (uint32_t)((r * ld + (c ^ swz_kc(v * kRowsPerLoad + r)) * 8) * 2);
    }
    __device__ static __forceinline__ int kc_period(int q) { return BK == 64 ? (q & 1) : 0; }
    // ... into an MN sub-tile (load q fills k-rows 8*(q%kLoadsPerSub) + l/8)
    __device__ static __forceinline__ uint32_t lane_mn(int lane, int64_t ld) {
        return (uint32_t)(((lane >> 3) * ld + ((lane & 7) ^ swz_mn(lane >> 3)) * 8) * 2);
    }
};

__device__ __forceinline__ float sigmoid_f(float a) { return __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }
__device__ __forceinline__ float silu_f(float a) { return a * sigmoid_f(a); }

__device__ __forceinline__ int xcd_remap(int b, int G) { return (b & 7) * (G >> 3) + (b >> 3); }

// The lane id (0..63) read from the hardware where it is needed: the asm can be
// neither hoisted nor merged, so no lane-derived value stays live across the
// persistent tile loop (the large bodies would spill it, and every reload
// waits for all the loads and stores in flight).
__device__ __forceinline__ int lane_id_here() {
    int v;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
    return v;
}

// Block tile BM x BN (B columns; for SWIGLU the gate half then the up half),
// contraction step BK, a ring of STAGES LDS stages, WM x WN waves each owning a
// (BM/WM) x (BN/WN) tile of 32x32 MFMA tiles.
template <int BM, int BN, int BK, int WM, int WN, int LDS_BUDGET = kLdsBudget>
struct Tile {
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kMTW = BM / WM / 32;
    static constexpr int kNTW = BN / WN / 32;
    static constexpr int kABytes = BM * BK * 2;
    static constexpr int kStage = (BM + BN) * BK * 2;
    static constexpr int kStages = LDS_BUDGET / kStage < 4 ? LDS_BUDGET / kStage : 4;
    static constexpr int kLoads = kStage / 1024;  // 1 KiB LDS-direct loads per stage
    static constexpr int kALoads = kABytes / 1024;
    static constexpr int kLoadsPerWave = kLoads / kWaves;
    static constexpr int kKK = BK / 16;           // MFMA k-steps per stage
    static_assert(kStages >= 3, "the pipeline needs at least three stages");
    static_assert(kLoads % kWaves == 0 && kALoads % kWaves == 0, "loads must split evenly over the waves");
    static_assert(kLoadsPerWave * (kStages - 1) < 64, "vmcnt range");
};

// The GEMM of one workgroup for one tile shape.  smem is the stage ring;
// s_off holds the clamped row offsets (already loaded); s_start and s_wave are
// scratch for the schedule; s_idx (GATHER only) holds the prefetched source
// indices of the A rows.  FULLC: every tile's columns (and, for the weight
// gradient, rows) lie inside the output, so the loads skip those bounds
// checks.  NTB: every expert fits one row tile, so each weight
// byte is read once and the weight loads carry the non-temporal hint.
template <int BM, int BN, int BK, int WM, int WN, int LB, int EPI, int SCHED, int LDSB, bool GATHER, bool NTB,
          bool FULLC = false>
__device__ __forceinline__ void gg_body(const GemmParams& p, uint8_t* smem, const int* s_off, int* s_start,
                                        int* s_wave, int* s_idx) {
    using TL = Tile<BM, BN, BK, WM, WN, LDSB>;
    using LY = Lay<BK>;
    constexpr int MTW = TL::kMTW, NTW = TL::kNTW, LPW = TL::kLoadsPerWave, S = TL::kStages, KK = TL::kKK;
    constexpr int LA = TL::kALoads / TL::kWaves;  // A loads per wave and stage
    static_assert(!GATHER || (SCHED == SCHED_ROWS && EPI == EPI_SWIGLU) || (SCHED == SCHED_WGRAD && EPI == EPI_F32),
                  "gathered A rows: the gate/up GEMM and the weight gradient");
    // gathered rows of the weight gradient's contraction (GATHER with SCHED_WGRAD)
    constexpr bool kGW = GATHER && SCHED == SCHED_WGRAD;
    // The 256 x 256 body of the down dgrad (SwiGLU-backward epilogue) computes
    // with v_mfma_f32_16x16x32_bf16: its 128 x 128 wave tile is 8 x 8 blocks of
    // 16 x 16, one 32-deep MFMA step per stage.  Each lane then holds 4
    // consecutive output columns of 16 rows, so the epilogue's loads of the
    // saved (a, b) pairs and its stores of (da, db) cover 32 bytes of a row per
    // group of 4 lanes instead of 16, and this GEMM ran 5-8% faster (A/B on one
    // box: 3.55 against 3.75 ms for T = 131072, H = 7168; 0.64 against 0.69 ms
    // for T = 16384, H = 2048).  The other GEMMs ran as fast or faster with
    // 32x32x16, although back-to-back 16x16x32 MFMAs on random operands reach
    // 14% more flops on this chip: their time is set by the loads, not the
    // MFMA rate.  The smaller bodies keep 32x32x16, whose 32-row blocks their
    // idle-row scheme is built on.  The weight gradient can use the same body
    // (MOE_GEMM_MFMA16_WGRAD=1: MN-layout A fragments, and each lane stores its
    // 16 bytes of fp32 dW straight from the accumulators); it ran 5% slower
    // than its 32x32x16 body, whose staged epilogue stores whole lines.
    constexpr bool kMf16 = ((MOE_GEMM_MFMA16 && EPI == EPI_SWIGLU_BWD && SCHED == SCHED_ROWS) ||
                            (MOE_GEMM_MFMA16_WGRAD && EPI == EPI_F32 && SCHED == SCHED_WGRAD)) &&
                           BM == 256 && BN == 256 && WM == 2 && WN == 2 && BK == 32;
    constexpr int MB16 = kMf16 ? BM / WM / 16 : 1;  // 16-row blocks per wave
    // Past the last tile the cursor's loads read zeros: through descriptors of
    // range 0 (no per-load select), or, in the 16x16x32 body, whose registers
    // are the scarcest (the descriptors kept in scalar registers made it spill
    // in its stage loop), through the out-of-range offset chosen per load.
    constexpr bool kSrdLive = !kMf16;
    constexpr int NB16 = kMf16 ? BN / WN / 16 : 1;  // 16-column blocks per wave

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int wm = wave / WN, wn = wave % WN;
    const int EL = p.e_local;

    // ---- per-workgroup schedule setup (device-resident row counts) ----
    int n_tiles_total;
    int tiles_n;  // tiles along N (ROWS) ; tiles per group (WGRAD)
    int tiles_mw = 0;
    if (SCHED == SCHED_ROWS) {
        tiles_n = EPI == EPI_SWIGLU ? (p.N + BN / 2 - 1) / (BN / 2) : (p.N + BN - 1) / BN;
        // exclusive scan of per-expert m-tile counts; each thread owns a run of experts
        constexpr int PER = (kMaxGroups + TL::kThreads - 1) / TL::kThreads;
        const int j0 = tid * PER;
        int cnt[PER], sum = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            int j = j0 + i;
            cnt[i] = j < EL ? (s_off[j + 1] - s_off[j] + BM - 1) / BM : 0;
            sum += cnt[i];
        }
        int v = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            int t = __shfl_up(v, o, 64);
            if (lane >= o) v += t;
        }
        if (lane == 63) s_wave[wave] = v;
        __syncthreads();
        int add = 0;
        for (int w = 0; w < wave; ++w) add += s_wave[w];
        int run = add + v - sum;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (j0 + i < EL) s_start[j0 + i] = run;
            run += cnt[i];
        }
        if (tid == TL::kThreads - 1) s_start[EL] = run;
        __syncthreads();
        n_tiles_total = s_start[EL] * tiles_n * max(p.ksplit, 1);
    } else {
        tiles_mw = (p.M + BM - 1) / BM;
        tiles_n = tiles_mw * ((p.N + BN - 1) / BN);
        // order experts by row count, longest first (ties: lower id first)
        for (int j = tid; j < EL; j += TL::kThreads) {
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

    // per-lane parts of the LDS-direct load offsets
    uint32_t lt_a0, lt_a1 = 0, lt_b0, lt_b1 = 0;
    if (SCHED == SCHED_ROWS) {
        // gathered rows: the row term comes from the row's own offset
        lt_a0 = LY::lane_kc(lane, 0, GATHER ? 0 : p.lda);
        lt_a1 = LY::lane_kc(lane, 1, GATHER ? 0 : p.lda);
        if (LB == LAY_KC) {
            lt_b0 = LY::lane_kc(lane, 0, p.ldw);
            lt_b1 = LY::lane_kc(lane, 1, p.ldw);
        } else {
            lt_b0 = LY::lane_mn(lane, p.ldw);
        }
    } else {
        // gathered rows (kGW): the row term comes from the row's token
        lt_a0 = LY::lane_mn(lane, kGW ? 0 : p.lda);
        lt_b0 = LY::lane_mn(lane, p.ldb);
    }

    // B column (within the BN-wide tile) of this wave's nt-th 32-column MFMA tile
    // first row (within the tile) of the wave's mt-th 32-row MFMA tile.  In
    // bodies that leave MFMA rows idle past a tile's valid rows the row
    // blocks are dealt to the wave rows in turn (block mt*WM + wm), so both
    // wave rows keep an equal share; elsewhere each wave row owns a run.
    auto row_base = [&](int mt) {
        return (SCHED == SCHED_ROWS && BM < 256) ? (mt * WM + wm) * 32 : wm * (BM / WM) + mt * 32;
    };
    auto col_of = [&](int nt) {
        if (EPI == EPI_SWIGLU) {
            constexpr int HW = BN / 2 / WN;  // h columns per wave
            const int half = nt / (NTW / 2), i = nt % (NTW / 2);
            return half * (BN / 2) + wn * HW + 32 * i;
        }
        return wn * (BN / WN) + 32 * nt;
    };

    // ---- tile decode (identical in every lane) ----
    struct TileDesc {
        int j, row0, valid, ni, mi_w, KT, ks;
    };
    auto decode = [&](int tile) {
        int j, row0 = 0, valid = 0, ni = 0, mi_w = 0, KT, ks = 0;
        if (SCHED == SCHED_ROWS) {
            const int MT = s_start[EL];
            // contraction chunks outermost: the tiles in flight share the
            // chunk's columns of A and rows of B
            if (p.ksplit > 1) {
                ks = tile / (MT * tiles_n);
                tile -= ks * MT * tiles_n;
            }
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
            row0 = s_off[j] + (mi - s_start[j]) * BM;
            valid = min(BM, s_off[j + 1] - row0);
            const int kd = p.two_seg ? 2 * p.Kd : p.Kd;
            KT = (p.ksplit > 1 ? min(p.kchunk, kd - ks * p.kchunk) : kd) / BK;
        } else {
            j = s_start[tile / tiles_n];
            // within a group: runs of kGroupN output-column tiles, rows fastest,
            // so the tiles in flight on one XCD share few A and B column blocks
            const int r = tile % tiles_n;
            const int tnn = tiles_n / tiles_mw;
            const int g = r / (kGroupN * tiles_mw);
            const int gw = min(kGroupN, tnn - g * kGroupN);
            const int idx = r - g * kGroupN * tiles_mw;
            ni = g * kGroupN + idx % gw;
            mi_w = idx / gw;
            row0 = s_off[j];
            valid = s_off[j + 1] - row0;
            KT = (valid + BK - 1) / BK;
        }
        // tell the compiler the decode is uniform, so that the buffer
        // descriptors built from it live in scalar registers
        TileDesc d;
        d.j = __builtin_amdgcn_readfirstlane(j);
        d.row0 = __builtin_amdgcn_readfirstlane(row0);
        d.valid = __builtin_amdgcn_readfirstlane(valid);
        d.ni = __builtin_amdgcn_readfirstlane(ni);
        d.mi_w = __builtin_amdgcn_readfirstlane(mi_w);
        d.KT = __builtin_amdgcn_readfirstlane(KT);
        d.ks = __builtin_amdgcn_readfirstlane(ks);
        return d;
    };

    // ---- issue cursor: the tile and stage whose loads are issued next ----
    // It walks this workgroup's tiles (tile0, tile0 + G, ...) S-1 stages ahead
    // of the MFMAs, skipping tiles without stages, so the LDS ring runs on
    // across tile boundaries: a tile's first stages load during the previous
    // tile's last stages and its epilogue.
    const int G = gridDim.x;
    const int tile0 = xcd_remap(blockIdx.x, G);
    int itile = tile0, ik = 0;
    TileDesc ic = {0, 0, 0, 0, 0, 0, 0};
    // buffer descriptors of the issue cursor's tile (row-tiled GEMMs), built
    // once per tile: the A rows, and the B weight of each half / segment
    i32x4 c_srdA = {0, 0, 0, 0}, c_srdB0 = {0, 0, 0, 0}, c_srdB1 = {0, 0, 0, 0};
    // weight gradient: the group's first A and B rows
    // (c_stA, c_stB: the cursor stage's first A and B rows, c_rem the group's
    // rows from there on; stepped by one stage per advance rather than rebuilt
    // from the stage index, which took 64-bit products per stage)
    uint64_t c_stA = 0, c_stB = 0;
    int c_rem = 0;

    // Gathered A rows (GATHER): one descriptor over all of a; per lane, the
    // byte offset of the row behind each of its LA loads (kOOB past the
    // expert's rows).  The source indices of a tile's rows are fetched one
    // tile ahead, by LDS-direct loads into this wave's slice of one of two
    // buffers (alternating per tile), so the switch to the next tile never
    // waits for loads in flight: when the cursor reaches a tile, the KT >= 2
    // stages issued since its prefetch (the contraction is at least 64 long)
    // put it behind the (S-2)*LPW newest loads, which a free vmcnt wait then
    // covers.
    uint32_t c_rowoff[LA];
#pragma unroll
    for (int u = 0; u < LA; ++u) c_rowoff[u] = kOOB_GATHER;
    int idx_buf = 0;
    bool pf_issued = false;  // the last advance() issued a prefetch (LA more loads)
    i32x4 srd_src = {0, 0, 0, 0};
    if (GATHER) {
        c_srdA = make_srd(p.a, (uint32_t)(p.a_rows * p.lda * 2));
        srd_src = make_srd(p.src, (uint32_t)(p.cap * 4));
    }
    // Gathered rows of the weight gradient (kGW): a stage's A rows are rows
    // k0 .. k0+31 of the expert, wave w loading rows k0 + 8w + (l / 8), so
    // each wave needs 8 tokens per stage.  They are fetched by one LDS-direct
    // dword load per stage (lanes 0..7; the other lanes read nothing) into
    // the wave's slice of one of two buffers in s_idx, two stages ahead of
    // the cursor, so the end-of-stage wait that publishes the ring's stages
    // covers them too (that fetch is the newest load of its stage, one more
    // than the ring's count).  tk counts the cursor's stages: its tokens are
    // in buffer tk & 1.
    int tk = 0;
    int itile_n = 0;  // the cursor tile's successor with stages (kGW)
    TileDesc ic_n = {0, 0, 0, 0, 0, 0, 0};
    // lane's row in A load u of this wave: rows q*16 + l/4 of the tile, the
    // uniform part q*16 and the lane part l/4
    // (per-tile code reads the lane id afresh, so that nothing derived from
    // it is hoisted out of the loop and kept live)
    auto a_row0 = [&](int u) { return (u * TL::kWaves + wave) * LY::kRowsPerLoad; };
    auto prefetch_rows = [&](int tile, int buf) {
        const TileDesc d = decode(tile);
        const uint32_t base = lds_addr(s_idx) + (uint32_t)(((buf * TL::kWaves + wave) * LA) * 256);
        const int a_rowl = lane_id_here() / LY::kChunks;
#pragma unroll
        for (int u = 0; u < LA; ++u) {
            const uint32_t voff = (uint32_t)(d.row0 + a_row0(u)) * 4u + (uint32_t)a_rowl * 4u;
            lds_load4(srd_src, base + u * 256, a_rowl < d.valid - a_row0(u) ? voff : kOOB);
        }
    };

    auto seek = [&]() {
        for (; itile < n_tiles_total; itile += G) {
            ic = decode(itile);
            if (ic.KT > 0) break;
        }
        if (SCHED == SCHED_ROWS && itile < n_tiles_total) {
            if (GATHER) {
                wait_vmcnt_mem<(S - 2) * LPW>();
                const int ln = lane_id_here();
                const int a_rowl = ln / LY::kChunks;
                const int* si = s_idx + ((idx_buf * TL::kWaves + wave) * LA) * 64 + ln;
#pragma unroll
                for (int u = 0; u < LA; ++u) {
                    // src = t*K + k; the quotient estimate is t or t - 1
                    const uint32_t v = (uint32_t)si[u * 64];
                    uint32_t tok = __umulhi(v, p.topk_rcp);
                    if (v - tok * (uint32_t)p.topk >= (uint32_t)p.topk) ++tok;
                    // the lane's 16-byte column chunk (its swizzle by load index) is folded in here
                    const uint32_t lt = LY::kc_period(u * TL::kWaves + wave) ? lt_a1 : lt_a0;
                    c_rowoff[u] = a_rowl < ic.valid - a_row0(u) && tok < (uint32_t)p.a_rows
                                      ? tok * (uint32_t)(p.lda * 2) + lt
                                      : kOOB_GATHER;
                }
                idx_buf ^= 1;
                if (itile + G < n_tiles_total) {
                    prefetch_rows(itile + G, idx_buf);
                    pf_issued = true;
                }
            }
            // first contraction index of the tile's chunk (0 without a split):
            // the descriptors start there, and their ranges still end where the
            // rows end, since kofs + chunk <= Kd <= the row stride
            const int64_t kofs = (int64_t)ic.ks * p.kchunk;
            if (!GATHER)
                c_srdA = make_srd(p.a + (int64_t)ic.row0 * p.lda + kofs, (uint32_t)((ic.valid * p.lda - kofs) * 2));
            if (LB == LAY_MN) {
                const uint32_t range = (uint32_t)((p.Kd - kofs) * p.ldw * 2);
                c_srdB0 = make_srd(p.w0 + (int64_t)ic.j * p.w_stride + kofs * p.ldw, range);
                if (EPI == EPI_SWIGLU) c_srdB1 = make_srd(p.w1 + (int64_t)ic.j * p.w_stride + kofs * p.ldw, range);
            } else {
                const int n0 = ic.ni * BN;
                const uint32_t range = (uint32_t)((min(BN, p.N - n0) * p.ldw - kofs) * 2);
                c_srdB0 = make_srd(p.w0 + (int64_t)ic.j * p.w_stride + (int64_t)n0 * p.ldw + kofs, range);
                if (p.two_seg) c_srdB1 = make_srd(p.w1 + (int64_t)ic.j * p.w_stride + (int64_t)n0 * p.ldw, range);
            }
            // opaque from here on: kept in SGPRs rather than rebuilt from the
            // tile indices in every stage
            asm volatile("" : "+s"(c_srdA), "+s"(c_srdB0), "+s"(c_srdB1));
        } else if (SCHED == SCHED_ROWS && kSrdLive) {
            // no tile left: descriptors of range 0, so every load the cursor
            // still issues (to keep the count per stage fixed) reads zeros
            c_srdA = make_srd(p.a, 0);
            c_srdB0 = c_srdB1 = make_srd(p.a, 0);
            asm volatile("" : "+s"(c_srdA), "+s"(c_srdB0), "+s"(c_srdB1));
        }
        if (SCHED == SCHED_WGRAD && itile < n_tiles_total) {
            c_stA = (uint64_t)(p.a + (int64_t)ic.row0 * p.lda);
            c_stB = (uint64_t)(p.b + (int64_t)ic.row0 * p.ldb);
            c_rem = ic.valid;
            asm volatile("" : "+s"(c_stA), "+s"(c_stB), "+s"(c_rem));
        }
        if (kGW) {
            for (itile_n = itile + G; itile_n < n_tiles_total; itile_n += G) {
                ic_n = decode(itile_n);
                if (ic_n.KT > 0) break;
            }
        }
    };
    // kGW: fetch the 8 tokens of this wave's rows of the cursor's stage
    // (ahead = 0) or of the stage after it (ahead = 1: the next stage of its
    // tile, or the first of the next tile) into buffer (tk + ahead) & 1; a
    // load of nothing when there is no such stage.
    auto fetch_tokens = [&](int ahead) {
        if constexpr (kGW) {
            int row0 = 0, rows = 0, k0 = 0;
            if (itile < n_tiles_total) {
                if (ik + ahead < ic.KT) {
                    row0 = ic.row0, rows = ic.valid, k0 = (ik + ahead) * BK;
                } else if (itile_n < n_tiles_total) {
                    row0 = ic_n.row0, rows = ic_n.valid, k0 = 0;
                }
            }
            const int ln = lane_id_here();
            const int r = k0 + 8 * wave + ln;  // lanes 0..7: the wave's 8 rows
            const uint32_t base = lds_addr(s_idx) + (uint32_t)((((tk + ahead) & 1) * TL::kWaves + wave) * 256);
            lds_load4(srd_src, base, ln < 8 && r < rows ? (uint32_t)(row0 + r) * 4u : kOOB);
        }
    };
    auto advance = [&]() {
        if (itile < n_tiles_total && ++ik >= ic.KT) {
            ik = 0;
            itile += G;
            seek();
        } else if constexpr (SCHED == SCHED_WGRAD) {
            // the next stage of the same group (or no tile left: unused)
            c_stA += (uint64_t)(BK * 2) * (uint64_t)p.lda;
            c_stB += (uint64_t)(BK * 2) * (uint64_t)p.ldb;
            c_rem -= BK;
        }
        if constexpr (kGW) {
            ++tk;
            fetch_tokens(1);
        }
    };
    if (GATHER && !kGW && tile0 < n_tiles_total) {
        // the first tile's indices (row-tiled schedules skip no tile)
        prefetch_rows(tile0, 0);
        wait_vmcnt_mem<0>();
    }
    seek();

    // Load u (0..LPW-1) of this wave for stage kt of the issue cursor's tile
    // into LDS slot `slot`.  With no tile left the cursor's descriptors have
    // range 0 (seek, stage_srd), so its loads read zeros with no memory
    // traffic, and every stage keeps the same number of loads, so the vmcnt
    // bookkeeping stays fixed.
    // Weight gradient: the buffer descriptors of one stage (its BK rows of A
    // and of B, cut at the group's last row, so rows past it load zeros),
    // built once per stage rather than once per load.
    struct StageSrd {
        i32x4 a, b;
        uint32_t arow;  // kGW: byte offset of the lane's A row in a, or kOOB_GATHER
    };
    auto stage_srd = [&](int kt) {
        StageSrd r{};
        if constexpr (kGW) {
            // the lane's row of the stage and its token (fetched two stages ago);
            // no tile left: descriptors of range 0 (loads of zeros)
            (void)kt;  // the cursor's stage: c_stB, c_rem
            const bool live = itile < n_tiles_total;
            const uint32_t rows = live ? (uint32_t)max(0, min(BK, c_rem)) : 0u;
            r.a = live ? c_srdA : make_srd(p.a, 0);
            r.b = make_srd((const void*)c_stB, rows * (uint32_t)(p.ldb * 2));
            const int ln = lane_id_here();
            const uint32_t v = (uint32_t)*(const MOE_LDS int*)(s_idx + ((tk & 1) * TL::kWaves + wave) * 64 + (ln >> 3));
            // src = t*K + k; the quotient estimate is t or t - 1
            uint32_t tok = __umulhi(v, p.topk_rcp);
            if (v - tok * (uint32_t)p.topk >= (uint32_t)p.topk) ++tok;
            r.arow = 8 * wave + (ln >> 3) < c_rem && tok < (uint32_t)p.a_rows ? tok * (uint32_t)(p.lda * 2)
                                                                               : kOOB_GATHER;
        } else if constexpr (SCHED == SCHED_WGRAD) {
            // the cursor's stage (c_stA, c_stB, c_rem); no tile left: range 0 (loads of zeros)
            (void)kt;
            const uint32_t rows = itile < n_tiles_total ? (uint32_t)max(0, min(BK, c_rem)) : 0u;
            r.a = make_srd((const void*)c_stA, rows * (uint32_t)(p.lda * 2));
            r.b = make_srd((const void*)c_stB, rows * (uint32_t)(p.ldb * 2));
        }
        return r;
    };
    auto load_one = [&](int kt, int slot, int u, bool live, const StageSrd& ss) {
        const uint32_t sA = lds_addr(smem) + slot * TL::kStage;
        const uint32_t sB = sA + TL::kABytes;
        const int k0 = kt * BK;
        // re-materialise the lane terms each load (cheap adds) rather than
        // keeping one hoisted offset per load alive across the loop: the terms
        // pass through an opaque copy, one v_mov per load.  The row-tiled GEMMs
        // copy just the term each load needs; copying all four per load cost
        // the forward GEMMs 24 VALU instructions per stage, and with one wave
        // per SIMD the stage's instruction stream is what its time follows
        // (gate/up 4% slower).  The weight gradient copies two.
        uint32_t la0 = lt_a0, la1 = lt_a1, lb0 = lt_b0, lb1 = lt_b1;
        auto lane_term = [](uint32_t v) {
            asm volatile("" : "+v"(v));
            return v;
        };
        constexpr bool kEachLoad = SCHED == SCHED_ROWS;
        if constexpr (SCHED == SCHED_WGRAD) asm volatile("" : "+v"(la0), "+v"(lb0));
        else if constexpr (!kEachLoad) asm volatile("" : "+v"(la0), "+v"(la1), "+v"(lb0), "+v"(lb1));
        {
            // load u of wave w fills A block u*W + w (u < LA) or B block
            // (u - LA)*W + w: A/B and the sub-tile follow from u at compile
            // time, so the stream of loads has no branches
            constexpr int LA = TL::kALoads / TL::kWaves;
            constexpr bool kSubPerLoad = LY::kLoadsPerSub == TL::kWaves;
            // MN blocks: sub-tile (64 columns) and 8-k-row group of block v*W + w
            auto mn_sub = [&](int v) { return kSubPerLoad ? v : (v * TL::kWaves + wave) / LY::kLoadsPerSub; };
            auto mn_kr = [&](int v) { return kSubPerLoad ? wave : (v * TL::kWaves + wave) % LY::kLoadsPerSub; };
            if (u < LA) {
                const int q = u * TL::kWaves + wave;
                if (SCHED == SCHED_ROWS) {
                    uint32_t voff;
                    if (GATHER) {
                        voff = c_rowoff[u] + (uint32_t)(k0 * 2);
                    } else {
                        uint32_t lt = LY::kc_period(q) ? la1 : la0;
                        if (kEachLoad) lt = lane_term(lt);
                        voff = lt + (uint32_t)((q * LY::kRowsPerLoad * p.lda + k0) * 2);
                    }
                    lds_load16(c_srdA, sA + q * 1024, kSrdLive || live ? voff : (GATHER ? kOOB_GATHER : kOOB));
                } else if (kGW) {
                    // the row term is the lane's token row (mn_kr(u) is the wave, so the
                    // stage's row of this lane is the one stage_srd looked up)
                    const int col = ic.mi_w * BM + mn_sub(u) * 64;
                    const uint32_t voff = FULLC || col < p.M ? ss.arow + la0 + (uint32_t)(col * 2) : kOOB_GATHER;
                    lds_load16(ss.a, sA + q * 1024, voff);
                } else {
                    const int col = ic.mi_w * BM + mn_sub(u) * 64;
                    const uint32_t voff =
                        FULLC || col < p.M ? la0 + (uint32_t)((mn_kr(u) * 8 * p.lda + col) * 2) : kOOB;
                    lds_load16(ss.a, sA + q * 1024, voff);
                }
            } else {
                const int q = (u - LA) * TL::kWaves + wave;
                if (SCHED == SCHED_WGRAD) {
                    const int col = ic.ni * BN + mn_sub(u - LA) * 64;
                    const uint32_t voff =
                        FULLC || col < p.N ? lb0 + (uint32_t)((mn_kr(u - LA) * 8 * p.ldb + col) * 2) : kOOB;
                    lds_load16(ss.b, sB + q * 1024, voff);
                } else if (LB == LAY_MN) {
                    // weight [Kd][ldw], N contiguous: [BK][64] sub-tiles
                    const int sub = mn_sub(u - LA);
                    i32x4 r;
                    int col;
                    if (EPI == EPI_SWIGLU) {
                        constexpr int HS = BN / 128;  // sub-tiles per half
                        r = sub < HS ? c_srdB0 : c_srdB1;
                        col = ic.ni * (BN / 2) + (sub % HS) * 64;
                    } else {
                        r = c_srdB0;
                        col = ic.ni * BN + sub * 64;
                    }
                    const uint32_t lbt = kEachLoad ? lane_term(lb0) : lb0;
                    const uint32_t voff =
                        FULLC || col < p.N ? lbt + (uint32_t)(((mn_kr(u - LA) * 8 + k0) * p.ldw + col) * 2) : kOOB;
                    if constexpr (NTB) lds_load16_nt(r, sB + q * 1024, kSrdLive || live ? voff : kOOB);
                    else lds_load16(r, sB + q * 1024, kSrdLive || live ? voff : kOOB);
                } else {
                    // weight [N][Kd], contraction contiguous; second segment from w1
                    const bool seg1 = p.two_seg && k0 >= p.Kd;
                    const i32x4 r = seg1 ? c_srdB1 : c_srdB0;
                    const int kk0 = seg1 ? k0 - p.Kd : k0;
                    const uint32_t lt = lane_term(LY::kc_period(q) ? lb1 : lb0);
                    const uint32_t voff = lt + (uint32_t)((q * LY::kRowsPerLoad * p.ldw + kk0) * 2);
                    lds_load16(r, sB + q * 1024, kSrdLive || live ? voff : kOOB);
                }
            }
        }
    };
    auto issue = [&](int kt, int slot, bool live) {
        const StageSrd ss = stage_srd(kt);
#pragma unroll
        for (int u = 0; u < LPW; ++u) load_one(kt, slot, u, live, ss);
    };

    f32x16 acc[MTW][NTW];
    // Two fragment buffers: the fragments of k16 step s+1 are read while
    // the MFMAs of step s run.
    bf16x8 af[2][MTW], bfv[2][NTW];
    // Reading the fragments of NB of the wave's MFMA rows (the others stay
    // idle for tiles whose valid rows end before them).
    auto load_frags = [&](int slot, int kk, int buf, auto nb_tag) {
        constexpr int NB = decltype(nb_tag)::value;
        const uint8_t* sA = smem + slot * TL::kStage;
        const uint8_t* sB = sA + TL::kABytes;
#pragma unroll
        for (int mt = 0; mt < NB; ++mt) {
            const int rb = row_base(mt);
            af[buf][mt] = SCHED == SCHED_ROWS ? LY::frag_kc(sA, rb, kk, lane) : LY::frag_mn(sA, rb, kk, lane);
        }
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            const int cb = col_of(nt);
            bfv[buf][nt] = (SCHED == SCHED_ROWS && LB == LAY_KC) ? LY::frag_kc(sB, cb, kk, lane)
                                                                 : LY::frag_mn(sB, cb, kk, lane);
        }
    };
    static_assert(KK == 2, "two k16 steps per stage");

    // Pipeline over a ring of S LDS stages, loads S-1 stages ahead.  The k16
    // steps of a stage issue the loads of the issue cursor's stage (one every
    // few MFMAs) and read the next step's fragments (one LDS read per MFMA), so
    // LDS-direct writes, fragment reads and MFMAs overlap instead of coming in
    // bursts.  Every stage issues the same number of loads (zero loads once no
    // tile is left), so "stages up to gs+2 have landed" is a fixed vmcnt of S-3
    // stages at the end of stage gs.  The barrier after it publishes stage gs+2
    // (first read in the last step of stage gs+1) and frees the slot of stage
    // gs, which stage gs+1's loads refill.
    constexpr int kWaitLoads = (S - 3) * LPW + (kGW ? 1 : 0);
    if constexpr (kGW) {
        // the first cursor stage's tokens (buffer 0), then the next stage's
        fetch_tokens(0);
        fetch_tokens(1);
    }
#pragma unroll
    for (int t = 0; t < S - 1; ++t) {
        if constexpr (kGW) wait_vmcnt_mem<0>();  // this stage's tokens have landed
        issue(ik, t, itile < n_tiles_total);
        advance();
    }
    wait_vmcnt<kWaitLoads>();
    __syncthreads();
    pf_issued = false;  // the prologue's wait covered any prefetch

    unsigned gs = 0;  // global stage index of this workgroup; its LDS slot is gs % S
    // One stage of the current tile on NB of the wave's MFMA rows.
    auto stage = [&](auto nb_tag) {
        constexpr int NB = decltype(nb_tag)::value;
        // LDS reads one fragment set takes: a KC fragment is one 16-byte read,
        // an MN fragment two transposing 8-byte reads
        constexpr int kReadsA = SCHED == SCHED_ROWS ? NB : 2 * NB;
        constexpr int kReadsB = (SCHED == SCHED_ROWS && LB == LAY_KC) ? NTW : 2 * NTW;
        constexpr int kReads = kReadsA + kReadsB;
        constexpr int kMfma = NB * NTW;
        const bool live = itile < n_tiles_total;
        const int kn = ik;  // the issue cursor's stage, loaded into the slot of gs-1
        const StageSrd ss = stage_srd(kn);
        const int nslot = (int)((gs + S - 1) % S);
        const int slot = (int)(gs % S), slot1 = (int)((gs + 1) % S);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            // next step: (gs, 1) or (gs+1, 0)
            if (kk + 1 < KK) load_frags(slot, kk + 1, (kk + 1) & 1, nb_tag);
            else load_frags(slot1, 0, (kk + 1) & 1, nb_tag);
#pragma unroll
            for (int mt = 0; mt < NB; ++mt) {
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfv[kk & 1][nt], af[kk & 1][mt],
                                                                          acc[mt][nt], 0, 0, 0);
                // this step's share of the stage's loads, spread over its MFMA rows
                const int lo = kk * LPW / KK, n = (kk + 1) * LPW / KK - lo;
#pragma unroll
                for (int i = 0; i < LPW; ++i)
                    if (i < n && i * NB / n == mt) load_one(kn, nslot, lo + i, live, ss);
            }
            // each MFMA followed by its share of the LDS reads (at most one
            // per MFMA when there are more MFMAs than reads)
            constexpr int kPer = (kReads + kMfma - 1) / kMfma;
#pragma unroll
            for (int t = 0; t < kMfma; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                if (t * kPer < kReads) __builtin_amdgcn_sched_group_barrier(0x100, kPer, 0);  // LDS reads
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        advance();
        if (GATHER && pf_issued) {
            // the LA index loads advance() just issued are the newest
            pf_issued = false;
            wait_vmcnt<kWaitLoads + LA>();
        } else {
            wait_vmcnt<kWaitLoads>();
        }
        __syncthreads();
    };
    auto run_tile = [&](int KT, auto nb_tag) {
        if (KT > 0) load_frags((int)(gs % S), 0, 0, nb_tag);
        for (int kt = 0; kt < KT; ++kt, ++gs) stage(nb_tag);
    };

    for (int tile = tile0; tile < n_tiles_total; tile += G) {
        const TileDesc cd = decode(tile);
        const int j = cd.j, row0 = cd.row0, valid = cd.valid, ni = cd.ni, mi_w = cd.mi_w, KT = cd.KT, ks = cd.ks;

        if constexpr (kMf16) {
            // ---- the 256 x 256 body on 16x16x32 MFMAs ----
            f32x4 acc16[MB16][NB16];
#pragma unroll
            for (int a = 0; a < MB16; ++a)
#pragma unroll
                for (int b = 0; b < NB16; ++b) acc16[a][b] = f32x4{};
            // first row / column (within the tile) of the wave's 16-row block m and
            // 16-column block n
            auto row16 = [&](int m) { return wm * (BM / WM) + 16 * m; };
            auto col16 = [&](int n) { return wn * (BN / WN) + 16 * n; };
            auto frag_a = [&](int slot, int m) {
                const uint8_t* sA = smem + slot * TL::kStage;
                return SCHED == SCHED_ROWS ? LY::frag_kc16(sA, row16(m), lane) : LY::frag_mn16(sA, row16(m), lane);
            };
            auto frag_b = [&](int slot, int n) {
                const uint8_t* sB = smem + slot * TL::kStage + TL::kABytes;
                return LB == LAY_KC ? LY::frag_kc16(sB, col16(n), lane) : LY::frag_mn16(sB, col16(n), lane);
            };
            // Each stage runs in two column halves: rows 0..MB16-1 against B blocks
            // 0..NB16/2-1, then against the other half.  All A fragments of the stage
            // stay in registers; the B fragments of the second half are read early in
            // the first half (from this stage's slot), and in the second half each A
            // fragment is read again for the next stage right after its last use, and
            // the next stage's first-half B fragments early on.  Every fragment is
            // thus read at least 4 rows of MFMAs before its first use,
            // with as many fragment registers as the 32x32x16 bodies (16 of 4).  The
            // next stage's fragments come from its slot, published by the barrier
            // that ended the stage before.
            constexpr int NH = NB16 / 2;
            bf16x8 a16[MB16], b16[NB16];
            if (KT > 0) {
                const int slot = (int)(gs % S);
#pragma unroll
                for (int m = 0; m < MB16; ++m) a16[m] = frag_a(slot, m);
#pragma unroll
                for (int n = 0; n < NH; ++n) b16[n] = frag_b(slot, n);
            }
            for (int kt = 0; kt < KT; ++kt, ++gs) {
                const bool live = itile < n_tiles_total;
                const int kn = ik;  // the issue cursor's stage, loaded into the slot of gs-1
                const StageSrd ss = stage_srd(kn);
                const int nslot = (int)((gs + S - 1) % S);
                const int slot = (int)(gs % S), slot1 = (int)((gs + 1) % S);
                // first half: this stage's second-half B fragments are read along the way
#pragma unroll
                for (int m = 0; m < MB16; ++m) {
#pragma unroll
                    for (int n = 0; n < NH; ++n)
                        acc16[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b16[n], a16[m], acc16[m][n], 0, 0, 0);
                    if (m < NH) b16[NH + m] = frag_b(slot, NH + m);
#pragma unroll
                    for (int i = 0; i < LPW; ++i)
                        if (i * 2 * MB16 / LPW == m) load_one(kn, nslot, i, live, ss);
                }
                // the halves stay apart: mixed, some first-half MFMAs would wait for the
                // second half's B fragments, read moments before
                __builtin_amdgcn_sched_barrier(0);
                // second half: the next stage's A fragments, and its first-half B ones
#pragma unroll
                for (int m = 0; m < MB16; ++m) {
#pragma unroll
                    for (int n = NH; n < NB16; ++n)
                        acc16[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b16[n], a16[m], acc16[m][n], 0, 0, 0);
                    a16[m] = frag_a(slot1, m);
                    if (m < NH) b16[m] = frag_b(slot1, m);
#pragma unroll
                    for (int i = 0; i < LPW; ++i)
                        if (i * 2 * MB16 / LPW == MB16 + m) load_one(kn, nslot, i, live, ss);
                }
                __builtin_amdgcn_sched_barrier(0);
                advance();
                if (GATHER && pf_issued) {
                    pf_issued = false;
                    wait_vmcnt<kWaitLoads + LA>();
                } else {
                    wait_vmcnt<kWaitLoads>();
                }
                __syncthreads();
            }

            // ---- epilogue: lane holds row l%16 and columns 4*(l/16) + 0..3 of each 16 x 16 block ----
            if constexpr (SCHED == SCHED_WGRAD) {
                // fp32 dW: each lane stores its 4 columns of a row (16 bytes); a
                // store instruction covers 64 bytes of each of 16 rows, and L2
                // merges the pieces of a line before it writes it back
                const int cq = 4 * (lane >> 4);
#pragma unroll
                for (int m = 0; m < MB16; ++m) {
                    const int mrow = mi_w * BM + row16(m) + (lane & 15);
                    if (mrow >= p.M) continue;
#pragma unroll
                    for (int nb = 0; nb < NB16; ++nb) {
                        const int n = ni * BN + col16(nb) + cq;
                        if (n >= p.N) continue;
                        const bool second = n >= p.n_split;
                        float* base = second ? p.cf2 : p.cf;
                        const int nn = second ? n - p.n_split : n;
                        *(f32x4*)(base + ((int64_t)j * p.M + mrow) * p.n_split + nn) = acc16[m][nb];
                    }
                }
                continue;
            }
            static_assert(EPI == EPI_SWIGLU_BWD || SCHED == SCHED_WGRAD, "16x16x32 body: the down dgrad or dW");
            if constexpr (EPI == EPI_SWIGLU_BWD && MOE_GEMM_DGRAD_STAGED) {  // the accumulators are dh
                // The saved (a, b) pairs come in, and (da, db) go out, as whole
                // 256-byte row pieces through the wave's 8 KiB of the free slot:
                // one 16-row block at a time, a in its first 4 KiB and b in the
                // second (16 rows x 256 bytes each, 16-byte chunks XOR-swizzled by
                // row).  Each lane reads its MFMA-layout values from there, writes
                // (da, db) over them, and the rows go back out whole.  The rows of
                // the next kPre blocks are in flight while a block is worked on.
                static_assert(TL::kStage / TL::kWaves >= 8192 && BN / WN == 128, "staging space per wave");
                uint8_t* stg = smem + ((gs + S - 1) % S) * TL::kStage + wave * 8192;
                const int ln = lane_id_here();
                auto sa = [&](int hb, int row, int chunk) {
                    return (MOE_LDS uint8_t*)(stg + hb * 4096 + row * 256 + ((chunk ^ row) << 4));
                };
                // row-wise: instruction i covers rows 4i..4i+3, lane ln row 4i + ln/16 and chunk ln%16
                const int rw = ln >> 4, cc = ln & 15;
                const int ncol = ni * BN + wn * (BN / WN) + 8 * cc;  // the chunk's first column
                const bool col_ok = ncol < p.N;
                constexpr int kPre = MOE_GEMM_DGRAD_PREFETCH;
                u32x4 ld[kPre][2][4];
                auto issue_loads = [&](int m) {
                    u32x4(&l)[2][4] = ld[m % kPre];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int mloc = row16(m) + 4 * i + rw;
                        l[0][i] = l[1][i] = u32x4{0u, 0u, 0u, 0u};
                        if (mloc < valid && col_ok) {
                            const uint16_t* src = p.ab + (int64_t)(row0 + mloc) * 2 * p.N + ncol;
                            l[0][i] = *(const u32x4*)src;
                            l[1][i] = *(const u32x4*)(src + p.N);
                        }
                    }
                };
                // MFMA layout: row ln%16, columns 4q..4q+3 of each 16-column block
                const int r = ln & 15, q = ln >> 4;
#pragma unroll
                for (int m = 0; m < kPre && m < MB16; ++m) issue_loads(m);
#pragma unroll
                for (int m = 0; m < MB16; ++m) {
                    // An empty asm that reads and rewrites this block's accumulators in
                    // AGPRs keeps the compiler from copying later blocks into VGPRs at
                    // the start of the epilogue; without it the 256-row body ran out of
                    // VGPRs and spilled, and each reload waited for every store issued
                    // before it.  (The 32x32 epilogues do not gain from the same.)
#pragma unroll
                    for (int nb = 0; nb < NB16; ++nb) asm volatile("" : "+a"(acc16[m][nb]));
#pragma unroll
                    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) *(MOE_LDS u32x4*)sa(hb, 4 * i + rw, cc) = ld[m % kPre][hb][i];
                    asm volatile("" ::: "memory");  // a wave's LDS accesses execute in order
                    if (m + kPre < MB16) issue_loads(m + kPre);
#pragma unroll
                    for (int nb = 0; nb < NB16; ++nb) {
                        MOE_LDS uint8_t* pa = sa(0, r, 2 * nb + (q >> 1)) + 8 * (q & 1);
                        MOE_LDS uint8_t* pb = sa(1, r, 2 * nb + (q >> 1)) + 8 * (q & 1);
                        const u32x2 aw = *(const MOE_LDS u32x2*)pa, bw = *(const MOE_LDS u32x2*)pb;
                        float da[4], db[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float v = acc16[m][nb][i];
                            const float a = (i & 1) ? bf_hi(aw[i >> 1]) : bf_lo(aw[i >> 1]);
                            const float b = (i & 1) ? bf_hi(bw[i >> 1]) : bf_lo(bw[i >> 1]);
                            // da = dh b s (1 + a (1 - s)), db = dh a s, with s = sigmoid(a)
                            const float sg = sigmoid_f(a);
                            const float u = v * sg, w = u * b;
                            db[i] = u * a;
                            da[i] = __builtin_fmaf(w, __builtin_fmaf(-a, sg, a), w);
                        }
                        *(MOE_LDS u32x2*)pa = u32x2{pack_bf2x(da[0], da[1]), pack_bf2x(da[2], da[3])};
                        *(MOE_LDS u32x2*)pb = u32x2{pack_bf2x(db[0], db[1]), pack_bf2x(db[2], db[3])};
                    }
                    asm volatile("" ::: "memory");
#pragma unroll
                    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const u32x4 v = *(const MOE_LDS u32x4*)sa(hb, 4 * i + rw, cc);
                            const int mloc = row16(m) + 4 * i + rw;
                            if (mloc < valid && col_ok)
                                *(u32x4*)(p.c + (int64_t)(row0 + mloc) * p.ldc + hb * p.N + ncol) = v;
                        }
                    asm volatile("" ::: "memory");  // this block's rows are read before the next is written
                }
                __syncthreads();  // every wave is done with the slot before the next stage refills it
            } else if constexpr (EPI == EPI_SWIGLU_BWD) {  // the accumulators are dh
                const int cq = 4 * (lane >> 4);
#pragma unroll
                for (int mp = 0; mp < MB16 / 2; ++mp) {
                    // two 16-row blocks at a time: their saved (a, b) pairs are all
                    // loaded before any of their results is stored
                    u32x2 aw[2][NB16], bw[2][NB16];
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int mloc = row16(2 * mp + h2) + (lane & 15);
                        const int64_t row = row0 + mloc;
#pragma unroll
                        for (int nb = 0; nb < NB16; ++nb) {
                            const int n = ni * BN + col16(nb) + cq;
                            aw[h2][nb] = bw[h2][nb] = u32x2{0u, 0u};
                            if (mloc < valid && n < p.N) {
                                aw[h2][nb] = *(const u32x2*)(p.ab + row * 2 * p.N + n);
                                bw[h2][nb] = *(const u32x2*)(p.ab + row * 2 * p.N + p.N + n);
                            }
                        }
                    }
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                        for (int nb = 0; nb < NB16; ++nb) asm volatile("" ::"v"(aw[h2][nb]), "v"(bw[h2][nb]));
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int mloc = row16(2 * mp + h2) + (lane & 15);
                        if (mloc >= valid) continue;
                        const int64_t row = row0 + mloc;
#pragma unroll
                        for (int nb = 0; nb < NB16; ++nb) {
                            const int n = ni * BN + col16(nb) + cq;
                            if (n >= p.N) continue;
                            float da[4], db[4];
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const float v = acc16[2 * mp + h2][nb][i];
                                float a = (i & 1) ? bf_hi(aw[h2][nb][i >> 1]) : bf_lo(aw[h2][nb][i >> 1]);
                                float b = (i & 1) ? bf_hi(bw[h2][nb][i >> 1]) : bf_lo(bw[h2][nb][i >> 1]);
                                float sg = sigmoid_f(a);
                                da[i] = v * b * sg * (1.0f + a * (1.0f - sg));
                                db[i] = v * a * sg;
                            }
                            u32x2 dw = {pack_bf2(da[0], da[1]), pack_bf2(da[2], da[3])};
                            u32x2 ew = {pack_bf2(db[0], db[1]), pack_bf2(db[2], db[3])};
                            *(u32x2*)(p.c + row * p.ldc + n) = dw;
                            *(u32x2*)(p.c + row * p.ldc + p.N + n) = ew;
                        }
                    }
                }
            }
            continue;
        }
#pragma unroll
        for (int a = 0; a < MTW; ++a)
#pragma unroll
            for (int b = 0; b < NTW; ++b) acc[a][b] = f32x16{};
        // Row-tiled GEMMs: the wave's MFMA rows that hold valid rows (row
        // blocks are dealt to the waves in turn, so both wave rows keep an
        // equal share); the rest of the wave's rows stay idle.  Every wave
        // still issues its loads and meets every barrier of every stage.
        // Tiles whose rows fill every MFMA row of the wave (and every tile of
        // the 256-row body, the large workloads' body) run the loop written
        // out below; the stage lambda compiles into slower code for them.
        constexpr bool kIdleRows = SCHED == SCHED_ROWS && BM < 256;
        static_assert(!kIdleRows || MTW <= 3, "idle-row bodies have at most three MFMA rows per wave");
        int nb = MTW;
        if (kIdleRows) {
            const int blocks = (valid + 31) / 32;
            nb = __builtin_amdgcn_readfirstlane(min(MTW, max(1, (blocks - wm + WM - 1) / WM)));
        }
        if (!kIdleRows || nb >= MTW) {
            constexpr int kReadsA = SCHED == SCHED_ROWS ? MTW : 2 * MTW;
            constexpr int kReadsB = (SCHED == SCHED_ROWS && LB == LAY_KC) ? NTW : 2 * NTW;
            constexpr int kReads = kReadsA + kReadsB;
            constexpr int kMfma = MTW * NTW;
            constexpr auto kAll = std::integral_constant<int, MTW>{};
            if (KT > 0) load_frags((int)(gs % S), 0, 0, kAll);
            for (int kt = 0; kt < KT; ++kt, ++gs) {
                const bool live = itile < n_tiles_total;
                const int kn = ik;  // the issue cursor's stage, loaded into the slot of gs-1
                const StageSrd ss = stage_srd(kn);
                const int nslot = (int)((gs + S - 1) % S);
                const int slot = (int)(gs % S), slot1 = (int)((gs + 1) % S);
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    // next step: (gs, 1) or (gs+1, 0)
                    if (kk + 1 < KK) load_frags(slot, kk + 1, (kk + 1) & 1, kAll);
                    else load_frags(slot1, 0, (kk + 1) & 1, kAll);
#pragma unroll
                    for (int mt = 0; mt < MTW; ++mt) {
#pragma unroll
                        for (int nt = 0; nt < NTW; ++nt)
                            acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfv[kk & 1][nt], af[kk & 1][mt],
                                                                                  acc[mt][nt], 0, 0, 0);
                        // this step's share of the stage's loads, spread over its MFMA rows
                        const int lo = kk * LPW / KK, n = (kk + 1) * LPW / KK - lo;
#pragma unroll
                        for (int i = 0; i < LPW; ++i)
                            if (i < n && i * MTW / n == mt) load_one(kn, nslot, lo + i, live, ss);
                    }
                    constexpr int kPer = (kReads + kMfma - 1) / kMfma;
#pragma unroll
                    for (int t = 0; t < kMfma; ++t) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                        if (t * kPer < kReads) __builtin_amdgcn_sched_group_barrier(0x100, kPer, 0);  // LDS reads
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                advance();
                if (GATHER && pf_issued) {
                    pf_issued = false;
                    wait_vmcnt<kWaitLoads + LA>();
                } else {
                    wait_vmcnt<kWaitLoads>();
                }
                __syncthreads();
            }
        } else if constexpr (kIdleRows) {
            // fewer MFMA rows than the wave has (nb < MTW <= 3)
            if constexpr (MTW >= 3) {
                if (nb >= 2) run_tile(KT, std::integral_constant<int, 2>{});
                else run_tile(KT, std::integral_constant<int, 1>{});
            } else {
                run_tile(KT, std::integral_constant<int, 1>{});
            }
        }

        // ---- epilogue: lane holds row (l%32) and columns 8*j4 + 4*(l/32) + 0..3 ----
        if constexpr (EPI == EPI_BF16 || EPI == EPI_F32) {
            // Plain results go out through LDS so that every store writes whole
            // 128-byte row lines (stored straight from the MFMA layout, each
            // store touches 32 rows).  The stage slot of the last stage (gs-1)
            // is free until the next stage issues its loads; each wave stages
            // 32 rows x 128 bytes at a time in its own 4 KiB of that slot, with
            // 16-byte chunks XOR-swizzled by row.  Where the slot has 8 KiB per
            // wave (the 256-row body), two such blocks are written before either
            // is read back, so each wait for LDS data covers two blocks.
            static_assert(TL::kStage / TL::kWaves >= 4096, "staging space per wave");
            constexpr int kBufs = TL::kStage / TL::kWaves >= 8192 ? 2 : 1;
            uint8_t* stg = smem + ((gs + S - 1) % S) * TL::kStage + wave * (kBufs * 4096);
            // the addresses derived from the lane are rebuilt here, per tile,
            // instead of being hoisted out of the tile loop, where the 256-row
            // body has no registers left for them and spills them (each reload
            // then waits for every store issued before it)
            const int ln = lane_id_here();
            const int r = ln & 31, h = ln >> 5;
            auto stage_addr = [&](int buf, int row, int chunk) {
                return (MOE_LDS uint8_t*)(stg + buf * 4096 + row * 128 + ((chunk ^ (row & 7)) << 4));
            };
            // column groups per round: 64 bf16 (two MFMA tiles) or 32 fp32 (one)
            constexpr int kTilesPerRound = EPI == EPI_BF16 ? 2 : 1;
            // row-tiled fp32 output with a bias: the bias of this lane's
            // columns is loaded, and waited for once, before the tile's first
            // store (a load issued behind stores also waits for them)
            constexpr bool kBias = EPI == EPI_F32 && SCHED == SCHED_ROWS;
            f32x4 bias_v[kBias ? NTW : 1] = {};
            if constexpr (kBias) {
                if (p.bias) {
#pragma unroll
                    for (int np = 0; np < NTW; ++np) {
                        const int n = ni * BN + wn * (BN / WN) + 32 * np + 4 * (ln & 7);
                        if (n < p.N) bias_v[np] = *(const f32x4*)(p.bias + n);
                    }
#pragma unroll
                    for (int np = 0; np < NTW; ++np) asm volatile("" ::"v"(bias_v[np]));
                }
            }
            constexpr int kRounds = NTW / kTilesPerRound;
            static_assert(kRounds % kBufs == 0, "rounds in whole pairs");
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt) {
                // one row block after another (the scheduler does not interleave
                // blocks); with the packed pair conversion below, the 256-row
                // bodies of this epilogue do not spill
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int np0 = 0; np0 < kRounds; np0 += kBufs) {
#pragma unroll
                    for (int b = 0; b < kBufs; ++b) {
#pragma unroll
                        for (int q = 0; q < kTilesPerRound; ++q) {
                            const f32x16& a = acc[mt][(np0 + b) * kTilesPerRound + q];
#pragma unroll
                            for (int j4 = 0; j4 < 4; ++j4) {
                                if (EPI == EPI_BF16) {
                                    u32x2 w = {pack_bf2x(a[4 * j4], a[4 * j4 + 1]), pack_bf2x(a[4 * j4 + 2], a[4 * j4 + 3])};
                                    *(MOE_LDS u32x2*)(stage_addr(b, r, 4 * q + j4) + 8 * h) = w;
                                } else {
                                    f32x4 w = {a[4 * j4], a[4 * j4 + 1], a[4 * j4 + 2], a[4 * j4 + 3]};
                                    *(MOE_LDS f32x4*)stage_addr(b, r, 2 * j4 + h) = w;
                                }
                            }
                        }
                    }
#pragma unroll
                    for (int b = 0; b < kBufs; ++b) {
                    const int np = np0 + b;
                    // read back 8 rows x 128 bytes per instruction and store whole lines
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int rr = 8 * i + (ln >> 3), c = ln & 7;
                        const u32x4 v = *(const MOE_LDS u32x4*)stage_addr(b, rr, c);
                        const int mloc = row_base(mt) + rr;
                        if (EPI == EPI_BF16) {
                            const int n = ni * BN + wn * (BN / WN) + 64 * np + 8 * c;
                            if (mloc < valid && n < p.N) *(u32x4*)(p.c + (int64_t)(row0 + mloc) * p.ldc + n) = v;
                        } else if (SCHED == SCHED_WGRAD) {
                            const int m = mi_w * BM + mloc;
                            const int n = ni * BN + wn * (BN / WN) + 32 * np + 4 * c;
                            if (m < p.M && n < p.N) {
                                // a plain store: L2 merges the pieces of a row into whole
                                // lines (a non-temporal store doubled the HBM write traffic)
                                const bool second = n >= p.n_split;
                                float* base = second ? p.cf2 : p.cf;
                                const int nn = second ? n - p.n_split : n;
                                *(u32x4*)(base + ((int64_t)j * p.M + m) * p.n_split + nn) = v;
                            }
                        } else {
                            // row-tiled fp32 output: one partial per contraction chunk
                            const int n = ni * BN + wn * (BN / WN) + 32 * np + 4 * c;
                            if (mloc < valid && n < p.N) {
                                u32x4 w = v;
                                if (p.bias) {
                                    f32x4 f = __builtin_bit_cast(f32x4, v);
                                    f += bias_v[kBias ? np : 0];
                                    w = __builtin_bit_cast(u32x4, f);
                                }
                                *(u32x4*)(p.cf + ks * p.part_stride + (int64_t)(row0 + mloc) * p.ldc + n) = w;
                            }
                        }
                    }
                    }
                }
            }
            __syncthreads();  // every wave is done with the slot before the next stage refills it
            continue;
        }
        if constexpr (EPI == EPI_SWIGLU && NTW == 4 && !GATHER) {
            // SwiGLU outputs go out through LDS as the bf16 ones do: each wave
            // holds 64 columns of h (and of a and b) per 32-row block, one 4 KiB
            // staging block of 32 rows x 128 bytes, stored as whole lines.  Stored
            // straight from the MFMA layout, each store covers 16 bytes of 32
            // rows, and the tile's h and ab stores took about twice as long.  The
            // gathered-row bodies keep the direct stores: their extra per-lane row
            // offsets leave no registers for the staged form, which spilled there.
            constexpr int kBufs = TL::kStage / TL::kWaves >= 8192 ? 2 : 1;
            uint8_t* stg = smem + ((gs + S - 1) % S) * TL::kStage + wave * (kBufs * 4096);
            const int ln = lane_id_here();
            const int r = ln & 31, hh = ln >> 5;
            auto stage_addr = [&](int buf, int row, int chunk) {
                return (MOE_LDS uint8_t*)(stg + buf * 4096 + row * 128 + ((chunk ^ (row & 7)) << 4));
            };
            const int hc0 = ni * (BN / 2) + wn * (BN / 2 / WN);  // the wave's first h column
            // read the staged block back, 8 rows x 128 bytes per instruction
            auto flush = [&](int buf, int mt, uint16_t* dst, int64_t ld, int col0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = 8 * i + (ln >> 3), c = ln & 7;
                    const u32x4 v = *(const MOE_LDS u32x4*)stage_addr(buf, rr, c);
                    const int mloc = row_base(mt) + rr;
                    const int n = hc0 + 8 * c;
                    if (mloc < valid && n < p.N) *(u32x4*)(dst + (int64_t)(row0 + mloc) * ld + col0 + n) = v;
                }
            };
            // lane (r, hh) holds columns 8*j4 + 4*hh + 0..3 of 32-column block i2 in row r
            auto put = [&](int buf, int i2, int j4, u32x2 w) {
                *(MOE_LDS u32x2*)(stage_addr(buf, r, 4 * i2 + j4) + 8 * hh) = w;
            };
            // the saved a (or b) values of block mt, into staging block buf (with
            // single conversions: the packed form made this body spill)
            auto put_ab = [&](int buf, int mt, int half) {
#pragma unroll
                for (int i2 = 0; i2 < 2; ++i2) {
                    const f32x16& v = acc[mt][2 * half + i2];
#pragma unroll
                    for (int j4 = 0; j4 < 4; ++j4)
                        put(buf, i2, j4, u32x2{pack_bf2(v[4 * j4], v[4 * j4 + 1]), pack_bf2(v[4 * j4 + 2], v[4 * j4 + 3])});
                }
            };
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt) {
                if (row_base(mt) >= valid) continue;  // no valid row in this block (uniform)
#pragma unroll
                for (int i2 = 0; i2 < 2; ++i2) {
                    const f32x16& ga = acc[mt][i2];
                    const f32x16& ub = acc[mt][2 + i2];
#pragma unroll
                    for (int j4 = 0; j4 < 4; ++j4) {
                        float hv[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) hv[i] = silu_f(ga[4 * j4 + i]) * ub[4 * j4 + i];
                        put(0, i2, j4, u32x2{pack_bf2x(hv[0], hv[1]), pack_bf2x(hv[2], hv[3])});
                    }
                }
                if (p.c2) {
                    if (kBufs == 2) {
                        // h and a staged together, then b
                        put_ab(kBufs - 1, mt, 0);
                        flush(0, mt, p.c, p.ldc, 0);
                        flush(kBufs - 1, mt, p.c2, 2 * (int64_t)p.N, 0);
                    } else {
                        flush(0, mt, p.c, p.ldc, 0);
                        put_ab(0, mt, 0);
                        flush(0, mt, p.c2, 2 * (int64_t)p.N, 0);
                    }
                    put_ab(0, mt, 1);
                    flush(0, mt, p.c2, 2 * (int64_t)p.N, p.N);
                } else {
                    flush(0, mt, p.c, p.ldc, 0);
                }
            }
            __syncthreads();  // every wave is done with the slot before the next stage refills it
            continue;
        }
        const int cq = 4 * (lane >> 5);
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt) {
            const int mloc = row_base(mt) + (lane & 31);
            if (mloc >= valid) continue;
            const int64_t row = row0 + mloc;
            if (EPI == EPI_SWIGLU) {
#pragma unroll
                for (int i2 = 0; i2 < NTW / 2; ++i2) {
                    const f32x16& ga = acc[mt][i2];
                    const f32x16& ub = acc[mt][NTW / 2 + i2];
#pragma unroll
                    for (int j4 = 0; j4 < 4; ++j4) {
                        const int hc = ni * (BN / 2) + col_of(i2) + 8 * j4 + cq;
                        if (hc >= p.N) continue;
                        float hv[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) hv[i] = silu_f(ga[4 * j4 + i]) * ub[4 * j4 + i];
                        u32x2 hw = {pack_bf2(hv[0], hv[1]), pack_bf2(hv[2], hv[3])};
                        *(u32x2*)(p.c + row * p.ldc + hc) = hw;
                        if (p.c2) {
                            u32x2 aw = {pack_bf2(ga[4 * j4], ga[4 * j4 + 1]), pack_bf2(ga[4 * j4 + 2], ga[4 * j4 + 3])};
                            u32x2 bw = {pack_bf2(ub[4 * j4], ub[4 * j4 + 1]), pack_bf2(ub[4 * j4 + 2], ub[4 * j4 + 3])};
                            *(u32x2*)(p.c2 + row * 2 * p.N + hc) = aw;
                            *(u32x2*)(p.c2 + row * 2 * p.N + p.N + hc) = bw;
                        }
                    }
                }
            } else if (EPI == EPI_BF16) {
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                    for (int j4 = 0; j4 < 4; ++j4) {
                        const int n = ni * BN + col_of(nt) + 8 * j4 + cq;
                        if (n >= p.N) continue;
                        const f32x16& a = acc[mt][nt];
                        u32x2 w = {pack_bf2(a[4 * j4], a[4 * j4 + 1]), pack_bf2(a[4 * j4 + 2], a[4 * j4 + 3])};
                        *(u32x2*)(p.c + row * p.ldc + n) = w;
                    }
            } else {  // EPI_SWIGLU_BWD: the accumulators are dh
                // the row block's saved (a, b) pairs are all loaded before any
                // of its results is stored: a load issued behind stores also
                // waits for them
                u32x2 aw[NTW][4], bw[NTW][4];
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                    for (int j4 = 0; j4 < 4; ++j4) {
                        const int n = ni * BN + col_of(nt) + 8 * j4 + cq;
                        aw[nt][j4] = bw[nt][j4] = u32x2{0u, 0u};
                        if (n < p.N) {
                            aw[nt][j4] = *(const u32x2*)(p.ab + row * 2 * p.N + n);
                            bw[nt][j4] = *(const u32x2*)(p.ab + row * 2 * p.N + p.N + n);
                        }
                    }
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                    for (int j4 = 0; j4 < 4; ++j4) asm volatile("" ::"v"(aw[nt][j4]), "v"(bw[nt][j4]));
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                    for (int j4 = 0; j4 < 4; ++j4) {
                        const int n = ni * BN + col_of(nt) + 8 * j4 + cq;
                        if (n >= p.N) continue;
                        float da[4], db[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float v = acc[mt][nt][4 * j4 + i];
                            float a = (i & 1) ? bf_hi(aw[nt][j4][i >> 1]) : bf_lo(aw[nt][j4][i >> 1]);
                            float b = (i & 1) ? bf_hi(bw[nt][j4][i >> 1]) : bf_lo(bw[nt][j4][i >> 1]);
                            float s = sigmoid_f(a);
                            da[i] = v * b * s * (1.0f + a * (1.0f - s));
                            db[i] = v * a * s;
                        }
                        u32x2 dw = {pack_bf2(da[0], da[1]), pack_bf2(da[2], da[3])};
                        u32x2 ew = {pack_bf2(db[0], db[1]), pack_bf2(db[2], db[3])};
                        *(u32x2*)(p.c + row * p.ldc + n) = dw;
                        *(u32x2*)(p.c + row * p.ldc + p.N + n) = ew;
                    }
            }
        }
    }
    wait_vmcnt<0>();  // the zero loads issued past the last tile
}

// Whether tiles of ALT rows beat tiles of BM rows on this call's row counts:
// every workgroup evaluates the same device-resident counts, so all agree.
// Cost model: rounds of tiles over the grid times the tile's rows, with 10%
// added for the smaller tile, whose MFMAs run a little less efficiently.
template <int BM, int ALT, int BN, int EPI, int THREADS>
__device__ __forceinline__ bool prefer_alt(const GemmParams& p, const int* s_off, int* s_wave) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int mb = 0, ma = 0;
    for (int j = tid; j < p.e_local; j += THREADS) {
        const int c = s_off[j + 1] - s_off[j];
        mb += (c + BM - 1) / BM;
        ma += (c + ALT - 1) / ALT;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        mb += __shfl_xor(mb, o, 64);
        ma += __shfl_xor(ma, o, 64);
    }
    if (lane == 0) {
        s_wave[2 * wave] = mb;
        s_wave[2 * wave + 1] = ma;
    }
    __syncthreads();
    mb = ma = 0;
    for (int w = 0; w < THREADS / 64; ++w) {
        mb += s_wave[2 * w];
        ma += s_wave[2 * w + 1];
    }
    __syncthreads();  // s_wave is reused by the schedule
    const int64_t tn = EPI == EPI_SWIGLU ? (p.N + BN / 2 - 1) / (BN / 2) : (p.N + BN - 1) / BN;
    const int64_t G = gridDim.x;
    const int64_t rb = (mb * tn + G - 1) / G, ra = (ma * tn + G - 1) / G;
    return ra * ALT * 11 < rb * BM * 10;
}

// One launch: loads the row offsets, then runs the BM-row body, or the
// ALT-row body when ALT != 0 and prefer_alt says so.
template <int BM, int BN, int BK, int WM, int WN, int LB, int EPI, int SCHED, int LDSB, int ALT, bool GATHER>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(1, 2)))
void gg_kernel(GemmParams p) {
    using TL = Tile<BM, BN, BK, WM, WN, LDSB>;
    using TA = Tile<ALT ? ALT : BM, BN, BK, WM, WN, LDSB>;
    constexpr int kRing = TL::kStages * TL::kStage;
    constexpr int kRingA = TA::kStages * TA::kStage;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kRing > kRingA ? kRing : kRingA];
    __shared__ int s_off[kMaxGroups + 1];    // clamped row offsets
    __shared__ int s_start[kMaxGroups + 1];  // ROWS: first m-tile of each expert; WGRAD: sorted order
    __shared__ int s_wave[16];
    // GATHER: two buffers of 64 source indices per A load of each wave, and
    // 1 KiB of slack behind them
    __shared__ int s_idx[GATHER ? 2 * TL::kALoads * 64 + 256 : 1];
    __shared__ int s_maxrows;
    // Start stagger, a measurement knob (off unless MOE_GEMM_STAGGER_P > 1 and
    // MOE_GEMM_STAGGER_NS are set): workgroup b waits ((b / 8) % P) * NS
    // before it starts, so that the persistent workgroups reach their tile
    // epilogues, and issue their stores, at different times.  With P = 2..8
    // and steps of 3.75-30 us no GEMM of the layer ran faster (the delay
    // itself was the only change), so the workgroups' stores landing at once
    // do not set the epilogue's cost.
    if (p.stagger_ticks > 0) {
        const int phase = (int)((blockIdx.x >> 3) % (unsigned)p.stagger_phases);
        if (phase) {
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            const uint64_t wait = (uint64_t)phase * (uint64_t)p.stagger_ticks;
            while (__builtin_amdgcn_s_memrealtime() - t0 < wait) __builtin_amdgcn_s_sleep(2);
        }
    }
    if (threadIdx.x == 0) s_maxrows = 0;
    __syncthreads();
    for (int j = threadIdx.x; j <= p.e_local; j += TL::kThreads) {
        const int64_t o = p.offsets ? (int64_t)p.offsets[j] : min((int64_t)j * p.row_chunk, (int64_t)p.dense_rows);
        s_off[j] = (int)(o < p.cap ? o : p.cap);
    }
    __syncthreads();
    // the non-temporal weight path exists for the forward GEMMs (weights N-contiguous)
    constexpr bool kNtPath = SCHED == SCHED_ROWS && LB == LAY_MN && EPI != EPI_F32;
    if constexpr (kNtPath) {
        for (int j = threadIdx.x; j < p.e_local; j += TL::kThreads) atomicMax(&s_maxrows, s_off[j + 1] - s_off[j]);
        __syncthreads();
    }
    const int max_rows = s_maxrows;
    if constexpr (ALT != 0) {
        if (prefer_alt<BM, ALT, BN, EPI, TL::kThreads>(p, s_off, s_wave)) {
            if constexpr (kNtPath) {
                if (max_rows <= ALT) {
                    gg_body<ALT, BN, BK, WM, WN, LB, EPI, SCHED, LDSB, GATHER, true>(p, smem, s_off, s_start, s_wave,
                                                                                     s_idx);
                    return;
                }
            }
            gg_body<ALT, BN, BK, WM, WN, LB, EPI, SCHED, LDSB, GATHER, false>(p, smem, s_off, s_start, s_wave, s_idx);
            return;
        }
    }
    // the 256 x 256 body also comes without the loads' column bounds checks,
    // for outputs whose every tile is whole (all the layer's workloads)
    constexpr bool kFullBody = BM == 256 && BN == 256;
    const bool fullc = kFullBody && (SCHED == SCHED_WGRAD ? p.M % BM == 0 && p.N % BN == 0
                                                          : p.N % (EPI == EPI_SWIGLU ? BN / 2 : BN) == 0);
    if constexpr (kNtPath) {
        if (max_rows <= BM) {
            if constexpr (kFullBody) {
                if (fullc) {
                    gg_body<BM, BN, BK, WM, WN, LB, EPI, SCHED, LDSB, GATHER, true, true>(p, smem, s_off, s_start,
                                                                                          s_wave, s_idx);
                    return;
                }
            }
            gg_body<BM, BN, BK, WM, WN, LB, EPI, SCHED, LDSB, GATHER, true>(p, smem, s_off, s_start, s_wave, s_idx);
            return;
        }
    }
    if constexpr (kFullBody) {
        if (fullc) {
            gg_body<BM, BN, BK, WM, WN, LB, EPI, SCHED, LDSB, GATHER, false, true>(p, smem, s_off, s_start, s_wave,
                                                                                   s_idx);
            return;
        }
    }
    gg_body<BM, BN, BK, WM, WN, LB, EPI, SCHED, LDSB, GATHER, false>(p, smem, s_off, s_start, s_wave, s_idx);
}

// Tile configurations.
//   big    256x256, four 128x128 waves, 4-stage ring (128 KiB LDS, one workgroup
//          per CU).  A 128x128 wave tile is the largest the 256 accumulator
//          registers allow and moves the fewest LDS bytes per MFMA, which is what
//          bounds this kernel.
//   mid    192x256, four 96x128 waves, 4-stage ring (112 KiB): for experts of
//          about 100-190 rows, where a 256-row tile is mostly padding
//   auto   (default) the row-tiled GEMMs carry both big and mid bodies and pick
//          one per call on the device from the row counts; the weight-gradient
//          GEMM uses big
//   small  128x128, four 64x64 waves
// MOE_GEMM_TILE=256, 192 or 128 pins one configuration (for comparisons).
enum : int { CFG_AUTO = 0, CFG_BIG = 1, CFG_MID = 2, CFG_SMALL = 3 };

inline int env_int(const char* name, int dflt) {
    const char* e = getenv(name);
    return e ? atoi(e) : dflt;
}

// read on every call, so a process can compare configurations
inline int tile_config() {
    const int t = env_int("MOE_GEMM_TILE", 0);
    return t == 128 ? CFG_SMALL : t == 192 ? CFG_MID : t == 256 ? CFG_BIG : CFG_AUTO;
}

template <int BM, int BN, int BK, int WM, int WN, int LB, int EPI, int SCHED, int LDSB, int ALT = 0,
          bool GATHER = false>
static int launch_cfg(const GemmParams& p, hipStream_t s) {
    using TL = Tile<BM, BN, BK, WM, WN, LDSB>;
    int64_t total_upper;
    if (SCHED == SCHED_ROWS) {
        const int tn = EPI == EPI_SWIGLU ? (p.N + BN / 2 - 1) / (BN / 2) : (p.N + BN - 1) / BN;
        constexpr int bm = ALT && ALT < BM ? ALT : BM;
        total_upper = ((p.cap + bm - 1) / bm + p.e_local) * (int64_t)tn * std::max(p.ksplit, 1);
    } else {
        total_upper = (int64_t)p.e_local * ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    }
    const int per_cu = (TL::kStage * TL::kStages > 80 * 1024 || TL::kMTW * TL::kNTW >= 8) ? 1 : 2;
    int64_t g = std::min<int64_t>(total_upper, (int64_t)moe_host::num_cus() * per_cu);
    const int grid = (int)((g + 7) / 8 * 8);
    if (grid == 0) return MOE_OK;
    GemmParams q = p;
    q.stagger_phases = std::max(1, env_int("MOE_GEMM_STAGGER_P", 1));
    q.stagger_ticks = q.stagger_phases > 1 ? env_int("MOE_GEMM_STAGGER_NS", 0) / 10 : 0;
    gg_kernel<BM, BN, BK, WM, WN, LB, EPI, SCHED, LDSB, ALT, GATHER><<<grid, TL::kThreads, 0, s>>>(q);
    return moe_host::launch_status();
}

template <int LB, int EPI, int SCHED, bool GATHER = false>
static int launch(const GemmParams& p, hipStream_t s) {
    if (tile_config() == CFG_SMALL)
        return launch_cfg<128, 128, 32, 2, 2, LB, EPI, SCHED, kLdsBudget, 0, GATHER>(p, s);
    if constexpr (SCHED == SCHED_ROWS) {
        if (tile_config() == CFG_MID)
            return launch_cfg<192, 256, 32, 2, 2, LB, EPI, SCHED, kLdsBudget, 0, GATHER>(p, s);
        if (tile_config() == CFG_AUTO)
            return launch_cfg<256, 256, 32, 2, 2, LB, EPI, SCHED, kLdsBudget, 192, GATHER>(p, s);
    }
    return launch_cfg<256, 256, 32, 2, 2, LB, EPI, SCHED, kLdsBudget, 0, GATHER>(p, s);
}

// Launchers of the instantiations, each compiled in one translation unit
// (gemm_rows.hip, gemm_dgrad.hip, gemm_wgrad.hip), so that no kernel is
// instantiated twice in the library.
int launch_rows_mn(const GemmParams& p, int epi, hipStream_t s);  // B [Kd][N]; EPI_BF16 or EPI_SWIGLU_BWD
int launch_rows_kc(const GemmParams& p, int epi, hipStream_t s);  // B [N][Kd]; EPI_BF16 or EPI_SWIGLU_BWD
int launch_wgrad(const GemmParams& p, hipStream_t s);             // SCHED_WGRAD, fp32 out

}  // namespace moe
