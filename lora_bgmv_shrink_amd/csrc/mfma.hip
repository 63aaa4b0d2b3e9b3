// MFMA kernels: SGMV shrink/expand over segment tiles and the fused layer
// GEMM (base product + LoRA expand in the epilogue).
//
// SGMV groups rows by adapter and runs one small product per segment
// ("Serving multiple LoRAs: segmented matrix multiplies and adapter
// scheduling", section "Not merging the weights, computing in batches";
// "Serving Many LoRA Adapters" (praveentn.live), section "Punica: The
// Segmented Gather-Scatter Kernel").  Long segments are real contractions,
// so they run on the matrix cores.  The base product is computed once for
// the batch and the scaled expand is added to it before y is rounded
// ("Serving many LoRA adapters" (blog.ecitis.org), section "Replay":
// segmented gather, grouped GEMM, scatter-add, fused batch output).
//
// Engine.  A workgroup owns a BM x BN output tile split over WM x WN waves;
// each wave holds (BM/WM/16) x (BN/WN/16) 16x16 fp32 accumulators.  Operand
// tiles are staged in LDS K-contiguous ([row][k], rows padded by 16 bytes),
// double-buffered, with the next K-block prefetched into registers while
// the current one feeds the MFMAs:
//   bf16: v_mfma_f32_16x16x32_bf16, lane l supplies row l%16, k (l/16)*8..+8
//   fp32: v_mfma_f32_16x16x4_f32,   lane l supplies row l%16, k l/16
//   output: lane l holds rows (l/16)*4 + 0..3 of column l%16.
#include <atomic>
#include <climits>

#include "lora_internal.hpp"

namespace lora {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// MFMA shapes.  BLK x BLK output block, KSTEP reduction per instruction;
// lane l supplies operand row/column l % BLK and k (l / BLK) * KPL .. + KPL.
template <typename T, int BLK> struct MF;
template <> struct MF<bf16, 16> {
    static constexpr int KSTEP = 32, KPL = 8, NACC = 4;
    using frag = bf16x8_t;
    using acc = f32x4_t;
    static __device__ __forceinline__ frag ld(const bf16* p) { return *(const bf16x8_t*)p; }
    static __device__ __forceinline__ acc mma(frag a, frag b, acc c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // output element q of lane l sits at (row, col) of the block
    static __device__ __forceinline__ int row(int lane, int q) { return (lane >> 4) * 4 + q; }
};
template <> struct MF<bf16, 32> {
    static constexpr int KSTEP = 16, KPL = 8, NACC = 16;
    using frag = bf16x8_t;
    using acc = f32x16_t;
    static __device__ __forceinline__ frag ld(const bf16* p) { return *(const bf16x8_t*)p; }
    static __device__ __forceinline__ acc mma(frag a, frag b, acc c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ int row(int lane, int q) { return (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3); }
};
template <> struct MF<float, 16> {
    static constexpr int KSTEP = 4, KPL = 1, NACC = 4;
    using frag = float;
    using acc = f32x4_t;
    static __device__ __forceinline__ frag ld(const float* p) { return *p; }
    static __device__ __forceinline__ acc mma(frag a, frag b, acc c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ int row(int lane, int q) { return (lane >> 4) * 4 + q; }
};

template <typename T_, int BM_, int BN_, int BK_, int WM_, int WN_, int BLK_ = 16>
struct Cfg {
    using T = T_;
    using M = MF<T_, BLK_>;
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, BLK = BLK_;
    static constexpr int NT = WM * WN * 64;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int FM = WTM / BLK, FN = WTN / BLK;
    static constexpr int VE = 16 / sizeof(T);
    static constexpr int LDK = BK + VE;
    static constexpr int A_ELEMS = BM * LDK;
    static constexpr int B_ELEMS = BN * LDK;
    static constexpr int STAGE = A_ELEMS + B_ELEMS;
    // ranks covered by one K-extension step of the LoRA epilogue: bf16 splits
    // the fp32 operand into hi + lo halves, fp32 takes it as is
    static constexpr int KH = (sizeof(T) == 2) ? BK / 2 : BK;
    static_assert(FM >= 1 && FN >= 1, "wave tile smaller than one MFMA block");
    static_assert(WTM % BLK == 0 && WTN % BLK == 0, "wave tile not a multiple of the MFMA block");
    static_assert(BK % M::KSTEP == 0, "BK not a multiple of the MFMA K");
    static_assert(BK % VE == 0, "BK not a multiple of the vector width");
};

template <class C>
struct Acc {
    typename C::M::acc v[C::FM][C::FN];
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
#pragma unroll
                for (int q = 0; q < C::M::NACC; ++q) v[i][j][q] = 0.f;
    }
};

// acc += sA[wave rows][0:BK] x sB[wave cols][0:BK]^T.  The fragments of
// k-substep s+1 are requested from LDS before (or, for A with a large
// accumulator, right after) the MFMAs of substep s that last read them, so
// LDS latency overlaps the matrix-core work.  A wave whose accumulator takes
// more than 96 registers keeps one set of A fragments, reloading each as soon
// as its row of MFMAs has issued, so that the tile still fits 256 registers.
template <class C>
__device__ __forceinline__ void mma_block(Acc<C>& acc, const typename C::T* sA,
                                          const typename C::T* sB, int wm, int wn, int lane) {
    using T = typename C::T;
    using M = typename C::M;
    constexpr int NSUB = C::BK / M::KSTEP;
    constexpr bool ROLL_A = C::FM * C::FN * M::NACC > 96;
    constexpr int NA = ROLL_A ? 1 : 2;
    const int lr = lane % C::BLK;
    const int kq = (lane / C::BLK) * M::KPL;
    const T* pa = sA + (wm * C::WTM + lr) * C::LDK + kq;
    const T* pb = sB + (wn * C::WTN + lr) * C::LDK + kq;
    typename M::frag a[NA][C::FM], b[2][C::FN];
    // the wave in its MFMA block issues ahead of a wave of the same SIMD that
    // is loading or storing the next block (prefill and mixed batches 0.4-1.5%
    // faster)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < C::FM; ++i) a[0][i] = M::ld(pa + i * C::BLK * C::LDK);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) b[0][j] = M::ld(pb + j * C::BLK * C::LDK);
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
        const int cur = s & 1;
        const int ca = ROLL_A ? 0 : cur;
        const int kk = (s + 1) * M::KSTEP;
        if (s + 1 < NSUB) {
#pragma unroll
            for (int j = 0; j < C::FN; ++j) b[cur ^ 1][j] = M::ld(pb + j * C::BLK * C::LDK + kk);
            if (!ROLL_A) {
#pragma unroll
                for (int i = 0; i < C::FM; ++i) a[ca ^ 1][i] = M::ld(pa + i * C::BLK * C::LDK + kk);
            }
        }
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
#pragma unroll
            for (int j = 0; j < C::FN; ++j) acc.v[i][j] = M::mma(a[ca][i], b[cur][j], acc.v[i][j]);
            if (ROLL_A && s + 1 < NSUB) a[0][i] = M::ld(pa + i * C::BLK * C::LDK + kk);
        }
        if (ROLL_A && s + 1 < NSUB) {
            // keep the order as written: B reads first, then per row its MFMAs
            // and the reload of its A fragment (not sunk next to its next use)
            __builtin_amdgcn_sched_group_barrier(0x100, C::FN, 0);
#pragma unroll
            for (int i = 0; i < C::FM; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, C::FN, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __builtin_amdgcn_s_setprio(0);
}

// K-contiguous rows -> LDS [row][k].  sRow[r] is the source row or -1.
template <class C, int ROWS>
struct RowLoader {
    using T = typename C::T;
    static constexpr int VPR = C::BK / C::VE;
    static constexpr int TOT = ROWS * VPR;
    static constexpr int NV = (TOT + C::NT - 1) / C::NT;
    uint4 reg[NV];

    // Inside K (k0 + BK <= K, decided once per block) every lane issues its
    // vector load unconditionally; rows past the end read row 0 and are
    // zeroed afterwards, so no branch splits the batch of loads.
    __device__ __forceinline__ void load(const T* __restrict__ base, int64_t ld, const int* sRow,
                                         int k0, int K, int tid) {
        if (k0 + C::BK <= K) {
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int idx = tid + v * C::NT;
                if (TOT % C::NT != 0 && idx >= TOT) break;
                const int r = idx / VPR;
                const int k = k0 + (idx - r * VPR) * C::VE;
                // a row past the end reads row 0; it only feeds output rows that are
                // never stored
                const int gr = sRow[r];
                reg[v] = *(const uint4*)(base + (int64_t)(gr >= 0 ? gr : 0) * ld + k);
            }
            return;
        }
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int idx = tid + v * C::NT;
            if (TOT % C::NT != 0 && idx >= TOT) break;
            const int r = idx / VPR;
            const int k = k0 + (idx - r * VPR) * C::VE;
            const int gr = sRow[r];
            union { uint4 u; T e[C::VE]; } tmp;
#pragma unroll
            for (int e = 0; e < C::VE; ++e)
                tmp.e[e] = (gr >= 0 && k + e < K) ? base[(int64_t)gr * ld + k + e] : (T)0;
            reg[v] = tmp.u;
        }
    }
    // A whole K-block (k0 + BK <= K) through a buffer resource whose base is
    // the tile's first row and whose range ends after its last valid row:
    // rows past it read as 0 (they only feed outputs never stored).  The
    // row offset of each piece is a per-lane VGPR, the K position a scalar.
    __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t rs, int64_t ld, int k0, int tid) {
        static_assert(C::NT % VPR == 0, "pieces of a lane share one column");
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const int r0 = tid / VPR;
        const int c = (tid - r0 * VPR) * C::VE;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            if (TOT % C::NT != 0 && tid + v * C::NT >= TOT) break;
            const int voff = (int)(((int64_t)(r0 + v * (C::NT / VPR)) * ld + c) * (int64_t)sizeof(T));
            const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, k0 * (int)sizeof(T), 0);
            reg[v] = __builtin_bit_cast(uint4, x);
        }
    }
    // Byte offsets of this lane's pieces within a buffer resource: row
    // sRow[r] - base_row of the source, or `none` (past the resource's range,
    // so the piece reads as 0) for a row of -1.  Computed once per tile.
    __device__ __forceinline__ void row_offsets(const int* sRow, int base_row, int64_t ld, int none, int tid,
                                                int (&voff)[NV]) const {
        static_assert(C::NT % VPR == 0, "pieces of a lane share one column");
        const int r0 = tid / VPR;
        const int c = (tid - r0 * VPR) * C::VE;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int gr = (TOT % C::NT != 0 && tid + v * C::NT >= TOT) ? -1 : sRow[r0 + v * (C::NT / VPR)];
            voff[v] = gr >= 0 ? (int)(((int64_t)(gr - base_row) * ld + c) * (int64_t)sizeof(T)) : none;
        }
    }
    // A whole K-block (k0 + BK <= K) through a buffer resource, each piece at
    // its precomputed row offset (a VGPR) plus the K position (a scalar).
    __device__ __forceinline__ void load_buf_off(__amdgpu_buffer_rsrc_t rs, const int (&voff)[NV], int k0,
                                                 int tid) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            if (TOT % C::NT != 0 && tid + v * C::NT >= TOT) break;
            const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, voff[v], k0 * (int)sizeof(T), 0);
            reg[v] = __builtin_bit_cast(uint4, x);
        }
    }
    // A whole K-block (k0 + BK <= K) of rows row0 .. row0 + ROWS - 1, those at
    // or past nrows read as row 0 (they only feed outputs never stored):
    // unconditional loads, no row table, no branch.
    __device__ __forceinline__ void load_full(const T* __restrict__ base, int64_t ld, int row0, int nrows, int k0,
                                              int tid) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int idx = tid + v * C::NT;
            if (TOT % C::NT != 0 && idx >= TOT) break;
            const int r = idx / VPR;
            const int gr = row0 + r;
            reg[v] = *(const uint4*)(base + (int64_t)(gr < nrows ? gr : 0) * ld + k0 + (idx - r * VPR) * C::VE);
        }
    }
    // Rows row0 .. row0 + ROWS - 1 of the source, those at or past nrows read
    // as row 0 (they only feed outputs that are never stored); no row table.
    __device__ __forceinline__ void load_direct(const T* __restrict__ base, int64_t ld, int row0, int nrows,
                                                int k0, int K, int tid) {
        if (k0 + C::BK <= K) {
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int idx = tid + v * C::NT;
                if (TOT % C::NT != 0 && idx >= TOT) break;
                const int r = idx / VPR;
                const int k = k0 + (idx - r * VPR) * C::VE;
                const int gr = row0 + r;
                reg[v] = *(const uint4*)(base + (int64_t)(gr < nrows ? gr : 0) * ld + k);
            }
            return;
        }
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int idx = tid + v * C::NT;
            if (TOT % C::NT != 0 && idx >= TOT) break;
            const int r = idx / VPR;
            const int k = k0 + (idx - r * VPR) * C::VE;
            const int gr = row0 + r;
            union { uint4 u; T e[C::VE]; } tmp;
#pragma unroll
            for (int e = 0; e < C::VE; ++e)
                tmp.e[e] = (gr < nrows && k + e < K) ? base[(int64_t)gr * ld + k + e] : (T)0;
            reg[v] = tmp.u;
        }
    }
    // the K-extension operand: rows whose sId is u; the others read row 0,
    // and are zeroed here (MASK) or by store_masked.  Masking at the load
    // made the compiler wait for each load before issuing the next; the GEMM
    // over W stored [d_in, d_out] keeps it (its 256 x 256 tile spills more
    // with the mask at the store).
    template <bool MASK>
    __device__ __forceinline__ void load_masked(const T* __restrict__ base, int64_t ld, const int* sRow,
                                                const int* sId, int u, int k0, int tid) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int idx = tid + v * C::NT;
            if (TOT % C::NT != 0 && idx >= TOT) break;
            const int r = idx / VPR;
            const int k = k0 + (idx - r * VPR) * C::VE;
            const bool ok = sId[r] == u;   // implies sRow[r] >= 0
            const uint4 val = *(const uint4*)(base + (int64_t)(ok ? sRow[r] : 0) * ld + k);
            reg[v] = (!MASK || ok) ? val : uint4{0u, 0u, 0u, 0u};
        }
    }
    // store, rows whose sId differs from u as zeros
    __device__ __forceinline__ void store_masked(T* s, const int* sId, int u, int tid) const {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int idx = tid + v * C::NT;
            if (TOT % C::NT != 0 && idx >= TOT) break;
            const int r = idx / VPR;
            const int c = (idx - r * VPR) * C::VE;
            *(uint4*)(s + r * C::LDK + c) = sId[r] == u ? reg[v] : uint4{0u, 0u, 0u, 0u};
        }
    }
    __device__ __forceinline__ void store(T* s, int tid) const {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int idx = tid + v * C::NT;
            if (TOT % C::NT != 0 && idx >= TOT) break;
            const int r = idx / VPR;
            const int c = (idx - r * VPR) * C::VE;
            *(uint4*)(s + r * C::LDK + c) = reg[v];
        }
    }
};

// The B operand of one K-block, staged into LDS as [n][k]; one register set
// serves two sources:
//   rows:  K-contiguous rows n (W stored [d_out, d_in]),
//   trans: row-major [K][N] rows k (W stored [d_in, d_out], or an adapter's
//          B block [r, d_out] for the K-extension steps), transposed on the
//          way into LDS.
template <class C>
struct BLoader {
    using T = typename C::T;
    static constexpr int VE = C::VE;
    static constexpr int R_VPR = C::BK / VE;        // rows: vectors per row
    static constexpr int T_VPR = C::BN / VE;        // trans: vectors per k-row
    static constexpr int TOT = C::BN * C::BK / VE;  // same count for both
    static constexpr int NV = (TOT + C::NT - 1) / C::NT;
    uint4 reg[NV];

    __device__ __forceinline__ void load_rows(const T* __restrict__ base, int64_t ld, const int* sRow,
                                              int k0, int K, int tid) {
        if (k0 + C::BK <= K) {
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int idx = tid + v * C::NT;
                if (TOT % C::NT != 0 && idx >= TOT) break;
                const int r = idx / R_VPR;
                const int k = k0 + (idx - r * R_VPR) * VE;
                // a column past the end reads row 0; its outputs are never stored
                const int gr = sRow[r];
                reg[v] = *(const uint4*)(base + (int64_t)(gr >= 0 ? gr : 0) * ld + k);
            }
            return;
        }
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int idx = tid + v * C::NT;
            if (TOT % C::NT != 0 && idx >= TOT) break;
            const int r = idx / R_VPR;
            const int k = k0 + (idx - r * R_VPR) * VE;
            const int gr = sRow[r];
            union { uint4 u; T e[VE]; } tmp;
#pragma unroll
            for (int e = 0; e < VE; ++e)
                tmp.e[e] = (gr >= 0 && k + e < K) ? base[(int64_t)gr * ld + k + e] : (T)0;
            reg[v] = tmp.u;
        }
    }
    // k-row kr of the block reads source row j0 + (kr % kwrap), valid below kmax
    __device__ __forceinline__ void load_trans(const T* __restrict__ base, int64_t ld, int j0, int kwrap,
                                               int kmax, int n0, int N, bool vec, int tid) {
        if (vec && n0 + C::BN <= N) {
            // all columns in range: a row at or past kmax reads row j0 (a valid row
            // of the same matrix); the A side is exactly zero at those k (x past
            // d_in, t_ext past the rank), so it adds nothing
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int idx = tid + v * C::NT;
                if (TOT % C::NT != 0 && idx >= TOT) break;
                const int kr = idx / T_VPR;
                const int k = j0 + kr % kwrap;
                const int n = n0 + (idx - kr * T_VPR) * VE;
                reg[v] = *(const uint4*)(base + (int64_t)(k < kmax ? k : j0) * ld + n);
            }
            return;
        }
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int idx = tid + v * C::NT;
            if (TOT % C::NT != 0 && idx >= TOT) break;
            const int kr = idx / T_VPR;
            const int k = j0 + kr % kwrap;
            const int n = n0 + (idx - kr * T_VPR) * VE;
            if (vec && k < kmax && n + VE <= N) {
                reg[v] = *(const uint4*)(base + (int64_t)k * ld + n);
            } else {
                union { uint4 u; T e[VE]; } tmp;
#pragma unroll
                for (int e = 0; e < VE; ++e)
                    tmp.e[e] = (k < kmax && n + e < N) ? base[(int64_t)k * ld + n + e] : (T)0;
                reg[v] = tmp.u;
            }
        }
    }
    // bf16 transposed pieces in pairs of k-rows: piece idx owns k-rows 2p and
    // 2p+1 of one column vector (pair_piece gives p and the vector), so the
    // two rows' values of a column are written to LDS as one 32-bit word.
    // reg[2v] holds row 2p, reg[2v+1] row 2p+1.
    static constexpr int PAIRS = C::BK / 2;
    static constexpr int P_TOT = PAIRS * T_VPR;
    static constexpr int P_NV = (P_TOT + C::NT - 1) / C::NT;
    static_assert(sizeof(T) != 2 || 2 * P_NV == NV, "pair pieces use the same registers");
    // Lanes in groups of PF take consecutive pairs of one column vector and
    // the groups step along the columns, so that a wave's loads cover whole
    // 128-byte row pieces (8 column vectors of a row) instead of 16 bytes
    // of 32 rows; the LDS stores then meet 4-way bank conflicts.  PF = 8 was
    // measured against 16 and 32 (the pairs of one vector in a half-wave).
    static constexpr int PF = 8 < PAIRS ? 8 : PAIRS;
    static_assert(PAIRS % PF == 0, "pairs per lane group");
    __device__ __forceinline__ static void pair_piece(int idx, int& p, int& cv) {
        const int lo = idx % PF, rest = idx / PF;
        cv = rest % T_VPR;
        p = lo + PF * (rest / T_VPR);
    }
    // SPLIT: whole vectors (the usual case) go through a branch-free loop of
    // their own.  A bounds branch around each load made the compiler wait for
    // each load before issuing the next; the K-extension blocks of the GEMM
    // over W stored [d_out, d_in] take SPLIT.  The GEMM over W stored
    // [d_in, d_out] keeps the per-piece form: its 256 x 256 tile spills more
    // with SPLIT.
    template <bool SPLIT = false>
    __device__ __forceinline__ void load_trans_pairs(const T* __restrict__ base, int64_t ld, int j0, int kwrap,
                                                     int kmax, int n0, int N, bool vec, int tid) {
        const bool full = vec && n0 + C::BN <= N;
        if (SPLIT && full) {
#pragma unroll
            for (int v = 0; v < P_NV; ++v) {
                const int idx = tid + v * C::NT;
                if (P_TOT % C::NT != 0 && idx >= P_TOT) break;
                int p, cv;
                pair_piece(idx, p, cv);
                const int n = n0 + cv * VE;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int k = j0 + (2 * p + h) % kwrap;
                    // a row at or past kmax reads row j0; the A side is exactly zero there
                    reg[2 * v + h] = *(const uint4*)(base + (int64_t)(k < kmax ? k : j0) * ld + n);
                }
            }
            return;
        }
#pragma unroll
        for (int v = 0; v < P_NV; ++v) {
            const int idx = tid + v * C::NT;
            if (P_TOT % C::NT != 0 && idx >= P_TOT) break;
            int p, cv;
            pair_piece(idx, p, cv);
            const int n = n0 + cv * VE;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = j0 + (2 * p + h) % kwrap;
                if (full) {
                    reg[2 * v + h] = *(const uint4*)(base + (int64_t)(k < kmax ? k : j0) * ld + n);
                } else {
                    union { uint4 u; T e[VE]; } tmp;
#pragma unroll
                    for (int e = 0; e < VE; ++e)
                        tmp.e[e] = (k < kmax && n + e < N) ? base[(int64_t)k * ld + n + e] : (T)0;
                    reg[2 * v + h] = tmp.u;
                }
            }
        }
    }
    __device__ __forceinline__ void store_trans_pairs(T* s, int tid) const {
#pragma unroll
        for (int v = 0; v < P_NV; ++v) {
            const int idx = tid + v * C::NT;
            if (P_TOT % C::NT != 0 && idx >= P_TOT) break;
            int p, cv;
            pair_piece(idx, p, cv);
            const int c = cv * VE;
            union { uint4 u; unsigned short e[VE]; } r0, r1;
            r0.u = reg[2 * v];
            r1.u = reg[2 * v + 1];
#pragma unroll
            for (int e = 0; e < VE; ++e)
                *(unsigned int*)(s + (c + e) * C::LDK + 2 * p) = (unsigned int)r0.e[e] | ((unsigned int)r1.e[e] << 16);
        }
    }
    __device__ __forceinline__ void store_rows(T* s, int tid) const {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int idx = tid + v * C::NT;
            if (TOT % C::NT != 0 && idx >= TOT) break;
            const int r = idx / R_VPR;
            const int c = (idx - r * R_VPR) * VE;
            *(uint4*)(s + r * C::LDK + c) = reg[v];
        }
    }
    __device__ __forceinline__ void store_trans(T* s, int tid) const {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int idx = tid + v * C::NT;
            if (TOT % C::NT != 0 && idx >= TOT) break;
            const int kr = idx / T_VPR;
            const int c = (idx - kr * T_VPR) * VE;
            union { uint4 u; T e[VE]; } tmp;
            tmp.u = reg[v];
#pragma unroll
            for (int e = 0; e < VE; ++e) s[(c + e) * C::LDK + kr] = tmp.e[e];
        }
    }
};

// Row-major [K][N] source -> LDS [n][k] (transposed on the way in).  bf16
// pieces come in pairs of k-rows: piece p = idx % (BK/2) holds k-rows 2p and
// 2p+1 of column vector idx / (BK/2), so each column's two values go to LDS
// as one 32-bit word and a wave fills one LDS row with consecutive words (no
// bank conflicts).  fp32 pieces are single k-rows.
template <class C, int COLS>
struct TransLoader {
    using T = typename C::T;
    static constexpr bool PAIRS = sizeof(T) == 2;
    static constexpr int VPR = COLS / C::VE;
    static constexpr int KR = PAIRS ? C::BK / 2 : C::BK;   // pieces per column vector
    static constexpr int TOT = KR * VPR;
    static constexpr int NP = (TOT + C::NT - 1) / C::NT;
    static constexpr int NV = PAIRS ? 2 * NP : NP;
    static_assert(COLS % C::VE == 0, "tile width not a multiple of the vector width");
    uint4 reg[NV];

    __device__ __forceinline__ uint4 piece(const T* __restrict__ base, int64_t ld, int k, int K, int n, int N,
                                           bool vec) const {
        if (vec && k < K && n + C::VE <= N) return *(const uint4*)(base + (int64_t)k * ld + n);
        union { uint4 u; T e[C::VE]; } tmp;
#pragma unroll
        for (int e = 0; e < C::VE; ++e) tmp.e[e] = (k < K && n + e < N) ? base[(int64_t)k * ld + n + e] : (T)0;
        return tmp.u;
    }
    __device__ __forceinline__ void load(const T* __restrict__ base, int64_t ld, int k0, int K,
                                         int n0, int N, bool vec, int tid) {
#pragma unroll
        for (int v = 0; v < NP; ++v) {
            const int idx = tid + v * C::NT;
            if (TOT % C::NT != 0 && idx >= TOT) break;
            const int kp = idx % KR;
            const int n = n0 + (idx / KR) * C::VE;
            if constexpr (PAIRS) {
                reg[2 * v] = piece(base, ld, k0 + 2 * kp, K, n, N, vec);
                reg[2 * v + 1] = piece(base, ld, k0 + 2 * kp + 1, K, n, N, vec);
            } else {
                reg[v] = piece(base, ld, k0 + kp, K, n, N, vec);
            }
        }
    }
    __device__ __forceinline__ void store(T* s, int tid) const {
#pragma unroll
        for (int v = 0; v < NP; ++v) {
            const int idx = tid + v * C::NT;
            if (TOT % C::NT != 0 && idx >= TOT) break;
            const int kp = idx % KR;
            const int c = (idx / KR) * C::VE;
            if constexpr (PAIRS) {
                union { uint4 u; unsigned short e[8]; } r0, r1;
                r0.u = reg[2 * v];
                r1.u = reg[2 * v + 1];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    *(unsigned int*)(s + (c + e) * C::LDK + 2 * kp) =
                        (unsigned int)r0.e[e] | ((unsigned int)r1.e[e] << 16);
            } else {
                union { uint4 u; T e[C::VE]; } tmp;
                tmp.u = reg[v];
#pragma unroll
                for (int e = 0; e < C::VE; ++e) s[(c + e) * C::LDK + kp] = tmp.e[e];
            }
        }
    }
};


// ---------------------------------------------------------------------------
// Fused layer GEMM
// ---------------------------------------------------------------------------

struct GemmDev {
    const void* x;
    int64_t ldx;
    const void* W;
    int64_t ldw;
    const int32_t* ids;
    int32_t n;
    const float* t;       // fp32 t (skinny kernel's epilogue)
    int64_t ldt;
    const void* t_ext;    // K-extension operand (tiled kernel), or null
    int64_t lde;
    void* y;
    int64_t ldy;
    int32_t tiles_m;
    int32_t tiles_n;
    // tiled kernel: tile row m is row perm[m] of x, ids, t, t_ext and y
    // (null: row m); x holds x_rows addressable rows
    const int32_t* perm;
    int32_t x_rows;
    // 4-bit W (k_layer_gemm<..., Q4>): W is bytes [d_out][ldw], the scale of
    // inputs 128 g .. 128 g + 127 of output n is wscale[n * lds + g]
    const float* wscale;
    int64_t lds;
    // split K (part non-null): workgroup b takes K slice b / (tiles_m *
    // tiles_n) of kslice K-blocks and writes its fp32 partial product
    // (base only) to part[slice][tile row][ldp]; a finish launch adds the
    // slices and the adapter term
    float* part;
    int64_t ldp;
    int32_t kslice;
};

// Eight signed 4-bit values (element e in bits 4e .. 4e+3) times `sc`, each
// product rounded once to bf16 (the conversion instruction takes two at a time).
__device__ __forceinline__ uint4 widen8_q4_scaled(uint32_t w, float sc) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    uint32_t o[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const int q0 = ((int)(w << (28 - 8 * h))) >> 28;
        const int q1 = ((int)(w << (24 - 8 * h))) >> 28;
        const bf16x2_t v = {(__bf16)((float)q0 * sc), (__bf16)((float)q1 * sc)};
        o[h] = __builtin_bit_cast(uint32_t, v);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// 4-bit W rows of a tile ([d_out, d_in] storage): one BK-deep block of BN
// rows is BN x BK/2 bytes.  A thread takes QB bytes (2 QB consecutive
// inputs) of one row through a buffer resource over the tile's rows (rows
// past the range read as 0), and that row's scale of the block's 128-input
// group; it stores them to the LDS tile widened, bf16(q * scale).
template <class C>
struct Q4WLoader {
    static constexpr int RB = C::BK / 2;              // bytes of a row per block
    static constexpr int QB = C::BN * RB / C::NT;     // bytes per thread
    static constexpr int PPR = RB / QB;               // pieces per row
    static_assert((QB == 8 || QB == 16) && PPR * QB == RB && C::NT % PPR == 0 && 128 % C::BK == 0,
                  "4-bit pieces of 8 or 16 bytes, one scale group per block");
    uint32_t q[QB / 4];
    float sc;
    __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t rs, int64_t ldq, const float* srow, int k0,
                                             int tid) {
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
        const int voff = (int)((int64_t)(tid / PPR) * ldq) + (tid % PPR) * QB;
        if constexpr (QB == 16) {
            const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, k0 / 2, 0);
            q[0] = v.x;
            q[1] = v.y;
            q[2] = v.z;
            q[3] = v.w;
        } else {
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, k0 / 2, 0);
            q[0] = v.x;
            q[1] = v.y;
        }
        sc = srow[k0 >> 7];
    }
    __device__ __forceinline__ void store(bf16* s, int tid) const {
        bf16* d = s + (tid / PPR) * C::LDK + (tid % PPR) * QB * 2;
#pragma unroll
        for (int h = 0; h < QB / 4; ++h) *(uint4*)(d + h * 8) = widen8_q4_scaled(q[h], sc);
    }
};

// VE consecutive outputs of one row, rounded once; 8-, 16- or 32-byte
// pieces where the row is whole and aligned, else one element at a time.
template <typename TY, int VE>
__device__ __forceinline__ void store_row_piece(TY* p, const float* v, int valid, bool vec) {
    if (vec && valid >= VE) {
        union { TY e[VE]; uint2 h[VE * sizeof(TY) / 8]; } o;
#pragma unroll
        for (int e = 0; e < VE; ++e) o.e[e] = from_f32<TY>(v[e]);
        if constexpr (VE * sizeof(TY) == 8) {
            *(uint2*)p = o.h[0];
        } else {
#pragma unroll
            for (int h = 0; h < (int)(VE * sizeof(TY) / 16); ++h)
                ((uint4*)p)[h] = make_uint4(o.h[2 * h].x, o.h[2 * h].y, o.h[2 * h + 1].x, o.h[2 * h + 1].y);
        }
    } else {
        for (int e = 0; e < VE && e < valid; ++e) p[e] = from_f32<TY>(v[e]);
    }
}

// Row-wise expand epilogue, for tiles whose rows carry many different
// adapters (decode-style batches in arrival order), where the K-extension
// would add one block of MFMA work per distinct adapter:
//     y[m, n] = acc[m, n] + s_a * sum_j t[m, j] * B_a[j, n],   a = id of row m.
// Each wave stages one block-row of its accumulators (BLK x WTN fp32) in
// its own slice of LDS, then reads it back one output row piece per lane
// (VE columns, a 16-byte piece of a B row) and streams the r rows of B_a
// for that piece, RC rank rows at a time.  The tile's LDS stages must no
// longer be in use when this starts.
template <class C, typename TY>
__device__ __forceinline__ void gather_epilogue(const PoolDev& P, const GemmDev& g, Acc<C>& acc,
                                                float* sw_all, const RowRec* sRec, const int* sRow, int n0,
                                                int wm, int wn, int wave, int lane) {
    using T = typename C::T;
    constexpr int VE = C::VE;
    constexpr int LPR = C::WTN / VE;   // lanes per output row
    constexpr int RPI = 64 / LPR;      // rows per pass of the wave (lanes past BLK rows idle)
    constexpr int LDW = C::WTN + 4;    // fp32 pitch of a staged row
    // rank rows requested together: all 16 of a rank-16 adapter where the
    // tile's LDS already limits a CU to two workgroups and the accumulator is
    // small (registers to spare), else 8 so that the epilogue does not raise
    // the kernel's register count
    constexpr int RC =
        (2 * C::STAGE * (int)sizeof(T) > 64 * 1024 && C::FM * C::FN * C::M::NACC <= 64) ? 16 : 8;
    constexpr int PASSES = (C::BLK + RPI - 1) / RPI;
    static_assert(C::WTN % VE == 0 && 64 % LPR == 0 && (C::BLK % RPI == 0 || RPI % C::BLK == 0),
                  "epilogue lane map");
    static_assert(C::WM * C::WN * C::BLK * LDW * 4 <= 2 * C::STAGE * (int)sizeof(T), "epilogue staging");
    const int N = P.d_out;
    const int lr = lane / LPR;
    const int cc = (lane % LPR) * VE;
    const int col = n0 + wn * C::WTN + cc;
    const int valid_c = N - col;
    const bool full = valid_c >= VE;
    const bool vec_y = ((g.ldy * (int64_t)sizeof(TY)) & 15) == 0;
    TY* Y = (TY*)g.y;
    const int lc = lane % C::BLK;

    if constexpr (PASSES == 1 && RC == 16) {
        // rank rows [j0, j0 + RC) of one row piece: B pieces and t values requested
        auto request = [&](uint4 (&bv)[RC], float (&tv)[RC], const T* Bu, const float* trow, int r, int j0)
            __attribute__((always_inline)) {
#pragma unroll
            for (int q = 0; q < RC; ++q) {
                const int jj = j0 + q;
                const T* bj = Bu + (int64_t)jj * N;
                tv[q] = (jj < r) ? trow[jj] : 0.f;
                if (jj < r && full && P.vec_b) {
                    bv[q] = *(const uint4*)bj;
                } else {
                    union { uint4 u; T e[VE]; } w;
#pragma unroll
                    for (int e = 0; e < VE; ++e) w.e[e] = (jj < r && e < valid_c) ? bj[e] : (T)0;
                    bv[q] = w.u;
                }
            }
        };
        auto accumulate = [&](float (&ex)[VE], const uint4 (&bv)[RC], const float (&tv)[RC])
            __attribute__((always_inline)) {
#pragma unroll
            for (int q = 0; q < RC; ++q) {
                union { uint4 u; T e[VE]; } w;
                w.u = bv[q];
#pragma unroll
                for (int e = 0; e < VE; ++e) ex[e] += tv[q] * to_f32(w.e[e]);
            }
        };
        auto load_staged = [&](float (&v)[VE], const float* src) __attribute__((always_inline)) {
#pragma unroll
            for (int e = 0; e < VE; e += 4) {
                const float4 b4 = *(const float4*)(src + e);
                v[e] = b4.x;
                v[e + 1] = b4.y;
                v[e + 2] = b4.z;
                v[e + 3] = b4.w;
            }
        };

        {
            // Each lane's FM row pieces are known before the accumulators are
            // staged, so the first RC rank rows of all of them are requested in
            // one round, then the whole wave tile is staged.
            static_assert(C::WM * C::WN * C::WTM * LDW * 4 <= 2 * C::STAGE * (int)sizeof(T), "wave tile staging");
            float* sw = sw_all + wave * C::WTM * LDW;
            int rowp[C::FM];
            RowRec recp[C::FM];
            uint4 bv[C::FM][RC];
            float tv[C::FM][RC];
#pragma unroll
            for (int i = 0; i < C::FM; ++i) {
                const int tr = wm * C::WTM + i * C::BLK + lr;
                rowp[i] = (lr < C::BLK && valid_c > 0) ? sRow[tr] : -1;
                recp[i] = rowp[i] >= 0 ? sRec[tr] : RowRec{0, 0, 0.f};
                request(bv[i], tv[i], (const T*)P.B + recp[i].b_off + col,
                        g.t + (int64_t)(rowp[i] >= 0 ? rowp[i] : 0) * g.ldt, recp[i].rank, 0);
            }
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
#pragma unroll
                for (int j = 0; j < C::FN; ++j)
#pragma unroll
                    for (int q = 0; q < C::M::NACC; ++q)
                        sw[(i * C::BLK + C::M::row(lane, q)) * LDW + j * C::BLK + lc] = acc.v[i][j][q];
            __syncthreads();
#pragma unroll
            for (int i = 0; i < C::FM; ++i) {
                if (rowp[i] < 0) continue;
                float v[VE], ex[VE];
                load_staged(v, sw + (i * C::BLK + lr) * LDW + cc);
#pragma unroll
                for (int e = 0; e < VE; ++e) ex[e] = 0.f;
                accumulate(ex, bv[i], tv[i]);
                const int r = recp[i].rank;
                const T* Bu = (const T*)P.B + recp[i].b_off + col;
                const float* trow = g.t + (int64_t)rowp[i] * g.ldt;
                for (int j0 = RC; j0 < r; j0 += RC) {
                    uint4 bw[RC];
                    float tw[RC];
                    request(bw, tw, Bu, trow, r, j0);
                    accumulate(ex, bw, tw);
                }
#pragma unroll
                for (int e = 0; e < VE; ++e) v[e] += recp[i].scale * ex[e];
                store_row_piece<TY, VE>(Y + (int64_t)rowp[i] * g.ldy + col, v, valid_c, vec_y);
            }
        }
    } else {
        float* sw = sw_all + wave * C::BLK * LDW;
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
#pragma unroll
                for (int q = 0; q < C::M::NACC; ++q) sw[C::M::row(lane, q) * LDW + j * C::BLK + lc] = acc.v[i][j][q];
            __syncthreads();
#pragma unroll 1
            for (int it = 0; it < PASSES; ++it) {
                const int rl = it * RPI + lr;
                const int tr = wm * C::WTM + i * C::BLK + rl;   // row within the tile
                const int row = (rl < C::BLK) ? sRow[tr] : -1;    // its row of t and y
                if (row < 0 || valid_c <= 0) continue;
                float v[VE];
#pragma unroll
                for (int e = 0; e < VE; e += 4) {
                    const float4 b4 = *(const float4*)(sw + rl * LDW + cc + e);
                    v[e] = b4.x;
                    v[e + 1] = b4.y;
                    v[e + 2] = b4.z;
                    v[e + 3] = b4.w;
                }
                const RowRec rec = sRec[tr];
                if (rec.rank > 0) {
                    const int r = rec.rank;
                    const T* Bu = (const T*)P.B + rec.b_off + col;
                    const float* trow = g.t + (int64_t)row * g.ldt;
                    float ex[VE];
#pragma unroll
                    for (int e = 0; e < VE; ++e) ex[e] = 0.f;
                    for (int j0 = 0; j0 < r; j0 += RC) {
                        uint4 bv[RC];
                        float tv[RC];
#pragma unroll
                        for (int q = 0; q < RC; ++q) {
                            const int jj = j0 + q;
                            const T* bj = Bu + (int64_t)jj * N;
                            tv[q] = (jj < r) ? trow[jj] : 0.f;
                            if (jj < r && full && P.vec_b) {
                                bv[q] = *(const uint4*)bj;
                            } else {
                                union { uint4 u; T e[VE]; } w;
#pragma unroll
                                for (int e = 0; e < VE; ++e) w.e[e] = (jj < r && e < valid_c) ? bj[e] : (T)0;
                                bv[q] = w.u;
                            }
                        }
#pragma unroll
                        for (int q = 0; q < RC; ++q) {
                            union { uint4 u; T e[VE]; } w;
                            w.u = bv[q];
#pragma unroll
                            for (int e = 0; e < VE; ++e) ex[e] += tv[q] * to_f32(w.e[e]);
                        }
                    }
#pragma unroll
                    for (int e = 0; e < VE; ++e) v[e] += rec.scale * ex[e];
                }
                store_row_piece<TY, VE>(Y + (int64_t)row * g.ldy + col, v, valid_c, vec_y);
            }
            __syncthreads();
        }
    }
}

// The LoRA expand rides on the same K loop: after the d_in/BK blocks of
// x W come, for every distinct adapter u among the tile's rows (in the
// order they first appear down the rows), ceil(r_u / KH) blocks whose A
// side is t_ext (s_u * t split into bf16 hi | lo halves, written by the
// shrink; rows of other adapters masked to 0)
// and whose B side is B_u[j][n0:n0+BN] (each rank row twice for bf16, to
// meet the hi and the lo half).  y is rounded once at the end.
// Q4 (with OUT_IN, bf16 x and adapters): W is 4-bit, widened into the LDS
// tile as bf16(q * scale) (Q4WLoader); d_in is a multiple of 128.
template <class C, typename TY, bool OUT_IN, bool Q4 = false>
__global__ __launch_bounds__(C::NT) void k_layer_gemm(PoolDev P, GemmDev g) {
    using T = typename C::T;
    static_assert(!Q4 || (OUT_IN && sizeof(T) == 2), "4-bit W: bf16, stored [d_out, d_in]");
    // K-extension only where a K-block is one t_ext block; other tile shapes
    // always take the row-wise epilogue
    constexpr bool EXT = C::BK == ext_block_cols(sizeof(T)) && C::KH == EXT_RANKS;
    __shared__ __attribute__((aligned(16))) T smem[2 * C::STAGE];
    __shared__ int sRowA[C::BM];
    __shared__ int sRowB[OUT_IN ? C::BN : 1];
    __shared__ __attribute__((aligned(16))) int sId[C::BM];
    __shared__ int sExt[2 * C::BM];   // (u << 1) | block, in order
    __shared__ int sWaveSum[(C::BM + 63) / 64];
    __shared__ int sNExt;
    __shared__ int sRuns;
    __shared__ int sValid;
    __shared__ RowRec sRec[C::BM];   // per tile row: B offset, rank, scale (row-wise epilogue)
    static_assert(C::BM <= C::NT, "one tile row per thread in the set-up");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / C::WN;
    const int wn = wave - wm * C::WN;

    // XCD-aware order: consecutive workgroups land on different XCDs, so give
    // each XCD a contiguous run of tiles, then raster in groups of 8 row-tiles.
    int b = blockIdx.x;
    int ks = 0;
    const int T_all = g.part ? g.tiles_m * g.tiles_n : (int)gridDim.x;
    if (g.part) {
        ks = b / T_all;
        b -= ks * T_all;
    }
    const int T8 = T_all & ~7;
    if (b < T8) b = (b & 7) * (T8 >> 3) + (b >> 3);
    constexpr int GM = 8;
    const int per_group = GM * g.tiles_n;
    const int grp = b / per_group;
    const int first_m = grp * GM;
    const int gsz = min(GM, g.tiles_m - first_m);
    const int in_grp = b - grp * per_group;
    const int tm = first_m + in_grp % gsz;
    const int tn = in_grp / gsz;
    const int m0 = tm * C::BM;
    const int n0 = tn * C::BN;
    const int K = P.d_in;
    const int N = P.d_out;

    if (tid < C::BM) {
        const int row = m0 + tid;
        // a perm entry outside x's rows (a malformed descriptor) skips the row
        const int pr = row < g.n ? (g.perm ? g.perm[row] : row) : -1;
        const int src = (pr >= 0 && pr < g.x_rows) ? pr : -1;
        int id = INT_MAX;
        if (src >= 0) {
            const int a = g.ids[src];
            if (id_ok(a, P.n_adapters)) id = a;
            else if (a != -1 && tn == 0) flag_bad_id(P.err);
        }
        sRowA[tid] = src;
        sId[tid] = id;
        if (g.t || g.t_ext) {
            RowRec rec{0, 0, 0.f};
            if (id != INT_MAX) {
                rec.b_off = P.b_off[id];
                rec.rank = P.ranks[id];
                rec.scale = P.scales[id];
            }
            sRec[tid] = rec;
        }
    }
    if constexpr (OUT_IN)
        for (int r = tid; r < C::BN; r += C::NT) sRowB[r] = (n0 + r < N) ? n0 + r : -1;
    if (tid == 0) {
        sNExt = 0;
        sRuns = 0;
        sValid = 0;
    }
    __syncthreads();

    // Runs of one adapter id down the tile's rows (looking past a few
    // base-only rows) estimate its distinct adapters.  The K-extension costs
    // a block of MFMA work per adapter but reads each adapter's B once; the
    // row-wise epilogue reads B once per row.  Tiles whose runs average at
    // most two rows (decode-style rows in arrival order) take the epilogue.
    bool gather = false;
    if (g.t) {
        if (tid < C::BM) {
            const int v = sId[tid];
            if (v != INT_MAX) {
                int prev = INT_MAX;
                for (int k = tid - 1; k >= 0 && k >= tid - 8; --k)
                    if (sId[k] != INT_MAX) {
                        prev = sId[k];
                        break;
                    }
                atomicAdd(&sValid, 1);
                if (prev != v) atomicAdd(&sRuns, 1);
            }
        }
        __syncthreads();
        const int per_adapter = (P.r_max + EXT_RANKS - 1) / EXT_RANKS;
        gather = !EXT || !g.t_ext || (sRuns * per_adapter > 2 && 2 * sRuns >= sValid);
    }

    // K-extension blocks: one set per distinct adapter of the tile, in the
    // order in which the adapters first appear down its rows.  The first row
    // of each run of one id looks back for an earlier run of that id; a run
    // that finds none brings its adapter's blocks, placed by a prefix sum
    // over the rows.
    if (EXT && g.t_ext && !gather) {
        const int v = tid < C::BM ? sId[tid] : INT_MAX;
        int nb = 0;
        if (v != INT_MAX && (tid == 0 || sId[tid - 1] != v)) {
            bool seen = false;
            for (int k = 0; k < tid; k += 4) {
                const int4 q = *(const int4*)(sId + k);
                seen |= (q.x == v) | (k + 1 < tid && q.y == v) | (k + 2 < tid && q.z == v) |
                        (k + 3 < tid && q.w == v);
            }
            if (!seen) nb = (sRec[tid].rank + C::KH - 1) / C::KH;
        }
        // exclusive prefix sum of nb over the tile's rows
        int incl = nb;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(incl, d, 64);
            if (lane >= d) incl += o;
        }
        if (lane == 63 && wave < (C::BM + 63) / 64) sWaveSum[wave] = incl;
        __syncthreads();
        int before = incl - nb;
        for (int w = 0; w < wave && w < (C::BM + 63) / 64; ++w) before += sWaveSum[w];
        for (int e = 0; e < nb; ++e) sExt[before + e] = (v << 1) | e;
        if (tid == C::BM - 1) sNExt = before + nb;
        __syncthreads();
    }
    const int nk_all = (K + C::BK - 1) / C::BK;
    // this workgroup's K-blocks (all of them without a K split)
    const int kbeg = g.part ? ks * g.kslice : 0;
    const int nk = g.part ? min(nk_all, kbeg + g.kslice) : nk_all;
    const int total = nk + sNExt;

    Acc<C> acc;
    acc.zero();
    const T* X = (const T*)g.x;
    const T* Wp = (const T*)g.W;
    const T* TE = (const T*)g.t_ext;
    RowLoader<C, C::BM> la;
    BLoader<C> lb;
    // W rows (OUT_IN) share the B register set's shape; 4-bit rows their own
    using WLoader = typename std::conditional<Q4, Q4WLoader<C>, RowLoader<C, C::BN>>::type;
    WLoader lw;
    auto load_main = [&](int s) {
        if (g.perm) la.load(X, g.ldx, sRowA, s * C::BK, K, tid);
        else la.load_direct(X, g.ldx, m0, g.n, s * C::BK, K, tid);
        if constexpr (Q4) {
            // not reached: a 4-bit K is whole blocks (the loop below takes them all)
        } else if constexpr (OUT_IN) {
            lw.load_direct(Wp, g.ldw, n0, N, s * C::BK, K, tid);
        } else if constexpr (sizeof(T) == 2) {
            lb.load_trans_pairs(Wp, g.ldw, s * C::BK, C::BK, K, n0, N, true, tid);
        } else {
            lb.load_trans(Wp, g.ldw, s * C::BK, C::BK, K, n0, N, true, tid);
        }
    };
    constexpr bool PAIRS = sizeof(T) == 2;
    auto load_ext = [&](int s) {
        const int code = sExt[s];
        const int u = code >> 1;
        const int e = code & 1;
        la.template load_masked<!OUT_IN>(TE, g.lde, sRowA, sId, u, e * C::BK, tid);
        if constexpr (PAIRS)
            lb.template load_trans_pairs<OUT_IN>((const T*)P.B + P.b_off[u], N, e * C::KH, C::KH, P.ranks[u], n0,
                                                 N, P.vec_b, tid);
        else
            lb.load_trans((const T*)P.B + P.b_off[u], N, e * C::KH, C::KH, P.ranks[u], n0, N, P.vec_b, tid);
    };
    auto store_trans = [&](T* sB) {
        if constexpr (PAIRS) lb.store_trans_pairs(sB, tid);
        else lb.store_trans(sB, tid);
    };
    const int n_ext = total - nk;
    // x W over d_in, two LDS stages, next block prefetched into registers
    if constexpr (OUT_IN) {
        // whole K-blocks in a branch-free loop (both operands K-contiguous);
        // the last whole block and a ragged tail block after it
        const int nkf = min(K / C::BK, nk);
        // buffer resources over the tile's rows (raw, 16-byte pieces); their
        // fields are workgroup-uniform, said so with readfirstlane so that the
        // loads take the descriptor from scalar registers directly
        auto rsrc = [](const T* base, int rows, int64_t ld) {
            const uint64_t a = (uint64_t)base;
            const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
            const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
            const int bytes = __builtin_amdgcn_readfirstlane((int)((int64_t)rows * ld * (int64_t)sizeof(T)));
            return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, bytes,
                                                     0x00020000);
        };
        // x rows: relative to the tile's first row, or (rows gathered through
        // perm) to row 0 of x; a row of -1 reads past the range
        const int a_base = g.perm ? 0 : m0;
        const int a_rows = g.perm ? g.x_rows : max(0, min(C::BM, g.n - m0));
        const __amdgpu_buffer_rsrc_t rs_a = rsrc(X + (int64_t)a_base * g.ldx, a_rows, g.ldx);
        // W: the tile's rows (4-bit: bytes, a row of ldw bytes; the scale row
        // of this thread's W row, clamped into W's rows)
        const __amdgpu_buffer_rsrc_t rs_w =
            Q4 ? rsrc((const T*)((const uint8_t*)g.W + (int64_t)n0 * g.ldw), max(0, min(C::BN, N - n0)),
                      g.ldw / (int64_t)sizeof(T))
               : rsrc(Wp + (int64_t)n0 * g.ldw, max(0, min(C::BN, N - n0)), g.ldw);
        const float* srow = nullptr;
        if constexpr (Q4) srow = g.wscale + (int64_t)min(n0 + tid / Q4WLoader<C>::PPR, N - 1) * g.lds;
        int a_off[RowLoader<C, C::BM>::NV];
        la.row_offsets(sRowA, a_base, g.ldx, (int)((int64_t)a_rows * g.ldx * (int64_t)sizeof(T)), tid, a_off);
        auto load_w = [&](WLoader& l, int s) __attribute__((always_inline)) {
            if constexpr (Q4) l.load_buf(rs_w, g.ldw, srow, s * C::BK, tid);
            else l.load_buf(rs_w, g.ldw, s * C::BK, tid);
        };
        auto load_full = [&](int s) {
            la.load_buf_off(rs_a, a_off, s * C::BK, tid);
            load_w(lw, s);
        };
        auto step = [&](int kb) {
            T* sA = smem + (kb & 1) * C::STAGE;
            T* sB = sA + C::A_ELEMS;
            la.store(sA, tid);
            lw.store(sB, tid);
            __syncthreads();
            return sA;
        };
        int kb = kbeg;
        if constexpr (C::NT <= 256 || (C::BM + C::BN) * C::BK * (int)sizeof(T) <= 64 * C::NT) {
            // registers to spare (4 waves, or at most 64 staged bytes a
            // thread): two blocks in flight, in two register sets used
            // alternately (the loop is unrolled by two)
            RowLoader<C, C::BM> la2;
            WLoader lw2;
            auto load_full2 = [&](int s) {
                la2.load_buf_off(rs_a, a_off, s * C::BK, tid);
                load_w(lw2, s);
            };
            auto step2 = [&](int k) {
                T* sA = smem + (k & 1) * C::STAGE;
                la2.store(sA, tid);
                lw2.store(sA + C::A_ELEMS, tid);
                __syncthreads();
                return sA;
            };
            if (nkf - kb >= 2) {
                load_full(kb);
                load_full2(kb + 1);
                for (; kb + 3 < nkf; kb += 2) {
                    T* sA = step(kb);
                    load_full(kb + 2);
                    mma_block<C>(acc, sA, sA + C::A_ELEMS, wm, wn, lane);
                    sA = step2(kb + 1);
                    load_full2(kb + 3);
                    mma_block<C>(acc, sA, sA + C::A_ELEMS, wm, wn, lane);
                }
                // two whole blocks left in the two register sets
                T* sA = step(kb);
                if (kb + 2 < nk) load_main(kb + 2);
                mma_block<C>(acc, sA, sA + C::A_ELEMS, wm, wn, lane);
                ++kb;
                sA = step2(kb);
                mma_block<C>(acc, sA, sA + C::A_ELEMS, wm, wn, lane);
                ++kb;
            } else {
                if (kb < nkf) load_full(kb);
                else load_main(kb);
            }
        } else {
            if (kb < nkf) load_full(kb);
            else load_main(kb);
            for (; kb + 1 < nkf; ++kb) {
                T* sA = step(kb);
                load_full(kb + 1);
                mma_block<C>(acc, sA, sA + C::A_ELEMS, wm, wn, lane);
            }
        }
        for (; kb < nk; ++kb) {
            T* sA = step(kb);
            if (kb + 1 < nk) load_main(kb + 1);
            mma_block<C>(acc, sA, sA + C::A_ELEMS, wm, wn, lane);
        }
    } else {
        load_main(kbeg);
        for (int kb = kbeg; kb < nk; ++kb) {
            T* sA = smem + (kb & 1) * C::STAGE;
            T* sB = sA + C::A_ELEMS;
            la.store(sA, tid);
            store_trans(sB);
            __syncthreads();
            if (kb + 1 < nk) load_main(kb + 1);
            mma_block<C>(acc, sA, sB, wm, wn, lane);
        }
    }
    // the LoRA K-extension blocks, same pipeline (their first block is fetched
    // here; the stage it goes to was last read two blocks ago)
    if constexpr (EXT) {
        if (n_ext > 0) load_ext(0);
        for (int e = 0; e < n_ext; ++e) {
            const int kb = nk + e;
            T* sA = smem + (kb & 1) * C::STAGE;
            T* sB = sA + C::A_ELEMS;
            if constexpr (OUT_IN) la.store_masked(sA, sId, sExt[e] >> 1, tid);
            else la.store(sA, tid);
            store_trans(sB);
            __syncthreads();
            if (e + 1 < n_ext) load_ext(e + 1);
            mma_block<C>(acc, sA, sB, wm, wn, lane);
        }
    }

    if (g.part) {
        // this K slice's fp32 partial product, by tile row, for the finish
        float* pp = g.part + (int64_t)ks * g.n * g.ldp;
        const int lcp = lane % C::BLK;
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j) {
                const int col = n0 + wn * C::WTN + j * C::BLK + lcp;
#pragma unroll
                for (int q = 0; q < C::M::NACC; ++q) {
                    const int m = m0 + wm * C::WTM + i * C::BLK + C::M::row(lane, q);
                    if (m < g.n && col < N) pp[(int64_t)m * g.ldp + col] = acc.v[i][j][q];
                }
            }
        return;
    }
    if (gather) {
        __syncthreads();   // every wave is done with the LDS stages
        gather_epilogue<C, TY>(P, g, acc, (float*)smem, sRec, sRowA, n0, wm, wn, wave, lane);
        return;
    }

    TY* Y = (TY*)g.y;
    const int lc = lane % C::BLK;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            const int col = n0 + wn * C::WTN + j * C::BLK + lc;
#pragma unroll
            for (int q = 0; q < C::M::NACC; ++q) {
                const int row = sRowA[wm * C::WTM + i * C::BLK + C::M::row(lane, q)];
                if (row >= 0 && col < N) Y[(int64_t)row * g.ldy + col] = from_f32<TY>(acc.v[i][j][q]);
            }
        }
}

// Finish of a split-K launch: workgroup (tile row m, 256 columns), lane l
// columns c .. c + 3:
//     y[row] = sum over slices (in order) of part[slice][m] + s_a * t[row] B_a,
// row = perm[m] (or m), a = ids[row], y rounded once.  The partial sums go
// out first (they need nothing), then, once the row's adapter is known, its
// t values (into LDS) and B rows; rank rows past r read row 0 again and meet
// t = 0.
struct SplitFinishArgs {
    const float* part;      // [S][n][ldp]
    int64_t ldp;
    int32_t S;
    int32_t n;
    const int32_t* perm;    // tile row -> row, or null
    int32_t x_rows;         // rows of ids, t and y; a perm entry outside them skips the tile row
    const int32_t* ids;     // by row
    const float* t;         // [row][ldt], unscaled x A
    int64_t ldt;
    void* y;
    int64_t ldy;
};
constexpr int SF_SLICES = 8;   // K slices of a split launch at most
constexpr int SF_RCHUNK = 16;  // rank rows of B requested together

template <typename TY>
__global__ __launch_bounds__(64) void k_gemm_split_finish(PoolDev P, SplitFinishArgs f) {
    __shared__ float st[64];
    const int lane = threadIdx.x;
    const int N = P.d_out;
    const int nch = (N + 255) / 256;
    const int m = blockIdx.x / nch;
    const int c0 = (blockIdx.x - m * nch) * 256 + lane * 4;
    const bool in = c0 < N;
    const int cc = in ? c0 : 0;   // columns past d_out read column 0 and are not stored
    const bool vec = (N & 3) == 0;
    float4 u[SF_SLICES];
#pragma unroll
    for (int q = 0; q < SF_SLICES; ++q) {
        const float* pp = f.part + ((int64_t)(q < f.S ? q : 0) * f.n + m) * f.ldp + cc;
        if (vec) {
            u[q] = *(const float4*)pp;
        } else {
            u[q].x = pp[0];
            u[q].y = cc + 1 < N ? pp[1] : 0.f;
            u[q].z = cc + 2 < N ? pp[2] : 0.f;
            u[q].w = cc + 3 < N ? pp[3] : 0.f;
        }
    }
    const int row = f.perm ? f.perm[m] : m;
    if (row < 0 || row >= f.x_rows) return;   // the GEMM skipped it too (whole workgroup, before the barrier)
    const int a = f.ids[row];
    const bool ok = id_ok(a, P.n_adapters);
    const int r = ok ? uload(P.ranks, a) : 0;
    const int64_t boff = ok ? uload(P.b_off, a) : 0;
    const float sc = ok ? uload(P.scales, a) : 0.f;
    if (lane < r) st[lane] = f.t[(int64_t)row * f.ldt + lane];
    const bf16* Bu = (const bf16*)P.B + boff + cc;
    const bool vb = P.vec_b != 0;
    uint2 bv[SF_RCHUNK];
    auto load_b = [&](int j0) {
#pragma unroll
        for (int q = 0; q < SF_RCHUNK; ++q) {
            const int j = j0 + q;
            if (vb) {
                bv[q] = *(const uint2*)(Bu + (int64_t)(j < r ? j : 0) * N);
            } else {
                union { uint2 u; bf16 e[4]; } w;
                for (int e = 0; e < 4; ++e) w.e[e] = (j < r && cc + e < N) ? Bu[(int64_t)j * N + e] : (bf16)0;
                bv[q] = w.u;
            }
        }
    };
    if (r > 0) load_b(0);
    float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < SF_SLICES; ++q)
        if (q < f.S) {
            v[0] += u[q].x; v[1] += u[q].y; v[2] += u[q].z; v[3] += u[q].w;
        }
    __syncthreads();
    if (!in) return;
    if (r > 0) {
        float e4[4] = {0.f, 0.f, 0.f, 0.f};
        for (int j0 = 0;;) {
#pragma unroll
            for (int q = 0; q < SF_RCHUNK; ++q) {
                const float tj = (j0 + q < r) ? st[j0 + q] : 0.f;
                union { uint2 u; bf16 e[4]; } w;
                w.u = bv[q];
#pragma unroll
                for (int e = 0; e < 4; ++e) e4[e] += tj * to_f32(w.e[e]);
            }
            j0 += SF_RCHUNK;
            if (j0 >= r) break;
            load_b(j0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += sc * e4[e];
    }
    const bool vec_y = ((f.ldy * (int64_t)sizeof(TY)) & 15) == 0 && ((uintptr_t)f.y & 15) == 0;
    store_row_piece<TY, 4>((TY*)f.y + (int64_t)row * f.ldy + c0, v, N - c0, vec_y);
}

// ---------------------------------------------------------------------------
// Skinny layer GEMM for decode batches (n_rows <= 64, W stored [d_out, d_in])
// ---------------------------------------------------------------------------
//
// At decode sizes the base product is a stream of W with almost no reuse,
// so the kernel is shaped for bytes in flight rather than for reuse: a
// workgroup owns 16 output columns (16 rows of W^T) and all batch rows; its
// NW waves split K, and every lane loads its MFMA operands straight from
// global memory into registers, U K-steps at a time (U 16-byte loads of W
// in flight per lane, with the matching x fragments, which stay in L2).
// The per-wave partial tiles are added in LDS in wave order, then the scaled
// expand s * t_m B_a[:, n] is added per row and y is rounded once.

__device__ __forceinline__ bf16x8_t load8_bf16(const bf16* p, int valid) {
    if (valid >= 8) return *(const bf16x8_t*)p;
    union { bf16x8_t v; bf16 e[8]; } u;
#pragma unroll
    for (int e = 0; e < 8; ++e) u.e[e] = (e < valid) ? p[e] : (bf16)0;
    return u.v;
}

template <typename TY, int MB, int NW>
__global__ __launch_bounds__(NW * 64) void k_gemm_skinny(PoolDev P, GemmDev g) {
    // K-steps loaded per pass: bounded by the registers a lane has at NW waves
    constexpr int U = (NW >= 16) ? ((MB >= 2) ? 4 : 8) : ((MB >= 4) ? 8 : 16);
    constexpr int MT = MB * 16;
    __shared__ float red[NW][MT][17];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n0 = blockIdx.x * 16;
    const int K = P.d_in;
    const int N = P.d_out;
    const int M = g.n;
    const bf16* X = (const bf16*)g.x;
    const bf16* Wt = (const bf16*)g.W;
    const int lr = lane & 15;
    const int kq = (lane >> 4) * 8;
    const bool n_ok = n0 + lr < N;
    const bf16* wrow = Wt + (int64_t)(n_ok ? n0 + lr : 0) * g.ldw;

    f32x4_t acc[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nsteps = (K + 31) / 32;
    const int spw = (nsteps + NW - 1) / NW;
    const int s0 = wave * spw;
    const int s1 = min(nsteps, s0 + spw);
    for (int sb = s0; sb < s1; sb += U) {
        bf16x8_t bw[U];
        bf16x8_t ax[U][MB];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = (sb + u) * 32 + kq;
            const int valid = (sb + u < s1) ? min(8, K - k) : 0;
            bw[u] = (n_ok && valid > 0) ? load8_bf16(wrow + k, valid) : bf16x8_t{};
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const int m = i * 16 + lr;
                ax[u][i] = (m < M && valid > 0) ? load8_bf16(X + (int64_t)m * g.ldx + k, valid) : bf16x8_t{};
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < MB; ++i)
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax[u][i], bw[u], acc[i], 0, 0, 0);
    }

    const int lq = (lane >> 4) * 4;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) red[wave][i * 16 + lq + q][lr] = acc[i][q];
    __syncthreads();

    TY* Y = (TY*)g.y;
    for (int o = tid; o < MT * 16; o += NW * 64) {
        const int m = o >> 4;
        const int n = o & 15;
        const int col = n0 + n;
        if (m >= M || col >= N) continue;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) v += red[w][m][n];
        const int a = g.ids[m];
        if (id_ok(a, P.n_adapters)) {
            if (g.t) {
                const int r = P.ranks[a];
                const bf16* Bu = (const bf16*)P.B + P.b_off[a] + col;
                const float* tm = g.t + (int64_t)m * g.ldt;
                float e = 0.f;
                for (int j = 0; j < r; ++j) e += tm[j] * to_f32(Bu[(int64_t)j * N]);
                v += P.scales[a] * e;
            }
        } else if (a != -1 && blockIdx.x == 0) {
            flag_bad_id(P.err);
        }
        Y[(int64_t)m * g.ldy + col] = from_f32<TY>(v);
    }
}

// ---------------------------------------------------------------------------
// SGMV shrink: t[rows of segment] = x[rows] A_u   (BN = 64 covers r <= 64)
// ---------------------------------------------------------------------------

template <class C>
__global__ __launch_bounds__(C::NT) void k_sgmv_shrink(PoolDev P, const typename C::T* __restrict__ x,
                                                       int64_t ldx, const int32_t* __restrict__ perm,
                                                       const int32_t* __restrict__ seg_ids,
                                                       const int32_t* __restrict__ seg_off,
                                                       const int32_t* __restrict__ n_seg_p,
                                                       float* __restrict__ t, int64_t ldt,
                                                       typename C::T* __restrict__ t_ext, int64_t lde,
                                                       float* __restrict__ part, int32_t n_rows,
                                                       int32_t ks_len) {
    // part != nullptr: K is cut into slices of ks_len (a multiple of BK);
    // workgroup (tile, blockIdx.y) writes the slice's partial
    // part[slice][row][0:64] and the reduce pass forms t and t_ext.
    using T = typename C::T;
    static_assert(C::BN == 64, "shrink tile covers ranks up to 64");
    __shared__ __attribute__((aligned(16))) T smem[2 * C::STAGE];
    __shared__ int sRow[C::BM];
    __shared__ int sInfo[3];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / C::WN;
    const int wn = wave - wm * C::WN;

    if (wave == 0) {
        int s = 0, c = 0;
        const bool found = find_seg_tile(seg_off, *n_seg_p, C::BM, blockIdx.x, lane, s, c);
        if (lane == 0) {
            sInfo[0] = found ? 1 : 0;
            sInfo[1] = s;
            sInfo[2] = c;
        }
    }
    __syncthreads();
    if (!sInfo[0]) return;
    const int s = sInfo[1];
    const int row0 = seg_off[s] + sInfo[2] * C::BM;
    const int cnt = min(C::BM, seg_off[s + 1] - row0);
    const int u = seg_ids[s];
    for (int r = tid; r < C::BM; r += C::NT) sRow[r] = r < cnt ? perm[row0 + r] : -1;
    __syncthreads();

    const int r_max = P.r_max;
    const int slice = blockIdx.y;
    if (!id_ok(u, P.n_adapters)) {
        if (part) {
            for (int idx = tid; idx < cnt * 64; idx += C::NT) {
                const int m = idx / 64;
                part[((int64_t)slice * n_rows + sRow[m]) * 64 + (idx - m * 64)] = 0.f;
            }
            return;
        }
        for (int idx = tid; idx < cnt * r_max; idx += C::NT) {
            const int m = idx / r_max;
            t[(int64_t)sRow[m] * ldt + (idx - m * r_max)] = 0.f;
        }
        return;
    }
    const int r = P.ranks[u];
    const float sc = P.scales[u];
    const int ext_rank_cols = EXT_RANKS * ((r_max + EXT_RANKS - 1) / EXT_RANKS);
    const T* Au = (const T*)P.A + P.a_off[u];
    const bool vec = P.vec_a && ((r * (int)sizeof(T)) % 16) == 0;
    // this workgroup's K range; the loaders zero everything at or past kend
    const int kbeg = part ? slice * ks_len : 0;
    const int kend = part ? min(P.d_in, kbeg + ks_len) : P.d_in;

    Acc<C> acc;
    acc.zero();
    // Two K-blocks in flight: even blocks go through register set 0 and LDS
    // stage 0, odd blocks through set 1 and stage 1; block kb + 2 is
    // requested as soon as block kb is in LDS, so each wave waits on memory
    // once per two blocks' worth of loads.  One barrier per block: a wave
    // that writes a stage has passed the barrier after which every wave is
    // done with the block that stage held before.
    RowLoader<C, C::BM> la0, la1;
    TransLoader<C, C::BN> lb0, lb1;
    const int nk = (kend - kbeg + C::BK - 1) / C::BK;
    la0.load(x, ldx, sRow, kbeg, kend, tid);
    lb0.load(Au, r, kbeg, kend, 0, r, vec, tid);
    if (nk > 1) {
        la1.load(x, ldx, sRow, kbeg + C::BK, kend, tid);
        lb1.load(Au, r, kbeg + C::BK, kend, 0, r, vec, tid);
    }
    for (int kb = 0; kb < nk; kb += 2) {
        {
            T* sA = smem;
            T* sB = sA + C::A_ELEMS;
            la0.store(sA, tid);
            lb0.store(sB, tid);
            __syncthreads();
            if (kb + 2 < nk) {
                la0.load(x, ldx, sRow, kbeg + (kb + 2) * C::BK, kend, tid);
                lb0.load(Au, r, kbeg + (kb + 2) * C::BK, kend, 0, r, vec, tid);
            }
            mma_block<C>(acc, sA, sB, wm, wn, lane);
        }
        if (kb + 1 < nk) {
            T* sA = smem + C::STAGE;
            T* sB = sA + C::A_ELEMS;
            la1.store(sA, tid);
            lb1.store(sB, tid);
            __syncthreads();
            if (kb + 3 < nk) {
                la1.load(x, ldx, sRow, kbeg + (kb + 3) * C::BK, kend, tid);
                lb1.load(Au, r, kbeg + (kb + 3) * C::BK, kend, 0, r, vec, tid);
            }
            mma_block<C>(acc, sA, sB, wm, wn, lane);
        }
    }

    const int lc = lane % C::BLK;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            const int col = wn * C::WTN + j * C::BLK + lc;
#pragma unroll
            for (int q = 0; q < C::M::NACC; ++q) {
                const int m = wm * C::WTM + i * C::BLK + C::M::row(lane, q);
                if (m >= cnt) continue;
                const float v = acc.v[i][j][q];
                if (part) {
                    // columns past rank r are exact zeros (B side of the shrink was zero there)
                    part[((int64_t)slice * n_rows + sRow[m]) * 64 + col] = v;
                    continue;
                }
                if (col < r_max) t[(int64_t)sRow[m] * ldt + col] = v;
                if (t_ext && col < ext_rank_cols) {
                    // columns past rank r are exact zeros (B side of the shrink was zero there)
                    T* er = t_ext + (int64_t)sRow[m] * lde;
                    const float sv = sc * v;
                    if constexpr (sizeof(T) == 2) {
                        const int e = col / EXT_RANKS;
                        const int jj = col - e * EXT_RANKS;
                        const bf16 hi = f32_to_bf16(sv);
                        er[e * 64 + jj] = (T)hi;
                        er[e * 64 + 32 + jj] = (T)f32_to_bf16(sv - to_f32(hi));
                    } else {
                        er[col] = (T)sv;
                    }
                }
            }
        }
}

// t[row][j] = sum over slices (in order) of part[slice][row][j], and the
// K-extension operand s * t (bf16 hi | lo blocks, or fp32) for the row.
// Thread = (row, 4 columns); the slices' 16-byte pieces are requested four
// at a time before any is added.  S_dev (when set) holds the slice count
// the shrink launch chose on the device; S is then its upper bound.
template <typename T>
__global__ __launch_bounds__(256) void k_shrink_reduce(PoolDev P, const float* __restrict__ part, int32_t S,
                                                       int32_t n_rows, const int32_t* __restrict__ ids,
                                                       float* __restrict__ t, int64_t ldt,
                                                       T* __restrict__ t_ext, int64_t lde,
                                                       const int32_t* __restrict__ S_dev = nullptr) {
    const int idx = blockIdx.x * 256 + threadIdx.x;
    const int row = idx >> 4;
    const int c0 = (idx & 15) * 4;
    if (row >= n_rows) return;
    if (S_dev) S = min(S, *S_dev);
    const f32x4_t* pp = (const f32x4_t*)(part + (int64_t)row * 64 + c0);
    const int64_t sstride = (int64_t)n_rows * 16;   // one slice, in 16-byte pieces
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += 4) {
        f32x4_t q[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) q[j] = pp[(int64_t)min(s0 + j, S - 1) * sstride];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (s0 + j < S) v += q[j];
    }
    const int ext_rank_cols = EXT_RANKS * ((P.r_max + EXT_RANKS - 1) / EXT_RANKS);
    const int a = t_ext ? ids[row] : -1;
    const float sc = id_ok(a, P.n_adapters) ? P.scales[a] : 0.f;
    T* er = t_ext ? t_ext + (int64_t)row * lde : nullptr;
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
        const int col = c0 + e4;
        if (col < P.r_max) t[(int64_t)row * ldt + col] = v[e4];
        if (!er || col >= ext_rank_cols) continue;
        const float sv = sc * v[e4];
        if constexpr (sizeof(T) == 2) {
            const int e = col / EXT_RANKS;
            const int jj = col - e * EXT_RANKS;
            const bf16 hi = f32_to_bf16(sv);
            er[e * 64 + jj] = (T)hi;
            er[e * 64 + 32 + jj] = (T)f32_to_bf16(sv - to_f32(hi));
        } else {
            er[col] = (T)sv;
        }
    }
}

// ---------------------------------------------------------------------------
// SGMV shrink for long segments: bf16 pools whose ranks are multiples of 8
// ---------------------------------------------------------------------------
//
// part[slice][row][0:64] = x[row, K slice] A_u[K slice, 0:64] over segment
// tiles of 32 NW rows ("Serving multiple LoRAs: segmented matrix multiplies
// and adapter scheduling", section "Not merging the weights, computing in
// batches": a segment's shrink is one small matrix product).  The shrink of
// a prefill batch reads x once and each A_u once per tile, so it is a
// stream of x; everything here is arranged to keep many bytes of x in
// flight per CU:
//   - NW waves, each 32 rows x 64 ranks of 16x16x32 bf16 MFMAs;
//   - K-blocks of 64 go through a RING-deep register ring (block kb + RING
//     is requested as soon as block kb is in LDS) into two LDS stages, one
//     barrier per block;
//   - x is staged [row][k] (whole 128-byte lines per load), with
//     nontemporal loads: x is read once, and marked as streaming it leaves
//     L2 to A, which every tile of a segment re-reads;
//   - A_u's rows kbeg .. kbeg + 63 are one contiguous run of 64 r elements,
//     copied as they lie ([k][n], whole lines) into a [k][64] LDS block
//     whose 32-byte units are XOR-swizzled per row, and read as MFMA
//     operands with the LDS transpose read: lane i of a 16-lane group
//     points at row k0 + i / 4, columns n0 + 4 (i % 4) .. + 3 and receives
//     column n0 + i of rows k0 .. k0 + 3, so no transpose happens on the
//     way in.  The swizzle (unit ^= (k & 3) ^ ((k >> 3) & 1)) puts the rows
//     one transpose read touches in distinct banks;
//   - the grid is the number of workgroups the GPU holds at once; every
//     workgroup counts the batch's tiles T (from the segment descriptor)
//     and takes the same slice count S = min(s_max, grid / T), so the
//     T x S (tile, slice) items fill the GPU once whatever the segments;
//     workgroup 0 stores S for the reduce pass.
// Ranks past r are exact zeros in part (the LDS columns past r are zeroed).
constexpr int SX_KB = 64;
constexpr int SX_LDK = SX_KB + 8;                       // x rows padded by 16 bytes

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

struct ShrinkXArgs {
    const bf16* x;
    int64_t ldx;
    const int32_t* perm;
    const int32_t* seg_ids;
    const int32_t* seg_off;
    const int32_t* n_seg;
    float* part;        // [s_max][n_rows][64]
    int32_t* s_used;    // the slice count chosen (read by the reduce pass)
    int32_t n_rows;
    int32_t s_max;
};

// element offset of (k, n) in a swizzled [64][64] A block
__device__ __forceinline__ int sx_a_at(int k, int n) {
    return k * 64 + ((((n >> 4) ^ (k & 3) ^ ((k >> 3) & 1))) << 4) + (n & 15);
}

// NW waves of 32 rows (tile of 32 NW rows); a RING-deep register ring.
template <int NW, int RING>
__global__ __launch_bounds__(NW * 64) void k_sgmv_shrink_x(PoolDev P, ShrinkXArgs a) {
    constexpr int BM = 32 * NW;
    constexpr int NT = 64 * NW;
    constexpr int XPT = BM * (SX_KB / 8) / NT;     // 16-byte x pieces per thread per block
    constexpr int APT = SX_KB * 8 / NT;            // 16-byte A pieces per thread per block (r = 64)
    static_assert(XPT * NT == BM * SX_KB / 8 && APT * NT == SX_KB * 8 && APT >= 1, "blocks do not split evenly");
    static_assert(RING >= 2 && RING <= 8, "register ring of 2 to 8 blocks");
    __shared__ __attribute__((aligned(16))) bf16 sX[2][BM * SX_LDK];
    __shared__ __attribute__((aligned(16))) bf16 sA[2][SX_KB * 64];
    __shared__ int sRow[BM];
    __shared__ int sInfo[4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lr = lane & 15;
    const int G = gridDim.x;
    const int n_seg = *a.n_seg;

    if (wave == 0) {
        int tot = 0;
        for (int s0 = 0; s0 < n_seg; s0 += 64) {
            const int s = s0 + lane;
            const int c = s < n_seg ? (a.seg_off[s + 1] - a.seg_off[s] + BM - 1) / BM : 0;
            tot += __shfl(wave_incl_scan(c, lane), 63, 64);
        }
        if (lane == 0) sInfo[0] = tot;
    }
    __syncthreads();
    const int T = __builtin_amdgcn_readfirstlane(sInfo[0]);
    const int S0 = max(1, min(a.s_max, G / max(T, 1)));
    const int kslice = ((P.d_in + S0 - 1) / S0 + SX_KB - 1) / SX_KB * SX_KB;
    const int S = (P.d_in + kslice - 1) / kslice;   // every slice non-empty
    if (blockIdx.x == 0 && tid == 0) *a.s_used = S;

    // lane constants of the transpose reads: group g = lane / 16 takes k
    // rows g * 8 .. g * 8 + 7 of each 32-deep step (reads of rows + 0..3 and
    // + 4..7); the swizzle of those rows is (lr / 4) ^ (g & 1)
    const int g = lane >> 4;
    const int a_lane = (g * 8 + (lr >> 2)) * 64 + (lr & 3) * 4;
    const int a_sw = (lr >> 2) ^ (g & 1);

    for (int item = blockIdx.x; item < T * S; item += G) {
        const int tile = item / S;
        const int ks = item - tile * S;
        __syncthreads();   // the previous item is done with sRow, sInfo and both stages
        if (wave == 0) {
            int s = 0, c = 0;
            find_seg_tile(a.seg_off, n_seg, BM, tile, lane, s, c);
            if (lane == 0) {
                sInfo[1] = s;
                sInfo[2] = c;
            }
        }
        __syncthreads();
        const int s = __builtin_amdgcn_readfirstlane(sInfo[1]);
        const int row0 = a.seg_off[s] + __builtin_amdgcn_readfirstlane(sInfo[2]) * BM;
        const int cnt = min(BM, a.seg_off[s + 1] - row0);
        const int u = a.seg_ids[s];
        if (tid < BM) sRow[tid] = tid < cnt ? a.perm[row0 + tid] : -1;
        float* out = a.part + (int64_t)ks * a.n_rows * 64;
        if (!id_ok(u, P.n_adapters)) {
            __syncthreads();
            for (int idx = tid; idx < cnt * 64; idx += NT) out[(int64_t)sRow[idx >> 6] * 64 + (idx & 63)] = 0.f;
            continue;
        }
        const int r = pool_rank(P, u);
        const bf16* Au = (const bf16*)P.A + pool_a_off(P, u);
        const int kbeg = ks * kslice;
        const int klen = min(P.d_in, kbeg + kslice) - kbeg;
        const int nfull = klen / SX_KB;
        // the item walks its whole blocks from a tile-dependent start (fixed
        // per tile, so the sum order is too): tiles that run side by side
        // read different columns of their rows at any moment
        const int rot = nfull > 0 ? (tile * 3) % nfull : 0;
        // LDS columns past r hold zeros for the whole item (no block writes them)
        if (r < 64) {
            const int w = 64 - r;
            for (int idx = tid; idx < 2 * SX_KB * w; idx += NT) {
                const int st = idx / (SX_KB * w);
                const int rem = idx - st * SX_KB * w;
                const int k = rem / w;
                sA[st][sx_a_at(k, r + rem - k * w)] = 0;
            }
        }
        __syncthreads();   // sRow

        // piece v = tid + NT p: x row v / 8, k-piece v % 8; A element 8 v of
        // the block's run (row 8 v / r, column 8 v % r), valid for v < 8 r
        const bf16* xp[XPT];
        int xs[XPT];
#pragma unroll
        for (int p = 0; p < XPT; ++p) {
            const int v = tid + NT * p;
            const int m = v >> 3;
            const int gr = sRow[m] >= 0 ? sRow[m] : sRow[0];   // rows past cnt read row 0 (never stored)
            xp[p] = a.x + (int64_t)gr * a.ldx + kbeg + (v & 7) * 8;
            xs[p] = m * SX_LDK + (v & 7) * 8;
        }
        const bf16* ap[APT];
        int as[APT];
        bool aok[APT];
#pragma unroll
        for (int p = 0; p < APT; ++p) {
            const int v = tid + NT * p;
            aok[p] = v < 8 * r;
            const int e = aok[p] ? 8 * v : 0;
            const int k = e / r;
            ap[p] = Au + (int64_t)kbeg * r + e;
            as[p] = sx_a_at(k, e - k * r);
        }
        const int64_t ablk = (int64_t)SX_KB * r;   // elements of A per block

        u32x4_t xr[RING][XPT], ar[RING][APT];
        f32x4_t acc[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        auto load = [&](u32x4_t (&dx)[XPT], u32x4_t (&da)[APT], int kb) __attribute__((always_inline)) {
            kb += rot;
            kb -= kb >= nfull ? nfull : 0;
#pragma unroll
            for (int p = 0; p < XPT; ++p) dx[p] = __builtin_nontemporal_load((const u32x4_t*)(xp[p] + kb * SX_KB));
#pragma unroll
            for (int p = 0; p < APT; ++p) da[p] = *(const u32x4_t*)(ap[p] + kb * ablk);
        };
        auto store = [&](const u32x4_t (&dx)[XPT], const u32x4_t (&da)[APT], int st) __attribute__((always_inline)) {
#pragma unroll
            for (int p = 0; p < XPT; ++p) *(u32x4_t*)(sX[st] + xs[p]) = dx[p];
#pragma unroll
            for (int p = 0; p < APT; ++p)
                if (aok[p]) *(u32x4_t*)(sA[st] + as[p]) = da[p];
        };
        auto mma = [&](int st) __attribute__((always_inline)) {
            const bf16* sx = sX[st] + (wave * 32 + lr) * SX_LDK + (lane >> 4) * 8;
            const bf16* sa = sA[st] + a_lane;
#pragma unroll
            for (int h = 0; h < SX_KB / 32; ++h) {
                bf16x8_t xa[2], b[4];
#pragma unroll
                for (int i = 0; i < 2; ++i) xa[i] = *(const bf16x8_t*)(sx + i * 16 * SX_LDK + h * 32);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bf16* q = sa + h * 32 * 64 + ((j ^ a_sw) << 4);
                    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4_t*)q);
                    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4_t*)(q + 4 * 64));
                    b[j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                }
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[i], b[j], acc[i][j], 0, 0, 0);
            }
        };
        // one block: registers -> LDS stage kb & 1 (last read by block
        // kb - 2, which every wave finished before the barrier of block
        // kb - 1), then block kb + RING into the freed registers (past the
        // last whole block: that block again, from cache, never stored), then
        // the MFMAs.  Ring slot q holds the blocks kb with kb % RING == q.
        auto step = [&](u32x4_t (&dx)[XPT], u32x4_t (&da)[APT], int kb, int last) __attribute__((always_inline)) {
            store(dx, da, kb & 1);
            __syncthreads();
            load(dx, da, min(kb + RING, last));
            mma(kb & 1);
        };
        if (nfull > 0) {
            const int last = nfull - 1;
#pragma unroll
            for (int q = 0; q < RING; ++q) load(xr[q], ar[q], min(q, last));
            int kb = 0;
            for (; kb + RING <= nfull; kb += RING) {
#pragma unroll
                for (int q = 0; q < RING; ++q) step(xr[q], ar[q], kb + q, last);
            }
#pragma unroll
            for (int q = 0; q < RING - 1; ++q)
                if (kb + q < nfull) step(xr[q], ar[q], kb + q, last);
        }
        if (klen > nfull * SX_KB) {
            // ragged last block: x element-wise up to klen, A rows past it zero
            const int k0 = nfull * SX_KB;
            const int rows = klen - k0;
#pragma unroll
            for (int p = 0; p < XPT; ++p) {
                const int v = tid + NT * p;
                const int valid = min(8, max(0, rows - (v & 7) * 8));
                xr[0][p] = __builtin_bit_cast(u32x4_t, ld8_guard(xp[p] + k0, valid));
            }
#pragma unroll
            for (int p = 0; p < APT; ++p) {
                const int v = tid + NT * p;
                const bool in = aok[p] && (8 * v) / r < rows;
                ar[0][p] = in ? *(const u32x4_t*)(ap[p] + nfull * ablk) : u32x4_t{0u, 0u, 0u, 0u};
            }
            store(xr[0], ar[0], nfull & 1);
            __syncthreads();
            mma(nfull & 1);
        }

        // lane l holds rows (l / 16) * 4 + q of column l % 16 of each block
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = wave * 32 + i * 16 + (lane >> 4) * 4 + q;
                if (m >= cnt) continue;
                float* o = out + (int64_t)sRow[m] * 64 + lr;
#pragma unroll
                for (int j = 0; j < 4; ++j) o[j * 16] = acc[i][j][q];
            }
    }
}

// ---------------------------------------------------------------------------
// SGMV expand: y[rows of segment tile] (+)= s_u * t[rows] B_u
// ---------------------------------------------------------------------------
//
// Per output element the expand does r <= 64 multiply-adds and moves y once
// (read and written when accumulating): a stream of y whose product belongs
// on the matrix cores (at rank 64 it would take the fp32 vector units longer
// than the stream).  Workgroup (tile, chunk) owns up to 64 rows of one
// segment and EXP_SPAN output columns, taken 128 at a time:
//   - the A side is s_u * t of the tile's rows as bf16 pairs (hi, lo) with
//     hi + lo = s_u * t to about 16 significant bits, in blocks of 32 ranks
//     laid [hi(32) | lo(32)] along K; the B side is B_u's rank rows for
//     the piece, staged as they lie ([rank][column], whole 256-byte rows)
//     and read as MFMA operands with LDS transpose reads, one fragment per
//     32 ranks serving both the hi and the lo half;
//   - 4 waves, each 64 rows x 32 columns of 16x16x32 bf16 MFMAs;
//   - the fp32 tile then goes through LDS so that y moves in 16-byte pieces,
//     read and written once, rounded once.
// Each workgroup sums its ranks in a fixed order: results do not depend on
// timing.  Only the bf16 pool dtype takes this kernel (fp32 pools take
// k_sgmv_expand_f32 below).
constexpr int EXP_ROWS = 64;
constexpr int EXP_COLS = 128;
constexpr int EXP_THREADS = 256;
constexpr int EXP_KMAX = 128;                  // 2 x 64 ranks
constexpr int EXP_KLD = EXP_KMAX + 8;          // bf16 pitch of the staged rows (16-byte pad)
constexpr int EXP_CLD = EXP_COLS + 4;          // fp32 pitch of the staged output tile
constexpr int EXP_SPAN = 512;                 // columns per workgroup, in pieces of EXP_COLS (256: slower; 1024: slower)

// element offset of (rank j, column c) in the staged [64][EXP_COLS] B block:
// 32-byte units XOR-swizzled per row so that the eight rows one half-wave's
// transpose read touches fall in distinct banks
__device__ __forceinline__ int exp_b_at(int j, int c) {
    return j * EXP_COLS + ((((c >> 4) ^ ((j & 3) | (((j >> 3) & 1) << 2)))) << 4) + (c & 15);
}
__device__ __forceinline__ int exp_kcols(int r) { return 64 * ((r + 31) / 32); }

template <typename TY>
__global__ __launch_bounds__(EXP_THREADS) void k_sgmv_expand(PoolDev P, const float* __restrict__ t,
                                                             int64_t ldt, const int32_t* __restrict__ perm,
                                                             const int32_t* __restrict__ seg_ids,
                                                             const int32_t* __restrict__ seg_off,
                                                             const int32_t* __restrict__ n_seg_p,
                                                             TY* __restrict__ y, int64_t ldy, int accumulate,
                                                             int vec_y) {
    // A [64 rows][KLD] bf16 stays for the workgroup's whole span; the second
    // region holds B_u [64 ranks][128 columns] bf16 of one 128-column piece
    // (swizzled), then that piece's fp32 output tile [64][CLD]
    constexpr int A_BYTES = EXP_ROWS * EXP_KLD * 2;
    constexpr int B_BYTES = (EXP_KMAX / 2) * EXP_COLS * 2;
    constexpr int C_BYTES = EXP_ROWS * EXP_CLD * 4;
    constexpr int R2_BYTES = B_BYTES > C_BYTES ? B_BYTES : C_BYTES;
    __shared__ __attribute__((aligned(16))) uint8_t lds[A_BYTES + R2_BYTES];
    __shared__ int sRow[EXP_ROWS];
    __shared__ int sInfo[3];
    bf16* sA = (bf16*)lds;
    bf16* sB = (bf16*)(lds + A_BYTES);
    float* sC = (float*)(lds + A_BYTES);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    if (wave == 0) {
        int s = 0, c = 0;
        const bool found = find_seg_tile(seg_off, *n_seg_p, EXP_ROWS, blockIdx.x, lane, s, c);
        if (lane == 0) {
            sInfo[0] = found ? 1 : 0;
            sInfo[1] = s;
            sInfo[2] = c;
        }
    }
    __syncthreads();
    if (!sInfo[0]) return;
    const int s = sInfo[1];
    const int row0 = seg_off[s] + sInfo[2] * EXP_ROWS;
    const int cnt = min(EXP_ROWS, seg_off[s + 1] - row0);
    const int u = seg_ids[s];
    const bool ok = id_ok(u, P.n_adapters);
    if (!ok && accumulate) return;   // base-only rows keep their y
    if (tid < EXP_ROWS) sRow[tid] = tid < cnt ? perm[row0 + tid] : -1;
    __syncthreads();

    const int N = P.d_out;
    const int rk = ok ? P.ranks[u] : 0;
    const int K = exp_kcols(rk);   // 0 for a base-only tile
    const bf16* Bu = (const bf16*)P.B + (ok ? P.b_off[u] : 0);
    const bool vb = P.vec_b != 0;
    if (ok) {
        const float sc = P.scales[u];
        // A: row m, K column 64 e + h * 32 + jj holds the hi (h = 0) or lo
        // (h = 1) part of s * t[m][32 e + jj] (0 past the rank and past cnt)
        // (every load of a thread requested before any is stored: at most
        // EXP_ROWS * 64 / EXP_THREADS = 16 per thread)
        constexpr int TPT = EXP_ROWS * (EXP_KMAX / 2) / EXP_THREADS;
        const int nA = EXP_ROWS * (K / 2);
        float tv[TPT];
#pragma unroll
        for (int q = 0; q < TPT; ++q) {
            const int idx = tid + q * EXP_THREADS;
            const int m = idx / (K / 2);
            const int j = idx - m * (K / 2);
            const bool in = idx < nA && m < cnt && j < rk;
            tv[q] = t[in ? (int64_t)sRow[m] * ldt + j : 0];
            tv[q] = in ? tv[q] : 0.f;
        }
#pragma unroll
        for (int q = 0; q < TPT; ++q) {
            const int idx = tid + q * EXP_THREADS;
            if (idx < nA) {
                const int m = idx / (K / 2);
                const int j = idx - m * (K / 2);
                const float v = sc * tv[q];
                const bf16 hi = f32_to_bf16(v);
                const bf16 lo = f32_to_bf16(v - to_f32(hi));
                const int e = j >> 5;
                const int jj = j & 31;
                sA[m * EXP_KLD + e * 64 + jj] = hi;
                sA[m * EXP_KLD + e * 64 + 32 + jj] = lo;
            }
        }
    }
    const int lr = lane & 15;
    const int kq = (lane >> 4) * 8;
    const int lq = (lane >> 4) * 4;
    // transpose-read lane constants: group g = lane / 16 reads rank rows
    // g * 8 + lr / 4 (+ 4) of each 32-rank block, whose swizzle is
    // (lr / 4) | ((g & 1) << 2)
    const int b_lane = ((lane >> 4) * 8 + (lr >> 2)) * EXP_COLS + (lr & 3) * 4;
    const int b_sw = (lr >> 2) | (((lane >> 4) & 1) << 2);
    const int span0 = blockIdx.y * EXP_SPAN;
    for (int piece = 0; piece < EXP_SPAN / EXP_COLS; ++piece) {
        const int n0 = span0 + piece * EXP_COLS;
        if (n0 >= N) break;   // uniform over the workgroup
        // 16 threads per row, 8 columns each: a wave moves 4 rows of 128
        // contiguous columns per pass; 16 rows per pass of the workgroup.
        // Whole 16-byte pieces of y (the usual case) are requested, for all
        // passes, before B is staged and the MFMAs run (the y round trip
        // overlaps them); ragged or unaligned pieces go element by element.
        constexpr int NPASS = EXP_ROWS / 16;
        constexpr int YV = 8 * (int)sizeof(TY) / 16;   // 16-byte pieces per 8 columns
        const int cl = (tid & 15) * 8;
        const int nc = n0 + cl;
        uint4 yv[NPASS][YV];
        bool whole[NPASS];
#pragma unroll
        for (int pass = 0; pass < NPASS; ++pass) whole[pass] = pass * 16 + (tid >> 4) < cnt && vec_y && nc + 8 <= N;
        if (accumulate && vec_y && N >= 8) {
            // no branch around the loads: a lane without a whole piece reads
            // one that is in bounds (the tile's first row, the last whole
            // piece of columns) and ignores it
            const int c = min(nc, N - 8);
#pragma unroll
            for (int pass = 0; pass < NPASS; ++pass) {
                const int m = pass * 16 + (tid >> 4);
                const TY* src = y + (int64_t)sRow[m < cnt ? m : 0] * ldy + c;
#pragma unroll
                for (int h = 0; h < YV; ++h) yv[pass][h] = *(const uint4*)(src + h * (16 / sizeof(TY)));
            }
        }
        if (ok) {
            // B_u rows 0 .. K/2 - 1, columns n0 .. n0 + 127, staged as they lie
            // ([rank][column], rows past the rank zero) in a swizzled block
            // read by the MFMAs with LDS transpose reads.  16 lanes move one
            // 256-byte rank row; every load of a thread is requested, without
            // a branch, before any is stored; ragged or unaligned pieces after.
            constexpr int BPT = (EXP_KMAX / 2) * (EXP_COLS / 8) / EXP_THREADS;
            const int nB = (K / 2) * (EXP_COLS / 8);
            uint4 bv[BPT];
            bool bw[BPT];
#pragma unroll
            for (int q = 0; q < BPT; ++q) {
                const int idx = tid + q * EXP_THREADS;
                const int j = idx >> 4;
                const int nc = n0 + (idx & 15) * 8;
                bw[q] = idx < nB && j < rk && vb && nc + 8 <= N;
                bv[q] = *(const uint4*)(bw[q] ? Bu + (int64_t)j * N + nc : Bu);
            }
#pragma unroll
            for (int q = 0; q < BPT; ++q) {
                const int idx = tid + q * EXP_THREADS;
                if (idx >= nB) continue;
                const int j = idx >> 4;
                const int c8 = (idx & 15) * 8;
                const int nc = n0 + c8;
                union { uint4 u4; bf16 e[8]; } v;
                if (bw[q]) {
                    v.u4 = bv[q];
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        v.e[e] = (j < rk && nc + e < N) ? Bu[(int64_t)j * N + nc + e] : (bf16)0;
                }
                *(uint4*)(sB + exp_b_at(j, c8)) = v.u4;
            }
        }
        __syncthreads();   // A (first piece) and B staged
        f32x4_t acc[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // per 32 ranks: the B fragments (transpose reads: lane l takes column
        // l % 16 of its 16-column block, ranks (l / 16) * 8 .. + 7) serve both
        // the hi and the lo half of s t
        for (int kb = 0; kb < K / 64; ++kb) {
            bf16x8_t bb[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const bf16* q = sB + b_lane + kb * 32 * EXP_COLS + (((wave * 2 + j) ^ b_sw) << 4);
                const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)q);
                const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4_t*)(q + 4 * EXP_COLS));
                bb[j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                bf16x8_t a[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    a[i] = *(const bf16x8_t*)(sA + (i * 16 + lr) * EXP_KLD + kb * 64 + h * 32 + kq);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bb[j], acc[i][j], 0, 0, 0);
            }
        }
        __syncthreads();   // every wave is done with B before sC overwrites it
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    sC[(i * 16 + lq + q) * EXP_CLD + wave * 32 + j * 16 + lr] = acc[i][j][q];
        __syncthreads();
        // y pieces of this thread (requested at the top of the piece)
#pragma unroll
        for (int pass = 0; pass < NPASS; ++pass) {
            const int m = pass * 16 + (tid >> 4);
            if (m >= cnt || nc >= N) continue;
            TY* yr = y + (int64_t)sRow[m] * ldy;
            const float* cr = sC + m * EXP_CLD;
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = cr[cl + e];
            if (whole[pass]) {
                union { uint4 u4[YV]; TY e[8]; } o;
                if (accumulate) {
#pragma unroll
                    for (int h = 0; h < YV; ++h) o.u4[h] = yv[pass][h];
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] += to_f32(o.e[e]);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) o.e[e] = from_f32<TY>(v[e]);
#pragma unroll
                for (int h = 0; h < YV; ++h) *(uint4*)(yr + nc + h * (16 / sizeof(TY))) = o.u4[h];
            } else {
                for (int e = 0; e < 8 && nc + e < N; ++e) {
                    float w = v[e];
                    if (accumulate) w += to_f32(yr[nc + e]);
                    yr[nc + e] = from_f32<TY>(w);
                }
            }
        }
        __syncthreads();   // sC read before the next piece's B overwrites it
    }
}

// The expand for long segments: the same tiles and operands as above, run
// as a stream.  A tile's setup (its segment, rows, rank, scale and s t) is a
// chain of dependent loads, so the grid is the number of workgroups the GPU
// holds at once and each workgroup streams an equal run of the batch's
// 128-column pieces, numbered tile-major (every workgroup counts the tiles
// from the segment descriptor); a run crosses at most a tile boundary or two.
// The runs are dealt out XCD by XCD (workgroups b with b % 8 == 0 take the
// first runs), so an XCD's L2 serves one or two segments.  Within a tile, y (whole 16-byte pieces of
// rows) and B run through register rings YR pieces deep; B and the fp32
// output tile have LDS regions of their own, so a piece needs two barriers.
// Requires d_out % 8 == 0 and y rows 16-byte aligned.
template <typename TY>
__global__ __launch_bounds__(EXP_THREADS) __attribute__((amdgpu_waves_per_eu(2))) void k_sgmv_expand_t(
    PoolDev P, const float* __restrict__ t, int64_t ldt, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ seg_ids, const int32_t* __restrict__ seg_off, const int32_t* __restrict__ n_seg_p,
    int32_t cap, TY* __restrict__ y, int64_t ldy, int accumulate) {
    constexpr int BPT = (EXP_KMAX / 2) * (EXP_COLS / 8) / EXP_THREADS;   // B pieces per thread
    constexpr int NPASS = EXP_ROWS / 16;                                 // y rows per thread
    constexpr int YV = 8 * (int)sizeof(TY) / 16;                         // 16-byte pieces per 8 columns
    constexpr int YR = sizeof(TY) == 2 ? 3 : 2;                          // ring depth (pieces in flight)
    __shared__ __attribute__((aligned(16))) bf16 sA[EXP_ROWS * EXP_KLD];
    __shared__ __attribute__((aligned(16))) bf16 sB[(EXP_KMAX / 2) * EXP_COLS];
    __shared__ __attribute__((aligned(16))) float sC[EXP_ROWS * EXP_CLD];
    __shared__ int sRow[EXP_ROWS];
    __shared__ int sInfo[8];
    __shared__ SegTileCache C;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int N = P.d_out;
    const int npieces = (N + EXP_COLS - 1) / EXP_COLS;
    // the run boundaries and ids, once per workgroup (tile lookups then
    // read LDS), and the batch's tile count
    const int n_seg = seg_tile_cache_load(seg_off, seg_ids, n_seg_p, cap, tid, EXP_THREADS, C);
    __syncthreads();
    if (wave == 0) {
        int tot = 0;
        for (int s0 = 0; s0 < n_seg; s0 += 64) {
            const int s = s0 + lane;
            int c = 0;
            if (s < n_seg) {
                const int l = s < SEG_CACHE ? C.lo[s] : seg_off[s];
                const int h = s < SEG_CACHE ? C.hi[s] : seg_off[s + 1];
                c = (h - l + EXP_ROWS - 1) / EXP_ROWS;
            }
            tot += __shfl(wave_incl_scan(c, lane), 63, 64);
        }
        if (lane == 0) sInfo[0] = tot;
    }
    __syncthreads();
    const int T = __builtin_amdgcn_readfirstlane(sInfo[0]);
    const int G = gridDim.x;
    const int64_t total = (int64_t)T * npieces;
    // workgroups numbered XCD by XCD (those with b % 8 == 0 first), each
    // taking the next equal run of pieces [g_beg, g_end)
    const int xc = blockIdx.x & 7;
    const int64_t pos = (int64_t)xc * (G >> 3) + min(xc, G & 7) + (blockIdx.x >> 3);
    const int64_t g_beg = pos * total / G;
    const int64_t g_end = (pos + 1) * total / G;

    const int lr = lane & 15;
    const int kq = (lane >> 4) * 8;
    const int lq = (lane >> 4) * 4;
    const int b_lane = ((lane >> 4) * 8 + (lr >> 2)) * EXP_COLS + (lr & 3) * 4;
    const int b_sw = (lr >> 2) | (((lane >> 4) & 1) << 2);
    const int cl = (tid & 15) * 8;   // this thread's 8 columns of a piece, rows pass * 16 + tid / 16

    for (int64_t gp = g_beg; gp < g_end;) {
        const int tile = (int)(gp / npieces);
        const int p_beg = (int)(gp - (int64_t)tile * npieces);
        const int p_end = (int)min<int64_t>(npieces, p_beg + (g_end - gp));
        gp += p_end - p_beg;
        __syncthreads();   // the previous tile is done with sInfo, sRow, sA, sB and sC
        if (wave == 0) {
            // the tile from LDS, then its rows, B offset, rank and scale in one round trip
            int s = 0, c = 0, lo = 0, hi = 0, id = -1;
            seg_tile_find(C, n_seg, seg_off, seg_ids, EXP_ROWS, tile, lane, s, c, lo, hi, id);
            const int r0 = lo + c * EXP_ROWS;
            const int cn = min(EXP_ROWS, hi - r0);
            const bool v = id_ok(id, P.n_adapters);
            const int pr = lane < cn ? perm[r0 + lane] : -1;
            const int64_t bo = v ? P.b_off[id] : 0;
            const int rkk = v ? pool_rank(P, id) : 0;
            const float scv = v ? P.scales[id] : 0.f;
            sRow[lane] = pr;
            if (lane == 0) {
                sInfo[1] = cn;
                sInfo[2] = v ? 1 : 0;
                sInfo[3] = rkk;
                sInfo[4] = (int)(bo & 0xffffffff);
                sInfo[5] = (int)(bo >> 32);
                sInfo[6] = __float_as_int(scv);
            }
        }
        __syncthreads();
        const int cnt = __builtin_amdgcn_readfirstlane(sInfo[1]);
        const bool ok = __builtin_amdgcn_readfirstlane(sInfo[2]) != 0;
        if (!ok && accumulate) continue;   // base-only rows keep their y
        const int rk = __builtin_amdgcn_readfirstlane(sInfo[3]);
        const int64_t b_off = ((int64_t)__builtin_amdgcn_readfirstlane(sInfo[5]) << 32) |
                              (uint32_t)__builtin_amdgcn_readfirstlane(sInfo[4]);
        const int K = exp_kcols(rk);   // 0 for a base-only tile
        const bf16* Bu = (const bf16*)P.B + b_off;
        const bool vb = P.vec_b != 0;
        // this thread's y rows (pass p: row p * 16 + tid / 16; past cnt: the
        // tile's first row, read and never written)
        int yrow[NPASS];
        bool rin[NPASS];
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps) {
            const int m = ps * 16 + (tid >> 4);
            rin[ps] = m < cnt;
            yrow[ps] = sRow[rin[ps] ? m : 0];
        }
        auto load_y = [&](u32x4_t (&yv)[NPASS][YV], int pc) __attribute__((always_inline)) {
            if (!accumulate) return;
            const int c = pc * EXP_COLS + cl;
            const int cc = c + 8 <= N ? c : 0;   // d_out % 8 == 0: a piece is whole or past the end
#pragma unroll
            for (int ps = 0; ps < NPASS; ++ps)
#pragma unroll
                for (int h = 0; h < YV; ++h)
                    yv[ps][h] = *(const u32x4_t*)(y + (int64_t)yrow[ps] * ldy + cc + h * (16 / sizeof(TY)));
        };
        // B_u rows 0 .. K/2 - 1 of a piece's 128 columns, 16 lanes per
        // 256-byte rank row; whole aligned pieces only (others after, one
        // element at a time, in store_b)
        auto load_b = [&](u32x4_t (&bv)[BPT], int pc) __attribute__((always_inline)) {
            const int n0 = pc * EXP_COLS;
            int m = 0;
#pragma unroll
            for (int q = 0; q < BPT; ++q) {
                const int idx = tid + q * EXP_THREADS;
                const int j = idx >> 4;
                const int nc = n0 + (idx & 15) * 8;
                const bool w = j < K / 2 && j < rk && vb && nc + 8 <= N;
                bv[q] = *(const u32x4_t*)(w ? Bu + (int64_t)j * N + nc : Bu);
                m |= w ? 1 << q : 0;
            }
            return m;
        };
        auto store_b = [&](const u32x4_t (&bv)[BPT], int bw, int pc) __attribute__((always_inline)) {
            const int n0 = pc * EXP_COLS;
#pragma unroll
            for (int q = 0; q < BPT; ++q) {
                const int idx = tid + q * EXP_THREADS;
                const int j = idx >> 4;
                if (j >= K / 2) continue;
                const int c8 = (idx & 15) * 8;
                const int nc = n0 + c8;
                union { u32x4_t u4; bf16 e[8]; } v;
                if (bw & (1 << q)) {
                    v.u4 = bv[q];
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        v.e[e] = (j < rk && nc + e < N) ? Bu[(int64_t)j * N + nc + e] : (bf16)0;
                }
                *(u32x4_t*)(sB + exp_b_at(j, c8)) = v.u4;
            }
        };

        // the run's first YR pieces (in this tile) of y and first YR - 1 pieces of B are
        // requested before s t is staged (a base-only tile has rank 0: no B
        // piece is loaded or stored)
        const int np = p_end - p_beg;
        u32x4_t yr[YR][NPASS][YV];
        u32x4_t br[YR][BPT];
        int wb[YR];
#pragma unroll
        for (int q = 0; q < YR; ++q) load_y(yr[q], p_beg + min(q, np - 1));
#pragma unroll
        for (int q = 0; q < YR - 1; ++q) wb[q] = load_b(br[q], p_beg + min(q, np - 1));
        if (ok) {
            // A: row m, K column 64 e + h * 32 + jj holds the hi (h = 0) or lo
            // (h = 1) part of s * t[m][32 e + jj] (0 past the rank and past cnt)
            constexpr int TPT = EXP_ROWS * (EXP_KMAX / 2) / EXP_THREADS;
            const float sc = __int_as_float(__builtin_amdgcn_readfirstlane(sInfo[6]));
            const int nA = EXP_ROWS * (K / 2);
            float tv[TPT];
#pragma unroll
            for (int q = 0; q < TPT; ++q) {
                const int idx = tid + q * EXP_THREADS;
                const int m = idx / (K / 2);
                const int j = idx - m * (K / 2);
                const bool in = idx < nA && m < cnt && j < rk;
                tv[q] = t[in ? (int64_t)sRow[m] * ldt + j : 0];
                tv[q] = in ? tv[q] : 0.f;
            }
#pragma unroll
            for (int q = 0; q < TPT; ++q) {
                const int idx = tid + q * EXP_THREADS;
                if (idx < nA) {
                    const int m = idx / (K / 2);
                    const int j = idx - m * (K / 2);
                    const float v = sc * tv[q];
                    const bf16 hi = f32_to_bf16(v);
                    const bf16 lo = f32_to_bf16(v - to_f32(hi));
                    const int e = j >> 5;
                    const int jj = j & 31;
                    sA[m * EXP_KLD + e * 64 + jj] = hi;
                    sA[m * EXP_KLD + e * 64 + 32 + jj] = lo;
                }
            }
        }

        // piece kk of the run (ring slot kk % YR): its B into LDS (whose
        // last reader, the previous piece's MFMAs, every wave finished before
        // the previous piece's second barrier), barrier, piece kk + YR - 1's
        // B requested into the slot the previous piece freed, MFMAs, the fp32
        // tile into sC (whose last reads, the previous piece's, every wave
        // finished before this piece's first barrier), barrier, y added from
        // sC and written, piece kk + YR's y requested into this slot (past
        // the run's last piece: that piece again, never used)
        auto step = [&](u32x4_t (&yc)[NPASS][YV], u32x4_t (&bc)[BPT], int wcur, u32x4_t (&bn)[BPT], int& wn,
                        int kk) __attribute__((always_inline)) {
            const int pc = p_beg + kk;
            store_b(bc, wcur, pc);
            __syncthreads();
            wn = load_b(bn, p_beg + min(kk + YR - 1, np - 1));
            f32x4_t acc[4][2];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            for (int kb = 0; kb < K / 64; ++kb) {
                bf16x8_t bb[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const bf16* q = sB + b_lane + kb * 32 * EXP_COLS + (((wave * 2 + j) ^ b_sw) << 4);
                    const i16x4_t lo =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)q);
                    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4_t*)(q + 4 * EXP_COLS));
                    bb[j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    bf16x8_t a[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        a[i] = *(const bf16x8_t*)(sA + (i * 16 + lr) * EXP_KLD + kb * 64 + h * 32 + kq);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 2; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bb[j], acc[i][j], 0, 0, 0);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        sC[(i * 16 + lq + q) * EXP_CLD + wave * 32 + j * 16 + lr] = acc[i][j][q];
            __syncthreads();
            const int nc = pc * EXP_COLS + cl;
#pragma unroll
            for (int ps = 0; ps < NPASS; ++ps) {
                if (!rin[ps] || nc >= N) continue;
                const float* cr = sC + (ps * 16 + (tid >> 4)) * EXP_CLD + cl;
                union { u32x4_t u4[YV]; TY e[8]; } o;
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = cr[e];
                if (accumulate) {
#pragma unroll
                    for (int h = 0; h < YV; ++h) o.u4[h] = yc[ps][h];
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] += to_f32(o.e[e]);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) o.e[e] = from_f32<TY>(v[e]);
                TY* dst = y + (int64_t)yrow[ps] * ldy + nc;
#pragma unroll
                for (int h = 0; h < YV; ++h) *(u32x4_t*)(dst + h * (16 / sizeof(TY))) = o.u4[h];
            }
            load_y(yc, p_beg + min(kk + YR, np - 1));
        };
        int kk = 0;
        for (; kk + YR <= np; kk += YR) {
#pragma unroll
            for (int q = 0; q < YR; ++q)
                step(yr[q], br[q], wb[q], br[(q + YR - 1) % YR], wb[(q + YR - 1) % YR], kk + q);
        }
#pragma unroll
        for (int q = 0; q < YR - 1; ++q)
            if (kk + q < np) step(yr[q], br[q], wb[q], br[(q + YR - 1) % YR], wb[(q + YR - 1) % YR], kk + q);
    }
}

// fp32 pools: the same tiling on the vector units (fp32 products, no split).
constexpr int EXPF_ROWS = 64;
constexpr int EXPF_COLS = 256;
constexpr int EXPF_THREADS = 256;

template <typename TY>
__global__ __launch_bounds__(EXPF_THREADS) void k_sgmv_expand_f32(PoolDev P, const float* __restrict__ t,
                                                                  int64_t ldt, const int32_t* __restrict__ perm,
                                                                  const int32_t* __restrict__ seg_ids,
                                                                  const int32_t* __restrict__ seg_off,
                                                                  const int32_t* __restrict__ n_seg_p,
                                                                  TY* __restrict__ y, int64_t ldy,
                                                                  int accumulate) {
    __shared__ __attribute__((aligned(16))) float sT[64][EXPF_ROWS];   // s_u * t: [rank][row]
    __shared__ int sRow[EXPF_ROWS];
    __shared__ int sInfo[3];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    if (wave == 0) {
        int s = 0, c = 0;
        const bool found = find_seg_tile(seg_off, *n_seg_p, EXPF_ROWS, blockIdx.x, lane, s, c);
        if (lane == 0) {
            sInfo[0] = found ? 1 : 0;
            sInfo[1] = s;
            sInfo[2] = c;
        }
    }
    __syncthreads();
    if (!sInfo[0]) return;
    const int s = sInfo[1];
    const int row0 = seg_off[s] + sInfo[2] * EXPF_ROWS;
    const int cnt = min(EXPF_ROWS, seg_off[s + 1] - row0);
    const int u = seg_ids[s];
    const bool ok = id_ok(u, P.n_adapters);
    if (!ok && accumulate) return;
    if (tid < EXPF_ROWS) sRow[tid] = tid < cnt ? perm[row0 + tid] : -1;
    __syncthreads();
    const int N = P.d_out;
    const int col = blockIdx.y * EXPF_COLS + tid;
    const int rk = ok ? P.ranks[u] : 0;
    if (ok) {
        const float sc = P.scales[u];
        for (int idx = tid; idx < 64 * EXPF_ROWS; idx += EXPF_THREADS) {
            const int j = idx / EXPF_ROWS;
            const int m = idx - j * EXPF_ROWS;
            sT[j][m] = (m < cnt && j < rk) ? sc * t[(int64_t)sRow[m] * ldt + j] : 0.f;
        }
    }
    __syncthreads();
    if (col >= N) return;
    float acc[EXPF_ROWS];
#pragma unroll
    for (int m = 0; m < EXPF_ROWS; ++m) acc[m] = 0.f;
    const float* Bc = (const float*)P.B + (ok ? P.b_off[u] : 0) + col;
    for (int j = 0; j < rk; ++j) {
        const float b = Bc[(int64_t)j * N];
#pragma unroll
        for (int m = 0; m < EXPF_ROWS; m += 4) {
            const float4 tv = *(const float4*)&sT[j][m];
            acc[m] += tv.x * b;
            acc[m + 1] += tv.y * b;
            acc[m + 2] += tv.z * b;
            acc[m + 3] += tv.w * b;
        }
    }
#pragma unroll
    for (int m = 0; m < EXPF_ROWS; ++m) {
        if (m < cnt) {
            TY* p = y + (int64_t)sRow[m] * ldy + col;
            float v = acc[m];
            if (accumulate) v += to_f32(*p);
            *p = from_f32<TY>(v);
        }
    }
}

// ---------------------------------------------------------------------------
// Tile configurations
// ---------------------------------------------------------------------------

using GemmHuge = Cfg<bf16, 256, 256, 64, 2, 4, 32>;
using GemmBig = Cfg<bf16, 128, 128, 64, 2, 4, 32>;
using GemmMid = Cfg<bf16, 64, 64, 64, 2, 2>;
// base products and decode-style batches of a few hundred rows: the tiles
// are small to reach every CU, so each K-block is made 256 deep to keep
// 64 KiB per workgroup in flight (too deep for the K-extension: the LoRA
// term is added row by row after the K loop)
using GemmMed = Cfg<bf16, 64, 64, 256, 2, 2>;
using GemmSmall = Cfg<bf16, 32, 64, 64, 2, 2>;
using GemmF32 = Cfg<float, 64, 64, 32, 2, 2>;
// K-blocks of 64 (16 KiB of x and A per block, two in flight): four
// workgroups fit a CU (64: 102.7 us on the 70B prefill q/o shrink, against
// 112.5 at 128 and 144.7 at 32)
using ShrinkB = Cfg<bf16, 64, 64, 64, 4, 1>;
using ShrinkF = Cfg<float, 64, 64, 32, 4, 1>;

// part non-null: a K split into S slices of kslice K-blocks, base product
// only, fp32 partial sums into part (see GemmDev)
template <class C, typename TY, bool Q4 = false>
hipError_t run_gemm(const PoolDev& P, const GemmArgs& a, hipStream_t stream, float* part = nullptr,
                    int64_t ldp = 0, int S = 1, int kslice = 0) {
    static_assert(!Q4 || sizeof(typename C::T) == 2, "4-bit W with bf16 tiles");
    GemmDev g;
    g.part = part;
    g.ldp = ldp;
    g.kslice = kslice;
    g.x = a.x;
    g.ldx = a.ldx;
    g.W = a.W;
    g.ldw = a.ldw;
    g.ids = a.ids;
    g.n = a.n_rows;
    g.t = a.t;
    g.ldt = a.ldt;
    g.t_ext = a.t_ext;
    g.lde = a.lde;
    g.y = a.y;
    g.ldy = a.ldy;
    g.tiles_m = (int32_t)ceil_div(a.n_rows, C::BM);
    g.tiles_n = (int32_t)ceil_div(P.d_out, C::BN);
    g.perm = a.perm;
    g.x_rows = a.x_rows > 0 ? a.x_rows : a.n_rows;
    g.wscale = a.wscale;
    g.lds = a.lds;
    if (part) {   // the base product alone; the finish adds the adapter term
        g.t = nullptr;
        g.t_ext = nullptr;
    }
    dim3 grid((unsigned)((int64_t)g.tiles_m * g.tiles_n * (part ? S : 1)));
    if constexpr (Q4) {
        hipLaunchKernelGGL((k_layer_gemm<C, TY, true, true>), grid, dim3(C::NT), 0, stream, P, g);
    } else if (a.w_out_in) {
        hipLaunchKernelGGL((k_layer_gemm<C, TY, true>), grid, dim3(C::NT), 0, stream, P, g);
    } else {
        hipLaunchKernelGGL((k_layer_gemm<C, TY, false>), grid, dim3(C::NT), 0, stream, P, g);
    }
    return hipGetLastError();
}

template <typename TY, int MB>
hipError_t run_skinny(const PoolDev& P, const GemmArgs& a, hipStream_t stream) {
    GemmDev g;
    g.x = a.x;
    g.ldx = a.ldx;
    g.W = a.W;
    g.ldw = a.ldw;
    g.ids = a.ids;
    g.n = a.n_rows;
    g.t = a.t;
    g.ldt = a.ldt;
    g.t_ext = nullptr;
    g.lde = 0;
    g.y = a.y;
    g.ldy = a.ldy;
    g.perm = nullptr;
    g.x_rows = a.n_rows;
    g.tiles_m = 1;
    g.tiles_n = (int32_t)ceil_div(P.d_out, 16);
    dim3 grid((unsigned)g.tiles_n);
    // fewer column tiles than CUs: more waves per tile to keep bytes in flight
    if (g.tiles_n < 256)
        hipLaunchKernelGGL((k_gemm_skinny<TY, MB, 16>), grid, dim3(16 * 64), 0, stream, P, g);
    else
        hipLaunchKernelGGL((k_gemm_skinny<TY, MB, 8>), grid, dim3(8 * 64), 0, stream, P, g);
    return hipGetLastError();
}

// Tile rows [r0, n) of a GEMM call as a call of their own (the row tiles of
// the two calls are disjoint).  With perm only perm moves; otherwise every
// row pointer moves by r0 rows.
template <typename TY>
GemmArgs rows_from(const GemmArgs& a, int32_t r0) {
    GemmArgs b = a;
    b.n_rows = a.n_rows - r0;
    if (a.perm) {
        b.perm = a.perm + r0;
        b.x_rows = a.x_rows > 0 ? a.x_rows : a.n_rows;
        return b;
    }
    b.x = (const bf16*)a.x + (int64_t)r0 * a.ldx;
    b.x_rows = 0;
    b.ids = a.ids + r0;
    if (a.t) b.t = a.t + (int64_t)r0 * a.ldt;
    if (a.t_ext) b.t_ext = (const bf16*)a.t_ext + (int64_t)r0 * a.lde;
    b.y = (TY*)a.y + (int64_t)r0 * a.ldy;
    return b;
}

// K slices for a 128x128 launch of n_rows rows (1: no split).  With fewer
// tiles than CUs and a long K, each workgroup walks all of K one block at a
// time, about a microsecond a block whatever the tile size (the 2,218-row
// mixed batch: its k and v projections and the rows past the 256x256 rounds
// took 130-400 us each).  The split takes the slice count that minimises
// (rounds of one workgroup per CU) x (K-blocks per slice), plus two blocks'
// worth per slice for the partial sums, each slice at least 16 blocks deep.
int gemm_big_slices(const PoolDev& P, int32_t n_rows) {
    const int64_t T = ceil_div(n_rows, GemmBig::BM) * ceil_div(P.d_out, GemmBig::BN);
    const int64_t nk = ceil_div(P.d_in, GemmBig::BK);
    if (T >= 256 || nk < 32) return 1;
    int best = 1;
    int64_t best_cost = ceil_div(T, 256) * nk;
    for (int S = 2; S <= SF_SLICES && nk / S >= 16; ++S) {
        const int64_t cost = ceil_div(T * S, 256) * ceil_div(nk, S) + 2 * S;
        if (cost < best_cost) {
            best_cost = cost;
            best = S;
        }
    }
    return best;
}

size_t gemm_big_split_bytes(const PoolDev& P, int32_t n_rows) {
    const int S = gemm_big_slices(P, n_rows);
    return S > 1 ? align_up((size_t)S * n_rows * align_up((size_t)P.d_out, 4) * 4, 256) : 0;
}

// Rows of the 256x256 launch when the rows past its whole rounds take a
// second launch (0: one launch)
int32_t huge_head_rows(const PoolDev& P, int32_t n_rows) {
    auto tiles = [&](int bm, int bn) { return ceil_div(n_rows, bm) * ceil_div(P.d_out, bn); };
    const int64_t th = tiles(GemmHuge::BM, GemmHuge::BN);
    const int64_t tn = ceil_div(P.d_out, GemmHuge::BN);
    const int64_t tm_h = (th / 256) * 256 / tn;
    const int32_t r0 = (int32_t)(tm_h * GemmHuge::BM);
    if (tm_h > 0 && r0 < n_rows) {
        const double rounds = (double)ceil_div(th, 256);
        const double rounds_h = (double)ceil_div(tm_h * tn, 256);
        const double tail_rounds =
            0.35 * (double)ceil_div(ceil_div(n_rows - r0, GemmBig::BM) * ceil_div(P.d_out, GemmBig::BN), 256);
        if (rounds_h + tail_rounds < rounds - 0.25) return r0;
    }
    return 0;
}

// 128x128 tiles, K split when gemm_big_slices says so and the caller gave
// room for the partial sums (W stored [d_out, d_in], bf16 W): the split
// launch computes x W alone, the finish adds the slices and s t B_a
template <typename TY>
hipError_t run_gemm_big(const PoolDev& P, const GemmArgs& a, hipStream_t stream) {
    const int S = (a.split_part && a.w_out_in && !a.w_q4 && a.t) ? gemm_big_slices(P, a.n_rows) : 1;
    if (S < 2 || gemm_big_split_bytes(P, a.n_rows) > a.split_bytes) return run_gemm<GemmBig, TY>(P, a, stream);
    const int nk = (int)ceil_div(P.d_in, GemmBig::BK);
    const int kslice = (nk + S - 1) / S;
    const int Sr = (nk + kslice - 1) / kslice;   // every slice non-empty
    const int64_t ldp = (int64_t)align_up((size_t)P.d_out, 4);
    hipError_t e = run_gemm<GemmBig, TY>(P, a, stream, a.split_part, ldp, Sr, kslice);
    if (e != hipSuccess) return e;
    SplitFinishArgs f;
    f.part = a.split_part;
    f.ldp = ldp;
    f.S = Sr;
    f.n = a.n_rows;
    f.perm = a.perm;
    f.x_rows = a.x_rows > 0 ? a.x_rows : a.n_rows;
    f.ids = a.ids;
    f.t = a.t;
    f.ldt = a.ldt;
    f.y = a.y;
    f.ldy = a.ldy;
    const int nch = (int)ceil_div(P.d_out, 256);
    hipLaunchKernelGGL(k_gemm_split_finish<TY>, dim3((unsigned)((int64_t)a.n_rows * nch)), dim3(64), 0, stream, P,
                       f);
    return hipGetLastError();
}

template <typename TY>
hipError_t run_gemm_bf16(const PoolDev& P, const GemmArgs& a, hipStream_t stream, bool tail = false) {
    if (a.w_q4) {
        // 4-bit W: 256x256 tiles (the row tiles past whole rounds in 128x128
        // tiles when the last round would be mostly idle), else 128x128
        auto tiles = [&](int bm, int bn) { return ceil_div(a.n_rows, bm) * ceil_div(P.d_out, bn); };
        const int64_t th = tiles(GemmHuge::BM, GemmHuge::BN);
        if (!tail && th >= 200) {
            const int64_t tn = ceil_div(P.d_out, GemmHuge::BN);
            const int64_t tm_h = (th / 256) * 256 / tn;
            const int32_t r0 = (int32_t)(tm_h * GemmHuge::BM);
            if (tm_h > 0 && r0 < a.n_rows && ceil_div(tm_h * tn, 256) < ceil_div(th, 256)) {
                GemmArgs h = a;
                h.n_rows = r0;
                const hipError_t e = run_gemm<GemmHuge, TY, true>(P, h, stream);
                if (e != hipSuccess) return e;
                return run_gemm_bf16<TY>(P, rows_from<TY>(a, r0), stream, true);
            }
            return run_gemm<GemmHuge, TY, true>(P, a, stream);
        }
        return run_gemm<GemmBig, TY, true>(P, a, stream);
    }
    if (a.w_out_in && a.n_rows <= 64 && !a.t_ext && !a.perm) {
        if (a.n_rows <= 16) return run_skinny<TY, 1>(P, a, stream);
        if (a.n_rows <= 32) return run_skinny<TY, 2>(P, a, stream);
        return run_skinny<TY, 4>(P, a, stream);
    }
    // Largest tile that still gives about one workgroup per CU.
    auto tiles = [&](int bm, int bn) { return ceil_div(a.n_rows, bm) * ceil_div(P.d_out, bn); };
    const int64_t th = tiles(GemmHuge::BM, GemmHuge::BN);
    if (th >= 200) {
        // The 256x256 tiles run one per CU, in rounds of 256.  When the last
        // round would be mostly idle, the row tiles that fill whole rounds
        // take the 256x256 launch and the remaining rows a launch of 128x128
        // tiles (a quarter of the work each).
        const int32_t r0 = huge_head_rows(P, a.n_rows);
        if (r0 > 0) {
            GemmArgs h = a;
            h.n_rows = r0;
            const hipError_t e = run_gemm<GemmHuge, TY>(P, h, stream);
            if (e != hipSuccess) return e;
            return run_gemm_bf16<TY>(P, rows_from<TY>(a, r0), stream, true);
        }
        return run_gemm<GemmHuge, TY>(P, a, stream);
    }
    // 128x128 tiles from 96 of them: fewer workgroups than CUs, but a
    // 128x128 tile moves half the x and W bytes per flop of a 64x64 tile
    if (tiles(GemmBig::BM, GemmBig::BN) >= (tail ? 64 : 96)) return run_gemm_big<TY>(P, a, stream);
    if (a.w_out_in && (!a.t_ext || (a.t && a.rows_distinct))) return run_gemm<GemmMed, TY>(P, a, stream);
    if (tiles(GemmMid::BM, GemmMid::BN) >= 128 || a.n_rows > 32) return run_gemm<GemmMid, TY>(P, a, stream);
    return run_gemm<GemmSmall, TY>(P, a, stream);
}

}  // namespace

hipError_t launch_layer_gemm(const PoolDev& P, lora_dtype_t dt, lora_dtype_t ydt, const GemmArgs& a,
                             hipStream_t stream) {
    if (dt == LORA_BF16)
        return ydt == LORA_BF16 ? run_gemm_bf16<bf16>(P, a, stream) : run_gemm_bf16<float>(P, a, stream);
    return ydt == LORA_BF16 ? run_gemm<GemmF32, bf16>(P, a, stream) : run_gemm<GemmF32, float>(P, a, stream);
}

size_t layer_gemm_split_bytes(const PoolDev& P, int32_t n_rows) {
    // the 128x128 launch that run_gemm_bf16 may split: all rows, or the rows
    // past the 256x256 rounds
    if (n_rows <= 0) return 0;
    auto tiles = [&](int32_t rows, int bm, int bn) { return ceil_div(rows, bm) * ceil_div(P.d_out, bn); };
    if (tiles(n_rows, GemmHuge::BM, GemmHuge::BN) >= 200) {
        const int32_t r0 = huge_head_rows(P, n_rows);
        if (r0 <= 0) return 0;
        const int32_t rest = n_rows - r0;
        if (tiles(rest, GemmHuge::BM, GemmHuge::BN) >= 200) return 0;
        return tiles(rest, GemmBig::BM, GemmBig::BN) >= 64 ? gemm_big_split_bytes(P, rest) : 0;
    }
    return tiles(n_rows, GemmBig::BM, GemmBig::BN) >= 96 ? gemm_big_split_bytes(P, n_rows) : 0;
}

static int64_t seg_tiles(int32_t n_rows, int32_t n_bins, int bm) {
    return ceil_div(n_rows, bm) + std::min<int64_t>(n_rows, n_bins);
}

int32_t sgmv_shrink_slices(const PoolDev& P, int32_t n_rows) {
    // about 1024 workgroups over the row tiles (one round at four per CU;
    // 2048 measured slower), each slice at least 1024 k-rows
    const int64_t tiles = std::max<int64_t>(1, ceil_div(n_rows, ShrinkB::BM));
    const int64_t want = ceil_div(1024, tiles);
    return (int32_t)std::max<int64_t>(1, std::min<int64_t>(want, P.d_in / 1024));
}

size_t sgmv_shrink_part_bytes(const PoolDev& P, int32_t n_rows) {
    // the slices' partial sums, then (k_sgmv_shrink_x) the slice count it chose
    const int32_t S = sgmv_shrink_slices(P, n_rows);
    return S > 1 ? align_up((size_t)S * n_rows * 64 * 4, 256) + 256 : 0;
}

// k_sgmv_shrink_x launch shape: 8 waves (256-row tiles), a 4-block ring (6 measured no faster).
constexpr int SX_NW = 8, SX_RING = 4;

// Workgroups of k_sgmv_shrink_x the current device holds at once.
static int shrink_x_slots() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0, per = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_sgmv_shrink_x<SX_NW, SX_RING>, SX_NW * 64, 0) !=
            hipSuccess)
            per = 0;
        v = std::max(1, cus) * std::max(1, per);
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// k_sgmv_shrink_x takes bf16 pools whose A blocks are 16-byte aligned and
// whose ranks are multiples of 8, when the K split is on.
static hipError_t run_shrink_x(const PoolDev& P, const void* x, int64_t ldx, const lora_segments_t* seg,
                               int32_t n_rows, int32_t n_bins, float* t, int64_t ldt, void* t_ext, int64_t lde,
                               const int32_t* ids, float* part, hipStream_t stream) {
    const int32_t s_max = sgmv_shrink_slices(P, n_rows);
    int32_t* s_used = (int32_t*)((uint8_t*)part + align_up((size_t)s_max * n_rows * 64 * 4, 256));
    const int64_t items = seg_tiles(n_rows, n_bins, 32 * SX_NW) * s_max;
    const int G = (int)std::max<int64_t>(1, std::min<int64_t>(shrink_x_slots(), items));
    ShrinkXArgs a{(const bf16*)x, ldx, seg->perm, seg->seg_ids, seg->seg_off, seg->n_seg, part, s_used, n_rows, s_max};
    hipLaunchKernelGGL((k_sgmv_shrink_x<SX_NW, SX_RING>), dim3((unsigned)G), dim3(SX_NW * 64), 0, stream, P, a);
    dim3 rgrid((unsigned)ceil_div((int64_t)n_rows * 16, 256));
    hipLaunchKernelGGL(k_shrink_reduce<bf16>, rgrid, dim3(256), 0, stream, P, (const float*)part, s_max, n_rows,
                       ids, t, ldt, (bf16*)t_ext, lde, (const int32_t*)s_used);
    return hipGetLastError();
}

template <class C, typename T>
static hipError_t run_shrink(const PoolDev& P, const void* x, int64_t ldx, const lora_segments_t* seg,
                             int32_t n_rows, int32_t n_bins, float* t, int64_t ldt, void* t_ext, int64_t lde,
                             const int32_t* ids, float* part, hipStream_t stream) {
    int32_t S = part ? sgmv_shrink_slices(P, n_rows) : 1;
    int32_t ks_len = P.d_in;
    if (S > 1) {
        ks_len = (int32_t)align_up((size_t)ceil_div(P.d_in, S), C::BK);
        S = (int32_t)ceil_div(P.d_in, ks_len);
    }
    float* pt = S > 1 ? part : nullptr;
    dim3 grid((unsigned)seg_tiles(n_rows, n_bins, C::BM), (unsigned)S);
    hipLaunchKernelGGL(k_sgmv_shrink<C>, grid, dim3(C::NT), 0, stream, P, (const T*)x, ldx, seg->perm,
                       seg->seg_ids, seg->seg_off, seg->n_seg, t, ldt, (T*)t_ext, lde, pt, n_rows, ks_len);
    if (pt) {
        dim3 rgrid((unsigned)ceil_div((int64_t)n_rows * 16, 256));
        hipLaunchKernelGGL(k_shrink_reduce<T>, rgrid, dim3(256), 0, stream, P, (const float*)pt, S, n_rows, ids,
                           t, ldt, (T*)t_ext, lde);
    }
    return hipGetLastError();
}

hipError_t launch_sgmv_shrink(const PoolDev& P, lora_dtype_t dt, const void* x, int64_t ldx,
                              const lora_segments_t* seg, int32_t n_rows, int32_t n_bins, float* t,
                              int64_t ldt, bool, hipStream_t stream, void* t_ext, int64_t lde,
                              const int32_t* ids, float* part) {
    if (dt == LORA_BF16) {
        if (part && P.vec_a && P.vec_rank && sgmv_shrink_slices(P, n_rows) > 1)
            return run_shrink_x(P, x, ldx, seg, n_rows, n_bins, t, ldt, t_ext, lde, ids, part, stream);
        return run_shrink<ShrinkB, bf16>(P, x, ldx, seg, n_rows, n_bins, t, ldt, t_ext, lde, ids, part, stream);
    }
    return run_shrink<ShrinkF, float>(P, x, ldx, seg, n_rows, n_bins, t, ldt, t_ext, lde, ids, part, stream);
}

// Workgroups of k_sgmv_expand_t (bf16 or fp32 y) the current device holds at once.
static int expand_t_slots(bool bf16_y) {
    static std::atomic<int> cache[2][64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int v = cache[bf16_y][dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0, per = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
        const hipError_t e = bf16_y ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_sgmv_expand_t<bf16>,
                                                                                   EXP_THREADS, 0)
                                    : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_sgmv_expand_t<float>,
                                                                                   EXP_THREADS, 0);
        if (e != hipSuccess) per = 0;
        v = std::max(1, cus) * std::max(1, per);
        cache[bf16_y][dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

hipError_t launch_sgmv_expand(const PoolDev& P, lora_dtype_t dt, const float* t, int64_t ldt,
                              const lora_segments_t* seg, int32_t n_rows, int32_t n_bins, void* y,
                              lora_dtype_t ydt, int64_t ldy, int accumulate, hipStream_t stream) {
    const unsigned row_tiles = (unsigned)seg_tiles(n_rows, n_bins, EXP_ROWS);
    if (dt == LORA_BF16) {
        const dim3 grid(row_tiles, (unsigned)ceil_div(P.d_out, EXP_SPAN));
        // 16-byte y pieces when y and its rows are 16-byte aligned
        const size_t yb = ydt == LORA_BF16 ? 2 : 4;
        const int vec_y = (((uintptr_t)y & 15u) == 0 && (ldy * (int64_t)yb) % 16 == 0) ? 1 : 0;
        // the streaming kernel: whole 16-byte pieces of y rows
        const bool piece_y = P.d_out % 8 == 0 && vec_y;
        if (piece_y) {
            const int64_t most = (int64_t)row_tiles * ceil_div(P.d_out, EXP_COLS);   // items never exceed this
            const int G = (int)std::max<int64_t>(1, std::min<int64_t>(expand_t_slots(ydt == LORA_BF16), most));
            const int32_t cap = std::min<int32_t>(seg->cap, std::max<int32_t>(1, std::min<int32_t>(n_rows, n_bins)));
            if (ydt == LORA_BF16)
                hipLaunchKernelGGL(k_sgmv_expand_t<bf16>, dim3((unsigned)G), dim3(EXP_THREADS), 0, stream, P, t,
                                   ldt, seg->perm, seg->seg_ids, seg->seg_off, seg->n_seg, cap, (bf16*)y, ldy,
                                   accumulate);
            else
                hipLaunchKernelGGL(k_sgmv_expand_t<float>, dim3((unsigned)G), dim3(EXP_THREADS), 0, stream, P, t,
                                   ldt, seg->perm, seg->seg_ids, seg->seg_off, seg->n_seg, cap, (float*)y, ldy,
                                   accumulate);
        } else if (ydt == LORA_BF16)
            hipLaunchKernelGGL(k_sgmv_expand<bf16>, grid, dim3(EXP_THREADS), 0, stream, P, t, ldt, seg->perm,
                               seg->seg_ids, seg->seg_off, seg->n_seg, (bf16*)y, ldy, accumulate, vec_y);
        else
            hipLaunchKernelGGL(k_sgmv_expand<float>, grid, dim3(EXP_THREADS), 0, stream, P, t, ldt, seg->perm,
                               seg->seg_ids, seg->seg_off, seg->n_seg, (float*)y, ldy, accumulate, vec_y);
    } else {
        const dim3 grid(row_tiles, (unsigned)ceil_div(P.d_out, EXPF_COLS));
        if (ydt == LORA_BF16)
            hipLaunchKernelGGL(k_sgmv_expand_f32<bf16>, grid, dim3(EXPF_THREADS), 0, stream, P, t, ldt,
                               seg->perm, seg->seg_ids, seg->seg_off, seg->n_seg, (bf16*)y, ldy, accumulate);
        else
            hipLaunchKernelGGL(k_sgmv_expand_f32<float>, grid, dim3(EXPF_THREADS), 0, stream, P, t, ldt,
                               seg->perm, seg->seg_ids, seg->seg_off, seg->n_seg, (float*)y, ldy, accumulate);
    }
    return hipGetLastError();
}

}  // namespace lora
