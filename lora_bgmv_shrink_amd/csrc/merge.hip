// Folding one adapter into a base weight, in place:
//
//     W += sign * s_a * A_a B_a
//
// ("Serving many LoRA adapters" (blog.ecitis.org), section "Merge or keep
// separate": a merged replica serves its adapter as plain base-model
// inference; taking the adapter back out is the same update with the
// opposite sign.)  W is the caller's weight in either storage layout:
//   IN_OUT  W [d_in, d_out]:  element (k, c) at W[k * ldw + c]
//   OUT_IN  W [d_out, d_in]:  element (k, c) at W[c * ldw + k]
// Every element is read once, updated in fp32 and rounded once.
//
// The update streams W twice (read + write) and is HBM-bound, except that a
// rank-64 update of a bf16 weight asks 32 flop per byte, more than the fp32
// vector units deliver at HBM speed: the bf16 kernel forms A_a B_a on the
// matrix cores (16x16x32 MFMA over the rank), the fp32 kernel (8 bytes per
// element, 16 flop per byte at rank 64) on the vector units.
#include <hip/hip_runtime.h>

#include "lora_internal.hpp"

namespace lora {
namespace {

// bf16 tile: 64 rows x 128 columns of W as stored, four waves of 32 x 64.
constexpr int MG_ROWS = 64;
constexpr int MG_COLS = 128;
constexpr int MG_THREADS = 256;
constexpr int MG_LDT = MG_COLS + 4;           // fp32 pitch of the staged product
constexpr int MG_PIECES = MG_ROWS * MG_COLS / 8 / MG_THREADS;   // 16-byte W pieces per thread

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// element offset of (rank j, column c) in a staged [64][NC] block of B_a:
// 32-byte units XOR-swizzled per row so that the rows one transpose read
// touches fall in distinct banks (NC = 128: 8 units a row, the eight rows of
// a half-wave in distinct units; NC = 64: 4 units, two rows per 64 banks)
template <int NC>
__device__ __forceinline__ int mg_b_at(int j, int c) {
    const int sw = NC == 128 ? ((j & 3) | (((j >> 3) & 1) << 2)) : ((j & 3) ^ ((j >> 3) & 1));
    return j * NC + ((((c >> 4) ^ sw)) << 4) + (c & 15);
}

// One 16-byte W piece of the tile: stored row `row`, columns col .. col + 7.
struct Piece {
    int row, col;
};
__device__ __forceinline__ Piece piece_of(int tid, int p) {
    const int idx = tid + p * MG_THREADS;
    return Piece{idx / (MG_COLS / 8), (idx % (MG_COLS / 8)) * 8};
}

// Rows and columns below are those of W as stored.  The product term of
// stored element (row, col) is sum_j L[row][j] * R[j][col] with
//   IN_OUT: L = A_a (row = k), R = B_a (col = c)
//   OUT_IN: L = B_a^T (row = c), R = A_a^T (col = k)
// A_a rows are j-contiguous, so its MFMA operand comes straight from global
// memory.  B_a is staged into LDS as it lies ([j][c], 16-byte pieces of its
// rows) and read as MFMA operands with the LDS transpose read (lane i of a
// 16-lane group points at row j0 + i / 4, columns c0 + 4 (i % 4) and
// receives column c0 + i of rows j0 .. j0 + 3).
//
// A workgroup walks tiles t = blockIdx.x, blockIdx.x + gridDim.x, ...; the
// next tile's W pieces are requested before the current tile is worked on,
// so W reads stay in flight across tiles.
template <bool OUT_IN>
__global__ __launch_bounds__(MG_THREADS) __attribute__((amdgpu_waves_per_eu(3))) void k_merge_bf16(PoolDev P, int32_t adapter, float sign,
                                                            bf16* __restrict__ W, int64_t ldw, int32_t tiles_c,
                                                            int32_t n_tiles) {
    constexpr int NC = OUT_IN ? MG_ROWS : MG_COLS;   // c values per tile
    __shared__ __attribute__((aligned(16))) bf16 sB[64 * NC];
    __shared__ __attribute__((aligned(16))) float sAcc[MG_ROWS * MG_LDT];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave >> 1;   // 32-row half of the tile
    const int wc = wave & 1;    // 64-column half of the tile
    const int n_rows = OUT_IN ? P.d_out : P.d_in;   // stored rows
    const int n_cols = OUT_IN ? P.d_in : P.d_out;   // stored columns
    const int r = uload(P.ranks, adapter);
    const float s = sign * uload(P.scales, adapter);
    const bf16* Aa = (const bf16*)P.A + uload(P.a_off, adapter);
    const bf16* Ba = (const bf16*)P.B + uload(P.b_off, adapter);
    const int d_in = P.d_in;
    const int d_out = P.d_out;
    const int steps = (r + 31) / 32;   // 32 ranks per MFMA step

    auto load_w = [&](uint4 (&wv)[MG_PIECES], int t) __attribute__((always_inline)) {
        const int row0 = (t / tiles_c) * MG_ROWS;
        const int col0 = (t % tiles_c) * MG_COLS;
#pragma unroll
        for (int p = 0; p < MG_PIECES; ++p) {
            const Piece q = piece_of(tid, p);
            const int row = row0 + q.row, col = col0 + q.col;
            const bf16* src = W + (int64_t)(row < n_rows ? row : 0) * ldw + col;
            if (row < n_rows && col + 8 <= n_cols) {
                wv[p] = *(const uint4*)src;
            } else {
                union { uint4 u; bf16 e[8]; } v;
#pragma unroll
                for (int e = 0; e < 8; ++e) v.e[e] = (row < n_rows && col + e < n_cols) ? src[e] : (bf16)0;
                wv[p] = v.u;
            }
        }
    };

    // L and R operands of 16x16x32 steps over j; lane l takes row/column
    // l % 16 and ranks (l / 16) * 8 .. + 8
    const int lr = lane & 15;
    const int kq = (lane >> 4) * 8;
    const bool vec_a = P.vec_a && (r % 8) == 0;
    auto a_frag = [&](int k, int j0) __attribute__((always_inline)) {
        const int j = j0 + kq;
        if (vec_a && k < d_in && j < r) return *(const bf16x8_t*)(Aa + (int64_t)k * r + j);
        union { bf16x8_t v; bf16 e[8]; } t;
#pragma unroll
        for (int e = 0; e < 8; ++e) t.e[e] = (k < d_in && j + e < r) ? Aa[(int64_t)k * r + j + e] : (bf16)0;
        return t.v;
    };
    // transpose-read operand: columns cb .. cb + 15 of the staged block,
    // ranks j0 + (l / 16) * 8 .. + 8
    const int b_lane = ((lane >> 4) * 8 + (lr >> 2)) * NC + (lr & 3) * 4;
    const int b_sw = NC == 128 ? ((lr >> 2) | (((lane >> 4) & 1) << 2)) : ((lr >> 2) ^ ((lane >> 4) & 1));
    auto b_frag = [&](int cb, int j0) __attribute__((always_inline)) {
        const bf16* q = sB + b_lane + j0 * NC + (((cb >> 4) ^ b_sw) << 4);
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)q);
        const i16x4_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(q + 4 * NC));
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    uint4 wv[MG_PIECES], wn[MG_PIECES];
    int t = blockIdx.x;
    if (t < n_tiles) load_w(wv, t);
    for (; t < n_tiles; t += gridDim.x) {
        const int row0 = (t / tiles_c) * MG_ROWS;
        const int col0 = (t % tiles_c) * MG_COLS;
        if (t + (int)gridDim.x < n_tiles) load_w(wn, t + gridDim.x);

        // this tile's A_a operands (two rank steps at most)
        bf16x8_t Ag[2][OUT_IN ? 4 : 2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            if (st >= steps) break;
#pragma unroll
            for (int f = 0; f < (OUT_IN ? 4 : 2); ++f) {
                const int k = OUT_IN ? col0 + wc * 64 + f * 16 + lr : row0 + wr * 32 + f * 16 + lr;
                Ag[st][f] = a_frag(k, st * 32);
            }
        }
        // B_a[j][c] for the tile's c range -> sB (16-byte pieces of B rows,
        // as they lie); ranks past r are 0 up to the last 32-rank step
        // (whole pieces requested together, without a branch, before any is
        // stored: a load-then-store loop waited one round trip per piece)
        const int c0 = OUT_IN ? row0 : col0;
        constexpr int BPR = NC / 8;   // pieces per B row
        constexpr int BPT = 64 * BPR / MG_THREADS;
        uint4 bv[BPT];
        bool bw[BPT];
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            const int idx = tid + q * MG_THREADS;
            const int j = idx / BPR;
            const int c = (idx - j * BPR) * 8;
            bw[q] = j < r && c0 + c + 8 <= d_out && P.vec_b;
            bv[q] = *(const uint4*)(bw[q] ? Ba + (int64_t)j * d_out + c0 + c : Ba);
        }
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            const int idx = tid + q * MG_THREADS;
            const int j = idx / BPR;
            if (j >= 32 * steps) continue;
            const int c = (idx - j * BPR) * 8;
            union { uint4 u; bf16 e[8]; } v;
            if (bw[q]) {
                v.u = bv[q];
            } else {
                const bf16* src = Ba + (int64_t)j * d_out + c0 + c;
#pragma unroll
                for (int e = 0; e < 8; ++e) v.e[e] = (j < r && c0 + c + e < d_out) ? src[e] : (bf16)0;
            }
            *(uint4*)(sB + mg_b_at<NC>(j, c)) = v.u;
        }
        __syncthreads();

        f32x4_t acc[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) acc[i][jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            if (st >= steps) break;
            const int j0 = st * 32;
            bf16x8_t L[2], R[4];
#pragma unroll
            for (int i = 0; i < 2; ++i) L[i] = OUT_IN ? b_frag(wr * 32 + i * 16, j0) : Ag[st][i];
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) R[jb] = OUT_IN ? Ag[st][jb] : b_frag(wc * 64 + jb * 16, j0);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jb = 0; jb < 4; ++jb)
                    acc[i][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(L[i], R[jb], acc[i][jb], 0, 0, 0);
        }

        // the product into LDS in W's layout, then W + s * product per piece
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int jb = 0; jb < 4; ++jb)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    sAcc[(wr * 32 + i * 16 + (lane >> 4) * 4 + q) * MG_LDT + wc * 64 + jb * 16 + lr] = acc[i][jb][q];
        __syncthreads();
#pragma unroll
        for (int p = 0; p < MG_PIECES; ++p) {
            const Piece q = piece_of(tid, p);
            const int row = row0 + q.row, col = col0 + q.col;
            if (row >= n_rows || col >= n_cols) continue;
            const float* pr = sAcc + q.row * MG_LDT + q.col;
            union { uint4 u; bf16 e[8]; } v;
            v.u = wv[p];
#pragma unroll
            for (int e = 0; e < 8; ++e) v.e[e] = f32_to_bf16(to_f32(v.e[e]) + s * pr[e]);
            bf16* dst = W + (int64_t)row * ldw + col;
            if (col + 8 <= n_cols) {
                *(uint4*)dst = v.u;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (col + e < n_cols) dst[e] = v.e[e];
            }
        }
#pragma unroll
        for (int p = 0; p < MG_PIECES; ++p) wv[p] = wn[p];
        __syncthreads();   // sB and sAcc are rewritten for the next tile
    }
}

// Whole tiles (the stored rows a multiple of 64, the stored columns of 128)
// and 16-byte A_a and B_a pieces: the same update with no bounds branch.
// A workgroup takes a run of consecutive tiles numbered column-major, so the
// run keeps its stored columns, on which one operand depends (OUT_IN: A_a,
// whose fragments stay in registers; IN_OUT: B_a, whose staged block stays
// in LDS); the next tile's W pieces and its other operand are requested
// before the current tile is worked on.  Every load of a tile goes out
// unconditionally (ranks past r read rank 0 of their row; the values are
// masked where they are used), so the loads stay in flight together and a
// wait for one of them does not wait for the next tile's.
template <bool OUT_IN>
__global__ __launch_bounds__(MG_THREADS) __attribute__((amdgpu_waves_per_eu(3))) void k_merge_bf16_run(
    PoolDev P, int32_t adapter, float sign, bf16* __restrict__ W, int64_t ldw, int32_t tiles_r, int32_t n_tiles) {
    constexpr int NC = OUT_IN ? MG_ROWS : MG_COLS;   // c values per tile
    constexpr int NAF = OUT_IN ? 4 : 2;              // A_a fragments per rank step
    constexpr int BPR = NC / 8;                      // 16-byte pieces per B_a row
    constexpr int BPT = 64 * BPR / MG_THREADS;       // B_a pieces per thread
    __shared__ __attribute__((aligned(16))) bf16 sB[64 * NC];
    __shared__ __attribute__((aligned(16))) float sAcc[MG_ROWS * MG_LDT];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave >> 1;   // 32-row half of the tile
    const int wc = wave & 1;    // 64-column half of the tile
    const int lr = lane & 15;
    const int kq = (lane >> 4) * 8;
    const int r = uload(P.ranks, adapter);
    const float s = sign * uload(P.scales, adapter);
    const bf16* Aa = (const bf16*)P.A + uload(P.a_off, adapter);
    const bf16* Ba = (const bf16*)P.B + uload(P.b_off, adapter);
    const int d_out = P.d_out;
    const int steps = (r + 31) / 32;   // 32 ranks per MFMA step

    auto tile_at = [&](int t, int& row0, int& col0) __attribute__((always_inline)) {
        const int tc = t / tiles_r;
        row0 = (t - tc * tiles_r) * MG_ROWS;
        col0 = tc * MG_COLS;
    };
    auto load_w = [&](u32x4_t (&w)[MG_PIECES], int t) __attribute__((always_inline)) {
        int row0, col0;
        tile_at(t, row0, col0);
#pragma unroll
        for (int p = 0; p < MG_PIECES; ++p) {
            const Piece q = piece_of(tid, p);
            w[p] = *(const u32x4_t*)(W + (int64_t)(row0 + q.row) * ldw + col0 + q.col);
        }
    };
    // A_a fragments of tile t: lane l takes row/column l % 16 of its block
    // and ranks (l / 16) * 8 .. + 8 of each 32-rank step
    auto load_a = [&](bf16x8_t (&a)[2][NAF], int t) __attribute__((always_inline)) {
        int row0, col0;
        tile_at(t, row0, col0);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            if (st >= steps) break;
            const int j = st * 32 + kq;
#pragma unroll
            for (int f = 0; f < NAF; ++f) {
                const int k = OUT_IN ? col0 + wc * 64 + f * 16 + lr : row0 + wr * 32 + f * 16 + lr;
                a[st][f] = *(const bf16x8_t*)(Aa + (int64_t)k * r + (j < r ? j : 0));
            }
        }
    };
    // B_a[j][c] pieces of the tile's c range, as they lie
    auto load_b = [&](u32x4_t (&b)[BPT], int t) __attribute__((always_inline)) {
        int row0, col0;
        tile_at(t, row0, col0);
        const int c0 = OUT_IN ? row0 : col0;
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            const int idx = tid + q * MG_THREADS;
            const int j = idx / BPR;
            const int c = (idx - j * BPR) * 8;
            b[q] = *(const u32x4_t*)(Ba + (int64_t)(j < r ? j : 0) * d_out + c0 + c);
        }
    };
    // -> sB; ranks past r are 0 up to the last 32-rank step
    auto stage_b = [&](const u32x4_t (&b)[BPT]) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            const int idx = tid + q * MG_THREADS;
            const int j = idx / BPR;
            if (j >= 32 * steps) continue;
            const int c = (idx - j * BPR) * 8;
            *(u32x4_t*)(sB + mg_b_at<NC>(j, c)) = j < r ? b[q] : u32x4_t{0u, 0u, 0u, 0u};
        }
    };
    // transpose-read operand: columns cb .. cb + 15 of the staged block,
    // ranks j0 + (l / 16) * 8 .. + 8
    const int b_lane = ((lane >> 4) * 8 + (lr >> 2)) * NC + (lr & 3) * 4;
    const int b_sw = NC == 128 ? ((lr >> 2) | (((lane >> 4) & 1) << 2)) : ((lr >> 2) ^ ((lane >> 4) & 1));
    auto b_frag = [&](int cb, int j0) __attribute__((always_inline)) {
        const bf16* q = sB + b_lane + j0 * NC + (((cb >> 4) ^ b_sw) << 4);
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)q);
        const i16x4_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(q + 4 * NC));
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // the tile's product on the matrix cores into sAcc (W's layout), then
    // W + s * product per piece, rounded once.  The A_a fragments and W
    // pieces are made opaque where they are used, so that nothing derived
    // from them (and no wait for them) moves up to their loads.
    auto work_tile = [&](int row0, int col0, bf16x8_t (&a)[2][NAF], u32x4_t (&w)[MG_PIECES])
                         __attribute__((always_inline)) {
        f32x4_t acc[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) acc[i][jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            if (st >= steps) break;
            const int j0 = st * 32;
            const bool aok = j0 + kq < r;
            bf16x8_t Am[NAF];
#pragma unroll
            for (int f = 0; f < NAF; ++f) {
                bf16x8_t v = a[st][f];
                asm volatile("" : "+v"(v));
                Am[f] = aok ? v : bf16x8_t{};
            }
            bf16x8_t L[2], R[4];
#pragma unroll
            for (int i = 0; i < 2; ++i) L[i] = OUT_IN ? b_frag(wr * 32 + i * 16, j0) : Am[i % NAF];
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) R[jb] = OUT_IN ? Am[jb % NAF] : b_frag(wc * 64 + jb * 16, j0);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jb = 0; jb < 4; ++jb)
                    acc[i][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(L[i], R[jb], acc[i][jb], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int jb = 0; jb < 4; ++jb)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    sAcc[(wr * 32 + i * 16 + (lane >> 4) * 4 + q) * MG_LDT + wc * 64 + jb * 16 + lr] = acc[i][jb][q];
        __syncthreads();
#pragma unroll
        for (int p = 0; p < MG_PIECES; ++p) {
            const Piece q = piece_of(tid, p);
            const float* pr = sAcc + q.row * MG_LDT + q.col;
            union { u32x4_t u; bf16 e[8]; } v;
            v.u = w[p];
            asm volatile("" : "+v"(v.u));
#pragma unroll
            for (int e = 0; e < 8; ++e) v.e[e] = f32_to_bf16(to_f32(v.e[e]) + s * pr[e]);
            *(u32x4_t*)(W + (int64_t)(row0 + q.row) * ldw + col0 + q.col) = v.u;
        }
    };

    const int t_beg = (int)((int64_t)blockIdx.x * n_tiles / gridDim.x);
    const int t_end = (int)((int64_t)(blockIdx.x + 1) * n_tiles / gridDim.x);
    if (t_beg >= t_end) return;
    u32x4_t wv[MG_PIECES], wn[MG_PIECES];
    bf16x8_t Ag[2][NAF];
    int held = -1;   // stored columns of the operand held along the run
    if constexpr (OUT_IN) {
        u32x4_t bv[BPT], bn[BPT];
        load_w(wv, t_beg);
        load_b(bv, t_beg);
        for (int t = t_beg; t < t_end; ++t) {
            int row0, col0;
            tile_at(t, row0, col0);
            if (col0 != held) {   // the run enters other columns: their A_a fragments
                held = col0;
                load_a(Ag, t);
            }
            // the next tile (the last tile again at the end of the run: an
            // unconditional request keeps every wait count exact)
            const int tn = t + 1 < t_end ? t + 1 : t;
            load_b(bn, tn);
            load_w(wn, tn);
            stage_b(bv);
            __syncthreads();
            work_tile(row0, col0, Ag, wv);
#pragma unroll
            for (int p = 0; p < MG_PIECES; ++p) wv[p] = wn[p];
#pragma unroll
            for (int q = 0; q < BPT; ++q) bv[q] = bn[q];
            __syncthreads();   // sB and sAcc are rewritten for the next tile
        }
    } else {
        bf16x8_t An[2][NAF];
        load_w(wv, t_beg);
        load_a(Ag, t_beg);
        for (int t = t_beg; t < t_end; ++t) {
            int row0, col0;
            tile_at(t, row0, col0);
            if (col0 != held) {   // the run enters other columns: their B_a block
                held = col0;
                u32x4_t bt[BPT];
                load_b(bt, t);
                stage_b(bt);
                __syncthreads();
            }
            const int tn = t + 1 < t_end ? t + 1 : t;
            load_a(An, tn);
            load_w(wn, tn);
            work_tile(row0, col0, Ag, wv);
#pragma unroll
            for (int p = 0; p < MG_PIECES; ++p) wv[p] = wn[p];
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int f = 0; f < NAF; ++f) Ag[st][f] = An[st][f];
            __syncthreads();   // sAcc (and sB at a change of columns) is rewritten for the next tile
        }
    }
}

// fp32: each thread updates four consecutive stored elements, summing over
// the rank in order.
template <bool OUT_IN>
__global__ __launch_bounds__(256) void k_merge_f32(PoolDev P, int32_t adapter, float sign, float* __restrict__ W,
                                                   int64_t ldw) {
    const int n_rows = OUT_IN ? P.d_out : P.d_in;
    const int n_cols = OUT_IN ? P.d_in : P.d_out;
    const int per_row = (n_cols + 3) / 4;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)n_rows * per_row) return;
    const int row = (int)(idx / per_row);
    const int col = (int)(idx - (int64_t)row * per_row) * 4;
    const int r = uload(P.ranks, adapter);
    const float s = sign * uload(P.scales, adapter);
    const float* Aa = (const float*)P.A + uload(P.a_off, adapter);
    const float* Ba = (const float*)P.B + uload(P.b_off, adapter);
    const int d_out = P.d_out;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < r; ++j) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (col + e >= n_cols) break;
            // IN_OUT: element (k = row, c = col + e); OUT_IN: (k = col + e, c = row)
            const int k = OUT_IN ? col + e : row;
            const int c = OUT_IN ? row : col + e;
            acc[e] += Aa[(int64_t)k * r + j] * Ba[(int64_t)j * d_out + c];
        }
    }
    float* w = W + (int64_t)row * ldw + col;
    for (int e = 0; e < 4 && col + e < n_cols; ++e) w[e] += s * acc[e];
}

}  // namespace

hipError_t launch_merge(const PoolDev& P, lora_dtype_t dt, int32_t adapter, float sign, void* W, int64_t ldw,
                        bool out_in, hipStream_t stream) {
    const int n_rows = out_in ? P.d_out : P.d_in;
    const int n_cols = out_in ? P.d_in : P.d_out;
    if (dt == LORA_BF16) {
        // about three workgroups per CU (the LDS of one is ~52 KiB), each
        // walking its share of the tiles
        const int tiles_c = (int)ceil_div(n_cols, MG_COLS);
        const int tiles_r = (int)ceil_div(n_rows, MG_ROWS);
        const int64_t n_tiles = (int64_t)tiles_r * tiles_c;
        dim3 grid((unsigned)std::min<int64_t>(n_tiles, 768));
        // whole tiles and 16-byte A_a and B_a pieces take the branch-free kernel
        const bool whole_tiles =
            n_rows % MG_ROWS == 0 && n_cols % MG_COLS == 0 && P.vec_a && P.vec_b && P.vec_rank;
        if (whole_tiles) {
            if (out_in)
                hipLaunchKernelGGL(k_merge_bf16_run<true>, grid, dim3(MG_THREADS), 0, stream, P, adapter, sign,
                                   (bf16*)W, ldw, tiles_r, (int32_t)n_tiles);
            else
                hipLaunchKernelGGL(k_merge_bf16_run<false>, grid, dim3(MG_THREADS), 0, stream, P, adapter, sign,
                                   (bf16*)W, ldw, tiles_r, (int32_t)n_tiles);
        } else if (out_in)
            hipLaunchKernelGGL(k_merge_bf16<true>, grid, dim3(MG_THREADS), 0, stream, P, adapter, sign, (bf16*)W,
                               ldw, tiles_c, (int32_t)n_tiles);
        else
            hipLaunchKernelGGL(k_merge_bf16<false>, grid, dim3(MG_THREADS), 0, stream, P, adapter, sign, (bf16*)W,
                               ldw, tiles_c, (int32_t)n_tiles);
    } else {
        dim3 grid((unsigned)ceil_div((int64_t)n_rows * ceil_div(n_cols, 4), 256));
        if (out_in)
            hipLaunchKernelGGL(k_merge_f32<true>, grid, dim3(256), 0, stream, P, adapter, sign, (float*)W, ldw);
        else
            hipLaunchKernelGGL(k_merge_f32<false>, grid, dim3(256), 0, stream, P, adapter, sign, (float*)W, ldw);
    }
    return hipGetLastError();
}

}  // namespace lora
