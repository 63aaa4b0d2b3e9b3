// Batches of a few hundred rows: the base product x W, and the adapter term
// grouped by adapter, in three launches.
//
// At a few hundred rows x W does about as many flops per byte of W as the
// matrix cores deliver per byte of HBM bandwidth (256 rows: 256 flop/byte
// against a ridge near 310), so the product has to keep the matrix cores and
// the memory pipeline of every CU busy at once.  A CU's vector-memory path
// (about 64 bytes a clock) is then the tightest limit, so the tile is chosen
// for the bytes it moves per MFMA, and the launch is cut into enough
// independent tiles (row tiles, column tiles, K slices) to cover every CU:
//
//   k_rows_gemm_x tile = 128 rows x 64 columns (4 waves) or 256 x 128 (8
//                 waves) x one K slice; wave w owns rows 32w .. 32w + 31 and
//                 all the tile's columns.  x and W blocks are loaded in whole
//                 lines, four blocks ahead in registers, and go through LDS
//                 to the matrix cores; W comes from HBM and is read once per
//                 row tile, x stays in L2.  Writes fp32 partial sums
//                 part[slice][row][col].
//                 A 4-bit W (signed nibbles, one fp32 scale per output and
//                 128 inputs) is widened exactly to bf16 on its way into LDS;
//                 a 128-deep block is one scale group, so each block's sums
//                 are scaled once and added ("Serving Many LoRA Adapters"
//                 (praveentn.live), section "When It Falls Down": a 4-bit base
//                 with BF16 adapters).
//
// The adapter term costs the reads of each distinct adapter's A and B
// ("Serving many LoRA adapters" (blog.ecitis.org), section "Batching across
// different adapters").  With skewed ids a row-by-row gather reads a popular
// adapter once per row, so the shrink and the expand run over the segments
// of lora_segments_build (rows grouped by adapter id, "Serving multiple
// LoRAs: segmented matrix multiplies and adapter scheduling", section "Not
// merging the weights, computing in batches"), and each segment tile reads
// its adapter's slice once:
//
//   k_seg_shrink  (segment tile of 16 rows, K slice): t partials = x_rows A_u
//                 on the matrix cores, A_u's slice transposed into LDS; slice
//                 0 also writes each row's record (B offset, rank, scale).
//   k_seg_finish  (one wave per row and 256 columns): y = sum of the base
//                 partials in slice order + s_u * (t summed in slice order)
//                 B_u, rounded once; base-only rows get the base alone.  The
//                 partials need only the row, so they are requested at once;
//                 B follows the row's record.  A column chunk always runs on
//                 one XCD, so the rows of a popular adapter read its B piece
//                 from that XCD's L2.
//
// Every sum runs in a fixed order, so results do not depend on timing.
#include "lora_internal.hpp"

namespace lora {
namespace {

constexpr int RG_KB = 128;            // K slices are whole 128-deep groups (the 4-bit scale group)

struct RowsGemmArgs {
    const bf16* x;
    int64_t ldx;
    const void* W;        // bf16 [N][ldw] elements, or 4-bit bytes [N][ldw]
    int64_t ldw;
    const float* wscale;  // 4-bit: [N][lds]
    int64_t lds;
    float* part;          // [S][M][ldp]
    int64_t ldp;
    int32_t M, N, K;
    int32_t tiles_m, tiles_n, S, kslice;
};

// Workgroup b -> logical tile.  Consecutive workgroups are dispatched to
// different XCDs (b % 8), so each XCD is given a contiguous run of logical
// tiles: the row tiles of one column tile (which read the same W block) and
// neighbouring column tiles (which read the same x slice) share its L2.
__device__ __forceinline__ int xcd_tile(int b, int G) {
    const int q = G >> 3, rem = G & 7;
    const int xc = b & 7, local = b >> 3;
    return xc * q + min(xc, rem) + local;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Eight signed 4-bit values (element e in bits 4e .. 4e+3) as exact bf16.
__device__ __forceinline__ u32x4 widen8_q4(uint32_t w) {
    union { u32x4 v; bf16 e[8]; } u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int q = ((int)(w << (28 - 4 * e))) >> 28;
        u.e[e] = (bf16)(__float_as_uint((float)q) >> 16);
    }
    return u.v;
}

// The same tile with x staged through LDS as well.  A wave's MFMA operand
// holds 16 rows x 8 k per load, so x fragments loaded straight from memory
// touch 16 rows (half a 128-byte line each) per instruction; on L2-resident
// data that pattern measured 2.8x slower than whole-line loads, and x is
// most of what a few-hundred-row tile reads (it is re-read once per column
// tile).  Here x and W blocks (KB k) are loaded in whole lines (a wave's
// load: rows or columns x 128 bytes) into a RING_X-deep register ring,
// stored to double-buffered LDS (pitch KB + 8: the fragment reads of 16 rows
// hit distinct banks), and the MFMAs read both from LDS.  Q4: a block is one
// 128-input scale group; its 4-bit W (16 bytes = 32 inputs of one column a
// piece) is widened exactly to bf16 on its way into LDS, and the block's
// sums are scaled once per column and added.
constexpr int RING_X = 4;

template <bool Q4, int NW, int BN, int KB>
__global__ __launch_bounds__(NW * 64) void k_rows_gemm_x(RowsGemmArgs a) {
    constexpr int BM = 32 * NW;
    constexpr int NT = NW * 64;
    constexpr int NB = BN / 16;
    constexpr int LDK = KB + 8;
    constexpr int PPR = KB / 8;                              // 16-byte bf16 pieces per row of a block
    constexpr int XPT = BM * PPR / NT;                       // x pieces per thread per block
    constexpr int WPR = Q4 ? KB / 32 : PPR;                  // 16-byte W pieces per column of a block
    constexpr int WPT = BN * WPR / NT;                       // W pieces per thread per block
    static_assert(XPT * NT == BM * PPR && WPT * NT == BN * WPR && WPT >= 1, "blocks do not split evenly");
    static_assert(!Q4 || (KB == 128 && WPT == 1), "4-bit blocks: one scale group, one piece per thread");
    __shared__ __attribute__((aligned(16))) bf16 sX[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) bf16 sW[2][BN * LDK];
    __shared__ float sSc[2][Q4 ? BN : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lr = lane & 15;
    const int kq = (lane >> 4) * 8;
    const int G = a.tiles_m * a.tiles_n * a.S;
    const int L = xcd_tile(blockIdx.x, G);
    const int tm = L % a.tiles_m;
    const int rest = L / a.tiles_m;
    const int tn = rest % a.tiles_n;
    const int ks = rest / a.tiles_n;
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int kbeg = ks * a.kslice;
    const int klen = min(a.K, kbeg + a.kslice) - kbeg;

    // piece v = tid + NT p: row (column) v / PPR (v / WPR), piece v % PPR
    // (v % WPR); rows past M and columns past N read the last one (never
    // stored)
    const bf16* xp[XPT];
    const uint8_t* wp[WPT];
    const float* scp = nullptr;
#pragma unroll
    for (int p = 0; p < XPT; ++p) {
        const int v = tid + NT * p;
        xp[p] = a.x + (int64_t)min(m0 + v / PPR, a.M - 1) * a.ldx + kbeg + (v % PPR) * 8;
    }
#pragma unroll
    for (int p = 0; p < WPT; ++p) {
        const int v = tid + NT * p;
        const int n = min(n0 + v / WPR, a.N - 1);
        if constexpr (Q4) wp[p] = (const uint8_t*)a.W + (int64_t)n * a.ldw + kbeg / 2 + (v % WPR) * 16;
        else wp[p] = (const uint8_t*)((const bf16*)a.W + (int64_t)n * a.ldw + kbeg + (v % WPR) * 8);
    }
    if constexpr (Q4) scp = a.wscale + (int64_t)min(n0 + tid / WPR, a.N - 1) * a.lds + kbeg / KB;

    const int nfull = klen / KB;
    // the register ring, as separate named arrays so that every index is static
    u32x4 x0[XPT], x1[XPT], x2[XPT], x3[XPT];
    u32x4 w0[WPT], w1[WPT], w2[WPT], w3[WPT];
    float c0 = 0.f, c1 = 0.f, c2 = 0.f, c3 = 0.f;
    f32x4_t acc[2][NB];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto load = [&](u32x4 (&dx)[XPT], u32x4 (&dw)[WPT], float& sc, int kb) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < XPT; ++p) dx[p] = *(const u32x4*)(xp[p] + kb * KB);
#pragma unroll
        for (int p = 0; p < WPT; ++p) dw[p] = *(const u32x4*)(wp[p] + (Q4 ? kb * KB / 2 : kb * KB * 2));
        if constexpr (Q4) sc = scp[kb];
    };
    auto store = [&](const u32x4 (&dx)[XPT], const u32x4 (&dw)[WPT], float sc, int stage)
                     __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < XPT; ++p) {
            const int v = tid + NT * p;
            *(u32x4*)(sX[stage] + (v / PPR) * LDK + (v % PPR) * 8) = dx[p];
        }
#pragma unroll
        for (int p = 0; p < WPT; ++p) {
            const int v = tid + NT * p;
            if constexpr (Q4) {
                bf16* d = sW[stage] + (v / WPR) * LDK + (v % WPR) * 32;
#pragma unroll
                for (int h = 0; h < 4; ++h) *(u32x4*)(d + h * 8) = widen8_q4(dw[p][h]);
                if (v % WPR == 0) sSc[stage][v / WPR] = sc;
            } else {
                *(u32x4*)(sW[stage] + (v / WPR) * LDK + (v % WPR) * 8) = dw[p];
            }
        }
    };
    auto mma = [&](int stage) __attribute__((always_inline)) {
        const bf16* sx = sX[stage] + (wave * 32 + lr) * LDK + kq;
        const bf16* sw = sW[stage] + lr * LDK + kq;
        f32x4_t g[2][NB];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) g[i][j] = Q4 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc[i][j];
#pragma unroll
        for (int st = 0; st < KB / 32; ++st) {
            bf16x8_t xa[2], b[NB];
#pragma unroll
            for (int i = 0; i < 2; ++i) xa[i] = *(const bf16x8_t*)(sx + i * 16 * LDK + st * 32);
#pragma unroll
            for (int j = 0; j < NB; ++j) b[j] = *(const bf16x8_t*)(sw + j * 16 * LDK + st * 32);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    g[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[i], b[j], g[i][j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            if constexpr (Q4) {
                const float sc = sSc[stage][j * 16 + lr];
#pragma unroll
                for (int i = 0; i < 2; ++i) acc[i][j] += sc * g[i][j];
            } else {
#pragma unroll
                for (int i = 0; i < 2; ++i) acc[i][j] = g[i][j];
            }
        }
    };
    // One block: registers -> LDS stage kb & 1 (last read by block kb - 2,
    // whose MFMAs every wave finished before the barrier of block kb - 1),
    // then block kb + RING_X is requested into the freed registers, then the
    // MFMAs.  Requests past the last whole block fetch that block again (from
    // cache, never used), so the loop has no branch around its loads.
#define RX_STEP(X_, W_, C_, KB_)                         \
    {                                                    \
        const int kb_ = (KB_);                           \
        store(X_, W_, C_, kb_ & 1);                      \
        __syncthreads();                                 \
        load(X_, W_, C_, min(kb_ + RING_X, last));       \
        mma(kb_ & 1);                                    \
    }
    if (nfull > 0) {
        const int last = nfull - 1;
        load(x0, w0, c0, 0);
        load(x1, w1, c1, min(1, last));
        load(x2, w2, c2, min(2, last));
        load(x3, w3, c3, min(3, last));
        int kb = 0;
        for (; kb + RING_X <= nfull; kb += RING_X) {
            RX_STEP(x0, w0, c0, kb);
            RX_STEP(x1, w1, c1, kb + 1);
            RX_STEP(x2, w2, c2, kb + 2);
            RX_STEP(x3, w3, c3, kb + 3);
        }
        if (kb < nfull) RX_STEP(x0, w0, c0, kb);
        if (kb + 1 < nfull) RX_STEP(x1, w1, c1, kb + 1);
        if (kb + 2 < nfull) RX_STEP(x2, w2, c2, kb + 2);
    }
#undef RX_STEP
    if (!Q4 && klen > nfull * KB) {
        // ragged last block (bf16 W only; a 4-bit K is whole blocks):
        // element-wise loads, zero past the slice
        const int k0 = nfull * KB;
#pragma unroll
        for (int p = 0; p < XPT; ++p) {
            const int v = tid + NT * p;
            const int valid = min(8, max(0, klen - k0 - (v % PPR) * 8));
            x0[p] = __builtin_bit_cast(u32x4, ld8_guard(xp[p] + k0, valid));
        }
#pragma unroll
        for (int p = 0; p < WPT; ++p) {
            const int v = tid + NT * p;
            const int valid = min(8, max(0, klen - k0 - (v % PPR) * 8));
            w0[p] = __builtin_bit_cast(u32x4, ld8_guard((const bf16*)wp[p] + k0, valid));
        }
        store(x0, w0, 0.f, nfull & 1);
        __syncthreads();
        mma(nfull & 1);
    }

    // partial sums: lane l holds rows (l / 16) * 4 + q of column l % 16 of
    // each 16 x 16 block
    float* out = a.part + (int64_t)ks * a.M * a.ldp;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int n = n0 + j * 16 + lr;
            if (n >= a.N) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = m0 + wave * 32 + i * 16 + (lane >> 4) * 4 + q;
                if (m < a.M) out[(int64_t)m * a.ldp + n] = acc[i][j][q];
            }
        }
}

// ---------------------------------------------------------------------------
// Shrink over segment tiles
// ---------------------------------------------------------------------------

constexpr int SS_ROWS = 16;    // rows per segment tile (one MFMA block)
constexpr int SS_NT = 256;
constexpr int SS_MAX_LDS = 40 * 1024;   // transposed A staging (four workgroups per CU)
constexpr int SS_LB = 8;       // 16-byte pieces of x and of A per thread per staging batch
constexpr int SS_MU = 4;       // k-steps per wave whose LDS fragments are read together
constexpr int SS_XS = 8;       // x fragments per lane: a slice of at most 32 k-steps over 4 waves

struct SegShrinkArgs {
    RowRec* recs;      // [M], the finish's record of each row (slice 0 writes it)
    const int32_t* ids;
    const bf16* x;
    int64_t ldx;
    const int32_t* perm;
    const int32_t* seg_ids;
    const int32_t* seg_off;
    const int32_t* n_seg;
    int32_t cap;       // capacity of the descriptor (>= its run count)
    float* tpart;      // [St][M][rtp]
    int64_t rtp;
    int32_t M;
    int32_t ks_len;    // k per slice (multiple of 128)
    int32_t kp;        // LDS pitch (bf16) of a staged row: ks_len + 8
    int32_t St;        // K slices
};

// Stores one batch of A pieces (16 bytes: 8 ranks of one k-row) transposed,
// sA[j][k]; pieces past the slice are 0.
__device__ __forceinline__ void stage_a(const u32x4 (&av)[SS_LB], const bool (&aok)[SS_LB], int b0, int tid, int G,
                                        int na, int KP, bf16* sA) {
#pragma unroll
    for (int q = 0; q < SS_LB; ++q) {
        const int v = b0 + q * SS_NT + tid;
        if (v < na) {
            const int k = v / G;
            const int j0 = (v - k * G) * 8;
            union { u32x4 q4; bf16 e[8]; } w;
            w.q4 = aok[q] ? av[q] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e) sA[(j0 + e) * KP + k] = w.e[e];
        }
    }
}

// The shrink's matrix-core phase: wave w takes k-steps w, w + 4, ... of the
// slice (nsteps a multiple of 4, at most 4 SS_XS); its x fragments are in
// registers, and the A fragments of SS_MU steps are read from LDS before
// their MFMAs, so a round costs one LDS round trip (one step at a time, the
// eight steps of a 1024-deep slice took 1.6 us).  acc[jb] = x rows x ranks
// 16 jb .. 16 jb + 15.
template <int RB>
__device__ __forceinline__ void shrink_mma(const u32x4 (&xf)[SS_XS], const bool (&xok)[SS_XS], const bf16* sA,
                                           int KP, int nsteps, int wave, int lane, f32x4_t (&acc)[4]) {
    const int lr = lane & 15;
    const int kq = (lane >> 4) * 8;
#pragma unroll
    for (int q0 = 0; q0 < SS_XS; q0 += SS_MU) {
        if (wave + 4 * q0 >= nsteps) break;
        bf16x8_t xa[SS_MU], bb[SS_MU][RB];
#pragma unroll
        for (int q = 0; q < SS_MU; ++q) {
            const int st = wave + 4 * (q0 + q);
            const int sr = st < nsteps ? st : wave;   // past the slice: read a valid step (x is 0 there)
#pragma unroll
            for (int jb = 0; jb < RB; ++jb) bb[q][jb] = *(const bf16x8_t*)(sA + (jb * 16 + lr) * KP + sr * 32 + kq);
            xa[q] = __builtin_bit_cast(bf16x8_t, xok[q0 + q] ? xf[q0 + q] : u32x4{0u, 0u, 0u, 0u});
        }
#pragma unroll
        for (int q = 0; q < SS_MU; ++q)
#pragma unroll
            for (int jb = 0; jb < RB; ++jb)
                acc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[q], bb[q][jb], acc[jb], 0, 0, 0);
    }
}

// The shrink of one segment tile (from sInfo) over K slice ks.
__device__ __forceinline__ void shrink_task(const PoolDev& P, const SegShrinkArgs& a, int ks, const int* sInfo,
                                            int* sRow, uint8_t* smem, int tid, int lane, int wave) {
    // tile-uniform values, read from LDS by every lane: made visibly uniform
    // so that the pool tables come through scalar loads
    const int u = __builtin_amdgcn_readfirstlane(sInfo[1]);
    const bool ok = id_ok(u, P.n_adapters);
    const int row0 = __builtin_amdgcn_readfirstlane(sInfo[2]);
    const int cnt = min(SS_ROWS, __builtin_amdgcn_readfirstlane(sInfo[3]) - row0);
    const int r = ok ? (P.uniform ? P.r_max : uload(P.ranks, u)) : 0;
    const int64_t aoff = ok ? (P.uniform ? (int64_t)u * P.d_in * P.r_max : uload(P.a_off, u)) : 0;
    if (ks == 0 && tid < cnt) {
        // the finish's record of the row: B offset, rank (0: no term), scale
        const int row = a.perm[row0 + tid];
        RowRec rec;
        rec.b_off = ok ? P.b_off[u] : 0;
        rec.rank = r;
        rec.scale = ok ? P.scales[u] : 0.f;
        a.recs[row] = rec;
        if (!ok && a.ids[row] != -1) flag_bad_id(P.err);   // invalid ids run as base-only rows
    }
    if (!ok) return;   // base-only rows (and invalid ids): no t
    const int RB = (r + 15) / 16;   // 16-rank blocks
    const int kbeg = ks * a.ks_len;
    const int klen = min(P.d_in, kbeg + a.ks_len) - kbeg;
    const int KP = a.kp;
    bf16* sA = (bf16*)smem;   // [RB * 16][KP], A_u's slice transposed
    const bf16* Au = (const bf16*)P.A + aoff + (int64_t)kbeg * r;
    const bool va = P.vec_a && r % 8 == 0;
    const int G = va ? r / 8 : 1;
    const int na = va ? a.ks_len * G : 0;

    // Requests in dependency order, none waiting on a later one: the tile
    // row of this lane's x fragments (perm), the first SS_LB 16-byte A
    // pieces per thread (all of a rank-16 slice), then, once perm is in, the
    // x fragments of this wave's k-steps.  The loads carry no branch (out-of-
    // range pieces read a valid address and are masked), so all stay in
    // flight.  x is not staged: lane l of wave w holds row l % 16 of the tile
    // at k-group (l / 16) * 8 of steps w, w + 4, ... in registers, which is
    // the matrix cores' operand layout, and LDS holds A alone (four
    // workgroups per CU).
    const int lr = lane & 15;
    const int kq = (lane >> 4) * 8;
    const int xrow = lr < cnt ? a.perm[row0 + lr] : -1;
    u32x4 av[SS_LB];
    bool aok[SS_LB];
#pragma unroll
    for (int q = 0; q < SS_LB; ++q) {
        const int v = q * SS_NT + tid;
        const int ka = v / G;
        aok[q] = v < na && ka < klen;
        av[q] = *(const u32x4*)(aok[q] ? Au + (int64_t)ka * r + (v - ka * G) * 8 : Au);
    }
    const int nsteps = a.ks_len / 32;
    u32x4 xf[SS_XS];
    bool xok[SS_XS];
#pragma unroll
    for (int q = 0; q < SS_XS; ++q) {
        const int k = (wave + 4 * q) * 32 + kq;
        xok[q] = xrow >= 0 && k + 8 <= klen;   // also false past the slice's steps
        xf[q] = *(const u32x4*)(xok[q] ? a.x + (int64_t)xrow * a.ldx + kbeg + k : a.x);
    }
    if (klen % 8) {   // the piece cut by the end of the slice (d_in not a multiple of 8)
        const int k = klen / 8 * 8;
#pragma unroll
        for (int q = 0; q < SS_XS; ++q)
            if (xrow >= 0 && (wave + 4 * q) * 32 + kq == k) {
                xf[q] = __builtin_bit_cast(u32x4, ld8_guard(a.x + (int64_t)xrow * a.ldx + kbeg + k, klen - k));
                xok[q] = true;
            }
    }
    stage_a(av, aok, 0, tid, G, na, KP, sA);
    for (int b0 = SS_NT * SS_LB; b0 < na; b0 += SS_NT * SS_LB) {   // ranks above 16
#pragma unroll
        for (int q = 0; q < SS_LB; ++q) {
            const int v = b0 + q * SS_NT + tid;
            const int ka = v / G;
            aok[q] = v < na && ka < klen;
            av[q] = *(const u32x4*)(aok[q] ? Au + (int64_t)ka * r + (v - ka * G) * 8 : Au);
        }
        stage_a(av, aok, b0, tid, G, na, KP, sA);
    }
    if (va) {   // ranks r .. 16 RB - 1 are 0
        for (int v = tid; v < (RB * 16 - r) * a.ks_len; v += SS_NT) {
            const int j = r + v / a.ks_len;
            sA[j * KP + v % a.ks_len] = 0;
        }
    } else {
        for (int v = tid; v < RB * 16 * a.ks_len; v += SS_NT) {
            const int k = v / (RB * 16);
            const int j = v - k * (RB * 16);
            sA[j * KP + k] = (j < r && k < klen) ? Au[(int64_t)k * r + j] : (bf16)0;
        }
    }
    if (tid < SS_ROWS) sRow[tid] = tid < cnt ? a.perm[row0 + tid] : -1;
    __syncthreads();

    f32x4_t acc[4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) acc[jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    switch (RB) {
        case 1: shrink_mma<1>(xf, xok, sA, KP, nsteps, wave, lane, acc); break;
        case 2: shrink_mma<2>(xf, xok, sA, KP, nsteps, wave, lane, acc); break;
        case 3: shrink_mma<3>(xf, xok, sA, KP, nsteps, wave, lane, acc); break;
        default: shrink_mma<4>(xf, xok, sA, KP, nsteps, wave, lane, acc); break;
    }
    __syncthreads();   // staging no longer read: reuse it for the wave sums
    float* red = (float*)smem;   // [4][16][64]
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
        if (jb < RB)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                red[(wave * SS_ROWS + (lane >> 4) * 4 + q) * 64 + jb * 16 + (lane & 15)] = acc[jb][q];
    __syncthreads();
    for (int v = tid; v < SS_ROWS * 64; v += SS_NT) {
        const int m = v >> 6;
        const int j = v & 63;
        if (m >= cnt || j >= r) continue;
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) t += red[(w * SS_ROWS + m) * 64 + j];
        a.tpart[((int64_t)ks * a.M + sRow[m]) * a.rtp + j] = t;
    }
}


// Workgroup b: tile b / St, K slice b % St (tile-major, so that every real
// tile is dispatched before the empty ones: the grid is sized without the
// run count, and in slice-major order the empty tiles held LDS slots that
// real ones waited for).
__global__ __launch_bounds__(SS_NT) void k_seg_shrink(PoolDev P, SegShrinkArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ int sRow[SS_ROWS];
    __shared__ int sInfo[4];
    __shared__ SegTileCache C;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n_seg = seg_tile_cache_load(a.seg_off, a.seg_ids, a.n_seg, a.cap, tid, SS_NT, C);
    __syncthreads();
    if (wave == 0) {
        int s = 0, c = 0, lo = 0, hi = 0, u = -1;
        const bool found = seg_tile_find(C, n_seg, a.seg_off, a.seg_ids, SS_ROWS, blockIdx.x / a.St, lane, s, c, lo,
                                         hi, u);
        if (lane == 0) {
            sInfo[0] = found ? 1 : 0;
            sInfo[1] = u;
            sInfo[2] = lo + c * SS_ROWS;
            sInfo[3] = hi;
        }
    }
    __syncthreads();
    if (!sInfo[0]) return;   // past the last tile
    shrink_task(P, a, blockIdx.x % a.St, sInfo, sRow, smem, tid, lane, wave);
}

// ---------------------------------------------------------------------------
// Finish over segment tiles: partial sums + scaled expand, y rounded once
// ---------------------------------------------------------------------------

constexpr int FS_NT = 256;             // 4 waves, one row each
constexpr int FS_VE = 4;               // columns per lane
constexpr int FS_COLS = 64 * FS_VE;    // columns per wave
constexpr int FS_RC = 16;              // rank rows of B requested together
constexpr int FS_TB = 16;              // shrink slices of t requested together

struct SegFinishArgs {
    const RowRec* recs;   // [M]
    const float* part;    // [S][M][ldp], ldp a multiple of 4
    int64_t ldp;
    int32_t S;
    const float* tpart;   // [St][M][rtp]
    int64_t rtp;
    int32_t St;
    int32_t M;
    int32_t n_chunks;     // column chunks of FS_COLS
    void* y;
    int64_t ldy;
};

// Wave (row i, FS_COLS columns), lane l: columns c .. c + 3 (c = chunk *
// FS_COLS + 4 l) and, for the expand, rank column j = l of t.  Everything but
// B is addressed by the row alone, so the row's record (scalar loads), its
// base partials (all SB >= S slices; slices past S are clamped and masked),
// and t's first FS_TB shrink slices go out together, with no branch between
// them; B's r rows follow the record.  Rows run in the caller's order (rows
// in adapter order, so that neighbouring waves share B, measured 10-20%
// slower on the 14336-column projections).  t_j is summed in slice order in lane
// j and read by every lane with readlane.  VEC: d_out % 8 == 0 and 16-byte
// B blocks (y and ldy are 16-byte aligned at the API), so every lane's four
// columns are whole; otherwise each element is read on its own.
template <typename TY, int SB, bool VEC>
__global__ __launch_bounds__(FS_NT) void k_seg_finish(PoolDev P, SegFinishArgs a) {
    const int lane = threadIdx.x & 63;
    const int rg = blockIdx.x / a.n_chunks;
    const int ch = blockIdx.x - rg * a.n_chunks;
    // the wave's row, made visibly uniform so that its record comes through
    // scalar loads
    const int i = __builtin_amdgcn_readfirstlane(rg * (FS_NT / 64) + (int)(threadIdx.x >> 6));
    if (i >= a.M) return;   // whole waves
    const int N = P.d_out;
    const int col = ch * FS_COLS + lane * FS_VE;
    const int cc = col < N ? col : 0;   // lanes past d_out read column 0; nothing is stored
    const RowRec* rp = a.recs + i;
    const int r = uload(&rp->rank, 0);
    const int64_t boff = uload(&rp->b_off, 0);
    const float sc = uload(&rp->scale, 0);

    const int64_t slice = (int64_t)a.M * a.ldp;
    const float* __restrict__ prow = a.part + (int64_t)i * a.ldp + cc;
    float pv[SB][FS_VE];
#pragma unroll
    for (int k = 0; k < SB; ++k) {
        const float* q = prow + (int64_t)min(k, a.S - 1) * slice;
        if constexpr (VEC) {
            const float4 f = *(const float4*)q;
            pv[k][0] = f.x; pv[k][1] = f.y; pv[k][2] = f.z; pv[k][3] = f.w;
        } else {
#pragma unroll
            for (int e = 0; e < FS_VE; ++e) pv[k][e] = q[cc + e < N ? e : 0];
        }
    }
    const int64_t tsl = (int64_t)a.M * a.rtp;
    const float* __restrict__ trow = a.tpart + (int64_t)i * a.rtp + min(lane, (int)a.rtp - 1);
    float tq[FS_TB];
#pragma unroll
    for (int q = 0; q < FS_TB; ++q) tq[q] = trow[(int64_t)min(q, a.St - 1) * tsl];

    // B rows j0 .. j0 + FS_RC - 1 of the lane's columns (rows past r read
    // row r - 1 again; they meet t = 0); rows without a term skip B
    const int rr = max(r, 1);
    const bf16* __restrict__ Bu = (const bf16*)P.B + boff + cc;
    uint2 bv[FS_RC];
    auto load_b = [&](int j0) {
#pragma unroll
        for (int q = 0; q < FS_RC; ++q) {
            const bf16* src = Bu + (int64_t)min(j0 + q, rr - 1) * N;
            if constexpr (VEC) {
                bv[q] = *(const uint2*)src;
            } else {
                union { uint2 u; bf16 e[4]; } w;
#pragma unroll
                for (int e = 0; e < FS_VE; ++e) w.e[e] = src[cc + e < N ? e : 0];
                bv[q] = w.u;
            }
        }
    };
    if (r > 0) load_b(0);

    float t = 0.f;
#pragma unroll
    for (int q = 0; q < FS_TB; ++q) t += (q < a.St) ? tq[q] : 0.f;
    for (int k0 = FS_TB; k0 < a.St; k0 += FS_TB) {
#pragma unroll
        for (int q = 0; q < FS_TB; ++q) tq[q] = trow[(int64_t)min(k0 + q, a.St - 1) * tsl];
#pragma unroll
        for (int q = 0; q < FS_TB; ++q) t += (k0 + q < a.St) ? tq[q] : 0.f;
    }

    float v[FS_VE];
#pragma unroll
    for (int e = 0; e < FS_VE; ++e) v[e] = 0.f;
#pragma unroll
    for (int k = 0; k < SB; ++k)
        if (k < a.S)
#pragma unroll
            for (int e = 0; e < FS_VE; ++e) v[e] += pv[k][e];

    float ex[FS_VE];
#pragma unroll
    for (int e = 0; e < FS_VE; ++e) ex[e] = 0.f;
    for (int j0 = 0; r > 0;) {
#pragma unroll
        for (int q = 0; q < FS_RC; ++q) {
            const int j = j0 + q;
            const float tj = (j < r) ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), j)) : 0.f;
            union { uint2 u; bf16 e[4]; } w;
            w.u = bv[q];
#pragma unroll
            for (int e = 0; e < FS_VE; ++e) ex[e] += tj * to_f32(w.e[e]);
        }
        j0 += FS_RC;
        if (j0 >= r) break;
        load_b(j0);
    }
    if (col >= N) return;
    TY* yr = (TY*)a.y + (int64_t)i * a.ldy + col;
    float o[FS_VE];
#pragma unroll
    for (int e = 0; e < FS_VE; ++e) o[e] = v[e] + sc * ex[e];
    if constexpr (VEC) {
        if constexpr (sizeof(TY) == 2) {
            union { uint2 u; bf16 e[4]; } w;
#pragma unroll
            for (int e = 0; e < FS_VE; ++e) w.e[e] = f32_to_bf16(o[e]);
            *(uint2*)yr = w.u;
        } else {
            *(float4*)yr = make_float4(o[0], o[1], o[2], o[3]);
        }
    } else {
        for (int e = 0; e < FS_VE && col + e < N; ++e) yr[e] = from_f32<TY>(o[e]);
    }
}

// segment tiles of SS_ROWS rows: at most one partial tile per segment on top
// of the full ones (the grid is sized without reading the segment count)
int64_t rows_tiles(int32_t n_rows, int32_t n_bins) {
    return ceil_div(n_rows, SS_ROWS) + std::min<int64_t>(n_rows, n_bins);
}

}  // namespace

RowsPlan plan_rows(const PoolDev& P, int32_t n_rows, bool q4) {
    RowsPlan R;
    const int K = P.d_in, N = P.d_out;
    // long or wide projections: 256 x 128 tiles (x re-read once per 128
    // columns, W once per 256 rows; split K covers the CUs); the others
    // 128 x 64 tiles, for more workgroups.  On the skewed 256-row 8B batch
    // the 4096 x 4096 projections were slower with 256 x 128 or 256 x 64
    // tiles (their fp32 partials grow with the split) and with eight waves
    // and a deeper register ring on 128 x 64.
    R.shape = (!q4 && (N >= 8192 || K >= 8192)) ? 1 : 0;   // 4-bit W: 128 x 64 tiles
    const int bm = R.shape ? 256 : 128, bn = R.shape ? 128 : 64;
    R.tiles_m = (int32_t)ceil_div(n_rows, bm);
    R.tiles_n = (int32_t)ceil_div(N, bn);
    // split K (into at most 8 slices) until the launch covers the CUs
    const int kblocks = (int)ceil_div(K, RG_KB);
    int S = 1;
    while ((int64_t)R.tiles_m * R.tiles_n * S < 200 && kblocks / (2 * S) >= 4 && S < 8) S *= 2;
    R.kslice = (int32_t)(ceil_div(kblocks, S) * RG_KB);
    R.S = (int32_t)ceil_div(K, R.kslice);
    R.ldp = (int64_t)align_up((size_t)N, 4);
    // shrink: K slices sized so that the transposed A fits the LDS budget
    const int rb = (int)ceil_div(P.r_max, 16) * 16;
    // (1024-deep slices also for long K: the launch rate of workgroups,
    // about 190 per us, bounds a grid of thousands)
    int ks_len = 1024;
    while (ks_len > 128 && rb * (ks_len + 8) * 2 > SS_MAX_LDS) ks_len /= 2;
    R.ks_len = ks_len;
    R.St = (int32_t)ceil_div(K, ks_len);
    R.rtp = (int64_t)align_up((size_t)P.r_max, 4);
    const size_t part = align_up((size_t)R.S * n_rows * R.ldp * 4, 256);
    const size_t tpart = align_up((size_t)R.St * n_rows * R.rtp * 4, 256);
    const size_t recs = align_up((size_t)n_rows * sizeof(RowRec), 256);   // the finish's row records
    R.part_off = 0;
    R.tpart_off = part;
    R.recs_off = part + tpart;
    R.bytes = part + tpart + recs;
    return R;
}

hipError_t launch_rows_gemm(const PoolDev& P, const RowsPlan& R, const void* x, int64_t ldx, const void* W,
                            int64_t ldw, const float* wscale, int64_t lds, bool q4, int32_t n_rows, float* part,
                            hipStream_t stream) {
    RowsGemmArgs a;
    a.x = (const bf16*)x;
    a.ldx = ldx;
    a.W = W;
    a.ldw = ldw;
    a.wscale = wscale;
    a.lds = lds;
    a.part = part;
    a.ldp = R.ldp;
    a.M = n_rows;
    a.N = P.d_out;
    a.K = P.d_in;
    a.tiles_m = R.tiles_m;
    a.tiles_n = R.tiles_n;
    a.S = R.S;
    a.kslice = R.kslice;
    dim3 grid((unsigned)(R.tiles_m * R.tiles_n * R.S));
    if (q4) hipLaunchKernelGGL((k_rows_gemm_x<true, 4, 64, 128>), grid, dim3(256), 0, stream, a);
    else if (R.shape == 1) hipLaunchKernelGGL((k_rows_gemm_x<false, 8, 128, 64>), grid, dim3(512), 0, stream, a);
    else hipLaunchKernelGGL((k_rows_gemm_x<false, 4, 64, 64>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_rows_adapter(const PoolDev& P, const RowsPlan& R, const void* x, int64_t ldx,
                               const int32_t* ids, const lora_segments_t* seg, int32_t n_rows,
                               const float* part, float* tpart, void* y, lora_dtype_t ydt, int64_t ldy,
                               hipStream_t stream, bool shrink, bool finish) {
    const int n_bins = P.n_adapters + 1;
    // the row records follow the t partials (RowsPlan::recs_off)
    RowRec* recs = (RowRec*)((uint8_t*)tpart + (R.recs_off - R.tpart_off));
    if (shrink) {
        SegShrinkArgs s;
        s.recs = recs;
        s.ids = ids;
        s.x = (const bf16*)x;
        s.ldx = ldx;
        s.perm = seg->perm;
        s.seg_ids = seg->seg_ids;
        s.seg_off = seg->seg_off;
        s.n_seg = seg->n_seg;
        s.cap = std::min<int32_t>(seg->cap, std::max<int32_t>(1, std::min<int32_t>(n_rows, n_bins)));
        s.tpart = tpart;
        s.rtp = R.rtp;
        s.M = n_rows;
        s.ks_len = R.ks_len;
        s.kp = R.ks_len + 8;
        const int rb = (int)ceil_div(P.r_max, 16) * 16;
        const size_t lds = std::max<size_t>((size_t)rb * s.kp * 2, 4 * SS_ROWS * 64 * 4);
        s.St = R.St;
        dim3 grid((unsigned)(rows_tiles(n_rows, n_bins) * R.St));
        hipLaunchKernelGGL(k_seg_shrink, grid, dim3(SS_NT), lds, stream, P, s);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (finish) {
        SegFinishArgs f;
        f.recs = recs;
        f.part = part;
        f.ldp = R.ldp;
        f.S = R.S;
        f.tpart = tpart;
        f.rtp = R.rtp;
        f.St = R.St;
        f.M = n_rows;
        f.n_chunks = (int32_t)ceil_div(P.d_out, FS_COLS);
        f.y = y;
        f.ldy = ldy;
        // chunk-minor: with a multiple of 8 chunks a chunk stays on one XCD
        dim3 grid((unsigned)(ceil_div(n_rows, FS_NT / 64) * f.n_chunks));
        const bool vec = P.vec_b != 0;
#define LORA_FIN(TY_, SB_)                                                                           \
    do {                                                                                             \
        if (vec) hipLaunchKernelGGL((k_seg_finish<TY_, SB_, true>), grid, dim3(FS_NT), 0, stream, P, f);  \
        else hipLaunchKernelGGL((k_seg_finish<TY_, SB_, false>), grid, dim3(FS_NT), 0, stream, P, f);     \
    } while (0)
        if (ydt == LORA_BF16) {
            if (R.S <= 1) LORA_FIN(bf16, 1);
            else if (R.S <= 2) LORA_FIN(bf16, 2);
            else if (R.S <= 4) LORA_FIN(bf16, 4);
            else LORA_FIN(bf16, 8);
        } else {
            if (R.S <= 1) LORA_FIN(float, 1);
            else if (R.S <= 2) LORA_FIN(float, 2);
            else if (R.S <= 4) LORA_FIN(float, 4);
            else LORA_FIN(float, 8);
        }
#undef LORA_FIN
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace lora
