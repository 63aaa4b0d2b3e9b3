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
#include <climits>

#include "lora_internal.hpp"

namespace lora {
namespace {

template <typename T> struct MF;
template <> struct MF<bf16> {
    static constexpr int KSTEP = 32;
    static constexpr int KPL = 8;
    using frag = bf16x8_t;
    static __device__ __forceinline__ frag ld(const bf16* p) { return *(const bf16x8_t*)p; }
    static __device__ __forceinline__ f32x4_t mma(frag a, frag b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct MF<float> {
    static constexpr int KSTEP = 4;
    static constexpr int KPL = 1;
    using frag = float;
    static __device__ __forceinline__ frag ld(const float* p) { return *p; }
    static __device__ __forceinline__ f32x4_t mma(frag a, frag b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

template <typename T_, int BM_, int BN_, int BK_, int WM_, int WN_>
struct Cfg {
    using T = T_;
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int NT = WM * WN * 64;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int FM = WTM / 16, FN = WTN / 16;
    static constexpr int VE = 16 / sizeof(T);
    static constexpr int LDK = BK + VE;
    static constexpr int A_ELEMS = BM * LDK;
    static constexpr int B_ELEMS = BN * LDK;
    static constexpr int STAGE = A_ELEMS + B_ELEMS;
    // ranks covered by one K-extension step of the LoRA epilogue: bf16 splits
    // the fp32 operand into hi + lo halves, fp32 takes it as is
    static constexpr int KH = (sizeof(T) == 2) ? BK / 2 : BK;
    static_assert(FM >= 1 && FN >= 1, "wave tile smaller than 16x16");
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile not a multiple of 16");
    static_assert(BK % MF<T>::KSTEP == 0, "BK not a multiple of the MFMA K");
    static_assert(BK % VE == 0, "BK not a multiple of the vector width");
};

template <class C>
struct Acc {
    f32x4_t v[C::FM][C::FN];
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j) v[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
};

// acc += sA[wave rows][0:BK] x sB[wave cols][0:BK]^T
template <class C>
__device__ __forceinline__ void mma_block(Acc<C>& acc, const typename C::T* sA,
                                          const typename C::T* sB, int wm, int wn, int lane) {
    using T = typename C::T;
    using M = MF<T>;
    const int lr = lane & 15;
    const int kq = (lane >> 4) * M::KPL;
    const T* pa = sA + (wm * C::WTM + lr) * C::LDK + kq;
    const T* pb = sB + (wn * C::WTN + lr) * C::LDK + kq;
#pragma unroll
    for (int kk = 0; kk < C::BK; kk += M::KSTEP) {
        typename M::frag a[C::FM], b[C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; ++i) a[i] = M::ld(pa + i * 16 * C::LDK + kk);
#pragma unroll
        for (int j = 0; j < C::FN; ++j) b[j] = M::ld(pb + j * 16 * C::LDK + kk);
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j) acc.v[i][j] = M::mma(a[i], b[j], acc.v[i][j]);
    }
}

// K-contiguous rows -> LDS [row][k].  sRow[r] is the source row or -1.
template <class C, int ROWS>
struct RowLoader {
    using T = typename C::T;
    static constexpr int VPR = C::BK / C::VE;
    static constexpr int TOT = ROWS * VPR;
    static constexpr int NV = (TOT + C::NT - 1) / C::NT;
    uint4 reg[NV];

    __device__ __forceinline__ void load(const T* __restrict__ base, int64_t ld, const int* sRow,
                                         int k0, int K, int tid) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int idx = tid + v * C::NT;
            if (TOT % C::NT != 0 && idx >= TOT) break;
            const int r = idx / VPR;
            const int k = k0 + (idx - r * VPR) * C::VE;
            const int gr = sRow[r];
            if (gr >= 0 && k + C::VE <= K) {
                reg[v] = *(const uint4*)(base + (int64_t)gr * ld + k);
            } else {
                union { uint4 u; T e[C::VE]; } tmp;
#pragma unroll
                for (int e = 0; e < C::VE; ++e)
                    tmp.e[e] = (gr >= 0 && k + e < K) ? base[(int64_t)gr * ld + k + e] : (T)0;
                reg[v] = tmp.u;
            }
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

// Row-major [K][N] source -> LDS [n][k] (transposed on the way in).
template <class C, int COLS>
struct TransLoader {
    using T = typename C::T;
    static constexpr int VPR = COLS / C::VE;
    static constexpr int TOT = C::BK * VPR;
    static constexpr int NV = (TOT + C::NT - 1) / C::NT;
    static_assert(COLS % C::VE == 0, "tile width not a multiple of the vector width");
    uint4 reg[NV];

    __device__ __forceinline__ void load(const T* __restrict__ base, int64_t ld, int k0, int K,
                                         int n0, int N, bool vec, int tid) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int idx = tid + v * C::NT;
            if (TOT % C::NT != 0 && idx >= TOT) break;
            const int kr = idx / VPR;
            const int k = k0 + kr;
            const int n = n0 + (idx - kr * VPR) * C::VE;
            if (vec && k < K && n + C::VE <= N) {
                reg[v] = *(const uint4*)(base + (int64_t)k * ld + n);
            } else {
                union { uint4 u; T e[C::VE]; } tmp;
#pragma unroll
                for (int e = 0; e < C::VE; ++e)
                    tmp.e[e] = (k < K && n + e < N) ? base[(int64_t)k * ld + n + e] : (T)0;
                reg[v] = tmp.u;
            }
        }
    }
    __device__ __forceinline__ void store(T* s, int tid) const {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int idx = tid + v * C::NT;
            if (TOT % C::NT != 0 && idx >= TOT) break;
            const int kr = idx / VPR;
            const int c = (idx - kr * VPR) * C::VE;
            union { uint4 u; T e[C::VE]; } tmp;
            tmp.u = reg[v];
#pragma unroll
            for (int e = 0; e < C::VE; ++e) s[(c + e) * C::LDK + kr] = tmp.e[e];
        }
    }
};

// LoRA expand as extra K-steps on the accumulator.  For every distinct
// adapter u among the tile's rows (ascending id), the tile is extended by
//   A-side: s_u * t[row][j] for rows with id u, 0 elsewhere   (BM x r_u)
//   B-side: B_u[j][n0 + n]                                   (r_u x BN)
// bf16 operands carry the fp32 s*t as hi + lo bf16 halves against B_u
// twice, so the intermediate keeps ~16 significant bits.  sId[m] holds the
// row's adapter id or INT_MAX (base-only, invalid or past the end); sRow[m]
// is the row's index into t.
template <class C>
__device__ void lora_kext(Acc<C>& acc, const PoolDev& P, const float* __restrict__ t, int64_t ldt,
                          const int* sRow, const int* sId, int* sNext, typename C::T* smem, int n0,
                          int tid, int wm, int wn, int lane) {
    using T = typename C::T;
    constexpr bool HL = sizeof(T) == 2;
    T* sA = smem;
    T* sB = smem + C::A_ELEMS;
    const int d_out = P.d_out;
    int prev = -1;
    for (;;) {
        if (tid == 0) *sNext = INT_MAX;
        __syncthreads();
        for (int m = tid; m < C::BM; m += C::NT) {
            const int v = sId[m];
            if (v > prev && v != INT_MAX) atomicMin(sNext, v);
        }
        __syncthreads();
        const int u = *sNext;
        if (u == INT_MAX) break;
        const int r = P.ranks[u];
        const float sc = P.scales[u];
        const T* Bu = (const T*)P.B + P.b_off[u];
        for (int j0 = 0; j0 < r; j0 += C::KH) {
            for (int idx = tid; idx < C::BM * C::KH; idx += C::NT) {
                const int m = idx / C::KH;
                const int kk = idx - m * C::KH;
                const int j = j0 + kk;
                float v = 0.f;
                if (sId[m] == u && j < r) v = sc * t[(int64_t)sRow[m] * ldt + j];
                if constexpr (HL) {
                    const bf16 hi = f32_to_bf16(v);
                    const bf16 lo = f32_to_bf16(v - to_f32(hi));
                    sA[m * C::LDK + kk] = (T)hi;
                    sA[m * C::LDK + C::KH + kk] = (T)lo;
                } else {
                    sA[m * C::LDK + kk] = (T)v;
                }
            }
            for (int idx = tid; idx < C::KH * C::BN; idx += C::NT) {
                const int kk = idx / C::BN;
                const int nn = idx - kk * C::BN;
                const int j = j0 + kk;
                const int col = n0 + nn;
                T v = (T)0;
                if (j < r && col < d_out) v = Bu[(int64_t)j * d_out + col];
                sB[nn * C::LDK + kk] = v;
                if constexpr (HL) sB[nn * C::LDK + C::KH + kk] = v;
            }
            __syncthreads();
            mma_block<C>(acc, sA, sB, wm, wn, lane);
            __syncthreads();
        }
        prev = u;
    }
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(v, d, 64);
        if (lane >= d) v += o;
    }
    return v;
}

// Map workgroup b to (segment s, chunk c) over the segment tiles of height
// BM.  Run by one whole wave; returns false past the last tile.
__device__ bool find_seg_tile(const int32_t* __restrict__ seg_off, int n_seg, int BM, int b,
                              int lane, int& s_out, int& c_out) {
    int base = 0;
    for (int s0 = 0; s0 < n_seg; s0 += 64) {
        const int s = s0 + lane;
        int cnt = 0;
        if (s < n_seg) cnt = (seg_off[s + 1] - seg_off[s] + BM - 1) / BM;
        const int incl = wave_incl_scan(cnt, lane);
        const int excl = base + incl - cnt;
        const uint64_t hit = __ballot(s < n_seg && b >= excl && b < base + incl);
        if (hit) {
            const int L = __ffsll((unsigned long long)hit) - 1;
            s_out = s0 + L;
            c_out = b - __shfl(excl, L, 64);
            return true;
        }
        base += __shfl(incl, 63, 64);
    }
    return false;
}

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
    const float* t;
    int64_t ldt;
    void* y;
    int64_t ldy;
    int32_t tiles_m;
    int32_t tiles_n;
};

template <class C, typename TY, bool OUT_IN>
__global__ __launch_bounds__(C::NT) void k_layer_gemm(PoolDev P, GemmDev g) {
    using T = typename C::T;
    __shared__ __attribute__((aligned(16))) T smem[2 * C::STAGE];
    __shared__ int sRowA[C::BM];
    __shared__ int sRowB[OUT_IN ? C::BN : 1];
    __shared__ int sId[C::BM];
    __shared__ int sNext;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / C::WN;
    const int wn = wave - wm * C::WN;

    // XCD-aware order: consecutive workgroups land on different XCDs, so give
    // each XCD a contiguous run of tiles, then raster in groups of 8 row-tiles.
    int b = blockIdx.x;
    const int T_all = gridDim.x;
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

    for (int r = tid; r < C::BM; r += C::NT) {
        const int row = m0 + r;
        int id = INT_MAX;
        if (row < g.n) {
            const int a = g.ids[row];
            if (id_ok(a, P.n_adapters)) id = a;
            else if (a != -1 && tn == 0) flag_bad_id(P.err);
        }
        sRowA[r] = row < g.n ? row : -1;
        sId[r] = id;
    }
    if constexpr (OUT_IN)
        for (int r = tid; r < C::BN; r += C::NT) sRowB[r] = (n0 + r < N) ? n0 + r : -1;
    __syncthreads();

    Acc<C> acc;
    acc.zero();
    const T* X = (const T*)g.x;
    const T* Wp = (const T*)g.W;
    RowLoader<C, C::BM> la;
    using LB = typename std::conditional<OUT_IN, RowLoader<C, C::BN>, TransLoader<C, C::BN>>::type;
    LB lb;
    auto load_b = [&](int k0) {
        if constexpr (OUT_IN) lb.load(Wp, g.ldw, sRowB, k0, K, tid);
        else lb.load(Wp, g.ldw, k0, K, n0, N, true, tid);
    };
    const int nk = (K + C::BK - 1) / C::BK;
    la.load(X, g.ldx, sRowA, 0, K, tid);
    load_b(0);
    for (int kb = 0; kb < nk; ++kb) {
        T* sA = smem + (kb & 1) * C::STAGE;
        T* sB = sA + C::A_ELEMS;
        la.store(sA, tid);
        lb.store(sB, tid);
        __syncthreads();
        if (kb + 1 < nk) {
            la.load(X, g.ldx, sRowA, (kb + 1) * C::BK, K, tid);
            load_b((kb + 1) * C::BK);
        }
        mma_block<C>(acc, sA, sB, wm, wn, lane);
    }
    __syncthreads();
    if (g.t) lora_kext<C>(acc, P, g.t, g.ldt, sRowA, sId, &sNext, smem, n0, tid, wm, wn, lane);

    TY* Y = (TY*)g.y;
    const int lr = lane & 15;
    const int lq = (lane >> 4) * 4;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            const int col = n0 + wn * C::WTN + j * 16 + lr;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = m0 + wm * C::WTM + i * 16 + lq + q;
                if (row < g.n && col < N) Y[(int64_t)row * g.ldy + col] = from_f32<TY>(acc.v[i][j][q]);
            }
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
                                                       float* __restrict__ t, int64_t ldt) {
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
    if (!id_ok(u, P.n_adapters)) {
        for (int idx = tid; idx < cnt * r_max; idx += C::NT) {
            const int m = idx / r_max;
            t[(int64_t)sRow[m] * ldt + (idx - m * r_max)] = 0.f;
        }
        return;
    }
    const int r = P.ranks[u];
    const T* Au = (const T*)P.A + P.a_off[u];
    const bool vec = P.vec_a && ((r * (int)sizeof(T)) % 16) == 0;
    const int K = P.d_in;

    Acc<C> acc;
    acc.zero();
    RowLoader<C, C::BM> la;
    TransLoader<C, C::BN> lb;
    const int nk = (K + C::BK - 1) / C::BK;
    la.load(x, ldx, sRow, 0, K, tid);
    lb.load(Au, r, 0, K, 0, r, vec, tid);
    for (int kb = 0; kb < nk; ++kb) {
        T* sA = smem + (kb & 1) * C::STAGE;
        T* sB = sA + C::A_ELEMS;
        la.store(sA, tid);
        lb.store(sB, tid);
        __syncthreads();
        if (kb + 1 < nk) {
            la.load(x, ldx, sRow, (kb + 1) * C::BK, K, tid);
            lb.load(Au, r, (kb + 1) * C::BK, K, 0, r, vec, tid);
        }
        mma_block<C>(acc, sA, sB, wm, wn, lane);
    }

    const int lr = lane & 15;
    const int lq = (lane >> 4) * 4;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            const int col = wn * C::WTN + j * 16 + lr;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = wm * C::WTM + i * 16 + lq + q;
                if (m < cnt && col < r_max) t[(int64_t)sRow[m] * ldt + col] = acc.v[i][j][q];
            }
        }
}

// ---------------------------------------------------------------------------
// SGMV expand: y[rows of segment, n-tile] (+)= s_u * t[rows] B_u
// ---------------------------------------------------------------------------

template <class C, typename TY>
__global__ __launch_bounds__(C::NT) void k_sgmv_expand(PoolDev P, const float* __restrict__ t,
                                                       int64_t ldt, const int32_t* __restrict__ perm,
                                                       const int32_t* __restrict__ seg_ids,
                                                       const int32_t* __restrict__ seg_off,
                                                       const int32_t* __restrict__ n_seg_p,
                                                       TY* __restrict__ y, int64_t ldy,
                                                       int accumulate, int tiles_n) {
    using T = typename C::T;
    __shared__ __attribute__((aligned(16))) T smem[C::STAGE];
    __shared__ int sRow[C::BM];
    __shared__ int sId[C::BM];
    __shared__ int sInfo[3];
    __shared__ int sNext;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / C::WN;
    const int wn = wave - wm * C::WN;
    const int tb = blockIdx.x / tiles_n;
    const int tn = blockIdx.x - tb * tiles_n;
    const int n0 = tn * C::BN;
    const int N = P.d_out;

    if (wave == 0) {
        int s = 0, c = 0;
        const bool found = find_seg_tile(seg_off, *n_seg_p, C::BM, tb, lane, s, c);
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
    const bool ok = id_ok(u, P.n_adapters);
    for (int r = tid; r < C::BM; r += C::NT) {
        sRow[r] = r < cnt ? perm[row0 + r] : -1;
        sId[r] = (r < cnt && ok) ? u : INT_MAX;
    }
    __syncthreads();
    if (!ok && accumulate) return;

    Acc<C> acc;
    acc.zero();
    if (ok) lora_kext<C>(acc, P, t, ldt, sRow, sId, &sNext, smem, n0, tid, wm, wn, lane);

    const int lr = lane & 15;
    const int lq = (lane >> 4) * 4;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            const int col = n0 + wn * C::WTN + j * 16 + lr;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = wm * C::WTM + i * 16 + lq + q;
                if (m < cnt && col < N) {
                    TY* p = y + (int64_t)sRow[m] * ldy + col;
                    float v = acc.v[i][j][q];
                    if (accumulate) v += to_f32(*p);
                    *p = from_f32<TY>(v);
                }
            }
        }
}

// ---------------------------------------------------------------------------
// Tile configurations
// ---------------------------------------------------------------------------

using GemmBig = Cfg<bf16, 128, 128, 64, 2, 2>;
using GemmMid = Cfg<bf16, 64, 64, 64, 2, 2>;
using GemmSmall = Cfg<bf16, 32, 64, 64, 2, 2>;
using GemmF32 = Cfg<float, 64, 64, 32, 2, 2>;
using ShrinkB = Cfg<bf16, 64, 64, 64, 4, 1>;
using ShrinkF = Cfg<float, 64, 64, 32, 4, 1>;
using ExpandB = Cfg<bf16, 64, 64, 64, 2, 2>;
using ExpandF = Cfg<float, 64, 64, 32, 2, 2>;

template <class C, typename TY>
hipError_t run_gemm(const PoolDev& P, const GemmArgs& a, hipStream_t stream) {
    GemmDev g;
    g.x = a.x;
    g.ldx = a.ldx;
    g.W = a.W;
    g.ldw = a.ldw;
    g.ids = a.ids;
    g.n = a.n_rows;
    g.t = a.t;
    g.ldt = a.ldt;
    g.y = a.y;
    g.ldy = a.ldy;
    g.tiles_m = (int32_t)ceil_div(a.n_rows, C::BM);
    g.tiles_n = (int32_t)ceil_div(P.d_out, C::BN);
    dim3 grid((unsigned)((int64_t)g.tiles_m * g.tiles_n));
    if (a.w_out_in)
        hipLaunchKernelGGL((k_layer_gemm<C, TY, true>), grid, dim3(C::NT), 0, stream, P, g);
    else
        hipLaunchKernelGGL((k_layer_gemm<C, TY, false>), grid, dim3(C::NT), 0, stream, P, g);
    return hipGetLastError();
}

template <typename TY>
hipError_t run_gemm_bf16(const PoolDev& P, const GemmArgs& a, hipStream_t stream) {
    // Largest tile that still gives about one workgroup per CU.
    const int64_t n_big = ceil_div(a.n_rows, GemmBig::BM) * ceil_div(P.d_out, GemmBig::BN);
    const int64_t n_mid = ceil_div(a.n_rows, GemmMid::BM) * ceil_div(P.d_out, GemmMid::BN);
    if (n_big >= 256) return run_gemm<GemmBig, TY>(P, a, stream);
    if (n_mid >= 256 || a.n_rows > 32) return run_gemm<GemmMid, TY>(P, a, stream);
    return run_gemm<GemmSmall, TY>(P, a, stream);
}

}  // namespace

hipError_t launch_layer_gemm(const PoolDev& P, lora_dtype_t dt, lora_dtype_t ydt, const GemmArgs& a,
                             hipStream_t stream) {
    if (dt == LORA_BF16)
        return ydt == LORA_BF16 ? run_gemm_bf16<bf16>(P, a, stream) : run_gemm_bf16<float>(P, a, stream);
    return ydt == LORA_BF16 ? run_gemm<GemmF32, bf16>(P, a, stream) : run_gemm<GemmF32, float>(P, a, stream);
}

static int64_t seg_tiles(int32_t n_rows, int32_t n_bins, int bm) {
    return ceil_div(n_rows, bm) + std::min<int64_t>(n_rows, n_bins);
}

hipError_t launch_sgmv_shrink(const PoolDev& P, lora_dtype_t dt, const void* x, int64_t ldx,
                              const lora_segments_t* seg, int32_t n_rows, int32_t n_bins, float* t,
                              int64_t ldt, bool, hipStream_t stream) {
    if (dt == LORA_BF16) {
        dim3 grid((unsigned)seg_tiles(n_rows, n_bins, ShrinkB::BM));
        hipLaunchKernelGGL(k_sgmv_shrink<ShrinkB>, grid, dim3(ShrinkB::NT), 0, stream, P,
                           (const bf16*)x, ldx, seg->perm, seg->seg_ids, seg->seg_off, seg->n_seg, t,
                           ldt);
    } else {
        dim3 grid((unsigned)seg_tiles(n_rows, n_bins, ShrinkF::BM));
        hipLaunchKernelGGL(k_sgmv_shrink<ShrinkF>, grid, dim3(ShrinkF::NT), 0, stream, P,
                           (const float*)x, ldx, seg->perm, seg->seg_ids, seg->seg_off, seg->n_seg, t,
                           ldt);
    }
    return hipGetLastError();
}

template <class C, typename TY>
static hipError_t run_expand(const PoolDev& P, const float* t, int64_t ldt, const lora_segments_t* seg,
                             int32_t n_rows, int32_t n_bins, void* y, int64_t ldy, int accumulate,
                             hipStream_t stream) {
    const int tiles_n = (int)ceil_div(P.d_out, C::BN);
    dim3 grid((unsigned)(seg_tiles(n_rows, n_bins, C::BM) * tiles_n));
    hipLaunchKernelGGL((k_sgmv_expand<C, TY>), grid, dim3(C::NT), 0, stream, P, t, ldt, seg->perm,
                       seg->seg_ids, seg->seg_off, seg->n_seg, (TY*)y, ldy, accumulate, tiles_n);
    return hipGetLastError();
}

hipError_t launch_sgmv_expand(const PoolDev& P, lora_dtype_t dt, const float* t, int64_t ldt,
                              const lora_segments_t* seg, int32_t n_rows, int32_t n_bins, void* y,
                              lora_dtype_t ydt, int64_t ldy, int accumulate, hipStream_t stream) {
    if (dt == LORA_BF16)
        return ydt == LORA_BF16
                   ? run_expand<ExpandB, bf16>(P, t, ldt, seg, n_rows, n_bins, y, ldy, accumulate, stream)
                   : run_expand<ExpandB, float>(P, t, ldt, seg, n_rows, n_bins, y, ldy, accumulate, stream);
    return ydt == LORA_BF16
               ? run_expand<ExpandF, bf16>(P, t, ldt, seg, n_rows, n_bins, y, ldy, accumulate, stream)
               : run_expand<ExpandF, float>(P, t, ldt, seg, n_rows, n_bins, y, ldy, accumulate, stream);
}

}  // namespace lora
