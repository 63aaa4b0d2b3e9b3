// Decode layer in two launches (n_rows <= 64, bf16, W stored [d_out, d_in]).
//
// At decode sizes the layer is a stream of W (and of the adapters' A and B
// blocks) with almost no reuse; the adapter term is bandwidth bound and its
// cost is reading A and B ("Serving many LoRA adapters" (blog.ecitis.org),
// section "Batching across different adapters").  A single pass over W per
// CU is limited by how many misses a CU keeps in flight, so the work is cut
// into many small independent pieces, and partial sums meet at the kernel
// boundary (an in-kernel cross-XCD hand-off costs more than the whole pass):
//
//   stream: workgroup (tn, ks) owns 128 output columns and K slice ks.  The
//           x rows of the slice are staged once in LDS; each wave streams the
//           W rows of 16 columns and the workgroup writes the fp32 partial
//           part_base[ks][m][n].  Over the same staged x it also shrinks the
//           rows i = tn, tn + tiles_n, ... : x_i A_a over the slice (BGMV: the
//           row gathers its own adapter), written as part_t[ks][i][j].
//   finish: y[m][n] = sum_slices part_base + s_a * sum_j (sum_slices part_t)[j]
//           * B_a[j][n], rounded once.
//
// Every sum runs in a fixed order, so results do not depend on timing.
#include <climits>

#include "lora_internal.hpp"

namespace lora {
namespace {

constexpr int DS_BASE_THREADS = 512;                // 8 base waves, 16 columns each
constexpr int DS_THREADS = DS_BASE_THREADS + 64;    // + the shrink wave
constexpr int DS_NB = 8;            // 16-column MFMA blocks per base workgroup, one per wave
constexpr int DS_COLS = DS_NB * 16;
constexpr int DS_USTEPS = 16;       // k-steps (of 32) per base slice at most
constexpr int DS_SHRINK_LOADS = 16; // 16-byte A pieces in flight per lane of the shrink wave
constexpr int FIN_THREADS = 64;     // finish workgroup (one wave), 4 columns per thread
constexpr int FIN_COLS = FIN_THREADS * 4;
static_assert(FIN_THREADS >= 64 && FIN_THREADS % 64 == 0, "the t partials need one thread per rank");
constexpr int FIN_RCHUNK = 16;      // rank rows of B loaded together in the finish
constexpr int FIN_SCHUNK = 8;       // partial slices loaded together in the finish

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16 bytes, nontemporal or ordinary
template <bool NT>
__device__ __forceinline__ u32x4_t ld16(const void* p) {
    if constexpr (NT) return __builtin_nontemporal_load((const u32x4_t*)p);
    else return *(const u32x4_t*)p;
}

template <bool NT = false>
__device__ __forceinline__ bf16x8_t ld8(const bf16* p, int valid) {
    if (valid >= 8) return __builtin_bit_cast(bf16x8_t, ld16<NT>(p));
    union { bf16x8_t v; bf16 e[8]; } u;
#pragma unroll
    for (int e = 0; e < 8; ++e) u.e[e] = (e < valid) ? p[e] : (bf16)0;
    return u.v;
}

// Eight signed 4-bit weights (two's complement, element e in bits 4e..4e+3)
// as bf16.  Integers in [-8, 7] are exact in fp32 and in bf16, so the high
// half of the fp32 pattern is the bf16 value.
__device__ __forceinline__ bf16x8_t dequant8_q4(uint32_t w) {
    union { bf16x8_t v; bf16 e[8]; } u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int q = ((int)(w << (28 - 4 * e))) >> 28;
        u.e[e] = (bf16)(__float_as_uint((float)q) >> 16);
    }
    return u.v;
}

// Shrink wave of workgroup (tn, ks): rows i = tn, tn + tiles_n, ...; for
// each, part_t[ks][i][0:r] = x_i[slice] A_a[slice] over the staged x row, and
// (slice 0) the row record for the finish pass.  A wave of its own, with its
// own load counter, so its A pieces stream while the base waves still wait
// for W.  Ranks the pool holds that divide 4096 (G = r / 8 lanes per k-row, a
// power of two) take 16-byte pieces: lane l owns columns (l % G) * 8 .. + 8 of
// k-rows l / G + p * (64 / G).
__device__ __forceinline__ void shrink_wave(const PoolDev& P, const DecodePlan& D, const DecodeArgs& g, int tn,
                                            int ks, int kbeg, int klen, const bf16* xs, int xld, int lane) {
    const int M = g.n;
    // the first row's lookups (scalar loads) and row record go out before
    // the x barrier; its A pieces after it
    int i = tn;
    int a = i < M ? uload(g.ids, i) : -1;
    bool ok = id_ok(a, P.n_adapters);
    int r = ok ? uload(P.ranks, a) : 0;
    int64_t aoff = ok ? uload(P.a_off, a) : 0;
    __syncthreads();   // x staged by the base waves
    for (; i < M;) {
        if (ks == 0 && lane == 0) {
            // row record for the finish pass: B block offset, rank (0: no term), scale
            RowRec rec;
            rec.b_off = ok ? uload(P.b_off, a) : 0;
            rec.rank = r;
            rec.scale = ok ? uload(P.scales, a) : 0.f;
            g.rows[i] = rec;
            if (!ok && a != -1) flag_bad_id(P.err);
        }
        if (r > 0) {   // the finish pass never reads t for rows without a term
            const bf16* Au = (const bf16*)P.A + aoff + (int64_t)kbeg * r;
            const bf16* xi = xs + i * xld;
            float* outp = g.part_t + ((int64_t)ks * M + i) * 64;
            if (P.stream_ok) {
                const int G = r / 8;
                const int RPP = 64 / G;   // k-rows per pass
                const int passes = (klen + RPP - 1) / RPP;
                const int jv = lane % G;
                const int ksub = lane / G;
                float acc[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = 0.f;
                for (int p0 = 0; p0 < passes; p0 += DS_SHRINK_LOADS) {
                    uint4 av[DS_SHRINK_LOADS];
#pragma unroll
                    for (int q = 0; q < DS_SHRINK_LOADS; ++q) {
                        const int kk = ksub + (p0 + q) * RPP;
                        // past the slice: read its first k-row again; it meets x = 0 below
                        av[q] = *(const uint4*)(Au + (int64_t)(kk < klen ? kk : 0) * r + jv * 8);
                    }
#pragma unroll
                    for (int q = 0; q < DS_SHRINK_LOADS; ++q) {
                        const int kk = ksub + (p0 + q) * RPP;
                        const float xv = (kk < klen) ? to_f32(xi[kk]) : 0.f;
                        union { uint4 u; bf16 e[8]; } v;
                        v.u = av[q];
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[e] += xv * to_f32(v.e[e]);
                    }
                }
                for (int d = G; d < 64; d <<= 1)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], d, 64);
                if (lane < G)
#pragma unroll
                    for (int e = 0; e < 8; ++e) outp[lane * 8 + e] = acc[e];
            } else {
                // any rank: lane (j, gq) sums column j over k-rows gq, gq + Gs, ...;
                // the groups are then added in order gq = 0, 1, ...
                const int Gs = 64 / r;
                const int j = lane % r;
                const int gq = lane / r;
                float acc = 0.f;
                if (gq < Gs)
                    for (int kk = gq; kk < klen; kk += Gs) acc += to_f32(xi[kk]) * to_f32(Au[(int64_t)kk * r + j]);
                float v = acc;
                for (int q = 1; q < Gs; ++q) v += __shfl(acc, j + q * r, 64);
                if (lane < r) outp[lane] = v;
            }
        }
        i += D.tiles_n;
        if (i >= M) break;
        a = uload(g.ids, i);
        ok = id_ok(a, P.n_adapters);
        r = ok ? uload(P.ranks, a) : 0;
        aoff = ok ? uload(P.a_off, a) : 0;
    }
}

// Workgroup (tn, ks): base wave w < 8 streams the 16 rows of W^T for column
// block w (all of the slice's k-steps in flight) and keeps the whole 16-column
// partial; x of the slice is staged in LDS and serves the MFMAs and the shrink
// wave.  W is read once.  With the shrink wave, W goes through nontemporal
// loads, which leave the caches to the adapter blocks that rows of one adapter
// share; without it, ordinary loads measured 5-7% faster (a wave's load takes
// 64 bytes of each of 16 rows, the two halves of a 128-byte line coming from
// two loads, and an ordinary load keeps the line for the second).  The shrink
// wave's A pieces go out after the x barrier: requested beside x they slowed
// the staging of x, which every MFMA waits for, by more than they gained.
//
// Q4: W holds signed 4-bit weights, row n of bytes at W + n * ldw (input k
// in the low nibble when even), with scale wscale[n * lds + k / 128].  The
// k order of a dot product is free, so lane group g = lane / 16 loads 16
// bytes (32 inputs) per 128-input group j of the slice: inputs
// j * 128 + g * 32 .. + 32, taken 8 at a time in four MFMA steps, with x read
// from LDS at the same inputs.  The four steps of group j thus cover exactly
// that group in every lane; its sums are scaled once and added.
template <int MB, bool FULL, bool LORA, bool Q4>
__device__ __forceinline__ void stream_body(const PoolDev& P, const DecodePlan& D, const DecodeArgs& g, int b,
                                            uint8_t* lds) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int tn = b % D.tiles_n;
    const int ks = b / D.tiles_n;
    const int K = P.d_in;
    const int N = P.d_out;
    const int M = g.n;
    const int kbeg = ks * D.kslice;
    const int kend = min(K, kbeg + D.kslice);
    const int klen = kend - kbeg;
    const int nsteps = (klen + 31) / 32;
    const int lr = lane & 15;
    const int kq = (lane >> 4) * 8;
    const int n = tn * DS_COLS + wave * 16 + lr;
    const int nc = n < N ? n : 0;   // a column past d_out reads row 0; its output is never stored

    // x[0:16*MB][slice] -> LDS as [m][k] bf16, rows padded by 16 bytes.  The
    // x pieces are requested before W: they come from L2 and return first, so
    // they are staged while the W stream is still in flight.
    constexpr int XLD = DS_USTEPS * 32 + 8;
    static_assert(MB * 16 * XLD * 2 <= DS_LDS_BYTES, "staged x does not fit the LDS block");
    constexpr int PER_ROW = DS_USTEPS * 32 / 8;    // 16-byte pieces per staged row
    constexpr int XV = MB * 16 * PER_ROW / DS_BASE_THREADS;
    static_assert(MB * 16 * PER_ROW % DS_BASE_THREADS == 0, "x pieces do not split evenly");
    bf16* xs = (bf16*)lds;
    if (LORA && wave == DS_NB) {
        shrink_wave(P, D, g, tn, ks, kbeg, klen, xs, XLD, lane);
        return;
    }
    const bf16* X = (const bf16*)g.x;
    bf16x8_t xv[XV];
#pragma unroll
    for (int q = 0; q < XV; ++q) {
        const int v = tid + q * DS_BASE_THREADS;
        const int m = v / PER_ROW;
        const int k = kbeg + (v - m * PER_ROW) * 8;
        if constexpr (FULL) {
            // rows past the batch read row 0; they only feed rows that are never stored
            xv[q] = *(const bf16x8_t*)(X + (int64_t)(m < M ? m : 0) * g.ldx + k);
        } else {
            const int valid = min(8, kend - k);
            xv[q] = (m < M && valid > 0) ? ld8(X + (int64_t)m * g.ldx + k, valid) : bf16x8_t{};
        }
    }

    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    constexpr int NW = Q4 ? 1 : DS_USTEPS;
    constexpr int NQ = Q4 ? DS_USTEPS / 4 : 1;
    bf16x8_t bw[NW];
    u32x4 wq[NQ];
    float wsc[NQ];
    // 4-bit: 128-input groups in the slice (klen is a multiple of 128)
    const int ngrp = FULL ? DS_USTEPS / 4 : klen / 128;
    if constexpr (Q4) {
        const uint8_t* Wq = (const uint8_t*)g.W + (int64_t)nc * g.ldw + kbeg / 2 + (lane >> 4) * 16;
        const float* Sc = g.wscale + (int64_t)nc * g.lds + kbeg / 128;
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            if (FULL || j < ngrp) {
                wq[j] = ld16<LORA>(Wq + j * 64);
                wsc[j] = Sc[j];
            } else {
                wq[j] = u32x4{0u, 0u, 0u, 0u};
                wsc[j] = 0.f;
            }
        }
    } else if constexpr (FULL) {
        const bf16* Wt = (const bf16*)g.W + (int64_t)nc * g.ldw;
#pragma unroll
        for (int u = 0; u < DS_USTEPS; ++u) {
            bw[u] = __builtin_bit_cast(bf16x8_t, ld16<LORA>(Wt + kbeg + u * 32 + kq));
        }
    } else {
        const bf16* Wt = (const bf16*)g.W + (int64_t)nc * g.ldw;
#pragma unroll
        for (int u = 0; u < DS_USTEPS; ++u) {
            const int k = kbeg + u * 32 + kq;
            const int valid = (u < nsteps) ? min(8, kend - k) : 0;
            bw[u] = (valid > 0 && n < N) ? ld8<LORA>(Wt + k, valid) : bf16x8_t{};
        }
    }

#pragma unroll
    for (int q = 0; q < XV; ++q) {
        const int v = tid + q * DS_BASE_THREADS;
        const int m = v / PER_ROW;
        *(bf16x8_t*)(xs + m * XLD + (v - m * PER_ROW) * 8) = xv[q];
    }
    __syncthreads();

    f32x4_t acc[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (Q4) {
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            if (FULL || j < ngrp) {
                f32x4_t ag[MB];
#pragma unroll
                for (int i = 0; i < MB; ++i) ag[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                const int k0 = j * 128 + (lane >> 4) * 32;   // this lane's 32 inputs of group j
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    const bf16x8_t b = dequant8_q4(wq[j][st]);
#pragma unroll
                    for (int i = 0; i < MB; ++i) {
                        const bf16x8_t a = *(const bf16x8_t*)(xs + (i * 16 + lr) * XLD + k0 + st * 8);
                        ag[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, ag[i], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int i = 0; i < MB; ++i) acc[i] += wsc[j] * ag[i];
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < DS_USTEPS; ++u) {
            if (FULL || u < nsteps) {
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    const bf16x8_t a = *(const bf16x8_t*)(xs + (i * 16 + lr) * XLD + u * 32 + kq);
                    acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bw[u], acc[i], 0, 0, 0);
                }
            }
        }
    }

    if (n < N) {
        float* out = g.part_base + (int64_t)ks * M * N + n;
        const int lq = (lane >> 4) * 4;
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = i * 16 + lq + q;
                if (m < M) out[(int64_t)m * N] = acc[i][q];
            }
    }
}

// LORA: the workgroup has the shrink wave (the layer with its adapter term);
// without it the stream is the base product alone.
template <int MB, bool LORA, bool Q4 = false>
__global__ __launch_bounds__(LORA ? DS_THREADS : DS_BASE_THREADS) void k_decode_stream(PoolDev P, DecodePlan D,
                                                                                    DecodeArgs g) {
    // staged x; sized over half a CU's LDS so that each CU runs one
    // workgroup and the grid (about one workgroup per CU) spreads over all
    __shared__ __attribute__((aligned(16))) uint8_t lds[DS_LDS_BYTES];
    // a slice wholly inside K (the usual case) takes the branch-free form,
    // whose wait counts let x be staged while W is still arriving
    const int b = blockIdx.x;
    const int kbeg = (b / D.tiles_n) * D.kslice;
    if (min(P.d_in, kbeg + D.kslice) - kbeg == DS_USTEPS * 32) stream_body<MB, true, LORA, Q4>(P, D, g, b, lds);
    else stream_body<MB, false, LORA, Q4>(P, D, g, b, lds);
}

// Finish: workgroup (m, chunk) owns FIN_COLS columns of row m, 4 per thread.
// Loads go out in the order their addresses are known: the base partials
// first (they need nothing), then, after the row record (a scalar load), the
// row's t partials and B rows.  The t partials are summed into LDS in slice
// order while the other loads are in flight.  VEC (d_out and every B block
// 16-byte aligned) takes whole 4-column vectors without branches.
template <typename TY, bool VEC, bool LORA>
__global__ __launch_bounds__(FIN_THREADS) void k_decode_finish(PoolDev P, DecodePlan D, DecodeArgs g) {
    __shared__ float st[64];
    const int tid = threadIdx.x;
    const int nch = (P.d_out + FIN_COLS - 1) / FIN_COLS;
    const int m = blockIdx.x / nch;
    const int c0 = (blockIdx.x - m * nch) * FIN_COLS + tid * 4;
    const int N = P.d_out;
    const int M = g.n;
    const bool in = c0 < N;
    const int cc = in ? c0 : 0;   // columns past d_out read column 0 and are not stored

    auto load4 = [&](const float* p) {
        float4 u;
        if constexpr (VEC) {
            u = *(const float4*)p;
        } else {
            u.x = p[0];
            u.y = (cc + 1 < N) ? p[1] : 0.f;
            u.z = (cc + 2 < N) ? p[2] : 0.f;
            u.w = (cc + 3 < N) ? p[3] : 0.f;
        }
        return u;
    };
    // base partials, FIN_SCHUNK slices requested together, added in slice order
    float4 u[FIN_SCHUNK];
    auto load_part = [&](int s0) {
#pragma unroll
        for (int q = 0; q < FIN_SCHUNK; ++q)
            u[q] = load4(g.part_base + ((int64_t)(s0 + q < D.base_slices ? s0 + q : 0) * M + m) * N + cc);
    };
    load_part(0);

    int r = 0;
    int64_t boff = 0;
    float sc = 0.f;
    if (LORA) {
        const RowRec* rec = g.rows + m;
        r = uload(&rec->rank, 0);
        boff = uload(&rec->b_off, 0);
        sc = uload(&rec->scale, 0);
    }
    float tp[FIN_SCHUNK];
    if (tid < r) {
#pragma unroll
        for (int q = 0; q < FIN_SCHUNK; ++q)
            tp[q] = g.part_t[((int64_t)(q < D.t_slices ? q : 0) * M + m) * 64 + tid];
    }
    const bf16* Bu = (const bf16*)P.B + boff + cc;
    uint2 bv[FIN_RCHUNK];
    auto load_b = [&](int j0) {
#pragma unroll
        for (int q = 0; q < FIN_RCHUNK; ++q) {
            const int j = j0 + q;
            if constexpr (VEC) {
                // rank rows past r read row 0 again; they meet t = 0
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
    for (int s0 = 0;;) {
#pragma unroll
        for (int q = 0; q < FIN_SCHUNK; ++q) {
            if (s0 + q < D.base_slices) {
                v[0] += u[q].x; v[1] += u[q].y; v[2] += u[q].z; v[3] += u[q].w;
            }
        }
        s0 += FIN_SCHUNK;
        if (s0 >= D.base_slices) break;
        load_part(s0);
    }
    if (tid < r) {
        float t = 0.f;
#pragma unroll
        for (int q = 0; q < FIN_SCHUNK; ++q)
            if (q < D.t_slices) t += tp[q];
        for (int s = FIN_SCHUNK; s < D.t_slices; ++s) t += g.part_t[((int64_t)s * M + m) * 64 + tid];
        st[tid] = t;
    }
    __syncthreads();
    if (!in) return;
    if (r > 0) {
        float e4[4] = {0.f, 0.f, 0.f, 0.f};
        for (int j0 = 0;;) {
#pragma unroll
            for (int q = 0; q < FIN_RCHUNK; ++q) {
                const float tj = (j0 + q < r) ? st[j0 + q] : 0.f;
                union { uint2 u; bf16 e[4]; } w;
                w.u = bv[q];
#pragma unroll
                for (int e = 0; e < 4; ++e) e4[e] += tj * to_f32(w.e[e]);
            }
            j0 += FIN_RCHUNK;
            if (j0 >= r) break;
            load_b(j0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += sc * e4[e];
    }
    TY* yr = (TY*)g.y + (int64_t)m * g.ldy;
    for (int e = 0; e < 4 && c0 + e < N; ++e) yr[c0 + e] = from_f32<TY>(v[e]);
}

}  // namespace

DecodePlan plan_decode(const PoolDev& P, int32_t n_rows, bool with_lora) {
    DecodePlan D;
    const int K = P.d_in;
    D.tiles_n = (int32_t)ceil_div(P.d_out, DS_COLS);
    const int ksteps = (int)ceil_div(K, 32);
    // K slices: about 256 workgroups, at most DS_USTEPS k-steps each
    const int want = (int)std::max<int64_t>(1, ceil_div(256, D.tiles_n));
    int steps = (int)ceil_div(ksteps, want);
    steps = std::max(1, std::min(steps, DS_USTEPS));
    steps = (int)ceil_div(steps, 4) * 4;   // whole groups of 128 k-rows (the 4-bit scale groups)
    D.kslice = steps * 32;
    D.base_slices = (int32_t)ceil_div(K, D.kslice);
    D.base_wgs = D.tiles_n * D.base_slices;
    // the shrink partials follow the base slices (workgroup (tn, ks) shrinks
    // rows tn, tn + tiles_n, ... over slice ks)
    D.t_slices = (with_lora && n_rows > 0) ? D.base_slices : 0;
    return D;
}

size_t decode_ws_bytes(const PoolDev& P, int32_t n_rows, const DecodePlan& D) {
    const size_t base = align_up((size_t)D.base_slices * n_rows * P.d_out * 4, 256);
    const size_t t = align_up((size_t)D.t_slices * n_rows * 64 * 4, 256);
    const size_t rows = D.t_slices ? align_up((size_t)n_rows * sizeof(RowRec), 256) : 0;
    return base + t + rows;
}

void decode_carve(const PoolDev& P, int32_t n_rows, const DecodePlan& D, void* ws, DecodeArgs& g) {
    uint8_t* w = (uint8_t*)ws;
    const size_t base = align_up((size_t)D.base_slices * n_rows * P.d_out * 4, 256);
    const size_t t = align_up((size_t)D.t_slices * n_rows * 64 * 4, 256);
    g.part_base = (float*)w;
    g.part_t = (float*)(w + base);
    g.rows = (RowRec*)(w + base + t);
}

hipError_t launch_decode_stream(const PoolDev& P, const DecodePlan& D, const DecodeArgs& g,
                                hipStream_t stream) {
    dim3 grid((unsigned)D.base_wgs);
    const int MB = g.n <= 16 ? 1 : (g.n <= 32 ? 2 : 4);
#define LORA_DS(mb)                                                                                        \
    if (g.w_q4) {                                                                                          \
        if (g.with_lora)                                                                                   \
            hipLaunchKernelGGL((k_decode_stream<mb, true, true>), grid, dim3(DS_THREADS), 0, stream, P, D, \
                               g);                                                                         \
        else                                                                                               \
            hipLaunchKernelGGL((k_decode_stream<mb, false, true>), grid, dim3(DS_BASE_THREADS), 0, stream, \
                               P, D, g);                                                                   \
    } else if (g.with_lora)                                                                                \
        hipLaunchKernelGGL((k_decode_stream<mb, true>), grid, dim3(DS_THREADS), 0, stream, P, D, g);       \
    else                                                                                                   \
        hipLaunchKernelGGL((k_decode_stream<mb, false>), grid, dim3(DS_BASE_THREADS), 0, stream, P, D, g)
    if (MB == 1) {
        LORA_DS(1);
    } else if (MB == 2) {
        LORA_DS(2);
    } else {
        LORA_DS(4);
    }
#undef LORA_DS
    return hipGetLastError();
}

hipError_t launch_decode_finish(const PoolDev& P, const DecodePlan& D, const DecodeArgs& g,
                                lora_dtype_t ydt, hipStream_t stream) {
    const int nch = (int)ceil_div(P.d_out, FIN_COLS);
    dim3 grid((unsigned)(g.n * nch));
    const bool vec = P.vec_b != 0;   // d_out % 8 == 0 and 16-byte B blocks
#define LORA_FIN(ty, v, l) hipLaunchKernelGGL((k_decode_finish<ty, v, l>), grid, dim3(FIN_THREADS), 0, stream, P, D, g)
    if (ydt == LORA_BF16) {
        if (g.with_lora) {
            if (vec) LORA_FIN(bf16, true, true);
            else LORA_FIN(bf16, false, true);
        } else {
            if (vec) LORA_FIN(bf16, true, false);
            else LORA_FIN(bf16, false, false);
        }
    } else {
        if (g.with_lora) {
            if (vec) LORA_FIN(float, true, true);
            else LORA_FIN(float, false, true);
        } else {
            if (vec) LORA_FIN(float, true, false);
            else LORA_FIN(float, false, false);
        }
    }
#undef LORA_FIN
    return hipGetLastError();
}

}  // namespace lora
