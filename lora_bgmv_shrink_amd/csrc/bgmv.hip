// BGMV: every row gathers its own adapter by index (decode batches).
//
// The per-row form of the batched adapter term ("Serving multiple LoRAs:
// segmented matrix multiplies and adapter scheduling", section "Not merging
// the weights, computing in batches"): row i looks up A and B of adapter a_i
// through the pool tables, forms t_i = x_i A (the rank-r shrink) and later
// adds s * t_i B (the expand).  Neither step has enough arithmetic per byte
// to need the matrix cores; both are limited by how fast the adapter blocks
// stream in ("Serving many LoRA adapters" (blog.ecitis.org), section
// "Batching across different adapters"), so the kernels are organised around
// wide, coalesced loads of A and B and do their sums on the vector units.
#include "lora_internal.hpp"

namespace lora {
namespace {

constexpr int SHRINK_THREADS = 512;     // one workgroup (8 waves) per row
constexpr int SHRINK_LOADS = 16;        // 16-byte loads of A in flight per thread
constexpr int SHRINK_X_FLOATS = 8192;   // x chunk staged in LDS (32 KiB)
constexpr int SHRINK_A_ELEMS = 8192;    // generic path: A chunk staged in LDS
constexpr int SHRINK_XV = 4;            // 16-byte x pieces per thread requested together

// One row of the K-extension operand from the row's t (in LDS), after a
// workgroup barrier.
__device__ __forceinline__ void write_t_ext(bf16* out, float* sv, int r, float s, int cols) {
    __syncthreads();
    for (int c = threadIdx.x; c < cols; c += blockDim.x) out[c] = ext_value_bf16(sv, r, s, c);
}
__device__ __forceinline__ void write_t_ext(float* out, float* sv, int r, float s, int cols) {
    __syncthreads();
    for (int c = threadIdx.x; c < cols; c += blockDim.x) out[c] = ext_value_f32(sv, r, s, c);
}

// x[0:kn] -> xs as fp32 (row start 16-byte aligned): 16-byte pieces, each
// thread's SHRINK_XV pieces requested before any is stored (a loop of
// element loads and stores waited for one round trip per iteration), then
// the elements past the last whole piece.
template <typename T>
__device__ __forceinline__ void stage_x(const T* __restrict__ x, int kn, float* xs, int tid) {
    constexpr int VE = 16 / sizeof(T);
    const int npc = kn / VE;
    for (int p0 = tid; p0 < npc; p0 += SHRINK_THREADS * SHRINK_XV) {
        uint4 v[SHRINK_XV];
#pragma unroll
        for (int q = 0; q < SHRINK_XV; ++q) {
            const int p = p0 + q * SHRINK_THREADS;
            v[q] = *(const uint4*)(x + (int64_t)(p < npc ? p : 0) * VE);
        }
#pragma unroll
        for (int q = 0; q < SHRINK_XV; ++q) {
            const int p = p0 + q * SHRINK_THREADS;
            if (p < npc) {
                union { uint4 u; T e[VE]; } w;
                w.u = v[q];
#pragma unroll
                for (int e = 0; e < VE; ++e) xs[p * VE + e] = to_f32(w.e[e]);
            }
        }
    }
    for (int k = npc * VE + tid; k < kn; k += SHRINK_THREADS) xs[k] = to_f32(x[k]);
}

// Streaming shrink, for ranks where 16-byte vectors tile every k-row
// (r % VE == 0) and a pass of the workgroup covers whole k-rows
// ((SHRINK_THREADS * VE) % r == 0): r in {8, 16, 32, 64} for bf16,
// {4, 8, 16, 32, 64} for fp32.
//
// Row i reads A_a ([d_in, r] row-major, contiguous) once, front to back:
// thread t owns the VE columns j0 = (t % G) * VE (G = r / VE vectors per
// k-row) of k-rows t / G, t / G + KPT, ... (KPT = SHRINK_THREADS / G), and
// keeps SHRINK_LOADS of those loads in flight while the matching x chunk
// is staged in LDS.  Per-thread partial sums are folded over the lanes of a
// wave that share j0 (butterfly), then over the waves in order; the result
// does not depend on timing.
template <typename T>
__global__ __launch_bounds__(SHRINK_THREADS) void k_bgmv_shrink_stream(PoolDev P, const T* __restrict__ x,
                                                                      int64_t ldx,
                                                                      const int32_t* __restrict__ ids,
                                                                      float* __restrict__ t, int64_t ldt,
                                                                      T* __restrict__ t_ext, int64_t lde) {
    constexpr int VE = 16 / sizeof(T);
    __shared__ float xs[SHRINK_X_FLOATS];
    __shared__ float red[SHRINK_THREADS / 64][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int i = blockIdx.x;
    const int a = ids[i];
    const int r_max = P.r_max;
    float* ti = t + (int64_t)i * ldt;
    if (!id_ok(a, P.n_adapters)) {
        if (tid == 0 && a != -1) flag_bad_id(P.err);
        if (tid < r_max) ti[tid] = 0.f;
        return;
    }
    const int r = pool_rank(P, a);
    const int G = r / VE;
    const int KPT = SHRINK_THREADS / G;
    const int KC = KPT * SHRINK_LOADS;   // k-rows per chunk (<= SHRINK_X_FLOATS)
    const int jv = tid % G;
    const int ksub = tid / G;
    const int d_in = P.d_in;
    const T* Au = (const T*)P.A + pool_a_off(P, a) + jv * VE;
    const T* xi = x + (int64_t)i * ldx;

    float acc[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] = 0.f;

    for (int kc0 = 0; kc0 < d_in; kc0 += KC) {
        uint4 av[SHRINK_LOADS];
#pragma unroll
        for (int l = 0; l < SHRINK_LOADS; ++l) {
            const int k = kc0 + ksub + l * KPT;
            // past d_in: read row 0 again; it meets x = 0 below
            av[l] = *(const uint4*)(Au + (int64_t)(k < d_in ? k : 0) * r);
        }
        const int kn = min(KC, d_in - kc0);
        stage_x(xi + kc0, kn, xs, tid);
        __syncthreads();
#pragma unroll
        for (int l = 0; l < SHRINK_LOADS; ++l) {
            const int kk = ksub + l * KPT;
            const float xv = (kk < kn) ? xs[kk] : 0.f;
            union { uint4 u; T e[VE]; } v;
            v.u = av[l];
#pragma unroll
            for (int e = 0; e < VE; ++e) acc[e] += xv * to_f32(v.e[e]);
        }
        __syncthreads();
    }

    // lanes sharing j0 differ in the lane bits >= log2(G)
    for (int d = G; d < 64; d <<= 1)
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[e] += __shfl_xor(acc[e], d, 64);
    if (lane < G)
#pragma unroll
        for (int e = 0; e < VE; ++e) red[wave][lane * VE + e] = acc[e];
    __syncthreads();
    __shared__ float sv[64];
    if (tid < 64) {
        float v = 0.f;
        if (tid < r)
            for (int w = 0; w < SHRINK_THREADS / 64; ++w) v += red[w][tid];
        if (tid < r_max) ti[tid] = v;
        sv[tid] = v;
    }
    if (t_ext) write_t_ext(t_ext + (int64_t)i * lde, sv, r, P.scales[a], ext_cols(sizeof(T), r_max));
}

// Generic shrink for any rank 1..64: k-chunks of A_a are staged in LDS and
// thread (j, g) sums column j over k = g, g + Gs, ... (Gs = threads / r),
// then the Gs partial sums are added in order.
template <typename T>
__global__ __launch_bounds__(SHRINK_THREADS) void k_bgmv_shrink_lds(PoolDev P, const T* __restrict__ x,
                                                                   int64_t ldx,
                                                                   const int32_t* __restrict__ ids,
                                                                   float* __restrict__ t, int64_t ldt,
                                                                   T* __restrict__ t_ext, int64_t lde) {
    __shared__ __attribute__((aligned(16))) T as[SHRINK_A_ELEMS];
    __shared__ float xs[SHRINK_A_ELEMS];
    __shared__ float red[SHRINK_THREADS];

    const int tid = threadIdx.x;
    const int i = blockIdx.x;
    const int a = ids[i];
    const int r_max = P.r_max;
    float* ti = t + (int64_t)i * ldt;
    if (!id_ok(a, P.n_adapters)) {
        if (tid == 0 && a != -1) flag_bad_id(P.err);
        if (tid < r_max) ti[tid] = 0.f;
        return;
    }
    const int r = P.ranks[a];
    const int d_in = P.d_in;
    const int KC = SHRINK_A_ELEMS / r / 8 * 8;   // k-rows per chunk, multiple of 8
    const T* Au = (const T*)P.A + P.a_off[a];
    const T* xi = x + (int64_t)i * ldx;
    const int Gs = SHRINK_THREADS / r;
    const int j = tid % r;
    const int g = tid / r;
    constexpr int VE = 16 / sizeof(T);
    float acc = 0.f;
    for (int k0 = 0; k0 < d_in; k0 += KC) {
        const int nk = min(KC, d_in - k0);
        const int F = nk * r;
        const T* src = Au + (int64_t)k0 * r;
        int done = 0;
        if (P.vec_a) {   // block start 16-byte aligned and k0 * r * elem a multiple of 16
            const int nv = F / VE;
            // SHRINK_XV pieces per thread requested before any is stored
            for (int v0 = tid; v0 < nv; v0 += SHRINK_THREADS * SHRINK_XV) {
                uint4 w[SHRINK_XV];
#pragma unroll
                for (int q = 0; q < SHRINK_XV; ++q) {
                    const int v = v0 + q * SHRINK_THREADS;
                    w[q] = *(const uint4*)(src + (int64_t)(v < nv ? v : 0) * VE);
                }
#pragma unroll
                for (int q = 0; q < SHRINK_XV; ++q) {
                    const int v = v0 + q * SHRINK_THREADS;
                    if (v < nv) *(uint4*)(as + v * VE) = w[q];
                }
            }
            done = nv * VE;
        }
        for (int e = done + tid; e < F; e += SHRINK_THREADS) as[e] = src[e];
        stage_x(xi + k0, nk, xs, tid);
        __syncthreads();
        if (g < Gs)
            for (int k = g; k < nk; k += Gs) acc += xs[k] * to_f32(as[k * r + j]);
        __syncthreads();
    }
    red[tid] = (g < Gs) ? acc : 0.f;
    __syncthreads();
    __shared__ float sv[64];
    if (tid < 64) {
        float v = 0.f;
        if (tid < r)
            for (int q = 0; q < Gs; ++q) v += red[q * r + tid];
        if (tid < r_max) ti[tid] = v;
        sv[tid] = v;
    }
    if (t_ext) write_t_ext(t_ext + (int64_t)i * lde, sv, r, P.scales[a], ext_cols(sizeof(T), r_max));
}

// Expand.  One wave per (row, chunk of 64*VE output columns); lane l owns VE
// consecutive columns and streams the matching 16-byte pieces of the r rows
// of B_a:  y_i[c] (+)= s_a * sum_j t_i[j] * B_a[j][c].
template <typename T, typename TY>
__global__ __launch_bounds__(256) void k_bgmv_expand(PoolDev P, const float* __restrict__ t,
                                                     int64_t ldt, const int32_t* __restrict__ ids,
                                                     int n, TY* __restrict__ y, int64_t ldy,
                                                     int accumulate, int vec_y, int n_chunks) {
    constexpr int VE = 16 / sizeof(T);
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int rg = blockIdx.x / n_chunks;
    const int ch = blockIdx.x - rg * n_chunks;
    const int i = rg * 4 + wave;
    if (i >= n) return;
    const int d_out = P.d_out;
    const int c0 = (ch * 64 + lane) * VE;
    if (c0 >= d_out) return;
    const int a = ids[i];
    TY* yi = y + (int64_t)i * ldy;
    const bool full = (c0 + VE <= d_out);

    float acc[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] = 0.f;

    if (!id_ok(a, P.n_adapters)) {
        if (lane == 0 && ch == 0 && a != -1) flag_bad_id(P.err);
        if (accumulate) return;
    } else {
        const int r = P.ranks[a];
        const float sc = P.scales[a];
        const T* Bu = (const T*)P.B + P.b_off[a] + c0;
        const float* ti = t + (int64_t)i * ldt;
        constexpr int RC = 16;   // rank rows requested together
        for (int j0 = 0; j0 < r; j0 += RC) {
            uint4 bv[RC];
            float tv[RC];
#pragma unroll
            for (int q = 0; q < RC; ++q) {
                const int j = j0 + q;
                const T* bj = Bu + (int64_t)j * d_out;
                tv[q] = (j < r) ? ti[j] : 0.f;
                if (j < r && full && P.vec_b) {
                    bv[q] = *(const uint4*)bj;
                } else {
                    union { uint4 u; T e[VE]; } w;
                    for (int e = 0; e < VE; ++e) w.e[e] = (j < r && c0 + e < d_out) ? bj[e] : (T)0;
                    bv[q] = w.u;
                }
            }
#pragma unroll
            for (int q = 0; q < RC; ++q) {
                union { uint4 u; T e[VE]; } w;
                w.u = bv[q];
#pragma unroll
                for (int e = 0; e < VE; ++e) acc[e] += tv[q] * to_f32(w.e[e]);
            }
        }
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[e] *= sc;
    }
    if (full && vec_y && (int)(16 / sizeof(TY)) <= VE) {
        // VE * sizeof(TY) bytes per lane: one or two 16-byte stores
        constexpr int YV = 16 / sizeof(TY);
#pragma unroll
        for (int h = 0; h < VE / YV; ++h) {
            union { uint4 u; TY e[YV]; } o;
            if (accumulate) o.u = *(const uint4*)(yi + c0 + h * YV);
#pragma unroll
            for (int e = 0; e < YV; ++e) {
                float v = acc[h * YV + e];
                if (accumulate) v += to_f32(o.e[e]);
                o.e[e] = from_f32<TY>(v);
            }
            *(uint4*)(yi + c0 + h * YV) = o.u;
        }
    } else {
        for (int e = 0; e < VE; ++e) {
            if (c0 + e >= d_out) break;
            float v = acc[e];
            if (accumulate) v += to_f32(yi[c0 + e]);
            yi[c0 + e] = from_f32<TY>(v);
        }
    }
}

}  // namespace

BgmvShrinkPlan plan_bgmv_shrink(const PoolDev& P, int, int32_t) {
    // The streaming kernel needs every rank in the pool to tile 16-byte
    // vectors and whole k-rows per pass; uniform pools check one rank.
    BgmvShrinkPlan plan;
    plan.ks = (P.vec_a && P.stream_ok) ? 1 : 0;
    return plan;
}

hipError_t launch_bgmv_shrink(const PoolDev& P, lora_dtype_t dt, const void* x, int64_t ldx,
                              const int32_t* ids, int32_t n_rows, float* t, int64_t ldt,
                              const BgmvShrinkPlan& plan, hipStream_t stream, void* t_ext, int64_t lde) {
    dim3 grid((unsigned)n_rows);
    const bool stream_path = plan.ks == 1;
    if (dt == LORA_BF16) {
        if (stream_path)
            hipLaunchKernelGGL(k_bgmv_shrink_stream<bf16>, grid, dim3(SHRINK_THREADS), 0, stream, P,
                               (const bf16*)x, ldx, ids, t, ldt, (bf16*)t_ext, lde);
        else
            hipLaunchKernelGGL(k_bgmv_shrink_lds<bf16>, grid, dim3(SHRINK_THREADS), 0, stream, P,
                               (const bf16*)x, ldx, ids, t, ldt, (bf16*)t_ext, lde);
    } else {
        if (stream_path)
            hipLaunchKernelGGL(k_bgmv_shrink_stream<float>, grid, dim3(SHRINK_THREADS), 0, stream, P,
                               (const float*)x, ldx, ids, t, ldt, (float*)t_ext, lde);
        else
            hipLaunchKernelGGL(k_bgmv_shrink_lds<float>, grid, dim3(SHRINK_THREADS), 0, stream, P,
                               (const float*)x, ldx, ids, t, ldt, (float*)t_ext, lde);
    }
    return hipGetLastError();
}

// t_ext from an existing t: one workgroup per row.
template <typename T>
__global__ __launch_bounds__(256) void k_make_t_ext(PoolDev P, const float* __restrict__ t, int64_t ldt,
                                                    const int32_t* __restrict__ ids, T* __restrict__ t_ext,
                                                    int64_t lde) {
    __shared__ float sv[64];
    const int i = blockIdx.x;
    const int a = ids[i];
    if (!id_ok(a, P.n_adapters)) return;
    const int r = P.ranks[a];
    if (threadIdx.x < 64) sv[threadIdx.x] = (threadIdx.x < r) ? t[(int64_t)i * ldt + threadIdx.x] : 0.f;
    write_t_ext(t_ext + (int64_t)i * lde, sv, r, P.scales[a], ext_cols(sizeof(T), P.r_max));
}

hipError_t launch_make_t_ext(const PoolDev& P, lora_dtype_t dt, const float* t, int64_t ldt,
                             const int32_t* ids, int32_t n_rows, void* t_ext, int64_t lde,
                             hipStream_t stream) {
    if (dt == LORA_BF16)
        hipLaunchKernelGGL(k_make_t_ext<bf16>, dim3((unsigned)n_rows), dim3(256), 0, stream, P, t, ldt, ids,
                           (bf16*)t_ext, lde);
    else
        hipLaunchKernelGGL(k_make_t_ext<float>, dim3((unsigned)n_rows), dim3(256), 0, stream, P, t, ldt, ids,
                           (float*)t_ext, lde);
    return hipGetLastError();
}

hipError_t launch_bgmv_expand(const PoolDev& P, lora_dtype_t dt, const float* t, int64_t ldt,
                              const int32_t* ids, int32_t n_rows, void* y, lora_dtype_t ydt,
                              int64_t ldy, int accumulate, bool vec_y, hipStream_t stream) {
    const int VE = (dt == LORA_BF16) ? 8 : 4;
    const int n_chunks = (int)ceil_div(P.d_out, 64 * VE);
    dim3 grid((unsigned)(ceil_div(n_rows, 4) * n_chunks));
    const int vy = vec_y ? 1 : 0;
    if (dt == LORA_BF16) {
        if (ydt == LORA_BF16)
            hipLaunchKernelGGL((k_bgmv_expand<bf16, bf16>), grid, dim3(256), 0, stream, P, t, ldt, ids,
                               n_rows, (bf16*)y, ldy, accumulate, vy, n_chunks);
        else
            hipLaunchKernelGGL((k_bgmv_expand<bf16, float>), grid, dim3(256), 0, stream, P, t, ldt,
                               ids, n_rows, (float*)y, ldy, accumulate, vy, n_chunks);
    } else {
        if (ydt == LORA_BF16)
            hipLaunchKernelGGL((k_bgmv_expand<float, bf16>), grid, dim3(256), 0, stream, P, t, ldt,
                               ids, n_rows, (bf16*)y, ldy, accumulate, vy, n_chunks);
        else
            hipLaunchKernelGGL((k_bgmv_expand<float, float>), grid, dim3(256), 0, stream, P, t, ldt,
                               ids, n_rows, (float*)y, ldy, accumulate, vy, n_chunks);
    }
    return hipGetLastError();
}

}  // namespace lora
