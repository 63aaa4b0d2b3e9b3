// BGMV: every row gathers its own adapter by index (decode batches).
//
// "Serving multiple LoRAs: segmented matrix multiplies and adapter
// scheduling", section "Not merging the weights, computing in batches": each
// token gathers its adapter's A and B by index and does a small
// matrix-vector product; the shrink (x -> xA, rank r) runs first, then the
// expand ((xA) -> (xA)B).  The adapter term is bound by reading A and B
// ("Serving many LoRA adapters" (blog.ecitis.org), section "Batching across
// different adapters"), so both kernels are built around wide, coalesced
// streaming of the adapter blocks; their arithmetic is VALU.
#include "lora_internal.hpp"

namespace lora {
namespace {

constexpr int SHRINK_THREADS = 256;
constexpr int SHRINK_A_BYTES = 32768;   // LDS staging of one slice of A
constexpr int SHRINK_KS_MAX = 256;      // k-rows per slice (x staged in LDS)
constexpr int SHRINK_PART_STRIDE = 64;  // floats per (row, slice) partial

// Shrink.  Workgroup b handles row i = b / S, K-slice s = b % S:
//   partial_s[j] = sum_{k in slice} x_i[k] * A_a[k][j]
// The slice of A is contiguous ([Ks, r] row-major) and is copied to LDS with
// 16-byte loads; thread (j, g) then sums k = g, g + G, ... for column j, and
// the G partial sums are added in order.  With S > 1 the slices of a row meet
// in a last-arriver step: each slice writes its partial to the workspace, and
// the slice that increments the row's counter last adds the S partials in
// slice order (deterministic) and resets the counter to zero.
template <typename T>
__global__ __launch_bounds__(SHRINK_THREADS) void k_bgmv_shrink(PoolDev P, const T* __restrict__ x,
                                                               int64_t ldx,
                                                               const int32_t* __restrict__ ids,
                                                               float* __restrict__ t, int64_t ldt,
                                                               int S, int Ks,
                                                               float* __restrict__ part,
                                                               int32_t* __restrict__ cnt) {
    __shared__ float xs[SHRINK_KS_MAX];
    __shared__ __attribute__((aligned(16))) T as[SHRINK_A_BYTES / sizeof(T)];
    __shared__ float red[SHRINK_THREADS];
    __shared__ int is_last;

    const int tid = threadIdx.x;
    const int i = blockIdx.x / S;
    const int s = blockIdx.x - i * S;
    const int a = ids[i];
    const int r_max = P.r_max;
    float* ti = t + (int64_t)i * ldt;

    if (!id_ok(a, P.n_adapters)) {
        if (s == 0) {
            if (tid == 0 && a != -1) flag_bad_id(P.err);
            if (tid < r_max) ti[tid] = 0.f;
        }
        return;
    }
    const int r = P.ranks[a];
    const int k0 = s * Ks;
    const int k1 = min(P.d_in, k0 + Ks);
    const int nk = k1 - k0;

    const T* xi = x + (int64_t)i * ldx + k0;
    for (int k = tid; k < nk; k += SHRINK_THREADS) xs[k] = to_f32(xi[k]);

    const T* src = (const T*)P.A + P.a_off[a] + (int64_t)k0 * r;
    const int F = nk * r;
    constexpr int VE = 16 / sizeof(T);
    int done = 0;
    if (P.vec_a) {
        const int nv = F / VE;
        for (int v = tid; v < nv; v += SHRINK_THREADS)
            *(uint4*)(as + v * VE) = *(const uint4*)(src + v * VE);
        done = nv * VE;
    }
    for (int e = done + tid; e < F; e += SHRINK_THREADS) as[e] = src[e];
    __syncthreads();

    const int G = SHRINK_THREADS / r;
    float acc = 0.f;
    if (tid < G * r) {
        const int j = tid % r;
        const int g = tid / r;
        for (int k = g; k < nk; k += G) acc += xs[k] * to_f32(as[k * r + j]);
    }
    red[tid] = acc;
    __syncthreads();
    float v = 0.f;
    if (tid < r)
        for (int g = 0; g < G; ++g) v += red[g * r + tid];

    if (S == 1) {
        if (tid < r_max) ti[tid] = (tid < r) ? v : 0.f;
        return;
    }
    if (tid < r) part[((int64_t)i * S + s) * SHRINK_PART_STRIDE + tid] = v;
    __threadfence();   // every writer releases its own partial at device scope
    __syncthreads();
    if (tid == 0) {
        // release our partial, acquire the others' if we arrive last
        const int prev = __hip_atomic_fetch_add(&cnt[i], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        is_last = (prev == S - 1);
    }
    __syncthreads();
    if (!is_last) return;
    __atomic_thread_fence(__ATOMIC_ACQUIRE);
    if (tid < r_max) {
        float sum = 0.f;
        if (tid < r) {
            const float* p = part + (int64_t)i * S * SHRINK_PART_STRIDE + tid;
            for (int q = 0; q < S; ++q)
                sum += __hip_atomic_load(p + q * SHRINK_PART_STRIDE, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
        }
        ti[tid] = sum;
    }
    if (tid == 0) __hip_atomic_store(&cnt[i], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
        for (int j = 0; j < r; ++j) {
            const float tj = ti[j];
            const T* bj = Bu + (int64_t)j * d_out;
            if (full && P.vec_b) {
                union { uint4 u; T e[VE]; } v;
                v.u = *(const uint4*)bj;
#pragma unroll
                for (int e = 0; e < VE; ++e) acc[e] += tj * to_f32(v.e[e]);
            } else {
                for (int e = 0; e < VE; ++e)
                    if (c0 + e < d_out) acc[e] += tj * to_f32(bj[e]);
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

BgmvShrinkPlan plan_bgmv_shrink(const PoolDev& P, int elem_bytes, int32_t n_rows) {
    // Largest slice the LDS staging buffer holds at the pool's widest rank.
    int ks_max = SHRINK_A_BYTES / (elem_bytes * P.r_max);
    ks_max = std::min(ks_max, SHRINK_KS_MAX) / 8 * 8;
    if (ks_max < 8) ks_max = 8;
    // Aim for about 1024 workgroups in flight, but no slice under 128 rows.
    int64_t want = std::max<int64_t>(1, ceil_div(1024, std::max(1, n_rows)));
    int64_t most = std::max<int64_t>(1, ceil_div(P.d_in, 128));
    int64_t s = std::min(want, most);
    s = std::max<int64_t>(s, ceil_div(P.d_in, ks_max));
    int ks = (int)align_up((size_t)ceil_div(P.d_in, s), 8);
    if (ks > ks_max) ks = ks_max;
    s = ceil_div(P.d_in, ks);
    return BgmvShrinkPlan{(int32_t)s, ks};
}

size_t bgmv_shrink_ws_bytes(const BgmvShrinkPlan& plan, int32_t n_rows) {
    if (plan.slices <= 1 || n_rows <= 0) return 0;
    size_t part = align_up((size_t)n_rows * plan.slices * SHRINK_PART_STRIDE * sizeof(float), 256);
    size_t cnt = align_up((size_t)n_rows * sizeof(int32_t), 256);
    return part + cnt;
}

hipError_t launch_bgmv_shrink(const PoolDev& P, lora_dtype_t dt, const void* x, int64_t ldx,
                              const int32_t* ids, int32_t n_rows, float* t, int64_t ldt, void* ws,
                              const BgmvShrinkPlan& plan, hipStream_t stream) {
    float* part = nullptr;
    int32_t* cnt = nullptr;
    if (plan.slices > 1) {
        part = (float*)ws;
        cnt = (int32_t*)((char*)ws + align_up((size_t)n_rows * plan.slices * SHRINK_PART_STRIDE *
                                                  sizeof(float), 256));
    }
    dim3 grid((unsigned)((int64_t)n_rows * plan.slices));
    if (dt == LORA_BF16)
        hipLaunchKernelGGL(k_bgmv_shrink<bf16>, grid, dim3(SHRINK_THREADS), 0, stream, P,
                           (const bf16*)x, ldx, ids, t, ldt, plan.slices, plan.ks, part, cnt);
    else
        hipLaunchKernelGGL(k_bgmv_shrink<float>, grid, dim3(SHRINK_THREADS), 0, stream, P,
                           (const float*)x, ldx, ids, t, ldt, plan.slices, plan.ks, part, cnt);
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
