// C ABI of liblora_mi355x: argument checks, pool tables, workspace layout and
// dispatch.  The semantics of every entry point are documented in
// include/lora_mi355x.h.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "lora_internal.hpp"
#include "pool.hpp"

using namespace lora;


namespace {

constexpr int kMaxRank = 64;
constexpr int kMaxAdaptersSegments = 16383;
constexpr int64_t kRaggedAlignElems = 128;   // 256 B in bf16, 512 B in fp32

int elem_bytes(lora_dtype_t d) { return d == LORA_BF16 ? 2 : 4; }
// Enum arguments come from C callers and may hold any int: validate their
// bits as an int (a value past the enumerators is not a valid enum value in
// C++, so it must not be read as one), then use the enum.
// (taken by reference: even copying an invalid value is a load of it)
template <typename E>
int raw(const E& e) {
    static_assert(sizeof(E) == sizeof(int), "enum arguments are int-sized");
    int v = 0;
    std::memcpy(&v, &e, sizeof v);
    return v;
}
bool dtype_ok(const lora_dtype_t& d) { return raw(d) == LORA_F32 || raw(d) == LORA_BF16; }
bool mode_ok(const lora_mode_t& m) {
    return raw(m) == LORA_MODE_AUTO || raw(m) == LORA_MODE_BGMV || raw(m) == LORA_MODE_SGMV;
}
bool w_layout_ok(const lora_w_layout_t& w) { return raw(w) == LORA_W_IN_OUT || raw(w) == LORA_W_OUT_IN; }
bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool ld_ok(int64_t ld, int64_t minv, int eb) { return ld >= minv && (ld * eb) % 16 == 0; }

lora_status_t dev_status(hipError_t e) { return e == hipSuccess ? LORA_OK : LORA_E_DEVICE; }

// Rank stride of the fp32 intermediate t inside layer workspaces.
int64_t t_stride(int32_t r_max) { return (int64_t)align_up((size_t)r_max, 4); }

// Bytes of the GEMM's K-extension operand for n_rows rows.
size_t ext_bytes(const lora_pool_s* pool, int32_t n_rows) {
    const int eb = pool->dtype == LORA_BF16 ? 2 : 4;
    return align_up((size_t)n_rows * ext_cols(eb, pool->dev.r_max) * eb, 256);
}

__global__ void k_fill_zero(uint4* __restrict__ p, size_t n16, uint8_t* __restrict__ tail,
                            size_t n_tail) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t k = i; k < n16; k += stride) p[k] = uint4{0u, 0u, 0u, 0u};
    if (i < n_tail) tail[i] = 0;
}

struct SegLayout {
    size_t perm, seg_ids, seg_off, n_seg, end;
    int32_t cap;
};

SegLayout seg_layout(size_t base, int32_t n_rows, int32_t n_adapters) {
    SegLayout L;
    L.cap = std::max<int32_t>(1, std::min<int32_t>(n_rows, n_adapters + 1));
    L.perm = align_up(base, 256);
    L.seg_ids = align_up(L.perm + (size_t)n_rows * 4, 256);
    L.seg_off = align_up(L.seg_ids + (size_t)L.cap * 4, 256);
    L.n_seg = align_up(L.seg_off + (size_t)(L.cap + 1) * 4, 256);
    L.end = align_up(L.n_seg + 4, 256);
    return L;
}

lora_status_t check_segments(const lora_segments_t* seg, int32_t n_rows, int32_t n_adapters) {
    if (!seg || !seg->seg_ids || !seg->seg_off || !seg->n_seg) return LORA_E_INVALID;
    if (n_rows > 0 && !seg->perm) return LORA_E_INVALID;
    if (seg->cap < std::min<int32_t>(n_rows, n_adapters + 1)) return LORA_E_INVALID;
    return LORA_OK;
}

lora_status_t check_pool(lora_pool_t p) { return p ? LORA_OK : LORA_E_INVALID; }

constexpr int32_t kDecodeMaxRows = 64;

bool decode_ok(const lora_pool_s* pool, int32_t n_rows) {
    return pool->dtype == LORA_BF16 && n_rows >= 1 && n_rows <= kDecodeMaxRows;
}

// BGMV batches of 65..kRowsMaxRows rows of a bf16 pool with W stored
// [d_out, d_in] take the few-hundred-row path (rows.hip): segments, the
// shrink per segment tile, the base product in split-K partial sums, and a
// finish that adds the partials and the scaled expand per segment tile.
constexpr int32_t kRowsMaxRows = 1024;

bool rows_ok(const lora_pool_s* pool, int32_t n_rows) {
    return pool->dtype == LORA_BF16 && n_rows > kDecodeMaxRows && n_rows <= kRowsMaxRows &&
           pool->dev.n_adapters <= kMaxAdaptersSegments;
}

// workspace of the few-hundred-row path: segments, then the plan's partials
// and row records
size_t rows_ws_bytes(const lora_pool_s* pool, int32_t n_rows, bool q4 = false) {
    const RowsPlan R = plan_rows(pool->dev, n_rows, q4);
    return align_up(seg_layout(0, n_rows, pool->dev.n_adapters).end, 256) + R.bytes;
}

// The few-hundred-row path, up to kRowsMaxRows rows (also the 4-bit base
// there).  seg:
// caller's segments of these ids, or NULL (built at the start of the
// workspace).  q4: W is 4-bit bytes with fp32 scales wscale [d_out][lds].
hipError_t run_rows(const lora_pool_s* pool, const void* x, int64_t ldx, const void* W, int64_t ldw,
                    const float* wscale, int64_t lds, bool q4, const int32_t* ids, const lora_segments_t* seg,
                    int32_t n_rows, void* y, lora_dtype_t y_dtype, int64_t ldy, void* ws, hipStream_t stream) {
    const PoolDev& P = pool->dev;
    uint8_t* base = (uint8_t*)ws;
    const SegLayout L = seg_layout(0, n_rows, P.n_adapters);
    lora_segments_t own;
    hipError_t e = hipSuccess;
    if (!seg) {
        own.perm = (int32_t*)(base + L.perm);
        own.seg_ids = (int32_t*)(base + L.seg_ids);
        own.seg_off = (int32_t*)(base + L.seg_off);
        own.n_seg = (int32_t*)(base + L.n_seg);
        own.cap = L.cap;
        e = launch_segments(ids, n_rows, P.n_adapters, &own, P.err, stream);
        seg = &own;
    }
    const RowsPlan R = plan_rows(P, n_rows, q4);
    uint8_t* rb = base + align_up(L.end, 256);
    float* part = (float*)(rb + R.part_off);
    float* tpart = (float*)(rb + R.tpart_off);
    if (e == hipSuccess)
        e = launch_rows_adapter(P, R, x, ldx, ids, seg, n_rows, part, tpart, y, y_dtype, ldy, stream, true, false);
    if (e == hipSuccess) e = launch_rows_gemm(P, R, x, ldx, W, ldw, wscale, lds, q4, n_rows, part, stream);
    if (e == hipSuccess)
        e = launch_rows_adapter(P, R, x, ldx, ids, seg, n_rows, part, tpart, y, y_dtype, ldy, stream, false, true);
    return e;
}

// The shrink (BGMV per row, or segments and the SGMV shrink) and the fused
// GEMM (x W plus the adapter term, y rounded once).  q4: W is 4-bit bytes
// stored [d_out, d_in] with fp32 scales wscale [d_out][lds] (SGMV only).
hipError_t run_fused(const lora_pool_s* pool, lora_mode_t m, const void* x, int64_t ldx, const void* W,
                     int64_t ldw, bool w_out_in, const float* wscale, int64_t lds, const int32_t* ids,
                     const lora_segments_t* seg, int32_t n_rows, void* y, lora_dtype_t y_dtype, int64_t ldy,
                     void* ws, hipStream_t stream) {
    const PoolDev& P = pool->dev;
    const int eb = elem_bytes(pool->dtype);
    uint8_t* base = (uint8_t*)ws;
    float* t = (float*)base;
    const int64_t ldt = t_stride(P.r_max);
    void* t_ext = base + align_up((size_t)n_rows * ldt * 4, 256);
    const int64_t lde = ext_cols(eb, P.r_max);
    const size_t after_t = align_up((size_t)n_rows * ldt * 4, 256) + ext_bytes(pool, n_rows);
    hipError_t e = hipSuccess;
    const int32_t* gemm_perm = nullptr;   // SGMV: the GEMM visits rows grouped by adapter
    size_t end = after_t;                  // end of this mode's layout; the GEMM's split partials follow
    if (m == LORA_MODE_BGMV) {
        BgmvShrinkPlan plan = plan_bgmv_shrink(P, eb, n_rows);
        e = launch_bgmv_shrink(P, pool->dtype, x, ldx, ids, n_rows, t, ldt, plan, stream, t_ext, lde);
    } else {
        lora_segments_t own;
        const lora_segments_t* sg = seg;
        const SegLayout SL = seg_layout(after_t, n_rows, P.n_adapters);
        float* part = sgmv_shrink_part_bytes(P, n_rows) ? (float*)(base + SL.end) : nullptr;
        end = SL.end + sgmv_shrink_part_bytes(P, n_rows);
        if (!sg) {
            SegLayout L = SL;
            own.perm = (int32_t*)(base + L.perm);
            own.seg_ids = (int32_t*)(base + L.seg_ids);
            own.seg_off = (int32_t*)(base + L.seg_off);
            own.n_seg = (int32_t*)(base + L.n_seg);
            own.cap = L.cap;
            e = launch_segments(ids, n_rows, P.n_adapters, &own, P.err, stream);
            sg = &own;
        }
        if (e == hipSuccess)
            e = launch_sgmv_shrink(P, pool->dtype, x, ldx, sg, n_rows, P.n_adapters + 1, t, ldt, true,
                                   stream, t_ext, lde, ids, part);
        if ((int64_t)n_rows * ldx * eb < ((int64_t)1 << 31)) gemm_perm = sg->perm;
    }
    if (e != hipSuccess) return e;
    GemmArgs g;
    g.x = x;
    g.ldx = ldx;
    g.W = W;
    g.ldw = ldw;
    g.w_out_in = w_out_in ? 1 : 0;
    g.w_q4 = wscale != nullptr;
    g.wscale = wscale;
    g.lds = lds;
    g.ids = ids;
    g.n_rows = n_rows;
    g.t = t;
    g.ldt = ldt;
    g.t_ext = t_ext;
    g.lde = lde;
    g.y = y;
    g.ldy = ldy;
    g.vec_x = true;
    g.vec_w = true;
    g.rows_distinct = (m == LORA_MODE_BGMV);
    g.perm = gemm_perm;
    g.x_rows = n_rows;
    if (pool->dtype == LORA_BF16) {
        g.split_bytes = layer_gemm_split_bytes(P, n_rows);
        g.split_part = g.split_bytes ? (float*)(base + align_up(end, 256)) : nullptr;
    }
    return launch_layer_gemm(P, pool->dtype, y_dtype, g, stream);
}

lora_mode_t resolve_mode(lora_mode_t m, int32_t n_rows, int32_t n_adapters) {
    if (m != LORA_MODE_AUTO) return m;
    return (n_rows <= 64 || n_rows <= 2 * (int64_t)n_adapters) ? LORA_MODE_BGMV : LORA_MODE_SGMV;
}

}  // namespace

namespace lora {
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream) {
    if (bytes == 0) return hipSuccess;
    const size_t n16 = bytes / 16;
    const size_t n_tail = bytes - n16 * 16;
    const size_t blocks = std::min<size_t>(std::max<size_t>(1, ceil_div((int64_t)n16, 256)), 4096);
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, stream, (uint4*)p, n16,
                       (uint8_t*)p + n16 * 16, n_tail);
    return hipGetLastError();
}
}  // namespace lora

// Scratch of lora_layer_apply_noalloc: one copy of this array per device,
// held by the device from the library's first use there until the process
// ends.  In host code `scratch` is only a stand-in for the symbol: its device
// address comes from hipGetSymbolAddress, once per device, and only that
// address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[LORA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the stream's device (fetched with that
// device current on first use, then kept).
lora_status_t scratch_address(hipStream_t stream, void** out) {
    int dev = -1;
    if (stream) {
        if (hipStreamGetDevice(stream, &dev) != hipSuccess) return LORA_E_DEVICE;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return LORA_E_DEVICE;
    }
    if (dev < 0 || dev >= kMaxDevices) return LORA_E_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return LORA_E_DEVICE;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return LORA_E_DEVICE;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return LORA_E_DEVICE;
        if (e != hipSuccess || !p) return LORA_E_DEVICE;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return LORA_OK;
}

}  // namespace

extern "C" {

const char* lora_status_string(lora_status_t status) {
    // a caller may pass any int: read the bits as an int, not as the enum
    // (values past the enumerators are not valid enum values in C++)
    int s = 0;
    std::memcpy(&s, &status, sizeof s);
    switch (s) {
        case LORA_OK: return "LORA_OK";
        case LORA_E_INVALID: return "LORA_E_INVALID: invalid argument";
        case LORA_E_UNSUPPORTED: return "LORA_E_UNSUPPORTED: valid but unsupported (alignment, rank, size)";
        case LORA_E_WORKSPACE: return "LORA_E_WORKSPACE: workspace missing or too small";
        case LORA_E_ID_RANGE: return "LORA_E_ID_RANGE: an adapter id was outside [-1, n_adapters)";
        case LORA_E_DEVICE: return "LORA_E_DEVICE: a HIP runtime call failed";
        case LORA_E_NOT_RESIDENT: return "LORA_E_NOT_RESIDENT: an adapter of the batch is not resident";
        case LORA_E_SCRATCH:
            return "LORA_E_SCRATCH: the call needs more scratch than the static array holds "
                   "(LORA_NOALLOC_SCRATCH_BYTES); use lora_layer_apply with a workspace";
    }
    return "unknown lora_status_t";
}

int64_t lora_adapter_param_count(int32_t rank, int32_t d_in, int32_t d_out) {
    if (rank <= 0 || d_in <= 0 || d_out <= 0) return -1;
    return (int64_t)rank * ((int64_t)d_in + (int64_t)d_out);
}

lora_status_t lora_pool_ragged_offsets(int32_t n_adapters, const int32_t* ranks, int32_t d_in,
                                       int32_t d_out, int64_t* a_off, int64_t* b_off,
                                       int64_t* a_total, int64_t* b_total) {
    if (n_adapters <= 0 || !ranks || d_in <= 0 || d_out <= 0 || !a_off || !b_off)
        return LORA_E_INVALID;
    int64_t pa = 0, pb = 0;
    for (int32_t u = 0; u < n_adapters; ++u) {
        if (ranks[u] < 1) return LORA_E_INVALID;
        if (ranks[u] > kMaxRank) return LORA_E_UNSUPPORTED;
        a_off[u] = pa;
        b_off[u] = pb;
        pa += ceil_div((int64_t)d_in * ranks[u], kRaggedAlignElems) * kRaggedAlignElems;
        pb += ceil_div((int64_t)ranks[u] * d_out, kRaggedAlignElems) * kRaggedAlignElems;
    }
    if (a_total) *a_total = pa;
    if (b_total) *b_total = pb;
    return LORA_OK;
}

lora_status_t lora_pool_create(lora_pool_t* out, lora_layout_t layout, lora_dtype_t dtype,
                               int32_t n_adapters, int32_t d_in, int32_t d_out, int32_t r_max,
                               const int32_t* ranks, const int64_t* a_off, const int64_t* b_off,
                               const void* A, const void* B, const float* scales) {
    if (!out) return LORA_E_INVALID;
    *out = nullptr;
    if (!dtype_ok(dtype) || (raw(layout) != LORA_LAYOUT_UNIFORM && raw(layout) != LORA_LAYOUT_RAGGED))
        return LORA_E_INVALID;
    if (n_adapters <= 0 || d_in <= 0 || d_out <= 0 || r_max <= 0 || !A || !B || !scales)
        return LORA_E_INVALID;
    if (r_max > kMaxRank) return LORA_E_UNSUPPORTED;
    if (!al16(A) || !al16(B)) return LORA_E_UNSUPPORTED;
    const int eb = elem_bytes(dtype);

    std::vector<int32_t> rk(n_adapters);
    std::vector<int64_t> ao(n_adapters), bo(n_adapters);
    if (layout == LORA_LAYOUT_UNIFORM) {
        if (ranks || a_off || b_off) return LORA_E_INVALID;
        for (int32_t u = 0; u < n_adapters; ++u) {
            rk[u] = r_max;
            ao[u] = (int64_t)u * d_in * r_max;
            bo[u] = (int64_t)u * r_max * d_out;
        }
    } else {
        if (!ranks || !a_off || !b_off) return LORA_E_INVALID;
        std::vector<std::pair<int64_t, int64_t>> sa, sb;
        for (int32_t u = 0; u < n_adapters; ++u) {
            if (ranks[u] < 1 || ranks[u] > r_max) return LORA_E_INVALID;
            if (a_off[u] < 0 || b_off[u] < 0) return LORA_E_INVALID;
            if ((a_off[u] * eb) % 16 != 0 || (b_off[u] * eb) % 16 != 0) return LORA_E_UNSUPPORTED;
            rk[u] = ranks[u];
            ao[u] = a_off[u];
            bo[u] = b_off[u];
            sa.push_back({a_off[u], a_off[u] + (int64_t)d_in * ranks[u]});
            sb.push_back({b_off[u], b_off[u] + (int64_t)ranks[u] * d_out});
        }
        std::sort(sa.begin(), sa.end());
        std::sort(sb.begin(), sb.end());
        for (size_t i = 1; i < sa.size(); ++i)
            if (sa[i].first < sa[i - 1].second || sb[i].first < sb[i - 1].second) return LORA_E_INVALID;
    }
    bool vec_a = true, vec_b = ((int64_t)d_out * eb) % 16 == 0, stream_ok = true, vec_rank = true;
    const int ve = 16 / eb;
    for (int32_t u = 0; u < n_adapters; ++u) {
        vec_a = vec_a && (ao[u] * eb) % 16 == 0;
        vec_b = vec_b && (bo[u] * eb) % 16 == 0;
        stream_ok = stream_ok && rk[u] % ve == 0 && (512 * ve) % rk[u] == 0;
        vec_rank = vec_rank && rk[u] % ve == 0;
    }

    const size_t o_ranks = 0;
    const size_t o_aoff = align_up(o_ranks + (size_t)n_adapters * 4, 256);
    const size_t o_boff = align_up(o_aoff + (size_t)n_adapters * 8, 256);
    const size_t o_scales = align_up(o_boff + (size_t)n_adapters * 8, 256);
    const size_t o_err = align_up(o_scales + (size_t)n_adapters * 4, 256);
    const size_t total = o_err + 256;
    std::vector<uint8_t> host(total, 0);
    std::memcpy(host.data() + o_ranks, rk.data(), (size_t)n_adapters * 4);
    std::memcpy(host.data() + o_aoff, ao.data(), (size_t)n_adapters * 8);
    std::memcpy(host.data() + o_boff, bo.data(), (size_t)n_adapters * 8);
    std::memcpy(host.data() + o_scales, scales, (size_t)n_adapters * 4);

    void* mem = nullptr;
    if (hipMalloc(&mem, total) != hipSuccess) return LORA_E_DEVICE;
    if (hipMemcpy(mem, host.data(), total, hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(mem);
        return LORA_E_DEVICE;
    }
    lora_pool_s* p = new lora_pool_s;
    p->owned_by_cache = false;
    p->layout = layout;
    p->dtype = dtype;
    p->ranks = rk;
    p->tables = mem;
    uint8_t* m = (uint8_t*)mem;
    p->dev.A = A;
    p->dev.B = B;
    p->dev.ranks = (const int32_t*)(m + o_ranks);
    p->dev.a_off = (const int64_t*)(m + o_aoff);
    p->dev.b_off = (const int64_t*)(m + o_boff);
    p->dev.scales = (const float*)(m + o_scales);
    p->dev.err = (int32_t*)(m + o_err);
    p->dev.n_adapters = n_adapters;
    p->dev.d_in = d_in;
    p->dev.d_out = d_out;
    p->dev.r_max = r_max;
    p->dev.vec_a = vec_a ? 1 : 0;
    p->dev.vec_b = vec_b ? 1 : 0;
    p->dev.stream_ok = stream_ok ? 1 : 0;
    p->dev.vec_rank = vec_rank ? 1 : 0;
    p->dev.uniform = layout == LORA_LAYOUT_UNIFORM ? 1 : 0;
    *out = p;
    return LORA_OK;
}

lora_status_t lora_pool_destroy(lora_pool_t pool) {
    if (!pool) return LORA_OK;
    if (pool->owned_by_cache) return LORA_E_INVALID;
    hipError_t e = hipDeviceSynchronize();
    hipError_t f = hipFree(pool->tables);
    delete pool;
    return (e == hipSuccess && f == hipSuccess) ? LORA_OK : LORA_E_DEVICE;
}

int64_t lora_pool_param_count(lora_pool_t pool, int32_t adapter) {
    if (!pool || adapter < 0 || adapter >= pool->dev.n_adapters) return -1;
    return lora_adapter_param_count(pool->ranks[adapter], pool->dev.d_in, pool->dev.d_out);
}

lora_status_t lora_pool_last_error(lora_pool_t pool, hipStream_t stream, int32_t* out) {
    if (!pool || !out) return LORA_E_INVALID;
    if (hipStreamSynchronize(stream) != hipSuccess) return LORA_E_DEVICE;
    int32_t v = 0, zero = 0;
    if (hipMemcpy(&v, pool->dev.err, 4, hipMemcpyDeviceToHost) != hipSuccess) return LORA_E_DEVICE;
    if (hipMemcpy(pool->dev.err, &zero, 4, hipMemcpyHostToDevice) != hipSuccess) return LORA_E_DEVICE;
    *out = v;
    return (v & 1) ? LORA_E_ID_RANGE : LORA_OK;
}

lora_status_t lora_workspace_clear(void* ws, size_t bytes, hipStream_t stream) {
    if (bytes == 0) return LORA_OK;
    if (!ws || !al16(ws)) return LORA_E_INVALID;
    return dev_status(launch_fill_zero(ws, bytes, stream));
}

lora_status_t lora_segments_workspace(int32_t n_rows, int32_t n_adapters, size_t* bytes) {
    if (!bytes || n_rows < 0 || n_adapters <= 0) return LORA_E_INVALID;
    if (n_adapters > kMaxAdaptersSegments) return LORA_E_UNSUPPORTED;
    *bytes = 0;
    return LORA_OK;
}

lora_status_t lora_segments_build(const int32_t* ids, int32_t n_rows, int32_t n_adapters,
                                  const lora_segments_t* seg, int32_t* status, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
    (void)ws;
    (void)ws_bytes;
    if (n_rows < 0 || n_adapters <= 0 || (n_rows > 0 && !ids)) return LORA_E_INVALID;
    if (n_adapters > kMaxAdaptersSegments) return LORA_E_UNSUPPORTED;
    lora_status_t st = check_segments(seg, n_rows, n_adapters);
    if (st != LORA_OK) return st;
    return dev_status(launch_segments(ids, n_rows, n_adapters, seg, status, stream));
}

lora_status_t lora_bgmv_shrink(lora_pool_t pool, const void* x, int64_t ldx, const int32_t* ids,
                               int32_t n_rows, float* t, int64_t ldt, hipStream_t stream) {
    if (check_pool(pool) != LORA_OK || n_rows < 0) return LORA_E_INVALID;
    if (n_rows == 0) return LORA_OK;
    const int eb = elem_bytes(pool->dtype);
    if (!x || !ids || !t) return LORA_E_INVALID;
    if (ldx < pool->dev.d_in || ldt < pool->dev.r_max) return LORA_E_INVALID;
    if (!al16(x) || !ld_ok(ldx, pool->dev.d_in, eb)) return LORA_E_UNSUPPORTED;
    BgmvShrinkPlan plan = plan_bgmv_shrink(pool->dev, eb, n_rows);
    return dev_status(launch_bgmv_shrink(pool->dev, pool->dtype, x, ldx, ids, n_rows, t, ldt, plan, stream));
}

lora_status_t lora_bgmv_expand(lora_pool_t pool, const float* t, int64_t ldt, const int32_t* ids,
                               int32_t n_rows, void* y, lora_dtype_t y_dtype, int64_t ldy,
                               int accumulate, hipStream_t stream) {
    if (check_pool(pool) != LORA_OK || n_rows < 0 || !dtype_ok(y_dtype)) return LORA_E_INVALID;
    if (n_rows == 0) return LORA_OK;
    if (!t || !ids || !y || ldt < pool->dev.r_max || ldy < pool->dev.d_out) return LORA_E_INVALID;
    const int ey = elem_bytes(y_dtype);
    if (!al16(y) || !ld_ok(ldy, pool->dev.d_out, ey)) return LORA_E_UNSUPPORTED;
    return dev_status(launch_bgmv_expand(pool->dev, pool->dtype, t, ldt, ids, n_rows, y, y_dtype, ldy,
                                         accumulate ? 1 : 0, true, stream));
}

lora_status_t lora_sgmv_shrink_workspace(lora_pool_t pool, int32_t n_rows, size_t* bytes) {
    if (!pool || !bytes || n_rows < 0) return LORA_E_INVALID;
    *bytes = sgmv_shrink_part_bytes(pool->dev, n_rows);
    return LORA_OK;
}

lora_status_t lora_sgmv_shrink(lora_pool_t pool, const void* x, int64_t ldx,
                               const lora_segments_t* seg, int32_t n_rows, float* t, int64_t ldt,
                               void* ws, size_t ws_bytes, hipStream_t stream) {
    if (check_pool(pool) != LORA_OK || n_rows < 0) return LORA_E_INVALID;
    if (n_rows == 0) return LORA_OK;
    const int eb = elem_bytes(pool->dtype);
    if (!x || !t || ldx < pool->dev.d_in || ldt < pool->dev.r_max) return LORA_E_INVALID;
    lora_status_t st = check_segments(seg, n_rows, pool->dev.n_adapters);
    if (st != LORA_OK) return st;
    if (!al16(x) || !ld_ok(ldx, pool->dev.d_in, eb)) return LORA_E_UNSUPPORTED;
    const size_t need = sgmv_shrink_part_bytes(pool->dev, n_rows);
    float* part = nullptr;
    if (ws) {
        if (!al16(ws) || ws_bytes < need) return LORA_E_WORKSPACE;
        if (need > 0) part = (float*)ws;
    }
    return dev_status(launch_sgmv_shrink(pool->dev, pool->dtype, x, ldx, seg, n_rows,
                                         pool->dev.n_adapters + 1, t, ldt, true, stream, nullptr, 0,
                                         nullptr, part));
}

lora_status_t lora_sgmv_expand(lora_pool_t pool, const float* t, int64_t ldt,
                               const lora_segments_t* seg, int32_t n_rows, void* y,
                               lora_dtype_t y_dtype, int64_t ldy, int accumulate,
                               hipStream_t stream) {
    if (check_pool(pool) != LORA_OK || n_rows < 0 || !dtype_ok(y_dtype)) return LORA_E_INVALID;
    if (n_rows == 0) return LORA_OK;
    if (!t || !y || ldt < pool->dev.r_max || ldy < pool->dev.d_out) return LORA_E_INVALID;
    lora_status_t st = check_segments(seg, n_rows, pool->dev.n_adapters);
    if (st != LORA_OK) return st;
    const int ey = elem_bytes(y_dtype);
    if (!al16(y) || !ld_ok(ldy, pool->dev.d_out, ey)) return LORA_E_UNSUPPORTED;
    return dev_status(launch_sgmv_expand(pool->dev, pool->dtype, t, ldt, seg, n_rows,
                                         pool->dev.n_adapters + 1, y, y_dtype, ldy,
                                         accumulate ? 1 : 0, stream));
}

lora_status_t lora_layer_workspace(lora_pool_t pool, int32_t n_rows, lora_mode_t mode,
                                   size_t* bytes) {
    if (!pool || !bytes || n_rows < 0) return LORA_E_INVALID;
    if (!mode_ok(mode)) return LORA_E_INVALID;
    const lora_mode_t m = resolve_mode(mode, n_rows, pool->dev.n_adapters);
    size_t off = align_up((size_t)n_rows * t_stride(pool->dev.r_max) * 4, 256) + ext_bytes(pool, n_rows);
    // the fused GEMM's K-split partial sums follow the layout of either mode
    const size_t split = pool->dtype == LORA_BF16 ? layer_gemm_split_bytes(pool->dev, n_rows) : 0;
    if (m == LORA_MODE_BGMV) {
        // the W layout is not known here: room for the few-hundred-row path
        // (W stored [d_out, d_in]) and for the fused GEMM (either layout)
        if (split) off = align_up(off, 256) + split;
        if (rows_ok(pool, n_rows)) off = std::max(off, rows_ws_bytes(pool, n_rows));
        if (decode_ok(pool, n_rows))
            off = std::max(off, decode_ws_bytes(pool->dev, n_rows, plan_decode(pool->dev, n_rows, true)));
    } else {
        if (pool->dev.n_adapters > kMaxAdaptersSegments) return LORA_E_UNSUPPORTED;
        off = seg_layout(off, n_rows, pool->dev.n_adapters).end;
        off += sgmv_shrink_part_bytes(pool->dev, n_rows);   // split-K partial sums of the shrink
        if (split) off = align_up(off, 256) + split;
    }
    *bytes = std::max<size_t>(off, 256);
    return LORA_OK;
}

lora_status_t lora_layer_apply(lora_pool_t pool, const void* x, int64_t ldx, const void* W,
                               int64_t ldw, lora_w_layout_t w_layout, const int32_t* ids,
                               const lora_segments_t* seg, int32_t n_rows, void* y,
                               lora_dtype_t y_dtype, int64_t ldy, lora_mode_t mode, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
    if (check_pool(pool) != LORA_OK || n_rows < 0 || !dtype_ok(y_dtype)) return LORA_E_INVALID;
    if (!mode_ok(mode)) return LORA_E_INVALID;
    if (!w_layout_ok(w_layout)) return LORA_E_INVALID;
    if (n_rows == 0) return LORA_OK;
    const PoolDev& P = pool->dev;
    const int eb = elem_bytes(pool->dtype);
    const int ey = elem_bytes(y_dtype);
    if (!x || !W || !ids || !y) return LORA_E_INVALID;
    const int64_t w_min = (w_layout == LORA_W_IN_OUT) ? P.d_out : P.d_in;
    if (ldx < P.d_in || ldw < w_min || ldy < P.d_out) return LORA_E_INVALID;
    if (!al16(x) || !al16(W) || !al16(y) || !ld_ok(ldx, P.d_in, eb) || !ld_ok(ldw, w_min, eb) ||
        !ld_ok(ldy, P.d_out, ey))
        return LORA_E_UNSUPPORTED;
    const lora_mode_t m = resolve_mode(mode, n_rows, pool->dev.n_adapters);
    if (m == LORA_MODE_SGMV && seg) {
        lora_status_t st = check_segments(seg, n_rows, P.n_adapters);
        if (st != LORA_OK) return st;
    }
    size_t need = 0;
    lora_status_t st = lora_layer_workspace(pool, n_rows, m, &need);
    if (st != LORA_OK) return st;
    if (!ws || ws_bytes < need || !al16(ws)) return LORA_E_WORKSPACE;

    if (m == LORA_MODE_BGMV && w_layout == LORA_W_OUT_IN && decode_ok(pool, n_rows)) {
        const DecodePlan D = plan_decode(P, n_rows, true);
        DecodeArgs g{};
        g.x = x;
        g.ldx = ldx;
        g.W = W;
        g.ldw = ldw;
        g.ids = ids;
        g.n = n_rows;
        g.with_lora = 1;
        g.y = y;
        g.ldy = ldy;
        decode_carve(P, n_rows, D, ws, g);
        hipError_t e = launch_decode_stream(P, D, g, stream);
        if (e == hipSuccess) e = launch_decode_finish(P, D, g, y_dtype, stream);
        return dev_status(e);
    }
    if (m == LORA_MODE_BGMV && w_layout == LORA_W_OUT_IN && rows_ok(pool, n_rows)) {
        if (seg) {
            lora_status_t sst = check_segments(seg, n_rows, P.n_adapters);
            if (sst != LORA_OK) return sst;
        }
        return dev_status(
            run_rows(pool, x, ldx, W, ldw, nullptr, 0, false, ids, seg, n_rows, y, y_dtype, ldy, ws, stream));
    }
    return dev_status(run_fused(pool, m, x, ldx, W, ldw, w_layout == LORA_W_OUT_IN, nullptr, 0, ids, seg, n_rows, y,
                                y_dtype, ldy, ws, stream));
}

lora_status_t lora_layer_apply_noalloc(lora_pool_t pool, const void* x, int64_t ldx, const void* W,
                                       int64_t ldw, lora_w_layout_t w_layout, const int32_t* ids,
                                       const lora_segments_t* seg, int32_t n_rows, void* y,
                                       lora_dtype_t y_dtype, int64_t ldy, lora_mode_t mode,
                                       hipStream_t stream) {
    if (check_pool(pool) != LORA_OK || n_rows < 0) return LORA_E_INVALID;
    if (!mode_ok(mode)) return LORA_E_INVALID;
    if (n_rows == 0) return LORA_OK;
    size_t need = 0;
    lora_status_t st = lora_layer_workspace(pool, n_rows, mode, &need);
    if (st != LORA_OK) return st;
    if (need > LORA_NOALLOC_SCRATCH_BYTES) return LORA_E_SCRATCH;
    void* ws = nullptr;
    st = scratch_address(stream, &ws);
    if (st != LORA_OK) return st;
    // the layer's workspace needs no zero fill: every value a kernel reads
    // from it was written earlier in the same call
    return lora_layer_apply(pool, x, ldx, W, ldw, w_layout, ids, seg, n_rows, y, y_dtype, ldy, mode, ws,
                            LORA_NOALLOC_SCRATCH_BYTES, stream);
}

lora_status_t lora_base_gemm_expand_workspace(lora_pool_t pool, int32_t n_rows, size_t* bytes) {
    if (!pool || !bytes || n_rows < 0) return LORA_E_INVALID;
    *bytes = ext_bytes(pool, n_rows);
    return LORA_OK;
}

lora_status_t lora_base_gemm_expand(lora_pool_t pool, const void* x, int64_t ldx, const void* W,
                                    int64_t ldw, lora_w_layout_t w_layout, const int32_t* ids,
                                    const float* t, int64_t ldt, int32_t n_rows, void* y,
                                    lora_dtype_t y_dtype, int64_t ldy, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
    if (check_pool(pool) != LORA_OK || n_rows < 0 || !dtype_ok(y_dtype)) return LORA_E_INVALID;
    if (!w_layout_ok(w_layout)) return LORA_E_INVALID;
    if (n_rows == 0) return LORA_OK;
    const PoolDev& P = pool->dev;
    const int eb = elem_bytes(pool->dtype);
    const int ey = elem_bytes(y_dtype);
    if (!x || !W || !ids || !y) return LORA_E_INVALID;
    if (t && ldt < P.r_max) return LORA_E_INVALID;
    const int64_t w_min = (w_layout == LORA_W_IN_OUT) ? P.d_out : P.d_in;
    if (ldx < P.d_in || ldw < w_min || ldy < P.d_out) return LORA_E_INVALID;
    if (!al16(x) || !al16(W) || !al16(y) || !ld_ok(ldx, P.d_in, eb) || !ld_ok(ldw, w_min, eb) ||
        !ld_ok(ldy, P.d_out, ey))
        return LORA_E_UNSUPPORTED;
    GemmArgs g;
    g.x = x;
    g.ldx = ldx;
    g.W = W;
    g.ldw = ldw;
    g.w_out_in = (w_layout == LORA_W_OUT_IN) ? 1 : 0;
    g.ids = ids;
    g.n_rows = n_rows;
    g.t = nullptr;
    g.ldt = 0;
    g.t_ext = nullptr;
    g.lde = 0;
    g.y = y;
    g.ldy = ldy;
    g.vec_x = true;
    g.vec_w = true;
    const bool skinny = pool->dtype == LORA_BF16 && g.w_out_in && n_rows <= 64;
    if (t && skinny) {
        g.t = t;       // the skinny kernel adds s * t B in a VALU epilogue
        g.ldt = ldt;
    } else if (t) {
        // tiles with few adapters fold t into the K loop, the others add it row by row
        if (!ws || !al16(ws) || ws_bytes < ext_bytes(pool, n_rows)) return LORA_E_WORKSPACE;
        g.t = t;
        g.ldt = ldt;
        g.t_ext = ws;
        g.lde = ext_cols(eb, P.r_max);
        hipError_t e = launch_make_t_ext(P, pool->dtype, t, ldt, ids, n_rows, ws, g.lde, stream);
        if (e != hipSuccess) return LORA_E_DEVICE;
    }
    return dev_status(launch_layer_gemm(P, pool->dtype, y_dtype, g, stream));
}

lora_status_t lora_merge_adapter(lora_pool_t pool, int32_t adapter, void* W, int64_t ldw,
                                 lora_w_layout_t w_layout, float sign, hipStream_t stream) {
    if (check_pool(pool) != LORA_OK || !W || !std::isfinite(sign)) return LORA_E_INVALID;
    if (!w_layout_ok(w_layout)) return LORA_E_INVALID;
    const PoolDev& P = pool->dev;
    if (adapter < 0 || adapter >= P.n_adapters) return LORA_E_ID_RANGE;
    const int64_t w_min = (w_layout == LORA_W_IN_OUT) ? P.d_out : P.d_in;
    if (ldw < w_min) return LORA_E_INVALID;
    if (!al16(W) || !ld_ok(ldw, w_min, elem_bytes(pool->dtype))) return LORA_E_UNSUPPORTED;
    return dev_status(launch_merge(P, pool->dtype, adapter, sign, W, ldw, w_layout == LORA_W_OUT_IN, stream));
}

lora_status_t lora_decode_workspace(lora_pool_t pool, int32_t n_rows, int with_lora, size_t* bytes) {
    if (!pool || !bytes || n_rows < 0) return LORA_E_INVALID;
    if (n_rows == 0) {
        *bytes = 0;
        return LORA_OK;
    }
    if (!decode_ok(pool, n_rows)) return LORA_E_UNSUPPORTED;
    *bytes = decode_ws_bytes(pool->dev, n_rows, plan_decode(pool->dev, n_rows, with_lora != 0));
    return LORA_OK;
}

lora_status_t lora_decode_stream(lora_pool_t pool, const void* x, int64_t ldx, const void* W,
                                 int64_t ldw, const int32_t* ids, int32_t n_rows, int with_lora,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
    if (check_pool(pool) != LORA_OK || n_rows < 0) return LORA_E_INVALID;
    if (n_rows == 0) return LORA_OK;
    if (!decode_ok(pool, n_rows)) return LORA_E_UNSUPPORTED;
    const PoolDev& P = pool->dev;
    if (!x || !W || !ids || ldx < P.d_in || ldw < P.d_in) return LORA_E_INVALID;
    if (!al16(x) || !al16(W) || !ld_ok(ldx, P.d_in, 2) || !ld_ok(ldw, P.d_in, 2)) return LORA_E_UNSUPPORTED;
    const DecodePlan D = plan_decode(P, n_rows, with_lora != 0);
    if (!ws || !al16(ws) || ws_bytes < decode_ws_bytes(P, n_rows, D)) return LORA_E_WORKSPACE;
    DecodeArgs g{};
    g.x = x;
    g.ldx = ldx;
    g.W = W;
    g.ldw = ldw;
    g.ids = ids;
    g.n = n_rows;
    g.with_lora = with_lora ? 1 : 0;
    decode_carve(P, n_rows, D, ws, g);
    return dev_status(launch_decode_stream(P, D, g, stream));
}

lora_status_t lora_decode_stream_q4(lora_pool_t pool, const void* x, int64_t ldx, const uint8_t* Wq,
                                    int64_t ldq, const float* w_scale, int64_t lds, const int32_t* ids,
                                    int32_t n_rows, int with_lora, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
    if (check_pool(pool) != LORA_OK || n_rows < 0) return LORA_E_INVALID;
    if (n_rows == 0) return LORA_OK;
    if (!decode_ok(pool, n_rows)) return LORA_E_UNSUPPORTED;
    const PoolDev& P = pool->dev;
    if (!x || !Wq || !w_scale || !ids || ldx < P.d_in || ldq < P.d_in / 2 || lds < P.d_in / 128)
        return LORA_E_INVALID;
    if (P.d_in % 128 != 0) return LORA_E_UNSUPPORTED;
    if (!al16(x) || !al16(Wq) || !ld_ok(ldx, P.d_in, 2) || ldq % 16 != 0 || ((uintptr_t)w_scale & 3u) != 0)
        return LORA_E_UNSUPPORTED;
    const DecodePlan D = plan_decode(P, n_rows, with_lora != 0);
    if (!ws || !al16(ws) || ws_bytes < decode_ws_bytes(P, n_rows, D)) return LORA_E_WORKSPACE;
    DecodeArgs g{};
    g.x = x;
    g.ldx = ldx;
    g.W = Wq;
    g.ldw = ldq;
    g.w_q4 = 1;
    g.wscale = w_scale;
    g.lds = lds;
    g.ids = ids;
    g.n = n_rows;
    g.with_lora = with_lora ? 1 : 0;
    decode_carve(P, n_rows, D, ws, g);
    return dev_status(launch_decode_stream(P, D, g, stream));
}

lora_status_t lora_decode_finish(lora_pool_t pool, const int32_t* ids, int32_t n_rows, int with_lora,
                                 void* y, lora_dtype_t y_dtype, int64_t ldy, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
    if (check_pool(pool) != LORA_OK || n_rows < 0 || !dtype_ok(y_dtype)) return LORA_E_INVALID;
    if (n_rows == 0) return LORA_OK;
    if (!decode_ok(pool, n_rows)) return LORA_E_UNSUPPORTED;
    const PoolDev& P = pool->dev;
    if (!ids || !y || ldy < P.d_out) return LORA_E_INVALID;
    if (!al16(y) || !ld_ok(ldy, P.d_out, elem_bytes(y_dtype))) return LORA_E_UNSUPPORTED;
    const DecodePlan D = plan_decode(P, n_rows, with_lora != 0);
    if (!ws || !al16(ws) || ws_bytes < decode_ws_bytes(P, n_rows, D)) return LORA_E_WORKSPACE;
    DecodeArgs g{};
    g.ids = ids;
    g.n = n_rows;
    g.with_lora = with_lora ? 1 : 0;
    g.y = y;
    g.ldy = ldy;
    decode_carve(P, n_rows, D, ws, g);
    return dev_status(launch_decode_finish(P, D, g, y_dtype, stream));
}

lora_status_t lora_layer_q4_workspace(lora_pool_t pool, int32_t n_rows, size_t* bytes) {
    if (!pool || !bytes || n_rows < 0) return LORA_E_INVALID;
    if (n_rows == 0) {
        *bytes = 0;
        return LORA_OK;
    }
    if (pool->dtype != LORA_BF16) return LORA_E_UNSUPPORTED;
    if (decode_ok(pool, n_rows)) {
        *bytes = decode_ws_bytes(pool->dev, n_rows, plan_decode(pool->dev, n_rows, true));
        return LORA_OK;
    }
    if (pool->dev.n_adapters > kMaxAdaptersSegments) return LORA_E_UNSUPPORTED;
    if (n_rows > kRowsMaxRows) return lora_layer_workspace(pool, n_rows, LORA_MODE_SGMV, bytes);
    *bytes = rows_ws_bytes(pool, n_rows, true);
    return LORA_OK;
}

lora_status_t lora_layer_apply_q4(lora_pool_t pool, const void* x, int64_t ldx, const uint8_t* Wq, int64_t ldq,
                                  const float* w_scale, int64_t lds, const int32_t* ids,
                                  const lora_segments_t* seg, int32_t n_rows, void* y, lora_dtype_t y_dtype,
                                  int64_t ldy, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (check_pool(pool) != LORA_OK || n_rows < 0 || !dtype_ok(y_dtype)) return LORA_E_INVALID;
    if (n_rows == 0) return LORA_OK;
    const PoolDev& P = pool->dev;
    if (pool->dtype != LORA_BF16) return LORA_E_UNSUPPORTED;
    if (!x || !Wq || !w_scale || !ids || !y || ldx < P.d_in || ldq < P.d_in / 2 || lds < P.d_in / 128 ||
        ldy < P.d_out)
        return LORA_E_INVALID;
    if (P.d_in % 128 != 0) return LORA_E_UNSUPPORTED;
    const int ey = elem_bytes(y_dtype);
    if (!al16(x) || !al16(Wq) || !al16(y) || !ld_ok(ldx, P.d_in, 2) || ldq % 16 != 0 ||
        ((uintptr_t)w_scale & 3u) != 0 || !ld_ok(ldy, P.d_out, ey))
        return LORA_E_UNSUPPORTED;
    if (seg) {
        lora_status_t sst = check_segments(seg, n_rows, P.n_adapters);
        if (sst != LORA_OK) return sst;
    }
    size_t need = 0;
    lora_status_t st = lora_layer_q4_workspace(pool, n_rows, &need);
    if (st != LORA_OK) return st;
    if (!ws || ws_bytes < need || !al16(ws)) return LORA_E_WORKSPACE;
    if (decode_ok(pool, n_rows)) {
        const DecodePlan D = plan_decode(P, n_rows, true);
        DecodeArgs g{};
        g.x = x;
        g.ldx = ldx;
        g.W = Wq;
        g.ldw = ldq;
        g.w_q4 = 1;
        g.wscale = w_scale;
        g.lds = lds;
        g.ids = ids;
        g.n = n_rows;
        g.with_lora = 1;
        g.y = y;
        g.ldy = ldy;
        decode_carve(P, n_rows, D, ws, g);
        hipError_t e = launch_decode_stream(P, D, g, stream);
        if (e == hipSuccess) e = launch_decode_finish(P, D, g, y_dtype, stream);
        return dev_status(e);
    }
    if (n_rows > kRowsMaxRows)
        return dev_status(run_fused(pool, LORA_MODE_SGMV, x, ldx, Wq, ldq, true, w_scale, lds, ids, seg, n_rows, y,
                                    y_dtype, ldy, ws, stream));
    return dev_status(run_rows(pool, x, ldx, Wq, ldq, w_scale, lds, true, ids, seg, n_rows, y, y_dtype, ldy, ws,
                               stream));
}

}  // extern "C"
