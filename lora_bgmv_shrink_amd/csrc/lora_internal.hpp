// Internal declarations shared by the HIP translation units of liblora_mi355x.
// Nothing here is part of the C ABI (include/lora_mi355x.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "../../include/lora_mi355x.h"

namespace lora {

// bf16 is carried as its raw 16-bit pattern.
using bf16 = uint16_t;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Device view of a pool: element offsets, ranks and scales live in device
// tables built once by lora_pool_create.
struct PoolDev {
    const void* A;
    const void* B;
    const int32_t* ranks;
    const int64_t* a_off;
    const int64_t* b_off;
    const float* scales;
    int32_t* err;        // bit 0: an id outside [-1, n_adapters) was seen
    int32_t n_adapters;
    int32_t d_in;
    int32_t d_out;
    int32_t r_max;
    int32_t vec_a;       // every A block starts 16-byte aligned
    int32_t vec_b;       // every B block 16-byte aligned and d_out*elem % 16 == 0
    int32_t stream_ok;   // every rank r: r*elem % 16 == 0 and (512*16/elem) % r == 0
    int32_t vec_rank = 0;   // every rank r: r*elem % 16 == 0 (rows of A are whole 16-byte pieces)
    // the uniform layout: every rank is r_max and adapter u's blocks start at
    // u * d_in * r_max (A) and u * r_max * d_out (B), so kernels whose path
    // waits on them form the rank and A offset without a table load
    int32_t uniform = 0;
};
__device__ __forceinline__ int pool_rank(const PoolDev& P, int u) { return P.uniform ? P.r_max : P.ranks[u]; }
__device__ __forceinline__ int64_t pool_a_off(const PoolDev& P, int u) {
    return P.uniform ? (int64_t)u * P.d_in * P.r_max : P.a_off[u];
}

// eight bf16 from p, those at or past `valid` read as zero (no access)
__device__ __forceinline__ bf16x8_t ld8_guard(const bf16* p, int valid) {
    union { bf16x8_t v; bf16 e[8]; } u;
#pragma unroll
    for (int e = 0; e < 8; ++e) u.e[e] = (e < valid) ? p[e] : (bf16)0;
    return u.v;
}

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even; NaN stays NaN (quieted).  The
// conversion instruction (v_cvt_pk_bf16_f32 on gfx950) does exactly this.
__device__ __forceinline__ bf16 f32_to_bf16(float f) { return __builtin_bit_cast(bf16, (__bf16)f); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return f32_to_bf16(v); }

__device__ __forceinline__ bool id_ok(int32_t a, int32_t n_adapters) {
    return a >= 0 && a < n_adapters;
}

// Read-only table entry at a workgroup-uniform index through the scalar
// cache (a scalar load: it waits on its own counter, not behind the vector
// loads in flight).  Only for data no kernel in flight writes.
template <typename T>
__device__ __forceinline__ T uload(const T* p, int64_t i) {
    return ((const __attribute__((address_space(4))) T*)p)[i];
}

__device__ __forceinline__ void flag_bad_id(int32_t* err) {
    __hip_atomic_fetch_or(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// K-extension operand of the tiled layer GEMM ("t_ext"): per row, s * t
// laid out in blocks of 32 ranks; a bf16 block is 64 columns [hi(32) | lo(32)]
// (the fp32 value v = hi + lo to about 16 significant bits), an fp32 block is
// the 32 values themselves.  Columns past the adapter's rank are 0.
constexpr int EXT_RANKS = 32;
__host__ __device__ constexpr int ext_block_cols(int elem_bytes) { return elem_bytes == 2 ? 64 : 32; }
__host__ __device__ inline int ext_cols(int elem_bytes, int r_max) {
    return ext_block_cols(elem_bytes) * ((r_max + EXT_RANKS - 1) / EXT_RANKS);
}
// column c of a row's t_ext, from the row's t (rank r, scale s)
__device__ __forceinline__ bf16 ext_value_bf16(const float* t, int r, float s, int c) {
    const int e = c >> 6;
    const int kk = c & 63;
    const int j = e * EXT_RANKS + (kk & 31);
    const float v = (j < r) ? s * t[j] : 0.f;
    const bf16 hi = f32_to_bf16(v);
    return (kk < 32) ? hi : f32_to_bf16(v - to_f32(hi));
}
__device__ __forceinline__ float ext_value_f32(const float* t, int r, float s, int c) {
    return (c < r) ? s * t[c] : 0.f;
}

// Inclusive prefix sum over the 64 lanes of a wave.
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
__device__ inline bool find_seg_tile(const int32_t* __restrict__ seg_off, int n_seg, int BM, int b,
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

// find_seg_tile for callers that know the descriptor's capacity (cap >=
// n_seg) and search many times: seg_tile_cache_load copies the first
// SEG_CACHE run boundaries and run ids to LDS (entries past n_seg are read
// but never used) and returns the run count, once per workgroup (all its
// threads, then a barrier); seg_tile_find then maps tile b to (run s, chunk
// c) from LDS, loading from memory only past SEG_CACHE runs.  Also returns
// the run's id and its first and one-past-last position in perm.  The find
// is run by one whole wave.
constexpr int SEG_CACHE = 256;
struct SegTileCache {
    int lo[SEG_CACHE], hi[SEG_CACHE], id[SEG_CACHE];
};
__device__ inline int seg_tile_cache_load(const int32_t* __restrict__ seg_off, const int32_t* __restrict__ seg_ids,
                                          const int32_t* __restrict__ n_seg_p, int cap, int tid, int nthreads,
                                          SegTileCache& C) {
    for (int s = tid; s < SEG_CACHE; s += nthreads) {
        C.lo[s] = s < cap ? seg_off[s] : 0;
        C.hi[s] = s < cap ? seg_off[s + 1] : 0;
        C.id[s] = s < cap ? seg_ids[s] : -1;
    }
    return *n_seg_p;
}
__device__ inline bool seg_tile_find(const SegTileCache& C, int n_seg, const int32_t* __restrict__ seg_off,
                                     const int32_t* __restrict__ seg_ids, int BM, int b, int lane, int& s_out,
                                     int& c_out, int& lo_out, int& hi_out, int& id_out) {
    int base = 0;
    for (int s0 = 0; s0 < n_seg; s0 += 64) {
        const int s = s0 + lane;
        int l = 0, h = 0, u = -1;
        if (s < n_seg) {
            if (s < SEG_CACHE) {
                l = C.lo[s];
                h = C.hi[s];
                u = C.id[s];
            } else {
                l = seg_off[s];
                h = seg_off[s + 1];
                u = seg_ids[s];
            }
        }
        const int cnt = s < n_seg ? (h - l + BM - 1) / BM : 0;
        const int incl = wave_incl_scan(cnt, lane);
        const int excl = base + incl - cnt;
        const uint64_t hit = __ballot(s < n_seg && b >= excl && b < base + incl);
        if (hit) {
            const int L = __ffsll((unsigned long long)hit) - 1;
            s_out = s0 + L;
            c_out = b - __shfl(excl, L, 64);
            lo_out = __shfl(l, L, 64);
            hi_out = __shfl(h, L, 64);
            id_out = __shfl(u, L, 64);
            return true;
        }
        base += __shfl(incl, 63, 64);
    }
    return false;
}

static inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
static inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// Launchers (host side, one per kernel family).  Shapes are validated by the
// C-ABI layer before these run.
// ---------------------------------------------------------------------------

// Segments: one workgroup of 1024 threads.
hipError_t launch_segments(const int32_t* ids, int32_t n_rows, int32_t n_adapters,
                           const lora_segments_t* seg, int32_t* status, hipStream_t stream);

// BGMV shrink: one workgroup per row (no workspace).
struct BgmvShrinkPlan {
    int32_t ks;       // 1: streaming kernel, 0: LDS-staged generic kernel
};
BgmvShrinkPlan plan_bgmv_shrink(const PoolDev& P, int elem_bytes, int32_t n_rows);
hipError_t launch_bgmv_shrink(const PoolDev& P, lora_dtype_t dt, const void* x, int64_t ldx,
                              const int32_t* ids, int32_t n_rows, float* t, int64_t ldt,
                              const BgmvShrinkPlan& plan, hipStream_t stream,
                              void* t_ext = nullptr, int64_t lde = 0);

hipError_t launch_bgmv_expand(const PoolDev& P, lora_dtype_t dt, const float* t, int64_t ldt,
                              const int32_t* ids, int32_t n_rows, void* y, lora_dtype_t ydt,
                              int64_t ldy, int accumulate, bool vec_y, hipStream_t stream);

// SGMV shrink / expand (MFMA over segment tiles).
// part (optional, sgmv_shrink_part_bytes of workspace): K is split into
// slices whose partial sums a reduce pass adds in order (ids then required).
hipError_t launch_sgmv_shrink(const PoolDev& P, lora_dtype_t dt, const void* x, int64_t ldx,
                              const lora_segments_t* seg, int32_t n_rows, int32_t n_bins,
                              float* t, int64_t ldt, bool vec_x, hipStream_t stream,
                              void* t_ext = nullptr, int64_t lde = 0, const int32_t* ids = nullptr,
                              float* part = nullptr);
int32_t sgmv_shrink_slices(const PoolDev& P, int32_t n_rows);
size_t sgmv_shrink_part_bytes(const PoolDev& P, int32_t n_rows);
// workspace for the K split of the layer GEMM's 128x128 launches (bf16 pool,
// W stored [d_out, d_in]); 0 when no launch of this batch is split
size_t layer_gemm_split_bytes(const PoolDev& P, int32_t n_rows);
// t_ext from an existing t (rows with invalid ids or -1 are left alone)
hipError_t launch_make_t_ext(const PoolDev& P, lora_dtype_t dt, const float* t, int64_t ldt,
                             const int32_t* ids, int32_t n_rows, void* t_ext, int64_t lde,
                             hipStream_t stream);
hipError_t launch_sgmv_expand(const PoolDev& P, lora_dtype_t dt, const float* t, int64_t ldt,
                              const lora_segments_t* seg, int32_t n_rows, int32_t n_bins,
                              void* y, lora_dtype_t ydt, int64_t ldy, int accumulate,
                              hipStream_t stream);

// Fused layer GEMM: y = x W (+ LoRA expand epilogue from t).
struct GemmArgs {
    const void* x;
    int64_t ldx;
    const void* W;
    int64_t ldw;
    int w_out_in;
    const int32_t* ids;
    int32_t n_rows;
    // LoRA term: fp32 t (unscaled x A_a) for the skinny kernel's epilogue and
    // the tiled kernel's row-wise epilogue; t_ext for the tiled kernel's
    // K-extension.  Both nullptr: base product only.  The tiled kernel picks
    // per tile among what is given.
    const float* t;
    int64_t ldt;
    const void* t_ext;
    int64_t lde;
    void* y;
    int64_t ldy;
    bool vec_x;
    bool vec_w;
    // the caller expects most rows to carry different adapters (decode-style
    // batches): a tile shape without the K-extension may be chosen
    bool rows_distinct = false;
    // tiled kernel: visit the rows in this order (tile row m is row perm[m];
    // null: in order), e.g. grouped by adapter so that a tile holds few
    // adapters.  x_rows: rows x holds (0: n_rows).  Needs x under 2 GiB.
    const int32_t* perm = nullptr;
    int32_t x_rows = 0;
    // 4-bit W (stored [d_out, d_in], bf16 pool): W holds bytes, ldw bytes per
    // row; wscale [d_out][lds] fp32, one scale per output and 128 inputs
    bool w_q4 = false;
    // room for the fp32 partial sums of a K split of the 128x128 launches
    // (layer_gemm_split_bytes); null: no split
    float* split_part = nullptr;
    size_t split_bytes = 0;
    const float* wscale = nullptr;
    int64_t lds = 0;
};
hipError_t launch_layer_gemm(const PoolDev& P, lora_dtype_t dt, lora_dtype_t ydt,
                             const GemmArgs& g, hipStream_t stream);

// Batches of a few hundred rows (bf16, W stored [d_out, d_in]): the base
// product in split-K partial sums over 128 x 64 tiles, and the adapter term
// over the segments of lora_segments_build (rows.hip).
struct RowsPlan {
    int32_t shape;              // tile: 0 128 x 64, 1 256 x 128
    int32_t tiles_m, tiles_n;
    int32_t S, kslice;          // K slices of the base product
    int32_t St, ks_len;         // K slices of the shrink
    int64_t ldp;                // fp32 pitch of a base partial row
    int64_t rtp;                // fp32 pitch of a t partial row
    size_t part_off, tpart_off, recs_off, bytes;   // workspace layout
};
RowsPlan plan_rows(const PoolDev& P, int32_t n_rows, bool q4 = false);
// base partials part[S][n_rows][ldp] = x W over each K slice; q4: W holds
// 4-bit weights (bytes [d_out][ldw]) with fp32 scales [d_out][lds] per 128
// inputs (d_in % 128 == 0)
hipError_t launch_rows_gemm(const PoolDev& P, const RowsPlan& R, const void* x, int64_t ldx, const void* W,
                            int64_t ldw, const float* wscale, int64_t lds, bool q4, int32_t n_rows, float* part,
                            hipStream_t stream);
// shrink: tpart[St][n_rows][rtp] = x_rows A_u over each K slice, per segment
// tile, and the tile records (or, without the segment-tile shrink, only the
// records: tpart is then t from the SGMV shrink, one slice of pitch rtp);
// finish: y = sum of part + s_u (sum of tpart) B_u, rounded once
hipError_t launch_rows_adapter(const PoolDev& P, const RowsPlan& R, const void* x, int64_t ldx,
                               const int32_t* ids, const lora_segments_t* seg, int32_t n_rows,
                               const float* part, float* tpart, void* y, lora_dtype_t ydt, int64_t ldy,
                               hipStream_t stream, bool shrink, bool finish);

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);

// W += sign * s_a * A_a B_a in place (W stored [d_out, d_in] when out_in).
hipError_t launch_merge(const PoolDev& P, lora_dtype_t dt, int32_t adapter, float sign, void* W, int64_t ldw,
                        bool out_in, hipStream_t stream);

// Decode layer in two launches (bf16, n_rows <= 64, W stored [d_out, d_in]).
constexpr int DS_LDS_BYTES = 84 * 1024;   // > half a CU: one stream workgroup per CU
struct DecodePlan {
    int32_t tiles_n;      // 128-column base tiles
    int32_t kslice;       // k-rows per slice (multiple of 128, at most 512)
    int32_t base_slices;  // partial base products per output
    int32_t base_wgs;     // tiles_n * base_slices
    int32_t t_slices;     // partial shrink sums per row (base_slices, or 0 without the LoRA term)
};
struct RowRec {
    int64_t b_off;   // element offset of the row's B block
    int32_t rank;    // 0: no adapter term (base-only or invalid id)
    float scale;
};
struct DecodeArgs {
    const void* x;
    int64_t ldx;
    const void* W;      // bf16 [d_out, ldw], or (w_q4) 4-bit bytes [d_out, ldw]
    int64_t ldw;        // elements, or bytes for a 4-bit W
    int32_t w_q4;       // W holds signed 4-bit weights with per-128-input scales
    const float* wscale;   // w_q4: [d_out, lds] fp32
    int64_t lds;
    const int32_t* ids;
    int32_t n;
    int32_t with_lora;
    float* part_base;   // [base_slices][n][d_out]
    float* part_t;      // [t_slices][n][64]
    RowRec* rows;       // [n], written by the shrink part
    void* y;
    int64_t ldy;
};
DecodePlan plan_decode(const PoolDev& P, int32_t n_rows, bool with_lora);
size_t decode_ws_bytes(const PoolDev& P, int32_t n_rows, const DecodePlan& D);
void decode_carve(const PoolDev& P, int32_t n_rows, const DecodePlan& D, void* ws, DecodeArgs& g);
hipError_t launch_decode_stream(const PoolDev& P, const DecodePlan& D, const DecodeArgs& g,
                                hipStream_t stream);
hipError_t launch_decode_finish(const PoolDev& P, const DecodePlan& D, const DecodeArgs& g,
                                lora_dtype_t ydt, hipStream_t stream);

}  // namespace lora
