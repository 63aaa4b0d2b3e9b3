// Stable GPU group-by of adapter ids (one launch, integer only).
//
// The group-by is the stable argsort of the per-token adapter ids followed
// by run detection ("Serving multiple LoRAs: segmented matrix multiplies and
// adapter scheduling", section "Not merging the weights, computing in
// batches").  Here it is a counting sort: ids map to bins 0..n_adapters
// (bin 0 holds id -1 and invalid ids), so ascending bins give ascending
// ids with the base-only run first.
//
// One workgroup of 16 waves.  Wave w owns a contiguous chunk of rows and its
// own histogram row in LDS, so after a bin-major exclusive scan every
// (bin, wave) pair has a private output cursor; each wave then walks its
// chunk in row order and places rows with a ballot-based rank, which keeps
// the sort stable without any cross-wave ordering.
#include "lora_internal.hpp"

namespace lora {
namespace {

constexpr int SEG_THREADS = 1024;
constexpr int SEG_WAVES = SEG_THREADS / 64;
constexpr int SEG_HIST_INTS = 16384;   // per-wave histograms, 64 KiB
constexpr int SEG_MAX_BINS = 16384;    // n_adapters + 1

__global__ __launch_bounds__(SEG_THREADS) void k_segments(const int32_t* __restrict__ ids, int32_t n,
                                                          int32_t n_ad, int32_t* __restrict__ perm,
                                                          int32_t* __restrict__ seg_ids,
                                                          int32_t* __restrict__ seg_off,
                                                          int32_t* __restrict__ n_seg,
                                                          int32_t* __restrict__ status) {
    __shared__ int32_t hist[SEG_HIST_INTS];   // [G][nb]: counts, then per-wave cursors
    __shared__ int32_t start[SEG_MAX_BINS];   // totals, then bin start offsets
    __shared__ int32_t wsum_c[SEG_WAVES];
    __shared__ int32_t wsum_f[SEG_WAVES];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int nb = n_ad + 1;
    const int G = min(SEG_WAVES, SEG_HIST_INTS / nb);   // >= 1 because nb <= 16384
    const int chunk = (n + G - 1) / G;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    for (int i = tid; i < G * nb; i += SEG_THREADS) hist[i] = 0;
    __syncthreads();

    // Phase 1: per-wave histograms (one LDS update per distinct bin per 64 rows).
    bool bad = false;
    if (wave < G) {
        const int r0 = wave * chunk;
        const int r1 = min(n, r0 + chunk);
        for (int base = r0; base < r1; base += 64) {
            const int row = base + lane;
            const bool act = row < r1;
            int b = 0;
            if (act) {
                const int a = ids[row];
                const bool v = a >= 0 && a < n_ad;
                bad |= (!v && a != -1);
                b = v ? a + 1 : 0;
            }
            uint64_t rem = __ballot(act);
            while (rem) {
                const int leader = __ffsll((unsigned long long)rem) - 1;
                const int vb = __shfl(b, leader, 64);
                const uint64_t m = __ballot(act && b == vb);
                if (lane == leader) hist[wave * nb + vb] += __popcll(m);
                rem &= ~m;
            }
        }
    }
    if (bad && status) atomicOr(status, 1);
    __syncthreads();

    // Phase 2a: per bin, exclusive prefix over waves; totals into start[].
    for (int b = tid; b < nb; b += SEG_THREADS) {
        int s = 0;
        for (int w = 0; w < G; ++w) {
            const int c = hist[w * nb + b];
            hist[w * nb + b] = s;
            s += c;
        }
        start[b] = s;
    }
    __syncthreads();

    // Phase 2b: exclusive scan of totals and of "bin non-empty" flags over
    // bins; each thread owns a contiguous range of bins.
    const int per = (nb + SEG_THREADS - 1) / SEG_THREADS;
    const int b0 = min(nb, tid * per);
    const int b1 = min(nb, b0 + per);
    int cs = 0, fs = 0;
    for (int b = b0; b < b1; ++b) {
        cs += start[b];
        fs += start[b] > 0;
    }
    const int ic = wave_incl_scan(cs, lane);
    const int iff = wave_incl_scan(fs, lane);
    if (lane == 63) {
        wsum_c[wave] = ic;
        wsum_f[wave] = iff;
    }
    __syncthreads();
    int pc = 0, pf = 0;
    for (int w = 0; w < wave; ++w) {
        pc += wsum_c[w];
        pf += wsum_f[w];
    }
    int run_c = pc + ic - cs;   // exclusive prefix of this thread's range
    int run_f = pf + iff - fs;
    for (int b = b0; b < b1; ++b) {
        const int tot = start[b];
        if (tot > 0) {
            seg_ids[run_f] = b - 1;
            seg_off[run_f] = run_c;
            ++run_f;
        }
        start[b] = run_c;
        run_c += tot;
    }
    if (tid == SEG_THREADS - 1) {
        // run_f / run_c of the last thread are the totals over all bins.
        *n_seg = run_f;
        seg_off[run_f] = run_c;
    }
    __syncthreads();

    // Phase 3: stable placement, each wave in row order through its chunk.
    if (wave < G) {
        const int r0 = wave * chunk;
        const int r1 = min(n, r0 + chunk);
        for (int base = r0; base < r1; base += 64) {
            const int row = base + lane;
            const bool act = row < r1;
            int b = 0;
            if (act) {
                const int a = ids[row];
                b = (a >= 0 && a < n_ad) ? a + 1 : 0;
            }
            uint64_t rem = __ballot(act);
            while (rem) {
                const int leader = __ffsll((unsigned long long)rem) - 1;
                const int vb = __shfl(b, leader, 64);
                const uint64_t m = __ballot(act && b == vb);
                const int cur = start[vb] + hist[wave * nb + vb];
                if (act && b == vb) perm[cur + __popcll(m & lt_mask)] = row;
                if (lane == leader) hist[wave * nb + vb] += __popcll(m);
                rem &= ~m;
            }
        }
    }
}

}  // namespace

hipError_t launch_segments(const int32_t* ids, int32_t n_rows, int32_t n_adapters,
                           const lora_segments_t* seg, int32_t* status, hipStream_t stream) {
    hipLaunchKernelGGL(k_segments, dim3(1), dim3(SEG_THREADS), 0, stream, ids, n_rows, n_adapters,
                       seg->perm, seg->seg_ids, seg->seg_off, seg->n_seg, status);
    return hipGetLastError();
}

}  // namespace lora
