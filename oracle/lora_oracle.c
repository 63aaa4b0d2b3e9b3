/*
 * fp64 CPU oracle for the multi-LoRA batched layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code with the HIP library.
 *
 * What it computes (plain definitions, written out):
 *
 *   LoRA layer, row-vector convention of "Serving multiple LoRAs: segmented
 *   matrix multiplies and adapter scheduling", section "Not merging the
 *   weights, computing in batches":  y = x W + s * (x A) B  with
 *   W [d_in, d_out], A [d_in, r], B [r, d_out], applied per request with that
 *   request's own adapter (the page's per-request loop).  A request of several
 *   tokens is several rows with one adapter id; rows of a matrix product are
 *   independent, so the loop below runs per row.
 *
 *   Base-only rows (adapter id -1; "Serving many LoRA adapters",
 *   blog.ecitis.org, section "Replay", has a request with no adapter served
 *   by the base model alone) get y = x W.
 *   Ids outside [-1, n_adapters) are counted as errors and treated as
 *   base-only.
 *
 *   The scale s is a per-adapter value that travels with the adapter
 *   (blog.ecitis.org, section "Correctness across tenants"); it multiplies
 *   the expanded term once.  The shrink output t = x A is returned unscaled.
 *
 *   Segments: the stable group-by of the same page section (stable argsort of
 *   the per-token adapter ids, then runs of equal ids).  Rows whose id is -1
 *   (or invalid) form the first run, with id -1.
 *
 * Every sum runs in fp64 over k = 0, 1, ... in order.  Inputs are the exact
 * values the GPU sees, widened to fp64 by the caller.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int id_valid(int32_t a, int32_t n_adapters) { return a >= 0 && a < n_adapters; }

/* Number of rows whose id lies outside [-1, n_adapters). */
int64_t oracle_count_bad_ids(const int32_t* ids, int64_t n_rows, int32_t n_adapters)
{
    int64_t bad = 0;
    for (int64_t i = 0; i < n_rows; ++i)
        if (ids[i] < -1 || ids[i] >= n_adapters) ++bad;
    return bad;
}

/*
 * Stable group-by of adapter ids.
 *   perm[n_rows]       : rows in ascending id order, original order inside a run
 *   seg_ids[n_seg]     : id of each run (-1 first when present)
 *   seg_off[n_seg + 1] : run boundaries into perm
 * Returns the number of invalid ids (those rows are grouped with -1).
 * Definition used: for every id value v = -1, 0, 1, ... in ascending order,
 * append the rows carrying v in their original order.
 */
int64_t oracle_segments(const int32_t* ids, int64_t n_rows, int32_t n_adapters,
                        int32_t* perm, int32_t* seg_ids, int32_t* seg_off, int32_t* n_seg)
{
    int64_t pos = 0;
    int32_t s = 0;
    for (int32_t v = -1; v < n_adapters; ++v) {
        int64_t start = pos;
        for (int64_t i = 0; i < n_rows; ++i) {
            int32_t key = id_valid(ids[i], n_adapters) ? ids[i] : -1;
            if (key == v) perm[pos++] = (int32_t)i;
        }
        if (pos > start) {
            seg_ids[s] = v;
            seg_off[s] = (int32_t)start;
            ++s;
        }
    }
    seg_off[s] = (int32_t)pos;
    *n_seg = s;
    return oracle_count_bad_ids(ids, n_rows, n_adapters);
}

/*
 * The layer, one row at a time.
 *
 *   x      [n_rows, d_in]                  row-major
 *   W      [d_in, d_out]                   row-major; may be NULL (no base term)
 *   ids    [n_rows]
 *   A, B   flat pools; adapter u is A[a_off[u] + k*ranks[u] + j]  (k < d_in, j < r_u)
 *                                  and B[b_off[u] + j*d_out + c]   (j < r_u, c < d_out)
 *   scales [n_adapters]
 *
 * Outputs (each may be NULL):
 *   t    [n_rows, r_max]   t[i][j] = sum_k x[i][k] A_a[k][j]   (0 past r_a and on base-only rows)
 *   lora [n_rows, d_out]   s_a * sum_j t[i][j] B_a[j][c]        (0 on base-only rows)
 *   y    [n_rows, d_out]   sum_k x[i][k] W[k][c] + lora[i][c]
 *
 * ``rows`` (may be NULL) lists the rows to compute; the others are left
 * untouched.  ``n_threads`` <= 0 keeps the OpenMP default.
 * Returns the number of invalid ids among the computed rows.
 */
int64_t oracle_layer(int64_t n_rows, int64_t d_in, int64_t d_out,
                     const double* x, const double* W,
                     const int32_t* ids, int32_t n_adapters,
                     const int32_t* ranks, const int64_t* a_off, const int64_t* b_off,
                     const double* A, const double* B, const double* scales,
                     int32_t r_max,
                     const int64_t* rows, int64_t n_sel,
                     double* t, double* lora, double* y, int n_threads)
{
    int64_t count = rows ? n_sel : n_rows;
    int64_t bad = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif

#pragma omp parallel reduction(+ : bad)
    {
        double* ti = (double*)malloc(sizeof(double) * (size_t)(r_max > 0 ? r_max : 1));
        double* li = (double*)malloc(sizeof(double) * (size_t)d_out);
        double* bi = (double*)malloc(sizeof(double) * (size_t)d_out);

#pragma omp for schedule(dynamic, 1)
        for (int64_t q = 0; q < count; ++q) {
            int64_t i = rows ? rows[q] : q;
            const double* xi = x + i * d_in;
            int32_t a = ids[i];
            int valid = id_valid(a, n_adapters);
            if (a != -1 && !valid) ++bad;

            /* shrink: t_i = x_i A_a */
            for (int32_t j = 0; j < r_max; ++j) ti[j] = 0.0;
            int32_t r = valid ? ranks[a] : 0;
            for (int32_t j = 0; j < r; ++j) {
                const double* Aa = A + a_off[a];
                double acc = 0.0;
                for (int64_t k = 0; k < d_in; ++k) acc += xi[k] * Aa[k * r + j];
                ti[j] = acc;
            }

            /* expand: lora_i = s_a * (t_i B_a) */
            for (int64_t c = 0; c < d_out; ++c) li[c] = 0.0;
            if (valid) {
                const double* Ba = B + b_off[a];
                double s = scales[a];
                for (int64_t c = 0; c < d_out; ++c) {
                    double acc = 0.0;
                    for (int32_t j = 0; j < r; ++j) acc += ti[j] * Ba[(int64_t)j * d_out + c];
                    li[c] = s * acc;
                }
            }

            /* base: x_i W, summed over k in order for every column */
            if (y) {
                for (int64_t c = 0; c < d_out; ++c) bi[c] = 0.0;
                if (W) {
                    for (int64_t k = 0; k < d_in; ++k) {
                        double xk = xi[k];
                        const double* Wk = W + k * d_out;
                        for (int64_t c = 0; c < d_out; ++c) bi[c] += xk * Wk[c];
                    }
                }
                for (int64_t c = 0; c < d_out; ++c) y[i * d_out + c] = bi[c] + li[c];
            }
            if (t)
                for (int32_t j = 0; j < r_max; ++j) t[i * r_max + j] = ti[j];
            if (lora)
                for (int64_t c = 0; c < d_out; ++c) lora[i * d_out + c] = li[c];
        }
        free(ti);
        free(li);
        free(bi);
    }
    return bad;
}

/*
 * Merged weights of one adapter ("Serving many LoRA adapters",
 * blog.ecitis.org, section "Merge or keep separate": the adapter folded into
 * the base weight, in this file's row-vector convention):
 *
 *   W[k][c] += sign * s_a * sum_j A_a[k][j] * B_a[j][c]      W [d_in, d_out]
 *
 * sign = +1 merges the adapter, -1 takes it back out.  W is updated in
 * place; each element's sum runs over j = 0 .. r_a-1 in order and is scaled
 * and added once.  Returns 1 (W untouched) for an adapter outside
 * [0, n_adapters), else 0.  ``n_threads`` <= 0 keeps the OpenMP default.
 */
int oracle_merge(int64_t d_in, int64_t d_out, double* W, int32_t adapter, int32_t n_adapters,
                 const int32_t* ranks, const int64_t* a_off, const int64_t* b_off,
                 const double* A, const double* B, const double* scales, double sign, int n_threads)
{
    if (!id_valid(adapter, n_adapters)) return 1;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    const int32_t r = ranks[adapter];
    const double* Aa = A + a_off[adapter];
    const double* Ba = B + b_off[adapter];
    const double s = sign * scales[adapter];
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < d_in; ++k) {
        const double* Ak = Aa + k * (int64_t)r;   /* row k of A_a */
        for (int64_t c = 0; c < d_out; ++c) {
            double acc = 0.0;
            for (int32_t j = 0; j < r; ++j) acc += Ak[j] * Ba[c + (int64_t)j * d_out];
            W[k * d_out + c] += s * acc;
        }
    }
    return 0;
}

/* Threads an OpenMP parallel region would use (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * A 4-bit base weight, widened.  The pages leave the 4-bit format open
 * ("Serving Many LoRA Adapters" (praveentn.live), section "When It Falls
 * Down": a 4-bit base with FP16/BF16 adapters); the one read here:
 *   q[n * ldq + k / 2] holds the weight of output column n and input k as a
 *   signed 4-bit two's-complement value, k even in the low nibble, k odd in
 *   the high nibble; scale[n * lds + k / group] is the scale of that weight's
 *   group of `group` consecutive inputs.  The weight is q * scale.
 * Writes W[k][n] ([d_in, d_out], the layer's orientation).  Each value is an
 * integer in [-8, 7] times a scale, exact in fp64.
 */
void oracle_dequant_q4(int64_t d_in, int64_t d_out, const uint8_t* q, int64_t ldq, const double* scale,
                       int64_t lds, int64_t group, double* W)
{
    for (int64_t n = 0; n < d_out; ++n) {
        for (int64_t k = 0; k < d_in; ++k) {
            const uint8_t byte = q[n * ldq + k / 2];
            const int nib = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
            const int v = nib >= 8 ? nib - 16 : nib;
            W[k * d_out + n] = (double)v * scale[n * lds + k / group];
        }
    }
}
