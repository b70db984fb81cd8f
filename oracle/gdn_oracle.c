/*
 * gdn_oracle.c -- fp64 token-by-token CPU oracle for the Gated DeltaNet layer.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * CPU-baseline leg of the benchmark, never by the product path.  Plain loops,
 * no blocking, no reordering beyond what the definitions state.  See
 * gdn_oracle.h for the definition and layouts.
 *
 * Readings where the pages leave a step open (each used below):
 *  - conv: cross-correlation over the K most recent raw tokens of one channel,
 *    w[c][K-1] multiplies the current token, w[c][0] the oldest; no bias;
 *    tokens before the sequence start come from the conv state (oldest
 *    first) or are zero.  SiLU follows the conv (hyper.ai story: causal
 *    convolution for local context; activation silu in the model-atlas key
 *    facts table).
 *  - order of steps on q, k: conv, SiLU, L2 normalisation, then q *= scale.
 *    v gets conv and SiLU only.
 *  - L2 normalisation: x / sqrt(sum x^2 + l2_eps).
 *  - key-head sharing: value head h reads key head h / (Hv/Hk).
 *  - g is the log-decay used as given: a = exp(g).  beta is b as given.
 *  - gated RMSNorm: normalise o over dv, multiply by norm_w (the effective
 *    weight, shared by all heads), then by SiLU(z).
 *  - the conv state written back holds the K-1 most recent raw tokens of the
 *    concatenation (old conv state, this sequence's tokens).
 */
#include "gdn_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- element access: exact widening of f32 / bf16 / f64 to double ---- */
static double ld(const void* p, int64_t i, int dtype)
{
    if (dtype == GDN_ORACLE_F64) return ((const double*)p)[i];
    if (dtype == GDN_ORACLE_F32) return (double)((const float*)p)[i];
    {
        uint32_t u = ((uint32_t)((const uint16_t*)p)[i]) << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
}

static void copy_elem(void* dst, int64_t di, const void* src, int64_t si, int dtype)
{
    if (dtype == GDN_ORACLE_F64) ((double*)dst)[di] = ((const double*)src)[si];
    else if (dtype == GDN_ORACLE_F32) ((float*)dst)[di] = ((const float*)src)[si];
    else ((uint16_t*)dst)[di] = ((const uint16_t*)src)[si];
}

static void zero_elem(void* dst, int64_t di, int dtype)
{
    if (dtype == GDN_ORACLE_F64) ((double*)dst)[di] = 0.0;
    else if (dtype == GDN_ORACLE_F32) ((float*)dst)[di] = 0.0f;
    else ((uint16_t*)dst)[di] = 0;
}

static double silu(double y) { return y / (1.0 + exp(-y)); }

/* ---- channel addressing: q | k | v ---- */
typedef struct {
    const void* q; const void* k; const void* v;
    int Hk, Hv, dk, dv, io;
} chan_src;

/* raw input of channel c at token t */
static double raw_at(const chan_src* s, int64_t t, int c)
{
    const int qk = s->Hk * s->dk;
    if (c < qk) return ld(s->q, t * qk + c, s->io);
    if (c < 2 * qk) return ld(s->k, t * qk + (c - qk), s->io);
    return ld(s->v, t * (int64_t)(s->Hv * s->dv) + (c - 2 * qk), s->io);
}

/* One token of the causal depthwise conv for one channel.
 * hist[0..K-2] holds the K-1 previous raw tokens, oldest first; x is the
 * current raw token.  Returns sum_j w[j]*window[j] over the K-token window
 * (window = hist followed by x) and shifts x into hist. */
static double conv_token(double* hist, const double* w, double x, int K)
{
    double acc = 0.0;
    for (int j = 0; j < K - 1; ++j) acc += w[j] * hist[j];
    acc += w[K - 1] * x;
    for (int j = 0; j + 1 < K - 1; ++j) hist[j] = hist[j + 1];
    if (K > 1) hist[K - 2] = x;
    return acc;
}

static int check_desc(const gdn_oracle_desc* d, const int32_t* cu)
{
    if (!d || !cu) return -1;
    if (d->num_seqs < 1 || d->num_k_heads < 1 || d->num_v_heads < 1) return -1;
    if (d->num_v_heads % d->num_k_heads) return -1;
    if (d->head_k_dim < 1 || d->head_v_dim < 1 || d->conv_kernel < 1) return -1;
    if (d->head_begin < 0 || d->head_end > d->num_v_heads || d->head_begin > d->head_end) return -1;
    if (cu[0] != 0 || (int64_t)cu[d->num_seqs] != d->total_tokens) return -1;
    for (int n = 0; n < d->num_seqs; ++n)
        if (cu[n + 1] < cu[n]) return -1;
    return 0;
}

/* Load the K-1 history values of channel c for sequence n (zeros if absent). */
static void load_hist(const gdn_oracle_desc* d, const void* conv_state_in, int n, int c,
                      int Cch, double* hist)
{
    const int K = d->conv_kernel;
    for (int j = 0; j < K - 1; ++j)
        hist[j] = conv_state_in
                      ? ld(conv_state_in, ((int64_t)n * (K - 1) + j) * Cch + c, d->io_dtype)
                      : 0.0;
}

/* ---- the recurrence for one (sequence, value head) ---- */
static void run_head(const gdn_oracle_desc* d, int n, int h,
                     const void* q, const void* k, const void* v,
                     const void* g, const void* beta,
                     const void* z, const void* conv_w, const void* norm_w,
                     const int32_t* cu, const void* S0, const void* conv_state_in,
                     double* out, double* final_state)
{
    const int Hk = d->num_k_heads, Hv = d->num_v_heads;
    const int dk = d->head_k_dim, dv = d->head_v_dim, K = d->conv_kernel;
    const int io = d->io_dtype;
    const int Cch = 2 * Hk * dk + Hv * dv;
    const int hk = h / (Hv / Hk);
    const int nh = d->head_end - d->head_begin;
    const int hl = h - d->head_begin;
    const int gate = (z != NULL) || (norm_w != NULL);
    const chan_src src = { q, k, v, Hk, Hv, dk, dv, io };

    /* this head's channels: q of key head hk, k of key head hk, v of value head h */
    const int nc = 2 * dk + dv;
    int* ch = (int*)malloc(sizeof(int) * nc);
    for (int i = 0; i < dk; ++i) ch[i] = hk * dk + i;
    for (int i = 0; i < dk; ++i) ch[dk + i] = Hk * dk + hk * dk + i;
    for (int i = 0; i < dv; ++i) ch[2 * dk + i] = 2 * Hk * dk + h * dv + i;

    double* S = (double*)calloc((size_t)dv * dk, sizeof(double));
    double* hist = (double*)calloc((size_t)nc * (K > 1 ? K - 1 : 1), sizeof(double));
    double* wt = (double*)calloc((size_t)nc * K, sizeof(double));
    double* y = (double*)malloc(sizeof(double) * nc);
    double* kvmem = (double*)malloc(sizeof(double) * dv);
    double* o = (double*)malloc(sizeof(double) * dv);

    if (S0)
        for (int64_t i = 0; i < (int64_t)dv * dk; ++i)
            S[i] = ld(S0, ((int64_t)n * Hv + h) * dv * dk + i, d->state_dtype);
    if (conv_w)
        for (int i = 0; i < nc; ++i) {
            load_hist(d, conv_state_in, n, ch[i], Cch, hist + (size_t)i * (K - 1));
            for (int j = 0; j < K; ++j) wt[(size_t)i * K + j] = ld(conv_w, (int64_t)ch[i] * K + j, io);
        }

    for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
        /* conv + SiLU (or the raw value when there is no conv) */
        for (int i = 0; i < nc; ++i) {
            const double x = raw_at(&src, t, ch[i]);
            y[i] = conv_w ? silu(conv_token(hist + (size_t)i * (K - 1), wt + (size_t)i * K, x, K)) : x;
        }
        double* yq = y;
        double* yk = y + dk;
        double* yv = y + 2 * dk;
        if (d->use_l2) {
            double sq = 0.0, sk = 0.0;
            for (int i = 0; i < dk; ++i) { sq += yq[i] * yq[i]; sk += yk[i] * yk[i]; }
            const double rq = 1.0 / sqrt(sq + d->l2_eps), rk = 1.0 / sqrt(sk + d->l2_eps);
            for (int i = 0; i < dk; ++i) { yq[i] *= rq; yk[i] *= rk; }
        }
        for (int i = 0; i < dk; ++i) yq[i] *= d->scale;

        const double a = exp(ld(g, t * Hv + h, d->gate_dtype));
        const double b = ld(beta, t * Hv + h, d->gate_dtype);

        /* S = a S ; kvmem = S k ; S += b (v - kvmem) k^T ; o = S q */
        for (int r = 0; r < dv; ++r)
            for (int c = 0; c < dk; ++c) S[(size_t)r * dk + c] *= a;
        for (int r = 0; r < dv; ++r) {
            double acc = 0.0;
            for (int c = 0; c < dk; ++c) acc += S[(size_t)r * dk + c] * yk[c];
            kvmem[r] = acc;
        }
        for (int r = 0; r < dv; ++r) {
            const double u = b * (yv[r] - kvmem[r]);
            for (int c = 0; c < dk; ++c) S[(size_t)r * dk + c] += u * yk[c];
        }
        for (int r = 0; r < dv; ++r) {
            double acc = 0.0;
            for (int c = 0; c < dk; ++c) acc += S[(size_t)r * dk + c] * yq[c];
            o[r] = acc;
        }

        double* dst = out + (t * nh + hl) * dv;
        if (gate) {
            double ms = 0.0;
            for (int r = 0; r < dv; ++r) ms += o[r] * o[r];
            ms /= dv;
            const double rinv = 1.0 / sqrt(ms + d->norm_eps);
            for (int r = 0; r < dv; ++r) {
                const double wn = norm_w ? ld(norm_w, r, io) : 1.0;
                const double gz = z ? silu(ld(z, (t * Hv + h) * dv + r, io)) : 1.0;
                dst[r] = o[r] * rinv * wn * gz;
            }
        } else {
            for (int r = 0; r < dv; ++r) dst[r] = o[r];
        }
    }

    if (final_state)
        memcpy(final_state + ((size_t)n * nh + hl) * dv * dk, S, sizeof(double) * dv * dk);

    free(ch); free(S); free(hist); free(wt); free(y); free(kvmem); free(o);
}

/* Conv state after a sequence: the K-1 most recent raw tokens of
 * (old conv state ++ sequence tokens), oldest first. */
static void write_conv_state(const gdn_oracle_desc* d, int n, const void* q, const void* k,
                             const void* v, const int32_t* cu, const void* conv_state_in,
                             void* conv_state_out)
{
    const int K = d->conv_kernel, io = d->io_dtype;
    const int Hk = d->num_k_heads, Hv = d->num_v_heads, dk = d->head_k_dim, dv = d->head_v_dim;
    const int Cch = 2 * Hk * dk + Hv * dv;
    const int qk = Hk * dk;
    const int64_t L = cu[n + 1] - cu[n];
    for (int j = 0; j < K - 1; ++j) {
        const int64_t pos = L + j;   /* index into the concatenation of length L + K - 1 */
        for (int c = 0; c < Cch; ++c) {
            const int64_t di = ((int64_t)n * (K - 1) + j) * Cch + c;
            if (pos < K - 1) {
                if (conv_state_in)
                    copy_elem(conv_state_out, di, conv_state_in,
                              ((int64_t)n * (K - 1) + pos) * Cch + c, io);
                else
                    zero_elem(conv_state_out, di, io);
            } else {
                const int64_t t = cu[n] + pos - (K - 1);
                if (c < qk) copy_elem(conv_state_out, di, q, t * qk + c, io);
                else if (c < 2 * qk) copy_elem(conv_state_out, di, k, t * qk + c - qk, io);
                else copy_elem(conv_state_out, di, v, t * (int64_t)(Hv * dv) + c - 2 * qk, io);
            }
        }
    }
}

int gdn_oracle_prefill(const gdn_oracle_desc* d,
                       const void* q, const void* k, const void* v,
                       const void* g, const void* beta,
                       const void* z, const void* conv_w, const void* norm_w,
                       const int32_t* cu_seqlens,
                       const void* initial_state, const void* conv_state_in,
                       double* out, double* final_state, void* conv_state_out)
{
    if (check_desc(d, cu_seqlens)) return -1;
    if (!q || !k || !v || !g || !beta || !out) return -1;
    const int N = d->num_seqs;
    const int nh = d->head_end - d->head_begin;
    const int units = N * nh;

#ifdef _OPENMP
    if (d->num_threads > 0) omp_set_num_threads(d->num_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int u = 0; u < units; ++u) {
        const int n = u / nh, h = d->head_begin + u % nh;
        run_head(d, n, h, q, k, v, g, beta, z, conv_w, norm_w, cu_seqlens,
                 initial_state, conv_state_in, out, final_state);
    }

    if (conv_state_out && d->conv_kernel > 1)
        for (int n = 0; n < N; ++n)
            write_conv_state(d, n, q, k, v, cu_seqlens, conv_state_in, conv_state_out);
    return 0;
}

int gdn_oracle_conv_silu(const gdn_oracle_desc* d,
                         const void* q, const void* k, const void* v,
                         const void* conv_w, const int32_t* cu_seqlens,
                         const void* conv_state_in, double* y)
{
    if (check_desc(d, cu_seqlens) || !q || !k || !v || !conv_w || !y) return -1;
    const int K = d->conv_kernel, io = d->io_dtype;
    const int Cch = 2 * d->num_k_heads * d->head_k_dim + d->num_v_heads * d->head_v_dim;
    const chan_src src = { q, k, v, d->num_k_heads, d->num_v_heads, d->head_k_dim,
                           d->head_v_dim, io };
    double* hist = (double*)calloc(K > 1 ? K - 1 : 1, sizeof(double));
    double* w = (double*)malloc(sizeof(double) * K);
    for (int n = 0; n < d->num_seqs; ++n)
        for (int c = 0; c < Cch; ++c) {
            load_hist(d, conv_state_in, n, c, Cch, hist);
            for (int j = 0; j < K; ++j) w[j] = ld(conv_w, (int64_t)c * K + j, io);
            for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t)
                y[t * Cch + c] = silu(conv_token(hist, w, raw_at(&src, t, c), K));
        }
    free(hist);
    free(w);
    return 0;
}

int gdn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
