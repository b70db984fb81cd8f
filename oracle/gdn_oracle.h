/*
 * gdn_oracle.h -- fp64 CPU oracle for the Gated DeltaNet layer.
 *
 * TEST INFRASTRUCTURE ONLY.  The oracle is the slow, plain reference that the
 * HIP library is checked against.  Only the tests, the smoke check and the
 * CPU-baseline leg of the benchmark may load it.  It shares no code with the
 * HIP library: neither includes, links or calls the other.
 *
 * What it computes (per sequence n, value head h, key head hk = h / (Hv/Hk)):
 *   causal depthwise conv (kernel K) + SiLU on the raw q, k, v channels
 *     (hyper.ai story on the Qwen3-Next Transformers merge: the Gated DeltaNet
 *      paragraph names the causal convolution; kernel 4 is
 *      linear_conv_kernel_dim in the raw config.json table of the model-atlas
 *      page for Qwen3-Coder-Next),
 *   L2 normalisation of q and k per token and key head, then q *= scale,
 *   the gated delta rule, written with the read-out of the old memory at the
 *   new key (the story's "kv_mem"):
 *     S     = a_t * S                      a_t = exp(g_t)
 *     kvmem = S k_t
 *     S     = S + b_t (v_t - kvmem) k_t^T  b_t = beta_t
 *     o_t   = S q_t
 *   which equals S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,
 *   and the z-gated RMSNorm of the output (rms_norm_eps 1e-6 in the same
 *   config table; Zero-Centered RMSNorm in the story):
 *     out_t = o_t / sqrt(mean(o_t^2) + eps) * w_norm * SiLU(z_t).
 * Readings where the pages are silent are listed with each step in
 * gdn_oracle.c.
 *
 * Layouts (row-major, last index contiguous):
 *   q, k [T][Hk][dk]; v, z [T][Hv][dv]; g, beta [T][Hv];
 *   conv_w [Cch][K] with Cch = 2*Hk*dk + Hv*dv, channels q | k | v;
 *   norm_w [dv]; states [N][Hv][dv][dk]; conv state [N][K-1][Cch], oldest first;
 *   cu_seqlens [N+1] (host memory).
 * Outputs cover value heads [head_begin, head_end) only:
 *   out [T][head_end-head_begin][dv], final_state [N][head_end-head_begin][dv][dk].
 *   conv_state_out covers every channel (exact copies of raw inputs).
 */
#ifndef GDN_ORACLE_H
#define GDN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { GDN_ORACLE_F32 = 0, GDN_ORACLE_BF16 = 1, GDN_ORACLE_F64 = 2 };

typedef struct {
    int32_t num_seqs;        /* N >= 1 */
    int64_t total_tokens;    /* must equal cu_seqlens[N] */
    int32_t num_k_heads;     /* Hk */
    int32_t num_v_heads;     /* Hv, a multiple of Hk */
    int32_t head_k_dim;      /* dk */
    int32_t head_v_dim;      /* dv */
    int32_t conv_kernel;     /* K >= 1 (used only when conv_w != NULL) */
    int32_t io_dtype;        /* q,k,v,z,conv_w,norm_w,conv states: F32, BF16 or F64 */
    int32_t gate_dtype;      /* g, beta: F32 or F64 */
    int32_t state_dtype;     /* initial_state: F32, BF16 or F64 */
    int32_t use_l2;          /* nonzero: L2-normalise q and k */
    double scale;            /* multiplies the (normalised) q */
    double l2_eps;
    double norm_eps;
    int32_t head_begin;      /* value heads computed: [head_begin, head_end) */
    int32_t head_end;
    int32_t num_threads;     /* OpenMP threads; 0 = runtime default */
} gdn_oracle_desc;

/* Prefill (and decode: one token per sequence).  z and norm_w both NULL: no
 * output gate (out = o).  conv_w NULL: no conv.  initial_state / conv_state_in
 * NULL: zeros.  final_state / conv_state_out may be NULL.  Returns 0 on
 * success, -1 on an invalid argument. */
int gdn_oracle_prefill(const gdn_oracle_desc* d,
                       const void* q, const void* k, const void* v,
                       const void* g, const void* beta,
                       const void* z, const void* conv_w, const void* norm_w,
                       const int32_t* cu_seqlens,
                       const void* initial_state, const void* conv_state_in,
                       double* out, double* final_state, void* conv_state_out);

/* The conv + SiLU step alone, for every channel: y [T][Cch] (q | k | v), using
 * the same per-token routine as gdn_oracle_prefill. */
int gdn_oracle_conv_silu(const gdn_oracle_desc* d,
                         const void* q, const void* k, const void* v,
                         const void* conv_w, const int32_t* cu_seqlens,
                         const void* conv_state_in, double* y);

/* Number of OpenMP threads a parallel region would use (for reporting). */
int gdn_oracle_max_threads(void);

#ifdef __cplusplus
}
#endif
#endif
