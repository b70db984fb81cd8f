/*
 * gdn.h -- C ABI of the Gated DeltaNet layer library (libgdn.so) for AMD
 * Instinct MI355X (gfx950).
 *
 * The layer (the linear-attention layer that makes up three of every four
 * layers of Qwen3-Next; hyper.ai story on the Qwen3-Next Transformers merge,
 * Gated DeltaNet paragraph) computes, per sequence n, value head h and key
 * head hk = h / (Hv/Hk):
 *   1. a causal depthwise conv over the last K = 4 raw tokens of every q, k, v
 *      channel, then SiLU (same story: causal convolution; model-atlas page for
 *      Qwen3-Coder-Next, raw config.json table: linear_conv_kernel_dim 4);
 *   2. L2 normalisation of q and k per token and key head, then q *= scale;
 *   3. the gated delta rule on a dv x dk state S per value head
 *        S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,  o_t = S_t q_t,
 *      a_t = exp(g_t) the decay gate, b_t = beta_t the update-strength gate
 *      (same story: beta gates the strength of the update; kv_mem is the
 *      memory read at the new key);
 *   4. the z-gated RMSNorm of o_t over dv (eps 1e-6: rms_norm_eps in the raw
 *      config.json table; Zero-Centered RMSNorm in the story):
 *        out_t = o_t / sqrt(mean(o_t^2) + norm_eps) * norm_w * SiLU(z_t).
 * Head shapes are those of the same config table: 16 key heads, 32 value
 * heads, key and value head dim 128.  Prefill uses the chunked form with
 * chunk 64 (FLA_CHUNK_SIZE in the SGLang cookbook's Mamba Radix Cache tip);
 * the recurrent state is fp32, optionally bf16 in decode (--mamba-ssm-dtype
 * in the cookbook's Configuration Tips: bf16 saves cache, fp32 is the more
 * accurate default).
 *
 * Conventions common to every entry point
 *  - Pointers to tensors are DEVICE pointers owned by the caller.  The library
 *    never allocates or frees device memory and never synchronises (except
 *    gdn_prefill_wait_status, a query that does so by definition); scratch
 *    memory comes from the caller's workspace (gdn_prefill_static: a static
 *    array inside the library, below).  Whatever a call leaves behind on the
 *    device lives in the caller's buffers (or that array); the host side keeps only
 *    thread-safe caches (CU counts per device, an epoch counter).  Concurrent
 *    calls on different streams are safe when their buffers (workspaces
 *    included) do not overlap.
 *  - Calls are asynchronous in the order of `stream`.  GDN_OK means the work
 *    was enqueued.
 *  - Every argument is validated on the host before anything is enqueued; on
 *    an error nothing runs and no output is touched.  The library never reads
 *    device memory from the host, so the contents of cu_seqlens and
 *    state_slots are preconditions (below), not checked.
 *  - Every tensor pointer must be 16-byte aligned; the workspace 256-byte
 *    aligned.
 *  - Layouts are row-major, last index contiguous.  Channel order of the conv
 *    weights and conv states: q (Hk*dk) | k (Hk*dk) | v (Hv*dv).
 *  - bf16 stores round to nearest even.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL_ARG = 1,     /* a required pointer is NULL, or z / norm_w given alone */
    GDN_ERR_BAD_SHAPE = 2,    /* counts out of range, Hv % Hk != 0, T_total != N in decode */
    GDN_ERR_UNSUPPORTED = 3,  /* head dims other than 128, conv kernel other than 4, unknown flags */
    GDN_ERR_BAD_DTYPE = 4,    /* unknown dtype, or a state dtype the call does not support */
    GDN_ERR_MISALIGNED = 5,   /* a tensor not 16-byte aligned, or workspace not 256-byte aligned */
    GDN_ERR_WORKSPACE = 6,    /* workspace NULL or smaller than gdn_prefill_workspace_size */
    GDN_ERR_HIP = 7,          /* a HIP launch or event call failed */
    GDN_ERR_ALIAS = 8,        /* an output overlaps an input in a way the call does not allow */
    GDN_ERR_BAD_VALUE = 9     /* a non-finite scale or eps, or a negative eps */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* L2-normalise q and k (step 2).  Without it q and k enter the recurrence as
 * they leave the conv (or as given, without conv); scale is still applied. */
#define GDN_FLAG_L2NORM_QK 0x1u
/* Prefill launch form (see gdn_prefill, "Launches"): never the pipelined
 * single launch, always separate kernels one after another (the plain ones,
 * or with GDN_FLAG_SEGMENTS also given, the segment-parallel ones). */
#define GDN_FLAG_SEPARATE_LAUNCHES 0x2u
/* Pipelined prefill: every prep unit writes its results back to memory
 * before publishing them, instead of leaving them in the L2 of the XCD that
 * all of their readers run on (same results; a diagnostic switch). */
#define GDN_FLAG_PREP_WRITE_BACK 0x4u
/* Testing the failure report: every wait of a pipelined launch gives up at
 * its first check instead of after about 2.7 s, so the call ends quickly with
 * invalid outputs and gdn_prefill_wait_status reports it.  No effect on
 * separate launches. */
#define GDN_FLAG_TEST_WAITS_GIVE_UP 0x8u
/* Prefill launch form for one sequence (no cu_seqlens) with bf16 io, an fp32
 * state, no state pool slots and no snapshots: segment-parallel separate
 * launches (see gdn_prefill, "Segments") at any head count and from 8 chunks
 * on.  Calls that do not qualify ignore it.  The workspace of a descriptor
 * that may take this form is larger (gdn_prefill_workspace_size takes the
 * flag and the default rule into account). */
#define GDN_FLAG_SEGMENTS 0x10u
/* Prefill launch form: the pipelined single launch wherever its conditions
 * hold (see gdn_prefill, "Launches"), also for the small calls that otherwise
 * take separate launches (one sequence with at most 16 value heads, or at
 * most 16 chunk slots, where separate launches are faster) and instead of the
 * default segment-parallel form.  GDN_FLAG_SEPARATE_LAUNCHES wins over it. */
#define GDN_FLAG_PIPELINED 0x20u

typedef struct {
    int32_t num_seqs;       /* N >= 1 */
    int64_t total_tokens;   /* prefill: T_total = cu_seqlens[N] >= 0, < 2^31;  decode: == N */
    int32_t num_k_heads;    /* Hk >= 1 */
    int32_t num_v_heads;    /* Hv >= 1, Hv % Hk == 0 */
    int32_t head_k_dim;     /* dk: 128 */
    int32_t head_v_dim;     /* dv: 128 */
    int32_t conv_kernel;    /* K: 4 */
    gdn_dtype io_dtype;     /* q, k, v, z, out, conv_w, norm_w, conv states */
    gdn_dtype state_dtype;  /* recurrent state storage: F32 or BF16 (gdn_prefill: F32) */
    float scale;            /* multiplies q after normalisation; 1.0 leaves q as is */
    float l2_eps;           /* step 2: x / sqrt(sum x^2 + l2_eps) */
    float norm_eps;         /* step 4 */
    uint32_t flags;         /* GDN_FLAG_* */
} gdn_desc;

/* Human-readable name of a status code (static storage). */
const char* gdn_status_string(gdn_status s);

/* Outcome of the last prefill call enqueued with `workspace` (see
 * gdn_prefill, "Launches"): waits for `stream` (the stream that call ran on),
 * then reads two words the call keeps at the start of its workspace.
 * *failed = 1 when a wait of that call's pipelined launch gave up (its
 * outputs are then invalid), 0 otherwise, and 0 for a workspace no prefill
 * call has used yet.  Synchronous: the one entry point that blocks the host.
 * GDN_ERR_WORKSPACE for a workspace smaller than 256 bytes, GDN_ERR_HIP when
 * the synchronisation or the copy fails. */
gdn_status gdn_prefill_wait_status(const void* workspace, size_t workspace_bytes,
                                   hipStream_t stream, int32_t* failed);

/* Bytes of device workspace gdn_prefill needs for descriptor d (a bound that
 * depends on N and T_total only through total_tokens / 64 + N chunks, plus,
 * for a descriptor the segment-parallel form may serve (one sequence, bf16
 * io, fp32 state; GDN_FLAG_SEGMENTS, or at most 16 value heads and at least
 * 2,048 tokens without GDN_FLAG_SEPARATE_LAUNCHES), 46 state-sized buffers
 * and 256 bytes per token and value head). */
gdn_status gdn_prefill_workspace_size(const gdn_desc* d, size_t* bytes);


/*
 * Prefill: every token of N packed sequences.
 *   q, k           [T_total, Hk, dk] io dtype, raw (before the conv)
 *   v              [T_total, Hv, dv] io dtype, raw
 *   g, beta        [T_total, Hv] fp32: g is the log-decay (a = exp(g)), beta is b
 *   z              [T_total, Hv, dv] io dtype, gate input        } both NULL:
 *   norm_w         [dv] io dtype, effective RMSNorm weight       } out = o
 *                  (with T_total == 0, q, k, v, g, beta, z, out may be NULL)
 *   conv_w         [Cch, K] io dtype, Cch = 2*Hk*dk + Hv*dv; NULL: no conv
 *   cu_seqlens     [N+1] int32 device; cu[0] = 0, non-decreasing, cu[N] =
 *                  T_total (precondition).  NULL allowed only when N == 1.
 *   initial_state  [N, Hv, dv, dk] fp32; NULL: zeros
 *   conv_state_in  [N, K-1, Cch] io dtype, oldest token first; NULL: zeros
 *   out            [T_total, Hv, dv] io dtype
 *   final_state    [N, Hv, dv, dk] fp32 or NULL; may equal initial_state
 *   conv_state_out [N, K-1, Cch] io dtype or NULL; may equal conv_state_in.
 *                  Holds the K-1 most recent raw tokens of (conv_state_in,
 *                  sequence tokens): a bit-exact copy of inputs.
 *   workspace      gdn_prefill_workspace_size bytes, contents ignored.
 * Zero-length sequences pass their states through.  Any other overlap
 * between outputs and inputs is GDN_ERR_ALIAS (out against q, k, v, z) or
 * undefined.
 *
 * Launches: with bf16 io, when the sweep's workgroups need more than an
 * eighth and at most half of the device's CUs and there are more than 16
 * chunk slots (one or a few long sequences at 32 value heads), the chunk prep
 * and the sweep run as one launch whose sweep workgroups wait for each chunk's prep
 * units, and whose gated-norm workgroups wait for the sweep's output, through
 * flags in the workspace (GDN_FLAG_SEPARATE_LAUNCHES selects separate
 * launches instead).  A chunk's prep results stay in the L2 of the XCD that
 * all of their readers run on, where each sweep workgroup records its XCD;
 * units whose readers are elsewhere write them back to memory first
 * (GDN_FLAG_PREP_WRITE_BACK: every unit does).  Every form gives the same
 * bits.
 * Forward progress of the pipelined launch rests on how the device dispatches
 * one launch's workgroups, which the library arranges for but cannot enforce:
 *  - workgroups start in increasing grid order, workgroup x on XCD x mod 8
 *    (eight XCDs, each dispatching from its own share of the grid);
 *  - one workgroup per CU (each takes more than half of a CU's 160 KB LDS);
 *  - the waiting workgroups (the sweep's, at most half of the CUs, and the
 *    gated norm's, together at most three quarters, counted per XCD) never
 *    hold every CU: the prep workgroups they wait for always find one, unless
 *    work on other streams occupies the remaining CUs until the waits give up.
 * Every wait is bounded (about 2.7 s of wall clock).  One that gives up marks
 * the call as failed in its workspace and stops waiting, so the launch still
 * ends; that call's outputs are then invalid, and gdn_prefill_wait_status
 * reports it.  Callers that cannot keep the CUs free for the call, or that
 * must not depend on the dispatch order, pass GDN_FLAG_SEPARATE_LAUNCHES: the
 * separate kernels never wait on each other.
 * Segments (GDN_FLAG_SEGMENTS, one qualifying sequence): the recurrence is
 * linear in the state (hyper.ai story, Gated DeltaNet paragraph: each token's
 * update multiplies the state by a_t (I - b_t k_t k_t^T) and adds
 * b_t v_t k_t^T), so over a run of chunks the state obeys S_end = S_start Phi
 * + S'_end and every output o_t = o'_t + S_start r_t, where S'_end and o'_t
 * come from a zero start and Phi, r_t from the identity start with v = 0.
 * The chunks are cut into P segments (P from 2 to 16: about sqrt(4 C / 3) for
 * C chunks, at most as many as one round of the device's CUs takes with
 * their identity chains); the sweep runs every segment from a zero state
 * (the first from initial_state) beside one such identity chain per later
 * segment, all at once, then one kernel chains the segments' start states
 * and the final state, and one adds S_start r_t to the outputs of the later
 * segments and applies their gated norm.  Results agree with the other forms
 * within rounding (not bit for bit).  Separate launches: no waits.  Taken by
 * default, without the flag, for one qualifying sequence of at least 32 chunks
 * with at most 16 value heads (one GPU's share of the 16 key / 32 value head
 * layer under 2-, 4- or 8-way head parallelism: the chain of chunk steps,
 * not the device's width, sets the time there), unless
 * GDN_FLAG_SEPARATE_LAUNCHES or GDN_FLAG_PIPELINED is given without it.
 */
gdn_status gdn_prefill(const gdn_desc* d,
                       const void* q, const void* k, const void* v,
                       const float* g, const float* beta,
                       const void* z, const void* conv_w, const void* norm_w,
                       const int32_t* cu_seqlens,
                       const float* initial_state, const void* conv_state_in,
                       void* out, float* final_state, void* conv_state_out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * gdn_prefill with per-kernel timing.  events: 2 + 2 * max_kernels
 * caller-created hipEvent_t.  events[0] and events[1] are recorded on
 * `stream` at the start and at the end of the call; kernel i ran between
 * events[2 + 2 i] and events[3 + 2 i], recorded on the stream it was
 * launched on.  stage_ids[i] (GDN_STAGE_*, max_kernels entries) names kernel
 * i's stage; *num_kernels receives the number of kernels.  A call that would
 * launch more than max_kernels kernels fails with GDN_ERR_HIP before
 * launching any.
 */
enum {
    GDN_STAGE_CHUNK_TABLE = 0,   /* chunk offsets of the packed sequences */
    GDN_STAGE_CHUNK_PREP = 1,    /* conv, SiLU, L2, gates, K K^T, UT transform: W, U~, P */
    GDN_STAGE_STATE_SWEEP = 2,   /* sequential chunk sweep: U, O, state update */
    GDN_STAGE_GATED_NORM = 3,    /* z-gated RMSNorm of the output */
    GDN_STAGE_CONV_STATE = 4,    /* conv state out */
    GDN_STAGE_PIPELINE = 5,      /* chunk prep and state sweep in one launch */
    GDN_STAGE_SEG_COMPOSE = 6,   /* segments: start states and final state */
    GDN_STAGE_SEG_FIXUP = 7      /* segments: start-state part of the outputs */
};
gdn_status gdn_prefill_profiled(const gdn_desc* d,
                                const void* q, const void* k, const void* v,
                                const float* g, const float* beta,
                                const void* z, const void* conv_w, const void* norm_w,
                                const int32_t* cu_seqlens,
                                const float* initial_state, const void* conv_state_in,
                                void* out, float* final_state, void* conv_state_out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream,
                                hipEvent_t* events, int32_t max_kernels, int32_t* num_kernels,
                                int32_t* stage_ids);

/*
 * Prefill with every option, arguments in one struct (fields as in
 * gdn_prefill unless stated; unused options zero / NULL).
 *
 * State pool.  state_slots [N] int32 device, or NULL: the row of
 * initial_state, final_state, conv_state_in and conv_state_out that sequence
 * n uses (NULL: row n).  Precondition: distinct, in [0, num_state_slots).
 * The four state tensors then have num_state_slots rows (>= N without
 * slots); rows no sequence names are not touched.  (SGLang cookbook,
 * Configuration Tips: the per-request state cache of --max-mamba-cache-size.)
 *
 * State dtype.  desc->state_dtype F32 or BF16 selects the storage of
 * initial_state, final_state and state_snapshots: [rows, Hv, dv, dk]; the
 * recurrence always runs on an fp32 state, bf16 is read widened and written
 * rounded to nearest even.  (Same page: --mamba-ssm-dtype.)
 *
 * Snapshots.  With state_snapshots non-NULL and snapshot_every = m >= 1, the
 * state after each chunk boundary 64 m j < L_n (j = 1, 2, ...) of sequence n
 * is also written, to row snapshot_base[n] + j - 1 of state_snapshots
 * [num_snapshot_slots, Hv, dv, dk] (state dtype).  snapshot_base [N] int32
 * device; precondition: rows in [0, num_snapshot_slots), not shared between
 * sequences.  The state after the last token is final_state, never a
 * snapshot.  (Same page, the branching-point cache of the radix cache.)
 *
 * Errors as gdn_prefill; in addition GDN_ERR_BAD_SHAPE for num_state_slots <
 * 1 (or < N without slots), snapshot_every < 1 or num_snapshot_slots < 1
 * with snapshots, GDN_ERR_NULL_ARG for snapshots without snapshot_base, and
 * GDN_ERR_ALIAS for a snapshot array that overlaps any other tensor.
 */
typedef struct {
    const void* q; const void* k; const void* v;
    const float* g; const float* beta;
    const void* z; const void* conv_w; const void* norm_w;
    const int32_t* cu_seqlens;
    const void* initial_state;      /* state dtype */
    void* final_state;              /* state dtype */
    const void* conv_state_in;
    void* conv_state_out;
    const int32_t* state_slots;
    int32_t num_state_slots;        /* 0: N */
    void* state_snapshots;          /* state dtype, or NULL */
    const int32_t* snapshot_base;
    int32_t snapshot_every;
    int32_t num_snapshot_slots;
    void* out;
    void* workspace;
    size_t workspace_bytes;
} gdn_prefill_args;

gdn_status gdn_prefill_ex(const gdn_desc* d, const gdn_prefill_args* args, hipStream_t stream);

/*
 * Prefill without a workspace and without any allocation, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Arguments as gdn_prefill_ex, except:
 *  - args->workspace must be NULL and args->workspace_bytes 0
 *    (GDN_ERR_BAD_VALUE otherwise).  The scratch is a static device array of
 *    GDN_STATIC_SCRATCH_BYTES inside the library, one per GPU, held from the
 *    library's loading on that GPU until the process ends.
 *  - A call whose workspace (gdn_prefill_workspace_size of d) exceeds
 *    GDN_STATIC_SCRATCH_BYTES fails with GDN_ERR_WORKSPACE before anything
 *    runs.  At 16 key / 32 value heads with bf16 io that is T_total / 64 + N
 *    <= 73 chunk slots: up to 4,671 tokens in one sequence.
 *  - The separate launches always run (GDN_FLAG_SEPARATE_LAUNCHES is implied):
 *    no kernel waits on another, so there is no failure to query.
 *  - Every call on one GPU uses that GPU's one array, which keeps the last
 *    call's contents (no call depends on them): calls that overlap in time on
 *    one GPU (unordered streams, several threads) race and give undefined
 *    results.  Calls in one stream's order do not overlap.
 * The library calls no hipMalloc, hipFree or allocating routine here.
 */
#define GDN_STATIC_SCRATCH_BYTES ((size_t)128 << 20)
gdn_status gdn_prefill_static(const gdn_desc* d, const gdn_prefill_args* args, hipStream_t stream);

/*
 * Decode: one new token for each of N sequences against cached states.
 *   q, k           [N, Hk, dk] io dtype, raw
 *   v, z           [N, Hv, dv] io dtype (z NULL together with norm_w: out = o)
 *   g, beta        [N, Hv] fp32
 *   conv_w, norm_w as in gdn_prefill
 *   state          [S, Hv, dv, dk] state dtype (F32 or BF16), updated in place
 *   conv_state     [S, K-1, Cch] io dtype, updated in place (shifted by one
 *                  token); NULL: zero history and nothing written
 *   state_slots    [N] int32 device: row of state / conv_state used by
 *                  sequence n; NULL: row n.  Precondition: distinct, in
 *                  [0, S).  num_state_slots = S (>= N when state_slots is NULL).
 *   out            [N, Hv, dv] io dtype
 */
gdn_status gdn_decode(const gdn_desc* d,
                      const void* q, const void* k, const void* v,
                      const float* g, const float* beta,
                      const void* z, const void* conv_w, const void* norm_w,
                      void* state, void* conv_state,
                      const int32_t* state_slots, int32_t num_state_slots,
                      void* out, hipStream_t stream);

/*
 * Multi-token decode for speculative-decoding verify (SGLang cookbook,
 * section 3.2: MTP / NEXTN with several draft tokens per step).  D new tokens
 * per sequence (1 <= D <= GDN_MAX_DRAFT) run through the conv and the
 * recurrence in order, starting from the cached state and conv state, which
 * this call only reads.  The state and the conv window after every token are
 * written as checkpoints, so that accepting the first j tokens is a copy of
 * checkpoint j - 1 into the cache (gdn_decode_commit).  desc: num_seqs = N,
 * total_tokens = N * D.
 *   q, k           [N, D, Hk, dk] io dtype, raw
 *   v, z           [N, D, Hv, dv] io dtype (z NULL together with norm_w)
 *   g, beta        [N, D, Hv] fp32
 *   conv_w, norm_w as in gdn_prefill
 *   state          [S, Hv, dv, dk] state dtype, read only
 *   conv_state     [S, K-1, Cch] io dtype, read only; NULL: zero history
 *   state_slots    [N] int32 device or NULL (row n), as in gdn_decode
 *   state_ckpt     [N, D, Hv, dv, dk] state dtype: the state after token j
 *   conv_ckpt      [N, D, K-1, Cch] io dtype or NULL: the K-1 most recent
 *                  raw tokens after token j (bit-exact copies of inputs)
 *   out            [N, D, Hv, dv] io dtype
 * Outputs must not overlap inputs (GDN_ERR_ALIAS).
 */
#define GDN_MAX_DRAFT 8
gdn_status gdn_decode_verify(const gdn_desc* d, int32_t num_draft,
                             const void* q, const void* k, const void* v,
                             const float* g, const float* beta,
                             const void* z, const void* conv_w, const void* norm_w,
                             const void* state, const void* conv_state,
                             const int32_t* state_slots, int32_t num_state_slots,
                             void* state_ckpt, void* conv_ckpt, void* out,
                             hipStream_t stream);

/*
 * Commit accepted draft tokens: for every sequence n with a_n = accepted[n]
 * in 1..D, copy checkpoint a_n - 1 of state_ckpt (and of conv_ckpt, when both
 * it and conv_state are non-NULL) into cache row state_slots[n] (NULL: n);
 * a_n = 0 leaves the row as it is.  accepted: [N] int32 device; values
 * outside 0..D are a precondition violation (the row is left as it is).
 */
gdn_status gdn_decode_commit(const gdn_desc* d, int32_t num_draft,
                             const void* state_ckpt, const void* conv_ckpt,
                             const int32_t* accepted, void* state, void* conv_state,
                             const int32_t* state_slots, int32_t num_state_slots,
                             hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H */
