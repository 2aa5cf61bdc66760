/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention forward library.
 *
 * KDA is the gated delta rule with one base-2 decay per key channel. For each sequence
 * n and value head hv (q/k head h = hv / (HV / H)), with S an fp32 [K, V] state:
 *
 *     S <- Diag(2^g_t) S                      decay every key row d by 2^g_t[d]
 *     S <- S + beta_t k_t (v_t - S^T k_t)^T    delta-rule erase + write
 *     o_t = scale * S^T q_t                    read the updated state
 *
 * Source: "kernel-fun 0.2.0.dev1 sdist", ALGORITHM.md (intro and section Forward:
 * base-2 gates <= 0, GVA head map h = hv // (HV // H), scale = K^-0.5, the chunk
 * stages); "Add fused recurrent_kda for decode and inference prefill" (attention-gym
 * PR #317, description: per-token log2 gate, packed int32 offsets, empty slots, state
 * per logical sequence, fp32 state and compute).
 *
 * Conventions for every entry point
 *   - Tensors are device pointers to contiguous row-major arrays (last index fastest),
 *     owned by the caller. The library never allocates, frees or synchronises; all
 *     work is enqueued on `stream` (NULL = the default stream).
 *   - Layouts: q, k [B, T, H, K]; v [B, T, HV, V]; g fp32 [B, T, HV, K] (per-token
 *     log2 decay, expected <= 0); beta [B, T, HV]; states fp32 [N, HV, K, V];
 *     o [B, T, HV, V] in the q/k/v dtype.
 *   - Dense mode (cu_seqlens == NULL): N must equal B; sequence n is row b = n, all T
 *     tokens. Packed mode (cu_seqlens != NULL): B must be 1; cu_seqlens is an int32
 *     device array [N + 1]; sequence n is tokens cu_seqlens[n] .. cu_seqlens[n+1]-1.
 *     Repeated offsets are empty slots: their final state is their initial state
 *     copied bitwise (zeros without an initial state). Rows at or past cu_seqlens[N]
 *     are neither read nor written.
 *   - initial_state == NULL means zeros. final_state == NULL means no final state is
 *     wanted: nothing is stored. final_state may equal initial_state (in place).
 *     o must not alias any input.
 *   - scale == 0.0f selects K^-0.5.
 *   - Return value: KDA_OK or a negative kda_status; kda_last_error() then gives a
 *     reason (thread-local, valid until the next call on the same thread). Argument
 *     errors are detected on the host before anything is enqueued.
 *   - Device-side checks never fault: a packed slot whose offsets break
 *     0 = cu[0] <= cu[n] <= cu[n+1] <= T is skipped (its rows of o and its final state
 *     are left untouched) and KDA_DEV_BAD_CU_SEQLENS is OR-ed into *dev_status when
 *     dev_status != NULL. The check runs on every call, including graph replays.
 *     Offsets that decrease always fail some slot's check; slots that pass may then
 *     overlap, and their shared rows of o are unspecified. kda_chunk_fwd also skips
 *     and flags any slot whose chunks would exceed its chunk table (T/64 + N chunks),
 *     which only overlapping slots can reach.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum kda_status {
    KDA_OK = 0,
    KDA_ERR_NULL = -1,         /* a required pointer is NULL */
    KDA_ERR_SHAPE = -2,        /* inconsistent or non-positive sizes, HV % H != 0, ... */
    KDA_ERR_DTYPE = -3,        /* unknown dtype code */
    KDA_ERR_UNSUPPORTED = -4,  /* K, V or chunk size outside what the kernels cover */
    KDA_ERR_WORKSPACE = -5,    /* workspace missing, too small or misaligned */
    KDA_ERR_HIP = -6,          /* a kernel launch failed */
    KDA_ERR_ARG = -7           /* an option outside its documented set (gate, preprocess) */
};

enum kda_dtype {
    KDA_F32 = 0,
    KDA_BF16 = 1
};

/* bit flags written into *dev_status by device-side checks */
#define KDA_DEV_BAD_CU_SEQLENS 1

/* Where the per-token log2 decay comes from (the `gate` argument of the _ex entry points). */
enum kda_gate {
    KDA_GATE_LOG2 = 0,      /* g: fp32 per-token log2 decay, used as given */
    KDA_GATE_RAW_F32 = 1,   /* g: fp32 raw gate input; the activation is fused (see below) */
    KDA_GATE_RAW_BF16 = 2   /* g: bf16 raw gate input; the same activation */
};

/*
 * Input preprocessing fused into the kernels' loads (the `preprocess` argument of the _ex
 * entry points, a bitwise OR; 0 = inputs used as given). Source: "kernel-fun 0.2.0.dev1
 * sdist", the autograd Function's forward (use_qk_l2norm: fla's l2norm of q and k before
 * the gate cumsum) and the chunk_kda wrapper (use_beta_sigmoid_in_kernel: beta through a
 * sigmoid, times 2 when negative eigenvalues are allowed); the deferred q normalisation
 * of attention-gym PR #345 (description).
 *   KDA_PRE_L2NORM_Q     q <- q / sqrt(sum_d q_d^2 + 1e-6), per (token, head); the pages
 *                        give no epsilon, 1e-6 is the reading taken. The row scale is
 *                        applied in fp32 (on the bf16 path it is folded into the fp32
 *                        products that feed the matrix cores, so nothing is re-rounded).
 *   KDA_PRE_L2NORM_K     the same for k.
 *   KDA_PRE_BETA_SIGMOID beta <- sigmoid(beta), in fp32.
 *   KDA_PRE_NEG_EIGVAL   with KDA_PRE_BETA_SIGMOID: beta <- 2 sigmoid(beta), in (0, 2).
 *                        Invalid without it.
 */
#define KDA_PRE_L2NORM_Q 1
#define KDA_PRE_L2NORM_K 2
#define KDA_PRE_BETA_SIGMOID 4
#define KDA_PRE_NEG_EIGVAL 8

/*
 * Chunked forward (prefill). The method of "kernel-fun 0.2.0.dev1 sdist",
 * ALGORITHM.md, section Forward: chunks of 64 tokens (restarting at every sequence
 * start), chunk-local log2 cumsum of the gate (Stage 1), intra-chunk Aqk / WY
 * transform (Stage 2, 16-row sub-chunks), then the serial state scan with the output
 * read-out (Stage 3+4).
 *
 *   qkv_dtype  KDA_BF16: bf16 q, k, v, o; bf16 matrix-core operands, fp32 accumulation
 *              and fp32 state. KDA_F32: fp32 everywhere.
 *   beta_dtype KDA_BF16 or KDA_F32 (independent of qkv_dtype).
 *   K          64 or 128.  V: 64 or 128.  chunk_size: must be 64.
 *   workspace  device buffer of at least kda_chunk_fwd_workspace_bytes(...) bytes,
 *              256-byte aligned, owned by the caller; it holds the per-chunk
 *              intermediates of one call and must not be shared by calls that may
 *              run concurrently.
 */
int kda_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                  const void* beta, const float* initial_state, const int32_t* cu_seqlens,
                  int N, void* o, float* final_state, int B, int T, int H, int HV, int K,
                  int V, int qkv_dtype, int beta_dtype, float scale, int chunk_size,
                  void* workspace, size_t workspace_bytes, int32_t* dev_status,
                  hipStream_t stream);

/*
 * kda_chunk_fwd with in-place timing: identical arguments, results and errors, plus
 * `events`, an array of four HIP events created by the caller. They are recorded on
 * `stream` before the first kernel (events[0]), after the packed-mode scheduler
 * (events[1]; same point as events[0] in dense mode), after the Stage 1+2 kernel
 * (events[2]) and after the Stage 3+4 scan (events[3]), so the caller can read each
 * kernel's duration with hipEventElapsedTime. A NULL entry is not recorded (each
 * record is a marker on the stream; a caller timing steps back to back can record only
 * events[2] and events[3] and take the previous step's events[3] as the start).
 * events == NULL behaves like kda_chunk_fwd.
 * For profiling callers (benchmarks); nothing is synchronised.
 */
int kda_chunk_fwd_timed(const void* q, const void* k, const void* v, const float* g,
                        const void* beta, const float* initial_state,
                        const int32_t* cu_seqlens, int N, void* o, float* final_state, int B,
                        int T, int H, int HV, int K, int V, int qkv_dtype, int beta_dtype,
                        float scale, int chunk_size, void* workspace, size_t workspace_bytes,
                        int32_t* dev_status, hipStream_t stream, hipEvent_t* events);

/*
 * kda_chunk_fwd with the gate activation fused into Stage 1. Instead of the per-token
 * log2 decay, the caller passes the raw gate input w_g(x) and the activation's
 * parameters; the Stage 1 loads form, per element,
 *     log2 decay = -exp(A_log[hv]) * softplus(g_raw[b,t,hv,d] + dt_bias[hv*K + d]) / ln 2
 * (softplus(x) = log(1 + e^x)) and the chunk cumsum proceeds as in kda_chunk_fwd. The
 * activation and its place in the cumsum: "kernel-fun 0.2.0.dev1 sdist", the chain
 * module's gate_cumsum helper (A_log [HV], dt_bias [HV*K]), and ALGORITHM.md, Forward,
 * on the activation fused into stage 1; the cumsum's 1/ln 2 gives the base-2 gate.
 *
 *   g_raw            device [B, T, HV, K], dtype g_dtype (KDA_BF16 or KDA_F32).
 *   A_log            device fp32 [HV]; required.
 *   dt_bias          device fp32 [HV * K], or NULL for zeros.
 *   has_lower_bound  nonzero: the natural-log activation is first clamped from below at
 *                    lower_bound, which must then be negative and finite (the pages name
 *                    the option without a formula; a clamp is the reading taken).
 * Everything else -- arguments, workspace, results, errors -- as kda_chunk_fwd; the
 * workspace size is the same.
 */
int kda_chunk_fwd_gated(const void* q, const void* k, const void* v, const void* g_raw,
                        int g_dtype, const float* A_log, const float* dt_bias,
                        int has_lower_bound, float lower_bound, const void* beta,
                        const float* initial_state, const int32_t* cu_seqlens, int N, void* o,
                        float* final_state, int B, int T, int H, int HV, int K, int V,
                        int qkv_dtype, int beta_dtype, float scale, int chunk_size,
                        void* workspace, size_t workspace_bytes, int32_t* dev_status,
                        hipStream_t stream);

/*
 * The chunked forward with every option: the gate source (`gate`, a kda_gate; for
 * KDA_GATE_LOG2, A_log and dt_bias must be NULL and has_lower_bound 0, otherwise the
 * activation and its arguments are those of kda_chunk_fwd_gated, with g the raw gate
 * input), the input preprocessing flags (`preprocess`, KDA_PRE_*), and the optional
 * `events` of kda_chunk_fwd_timed (NULL for none). Everything else as kda_chunk_fwd;
 * the workspace size is the same. kda_chunk_fwd, kda_chunk_fwd_timed and
 * kda_chunk_fwd_gated are this call with gate and preprocess at their plain values.
 */
int kda_chunk_fwd_ex(const void* q, const void* k, const void* v, const void* g, int gate,
                     const float* A_log, const float* dt_bias, int has_lower_bound,
                     float lower_bound, const void* beta, int preprocess,
                     const float* initial_state, const int32_t* cu_seqlens, int N, void* o,
                     float* final_state, int B, int T, int H, int HV, int K, int V,
                     int qkv_dtype, int beta_dtype, float scale, int chunk_size,
                     void* workspace, size_t workspace_bytes, int32_t* dev_status,
                     hipStream_t stream, hipEvent_t* events);

/*
 * Workspace bytes kda_chunk_fwd needs for these sizes (packed != 0 for packed mode,
 * N sequences). Returns 0 for invalid sizes.
 */
size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int HV, int K, int V, int N,
                                     int packed, int qkv_dtype);

/*
 * Chunked backward (training): the gradients of kda_chunk_fwd's outputs with respect to
 * q, k, v, g (the per-token log2 decay), beta and the initial state. The method of
 * "kernel-fun 0.2.0.dev1 sdist", ALGORITHM.md, section Backward: recompute of the
 * chunk records, a re-scan that checkpoints the state at every chunk start and v', the
 * reverse scan of the state gradient (dv' per chunk), then per chunk the products with
 * the checkpoints, the backward of the WY inverse and the intra-chunk pair terms with
 * one-sided decay factors only; dg comes out already reverse-cumsummed (it is the
 * gradient with respect to g itself), and GVA dq, dk are summed over each q/k head's
 * value heads. All arithmetic is fp32.
 *
 *   q, k, v, g, beta, initial_state, cu_seqlens, N, sizes, dtypes, scale, chunk_size:
 *                as kda_chunk_fwd (the forward being differentiated).
 *   dout         device [B, T, HV, V] in qkv_dtype: the gradient with respect to o.
 *   dht          device fp32 [N, HV, K, V]: with respect to the final state, or NULL
 *                (zeros).
 *   dq, dk       device [B, T, H, K] in qkv_dtype.   dv  device [B, T, HV, V] in qkv_dtype.
 *   dg           device fp32 [B, T, HV, K].           dbeta  device [B, T, HV] in beta_dtype.
 *   dh0          device fp32 [N, HV, K, V], or NULL when not wanted. It is the gradient
 *                with respect to the initial state (zeros stand in for a NULL one).
 *   workspace    at least kda_chunk_bwd_workspace_bytes(...) bytes, 256-byte aligned;
 *                one call's intermediates (records, per-chunk fp32 state checkpoints and
 *                gradients), not shared between calls that may overlap.
 * Gradients of rows outside every sequence (packed tail, slots that fail the offset
 * check) are not written. No output may alias an input.
 */
int kda_chunk_bwd(const void* q, const void* k, const void* v, const float* g,
                  const void* beta, const float* initial_state, const int32_t* cu_seqlens,
                  int N, const void* dout, const float* dht, void* dq, void* dk, void* dv,
                  float* dg, void* dbeta, float* dh0, int B, int T, int H, int HV, int K,
                  int V, int qkv_dtype, int beta_dtype, float scale, int chunk_size,
                  void* workspace, size_t workspace_bytes, int32_t* dev_status,
                  hipStream_t stream);

/*
 * Training forward: kda_chunk_fwd's outputs (o, and the final state when final_state is
 * non-NULL) computed the way kda_chunk_bwd recomputes the forward (the method's backward
 * in "kernel-fun 0.2.0.dev1 sdist", ALGORITHM.md, section Backward, starts with that
 * recompute), leaving in the workspace everything that recompute produces: the
 * schedule, the per-chunk records, Stage 2's M and T, the state at every chunk start
 * and v'. A kda_chunk_bwd_saved call with the same inputs and this workspace then skips
 * the recompute. Arguments as kda_chunk_fwd, except:
 *   workspace    at least kda_chunk_bwd_workspace_bytes(...) bytes (the backward's
 *                size), 256-byte aligned; it belongs to this forward and its backward
 *                until that backward has run.
 * o agrees with kda_chunk_fwd's to the tolerance of the bf16 path (bit for bit where
 * kda_chunk_fwd's scan takes 16-column slices: chains x V / 32 < 512).
 */
int kda_chunk_fwd_train(const void* q, const void* k, const void* v, const float* g,
                        const void* beta, const float* initial_state, const int32_t* cu_seqlens,
                        int N, void* o, float* final_state, int B, int T, int H, int HV, int K,
                        int V, int qkv_dtype, int beta_dtype, float scale, int chunk_size,
                        void* workspace, size_t workspace_bytes, int32_t* dev_status,
                        hipStream_t stream);

/*
 * kda_chunk_bwd from a kda_chunk_fwd_train workspace: the same arguments and results
 * (bit for bit), without the forward recompute. The inputs must be those of that
 * forward and the workspace untouched since; the workspace is then used as
 * kda_chunk_bwd uses its own.
 */
int kda_chunk_bwd_saved(const void* q, const void* k, const void* v, const float* g,
                        const void* beta, const float* initial_state, const int32_t* cu_seqlens,
                        int N, const void* dout, const float* dht, void* dq, void* dk, void* dv,
                        float* dg, void* dbeta, float* dh0, int B, int T, int H, int HV, int K,
                        int V, int qkv_dtype, int beta_dtype, float scale, int chunk_size,
                        void* workspace, size_t workspace_bytes, int32_t* dev_status,
                        hipStream_t stream);

/*
 * kda_chunk_bwd for a forward run with the options of kda_chunk_fwd_ex: the same `g`,
 * `gate`, A_log, dt_bias, has_lower_bound, lower_bound, beta and `preprocess` arguments
 * (and rules) as that forward. The gradients are with respect to the raw inputs:
 *   dq, dk     through the L2 normalisation when KDA_PRE_L2NORM_Q / _K is set
 *              (dx = r (dy - y (y . dy)), y = x r, r = (sum x^2 + 1e-6)^-1/2);
 *   dbeta      through the sigmoid when KDA_PRE_BETA_SIGMOID is set (c s (1 - s));
 *   dg         fp32 [B, T, HV, K]: with respect to g itself (the log2 decay, or the raw
 *              gate input), through the activation where the lower bound does not clamp;
 *   dA_log     device fp32 [HV], required with a raw gate (NULL otherwise);
 *   ddt_bias   device fp32 [HV * K], required when dt_bias is given.
 * The gate backward is the one of "kernel-fun 0.2.0.dev1 sdist" (the chain module's
 * gate_backward: dg with respect to the raw input, dA_log, ddt_bias); the normalisation
 * backward is fla's l2norm_bwd, which that page's autograd Function applies to dq and
 * dk. The options are applied in fp32 to the inputs each kernel stages, as in the fused
 * forward; the workspace (kda_chunk_bwd_ex_workspace_bytes) adds the fp32 gradients of
 * the transformed gate and beta. Everything else as kda_chunk_bwd.
 */
int kda_chunk_bwd_ex(const void* q, const void* k, const void* v, const void* g, int gate,
                     const float* A_log, const float* dt_bias, int has_lower_bound,
                     float lower_bound, const void* beta, int preprocess,
                     const float* initial_state, const int32_t* cu_seqlens, int N,
                     const void* dout, const float* dht, void* dq, void* dk, void* dv, float* dg,
                     void* dbeta, float* dh0, float* dA_log, float* ddt_bias, int B, int T,
                     int H, int HV, int K, int V, int qkv_dtype, int beta_dtype, float scale,
                     int chunk_size, void* workspace, size_t workspace_bytes,
                     int32_t* dev_status, hipStream_t stream);

/*
 * kda_chunk_fwd_train with the options of kda_chunk_fwd_ex (the same g, gate, A_log,
 * dt_bias, has_lower_bound, lower_bound, beta and preprocess arguments and rules), and
 * kda_chunk_bwd_ex from its workspace (at least kda_chunk_bwd_ex_workspace_bytes bytes):
 * the same arguments and results as kda_chunk_bwd_ex, without the forward recompute.
 * Everything else as kda_chunk_fwd_train and kda_chunk_bwd_saved.
 */
int kda_chunk_fwd_ex_train(const void* q, const void* k, const void* v, const void* g, int gate,
                           const float* A_log, const float* dt_bias, int has_lower_bound,
                           float lower_bound, const void* beta, int preprocess,
                           const float* initial_state, const int32_t* cu_seqlens, int N, void* o,
                           float* final_state, int B, int T, int H, int HV, int K, int V,
                           int qkv_dtype, int beta_dtype, float scale, int chunk_size,
                           void* workspace, size_t workspace_bytes, int32_t* dev_status,
                           hipStream_t stream);
int kda_chunk_bwd_ex_saved(const void* q, const void* k, const void* v, const void* g, int gate,
                           const float* A_log, const float* dt_bias, int has_lower_bound,
                           float lower_bound, const void* beta, int preprocess,
                           const float* initial_state, const int32_t* cu_seqlens, int N,
                           const void* dout, const float* dht, void* dq, void* dk, void* dv, float* dg,
                           void* dbeta, float* dh0, float* dA_log, float* ddt_bias, int B, int T,
                           int H, int HV, int K, int V, int qkv_dtype, int beta_dtype, float scale,
                           int chunk_size, void* workspace, size_t workspace_bytes,
                           int32_t* dev_status, hipStream_t stream);

/* Workspace bytes kda_chunk_bwd_ex needs; 0 for invalid sizes. */
size_t kda_chunk_bwd_ex_workspace_bytes(int B, int T, int H, int HV, int K, int V, int N,
                                        int packed, int qkv_dtype);

/* Workspace bytes kda_chunk_bwd needs for these sizes; 0 for invalid sizes. */
size_t kda_chunk_bwd_workspace_bytes(int B, int T, int H, int HV, int K, int V, int N,
                                     int packed, int qkv_dtype);

/*
 * Per-token recurrent forward (decode, or a token-by-token prefill): the contract of
 * "Add fused recurrent_kda for decode and inference prefill" (attention-gym PR #317):
 * each (sequence, value head, 64-column slice of V) walks its tokens in order with
 * its fp32 state slice in registers; fp32 arithmetic whatever the input dtype; one
 * flat 1-D grid, so N * HV may exceed 65,535.
 *
 *   qkv_dtype, beta_dtype  KDA_BF16 or KDA_F32.   K: 64 or 128.   V: a multiple of 64.
 */
int kda_recurrent_fwd(const void* q, const void* k, const void* v, const float* g,
                      const void* beta, const float* initial_state,
                      const int32_t* cu_seqlens, int N, void* o, float* final_state, int B,
                      int T, int H, int HV, int K, int V, int qkv_dtype, int beta_dtype,
                      float scale, int32_t* dev_status, hipStream_t stream);

/* State layouts of the recurrent entry points (the `state_layout` argument). */
enum kda_state_layout {
    KDA_STATE_KV = 0,   /* [N, HV, K, V] (the default everywhere) */
    KDA_STATE_VK = 1    /* [N, HV, V, K]: each state stored transposed */
};

/*
 * kda_recurrent_fwd with every decode option: the gate source and the input
 * preprocessing of kda_chunk_fwd_ex (the same `gate`, A_log, dt_bias, has_lower_bound,
 * lower_bound and `preprocess` arguments and rules), the layout of initial_state,
 * final_state and intermediate_states (`state_layout`, a kda_state_layout: the
 * transposed layout is fla's state_v_first / transpose_state_layout, named on the
 * "kernel-fun 0.2.0.dev1 sdist" page among the flags its op does not take), and
 * `intermediate_states`: NULL, or device fp32 [B*T, HV, K*V] receiving the state after
 * every token of every sequence (fla's return_intermediate_states; row r's entries are
 * written only for rows inside a sequence). The decode serving path of "Add fused
 * recurrent_kda for decode and inference prefill" (attention-gym PR #317).
 */
int kda_recurrent_fwd_ex(const void* q, const void* k, const void* v, const void* g, int gate,
                         const float* A_log, const float* dt_bias, int has_lower_bound,
                         float lower_bound, const void* beta, int preprocess, int state_layout,
                         const float* initial_state, const int32_t* cu_seqlens, int N,
                         void* o, float* final_state, float* intermediate_states, int B, int T,
                         int H, int HV, int K, int V, int qkv_dtype, int beta_dtype,
                         float scale, int32_t* dev_status, hipStream_t stream);

/*
 * kda_chunk_fwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same arguments,
 * results and errors minus the workspace. The per-chunk intermediates go to a scratch
 * array of KDA_NOALLOC_SCRATCH_MB MiB that the library's code object holds in device
 * memory, one copy per GPU, kept until the process ends. Nothing is allocated or freed.
 *   - Problems whose kda_chunk_fwd_workspace_bytes() exceeds kda_noalloc_scratch_bytes()
 *     are rejected with KDA_ERR_WORKSPACE before anything is enqueued (e.g. at K = V =
 *     128 in bf16 about 500 (value head, 64-token chunk) pairs fit).
 *   - Every call on one GPU shares that GPU's array and leaves its intermediates there:
 *     calls that may overlap on one GPU (other streams, other host threads) race and
 *     must be serialised by the caller.
 *   - The first call on each GPU looks the array's address up (with that GPU current).
 */
#define KDA_NOALLOC_SCRATCH_MB 64
int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g,
                          const void* beta, const float* initial_state,
                          const int32_t* cu_seqlens, int N, void* o, float* final_state, int B,
                          int T, int H, int HV, int K, int V, int qkv_dtype, int beta_dtype,
                          float scale, int chunk_size, int32_t* dev_status, hipStream_t stream);

/* Bytes of the scratch array behind kda_chunk_fwd_noalloc (KDA_NOALLOC_SCRATCH_MB MiB). */
size_t kda_noalloc_scratch_bytes(void);

/* Reason for the last non-KDA_OK return on this thread ("" if none). */
const char* kda_last_error(void);

/* ABI version of this header (bumped on any signature change or added entry point);
 * the library returns the KDA_ABI_VERSION it was built with. */
#define KDA_ABI_VERSION 7
int kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
