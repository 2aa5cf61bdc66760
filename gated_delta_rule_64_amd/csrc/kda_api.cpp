// C ABI of the KDA library: argument validation, error strings and dispatch to the
// kernel launchers. Nothing here allocates, frees or synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include "kda_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_last_error[0] = '\0'; }

bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Checks shared by both entry points. Returns KDA_OK or an error code (with the reason).
int check_common(const void* q, const void* k, const void* v, const float* g, const void* beta,
                 const float* initial_state, const int32_t* cu_seqlens, int N, const void* o,
                 const float* final_state, int B, int T, int H, int HV, int K, int V,
                 int qkv_dtype, int beta_dtype) {
    if (qkv_dtype != KDA_BF16 && qkv_dtype != KDA_F32)
        return fail(KDA_ERR_DTYPE, "qkv_dtype must be KDA_BF16 (1) or KDA_F32 (0), got %d", qkv_dtype);
    if (beta_dtype != KDA_BF16 && beta_dtype != KDA_F32)
        return fail(KDA_ERR_DTYPE, "beta_dtype must be KDA_BF16 (1) or KDA_F32 (0), got %d", beta_dtype);
    if (B < 0 || T < 0 || H <= 0 || HV <= 0 || K <= 0 || V <= 0 || N < 0)
        return fail(KDA_ERR_SHAPE, "sizes must be non-negative (H, HV, K, V positive): B=%d T=%d H=%d HV=%d K=%d V=%d N=%d",
                    B, T, H, HV, K, V, N);
    if (HV % H != 0)
        return fail(KDA_ERR_SHAPE, "HV=%d must be a multiple of H=%d", HV, H);
    if (cu_seqlens) {
        if (B != 1) return fail(KDA_ERR_SHAPE, "packed sequences (cu_seqlens given) need B == 1, got B=%d", B);
    } else if (N != B) {
        return fail(KDA_ERR_SHAPE, "without cu_seqlens N must equal B (N=%d, B=%d)", N, B);
    }
    const long long rows = (long long)B * T;
    if (rows > 0x7fffffffLL)
        return fail(KDA_ERR_SHAPE, "B*T=%lld exceeds 2^31-1 rows", rows);
    if ((long long)N * HV > 0x7fffffffLL / 4)
        return fail(KDA_ERR_SHAPE, "N*HV=%lld too large", (long long)N * HV);
    if (rows > 0) {
        if (!q || !k || !v || !g || !beta || !o)
            return fail(KDA_ERR_NULL, "q, k, v, g, beta and o must be non-NULL");
    }
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(o) ||
        !aligned16(initial_state) || !aligned16(final_state))
        return fail(KDA_ERR_SHAPE, "q, k, v, g, o and the states must be 16-byte aligned");
    return KDA_OK;
}

// Builds the kernels' InputSpec from the gate and preprocessing arguments and checks them
// (g itself, log2 decay or raw input, goes through the common pointer checks).
int make_input_spec(const void* g, int gate, const float* A_log, const float* dt_bias,
                    int has_lower_bound, float lower_bound, int preprocess, bool nonempty,
                    kda::InputSpec* in) {
    if (gate != KDA_GATE_LOG2 && gate != KDA_GATE_RAW_F32 && gate != KDA_GATE_RAW_BF16)
        return fail(KDA_ERR_ARG, "gate must be KDA_GATE_LOG2 (0), KDA_GATE_RAW_F32 (1) or KDA_GATE_RAW_BF16 (2), got %d", gate);
    if (preprocess & ~(KDA_PRE_L2NORM_Q | KDA_PRE_L2NORM_K | KDA_PRE_BETA_SIGMOID | KDA_PRE_NEG_EIGVAL))
        return fail(KDA_ERR_ARG, "preprocess has unknown bits: 0x%x", preprocess);
    if ((preprocess & KDA_PRE_NEG_EIGVAL) && !(preprocess & KDA_PRE_BETA_SIGMOID))
        return fail(KDA_ERR_ARG, "KDA_PRE_NEG_EIGVAL needs KDA_PRE_BETA_SIGMOID");
    if (gate == KDA_GATE_LOG2) {
        if (A_log || dt_bias || has_lower_bound)
            return fail(KDA_ERR_ARG, "A_log, dt_bias and a lower bound belong to a raw gate input (gate=%d is the log2 decay)", gate);
    } else {
        if (has_lower_bound && !(lower_bound < 0.0f && isfinite(lower_bound)))
            return fail(KDA_ERR_SHAPE, "lower_bound must be negative and finite, got %g", (double)lower_bound);
        if (nonempty && !A_log) return fail(KDA_ERR_NULL, "A_log must be non-NULL");
        if (!aligned16(dt_bias)) return fail(KDA_ERR_SHAPE, "dt_bias must be 16-byte aligned");
    }
    in->gate_mode = gate;
    in->g_raw = gate == KDA_GATE_LOG2 ? nullptr : g;
    in->A_log = gate == KDA_GATE_LOG2 ? nullptr : A_log;
    in->dt_bias = gate == KDA_GATE_LOG2 ? nullptr : dt_bias;
    in->has_lower_bound = gate != KDA_GATE_LOG2 && has_lower_bound ? 1 : 0;
    in->lower_bound = lower_bound;
    in->l2norm_q = (preprocess & KDA_PRE_L2NORM_Q) ? 1 : 0;
    in->l2norm_k = (preprocess & KDA_PRE_L2NORM_K) ? 1 : 0;
    in->beta_sig = (preprocess & KDA_PRE_BETA_SIGMOID) ? ((preprocess & KDA_PRE_NEG_EIGVAL) ? 2.0f : 1.0f) : 0.0f;
    return KDA_OK;
}

// The chunked forward behind every chunk entry point.
int chunk_impl(const void* q, const void* k, const void* v, const void* g, int gate,
               const float* A_log, const float* dt_bias, int has_lower_bound, float lower_bound,
               const void* beta, int preprocess, const float* initial_state,
               const int32_t* cu_seqlens, int N, void* o, float* final_state, int B, int T, int H,
               int HV, int K, int V, int qkv_dtype, int beta_dtype, float scale, int chunk_size,
               void* workspace, size_t workspace_bytes, int32_t* dev_status, hipStream_t stream,
               hipEvent_t* events) {
    int rc = check_common(q, k, v, static_cast<const float*>(g), beta, initial_state, cu_seqlens, N,
                          o, final_state, B, T, H, HV, K, V, qkv_dtype, beta_dtype);
    if (rc != KDA_OK) return rc;
    kda::InputSpec in;
    rc = make_input_spec(g, gate, A_log, dt_bias, has_lower_bound, lower_bound, preprocess,
                         (long long)B * T > 0, &in);
    if (rc != KDA_OK) return rc;
    if (chunk_size != 64)
        return fail(KDA_ERR_UNSUPPORTED, "chunk_size must be 64, got %d", chunk_size);
    if (K != 64 && K != 128)
        return fail(KDA_ERR_UNSUPPORTED, "K must be 64 or 128, got %d", K);
    if (V != 64 && V != 128)
        return fail(KDA_ERR_UNSUPPORTED, "V must be 64 or 128, got %d", V);
    if (cu_seqlens && (long long)T / 64 + N > 0x7fffffffLL / HV)
        return fail(KDA_ERR_SHAPE, "too many chunks");
    kda::ChunkLayout L;
    kda::chunk_layout(B, T, HV, K, V, N, cu_seqlens != nullptr, qkv_dtype, &L);
    if (N == 0) return KDA_OK;
    if (L.total > 0) {
        if (!workspace)
            return fail(KDA_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", L.total);
        if (workspace_bytes < L.total)
            return fail(KDA_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes, L.total);
        if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
            return fail(KDA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    }
    kda::ChunkArgs a;
    a.q = q; a.k = k; a.v = v; a.beta = beta;
    a.g = gate == KDA_GATE_LOG2 ? static_cast<const float*>(g) : nullptr;
    a.in = in;
    a.initial_state = initial_state; a.cu_seqlens = cu_seqlens;
    a.o = o; a.final_state = final_state;
    a.N = N; a.B = B; a.T = T; a.H = H; a.HV = HV; a.K = K; a.V = V;
    a.qkv_dtype = qkv_dtype; a.beta_dtype = beta_dtype;
    a.scale = scale == 0.0f ? 1.0f / sqrtf((float)K) : scale;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    a.dev_status = dev_status; a.stream = stream; a.events = events;
    hipError_t err = kda::launch_chunk(a, L);
    if (err != hipSuccess)
        return fail(KDA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return KDA_OK;
}

// The per-token forward behind both recurrent entry points.
int recurrent_impl(const void* q, const void* k, const void* v, const void* g, int gate,
                   const float* A_log, const float* dt_bias, int has_lower_bound,
                   float lower_bound, const void* beta, int preprocess, int state_layout,
                   const float* initial_state, const int32_t* cu_seqlens, int N, void* o,
                   float* final_state, float* inter_states, int B, int T, int H, int HV, int K,
                   int V, int qkv_dtype, int beta_dtype, float scale, int32_t* dev_status,
                   hipStream_t stream) {
    int rc = check_common(q, k, v, static_cast<const float*>(g), beta, initial_state, cu_seqlens, N,
                          o, final_state, B, T, H, HV, K, V, qkv_dtype, beta_dtype);
    if (rc != KDA_OK) return rc;
    kda::InputSpec in;
    rc = make_input_spec(g, gate, A_log, dt_bias, has_lower_bound, lower_bound, preprocess,
                         (long long)B * T > 0, &in);
    if (rc != KDA_OK) return rc;
    if (K != 64 && K != 128)
        return fail(KDA_ERR_UNSUPPORTED, "K must be 64 or 128, got %d", K);
    if (V % 64 != 0)
        return fail(KDA_ERR_UNSUPPORTED, "V must be a multiple of 64, got %d", V);
    if ((long long)N * HV * (V / 16) > 0x7fffffffLL * 4LL)
        return fail(KDA_ERR_SHAPE, "grid too large");
    if (state_layout != KDA_STATE_KV && state_layout != KDA_STATE_VK)
        return fail(KDA_ERR_ARG, "state_layout must be KDA_STATE_KV (0) or KDA_STATE_VK (1), got %d", state_layout);
    if (!aligned16(inter_states))
        return fail(KDA_ERR_SHAPE, "intermediate_states must be 16-byte aligned");
    if (N == 0) return KDA_OK;
    kda::RecurrentArgs a;
    a.q = q; a.k = k; a.v = v; a.beta = beta;
    a.g = gate == KDA_GATE_LOG2 ? static_cast<const float*>(g) : nullptr;
    a.in = in;
    a.initial_state = initial_state; a.cu_seqlens = cu_seqlens;
    a.o = o; a.final_state = final_state;
    a.N = N; a.B = B; a.T = T; a.H = H; a.HV = HV; a.K = K; a.V = V;
    a.qkv_dtype = qkv_dtype; a.beta_dtype = beta_dtype;
    a.scale = scale == 0.0f ? 1.0f / sqrtf((float)K) : scale;
    a.dev_status = dev_status; a.stream = stream;
    a.state_vk = state_layout == KDA_STATE_VK ? 1 : 0;
    a.inter_states = inter_states;
    hipError_t err = kda::launch_recurrent(a);
    if (err != hipSuccess)
        return fail(KDA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return KDA_OK;
}

// the backward (a.mode BWD_FULL or BWD_FROM_SAVED) or a training forward (BWD_FORWARD)
int chunk_bwd_impl(const kda::ChunkBwdArgs& a0, const float* g, int chunk_size) {
    kda::ChunkBwdArgs a = a0;
    const bool fwd = a.mode == kda::BWD_FORWARD;
    int rc = check_common(a.q, a.k, a.v, g, a.beta, a.initial_state, a.cu_seqlens, a.N,
                          fwd ? a.fwd_o : a.dv, fwd ? a.fwd_final_state : a.dh0, a.B, a.T, a.H,
                          a.HV, a.K, a.V, a.qkv_dtype, a.beta_dtype);
    if (rc != KDA_OK) return rc;
    if (fwd) {
        if ((long long)a.B * a.T > 0 && !a.fwd_o) return fail(KDA_ERR_NULL, "o must be non-NULL");
    } else {
        if ((long long)a.B * a.T > 0 && (!a.dout || !a.dq || !a.dk || !a.dv || !a.dg || !a.dbeta))
            return fail(KDA_ERR_NULL, "do, dq, dk, dv, dg and dbeta must be non-NULL");
        if (!aligned16(a.dht) || !aligned16(a.dout) || !aligned16(a.dq) || !aligned16(a.dk) ||
            !aligned16(a.dg) || !aligned16(a.dbeta))
            return fail(KDA_ERR_SHAPE, "dht, do, dq, dk, dg and dbeta must be 16-byte aligned");
    }
    if (chunk_size != 64)
        return fail(KDA_ERR_UNSUPPORTED, "chunk_size must be 64, got %d", chunk_size);
    if (a.K != 64 && a.K != 128)
        return fail(KDA_ERR_UNSUPPORTED, "K must be 64 or 128, got %d", a.K);
    if (a.V != 64 && a.V != 128)
        return fail(KDA_ERR_UNSUPPORTED, "V must be 64 or 128, got %d", a.V);
    if (a.cu_seqlens && (long long)a.T / 64 + a.N > 0x7fffffffLL / a.HV)
        return fail(KDA_ERR_SHAPE, "too many chunks");
    kda::ChunkBwdLayout L;
    kda::chunk_bwd_layout(a.B, a.T, a.HV, a.K, a.V, a.N, a.cu_seqlens != nullptr, a.qkv_dtype, &L);
    if (a.N == 0) return KDA_OK;
    if (!a.workspace)
        return fail(KDA_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", L.total);
    if (a.workspace_bytes < L.total)
        return fail(KDA_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", a.workspace_bytes, L.total);
    if ((reinterpret_cast<uintptr_t>(a.workspace) & 255) != 0)
        return fail(KDA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    a.g = g;
    a.scale = a.scale == 0.0f ? 1.0f / sqrtf((float)a.K) : a.scale;
    hipError_t err = kda::launch_chunk_bwd(a, L);
    if (err != hipSuccess)
        return fail(KDA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return KDA_OK;
}

}  // namespace

namespace kda {
int set_error(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return code;
}
}  // namespace kda

extern "C" {

size_t kda_chunk_bwd_ex_workspace_bytes(int B, int T, int H, int HV, int K, int V, int N,
                                        int packed, int qkv_dtype) {
    if (B < 0 || T < 0 || H <= 0 || HV <= 0 || N < 0 || (K != 64 && K != 128) ||
        (V != 64 && V != 128) || (qkv_dtype != KDA_BF16 && qkv_dtype != KDA_F32))
        return 0;
    kda::ChunkBwdExLayout L;
    if (!kda::chunk_bwd_ex_layout(B, T, H, HV, K, V, packed ? N : B, packed != 0, qkv_dtype, &L)) return 0;
    return L.total;
}

}  // extern "C"

namespace {

// kda_chunk_bwd_ex (mode BWD_FULL or BWD_FROM_SAVED) or its training forward (BWD_FORWARD:
// o and final_state are written, the gradient pointers are unused)
int chunk_bwd_ex_impl(int mode, const void* q, const void* k, const void* v, const void* g, int gate,
                      const float* A_log, const float* dt_bias, int has_lower_bound,
                      float lower_bound, const void* beta, int preprocess,
                      const float* initial_state, const int32_t* cu_seqlens, int N, void* o,
                      float* final_state, const void* dout, const float* dht, void* dq, void* dk,
                      void* dv, float* dg, void* dbeta, float* dh0, float* dA_log, float* ddt_bias,
                      int B, int T, int H, int HV, int K, int V, int qkv_dtype, int beta_dtype,
                      float scale, int chunk_size, void* workspace, size_t workspace_bytes,
                      int32_t* dev_status, hipStream_t stream) {
    clear_error();
    const bool fwd = mode == kda::BWD_FORWARD;
    int rc = check_common(q, k, v, static_cast<const float*>(g), beta, initial_state, cu_seqlens, N,
                          fwd ? o : dv, fwd ? final_state : dh0, B, T, H, HV, K, V, qkv_dtype, beta_dtype);
    if (rc != KDA_OK) return rc;
    kda::InputSpec in;
    const bool nonempty = (long long)B * T > 0;
    rc = make_input_spec(g, gate, A_log, dt_bias, has_lower_bound, lower_bound, preprocess, nonempty, &in);
    if (rc != KDA_OK) return rc;
    if (fwd) {
        if (nonempty && !o) return fail(KDA_ERR_NULL, "o must be non-NULL");
    } else {
        if (nonempty && (!dout || !dq || !dk || !dv || !dg || !dbeta))
            return fail(KDA_ERR_NULL, "do, dq, dk, dv, dg and dbeta must be non-NULL");
        if (gate != KDA_GATE_LOG2 && nonempty && !dA_log)
            return fail(KDA_ERR_NULL, "dA_log must be non-NULL with a raw gate");
        if (gate != KDA_GATE_LOG2 && dt_bias && nonempty && !ddt_bias)
            return fail(KDA_ERR_NULL, "ddt_bias must be non-NULL when dt_bias is given");
        if (!aligned16(dht) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
            !aligned16(dg) || !aligned16(dbeta) || !aligned16(dA_log) || !aligned16(ddt_bias))
            return fail(KDA_ERR_SHAPE, "dht, do, dq, dk, dg, dbeta, dA_log and ddt_bias must be 16-byte aligned");
    }
    if (chunk_size != 64)
        return fail(KDA_ERR_UNSUPPORTED, "chunk_size must be 64, got %d", chunk_size);
    if (K != 64 && K != 128)
        return fail(KDA_ERR_UNSUPPORTED, "K must be 64 or 128, got %d", K);
    if (V != 64 && V != 128)
        return fail(KDA_ERR_UNSUPPORTED, "V must be 64 or 128, got %d", V);
    if (cu_seqlens && (long long)T / 64 + N > 0x7fffffffLL / HV)
        return fail(KDA_ERR_SHAPE, "too many chunks");
    kda::ChunkBwdExLayout L;
    kda::chunk_bwd_ex_layout(B, T, H, HV, K, V, N, cu_seqlens != nullptr, qkv_dtype, &L);
    if (N == 0) return KDA_OK;
    if (!workspace)
        return fail(KDA_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", L.total);
    if (workspace_bytes < L.total)
        return fail(KDA_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes, L.total);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
        return fail(KDA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    kda::ChunkBwdExArgs x;
    kda::ChunkBwdArgs& a = x.core;
    a.q = q; a.k = k; a.v = v; a.g = static_cast<const float*>(g); a.beta = beta;
    a.initial_state = initial_state; a.cu_seqlens = cu_seqlens;
    a.dout = dout; a.dht = dht;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.dh0 = dh0;
    a.N = N; a.B = B; a.T = T; a.H = H; a.HV = HV; a.K = K; a.V = V;
    a.qkv_dtype = qkv_dtype; a.beta_dtype = beta_dtype;
    a.scale = scale == 0.0f ? 1.0f / sqrtf((float)K) : scale;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    a.dev_status = dev_status; a.stream = stream;
    a.mode = mode;
    a.fwd_o = o;
    a.fwd_final_state = final_state;
    x.g = g;
    x.gate_bf16 = gate == KDA_GATE_RAW_BF16 ? 1 : 0;
    x.in = in;
    x.dA_log = dA_log;
    x.ddt_bias = ddt_bias;
    hipError_t err = kda::launch_chunk_bwd_ex(x, L);
    if (err != hipSuccess)
        return fail(KDA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return KDA_OK;
}

}  // namespace

extern "C" {

int kda_chunk_bwd_ex(const void* q, const void* k, const void* v, const void* g, int gate,
                     const float* A_log, const float* dt_bias, int has_lower_bound,
                     float lower_bound, const void* beta, int preprocess,
                     const float* initial_state, const int32_t* cu_seqlens, int N,
                     const void* dout, const float* dht, void* dq, void* dk, void* dv, float* dg,
                     void* dbeta, float* dh0, float* dA_log, float* ddt_bias, int B, int T,
                     int H, int HV, int K, int V, int qkv_dtype, int beta_dtype, float scale,
                     int chunk_size, void* workspace, size_t workspace_bytes,
                     int32_t* dev_status, hipStream_t stream) {
    return chunk_bwd_ex_impl(kda::BWD_FULL, q, k, v, g, gate, A_log, dt_bias, has_lower_bound,
                             lower_bound, beta, preprocess, initial_state, cu_seqlens, N, nullptr,
                             nullptr, dout, dht, dq, dk, dv, dg, dbeta, dh0, dA_log, ddt_bias, B, T,
                             H, HV, K, V, qkv_dtype, beta_dtype, scale, chunk_size, workspace,
                             workspace_bytes, dev_status, stream);
}

int kda_chunk_bwd_ex_saved(const void* q, const void* k, const void* v, const void* g, int gate,
                           const float* A_log, const float* dt_bias, int has_lower_bound,
                           float lower_bound, const void* beta, int preprocess,
                           const float* initial_state, const int32_t* cu_seqlens, int N,
                           const void* dout, const float* dht, void* dq, void* dk, void* dv, float* dg,
                           void* dbeta, float* dh0, float* dA_log, float* ddt_bias, int B, int T,
                           int H, int HV, int K, int V, int qkv_dtype, int beta_dtype, float scale,
                           int chunk_size, void* workspace, size_t workspace_bytes,
                           int32_t* dev_status, hipStream_t stream) {
    return chunk_bwd_ex_impl(kda::BWD_FROM_SAVED, q, k, v, g, gate, A_log, dt_bias, has_lower_bound,
                             lower_bound, beta, preprocess, initial_state, cu_seqlens, N, nullptr,
                             nullptr, dout, dht, dq, dk, dv, dg, dbeta, dh0, dA_log, ddt_bias, B, T,
                             H, HV, K, V, qkv_dtype, beta_dtype, scale, chunk_size, workspace,
                             workspace_bytes, dev_status, stream);
}

int kda_chunk_fwd_ex_train(const void* q, const void* k, const void* v, const void* g, int gate,
                           const float* A_log, const float* dt_bias, int has_lower_bound,
                           float lower_bound, const void* beta, int preprocess,
                           const float* initial_state, const int32_t* cu_seqlens, int N, void* o,
                           float* final_state, int B, int T, int H, int HV, int K, int V,
                           int qkv_dtype, int beta_dtype, float scale, int chunk_size,
                           void* workspace, size_t workspace_bytes, int32_t* dev_status,
                           hipStream_t stream) {
    return chunk_bwd_ex_impl(kda::BWD_FORWARD, q, k, v, g, gate, A_log, dt_bias, has_lower_bound,
                             lower_bound, beta, preprocess, initial_state, cu_seqlens, N, o,
                             final_state, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                             nullptr, nullptr, nullptr, nullptr, B, T, H, HV, K, V, qkv_dtype,
                             beta_dtype, scale, chunk_size, workspace, workspace_bytes, dev_status,
                             stream);
}

const char* kda_last_error(void) { return g_last_error; }

size_t kda_chunk_bwd_workspace_bytes(int B, int T, int H, int HV, int K, int V, int N,
                                     int packed, int qkv_dtype) {
    if (B < 0 || T < 0 || H <= 0 || HV <= 0 || N < 0 || (K != 64 && K != 128) ||
        (V != 64 && V != 128) || (qkv_dtype != KDA_BF16 && qkv_dtype != KDA_F32))
        return 0;
    kda::ChunkBwdLayout L;
    if (!kda::chunk_bwd_layout(B, T, HV, K, V, packed ? N : B, packed != 0, qkv_dtype, &L)) return 0;
    return L.total;
}

int kda_chunk_bwd(const void* q, const void* k, const void* v, const float* g, const void* beta,
                  const float* initial_state, const int32_t* cu_seqlens, int N, const void* dout,
                  const float* dht, void* dq, void* dk, void* dv, float* dg, void* dbeta,
                  float* dh0, int B, int T, int H, int HV, int K, int V, int qkv_dtype,
                  int beta_dtype, float scale, int chunk_size, void* workspace,
                  size_t workspace_bytes, int32_t* dev_status, hipStream_t stream) {
    clear_error();
    kda::ChunkBwdArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.initial_state = initial_state; a.cu_seqlens = cu_seqlens;
    a.dout = dout; a.dht = dht;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.dh0 = dh0;
    a.N = N; a.B = B; a.T = T; a.H = H; a.HV = HV; a.K = K; a.V = V;
    a.qkv_dtype = qkv_dtype; a.beta_dtype = beta_dtype; a.scale = scale;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    a.dev_status = dev_status; a.stream = stream;
    return chunk_bwd_impl(a, g, chunk_size);
}

int kda_chunk_fwd_train(const void* q, const void* k, const void* v, const float* g,
                        const void* beta, const float* initial_state, const int32_t* cu_seqlens,
                        int N, void* o, float* final_state, int B, int T, int H, int HV, int K,
                        int V, int qkv_dtype, int beta_dtype, float scale, int chunk_size,
                        void* workspace, size_t workspace_bytes, int32_t* dev_status,
                        hipStream_t stream) {
    clear_error();
    kda::ChunkBwdArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.initial_state = initial_state; a.cu_seqlens = cu_seqlens;
    a.N = N; a.B = B; a.T = T; a.H = H; a.HV = HV; a.K = K; a.V = V;
    a.qkv_dtype = qkv_dtype; a.beta_dtype = beta_dtype; a.scale = scale;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    a.dev_status = dev_status; a.stream = stream;
    a.mode = kda::BWD_FORWARD;
    a.fwd_o = o;
    a.fwd_final_state = final_state;
    return chunk_bwd_impl(a, g, chunk_size);
}

int kda_chunk_bwd_saved(const void* q, const void* k, const void* v, const float* g, const void* beta,
                        const float* initial_state, const int32_t* cu_seqlens, int N, const void* dout,
                        const float* dht, void* dq, void* dk, void* dv, float* dg, void* dbeta,
                        float* dh0, int B, int T, int H, int HV, int K, int V, int qkv_dtype,
                        int beta_dtype, float scale, int chunk_size, void* workspace,
                        size_t workspace_bytes, int32_t* dev_status, hipStream_t stream) {
    clear_error();
    kda::ChunkBwdArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.initial_state = initial_state; a.cu_seqlens = cu_seqlens;
    a.dout = dout; a.dht = dht;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.dh0 = dh0;
    a.N = N; a.B = B; a.T = T; a.H = H; a.HV = HV; a.K = K; a.V = V;
    a.qkv_dtype = qkv_dtype; a.beta_dtype = beta_dtype; a.scale = scale;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    a.dev_status = dev_status; a.stream = stream;
    a.mode = kda::BWD_FROM_SAVED;
    return chunk_bwd_impl(a, g, chunk_size);
}

int kda_abi_version(void) { return KDA_ABI_VERSION; }

size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int HV, int K, int V, int N,
                                     int packed, int qkv_dtype) {
    if (B < 0 || T < 0 || H <= 0 || HV <= 0 || N < 0 || (K != 64 && K != 128) ||
        (V != 64 && V != 128) || (qkv_dtype != KDA_BF16 && qkv_dtype != KDA_F32))
        return 0;
    kda::ChunkLayout L;
    if (!kda::chunk_layout(B, T, HV, K, V, packed ? N : B, packed != 0, qkv_dtype, &L)) return 0;
    return L.total;
}

int kda_chunk_fwd_ex(const void* q, const void* k, const void* v, const void* g, int gate,
                     const float* A_log, const float* dt_bias, int has_lower_bound,
                     float lower_bound, const void* beta, int preprocess,
                     const float* initial_state, const int32_t* cu_seqlens, int N, void* o,
                     float* final_state, int B, int T, int H, int HV, int K, int V,
                     int qkv_dtype, int beta_dtype, float scale, int chunk_size,
                     void* workspace, size_t workspace_bytes, int32_t* dev_status,
                     hipStream_t stream, hipEvent_t* events) {
    clear_error();
    return chunk_impl(q, k, v, g, gate, A_log, dt_bias, has_lower_bound, lower_bound, beta,
                      preprocess, initial_state, cu_seqlens, N, o, final_state, B, T, H, HV, K,
                      V, qkv_dtype, beta_dtype, scale, chunk_size, workspace, workspace_bytes,
                      dev_status, stream, events);
}

int kda_chunk_fwd(const void* q, const void* k, const void* v, const float* g, const void* beta,
                  const float* initial_state, const int32_t* cu_seqlens, int N, void* o,
                  float* final_state, int B, int T, int H, int HV, int K, int V, int qkv_dtype,
                  int beta_dtype, float scale, int chunk_size, void* workspace,
                  size_t workspace_bytes, int32_t* dev_status, hipStream_t stream) {
    clear_error();
    return chunk_impl(q, k, v, g, KDA_GATE_LOG2, nullptr, nullptr, 0, 0.0f, beta, 0,
                      initial_state, cu_seqlens, N, o, final_state, B, T, H, HV, K, V, qkv_dtype,
                      beta_dtype, scale, chunk_size, workspace, workspace_bytes, dev_status,
                      stream, nullptr);
}

int kda_chunk_fwd_timed(const void* q, const void* k, const void* v, const float* g,
                        const void* beta, const float* initial_state,
                        const int32_t* cu_seqlens, int N, void* o, float* final_state, int B,
                        int T, int H, int HV, int K, int V, int qkv_dtype, int beta_dtype,
                        float scale, int chunk_size, void* workspace, size_t workspace_bytes,
                        int32_t* dev_status, hipStream_t stream, hipEvent_t* events) {
    clear_error();
    return chunk_impl(q, k, v, g, KDA_GATE_LOG2, nullptr, nullptr, 0, 0.0f, beta, 0,
                      initial_state, cu_seqlens, N, o, final_state, B, T, H, HV, K, V, qkv_dtype,
                      beta_dtype, scale, chunk_size, workspace, workspace_bytes, dev_status,
                      stream, events);
}

int kda_chunk_fwd_gated(const void* q, const void* k, const void* v, const void* g_raw,
                        int g_dtype, const float* A_log, const float* dt_bias,
                        int has_lower_bound, float lower_bound, const void* beta,
                        const float* initial_state, const int32_t* cu_seqlens, int N, void* o,
                        float* final_state, int B, int T, int H, int HV, int K, int V,
                        int qkv_dtype, int beta_dtype, float scale, int chunk_size,
                        void* workspace, size_t workspace_bytes, int32_t* dev_status,
                        hipStream_t stream) {
    clear_error();
    if (g_dtype != KDA_BF16 && g_dtype != KDA_F32)
        return fail(KDA_ERR_DTYPE, "g_dtype must be KDA_BF16 (1) or KDA_F32 (0), got %d", g_dtype);
    return chunk_impl(q, k, v, g_raw, g_dtype == KDA_BF16 ? KDA_GATE_RAW_BF16 : KDA_GATE_RAW_F32,
                      A_log, dt_bias, has_lower_bound, lower_bound, beta, 0, initial_state,
                      cu_seqlens, N, o, final_state, B, T, H, HV, K, V, qkv_dtype, beta_dtype,
                      scale, chunk_size, workspace, workspace_bytes, dev_status, stream, nullptr);
}

int kda_recurrent_fwd(const void* q, const void* k, const void* v, const float* g,
                      const void* beta, const float* initial_state, const int32_t* cu_seqlens,
                      int N, void* o, float* final_state, int B, int T, int H, int HV, int K,
                      int V, int qkv_dtype, int beta_dtype, float scale, int32_t* dev_status,
                      hipStream_t stream) {
    clear_error();
    return recurrent_impl(q, k, v, g, KDA_GATE_LOG2, nullptr, nullptr, 0, 0.0f, beta, 0,
                          KDA_STATE_KV, initial_state, cu_seqlens, N, o, final_state, nullptr, B,
                          T, H, HV, K, V, qkv_dtype, beta_dtype, scale, dev_status, stream);
}

int kda_recurrent_fwd_ex(const void* q, const void* k, const void* v, const void* g, int gate,
                         const float* A_log, const float* dt_bias, int has_lower_bound,
                         float lower_bound, const void* beta, int preprocess, int state_layout,
                         const float* initial_state, const int32_t* cu_seqlens, int N,
                         void* o, float* final_state, float* intermediate_states, int B, int T,
                         int H, int HV, int K, int V, int qkv_dtype, int beta_dtype,
                         float scale, int32_t* dev_status, hipStream_t stream) {
    clear_error();
    return recurrent_impl(q, k, v, g, gate, A_log, dt_bias, has_lower_bound, lower_bound, beta,
                          preprocess, state_layout, initial_state, cu_seqlens, N, o, final_state,
                          intermediate_states, B, T, H, HV, K, V, qkv_dtype, beta_dtype, scale,
                          dev_status, stream);
}

}  // extern "C"
