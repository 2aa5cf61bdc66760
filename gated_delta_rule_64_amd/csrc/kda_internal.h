// Host-side launch descriptors shared by the C ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/kda.h"

namespace kda {

// Records `fmt` as the thread's kda_last_error() reason and returns `code` (the C ABI
// layer's error path, shared with the entry points that live in other files).
int set_error(int code, const char* fmt, ...);

// How the loads obtain the per-token log2 decay (the public kda_gate values).
enum GateMode {
    GATE_LOG2 = KDA_GATE_LOG2,           // g: fp32 per-token log2 decay, as given
    GATE_RAW_F32 = KDA_GATE_RAW_F32,     // g_raw fp32: -exp(A_log) softplus(g_raw + dt_bias) / ln 2
    GATE_RAW_BF16 = KDA_GATE_RAW_BF16    // g_raw bf16: same activation
};

// Gate source and input preprocessing, as the kernels take them.
struct InputSpec {
    int gate_mode;             // GateMode
    const void* g_raw;         // GATE_RAW_*: raw gate input
    const float* A_log;        // [HV]
    const float* dt_bias;      // [HV * K] or NULL
    int has_lower_bound;
    float lower_bound;
    int l2norm_q, l2norm_k;    // normalise q / k rows in the loads
    float beta_sig;            // 0: beta as given; else beta = beta_sig * sigmoid(beta)
};

struct RecurrentArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    InputSpec in;
    const void* beta;
    const float* initial_state;
    const int32_t* cu_seqlens;
    void* o;
    float* final_state;
    int N, B, T, H, HV, K, V;
    int qkv_dtype, beta_dtype;
    float scale;
    int32_t* dev_status;
    hipStream_t stream;
    int state_vk = 0;                // states [V][K] instead of [K][V]
    float* inter_states = nullptr;   // [B*T][HV][K*V]: the state after every token, or NULL
};

struct ChunkArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    InputSpec in;
    const void* beta;
    const float* initial_state;
    const int32_t* cu_seqlens;
    void* o;
    float* final_state;
    int N, B, T, H, HV, K, V;
    int qkv_dtype, beta_dtype;
    float scale;
    void* workspace;
    size_t workspace_bytes;
    int32_t* dev_status;
    hipStream_t stream;
    hipEvent_t* events;   // optional: 4 events recorded around the kernels
    // optional checkpoints for the backward (o may then be null): the state at each
    // chunk's start [HV][NCmax][K][V] and v' [HV][NCmax][64][V], fp32
    float* h_out = nullptr;
    float* vn_out = nullptr;
    // and from Stage 1+2: M (the key Gram with decay, strictly lower, before beta) and
    // T = (I + diag(beta) M)^-1, [HV][NCmax][64][64] fp32 each
    float* m_out = nullptr;
    float* t_out = nullptr;
};

// Workspace layout of the chunked forward (all offsets 256-byte aligned):
//   [sched]  int32 first_chunk[N], int32 end_chunk[N], int32 slot_ok[N],
//            int32 n_chunks[1], int2 chunk_table[NCmax] (first row, rows); written in
//            packed mode only (dense mode computes positions), present in both
//   [inter]  per (value head hv, chunk c), one record of the Stage 2 results, in order:
//              w      [64][K]       element type of the compute path (TW)
//              qg     [NS][64][K]   TW, scale folded in
//              kgT    [NS][K][64]   TW (rows = key channels)
//              Aqk    [NS][64][64]  TW, scale folded in, zero above the diagonal
//              u      [64][V]       fp32, accumulator order (AccTile)
//              eG     [K]           fp32, 2^(chunk's total log2 decay)
//            w, qg, kgT and Aqk are in matrix-core fragment order (FragTile). The
//            forward leaves Aqk's two all-zero fragments (rows 0-31, columns 32-63)
//            unwritten, as its scan never reads them; the backward's records hold them.
//            NS = 2 on the bf16 path (tile 1 holds x - bf16(x) rounded to bf16, so
//            hi + lo carries about 16 significant bits), NS = 1 on the fp32 path.
//            records are ordered hv-major: record(hv, c) = hv * NCmax + c.
//            The bf16 forward's own records, where its scan takes 32-column slices
//            (scan_slice_width: many chains), are compact:
//            qg, kgT and Aqk keep only their bf16 tile in place (NS = 1) and their
//            residuals follow as fp8 tiles with per-lane scale words (Lo8Tile):
//              qg lo [64][K], kgT lo [K][64], Aqk lo [64][64]   1 byte per value
//              qg, kgT, Aqk scale words                         [bands][64] uint32
//            then u and eG as above (hi + lo carries about 12 significant bits).
struct ChunkLayout {
    int NCmax;            // chunk slots (dense: B * ceil(T/64); packed: T/64 + N)
    size_t elem;          // bytes per intermediate element (2 bf16, 4 fp32)
    size_t off_w, off_u, off_qg, off_kgT, off_aqk, off_eg, rec_bytes;
    // residual tiles (the bf16 tile's offset + its size unless compact) and, in compact
    // records, the fp8 residuals' scale words
    size_t off_qg_lo, off_kgT_lo, off_aqk_lo, off_qg_sc, off_kgT_sc, off_aqk_sc;
    bool lo8;             // compact records (fp8 residuals)
    size_t sched_bytes;   // bytes of the chunk schedule
    size_t total;
};

// Column-slice width of the scan: 16 while chains are few (so that chains x V / 16
// blocks cover the chip), 32 on the bf16 path once chains x V / 32 reaches 512 blocks
// (the fp32 path keeps 16: its operand tiles take twice the LDS).
inline int scan_slice_width(long long chains, int V, bool bf16) {
    return bf16 && chains * (V / 32) >= 512 ? 32 : 16;
}

// ckpt_records: the layout of the backward's recompute (bf16 residual tiles); otherwise
// the forward's, compact where the scan takes 32-column slices (bf16 path, many chains)
bool chunk_layout(int B, int T, int HV, int K, int V, int N, bool packed, int qkv_dtype,
                  ChunkLayout* out, bool ckpt_records = false);

constexpr int BWD_FULL = 0, BWD_FORWARD = 1, BWD_FROM_SAVED = 2;

// The chunked backward: forward inputs, the output gradient and the gradients out.
struct ChunkBwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const void* beta;
    const float* initial_state;
    const int32_t* cu_seqlens;
    const void* dout;          // [B, T, HV, V], q's dtype
    const float* dht;          // [N, HV, K, V] or NULL (zeros)
    void* dq;                  // [B, T, H, K], q's dtype
    void* dk;
    void* dv;                  // [B, T, HV, V]
    float* dg;                 // [B, T, HV, K]
    void* dbeta;               // [B, T, HV], beta's dtype
    float* dh0;                // [N, HV, K, V] or NULL
    int N, B, T, H, HV, K, V;
    int qkv_dtype, beta_dtype;
    float scale;
    void* workspace;
    size_t workspace_bytes;
    int32_t* dev_status;
    hipStream_t stream;
    bool skip_reduce = false;   // leave dq, dk per value head (fp32) in the workspace
    // BWD_FULL: the backward, the forward recomputed first into the workspace;
    // BWD_FORWARD: only that forward, writing o (fwd_o) and the final state
    // (fwd_final_state, or NULL) as well: a training forward whose workspace then holds
    // everything the backward recomputes; BWD_FROM_SAVED: the backward from such a
    // workspace (same inputs), without the recompute
    int mode = 0;
    void* fwd_o = nullptr;
    float* fwd_final_state = nullptr;
    // fused input options of the forward being differentiated (g unused for a raw gate);
    // the gradients then are with respect to the transformed inputs (q, k normalised,
    // the log2 gate, the activated beta), the last one written fp32 when dbeta_f32
    InputSpec in{GATE_LOG2, nullptr, nullptr, nullptr, 0, 0.f, 0, 0, 0.f};
    bool dbeta_f32 = false;
};

// Backward workspace: the forward's (schedule + records) first, then per (value head,
// chunk) fp32 checkpoints and intermediates, then per-value-head dq, dk (all offsets
// 256-byte aligned):
//   h [K][V] state at the chunk start, vn [64][V] v', mt (M [64][64] and T [64][64] of
//   Stage 2), dh [K][V] gradient at the chunk
//   end, dvn [64][V] dv', sops (the reverse scan's operands: kg, w^T, Aqk^T do, qg^T do),
//   gs (dqg, dw, dkg [64][K], dAqk [64][64], dG [K]),
//   wy (dkd [64][K], dM [64][64]); dq, dk [B*T][HV][K].
struct ChunkBwdLayout {
    ChunkLayout fwd;
    size_t off_h, off_vn, off_mt, off_dh, off_dvn, off_sops, off_gs, off_wy, off_dq, off_dk;
    size_t total;
};

bool chunk_bwd_layout(int B, int T, int HV, int K, int V, int N, bool packed, int qkv_dtype,
                      ChunkBwdLayout* out);
hipError_t launch_chunk_bwd(const ChunkBwdArgs& a, const ChunkBwdLayout& L);

// The backward with the fused input options: `core` holds the raw inputs (g unused when
// the gate is raw; then g below is the raw gate) and the final gradient outputs.
struct ChunkBwdExArgs {
    ChunkBwdArgs core;
    const void* g;          // log2 decay (fp32) or the raw gate input
    int gate_bf16;          // raw gate stored as bf16
    InputSpec in;
    float* dA_log;          // [HV] (raw gate)
    float* ddt_bias;        // [HV * K] or NULL
};

// the core backward's workspace, then the fp32 gradients of the log2 gate and of the
// activated beta, and the per-chunk partial sums of the gate parameters' gradients
struct ChunkBwdExLayout {
    ChunkBwdLayout core;
    size_t off_dg2, off_dba, off_part;
    size_t total;
};

bool chunk_bwd_ex_layout(int B, int T, int H, int HV, int K, int V, int N, bool packed, int qkv_dtype,
                         ChunkBwdExLayout* out);
hipError_t launch_chunk_bwd_ex(const ChunkBwdExArgs& x, const ChunkBwdExLayout& L);

hipError_t launch_recurrent(const RecurrentArgs& a);
hipError_t launch_chunk(const ChunkArgs& a, const ChunkLayout& L);

}  // namespace kda
