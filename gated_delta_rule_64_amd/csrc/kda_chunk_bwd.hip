// Chunked KDA backward for gfx950: the gradients of the chunked forward with respect to
// q, k, v, the per-token log2 decay g, beta and the initial state.
//
// The method is the backward of "kernel-fun 0.2.0.dev1 sdist", ALGORITHM.md, section
// Backward: the forward's Stage 1+2 is recomputed (the forward's own kernel writes the
// per-chunk records), the forward scan runs again and checkpoints the state at every
// chunk start and v' (its "re-scan"), a reverse scan carries the state gradient and
// gives dv' per chunk (its "dhu" stage), and per-chunk kernels turn those into the
// input gradients: the products with the state checkpoints (its wy_dqkg h/dh
// consumers), the backward of the WY inverse, and the intra-chunk pair terms with a
// reverse cumsum of the gate gradient folded in (its intra stage and dg cumsum). GVA
// gradients of q and k are summed over each q/k head's value heads (by the bf16 pair
// kernel itself, else by a last kernel).
//
// Per chunk (rows r, s of the chunk, Gamma the chunk-local cumsum of g, G its last
// row, S the state at the chunk start, dS the gradient at the chunk end, do the output
// gradient), with the forward's qg = scale q 2^Gamma, kd = k 2^Gamma,
// kg = k 2^(G - Gamma), Aqk[r,s] = scale sum_d q_r k_s 2^(Gamma_r - Gamma_s) (s <= r),
// M[r,s] = sum_d k_r k_s 2^(Gamma_r - Gamma_s) (s < r), T = (I + diag(beta) M)^-1,
// u = T diag(beta) v, w = T diag(beta) kd, v' = u - w S:
//   dv'  = Aqk^T do + kg dS                 dS_prev = 2^G dS + qg^T do - w^T dv'
//   dqg  = do S^T   dw = -dv' S^T   dkg = v' dS^T   dAqk = do v'^T (s <= r)
//   dG  += ln2 2^G sum_v dS S
//   Gu = T^T dv', Gw = T^T dw: dv = beta Gu, dkd = beta Gw,
//   dbeta = rowsum(Gu v) + rowsum(Gw kd) + rowsum(dL M),
//   dT = dv' (beta v)^T + dw (beta kd)^T, dL = -(T^T dT T^T) strictly lower, dM = beta dL
//   and the pair terms of Aqk and M with one one-sided 2^(Gamma_r - Gamma_s) <= 1 each.
// All of it in fp32 arithmetic. With bf16 inputs the dense products of the reverse scan
// (P1 and P2 included), the state, WY and pair stages run on the bf16 matrix cores, each
// fp32 operand carried as a hi + lo bf16 pair (three products per step; two where one
// operand is exact in bf16), and the prep only lays their operands out; the fp32-input
// path uses the fp32 matrix cores.
#include <atomic>
#include <type_traits>

#include "kda_chunk_common.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int BT = 256;                       // threads per block
constexpr float LN2F = 0.69314718055994531f;

// fp32 matrix-core tile product over contraction [0, nk): C[16x16] += sum_k A(i, k) B(j, k).
// Lane (lq, lr) supplies A(lr, k + lq) and B(lr, k + lq) and holds C[4 lq + r][lr] in
// register r (v_mfma_f32_16x16x4_f32).
template <class FA, class FB>
__device__ __forceinline__ f32x4 mma_f32(f32x4 acc, const FA& a, const FB& b, int nk, int lane) {
    const int r = lane & 15, kq = lane >> 4;
    for (int k = 0; k < nk; k += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a(r, k + kq), b(r, k + kq), acc, 0, 0, 0);
    return acc;
}

// Sum over the 16 lanes of a DPP row (the lanes that hold one row of a tile product).
__device__ __forceinline__ float sum16(float x) {
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 4, 64);
    x += __shfl_xor(x, 8, 64);
    return x;
}

// An R x KC record tile (fragment order; on the bf16 path the rounding residual tile
// follows at + R*KC when `split`) copied into fp32 LDS: dst[row * ld + col].
template <typename TW, int R, int KC>
__device__ __forceinline__ void stage_record(const TW* t, bool split, float* dst, int ld, int tid) {
    typedef Mma<TW> M;
    constexpr int NS = KC / M::KS;
    static_assert((R * KC) % (8 * BT) == 0, "whole 8-element groups per thread");
    // 8 consecutive elements (one 16-byte bf16 or two fp32 vectors) per thread and step
#pragma unroll 4
    for (int q = tid; q < R * KC / 8; q += BT) {
        const int e0 = 8 * q;
        float v[8];
        if constexpr (sizeof(TW) == 2) {
            const bf16x8 h = *reinterpret_cast<const bf16x8*>(t + e0);
            bf16x8 l8 = {};
            if (split) l8 = *reinterpret_cast<const bf16x8*>(t + e0 + R * KC);
#pragma unroll
            for (int x = 0; x < 8; ++x) v[x] = (float)h[x] + (float)l8[x];
        } else {
            const f32x4 a = *reinterpret_cast<const f32x4*>(t + e0);
            const f32x4 b = *reinterpret_cast<const f32x4*>(t + e0 + 4);
#pragma unroll
            for (int x = 0; x < 4; ++x) { v[x] = a[x]; v[4 + x] = b[x]; }
        }
#pragma unroll
        for (int x = 0; x < 8; ++x) {
            const int e = e0 + x;
            const int xi = e % M::KPL;
            const int l = (e / M::KPL) % 64;
            const int blk = e / (M::KPL * 64);
            const int row = 16 * (blk / NS) + (l & 15);
            const int col = (blk % NS) * M::KS + (l >> 4) * M::KPL + xi;
            dst[row * ld + col] = v[x];
        }
    }
}

// Rows [0, R) x columns [0, W) of a row-major fp32 array (row stride `gstride` floats)
// into LDS dst[r * ld + c]; 16-byte loads, several in flight per thread.
template <int R, int W, int NTH = BT>
__device__ __forceinline__ void stage_f32(const float* src, size_t gstride, float* dst, int ld, int tid) {
    constexpr int W4 = W / 4;
#pragma unroll 4
    for (int q = tid; q < R * W4; q += NTH) {
        const int r = q / W4, c4 = 4 * (q % W4);
        const f32x4 x = *reinterpret_cast<const f32x4*>(src + (size_t)r * gstride + c4);
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[r * ld + c4 + e] = x[e];
    }
}

// Rows of an input tensor as fp32 into LDS: row r at src + r * rstride (W contiguous
// elements of T), zeros from row `len` on.
template <int R, int W, typename T, int NTH = BT>
__device__ __forceinline__ void stage_rows(const T* src, size_t rstride, int len, float* dst, int ld, int tid) {
    constexpr int W4 = W / 4;
    // rows past len read row len - 1 (in bounds) and are stored as zeros: no branch
    // around the loads, so the unrolled loop issues them all before its first store
    if (len <= 0) {   // (block-uniform) no row to read
        for (int q = tid; q < R * W4; q += NTH)
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[(q / W4) * ld + 4 * (q % W4) + e] = 0.f;
        return;
    }
    const int last = len - 1;
#pragma unroll 4
    for (int q = tid; q < R * W4; q += NTH) {
        const int r = q / W4, c4 = 4 * (q % W4);
        const int rl = r < len ? r : last;
        float x[4];
        if constexpr (sizeof(T) == 2) {
            const bf16x4 h = *reinterpret_cast<const bf16x4*>(src + (size_t)rl * rstride + c4);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = r < len ? (float)h[e] : 0.f;
        } else {
            const f32x4 f = *reinterpret_cast<const f32x4*>(src + (size_t)rl * rstride + c4);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = r < len ? f[e] : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[r * ld + c4 + e] = x[e];
    }
}

// Rows of an input tensor (as stage_rows), in two steps: load() issues every load of
// the calling thread into registers, store() converts and writes them to LDS. Staging
// several tensors load-load-...-store-store keeps all their loads in flight together.
template <int R, int W, typename T, int NTH>
struct RowLoad {
    static constexpr int W4 = W / 4, N = R * W4 / NTH;
    static_assert(N * NTH == R * W4, "whole vectors per thread");
    typedef typename std::conditional<sizeof(T) == 2, bf16x4, f32x4>::type vec;
    vec x[N];
    __device__ __forceinline__ void load(const T* src, size_t rstride, int len, int tid) {
        const int last = len > 0 ? len - 1 : 0;   // rows past len re-read row len - 1
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int q = tid + NTH * i, r = q / W4, c4 = 4 * (q % W4);
            x[i] = len > 0 ? *reinterpret_cast<const vec*>(src + (size_t)(r < len ? r : last) * rstride + c4) : vec{};
        }
    }
    __device__ __forceinline__ void store(int len, float* dst, int ld, int tid) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int q = tid + NTH * i, r = q / W4, c4 = 4 * (q % W4);
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[r * ld + c4 + e] = r < len ? (float)x[i][e] : 0.f;
        }
    }
};

// A fp32 [R][W] tile (as stage_f32), in the same two steps.
template <int R, int W, int NTH>
struct TileLoad {
    static constexpr int W4 = W / 4, N = R * W4 / NTH;
    static_assert(N * NTH == R * W4, "whole vectors per thread");
    f32x4 x[N];
    __device__ __forceinline__ void load(const float* src, size_t gstride, int tid) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int q = tid + NTH * i;
            x[i] = *reinterpret_cast<const f32x4*>(src + (size_t)(q / W4) * gstride + 4 * (q % W4));
        }
    }
    __device__ __forceinline__ void store(float* dst, int ld, int tid) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int q = tid + NTH * i;
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[(q / W4) * ld + 4 * (q % W4) + e] = x[i][e];
        }
    }
};

struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const void* beta;
    const void* dout;
    const float* dht;
    void* dq;
    void* dk;
    void* dv;
    float* dg;
    void* dbeta;
    float* dh0;
    // schedule (packed mode) or dense positions
    const int32_t* nchunks;
    const int2* table;
    const int32_t* coff;
    const int32_t* cend;
    const int32_t* slot_ok;
    const int32_t* order;     // slots by descending chunk count (packed), or NULL
    int dense, NT, T, N, H, HV, NCmax;
    float scale;
    // forward records
    const char* rec;
    size_t rec_bytes, off_w, off_u, off_qg, off_kgT, off_aqk, off_eg;
    // checkpoints and intermediates, per (value head, chunk): index hv * NCmax + c
    const float* h;      // [K][V] state at the chunk start
    const float* vn;     // [64][V] v'
    const float* mt;     // M [64][64] per item, then T [64][64] per item (Stage 2)
    float* dh;           // [K][V] gradient at the chunk end
    float* dvn;          // [64][V] dv'
    float* sops;         // operands of the reverse scan (ScanOps)
    float* gs;           // dqg, dw, dkg [64][K] each, dAqk [64][64], dG [K]
    float* wy;           // dkd [64][K], dM [64][64]
    float* dq_hv;        // [B*T][HV][K]
    float* dk_hv;
    InputSpec in;        // fused options of the forward (applied to the staged inputs)
    int dbeta_f32;       // dbeta written as fp32
    int pair_gva;        // the bf16 pair kernel sums dq, dk over each q/k head's value heads itself
};

// The fused options applied to staged rows in LDS (64 rows of K, rows >= len zero):
// the L2 normalisation of each row, in fp32.
// Thread t in [0, 64) takes row t.
template <int K>
__device__ __forceinline__ void l2norm_rows_lds(float* X, int ld, int t) {
    if (t >= 0 && t < C) {
        // two passes over LDS, neither fully unrolled: fully unrolled, the pair kept the
        // whole row in registers between them (and spilled)
        float ss = 0.f;
#pragma unroll 8
        for (int d = 0; d < K; ++d) ss = fmaf(X[t * ld + d], X[t * ld + d], ss);
        const float rn = l2norm_rstd(ss);
#pragma unroll 8
        for (int d = 0; d < K; ++d) X[t * ld + d] *= rn;
    }
}

// The raw gate input staged into X (rows < len) turned into the log2 decay.
template <int K, int NTH>
__device__ __forceinline__ void gate_rows_lds(float* X, int ld, int len, const InputSpec& in, int hv, int tid) {
    const float amp = -expf(in.A_log[hv]);
    const float lb2 = in.lower_bound * LOG2E;
    for (int e = tid; e < C * K; e += NTH) {
        const int r = e / K, d = e % K;
        if (r < len) {
            const float x = X[r * ld + d] + (in.dt_bias ? in.dt_bias[(size_t)hv * K + d] : 0.f);
            X[r * ld + d] = gate_log2_from_raw(x, amp, in.has_lower_bound, lb2);
        }
    }
}

// In-place cumulative sum down the C rows of a C x K fp32 tile in LDS (X[r * ld + d]):
// NTH threads, each a run of C / (NTH / K) rows of one column; the runs' totals go
// through `tot` (NTH floats) and each run adds those above it. The caller's writes of X
// must be visible (a barrier) before the call; one barrier inside, none at the end.
template <int K, int NTH>
__device__ __forceinline__ void cumsum_rows_lds(float* X, int ld, float* tot, int tid) {
    constexpr int NS = NTH / K, RL = C / NS;
    static_assert(NTH % K == 0 && C % NS == 0, "runs must tile the chunk");
    const int d = tid % K, s = tid / K;
    float x[RL];
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < RL; ++i) x[i] = X[(s * RL + i) * ld + d];
#pragma unroll
    for (int i = 0; i < RL; ++i) { acc += x[i]; x[i] = acc; }
    tot[s * K + d] = acc;
    __syncthreads();
    float off = 0.f;
    for (int j = 0; j < s; ++j) off += tot[j * K + d];
#pragma unroll
    for (int i = 0; i < RL; ++i) X[(s * RL + i) * ld + d] = x[i] + off;
}

// rows of g (log2 decay, or the raw gate input by the options) into LDS
template <int K, int NTH>
__device__ __forceinline__ void stage_gate(const BwdParams& p, int2 pos, int hv, float* X, int ld, int tid) {
    const size_t o = ((size_t)pos.x * p.HV + hv) * K, st = (size_t)p.HV * K;
    if (p.in.gate_mode == GATE_RAW_BF16)
        stage_rows<C, K, __bf16, NTH>(static_cast<const __bf16*>(p.in.g_raw) + o, st, pos.y, X, ld, tid);
    else if (p.in.gate_mode == GATE_RAW_F32)
        stage_rows<C, K, float, NTH>(static_cast<const float*>(p.in.g_raw) + o, st, pos.y, X, ld, tid);
    else
        stage_rows<C, K, float, NTH>(p.g + o, st, pos.y, X, ld, tid);
}

template <int K>
struct GsLayout {
    static constexpr int DQG = 0, DW = C * K, DKG = 2 * C * K, DA = 3 * C * K, DG = 3 * C * K + C * C;
    static constexpr int FLOATS = 3 * C * K + C * C + K;
};
template <int K>
struct WyLayout {
    static constexpr int DKD = 0, DM = C * K;
    static constexpr int FLOATS = C * K + C * C;
};

// Work item b of a per-chunk-head kernel (G = NCmax * HV items, dealt to the XCDs by
// xcd_remap): its chunk c and value head hv, and whether it exists (nch = the number of
// chunks: NCmax in dense mode, the packed schedule's count otherwise).
__device__ __forceinline__ bool bwd_item(const BwdParams& p, int b, int nch, int& c, int& hv) {
    const int item = xcd_remap(b, p.NCmax * p.HV);
    hv = item % p.HV;
    c = item / p.HV;
    return c < nch;
}

// the chunk this block handles, or false when it is past the packed schedule's end
__device__ __forceinline__ bool bwd_chunk(const BwdParams& p, int& c, int& hv, int2& pos) {
    const int G = p.NCmax * p.HV;
    const int item = xcd_remap(blockIdx.x, G);
    hv = item % p.HV;
    c = item / p.HV;
    if (!p.dense && c >= p.nchunks[0]) return false;
    pos = chunk_pos(p.dense, p.NT, p.T, p.table, c);
    return true;
}

// Accumulator order of a K x V fp32 tile (rows d, columns v): block (16-column tile,
// 16-row band), lane l = (v % 16) + 16 ((d % 16) / 4) holds rows d .. d+3 of column v as
// one f32x4 -- the layout of a 16x16 matrix-core result, loaded with one 16-byte access.
template <int K>
__device__ __forceinline__ int acc_kv(int v, int d) {
    return (((v >> 4) * (K / 16) + (d >> 4)) * 64 + (v & 15) + 16 * ((d & 15) >> 2)) * 4 + (d & 3);
}

// Per (value head, chunk) operands of the reverse scan, fp32 inputs: kg in fragment
// order as the A operand of kg dS ([64][K]), w^T in fragment order as the A operand of
// w^T dv' ([K][64]), P1 = Aqk^T do ([64][V], AccTile order) and P2 = qg^T do ([K][V],
// acc_kv order), all fp32. P1 and P2 do not depend on the state gradient, so they are
// formed in parallel before the scan.
template <int K, int V>
struct ScanOps {
    static constexpr int KG = 0, WT = C * K, P1 = 2 * C * K, P2 = 2 * C * K + C * V;
    static constexpr int FLOATS = 2 * C * K + C * V + K * V;
};
// The same slot for bf16 inputs, in bf16 elements, every tile in 16x16x32 fragment
// order: kg (hi, lo), w^T, then the operands of P1 and P2, which the reverse scan forms
// on the matrix cores as it goes (64 KB of bf16 operands per chunk-head instead of 96 KB
// of fp32 products): Aqk^T (rows s, contraction r; hi, lo), qg^T (rows d, contraction
// r; hi, lo) and do^T (rows v, contraction r).
template <int K, int V>
struct ScanOpsB {
    static constexpr int KG = 0, WT = 2 * C * K, AQT = 3 * C * K, QGT = 3 * C * K + 2 * C * C;
    static constexpr int DOT = 5 * C * K + 2 * C * C, ELEMS = 5 * C * K + 2 * C * C + V * C;
    static_assert(ELEMS * 2 <= ScanOps<K, V>::FLOATS * 4, "fits the per-chunk slot");
    static_assert(ELEMS * 2 % 128 == 0, "whole 128-byte lines");
};

// ------------------------------------------------------------------------------------
// prep for the reverse scan, per (chunk, value head): P1, P2 and the transposed
// operands, from the forward records and do.
// ------------------------------------------------------------------------------------
template <int K, int V, typename TW, typename TIn>
__global__ __launch_bounds__(BT, 1) void bwd_prep_kernel(BwdParams p) {
    constexpr int LA = C + 1, LK = K + 1, LV = V + 1;
    constexpr bool SPLIT = sizeof(TW) == 2;
    typedef ScanOps<K, V> SO;
    typedef FragTile<float, C, K> FKG;
    typedef FragTile<float, K, C> FWT;
    __shared__ float R0[C * LK];     // qg [r][d], then w [r][d]
    __shared__ float R1[K * LA];     // Aqk [r][s], then kg^T [d][s]
    __shared__ float doL[C * LV];
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int c, hv;
    int2 pos;
    if (!bwd_chunk(p, c, hv, pos)) return;
    const size_t ci = (size_t)hv * p.NCmax + c;
    const char* rec = p.rec + ci * p.rec_bytes;
    const TIn* dout = reinterpret_cast<const TIn*>(p.dout);
    float* ops = p.sops + ci * (size_t)SO::FLOATS;

    stage_record<TW, C, K>(reinterpret_cast<const TW*>(rec + p.off_qg), SPLIT, R0, LK, tid);
    stage_record<TW, C, C>(reinterpret_cast<const TW*>(rec + p.off_aqk), SPLIT, R1, LA, tid);
    stage_rows<C, V>(dout + ((size_t)pos.x * p.HV + hv) * V, (size_t)p.HV * V, pos.y, doL, LV, tid);
    __syncthreads();
    // P1[s][v] = sum_r Aqk[r][s] do[r][v]: wave w owns rows 16w ..
    for (int nt = 0; nt < V / 16; ++nt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma_f32(acc, [&](int i, int k) { return R1[k * LA + 16 * wave + i]; },
                      [&](int j, int k) { return doL[k * LV + 16 * nt + j]; }, C, lane);
        *reinterpret_cast<f32x4*>(ops + SO::P1 + AccTile::quad(16 * nt + lr, 16 * wave + 4 * lq)) = acc;
    }
    // P2[d][v] = sum_r qg[r][d] do[r][v]: wave w owns bands w, w + 4, ..
    for (int db = wave; db < K / 16; db += 4)
        for (int nt = 0; nt < V / 16; ++nt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma_f32(acc, [&](int i, int k) { return R0[k * LK + 16 * db + i]; },
                          [&](int j, int k) { return doL[k * LV + 16 * nt + j]; }, C, lane);
            *reinterpret_cast<f32x4*>(ops + SO::P2 + acc_kv<K>(16 * nt + lr, 16 * db + 4 * lq)) = acc;
        }
    __syncthreads();
    stage_record<TW, C, K>(reinterpret_cast<const TW*>(rec + p.off_w), false, R0, LK, tid);
    stage_record<TW, K, C>(reinterpret_cast<const TW*>(rec + p.off_kgT), SPLIT, R1, LA, tid);
    __syncthreads();
    // kg in fragment order (rows s, contraction d) and w^T (rows d, contraction r)
    for (int e = tid; e < C * K; e += BT) {
        const int l = e % 64, blk = e / 64;
        {
            const int row = 16 * (blk / FKG::NS) + (l & 15), col = 4 * (blk % FKG::NS) + (l >> 4);
            ops[SO::KG + e] = R1[col * LA + row];
        }
        {
            const int row = 16 * (blk / FWT::NS) + (l & 15), col = 4 * (blk % FWT::NS) + (l >> 4);
            ops[SO::WT + e] = R0[col * LK + row];
        }
    }
}

// ------------------------------------------------------------------------------------
// reverse scan: dS (the state gradient) walks each chain's chunks backwards:
//   dh_c = dS,  dv' = P1 + kg dS,  dS <- 2^G dS + P2 - w^T dv'
// One block per (chain, 16-column slice of V); wave w owns rows 16w.. of dv' and state
// bands w, w + 4. The kg / w^T fragments are loaded straight from memory (fragment
// order), two chunks ahead; dS^T and dv'^T are shared through LDS.
// ------------------------------------------------------------------------------------
template <int K, int V>
struct DscanFrags {
    static constexpr int NKS = K / 4, NJS = C / 4, NDT = K / 64;
    float kg[NKS];
    float wt[NDT][NJS];
    f32x4 p1;
    f32x4 p2[NDT];
    f32x4 e[NDT];
};

template <int K, int V>
__device__ __forceinline__ void load_dscan(DscanFrags<K, V>& F, const BwdParams& p, int hv, int c,
                                           int wave, int lane, int v0) {
    typedef ScanOps<K, V> SO;
    typedef FragTile<float, C, K> FKG;
    typedef FragTile<float, K, C> FWT;
    const int lr = lane & 15, lq = lane >> 4;
    const size_t ci = (size_t)hv * p.NCmax + c;
    const float* ops = p.sops + ci * (size_t)SO::FLOATS;
    const float* eg = reinterpret_cast<const float*>(p.rec + ci * p.rec_bytes + p.off_eg);
#pragma unroll
    for (int kk = 0; kk < DscanFrags<K, V>::NKS; ++kk) F.kg[kk] = ops[SO::KG + FKG::frag(wave, kk, lane)];
#pragma unroll
    for (int a = 0; a < DscanFrags<K, V>::NDT; ++a) {
#pragma unroll
        for (int jj = 0; jj < DscanFrags<K, V>::NJS; ++jj)
            F.wt[a][jj] = ops[SO::WT + FWT::frag(wave + 4 * a, jj, lane)];
        F.p2[a] = *reinterpret_cast<const f32x4*>(ops + SO::P2 + acc_kv<K>(v0 + lr, 16 * (wave + 4 * a) + 4 * lq));
        F.e[a] = *reinterpret_cast<const f32x4*>(eg + 16 * (wave + 4 * a) + 4 * lq);
    }
    F.p1 = *reinterpret_cast<const f32x4*>(ops + SO::P1 + AccTile::quad(v0 + lr, 16 * wave + 4 * lq));
}

template <int K, int V>
__global__ __launch_bounds__(BT, 1) void bwd_scan_kernel(BwdParams p) {
    constexpr int BV = 16, NVT = V / BV, LDK = K + 1, LDC = C + 1, NDT = K / 64;
    typedef DscanFrags<K, V> DF;
    __shared__ float dSt[BV * LDK];   // dS^T [v][d]
    __shared__ float dvt[BV * LDC];   // dv'^T [v][r]
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = p.N * p.HV * NVT;
    int vt, hv, n;
    scan_item(blockIdx.x, G, NVT, p.HV, p.dense ? nullptr : p.order, vt, hv, n);
    const int v0 = vt * BV;
    if (!p.dense && !p.slot_ok[n]) return;
    const int c0 = p.dense ? n * p.NT : p.coff[n];
    const int c1 = p.dense ? c0 + p.NT : p.cend[n];
    const size_t sbase = ((size_t)n * p.HV + hv) * (size_t)K * V;

    f32x4 dS[NDT];
#pragma unroll
    for (int a = 0; a < NDT; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d = 16 * (wave + 4 * a) + 4 * lq + r;
            dS[a][r] = p.dht ? p.dht[sbase + (size_t)d * V + v0 + lr] : 0.f;
            dSt[lr * LDK + d] = dS[a][r];
        }
    // two-chunk ring: F0 holds chunk c, F1 chunk c - 1; past the first chunk a buffer
    // re-reads chunk c0 (in bounds, never used)
    auto clampc = [&](int c) { return c >= c0 ? c : c0; };
    DF F0, F1;
    if (c0 < c1) {
        load_dscan<K, V>(F0, p, hv, c1 - 1, wave, lane, v0);
        load_dscan<K, V>(F1, p, hv, clampc(c1 - 2), wave, lane, v0);
    }
    __syncthreads();
    auto step = [&](DF& F, int c) {
        const size_t ci = (size_t)hv * p.NCmax + c;
        float* dhb = p.dh + ci * (size_t)K * V;
#pragma unroll
        for (int a = 0; a < NDT; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r) dhb[(size_t)(16 * (wave + 4 * a) + 4 * lq + r) * V + v0 + lr] = dS[a][r];
        // dv' = P1 + kg dS (rows 16 wave + 4 lq + r, column lr of the slice)
        f32x4 acc = F.p1;
#pragma unroll
        for (int kk = 0; kk < DF::NKS; ++kk)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(F.kg[kk], dSt[lr * LDK + 4 * kk + lq], acc, 0, 0, 0);
        float* dvb = p.dvn + ci * (size_t)C * V;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int s = 16 * wave + 4 * lq + r;
            dvt[lr * LDC + s] = acc[r];
            dvb[(size_t)s * V + v0 + lr] = acc[r];
        }
        __syncthreads();
        // dS <- 2^G dS + P2 - w^T dv'
#pragma unroll
        for (int a = 0; a < NDT; ++a) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jj = 0; jj < DF::NJS; ++jj)
                x = __builtin_amdgcn_mfma_f32_16x16x4f32(F.wt[a][jj], dvt[lr * LDC + 4 * jj + lq], x, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                dS[a][r] = fmaf(F.e[a][r], dS[a][r], F.p2[a][r] - x[r]);
                dSt[lr * LDK + 16 * (wave + 4 * a) + 4 * lq + r] = dS[a][r];
            }
        }
        __syncthreads();
    };
    const int nsteps = c1 - c0;
    int c = c1 - 1;
    for (int t = 0; t < nsteps / 2; ++t, c -= 2) {
        step(F0, c);
        load_dscan<K, V>(F0, p, hv, clampc(c - 2), wave, lane, v0);
        step(F1, c - 1);
        load_dscan<K, V>(F1, p, hv, clampc(c - 3), wave, lane, v0);
    }
    if (nsteps & 1) step(F0, c);
    if (p.dh0) {
#pragma unroll
        for (int a = 0; a < NDT; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                p.dh0[sbase + (size_t)(16 * (wave + 4 * a) + 4 * lq + r) * V + v0 + lr] = dS[a][r];
    }
}

// The reverse scan for bf16 inputs: kg (hi, lo) and w^T in bf16 fragment order from the
// bf16 prep, dS and dv' exchanged through LDS as hi + lo bf16 rows, products on
// v_mfma_f32_16x16x32_bf16 (hi*hi + lo*hi + hi*lo; w^T is exact, two products). The
// chain per chunk is 4 + 2 dependent steps per wave instead of 32 + 16 fp32 ones. P1 and
// P2 of the slice's columns are formed from the prep's Aqk^T, qg^T (hi, lo) and do^T
// fragments (hi then lo per contraction step, in one accumulator): P1 as the start of
// the dv' accumulation, P2 after the v' barrier, where it overlaps the dv'^T reads.
constexpr int BWD_L2_AHEAD = 4;   // chunks beyond the current one the reverse scan's L2 prefetch touches

template <int K, int V>
struct DscanFragsB {
    static constexpr int NKS = K / 32, NJS = C / 32, NDT = K / 64;
    bf16x8 kg[2][NKS];        // hi, lo
    bf16x8 wt[NDT][NJS];
    f32x4 e[NDT];
};
template <int K, int V>
struct DscanPB {
    static constexpr int NJS = C / 32, NDT = K / 64;
    bf16x8 aq[2][NJS];        // Aqk^T band `wave`: hi, lo
    bf16x8 dt[NJS];           // do^T band of the slice
    bf16x8 qt[NDT][2][NJS];   // qg^T bands wave + 4a: hi, lo
};

// The operands of chunk c in two groups, two chunks ahead: those of the dv' products
// (kg) and those of the dS update (w^T, 2^G); the scan issues each group right after the
// products that last read it, so the loads queue up behind work in flight instead of in
// one burst. The operands of P1 and P2 (Aqk^T, do^T, qg^T) are held one chunk ahead
// only (their loads hit the lines the L2 prefetch touched), which keeps the scan within
// its registers.
template <int K, int V>
__device__ __forceinline__ void load_dscan_b_kg(DscanFragsB<K, V>& F, const BwdParams& p, int hv, int c,
                                                int wave, int lane, int v0) {
    typedef ScanOps<K, V> SO;
    typedef ScanOpsB<K, V> SB;
    typedef FragTile<__bf16, C, K> FKG;
    typedef DscanFragsB<K, V> DF;
    const size_t ci = (size_t)hv * p.NCmax + c;
    const __bf16* ops = reinterpret_cast<const __bf16*>(p.sops + ci * (size_t)SO::FLOATS);
#pragma unroll
    for (int kk = 0; kk < DF::NKS; ++kk) {
        F.kg[0][kk] = *reinterpret_cast<const bf16x8*>(ops + SB::KG + FKG::frag(wave, kk, lane));
        F.kg[1][kk] = *reinterpret_cast<const bf16x8*>(ops + SB::KG + C * K + FKG::frag(wave, kk, lane));
    }
}
template <int K, int V>
__device__ __forceinline__ void load_dscan_b_p(DscanPB<K, V>& F, const BwdParams& p, int hv, int c,
                                               int wave, int lane, int v0) {
    typedef ScanOps<K, V> SO;
    typedef ScanOpsB<K, V> SB;
    typedef FragTile<__bf16, C, C> FAT;
    typedef FragTile<__bf16, V, C> FDT;
    typedef FragTile<__bf16, K, C> FQT;
    typedef DscanPB<K, V> PF;
    const size_t ci = (size_t)hv * p.NCmax + c;
    const __bf16* ops = reinterpret_cast<const __bf16*>(p.sops + ci * (size_t)SO::FLOATS);
#pragma unroll
    for (int jj = 0; jj < PF::NJS; ++jj) {
        F.dt[jj] = *reinterpret_cast<const bf16x8*>(ops + SB::DOT + FDT::frag(v0 / 16, jj, lane));
        F.aq[0][jj] = *reinterpret_cast<const bf16x8*>(ops + SB::AQT + FAT::frag(wave, jj, lane));
        F.aq[1][jj] = *reinterpret_cast<const bf16x8*>(ops + SB::AQT + C * C + FAT::frag(wave, jj, lane));
    }
#pragma unroll
    for (int a = 0; a < PF::NDT; ++a)
#pragma unroll
        for (int jj = 0; jj < PF::NJS; ++jj) {
            F.qt[a][0][jj] = *reinterpret_cast<const bf16x8*>(ops + SB::QGT + FQT::frag(wave + 4 * a, jj, lane));
            F.qt[a][1][jj] = *reinterpret_cast<const bf16x8*>(ops + SB::QGT + K * C + FQT::frag(wave + 4 * a, jj, lane));
        }
}
template <int K, int V>
__device__ __forceinline__ void load_dscan_b_wt(DscanFragsB<K, V>& F, const BwdParams& p, int hv, int c,
                                                int wave, int lane, int v0) {
    typedef ScanOps<K, V> SO;
    typedef ScanOpsB<K, V> SB;
    typedef FragTile<__bf16, K, C> FWT;
    typedef DscanFragsB<K, V> DF;
    const int lq = lane >> 4;
    const size_t ci = (size_t)hv * p.NCmax + c;
    const __bf16* ops = reinterpret_cast<const __bf16*>(p.sops + ci * (size_t)SO::FLOATS);
    const float* eg = reinterpret_cast<const float*>(p.rec + ci * p.rec_bytes + p.off_eg);
#pragma unroll
    for (int a = 0; a < DF::NDT; ++a) {
#pragma unroll
        for (int jj = 0; jj < DF::NJS; ++jj) {
            F.wt[a][jj] = *reinterpret_cast<const bf16x8*>(ops + SB::WT + FWT::frag(wave + 4 * a, jj, lane));
        }
        F.e[a] = *reinterpret_cast<const f32x4*>(eg + 16 * (wave + 4 * a) + 4 * lq);
    }
}
template <int K, int V>
__device__ __forceinline__ void load_dscan_b(DscanFragsB<K, V>& F, const BwdParams& p, int hv, int c,
                                             int wave, int lane, int v0) {
    load_dscan_b_kg<K, V>(F, p, hv, c, wave, lane, v0);
    load_dscan_b_wt<K, V>(F, p, hv, c, wave, lane, v0);
}

template <int K, int V>
__global__ __launch_bounds__(BT, 1) void bwd_scan_bf16_kernel(BwdParams p) {
    constexpr int BV = 16, NVT = V / BV, NDT = K / 64;
    constexpr int LDK = K + 8, LDC = C + 8;   // bf16 row strides (16 distinct bank groups per fragment)
    typedef DscanFragsB<K, V> DF;
    typedef Mma<__bf16> M;
    __shared__ __attribute__((aligned(16))) __bf16 dSh[BV * LDK], dSl[BV * LDK];   // dS^T [v][d]
    __shared__ __attribute__((aligned(16))) __bf16 dvh[BV * LDC], dvl[BV * LDC];   // dv'^T [v][r]
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = p.N * p.HV * NVT;
    int vt, hv, n;
    scan_item(blockIdx.x, G, NVT, p.HV, p.dense ? nullptr : p.order, vt, hv, n);
    const int v0 = vt * BV;
    if (!p.dense && !p.slot_ok[n]) return;
    const int c0 = p.dense ? n * p.NT : p.coff[n];
    const int c1 = p.dense ? c0 + p.NT : p.cend[n];
    const size_t sbase = ((size_t)n * p.HV + hv) * (size_t)K * V;

    // four consecutive rows (d or r) of column lr: hi and lo
    auto put4 = [&](__bf16* hi, __bf16* lo, int off, f32x4 x) {
        bf16x4 h, l;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            h[r] = (__bf16)x[r];
            l[r] = (__bf16)(x[r] - (float)h[r]);
        }
        *reinterpret_cast<bf16x4*>(hi + off) = h;
        *reinterpret_cast<bf16x4*>(lo + off) = l;
    };
    f32x4 dS[NDT];
#pragma unroll
    for (int a = 0; a < NDT; ++a) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d = 16 * (wave + 4 * a) + 4 * lq + r;
            dS[a][r] = p.dht ? p.dht[sbase + (size_t)d * V + v0 + lr] : 0.f;
        }
        put4(dSh, dSl, lr * LDK + 16 * (wave + 4 * a) + 4 * lq, dS[a]);
    }
    // two-chunk ring: F0 holds chunk c, F1 chunk c - 1; past the first chunk a buffer
    // re-reads chunk c0 (in bounds, never used)
    auto clampc = [&](int c) { return c >= c0 ? c : c0; };
    DF F0, F1;
    DscanPB<K, V> PF;   // one chunk ahead (its loads hit the L2 lines the prefetch touched)
    if (c0 < c1) {
        load_dscan_b_p<K, V>(PF, p, hv, c1 - 1, wave, lane, v0);
        load_dscan_b<K, V>(F0, p, hv, c1 - 1, wave, lane, v0);
        load_dscan_b<K, V>(F1, p, hv, clampc(c1 - 2), wave, lane, v0);
    }
    // L2 prefetch of the operands BWD_L2_AHEAD chunks further down the walk: the chain's
    // NVT slice blocks share one XCD (scan_item) and block vt touches one word per
    // 128-byte line of its share of the bytes this kernel reads (the whole bf16 operand
    // slot); a loaded word is folded into `sink` when its ring slot comes round
    typedef ScanOps<K, V> SO;
    constexpr int LINES = ScanOpsB<K, V>::ELEMS * 2 / 128;
    static_assert((LINES + NVT - 1) / NVT <= BT, "one line per lane");
    const int l0 = vt * LINES / NVT, nl = (vt + 1) * LINES / NVT - l0;
    const int li = 64 * wave + lane;
    const size_t pbyte = (size_t)(l0 + li) * 128;
    uint32_t sink = 0, pf0 = 0, pf1 = 0;
    auto prefetch = [&](uint32_t& pf, int c) {
        sink ^= pf;
        if (li < nl) {
            const char* ops = reinterpret_cast<const char*>(p.sops + ((size_t)hv * p.NCmax + clampc(c - BWD_L2_AHEAD)) * (size_t)SO::FLOATS);
            pf = *reinterpret_cast<const uint32_t*>(ops + pbyte);
        }
    };
    __syncthreads();
    // one chunk of the walk; F's operands are then reloaded with chunk cn's, each group
    // right after its last use
    auto step = [&](DF& F, int c, int cn) {
        const size_t ci = (size_t)hv * p.NCmax + c;
        float* dhb = p.dh + ci * (size_t)K * V;
#pragma unroll
        for (int a = 0; a < NDT; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r) dhb[(size_t)(16 * (wave + 4 * a) + 4 * lq + r) * V + v0 + lr] = dS[a][r];
        // P1 = Aqk^T do at this wave's rows and the slice's columns (Aqk^T as hi + lo; do
        // is exact in bf16)
        f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = acc, p2[NDT];
#pragma unroll
        for (int jj = 0; jj < DF::NJS; ++jj) {
            acc = M::mma(PF.aq[0][jj], PF.dt[jj], acc);
            acc = M::mma(PF.aq[1][jj], PF.dt[jj], acc);
        }
        // dv' = P1 + kg dS (rows 16 wave + 4 lq + r, column lr of the slice)
#pragma unroll
        for (int kk = 0; kk < DF::NKS; ++kk) {
            const bf16x8 bh = *reinterpret_cast<const bf16x8*>(dSh + lr * LDK + 32 * kk + 8 * lq);
            const bf16x8 bl = *reinterpret_cast<const bf16x8*>(dSl + lr * LDK + 32 * kk + 8 * lq);
            acc = M::mma(F.kg[0][kk], bh, acc);
            acc2 = M::mma(F.kg[1][kk], bh, acc2);
            acc2 = M::mma(F.kg[0][kk], bl, acc2);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] += acc2[r];
        load_dscan_b_kg<K, V>(F, p, hv, cn, wave, lane, v0);
        float* dvb = p.dvn + ci * (size_t)C * V;
#pragma unroll
        for (int r = 0; r < 4; ++r) dvb[(size_t)(16 * wave + 4 * lq + r) * V + v0 + lr] = acc[r];
        put4(dvh, dvl, lr * LDC + 16 * wave + 4 * lq, acc);
        __syncthreads();
        // P2 = qg^T do (qg^T as hi + lo), then the next chunk's P operands; dS <- 2^G dS +
        // P2 - w^T dv'
#pragma unroll
        for (int a = 0; a < NDT; ++a) {
            p2[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jj = 0; jj < DF::NJS; ++jj) {
                p2[a] = M::mma(PF.qt[a][0][jj], PF.dt[jj], p2[a]);
                p2[a] = M::mma(PF.qt[a][1][jj], PF.dt[jj], p2[a]);
            }
        }
        load_dscan_b_p<K, V>(PF, p, hv, clampc(c - 1), wave, lane, v0);
#pragma unroll
        for (int a = 0; a < NDT; ++a) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jj = 0; jj < DF::NJS; ++jj) {
                x = M::mma(F.wt[a][jj], *reinterpret_cast<const bf16x8*>(dvh + lr * LDC + 32 * jj + 8 * lq), x);
                x = M::mma(F.wt[a][jj], *reinterpret_cast<const bf16x8*>(dvl + lr * LDC + 32 * jj + 8 * lq), x);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) dS[a][r] = fmaf(F.e[a][r], dS[a][r], p2[a][r] - x[r]);
            put4(dSh, dSl, lr * LDK + 16 * (wave + 4 * a) + 4 * lq, dS[a]);
        }
        load_dscan_b_wt<K, V>(F, p, hv, cn, wave, lane, v0);
        __syncthreads();
    };
    const int nsteps = c1 - c0;
    int c = c1 - 1;
    for (int t = 0; t < nsteps / 2; ++t, c -= 2) {
        step(F0, c, clampc(c - 2));
        prefetch(pf0, c);
        step(F1, c - 1, clampc(c - 3));
        prefetch(pf1, c - 1);
    }
    if (nsteps & 1) step(F0, c, clampc(c - 2));
    sink ^= pf0 ^ pf1;
    asm volatile("" ::"v"(sink));   // keeps the prefetch loads; emits no instruction
    if (p.dh0) {
#pragma unroll
        for (int a = 0; a < NDT; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                p.dh0[sbase + (size_t)(16 * (wave + 4 * a) + 4 * lq + r) * V + v0 + lr] = dS[a][r];
    }
}

// The prep for bf16 inputs: the reverse scan's operands as bf16 fragments for
// v_mfma_f32_16x16x32_bf16, no products. The records carry Aqk and qg as hi + lo bf16
// pairs and do is a bf16 input, so the scan's P1 = Aqk_hi^T do + Aqk_lo^T do and P2
// likewise are exact products accumulated in fp32 (the fp32 prep's result up to
// summation order). Their contraction runs over the chunk's rows, so Aqk, qg and do are
// staged transposed into bf16 LDS rows of 64 padded to 72 (144 bytes: the 16 rows of a
// fragment read start in 16 distinct four-bank groups) and copied out as Aqk^T, qg^T
// (hi, lo) and do^T fragments. The same LDS then stages w and kg^T: kg as hi + lo (rows
// s, contraction d), w^T (rows d, contraction r; w is a single bf16 in the record, so
// this copy is exact).
constexpr int PT_LD = 72;

// A fragment-order bf16 record tile (R rows, KC contraction, its residual tile at
// + R * KC) transposed into column-major LDS (dst[col * PT_LD + row]), in two steps:
// load() issues the thread's loads, store() writes them, so several tiles' loads are in
// flight together.
template <int R, int KC, int NTH>
struct FragTLoad {
    typedef Mma<__bf16> M;
    static constexpr int N = R * KC / 8 / NTH, NS = KC / M::KS;
    static_assert(N * NTH * 8 == R * KC, "whole runs per thread");
    bf16x8 h[N], l[N];
    __device__ __forceinline__ void load(const __bf16* t, int tid) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int e0 = 8 * (tid + NTH * i);
            h[i] = *reinterpret_cast<const bf16x8*>(t + e0);
            l[i] = *reinterpret_cast<const bf16x8*>(t + e0 + R * KC);
        }
    }
    __device__ __forceinline__ void store(__bf16* dh, __bf16* dl, int tid) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int q = tid + NTH * i, ln = q % 64, blk = q / 64;
            const int row = 16 * (blk / NS) + (ln & 15);
            const int col = (blk % NS) * M::KS + (ln >> 4) * M::KPL;
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                dh[(col + x) * PT_LD + row] = h[i][x];
                dl[(col + x) * PT_LD + row] = l[i][x];
            }
        }
    }
};

// A fragment-order bf16 record tile (R rows, KC contraction; with SPLIT its residual
// tile at + R * KC too) copied into row-major LDS (dst[row * ld + col]), in two steps
// like FragTLoad.
template <int R, int KC, int NTH, bool SPLIT>
struct FragRLoad {
    typedef Mma<__bf16> M;
    static constexpr int N = R * KC / 8 / NTH, NS = KC / M::KS;
    static_assert(N * NTH * 8 == R * KC, "whole runs per thread");
    bf16x8 h[N], l[SPLIT ? N : 1];
    __device__ __forceinline__ void load(const __bf16* t, int tid) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int e0 = 8 * (tid + NTH * i);
            h[i] = *reinterpret_cast<const bf16x8*>(t + e0);
            if constexpr (SPLIT) l[i] = *reinterpret_cast<const bf16x8*>(t + e0 + R * KC);
        }
    }
    __device__ __forceinline__ void store(__bf16* dh, __bf16* dl, int ld, int tid) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int q = tid + NTH * i, ln = q % 64, blk = q / 64;
            const int row = 16 * (blk / NS) + (ln & 15);
            const int col = (blk % NS) * M::KS + (ln >> 4) * M::KPL;
            *reinterpret_cast<bf16x8*>(dh + row * ld + col) = h[i];
            if constexpr (SPLIT) *reinterpret_cast<bf16x8*>(dl + row * ld + col) = l[i];
        }
    }
};

// R rows of W bf16 values (row r at src + r * rstride) transposed into LDS
// (dst[col * PT_LD + r]), zeros from row len on, in the same two steps; rows past len
// re-read row len - 1 (in bounds).
template <int R, int W, int NTH>
struct RowTLoad {
    static constexpr int W8 = W / 8, N = R * W8 / NTH;
    static_assert(N * NTH == R * W8, "whole runs per thread");
    bf16x8 x[N];
    __device__ __forceinline__ void load(const __bf16* src, size_t rstride, int len, int tid) {
        const int last = len > 0 ? len - 1 : 0;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int q = tid + NTH * i, r = q / W8, c0 = 8 * (q % W8);
            x[i] = len > 0 ? *reinterpret_cast<const bf16x8*>(src + (size_t)(r < len ? r : last) * rstride + c0)
                           : bf16x8{};
        }
    }
    __device__ __forceinline__ void store(int len, __bf16* dst, int tid) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int q = tid + NTH * i, r = q / W8, c0 = 8 * (q % W8);
#pragma unroll
            for (int e = 0; e < 8; ++e) dst[(c0 + e) * PT_LD + r] = r < len ? x[i][e] : (__bf16)0.f;
        }
    }
};

template <int K, int V>
__global__ __launch_bounds__(BT, 2) void bwd_prep_bf16_kernel(BwdParams p) {
    typedef ScanOps<K, V> SO;
    typedef ScanOpsB<K, V> SB;
    typedef Mma<__bf16> M;
    constexpr int T_BYTES = (2 * C + 2 * K + V) * PT_LD * 2;     // first phase
    constexpr int F_BYTES = 2 * K * PT_LD * 2 + C * (K + 8) * 2;  // second phase
    __shared__ __attribute__((aligned(16))) char smem[T_BYTES > F_BYTES ? T_BYTES : F_BYTES];
    __bf16* aTh = reinterpret_cast<__bf16*>(smem);   // Aqk^T [s][r], hi
    __bf16* aTl = aTh + C * PT_LD;                   //                lo
    __bf16* qTh = aTl + C * PT_LD;                   // qg^T [d][r], hi
    __bf16* qTl = qTh + K * PT_LD;                   //               lo
    __bf16* dT = qTl + K * PT_LD;                    // do^T [v][r]
    const int tid = threadIdx.x;
    int c, hv;
    int2 pos;
    if (!bwd_chunk(p, c, hv, pos)) return;
    const size_t ci = (size_t)hv * p.NCmax + c;
    const char* rec = p.rec + ci * p.rec_bytes;
    const __bf16* dout = reinterpret_cast<const __bf16*>(p.dout);
    float* ops = p.sops + ci * (size_t)SO::FLOATS;

    {
        // Aqk and qg (hi, lo) and the do rows: every load first, then the transposed stores
        FragTLoad<C, C, BT> la_;
        FragTLoad<C, K, BT> lq_;
        RowTLoad<C, V, BT> ld_;
        la_.load(reinterpret_cast<const __bf16*>(rec + p.off_aqk), tid);
        lq_.load(reinterpret_cast<const __bf16*>(rec + p.off_qg), tid);
        ld_.load(dout + ((size_t)pos.x * p.HV + hv) * V, (size_t)p.HV * V, pos.y, tid);
        la_.store(aTh, aTl, tid);
        lq_.store(qTh, qTl, tid);
        ld_.store(pos.y, dT, tid);
    }
    __syncthreads();
    // Aqk^T, qg^T (hi, lo) and do^T copied out in 16x16x32 fragment order (lane l of block
    // (band b, step st) holds row 16b + l % 16, columns 32st + 8(l / 16) ..): the reverse
    // scan's operands of P1 = Aqk^T do and P2 = qg^T do
    __bf16* ob = reinterpret_cast<__bf16*>(ops);
    auto copy_frags = [&](auto rows, const __bf16* t, __bf16* dst) {
        constexpr int N = decltype(rows)::value * C / 8 / BT;
        static_assert(N * BT * 8 == decltype(rows)::value * C, "whole runs per thread");
        bf16x8 x[N];
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int q = tid + BT * i, ln = q % 64, blk = q / 64;
            x[i] = *reinterpret_cast<const bf16x8*>(t + (16 * (blk / (C / 32)) + (ln & 15)) * PT_LD +
                                                    32 * (blk % (C / 32)) + 8 * (ln >> 4));
        }
#pragma unroll
        for (int i = 0; i < N; ++i) *reinterpret_cast<bf16x8*>(dst + 8 * (tid + BT * i)) = x[i];
    };
    copy_frags(std::integral_constant<int, C>(), aTh, ob + SB::AQT);
    copy_frags(std::integral_constant<int, C>(), aTl, ob + SB::AQT + C * C);
    copy_frags(std::integral_constant<int, K>(), qTh, ob + SB::QGT);
    copy_frags(std::integral_constant<int, K>(), qTl, ob + SB::QGT + K * C);
    copy_frags(std::integral_constant<int, V>(), dT, ob + SB::DOT);
    __syncthreads();
    // kg^T (rows d, contraction s; hi, lo) and w (rows r, contraction d) as row-major bf16
    __bf16* kTh = reinterpret_cast<__bf16*>(smem);   // kg^T [d][s], hi
    __bf16* kTl = kTh + K * PT_LD;                   //                lo
    __bf16* wR = kTl + K * PT_LD;                    // w [r][d]
    constexpr int WLD = K + 8;
    {
        // kg^T (hi, lo) and w from the record: every load first, then the LDS stores
        FragRLoad<K, C, BT, true> lk_;
        FragRLoad<C, K, BT, false> lw_;
        lk_.load(reinterpret_cast<const __bf16*>(rec + p.off_kgT), tid);
        lw_.load(reinterpret_cast<const __bf16*>(rec + p.off_w), tid);
        lk_.store(kTh, kTl, PT_LD, tid);
        lw_.store(wR, nullptr, WLD, tid);
    }
    __syncthreads();
    // kg (rows s, contraction d) and w^T (rows d, contraction r) in bf16 fragment order:
    // kg hi at KG, lo at KG + C K (bf16 elements); w^T at WT
    typedef FragTile<__bf16, C, K> FKGB;
    typedef FragTile<__bf16, K, C> FWTB;
    __bf16* okg = ob + SB::KG;
    __bf16* owt = ob + SB::WT;
    for (int q = tid; q < C * K / 8; q += BT) {
        const int l = q % 64, blk = q / 64;
        {
            const int srow = 16 * (blk / FKGB::NS) + (l & 15);
            const int d0 = (blk % FKGB::NS) * M::KS + (l >> 4) * M::KPL;
            bf16x8 h, lo;
#pragma unroll
            for (int x = 0; x < 8; ++x) { h[x] = kTh[(d0 + x) * PT_LD + srow]; lo[x] = kTl[(d0 + x) * PT_LD + srow]; }
            *reinterpret_cast<bf16x8*>(okg + 8 * q) = h;
            *reinterpret_cast<bf16x8*>(okg + C * K + 8 * q) = lo;
        }
        {
            const int drow = 16 * (blk / FWTB::NS) + (l & 15);
            const int r0 = (blk % FWTB::NS) * M::KS + (l >> 4) * M::KPL;
            bf16x8 h;
#pragma unroll
            for (int x = 0; x < 8; ++x) h[x] = wR[(r0 + x) * WLD + drow];
            *reinterpret_cast<bf16x8*>(owt + 8 * q) = h;
        }
    }
}

// ------------------------------------------------------------------------------------
// products with the state checkpoints, per (chunk, value head): dqg = do S^T,
// dw = -dv' S^T, dkg = v' dS^T, dAqk = do v'^T (s <= r), dG = ln2 2^G rowsum(dS S).
// Contraction over V in slices of 32 staged in LDS; wave w owns row band w.
// ------------------------------------------------------------------------------------
template <int K, int V, typename TIn>
__global__ __launch_bounds__(BT, 2) void bwd_state_kernel(BwdParams p) {
    constexpr int VC = 32, LV = VC + 1, NKT = K / 16;
    typedef GsLayout<K> GL;
    __shared__ float hL[K * LV];
    __shared__ float dhL[K * LV];
    __shared__ float doL[C * LV];
    __shared__ float vnL[C * LV];
    __shared__ float dvL[C * LV];
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int c, hv;
    int2 pos;
    if (!bwd_chunk(p, c, hv, pos)) return;
    const size_t ci = (size_t)hv * p.NCmax + c;
    const float* hC = p.h + ci * (size_t)K * V;
    const float* dhC = p.dh + ci * (size_t)K * V;
    const float* vnC = p.vn + ci * (size_t)C * V;
    const float* dvC = p.dvn + ci * (size_t)C * V;
    const TIn* dout = reinterpret_cast<const TIn*>(p.dout);
    const int r0 = 16 * wave;

    f32x4 aq[NKT], aw[NKT], ak[NKT], aA[4];
#pragma unroll
    for (int j = 0; j < NKT; ++j) { aq[j] = f32x4{0.f, 0.f, 0.f, 0.f}; aw[j] = aq[j]; ak[j] = aq[j]; }
#pragma unroll
    for (int j = 0; j < 4; ++j) aA[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float dgacc = 0.f;   // thread d < K: sum_v dS[d][v] S[d][v]
    for (int vb = 0; vb < V; vb += VC) {
        stage_f32<K, VC>(hC + vb, V, hL, LV, tid);
        stage_f32<K, VC>(dhC + vb, V, dhL, LV, tid);
        stage_rows<C, VC>(dout + ((size_t)pos.x * p.HV + hv) * V + vb, (size_t)p.HV * V, pos.y, doL, LV, tid);
        stage_f32<C, VC>(vnC + vb, V, vnL, LV, tid);
        stage_f32<C, VC>(dvC + vb, V, dvL, LV, tid);
        __syncthreads();
        if (tid < K)
            for (int vv = 0; vv < VC; ++vv) dgacc = fmaf(dhL[tid * LV + vv], hL[tid * LV + vv], dgacc);
#pragma unroll
        for (int j = 0; j < NKT; ++j) {
            auto bh = [&](int jj, int k) { return hL[(16 * j + jj) * LV + k]; };
            auto bdh = [&](int jj, int k) { return dhL[(16 * j + jj) * LV + k]; };
            aq[j] = mma_f32(aq[j], [&](int i, int k) { return doL[(r0 + i) * LV + k]; }, bh, VC, lane);
            aw[j] = mma_f32(aw[j], [&](int i, int k) { return dvL[(r0 + i) * LV + k]; }, bh, VC, lane);
            ak[j] = mma_f32(ak[j], [&](int i, int k) { return vnL[(r0 + i) * LV + k]; }, bdh, VC, lane);
        }
#pragma unroll
        for (int J = 0; J < 4; ++J)
            if (J <= wave)
                aA[J] = mma_f32(aA[J], [&](int i, int k) { return doL[(r0 + i) * LV + k]; },
                                [&](int jj, int k) { return vnL[(16 * J + jj) * LV + k]; }, VC, lane);
        __syncthreads();
    }
    float* out = p.gs + ci * (size_t)GL::FLOATS;
#pragma unroll
    for (int j = 0; j < NKT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = r0 + 4 * lq + r, d = 16 * j + lr;
            out[GL::DQG + row * K + d] = aq[j][r];
            out[GL::DW + row * K + d] = -aw[j][r];
            out[GL::DKG + row * K + d] = ak[j][r];
        }
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = r0 + 4 * lq + r, s = 16 * J + lr;
            out[GL::DA + row * C + s] = (J <= wave && s <= row) ? aA[J][r] : 0.f;
        }
    if (tid < K) {
        const float eg = reinterpret_cast<const float*>(p.rec + ci * p.rec_bytes + p.off_eg)[tid];
        out[GL::DG + tid] = LN2F * eg * dgacc;
    }
}

// The same products for bf16 inputs on the bf16 matrix cores: every fp32 operand is
// carried as a hi + lo bf16 pair and a product is hi*hi + lo*hi + hi*lo (do, a bf16
// input, is exact in bf16 and has no residual). Contraction over V in slices of 32: one
// v_mfma_f32_16x16x32_bf16 step per slice. The operands sit in LDS as bf16 rows of
// 32 values padded to 40 (80 bytes), so the 16 rows of a fragment read start in 16
// distinct four-bank groups. Sixteen waves (four per SIMD): wave w owns row band w % 4
// and a quarter of the 16-column tiles of K (part w / 4), and the band's dAqk tile
// J = part when J <= band.
constexpr int SB_LD = 40;          // bf16 row stride of the operand tiles
constexpr int SB_THREADS = 1024;

// The operand fragment of tile row `row`: lane (lq, lr) of a 16-row band reads values
// 8 lq .. 8 lq + 7 of its row.
__device__ __forceinline__ bf16x8 sb_frag(const __bf16* t, int row, int lq) {
    return *reinterpret_cast<const bf16x8*>(t + row * SB_LD + 8 * lq);
}

// One 32-column slice of the state kernel's operands, held in registers between its
// loads and its split stores (so that a slice's loads are in flight together, and the
// next slice's during this one's products): S and dS fp32 [K][32], v' and dv' fp32
// [64][32], do bf16 [64][32] (rows >= len zero). Thread t takes row t / 8, columns
// 4 (t % 8) .. + 3 of each tile, as stage_split and stage_rows_bf16 do.
__device__ __forceinline__ void put_split4(f32x4 x, __bf16* hi, __bf16* lo, int off) {
    bf16x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[e] = (__bf16)x[e];
        l[e] = (__bf16)(x[e] - (float)h[e]);
    }
    *reinterpret_cast<bf16x4*>(hi + off) = h;
    *reinterpret_cast<bf16x4*>(lo + off) = l;
}
template <int K, int V>
struct StateSlice {
    static_assert(K * 8 <= SB_THREADS && C * 8 <= SB_THREADS, "one vector per thread and tile");
    f32x4 h, dh, vn, dv;
    bf16x4 dO;
    __device__ __forceinline__ void load(const float* hC, const float* dhC, const float* vnC, const float* dvC,
                                         const __bf16* dorow, size_t dstride, int len, int vb, int tid) {
        const int r = tid >> 3, c4 = 4 * (tid & 7);
        if (r < K) {
            h = *reinterpret_cast<const f32x4*>(hC + (size_t)r * V + vb + c4);
            dh = *reinterpret_cast<const f32x4*>(dhC + (size_t)r * V + vb + c4);
        }
        if (r < C) {
            vn = *reinterpret_cast<const f32x4*>(vnC + (size_t)r * V + vb + c4);
            dv = *reinterpret_cast<const f32x4*>(dvC + (size_t)r * V + vb + c4);
            dO = bf16x4{};
            if (r < len) dO = *reinterpret_cast<const bf16x4*>(dorow + (size_t)r * dstride + vb + c4);
        }
    }
    __device__ __forceinline__ void store(__bf16* hH, __bf16* hLo, __bf16* dhH, __bf16* dhLo, __bf16* doH,
                                          __bf16* vnH, __bf16* vnLo, __bf16* dvH, __bf16* dvLo, int tid) const {
        const int r = tid >> 3, c4 = 4 * (tid & 7), o = r * SB_LD + c4;
        if (r < K) {
            put_split4(h, hH, hLo, o);
            put_split4(dh, dhH, dhLo, o);
        }
        if (r < C) {
            put_split4(vn, vnH, vnLo, o);
            put_split4(dv, dvH, dvLo, o);
            *reinterpret_cast<bf16x4*>(doH + o) = dO;
        }
    }
};

template <int K, int V>
__global__ __launch_bounds__(SB_THREADS, 4) void bwd_state_bf16_kernel(BwdParams p) {
    constexpr int VC = 32, NKH = K / 64;   // 16-column tiles of K per part
    typedef GsLayout<K> GL;
    typedef Mma<__bf16> M;
    __shared__ __attribute__((aligned(16))) __bf16 hH[K * SB_LD], hLo[K * SB_LD];
    __shared__ __attribute__((aligned(16))) __bf16 dhH[K * SB_LD], dhLo[K * SB_LD];
    __shared__ __attribute__((aligned(16))) __bf16 doH[C * SB_LD];
    __shared__ __attribute__((aligned(16))) __bf16 vnH[C * SB_LD], vnLo[C * SB_LD];
    __shared__ __attribute__((aligned(16))) __bf16 dvH[C * SB_LD], dvLo[C * SB_LD];
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int band = wave & 3, part = wave >> 2;
    int c, hv;
    int2 pos;
    if (!bwd_chunk(p, c, hv, pos)) return;
    const size_t ci = (size_t)hv * p.NCmax + c;
    const float* hC = p.h + ci * (size_t)K * V;
    const float* dhC = p.dh + ci * (size_t)K * V;
    const float* vnC = p.vn + ci * (size_t)C * V;
    const float* dvC = p.dvn + ci * (size_t)C * V;
    const __bf16* dout = reinterpret_cast<const __bf16*>(p.dout);
    const int r0 = 16 * band;
    const int j0 = NKH * part;

    f32x4 aq[NKH], aw[NKH], ak[NKH], aA;
#pragma unroll
    for (int j = 0; j < NKH; ++j) { aq[j] = f32x4{0.f, 0.f, 0.f, 0.f}; aw[j] = aq[j]; ak[j] = aq[j]; }
    aA = f32x4{0.f, 0.f, 0.f, 0.f};
    float dgacc = 0.f;   // thread d < K: sum_v dS[d][v] S[d][v]
    const __bf16* dorow = dout + ((size_t)pos.x * p.HV + hv) * V;
    StateSlice<K, V> cur, nxt;
    cur.load(hC, dhC, vnC, dvC, dorow, (size_t)p.HV * V, pos.y, 0, tid);
#pragma unroll
    for (int vb = 0; vb < V; vb += VC) {
        cur.store(hH, hLo, dhH, dhLo, doH, vnH, vnLo, dvH, dvLo, tid);
        __syncthreads();
        // the next slice's loads go out now and land during this slice's products
        if (vb + VC < V) nxt.load(hC, dhC, vnC, dvC, dorow, (size_t)p.HV * V, pos.y, vb + VC, tid);
        if (tid < K)
#pragma unroll 8   // (fully unrolled, its 128 LDS reads were all held in registers)
            for (int vv = 0; vv < VC; ++vv) {
                const int e = tid * SB_LD + vv;
                dgacc = fmaf((float)dhH[e] + (float)dhLo[e], (float)hH[e] + (float)hLo[e], dgacc);
            }
        const bf16x8 a_do = sb_frag(doH, r0 + lr, lq);
        const bf16x8 a_dvh = sb_frag(dvH, r0 + lr, lq), a_dvl = sb_frag(dvLo, r0 + lr, lq);
        const bf16x8 a_vnh = sb_frag(vnH, r0 + lr, lq), a_vnl = sb_frag(vnLo, r0 + lr, lq);
#pragma unroll
        for (int j = 0; j < NKH; ++j) {
            const int row = 16 * (j0 + j) + lr;
            const bf16x8 bh = sb_frag(hH, row, lq), bl = sb_frag(hLo, row, lq);
            const bf16x8 dh = sb_frag(dhH, row, lq), dl = sb_frag(dhLo, row, lq);
            aq[j] = M::mma(a_do, bh, aq[j]);
            aq[j] = M::mma(a_do, bl, aq[j]);
            aw[j] = M::mma(a_dvh, bh, aw[j]);
            aw[j] = M::mma(a_dvl, bh, aw[j]);
            aw[j] = M::mma(a_dvh, bl, aw[j]);
            ak[j] = M::mma(a_vnh, dh, ak[j]);
            ak[j] = M::mma(a_vnl, dh, ak[j]);
            ak[j] = M::mma(a_vnh, dl, ak[j]);
        }
        // dAqk tile (band, J = part), J <= band
        if (part <= band) {
            const bf16x8 vh = sb_frag(vnH, 16 * part + lr, lq), vl = sb_frag(vnLo, 16 * part + lr, lq);
            aA = M::mma(a_do, vh, aA);
            aA = M::mma(a_do, vl, aA);
        }
        __syncthreads();
        cur = nxt;
    }
    float* out = p.gs + ci * (size_t)GL::FLOATS;
#pragma unroll
    for (int j = 0; j < NKH; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = r0 + 4 * lq + r, d = 16 * (j0 + j) + lr;
            out[GL::DQG + row * K + d] = aq[j][r];
            out[GL::DW + row * K + d] = -aw[j][r];
            out[GL::DKG + row * K + d] = ak[j][r];
        }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = r0 + 4 * lq + r, s = 16 * part + lr;
        out[GL::DA + row * C + s] = (part <= band && s <= row) ? aA[r] : 0.f;
    }
    if (tid < K) {
        const float eg = reinterpret_cast<const float*>(p.rec + ci * p.rec_bytes + p.off_eg)[tid];
        out[GL::DG + tid] = LN2F * eg * dgacc;
    }
}

// ------------------------------------------------------------------------------------
// backward of the WY inverse, per (chunk, value head): with M and T from the recompute,
// writes dv and dbeta (final) and dkd, dM for the pair kernel. Eight waves; every product
// is split into 16x16 output tiles dealt round-robin to the waves, and the row sums
// that make dbeta are added into LDS.
// ------------------------------------------------------------------------------------
constexpr int WY_THREADS = 1024;

template <int K, int V, typename TIn, typename TB>
__global__ __launch_bounds__(WY_THREADS, 1) void bwd_wy_kernel(BwdParams p) {
    constexpr int NTH = WY_THREADS, NW = NTH / 64;
    constexpr int LA = C + 1, LK = K + 1, LX = (K > V ? K : V) + 1, LY = (V > C ? V : C) + 1;
    typedef GsLayout<K> GL;
    typedef WyLayout<K> WL;
    __shared__ float kL[C * LK];     // k, then kd = k 2^Gamma
    __shared__ float XL[C * LX];     // Gamma, then dv', then dw
    __shared__ float YL[C * LY];     // v, then T^T dT
    __shared__ float ML[C * LA];
    __shared__ float TL[C * LA];
    __shared__ float dTL[C * LA];
    __shared__ float bL[C];
    __shared__ float dbP[NW][C];     // each wave's row sums for dbeta (added in wave order at the end)
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int c, hv;
    int2 pos;
    if (!bwd_chunk(p, c, hv, pos)) return;
    const int h = hv / (p.HV / p.H);
    const int len = pos.y;
    const size_t ci = (size_t)hv * p.NCmax + c;
    const TIn* kin = reinterpret_cast<const TIn*>(p.k);
    const TIn* vin = reinterpret_cast<const TIn*>(p.v);
    const TB* bin = reinterpret_cast<const TB*>(p.beta);

    // ---- loads and the chunk-local cumsum of g ----
    RowLoad<C, K, TIn, NTH> lk_;
    lk_.load(kin + ((size_t)pos.x * p.H + h) * K, (size_t)p.H * K, len, tid);
    stage_gate<K, NTH>(p, pos, hv, XL, LX, tid);
    lk_.store(len, kL, LK, tid);
    if (tid < C) {
        float b = tid < len ? to_f32(bin[(size_t)(pos.x + tid) * p.HV + hv]) : 0.f;
        if (p.in.beta_sig != 0.f && tid < len) b = beta_from_logit(b, p.in.beta_sig);
        bL[tid] = b;
    }
    for (int e = tid; e < NW * C; e += NTH) dbP[e / C][e % C] = 0.f;
    __syncthreads();
    if (p.in.l2norm_k) l2norm_rows_lds<K>(kL, LK, tid);
    if (p.in.gate_mode != GATE_LOG2) gate_rows_lds<K, NTH>(XL, LX, len, p.in, hv, tid);
    __syncthreads();
    if (tid < K) {
        float acc = 0.f;
        for (int r = 0; r < C; ++r) { acc += XL[r * LX + tid]; XL[r * LX + tid] = acc; }
    }
    __syncthreads();
    // kd = k 2^Gamma; M and T = (I + diag(beta) M)^-1 as Stage 2 of the recompute left
    // them (their loads issued first, stored after the kd loop)
    {
        TileLoad<C, C, NTH> lm_, lt_;
        lm_.load(p.mt + ci * (size_t)(C * C), C, tid);
        lt_.load(p.mt + ((size_t)p.NCmax * p.HV + ci) * (C * C), C, tid);
        for (int e = tid; e < C * K; e += NTH) {
            const int r = e / K, d = e % K;
            kL[r * LK + d] *= exp2_fast(XL[r * LX + d]);
        }
        lm_.store(ML, LA, tid);
        lt_.store(TL, LA, tid);
    }
    __syncthreads();
    // row sums over one tile's columns (the 16 lanes of a row), added into the wave's own
    // partials (one lane per row: no atomics, so the sums do not depend on wave timing)
    auto add_rows = [&](int row0, const float (&x)[4]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float y = sum16(x[r]);
            if (lr == 0) dbP[wave][row0 + 4 * lq + r] += y;
        }
    };
    // dT tiles (I, J) owned by this wave: t = wave + NW i, I = t / 4, J = t % 4
    constexpr int NT_DT = 16 / NW;
    f32x4 dT[NT_DT];
#pragma unroll
    for (int i = 0; i < NT_DT; ++i) dT[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- value side: dv = beta T^T dv', dbeta += rowsum((T^T dv') v), dT = dv' (beta v)^T ----
    {
        TileLoad<C, V, NTH> ldv_;
        RowLoad<C, V, TIn, NTH> lv_;
        ldv_.load(p.dvn + ci * (size_t)C * V, V, tid);
        lv_.load(vin + ((size_t)pos.x * p.HV + hv) * V, (size_t)p.HV * V, len, tid);
        ldv_.store(XL, LX, tid);
        lv_.store(len, YL, LY, tid);
    }
    __syncthreads();
    // dw (for the key side) is loaded now and lands in XL once the value side is done
    const float* gsC = p.gs + ci * (size_t)GL::FLOATS;
    TileLoad<C, K, NTH> ldw_;
    ldw_.load(gsC + GL::DW, K, tid);
    TIn* dvout = reinterpret_cast<TIn*>(p.dv);
    for (int t = wave; t < 4 * (V / 16); t += NW) {
        const int sb = t / (V / 16), nt = t % (V / 16);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma_f32(acc, [&](int i, int k) { return TL[k * LA + 16 * sb + i]; },
                      [&](int j, int k) { return XL[k * LX + 16 * nt + j]; }, C, lane);
        float db[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int s = 16 * sb + 4 * lq + r, vv = 16 * nt + lr;
            db[r] = acc[r] * YL[s * LY + vv];
            if (s < len) dvout[((size_t)(pos.x + s) * p.HV + hv) * V + vv] = from_f32<TIn>(bL[s] * acc[r]);
        }
        add_rows(16 * sb, db);
    }
#pragma unroll
    for (int i = 0; i < NT_DT; ++i) {
        const int t = wave + NW * i, I = t / 4, J = t % 4;
        if (J <= I)
            dT[i] = mma_f32(dT[i], [&](int ii, int k) { return XL[(16 * I + ii) * LX + k]; },
                            [&](int j, int k) { return bL[16 * J + j] * YL[(16 * J + j) * LY + k]; }, V, lane);
    }
    __syncthreads();
    // ---- key side: dkd = beta T^T dw, dbeta += rowsum((T^T dw) kd), dT += dw (beta kd)^T ----
    ldw_.store(XL, LX, tid);
    __syncthreads();
    float* wyC = p.wy + ci * (size_t)WL::FLOATS;
    for (int t = wave; t < 4 * (K / 16); t += NW) {
        const int sb = t / (K / 16), nt = t % (K / 16);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma_f32(acc, [&](int i, int k) { return TL[k * LA + 16 * sb + i]; },
                      [&](int j, int k) { return XL[k * LX + 16 * nt + j]; }, C, lane);
        float db[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int s = 16 * sb + 4 * lq + r, d = 16 * nt + lr;
            db[r] = acc[r] * kL[s * LK + d];
            wyC[WL::DKD + s * K + d] = bL[s] * acc[r];
        }
        add_rows(16 * sb, db);
    }
#pragma unroll
    for (int i = 0; i < NT_DT; ++i) {
        const int t = wave + NW * i, I = t / 4, J = t % 4;
        if (J <= I)
            dT[i] = mma_f32(dT[i], [&](int ii, int k) { return XL[(16 * I + ii) * LX + k]; },
                            [&](int j, int k) { return bL[16 * J + j] * kL[(16 * J + j) * LK + k]; }, K, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * I + 4 * lq + r, s = 16 * J + lr;
            dTL[row * LA + s] = (J <= I && s < row) ? dT[i][r] : 0.f;
        }
    }
    __syncthreads();
    // ---- X = T^T dT (all tiles), then dL = -(X T^T) strictly lower ----
#pragma unroll
    for (int i = 0; i < NT_DT; ++i) {
        const int t = wave + NW * i, I = t / 4, J = t % 4;
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        x = mma_f32(x, [&](int ii, int k) { return TL[k * LA + 16 * I + ii]; },
                    [&](int j, int k) { return dTL[k * LA + 16 * J + j]; }, C, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) YL[(16 * I + 4 * lq + r) * LY + 16 * J + lr] = x[r];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NT_DT; ++i) {
        const int t = wave + NW * i, I = t / 4, J = t % 4;
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (J <= I)
            x = mma_f32(x, [&](int ii, int k) { return YL[(16 * I + ii) * LY + k]; },
                        [&](int j, int k) { return TL[(16 * J + j) * LA + k]; }, C, lane);
        float db[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * I + 4 * lq + r, s = 16 * J + lr;
            const float dl = (J <= I && s < row) ? -x[r] : 0.f;
            db[r] = dl * ML[row * LA + s];
            wyC[WL::DM + row * C + s] = bL[row] * dl;
        }
        add_rows(16 * I, db);
    }
    __syncthreads();
    if (tid < len) {
        float db = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) db += dbP[w][tid];
        const size_t e = (size_t)(pos.x + tid) * p.HV + hv;
        if (p.dbeta_f32) reinterpret_cast<float*>(p.dbeta)[e] = db;
        else reinterpret_cast<TB*>(p.dbeta)[e] = from_f32<TB>(db);
    }
}

// A chunk-head's k, v and gate rows and its beta, held in registers between their loads
// and their LDS stores (so that the next chunk-head's are in flight during this one's
// products). TG is the gate's element type (fp32 log2 decay or raw input, or a bf16 raw
// input). A scheduled chunk has at least one row: rows past its end re-read its last
// row (no branch around the loads) and are stored as zeros.
template <int K, int V, int NTH, typename TB, typename TG>
struct WyInputs {
    static constexpr int NK = C * K / (4 * NTH), NV = C * V / (4 * NTH);
    static_assert(NK * 4 * NTH == C * K && NV * 4 * NTH == C * V, "whole vectors per thread");
    typedef typename std::conditional<sizeof(TG) == 2, bf16x4, f32x4>::type gvec;
    bf16x4 k[NK], v[NV];
    gvec g[NK];
    TB b;
    __device__ __forceinline__ void load(const BwdParams& p, const TG* gsrc, int2 ps, int hv, int tid) {
        const int last = ps.y > 0 ? ps.y - 1 : 0, h = hv / (p.HV / p.H);
        const __bf16* kin = reinterpret_cast<const __bf16*>(p.k);
        const __bf16* vin = reinterpret_cast<const __bf16*>(p.v);
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int q = tid + NTH * i, r = min(q / (K / 4), last), c4 = 4 * (q % (K / 4));
            k[i] = *reinterpret_cast<const bf16x4*>(kin + ((size_t)(ps.x + r) * p.H + h) * K + c4);
            g[i] = *reinterpret_cast<const gvec*>(gsrc + ((size_t)(ps.x + r) * p.HV + hv) * K + c4);
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int q = tid + NTH * i, r = min(q / (V / 4), last), c4 = 4 * (q % (V / 4));
            v[i] = *reinterpret_cast<const bf16x4*>(vin + ((size_t)(ps.x + r) * p.HV + hv) * V + c4);
        }
        if (tid < C) b = reinterpret_cast<const TB*>(p.beta)[(size_t)(ps.x + min(tid, last)) * p.HV + hv];
    }
    // k and the gate as fp32 rows (row stride ld), v as bf16 rows (stride ldv), beta
    // (through its sigmoid with the option) into bL
    __device__ __forceinline__ void store(const BwdParams& p, int len, float* kS, float* GS, int ld, __bf16* vB,
                                          int ldv, float* bL, int tid) const {
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int q = tid + NTH * i, r = q / (K / 4), c4 = 4 * (q % (K / 4));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kS[r * ld + c4 + e] = r < len ? (float)k[i][e] : 0.f;
                GS[r * ld + c4 + e] = r < len ? (float)g[i][e] : 0.f;
            }
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int q = tid + NTH * i, r = q / (V / 4), c4 = 4 * (q % (V / 4));
            *reinterpret_cast<bf16x4*>(vB + r * ldv + c4) = r < len ? v[i] : bf16x4{};
        }
        if (tid < C) {
            float bt = tid < len ? to_f32(b) : 0.f;
            if (p.in.beta_sig != 0.f && tid < len) bt = beta_from_logit(bt, p.in.beta_sig);
            bL[tid] = bt;
        }
    }
};

// ------------------------------------------------------------------------------------
// The same backward of the WY inverse for bf16 inputs, its dense products on the bf16
// matrix cores. Each fp32 operand is split once into a hi + lo bf16 pair in LDS, laid
// out so that a lane's eight contraction values are one 16-byte read: T^T (for
// T^T dv', T^T dw, T^T dT) and T (for X T^T), dv' and dw both as rows (dT) and
// transposed (T^T dv', T^T dw), kd, v (a bf16 input, exact). A product is then
// hi*hi + lo*hi + hi*lo per 32-wide contraction step (hi*hi + lo*hi against v, and beta
// applied to the finished dT column). Sixteen waves, the tiles dealt as in the fp32
// kernel; the row sums for dbeta in per-wave partials. The blocks are persistent (one
// per CU, each looping over chunk-heads) and load the next chunk-head's k, v, gate and
// beta into registers during this one's products.
// ------------------------------------------------------------------------------------
// An fp32 [C][W] tile (row stride W) into registers, lane l of each wave taking row l:
// the transposed bf16 stores below then put a wave's 64 lanes on 32 distinct banks
// (lanes along a row would share four).
template <int W, int NTH>
struct ColLoad {
    static constexpr int WAVES = NTH / 64, N = C * W / (4 * NTH);
    static_assert(N * 4 * NTH == C * W, "whole vectors per thread");
    f32x4 x[N];
    __device__ __forceinline__ static int col(int tid, int i) { return 4 * ((tid >> 6) + WAVES * i); }
    __device__ __forceinline__ void load(const float* src, int tid) {
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] = *reinterpret_cast<const f32x4*>(src + (tid & 63) * W + col(tid, i));
    }
};

// That tile split into hi + lo bf16 rows (row r at r * ldr) and transposed rows (column
// c at c * ldt).
template <int W, int NTH>
__device__ __forceinline__ void store_split_rt(const ColLoad<W, NTH>& t, __bf16* rh, __bf16* rl, int ldr,
                                              __bf16* th, __bf16* tl, int ldt, int tid) {
#pragma unroll
    for (int i = 0; i < ColLoad<W, NTH>::N; ++i) {
        const int r = tid & 63, c4 = ColLoad<W, NTH>::col(tid, i);
        bf16x4 h, l;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            h[e] = (__bf16)t.x[i][e];
            l[e] = (__bf16)(t.x[i][e] - (float)h[e]);
            th[(c4 + e) * ldt + r] = h[e];
            tl[(c4 + e) * ldt + r] = l[e];
        }
        *reinterpret_cast<bf16x4*>(rh + r * ldr + c4) = h;
        *reinterpret_cast<bf16x4*>(rl + r * ldr + c4) = l;
    }
}

// The 16x16x32 operand fragment of row `row` at contraction offset k (k = k0 + 8 lq).
__device__ __forceinline__ bf16x8 wy_frag(const __bf16* t, int row, int ld, int k) {
    return *reinterpret_cast<const bf16x8*>(t + row * ld + k);
}

template <int K, int V, typename TB, typename TG>
__global__ __launch_bounds__(WY_THREADS, 1) void bwd_wy_bf16_kernel(BwdParams p) {
    constexpr int NTH = WY_THREADS, NW = NTH / 64;
    constexpr int MKV = K > V ? K : V;
    // bf16 row strides: 144 or 272 bytes, so the 16 rows of a fragment read start in 16
    // distinct four-bank groups
    constexpr int TP = C + 8, KP = K + 8, VP = V + 8, XP = MKV + 8, LK = K + 1;
    constexpr int A_ELEMS = 2 * C * XP, B_ELEMS = 4 * C * TP;
    static_assert(NTH == C * C / 4 && NTH / 64 == C / 4, "one float4 of T per thread");
    static_assert(2 * MKV * TP <= B_ELEMS, "transposed operand fits region B");
    static_assert(C * LK * 2 <= A_ELEMS && C * LK * 2 <= B_ELEMS, "fp32 staging fits regions A and B");
    static_assert(NW == 16, "one 16x16 tile of a 64x64 product per wave");
    typedef GsLayout<K> GL;
    typedef WyLayout<K> WL;
    typedef Mma<__bf16> M;
    __shared__ __attribute__((aligned(16))) __bf16 TtH[C * TP], TtL[C * TP];   // T^T
    __shared__ __attribute__((aligned(16))) __bf16 kdH[C * KP], kdL[C * KP];   // kd = k 2^Gamma
    __shared__ __attribute__((aligned(16))) __bf16 vB[C * VP];                // v
    // region A: Gamma (fp32), then dv' rows, then dw rows (hi, lo), then X = T^T dT
    // region B: k (fp32), then dv'^T, then dw^T (hi, lo), then T rows and dT^T
    __shared__ __attribute__((aligned(16))) __bf16 regA[A_ELEMS];
    __shared__ __attribute__((aligned(16))) __bf16 regB[B_ELEMS];
    __shared__ float bL[C];
    __shared__ float dbP[NW][C];     // each wave's row sums for dbeta (added in wave order at the end)
    __shared__ float runT[NTH];      // run totals of the gate cumsum
    float* GS = reinterpret_cast<float*>(regA);
    float* kS = reinterpret_cast<float*>(regB);
    __bf16 *AH = regA, *AL = regA + C * XP;
    __bf16 *BtH = regB, *BtL = regB + MKV * TP;
    __bf16 *ThH = regB, *ThL = regB + C * TP, *dTH = regB + 2 * C * TP, *dTL = regB + 3 * C * TP;
    __bf16 *XH = regA, *XLo = regA + C * TP;
    const int tid0 = threadIdx.x;
    const int G = p.NCmax * p.HV;
    const int nch = p.dense ? p.NCmax : p.nchunks[0];
    const TG* gsrc = static_cast<const TG*>(p.in.gate_mode == GATE_LOG2 ? static_cast<const void*>(p.g) : p.in.g_raw);
    // The block takes chunk-heads b, b + gridDim.x, ... and loads the next one's inputs
    // during this one's products.
    WyInputs<K, V, NTH, TB, TG> in_;
    int b = blockIdx.x, c = 0, hv = 0;
    while (b < G && !bwd_item(p, b, nch, c, hv)) b += gridDim.x;
    if (b < G) in_.load(p, gsrc, chunk_pos(p.dense, p.NT, p.T, p.table, c), hv, tid0);
    while (b < G) {
    // the lane indices re-derived from an opaque copy each chunk-head, so that the
    // compiler recomputes the lane-dependent LDS addresses in the body instead of keeping
    // them all live across the loop
    int tid = tid0;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tI = wave >> 2, tJ = wave & 3;   // this wave's tile of the 64 x 64 products
    const int2 pos = chunk_pos(p.dense, p.NT, p.T, p.table, c);
    const int len = pos.y;
    const size_t ci = (size_t)hv * p.NCmax + c;
    const float* gsC = p.gs + ci * (size_t)GL::FLOATS;
    float* wyC = p.wy + ci * (size_t)WL::FLOATS;
    // the next chunk-head this block takes
    int bn = b + gridDim.x, cn = 0, hvn = 0;
    while (bn < G && !bwd_item(p, bn, nch, cn, hvn)) bn += gridDim.x;

    // ---- this chunk-head's k, v, gate and beta into LDS; T and dv' into registers (they
    // land while the gate cumsum and kd run) ----
    in_.store(p, len, kS, GS, LK, vB, VP, bL, tid);
    // T[tr][tc .. tc + 3], lane l of each wave taking row l
    const int tr = tid & 63, tc = 4 * (tid >> 6);
    const f32x4 tq0 = *reinterpret_cast<const f32x4*>(p.mt + ((size_t)p.NCmax * p.HV + ci) * (C * C) + tr * C + tc);
    ColLoad<V, NTH> ldv_;
    ldv_.load(p.dvn + ci * (size_t)C * V, tid);
    for (int e = tid; e < NW * C; e += NTH) dbP[e / C][e % C] = 0.f;
    __syncthreads();
    if (p.in.l2norm_k) l2norm_rows_lds<K>(kS, LK, tid);
    if (p.in.gate_mode != GATE_LOG2) gate_rows_lds<K, NTH>(GS, LK, len, p.in, hv, tid);
    __syncthreads();
    cumsum_rows_lds<K, NTH>(GS, LK, runT, tid);
    __syncthreads();
    // kd = k 2^Gamma and T^T, split
    for (int e = tid; e < C * K; e += NTH) {
        const int r = e / K, d = e % K;
        const float x = kS[r * LK + d] * exp2_fast(GS[r * LK + d]);
        const __bf16 hx = (__bf16)x;
        kdH[r * KP + d] = hx;
        kdL[r * KP + d] = (__bf16)(x - (float)hx);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const __bf16 hx = (__bf16)tq0[e];
        TtH[(tc + e) * TP + tr] = hx;
        TtL[(tc + e) * TP + tr] = (__bf16)(tq0[e] - (float)hx);
    }
    __syncthreads();
    store_split_rt<V, NTH>(ldv_, AH, AL, XP, BtH, BtL, TP, tid);
    // dw (for the key side) is loaded now and lands during the value side, then the next
    // chunk-head's inputs
    ColLoad<K, NTH> ldw_;
    ldw_.load(gsC + GL::DW, tid);
    if (bn < G) in_.load(p, gsrc, chunk_pos(p.dense, p.NT, p.T, p.table, cn), hvn, tid);
    __syncthreads();

    auto add_rows = [&](int row0, const float (&x)[4]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float y = sum16(x[r]);
            if (lr == 0) dbP[wave][row0 + 4 * lq + r] += y;
        }
    };
    // T^T X for X = dv' or dw held transposed in region B: tile (sb, nt)
    auto tt_prod = [&](int sb, int nt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < C; k0 += 32) {
            const int k = k0 + 8 * lq;
            const bf16x8 ah = wy_frag(TtH, 16 * sb + lr, TP, k), al = wy_frag(TtL, 16 * sb + lr, TP, k);
            const bf16x8 bh = wy_frag(BtH, 16 * nt + lr, TP, k), bl = wy_frag(BtL, 16 * nt + lr, TP, k);
            acc = M::mma(ah, bh, acc);
            acc = M::mma(al, bh, acc);
            acc = M::mma(ah, bl, acc);
        }
        return acc;
    };
    // tiles (sb, nt) and (sb + 2, nt) together: one read of the X fragments serves both
    auto tt_prod2 = [&](int sb, int nt, f32x4& a0, f32x4& a1) {
        a0 = f32x4{0.f, 0.f, 0.f, 0.f};
        a1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < C; k0 += 32) {
            const int k = k0 + 8 * lq;
            const bf16x8 bh = wy_frag(BtH, 16 * nt + lr, TP, k), bl = wy_frag(BtL, 16 * nt + lr, TP, k);
            const bf16x8 ah0 = wy_frag(TtH, 16 * sb + lr, TP, k), al0 = wy_frag(TtL, 16 * sb + lr, TP, k);
            const bf16x8 ah1 = wy_frag(TtH, 16 * sb + 32 + lr, TP, k), al1 = wy_frag(TtL, 16 * sb + 32 + lr, TP, k);
            a0 = M::mma(ah0, bh, a0);
            a1 = M::mma(ah1, bh, a1);
            a0 = M::mma(al0, bh, a0);
            a1 = M::mma(al1, bh, a1);
            a0 = M::mma(ah0, bl, a0);
            a1 = M::mma(ah1, bl, a1);
        }
    };
    // every tile of T^T X (N / 16 column tiles) through epi(sb, nt, acc); with two tiles
    // per wave, wave w takes (w / (N / 16), w % (N / 16)) and the tile two row blocks down
    auto tt_all = [&](auto ncols, auto&& epi) {
        constexpr int NC = decltype(ncols)::value;
        if constexpr (4 * NC == 2 * NW) {
            const int sb = wave / NC, nt = wave % NC;
            f32x4 a0, a1;
            tt_prod2(sb, nt, a0, a1);
            epi(sb, nt, a0);
            epi(sb + 2, nt, a1);
        } else {
            for (int t = wave; t < 4 * NC; t += NW) epi(t / NC, t % NC, tt_prod(t / NC, t % NC));
        }
    };
    f32x4 dT = {0.f, 0.f, 0.f, 0.f};
    float mR[4];

    // ---- value side: dv = beta T^T dv', dbeta += rowsum((T^T dv') v), dT = dv' (beta v)^T ----
    __bf16* dvout = reinterpret_cast<__bf16*>(p.dv);
    tt_all(std::integral_constant<int, V / 16>(), [&](int sb, int nt, const f32x4& acc) {
        float db[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int s = 16 * sb + 4 * lq + r, vv = 16 * nt + lr;
            db[r] = acc[r] * (float)vB[s * VP + vv];
            if (s < len) dvout[((size_t)(pos.x + s) * p.HV + hv) * V + vv] = (__bf16)(bL[s] * acc[r]);
        }
        add_rows(16 * sb, db);
    });
    if (tJ <= tI) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < V; k0 += 32) {
            const int k = k0 + 8 * lq;
            const bf16x8 ah = wy_frag(AH, 16 * tI + lr, XP, k), al = wy_frag(AL, 16 * tI + lr, XP, k);
            const bf16x8 b = wy_frag(vB, 16 * tJ + lr, VP, k);
            acc = M::mma(ah, b, acc);
            acc = M::mma(al, b, acc);
        }
        const float bj = bL[16 * tJ + lr];
#pragma unroll
        for (int r = 0; r < 4; ++r) dT[r] = bj * acc[r];
    }
    __syncthreads();
    store_split_rt<K, NTH>(ldw_, AH, AL, XP, BtH, BtL, TP, tid);
    __syncthreads();
    // ---- key side: dkd = beta T^T dw, dbeta += rowsum((T^T dw) kd), dT += dw (beta kd)^T ----
    tt_all(std::integral_constant<int, K / 16>(), [&](int sb, int nt, const f32x4& acc) {
        float db[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int s = 16 * sb + 4 * lq + r, d = 16 * nt + lr;
            db[r] = acc[r] * ((float)kdH[s * KP + d] + (float)kdL[s * KP + d]);
            wyC[WL::DKD + s * K + d] = bL[s] * acc[r];
        }
        add_rows(16 * sb, db);
    });
    if (tJ <= tI) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += 32) {
            const int k = k0 + 8 * lq;
            const bf16x8 ah = wy_frag(AH, 16 * tI + lr, XP, k), al = wy_frag(AL, 16 * tI + lr, XP, k);
            const bf16x8 bh = wy_frag(kdH, 16 * tJ + lr, KP, k), bl = wy_frag(kdL, 16 * tJ + lr, KP, k);
            acc = M::mma(ah, bh, acc);
            acc = M::mma(al, bh, acc);
            acc = M::mma(ah, bl, acc);
        }
        const float bj = bL[16 * tJ + lr];
#pragma unroll
        for (int r = 0; r < 4; ++r) dT[r] = fmaf(bj, acc[r], dT[r]);
    }
    __syncthreads();
    // ---- dT (strictly lower) transposed and T as rows, split, into region B ----
    {
        // M at this lane's dL elements: loaded here rather than held in registers through
        // the products
#pragma unroll
        for (int r = 0; r < 4; ++r) mR[r] = p.mt[ci * (size_t)(C * C) + (16 * tI + 4 * lq + r) * C + 16 * tJ + lr];
        bf16x4 hv4, lv4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * tI + 4 * lq + r, s = 16 * tJ + lr;
            const float x = (tJ <= tI && s < row) ? dT[r] : 0.f;
            hv4[r] = (__bf16)x;
            lv4[r] = (__bf16)(x - (float)hv4[r]);
        }
        const int s = 16 * tJ + lr;
        *reinterpret_cast<bf16x4*>(dTH + s * TP + 16 * tI + 4 * lq) = hv4;
        *reinterpret_cast<bf16x4*>(dTL + s * TP + 16 * tI + 4 * lq) = lv4;
        // T as rows (hi, lo): T^T's split read transposed (the same bits as splitting T)
        bf16x4 th, tl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            th[e] = TtH[(tc + e) * TP + tr];
            tl[e] = TtL[(tc + e) * TP + tr];
        }
        *reinterpret_cast<bf16x4*>(ThH + tr * TP + tc) = th;
        *reinterpret_cast<bf16x4*>(ThL + tr * TP + tc) = tl;
    }
    __syncthreads();
    // ---- X = T^T dT (all tiles), split into region A ----
    {
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < C; k0 += 32) {
            const int k = k0 + 8 * lq;
            const bf16x8 ah = wy_frag(TtH, 16 * tI + lr, TP, k), al = wy_frag(TtL, 16 * tI + lr, TP, k);
            const bf16x8 bh = wy_frag(dTH, 16 * tJ + lr, TP, k), bl = wy_frag(dTL, 16 * tJ + lr, TP, k);
            x = M::mma(ah, bh, x);
            x = M::mma(al, bh, x);
            x = M::mma(ah, bl, x);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = (16 * tI + 4 * lq + r) * TP + 16 * tJ + lr;
            const __bf16 hx = (__bf16)x[r];
            XH[e] = hx;
            XLo[e] = (__bf16)(x[r] - (float)hx);
        }
    }
    __syncthreads();
    // ---- dL = -(X T^T) strictly lower; dM = beta dL, dbeta += rowsum(dL M) ----
    {
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (tJ <= tI) {
#pragma unroll
            for (int k0 = 0; k0 < C; k0 += 32) {
                const int k = k0 + 8 * lq;
                const bf16x8 ah = wy_frag(XH, 16 * tI + lr, TP, k), al = wy_frag(XLo, 16 * tI + lr, TP, k);
                const bf16x8 bh = wy_frag(ThH, 16 * tJ + lr, TP, k), bl = wy_frag(ThL, 16 * tJ + lr, TP, k);
                x = M::mma(ah, bh, x);
                x = M::mma(al, bh, x);
                x = M::mma(ah, bl, x);
            }
        }
        float db[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * tI + 4 * lq + r, s = 16 * tJ + lr;
            const float dl = (tJ <= tI && s < row) ? -x[r] : 0.f;
            db[r] = dl * mR[r];
            wyC[WL::DM + row * C + s] = bL[row] * dl;
        }
        add_rows(16 * tI, db);
    }
    __syncthreads();
    if (tid < len) {
        float db = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) db += dbP[w][tid];
        const size_t e = (size_t)(pos.x + tid) * p.HV + hv;
        if (p.dbeta_f32) reinterpret_cast<float*>(p.dbeta)[e] = db;
        else reinterpret_cast<TB*>(p.dbeta)[e] = from_f32<TB>(db);
    }
    __syncthreads();   // this chunk-head's LDS reads are done before the next one's stores
    b = bn;
    c = cn;
    hv = hvn;
    }
}

// ------------------------------------------------------------------------------------
// pair terms and the elementwise ones, per (chunk, value head): dq, dk (per value head,
// summed later) and dg (the chunk-local reverse cumsum of dGamma).
//   row side    dq_r  = sum_(s<=r) scale dAqk[r,s] k_s e(r,s),  dkr_r = sum_(s<r) dM[r,s] k_s e(r,s)
//   column side dkc_s = sum_(r>=s) (scale dAqk[r,s] q_r + dM[r,s] k_r) e(r,s)
// with e(r,s) = 2^(Gamma_r - Gamma_s) per channel. Pairs in different 16-row blocks run on
// the matrix cores, factored through a boundary row between them (both factors <= 1): the
// row side of block I through row 16I - 1, the column side of block J through row
// 16J + 15. Pairs inside a block keep one one-sided factor each. Two waves share each
// 16-channel tile (2K / 16 waves): one takes row blocks 0 and 1, the other 2 and 3 --
// block I's row side (8I products), column side (8(3 - I)) and diagonal (16) cost the
// same for every I -- and each lane holds its results in the matrix-core layout (rows
// 16I + 4lq .. +3 of channel 16 tile + lr) through the elementwise step.
// ------------------------------------------------------------------------------------
// largest decay spread (log2 units) of a 16-row block that the pair kernel anchors
constexpr float PAIR_SPREAD = 64.f;

template <int K>
constexpr int pair_threads() { return 8 * K; }   // two waves per 16-channel tile

template <int K, int V, typename TIn>
__global__ __launch_bounds__(pair_threads<K>(), 1) void bwd_pair_kernel(BwdParams p) {
    constexpr int LA = C + 1, LK = K + 1, NTH = pair_threads<K>();
    typedef GsLayout<K> GL;
    typedef WyLayout<K> WL;
    __shared__ float qL[C * LK];     // q, then dGamma
    __shared__ float kL[C * LK];
    __shared__ float GmL[C * LK];    // Gamma
    __shared__ float dAL[C * LA];    // dAqk (s <= r)
    __shared__ float dML[C * LA];    // dM (s < r)
    __shared__ float dGL[K];         // dG of the chunk end, from the state products
    __shared__ float dGP[2][K];      // each half's kg term of dG (added in a fixed order)
    __shared__ float runT[NTH];      // run totals of the two cumsums
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = wave % (K / 16), half = wave / (K / 16);   // channel tile; row blocks 2 half, 2 half + 1
    int c, hv;
    int2 pos;
    if (!bwd_chunk(p, c, hv, pos)) return;
    const int h = hv / (p.HV / p.H);
    const int len = pos.y;
    const size_t ci = (size_t)hv * p.NCmax + c;
    const TIn* qin = reinterpret_cast<const TIn*>(p.q);
    const TIn* kin = reinterpret_cast<const TIn*>(p.k);
    const float* gsC = p.gs + ci * (size_t)GL::FLOATS;
    const float* wyC = p.wy + ci * (size_t)WL::FLOATS;
    const float sc = p.scale;

    {
        // q, k, dAqk and dM loads go out together, the gate is staged meanwhile
        RowLoad<C, K, TIn, NTH> lq_, lk_;
        TileLoad<C, C, NTH> la_, lm_;
        lq_.load(qin + ((size_t)pos.x * p.H + h) * K, (size_t)p.H * K, len, tid);
        lk_.load(kin + ((size_t)pos.x * p.H + h) * K, (size_t)p.H * K, len, tid);
        la_.load(gsC + GL::DA, C, tid);   // dAqk (the scale is applied at use)
        lm_.load(wyC + WL::DM, C, tid);
        stage_gate<K, NTH>(p, pos, hv, GmL, LK, tid);
        if (tid < K) dGL[tid] = gsC[GL::DG + tid];
        lq_.store(len, qL, LK, tid);
        lk_.store(len, kL, LK, tid);
        la_.store(dAL, LA, tid);
        lm_.store(dML, LA, tid);
    }
    __syncthreads();
    if (p.in.l2norm_q) l2norm_rows_lds<K>(qL, LK, tid);        // threads 0 .. 63
    if (p.in.l2norm_k) l2norm_rows_lds<K>(kL, LK, tid - C);    // threads 64 .. 127
    if (p.in.gate_mode != GATE_LOG2) gate_rows_lds<K, NTH>(GmL, LK, len, p.in, hv, tid);
    __syncthreads();
    cumsum_rows_lds<K, NTH>(GmL, LK, runT, tid);
    __syncthreads();

    const int d = 16 * tile + lr;
    // the state products' and the WY backward's gradients at this lane's elements (rows
    // 16 I + 4 lq + rr of channel d), loaded now so that they land during the products
    float dqgR[2][4], dkgR[2][4], dkdR[2][4];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int r = 16 * (2 * half + ib) + 4 * lq + rr;
            dqgR[ib][rr] = gsC[GL::DQG + r * K + d];
            dkgR[ib][rr] = gsC[GL::DKG + r * K + d];
            dkdR[ib][rr] = wyC[WL::DKD + r * K + d];
        }

    // accumulators of the wave's two row blocks I = 2 half + ib
    f32x4 aq[2], akr[2], akc[2];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
        aq[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
        akr[ib] = aq[ib];
        akc[ib] = aq[ib];
    }
    // row side, pairs across blocks: block I against rows s < 16I, through row 16I - 1
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
        const int I = 2 * half + ib;
        if (I == 0) continue;
        const float P = GmL[(16 * I - 1) * LK + d];
        f32x4 yq = {0.f, 0.f, 0.f, 0.f}, yk = {0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < 16 * I; s0 += 4) {
            const int s = s0 + lq;
            const float b = kL[s * LK + d] * exp2_fast(P - GmL[s * LK + d]);
            yq = __builtin_amdgcn_mfma_f32_16x16x4f32(sc * dAL[(16 * I + lr) * LA + s], b, yq, 0, 0, 0);
            yk = __builtin_amdgcn_mfma_f32_16x16x4f32(dML[(16 * I + lr) * LA + s], b, yk, 0, 0, 0);
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const float f = exp2_fast(GmL[(16 * I + 4 * lq + rr) * LK + d] - P);
            aq[ib][rr] = fmaf(f, yq[rr], aq[ib][rr]);
            akr[ib][rr] = fmaf(f, yk[rr], akr[ib][rr]);
        }
    }
    // column side, pairs across blocks: block J against rows r >= 16J + 16, through
    // row 16J + 15
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
        const int J = 2 * half + ib;
        if (J == 3) continue;
        const float Q = GmL[(16 * J + 15) * LK + d];
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        for (int r0 = 16 * (J + 1); r0 < C; r0 += 4) {
            const int r = r0 + lq;
            const float e = exp2_fast(GmL[r * LK + d] - Q);
            z = __builtin_amdgcn_mfma_f32_16x16x4f32(sc * dAL[r * LA + 16 * J + lr], qL[r * LK + d] * e, z, 0, 0, 0);
            z = __builtin_amdgcn_mfma_f32_16x16x4f32(dML[r * LA + 16 * J + lr], kL[r * LK + d] * e, z, 0, 0, 0);
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const float f = exp2_fast(Q - GmL[(16 * J + 4 * lq + rr) * LK + d]);
            akc[ib][rr] = fmaf(f, z[rr], akc[ib][rr]);
        }
    }
    // pairs inside a block. Where the block's decay spread (Gamma of its first row minus
    // Gamma of its last, in every channel of the tile) is at most PAIR_SPREAD, anchor
    // the factors at a block boundary row and use the matrix cores:
    //   row side    2^(G_r - G_s) = 2^(G_r - G_last) 2^(G_last - G_s),
    //   column side 2^(G_s - G_r) = 2^(G_first - G_r) 2^(G_s - G_first),
    // the second factor (<= 1) scaling the operand and the first (<= 2^spread) the
    // finished sum. Otherwise one one-sided factor per pair (exact at any decay). In
    // both, pairs on the wrong side of the diagonal meet a zero dAqk / dM.
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
        const int I = 2 * half + ib;
        f32x4 xq4, xk4, xc4;
        const float gfirst = GmL[(16 * I) * LK + d], glast = GmL[(16 * I + 15) * LK + d];
        const bool steep = __builtin_amdgcn_ballot_w64(gfirst - glast > PAIR_SPREAD) != 0;   // wave-uniform
        if (!steep) {
            f32x4 yq = {0.f, 0.f, 0.f, 0.f}, yk = yq, yc = yq;
            const int ri = 16 * I + lr;   // A operand row of this lane
#pragma unroll
            for (int s0 = 0; s0 < 16; s0 += 4) {
                const int s = 16 * I + s0 + lq;   // contraction index of this lane
                const float gs = GmL[s * LK + d];
                const float ks = kL[s * LK + d];
                const float br = ks * exp2_fast(glast - gs);
                const float fc = exp2_fast(gs - gfirst);
                yq = __builtin_amdgcn_mfma_f32_16x16x4f32(dAL[ri * LA + s], br, yq, 0, 0, 0);
                yk = __builtin_amdgcn_mfma_f32_16x16x4f32(dML[ri * LA + s], br, yk, 0, 0, 0);
                yc = __builtin_amdgcn_mfma_f32_16x16x4f32(sc * dAL[s * LA + ri], qL[s * LK + d] * fc, yc, 0, 0, 0);
                yc = __builtin_amdgcn_mfma_f32_16x16x4f32(dML[s * LA + ri], ks * fc, yc, 0, 0, 0);
            }
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const float gr = GmL[(16 * I + 4 * lq + rr) * LK + d];
                const float fr = exp2_fast(gr - glast), fcol = exp2_fast(gfirst - gr);
                xq4[rr] = sc * fr * yq[rr];
                xk4[rr] = fr * yk[rr];
                xc4[rr] = fcol * yc[rr];
            }
        } else {
            // (the rows' k, q and Gamma are read from LDS inside the loop: this branch is
            // rare, and holding them in registers would crowd the 128-register budget)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int r = 16 * I + 4 * lq + rr;
                const float gr = GmL[r * LK + d];
                float xq = 0.f, xk = 0.f, xc = 0.f;
#pragma unroll 4
                for (int j = 0; j < 16; ++j) {
                    const int s = 16 * I + j;
                    const float kb = kL[s * LK + d], qb = qL[s * LK + d];
                    // row side (s <= r): 2^min(x, 0); column side (s >= r): 2^min(-x, 0),
                    // x = Gamma_r - Gamma_s; both are 2^-|x| on their own side and 1 on
                    // the other, so one exp2 serves the pair
                    const float x = gr - GmL[s * LK + d];
                    const float t2 = exp2_fast(-fabsf(x));
                    const float er = x <= 0.f ? t2 : 1.f;
                    const float ec = x >= 0.f ? t2 : 1.f;
                    const float ek = kb * er;
                    xq = fmaf(dAL[r * LA + s], ek, xq);
                    xk = fmaf(dML[r * LA + s], ek, xk);
                    xc = fmaf(fmaf(sc * dAL[s * LA + r], qb, dML[s * LA + r] * kb), ec, xc);
                }
                xq4[rr] = sc * xq;
                xk4[rr] = xk;
                xc4[rr] = xc;
            }
        }
        aq[ib] += xq4;
        akr[ib] += xk4;
        akc[ib] += xc4;
    }
    // elementwise terms of qg, kd, kg; dGamma; dq, dk per value head
    float dgam[2][4];
    {
        const float Gd = GmL[(C - 1) * LK + d];
        float dgk = 0.f;
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int r = 16 * (2 * half + ib) + 4 * lq + rr;
                const float qv = qL[r * LK + d], kv = kL[r * LK + d], gr = GmL[r * LK + d];
                const float e1 = exp2_fast(gr), e2 = exp2_fast(Gd - gr);
                const float dqg = dqgR[ib][rr], dkg = dkgR[ib][rr], dkd = dkdR[ib][rr];
                const float dqi = aq[ib][rr], dkr = akr[ib][rr], dkc = akc[ib][rr];
                const float dq = fmaf(sc * e1, dqg, dqi);
                const float dk = dkr + dkc + e1 * dkd + e2 * dkg;
                const float kge = kv * e2 * dkg;
                dgam[ib][rr] = LN2F * (qv * dq + kv * (dkr - dkc + e1 * dkd) - kge);
                if (r < len) {
                    dgk += kge;
                    const size_t row = (size_t)(pos.x + r);
                    p.dq_hv[(row * p.HV + hv) * K + d] = dq;
                    p.dk_hv[(row * p.HV + hv) * K + d] = dk;
                }
            }
        // the four lanes of channel d (lq = 0..3) summed in a fixed order
        dgk += __shfl_xor(dgk, 16, 64);
        dgk += __shfl_xor(dgk, 32, 64);
        if (lq == 0) dGP[half][d] = LN2F * dgk;
    }
    __syncthreads();   // qL becomes dGamma
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            qL[(16 * (2 * half + ib) + 4 * lq + rr) * LK + d] = dgam[ib][rr];
    __syncthreads();
    // dg = reverse cumsum of dGamma over the chunk's rows (rows >= len left out); dG
    // joins at the last row. Runs of RL rows per thread, as in the forward cumsum.
    {
        constexpr int NS = NTH / K, RL = C / NS;
        const int dc = tid % K, sg = tid / K;
        float x[RL];
        float acc = 0.f;
#pragma unroll
        for (int i = RL - 1; i >= 0; --i) {
            const int r = sg * RL + i;
            acc += r < len ? qL[r * LK + dc] : 0.f;
            x[i] = acc;
        }
        runT[sg * K + dc] = acc;
        __syncthreads();
        float off = dGL[dc] + dGP[0][dc] + dGP[1][dc];
        for (int j = NS - 1; j > sg; --j) off += runT[j * K + dc];
#pragma unroll
        for (int i = 0; i < RL; ++i) {
            const int r = sg * RL + i;
            if (r < len) p.dg[((size_t)(pos.x + r) * p.HV + hv) * K + dc] = x[i] + off;
        }
    }
}

// ------------------------------------------------------------------------------------
// The pair terms for bf16 inputs on the bf16 matrix cores (16x16x16: a 16-row block is
// one contraction step). scale dAqk and dM are split once into hi + lo bf16 tiles, as
// rows (the row side: contraction over s) and transposed (the column side: contraction
// over r); each lane's decayed k / q operand values are split as they are formed, and a
// product is hi*hi + lo*hi + hi*lo. q and k stay bf16 in LDS (exact) with the rows'
// normalisation factors beside them; the tiling, the anchoring and the elementwise
// step are those of the fp32 kernel.
// ------------------------------------------------------------------------------------
// 16x16x16 operand fragment: row `row`, contraction values k .. k + 3 (k = k0 + 4 lq)
__device__ __forceinline__ bf16x4 pair_frag(const __bf16* t, int row, int k) {
    return *reinterpret_cast<const bf16x4*>(t + row * (C + 8) + k);
}
__device__ __forceinline__ f32x4 mma16_3(bf16x4 ah, bf16x4 al, bf16x4 bh, bf16x4 bl, f32x4 c) {
    c = mma16(ah, bl, c);
    c = mma16(al, bh, c);
    return mma16(ah, bh, c);
}

template <int K, int V>
__global__ __launch_bounds__(pair_threads<K>(), 1) void bwd_pair_bf16_kernel(BwdParams p) {
    constexpr int NTH = pair_threads<K>(), LK = K + 1, KP = K + 8, TP = C + 8;
    typedef GsLayout<K> GL;
    typedef WyLayout<K> WL;
    __shared__ __attribute__((aligned(16))) __bf16 qB[C * KP], kB[C * KP];   // q, k (bf16 inputs)
    __shared__ float rnq[C], rnk[C];     // row normalisation factors (1 without the option)
    __shared__ float GmL[C * LK];        // Gamma
    // scale dAqk (s <= r) and dM (s < r): hi / lo, as rows then transposed; after the
    // products the region holds dGamma [C][LK] fp32
    __shared__ __attribute__((aligned(16))) __bf16 At[8 * C * TP];
    __shared__ float dGL[K];             // dG of the chunk end, from the state products
    __shared__ float dGP[2][K];          // each half's kg term of dG (added in a fixed order)
    __shared__ float runT[NTH];          // run totals of the two cumsums
    static_assert(C * LK * 4 <= 8 * C * TP * 2, "dGamma fits the operand region");
    __bf16 *aH = At, *aL = At + C * TP, *mH = At + 2 * C * TP, *mL = At + 3 * C * TP;
    __bf16 *atH = At + 4 * C * TP, *atL = At + 5 * C * TP, *mtH = At + 6 * C * TP, *mtL = At + 7 * C * TP;
    float* dGam = reinterpret_cast<float*>(At);
    // A block takes one chunk and, with pair_gva, one q/k head and all of its value
    // heads in turn (q, k and their normalisation factors staged once; dq, dk summed over
    // the value heads in the first one's slot of the per-value-head buffers, the last one
    // writing the bf16 results), else one (chunk, value head).
    const int grp = p.HV / p.H;
    const int nh = p.pair_gva ? p.H : p.HV;
    const int item = xcd_remap(blockIdx.x, p.NCmax * nh);
    const int c = item / nh, hh = item % nh;
    if (!p.dense && c >= p.nchunks[0]) return;
    const int2 pos = chunk_pos(p.dense, p.NT, p.T, p.table, c);
    const int h = p.pair_gva ? hh : hh / grp;
    const int ng = p.pair_gva ? grp : 1;
    const int len = pos.y;
    const __bf16* qin = reinterpret_cast<const __bf16*>(p.q);
    const __bf16* kin = reinterpret_cast<const __bf16*>(p.k);
    __bf16* dqo = reinterpret_cast<__bf16*>(p.dq);
    __bf16* dko = reinterpret_cast<__bf16*>(p.dk);
    const float sc = p.scale;
    const int tid0 = threadIdx.x;
    {
        // q, k (bf16, exact) and their rows' normalisation factors, once for the block
        RowLoad<C, K, __bf16, NTH> lq_, lk_;
        lq_.load(qin + ((size_t)pos.x * p.H + h) * K, (size_t)p.H * K, len, tid0);
        lk_.load(kin + ((size_t)pos.x * p.H + h) * K, (size_t)p.H * K, len, tid0);
#pragma unroll
        for (int i = 0; i < RowLoad<C, K, __bf16, NTH>::N; ++i) {
            const int q = tid0 + NTH * i, r = q / (K / 4), c4 = 4 * (q % (K / 4));
            *reinterpret_cast<bf16x4*>(qB + r * KP + c4) = r < len ? lq_.x[i] : bf16x4{};
            *reinterpret_cast<bf16x4*>(kB + r * KP + c4) = r < len ? lk_.x[i] : bf16x4{};
        }
        __syncthreads();
        // threads 0 .. 63 the q rows, 64 .. 127 the k rows (the sum of squares in channel
        // order, as the fp32 kernel's)
        if (tid0 < 2 * C) {
            const int r = tid0 & 63;
            const bool isq = tid0 < C;
            float f = 1.f;
            if (isq ? p.in.l2norm_q : p.in.l2norm_k) {
                const __bf16* row = (isq ? qB : kB) + r * KP;
                float ss = 0.f;
#pragma unroll 8
                for (int d = 0; d < K; ++d) ss = fmaf((float)row[d], (float)row[d], ss);
                f = l2norm_rstd(ss);
            }
            (isq ? rnq : rnk)[r] = f;
        }
    }
    for (int g = 0; g < ng; ++g) {
    // lane indices from an opaque copy each value head (the lane-dependent LDS addresses
    // are then recomputed in the body, not held live across the loop)
    int tid = tid0;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = wave % (K / 16), half = wave / (K / 16);   // channel tile; row blocks 2 half, 2 half + 1
    const int hv = p.pair_gva ? h * grp + g : hh;
    const size_t ci = (size_t)hv * p.NCmax + c;
    const float* gsC = p.gs + ci * (size_t)GL::FLOATS;
    const float* wyC = p.wy + ci * (size_t)WL::FLOATS;

    {
        // dAqk and dM loads go out together, the gate is staged meanwhile
        ColLoad<C, NTH> la_, lm_;
        la_.load(gsC + GL::DA, tid);
        lm_.load(wyC + WL::DM, tid);
        stage_gate<K, NTH>(p, pos, hv, GmL, LK, tid);
        if (tid < K) dGL[tid] = gsC[GL::DG + tid];
#pragma unroll
        for (int i = 0; i < ColLoad<C, NTH>::N; ++i) {
            f32x4 x = la_.x[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] *= sc;
            const int r = tid & 63, c4 = ColLoad<C, NTH>::col(tid, i);
            bf16x4 hh, ll;
            split4(x, hh, ll);
            *reinterpret_cast<bf16x4*>(aH + r * TP + c4) = hh;
            *reinterpret_cast<bf16x4*>(aL + r * TP + c4) = ll;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                atH[(c4 + e) * TP + r] = hh[e];
                atL[(c4 + e) * TP + r] = ll[e];
            }
            split4(lm_.x[i], hh, ll);
            *reinterpret_cast<bf16x4*>(mH + r * TP + c4) = hh;
            *reinterpret_cast<bf16x4*>(mL + r * TP + c4) = ll;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                mtH[(c4 + e) * TP + r] = hh[e];
                mtL[(c4 + e) * TP + r] = ll[e];
            }
        }
    }
    __syncthreads();
    if (p.in.gate_mode != GATE_LOG2) gate_rows_lds<K, NTH>(GmL, LK, len, p.in, hv, tid);
    __syncthreads();
    cumsum_rows_lds<K, NTH>(GmL, LK, runT, tid);
    __syncthreads();

    const int d = 16 * tile + lr;
    auto qval = [&](int r) { return (float)qB[r * KP + d] * rnq[r]; };
    auto kval = [&](int r) { return (float)kB[r * KP + d] * rnk[r]; };
    // The wave's two row blocks I = 2 half + ib one after the other: products, then the
    // elementwise step of the block's rows. The state products' and the WY backward's
    // gradients at a block's elements (rows 16 I + 4 lq + rr of channel d) are loaded
    // one block ahead, so they land during the products.
    float dgam[2][4];
    float dgk = 0.f;
    const float Gd = GmL[(C - 1) * LK + d];
    float dqgR[4], dkgR[4], dkdR[4];
    auto load_grads = [&](int I) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int r = 16 * I + 4 * lq + rr;
            dqgR[rr] = gsC[GL::DQG + r * K + d];
            dkgR[rr] = gsC[GL::DKG + r * K + d];
            dkdR[rr] = wyC[WL::DKD + r * K + d];
        }
    };
    load_grads(2 * half);
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
        const int I = 2 * half + ib;
        f32x4 aq = {0.f, 0.f, 0.f, 0.f}, akr = aq, akc = aq;
        // row side, pairs across blocks: block I against the blocks S < I, through row 16I - 1
        if (I > 0) {
            const float P = GmL[(16 * I - 1) * LK + d];
            f32x4 yq = {0.f, 0.f, 0.f, 0.f}, yk = {0.f, 0.f, 0.f, 0.f};
            for (int S = 0; S < I; ++S) {
                f32x4 b;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int s = 16 * S + 4 * lq + j;
                    b[j] = kval(s) * exp2_fast(P - GmL[s * LK + d]);
                }
                bf16x4 bh, bl;
                split4(b, bh, bl);
                const int k = 16 * S + 4 * lq;
                yq = mma16_3(pair_frag(aH, 16 * I + lr, k), pair_frag(aL, 16 * I + lr, k), bh, bl, yq);
                yk = mma16_3(pair_frag(mH, 16 * I + lr, k), pair_frag(mL, 16 * I + lr, k), bh, bl, yk);
            }
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const float f = exp2_fast(GmL[(16 * I + 4 * lq + rr) * LK + d] - P);
                aq[rr] = f * yq[rr];
                akr[rr] = f * yk[rr];
            }
        }
        // column side, pairs across blocks: block I against the blocks R > I, through row
        // 16I + 15
        if (I < 3) {
            const float Q = GmL[(16 * I + 15) * LK + d];
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
            for (int R = I + 1; R < 4; ++R) {
                f32x4 bq, bk;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * R + 4 * lq + j;
                    const float e = exp2_fast(GmL[r * LK + d] - Q);
                    bq[j] = qval(r) * e;
                    bk[j] = kval(r) * e;
                }
                bf16x4 bqh, bql, bkh, bkl;
                split4(bq, bqh, bql);
                split4(bk, bkh, bkl);
                const int k = 16 * R + 4 * lq;
                z = mma16_3(pair_frag(atH, 16 * I + lr, k), pair_frag(atL, 16 * I + lr, k), bqh, bql, z);
                z = mma16_3(pair_frag(mtH, 16 * I + lr, k), pair_frag(mtL, 16 * I + lr, k), bkh, bkl, z);
            }
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                akc[rr] = exp2_fast(Q - GmL[(16 * I + 4 * lq + rr) * LK + d]) * z[rr];
        }
        // pairs inside the block: anchored at a block boundary row on the matrix cores
        // where the block's decay spread is at most PAIR_SPREAD, else one one-sided factor
        // per pair (exact at any decay); pairs on the wrong side of the diagonal meet a
        // zero dAqk / dM.
        const float gfirst = GmL[(16 * I) * LK + d], glast = GmL[(16 * I + 15) * LK + d];
        const bool steep = __builtin_amdgcn_ballot_w64(gfirst - glast > PAIR_SPREAD) != 0;   // wave-uniform
        if (!steep) {
            // row side (anchored at the block's last row), then the column side (at its
            // first row), each operand split just before its products
            const int row = 16 * I + lr, k = 16 * I + 4 * lq;
            {
                f32x4 br;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int s = 16 * I + 4 * lq + j;
                    br[j] = kval(s) * exp2_fast(glast - GmL[s * LK + d]);
                }
                bf16x4 bh, bl;
                split4(br, bh, bl);
                f32x4 yq = {0.f, 0.f, 0.f, 0.f}, yk = yq;
                yq = mma16_3(pair_frag(aH, row, k), pair_frag(aL, row, k), bh, bl, yq);
                yk = mma16_3(pair_frag(mH, row, k), pair_frag(mL, row, k), bh, bl, yk);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const float fr = exp2_fast(GmL[(16 * I + 4 * lq + rr) * LK + d] - glast);
                    aq[rr] = fmaf(fr, yq[rr], aq[rr]);
                    akr[rr] = fmaf(fr, yk[rr], akr[rr]);
                }
            }
            {
                f32x4 bq, bk;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int s = 16 * I + 4 * lq + j;
                    const float fc = exp2_fast(GmL[s * LK + d] - gfirst);
                    bq[j] = qval(s) * fc;
                    bk[j] = kval(s) * fc;
                }
                bf16x4 bqh, bql, bkh, bkl;
                split4(bq, bqh, bql);
                split4(bk, bkh, bkl);
                f32x4 yc = {0.f, 0.f, 0.f, 0.f};
                yc = mma16_3(pair_frag(atH, row, k), pair_frag(atL, row, k), bqh, bql, yc);
                yc = mma16_3(pair_frag(mtH, row, k), pair_frag(mtL, row, k), bkh, bkl, yc);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    akc[rr] = fmaf(exp2_fast(gfirst - GmL[(16 * I + 4 * lq + rr) * LK + d]), yc[rr], akc[rr]);
            }
        } else {
            // (rare: operands read from LDS inside the loop, dAqk and dM as hi + lo)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int r = 16 * I + 4 * lq + rr;
                const float gr = GmL[r * LK + d];
                float xq = 0.f, xk = 0.f, xc = 0.f;
#pragma unroll 4
                for (int j = 0; j < 16; ++j) {
                    const int s = 16 * I + j;
                    const float kb = kval(s), qb = qval(s);
                    // row side (s <= r): 2^min(x, 0); column side (s >= r): 2^min(-x, 0)
                    const float x = gr - GmL[s * LK + d];
                    const float t2 = exp2_fast(-fabsf(x));
                    const float er = x <= 0.f ? t2 : 1.f;
                    const float ec = x >= 0.f ? t2 : 1.f;
                    const float ek = kb * er;
                    const float a_rs = (float)aH[r * TP + s] + (float)aL[r * TP + s];
                    const float m_rs = (float)mH[r * TP + s] + (float)mL[r * TP + s];
                    const float a_sr = (float)aH[s * TP + r] + (float)aL[s * TP + r];
                    const float m_sr = (float)mH[s * TP + r] + (float)mL[s * TP + r];
                    xq = fmaf(a_rs, ek, xq);
                    xk = fmaf(m_rs, ek, xk);
                    xc = fmaf(fmaf(a_sr, qb, m_sr * kb), ec, xc);
                }
                aq[rr] += xq;
                akr[rr] += xk;
                akc[rr] += xc;
            }
        }
        // elementwise terms of qg, kd, kg; dGamma; dq, dk per value head
        float dqg[4], dkg[4], dkd[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            dqg[rr] = dqgR[rr];
            dkg[rr] = dkgR[rr];
            dkd[rr] = dkdR[rr];
        }
        if (ib == 0) load_grads(I + 1);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int r = 16 * I + 4 * lq + rr;
            const float qv = qval(r), kv = kval(r), gr = GmL[r * LK + d];
            const float e1 = exp2_fast(gr), e2 = exp2_fast(Gd - gr);
            const float dqi = aq[rr], dkr = akr[rr], dkc = akc[rr];
            const float dq = fmaf(sc * e1, dqg[rr], dqi);
            const float dk = dkr + dkc + e1 * dkd[rr] + e2 * dkg[rr];
            const float kge = kv * e2 * dkg[rr];
            dgam[ib][rr] = LN2F * (qv * dq + kv * (dkr - dkc + e1 * dkd[rr]) - kge);
            if (r < len) {
                dgk += kge;
                const size_t row = (size_t)(pos.x + r);
                if (p.pair_gva) {
                    // the running sum over the value heads (each lane reads back only
                    // what it wrote for the value head before)
                    float* sq = p.dq_hv + (row * p.HV + h * grp) * K + d;
                    float* sk = p.dk_hv + (row * p.HV + h * grp) * K + d;
                    const float aq_ = g > 0 ? *sq + dq : dq, ak_ = g > 0 ? *sk + dk : dk;
                    if (g + 1 < ng) {
                        *sq = aq_;
                        *sk = ak_;
                    } else {
                        dqo[(row * p.H + h) * K + d] = (__bf16)aq_;
                        dko[(row * p.H + h) * K + d] = (__bf16)ak_;
                    }
                } else {
                    p.dq_hv[(row * p.HV + hv) * K + d] = dq;
                    p.dk_hv[(row * p.HV + hv) * K + d] = dk;
                }
            }
        }
    }
    // the four lanes of channel d (lq = 0..3) summed in a fixed order
    dgk += __shfl_xor(dgk, 16, 64);
    dgk += __shfl_xor(dgk, 32, 64);
    if (lq == 0) dGP[half][d] = LN2F * dgk;
    __syncthreads();   // the operand tiles become dGamma
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            dGam[(16 * (2 * half + ib) + 4 * lq + rr) * LK + d] = dgam[ib][rr];
    __syncthreads();
    // dg = reverse cumsum of dGamma over the chunk's rows (rows >= len left out); dG
    // joins at the last row. Runs of RL rows per thread, as in the forward cumsum.
    {
        constexpr int NS = NTH / K, RL = C / NS;
        const int dc = tid % K, sg = tid / K;
        float x[RL];
        float acc = 0.f;
#pragma unroll
        for (int i = RL - 1; i >= 0; --i) {
            const int r = sg * RL + i;
            acc += r < len ? dGam[r * LK + dc] : 0.f;
            x[i] = acc;
        }
        runT[sg * K + dc] = acc;
        __syncthreads();
        float off = dGL[dc] + dGP[0][dc] + dGP[1][dc];
        for (int j = NS - 1; j > sg; --j) off += runT[j * K + dc];
#pragma unroll
        for (int i = 0; i < RL; ++i) {
            const int r = sg * RL + i;
            if (r < len) p.dg[((size_t)(pos.x + r) * p.HV + hv) * K + dc] = x[i] + off;
        }
    }
    __syncthreads();   // this value head's LDS reads are done before the next one's stores
    }
}

// ------------------------------------------------------------------------------------
// GVA: dq, dk of a q/k head are the sums over its value heads; per (chunk, q/k head)
// ------------------------------------------------------------------------------------
template <int K, typename TIn>
__global__ __launch_bounds__(BT) void bwd_reduce_kernel(BwdParams p) {
    const int G = p.NCmax * p.H;
    const int item = blockIdx.x;
    if (item >= G) return;
    const int h = item % p.H, c = item / p.H;
    if (!p.dense && c >= p.nchunks[0]) return;
    const int2 pos = chunk_pos(p.dense, p.NT, p.T, p.table, c);
    const int grp = p.HV / p.H;
    TIn* dq = reinterpret_cast<TIn*>(p.dq);
    TIn* dk = reinterpret_cast<TIn*>(p.dk);
    for (int e = threadIdx.x; e < pos.y * K; e += BT) {
        const int r = e / K, d = e % K;
        const size_t row = (size_t)(pos.x + r);
        float sq = 0.f, sk = 0.f;
        for (int j = 0; j < grp; ++j) {
            sq += p.dq_hv[(row * p.HV + h * grp + j) * K + d];
            sk += p.dk_hv[(row * p.HV + h * grp + j) * K + d];
        }
        dq[(row * p.H + h) * K + d] = from_f32<TIn>(sq);
        dk[(row * p.H + h) * K + d] = from_f32<TIn>(sk);
    }
}


// Grid of a persistent kernel (one block per CU, each looping over its items): the
// current device's CU count, at most `items`.
long long persistent_blocks(long long items) {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    int n = dev >= 0 && dev < 64 ? cus[dev].load(std::memory_order_relaxed) : 0;
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        if (dev >= 0 && dev < 64) cus[dev].store(n, std::memory_order_relaxed);
    }
    return items < n ? items : n;
}

template <int K, int V, typename TIn, typename TB>
hipError_t launch_bwd_kv(const ChunkBwdArgs& a, const ChunkBwdLayout& L) {
    char* ws = reinterpret_cast<char*>(a.workspace);
    const bool dense = a.cu_seqlens == nullptr;
    const int NT = (a.T + C - 1) / C;
    // forward recompute: schedule (packed), records, and the re-scan with checkpoints (a
    // training forward also writes o and the final state; a backward from its workspace
    // skips this)
    if (a.mode != BWD_FROM_SAVED) {
        ChunkArgs f;
        f.q = a.q; f.k = a.k; f.v = a.v; f.g = a.g; f.beta = a.beta;
        f.in = a.in;   // the recompute runs with the forward's fused options
        f.initial_state = a.initial_state; f.cu_seqlens = a.cu_seqlens;
        const bool fwd = a.mode == BWD_FORWARD;
        f.o = fwd ? a.fwd_o : nullptr;
        f.final_state = fwd ? a.fwd_final_state : nullptr;
        f.N = a.N; f.B = a.B; f.T = a.T; f.H = a.H; f.HV = a.HV; f.K = a.K; f.V = a.V;
        f.qkv_dtype = a.qkv_dtype; f.beta_dtype = a.beta_dtype; f.scale = a.scale;
        f.workspace = a.workspace; f.workspace_bytes = a.workspace_bytes;
        f.dev_status = a.dev_status; f.stream = a.stream; f.events = nullptr;
        f.h_out = reinterpret_cast<float*>(ws + L.off_h);
        f.vn_out = reinterpret_cast<float*>(ws + L.off_vn);
        f.m_out = reinterpret_cast<float*>(ws + L.off_mt);                        // [items][64][64]
        f.t_out = f.m_out + (size_t)L.fwd.NCmax * a.HV * (C * C);                  // [items][64][64]
        hipError_t err = launch_chunk(f, L.fwd);
        if (err != hipSuccess || fwd) return err;
    }
    hipError_t err = hipSuccess;

    BwdParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.g = a.g; p.beta = a.beta; p.dout = a.dout; p.dht = a.dht;
    p.dq = a.dq; p.dk = a.dk; p.dv = a.dv; p.dg = a.dg; p.dbeta = a.dbeta; p.dh0 = a.dh0;
    if (!dense) {
        const int32_t* coff = reinterpret_cast<const int32_t*>(ws);
        p.coff = coff; p.cend = coff + a.N; p.slot_ok = coff + 2 * a.N; p.nchunks = coff + 3 * a.N;
        p.table = reinterpret_cast<const int2*>(ws + sched_table_offset(a.N));
        p.order = reinterpret_cast<const int32_t*>(ws + sched_order_offset(a.N, L.fwd.NCmax));
    } else {
        p.coff = p.cend = p.slot_ok = p.nchunks = p.order = nullptr;
        p.table = nullptr;
    }
    p.dense = dense; p.NT = NT; p.T = a.T; p.N = a.N; p.H = a.H; p.HV = a.HV; p.NCmax = L.fwd.NCmax;
    p.scale = a.scale;
    p.rec = ws + L.fwd.sched_bytes;
    p.rec_bytes = L.fwd.rec_bytes; p.off_w = L.fwd.off_w; p.off_u = L.fwd.off_u; p.off_qg = L.fwd.off_qg;
    p.off_kgT = L.fwd.off_kgT; p.off_aqk = L.fwd.off_aqk; p.off_eg = L.fwd.off_eg;
    p.h = reinterpret_cast<const float*>(ws + L.off_h);
    p.vn = reinterpret_cast<const float*>(ws + L.off_vn);
    p.mt = reinterpret_cast<const float*>(ws + L.off_mt);
    p.dh = reinterpret_cast<float*>(ws + L.off_dh);
    p.dvn = reinterpret_cast<float*>(ws + L.off_dvn);
    p.sops = reinterpret_cast<float*>(ws + L.off_sops);
    p.gs = reinterpret_cast<float*>(ws + L.off_gs);
    p.wy = reinterpret_cast<float*>(ws + L.off_wy);
    p.dq_hv = reinterpret_cast<float*>(ws + L.off_dq);
    p.dk_hv = reinterpret_cast<float*>(ws + L.off_dk);
    p.in = a.in;
    p.dbeta_f32 = a.dbeta_f32;

    const long long chains = (long long)a.N * a.HV;
    const long long nchunk_items = (long long)L.fwd.NCmax * a.HV;
    if (nchunk_items > 0) {
        // the records are in the input type (bf16 hi/lo pairs, or fp32)
        if constexpr (sizeof(TIn) == 2)
            hipLaunchKernelGGL((bwd_prep_bf16_kernel<K, V>), dim3((unsigned)nchunk_items), dim3(BT), 0, a.stream, p);
        else
            hipLaunchKernelGGL((bwd_prep_kernel<K, V, TIn, TIn>), dim3((unsigned)nchunk_items), dim3(BT), 0, a.stream, p);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (chains > 0) {
        if constexpr (sizeof(TIn) == 2)
            hipLaunchKernelGGL((bwd_scan_bf16_kernel<K, V>), dim3((unsigned)(chains * (V / 16))), dim3(BT), 0, a.stream, p);
        else
            hipLaunchKernelGGL((bwd_scan_kernel<K, V>), dim3((unsigned)(chains * (V / 16))), dim3(BT), 0, a.stream, p);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (nchunk_items > 0) {
        if constexpr (sizeof(TIn) == 2)
            hipLaunchKernelGGL((bwd_state_bf16_kernel<K, V>), dim3((unsigned)nchunk_items), dim3(SB_THREADS), 0, a.stream, p);
        else
            hipLaunchKernelGGL((bwd_state_kernel<K, V, TIn>), dim3((unsigned)nchunk_items), dim3(BT), 0, a.stream, p);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        if constexpr (sizeof(TIn) == 2) {
            if (p.in.gate_mode == GATE_RAW_BF16)
                hipLaunchKernelGGL((bwd_wy_bf16_kernel<K, V, TB, __bf16>), dim3((unsigned)persistent_blocks(nchunk_items)),
                                   dim3(WY_THREADS), 0, a.stream, p);
            else
                hipLaunchKernelGGL((bwd_wy_bf16_kernel<K, V, TB, float>), dim3((unsigned)persistent_blocks(nchunk_items)),
                                   dim3(WY_THREADS), 0, a.stream, p);
        }
        else
            hipLaunchKernelGGL((bwd_wy_kernel<K, V, TIn, TB>), dim3((unsigned)nchunk_items), dim3(WY_THREADS), 0, a.stream, p);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        // bf16 inputs without a following chain rule: the pair kernel sums dq, dk over the
        // value heads itself (one block per chunk and q/k head), no separate reduction
        const bool pair_gva = sizeof(TIn) == 2 && !a.skip_reduce;
        p.pair_gva = pair_gva ? 1 : 0;
        if constexpr (sizeof(TIn) == 2)
            hipLaunchKernelGGL((bwd_pair_bf16_kernel<K, V>),
                               dim3((unsigned)(pair_gva ? (long long)L.fwd.NCmax * a.H : nchunk_items)),
                               dim3(pair_threads<K>()), 0, a.stream, p);
        else
            hipLaunchKernelGGL((bwd_pair_kernel<K, V, TIn>), dim3((unsigned)nchunk_items), dim3(pair_threads<K>()), 0,
                               a.stream, p);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        if (!a.skip_reduce && !pair_gva) {
            hipLaunchKernelGGL((bwd_reduce_kernel<K, TIn>), dim3((unsigned)((long long)L.fwd.NCmax * a.H)), dim3(BT), 0,
                               a.stream, p);
            if ((err = hipGetLastError()) != hipSuccess) return err;
        }
    }
    return hipSuccess;
}

template <typename TIn, typename TB>
hipError_t launch_bwd_t(const ChunkBwdArgs& a, const ChunkBwdLayout& L) {
    if (a.K == 128) return a.V == 128 ? launch_bwd_kv<128, 128, TIn, TB>(a, L) : launch_bwd_kv<128, 64, TIn, TB>(a, L);
    return a.V == 128 ? launch_bwd_kv<64, 128, TIn, TB>(a, L) : launch_bwd_kv<64, 64, TIn, TB>(a, L);
}

size_t align256b(size_t x) { return (x + 255) / 256 * 256; }

// ------------------------------------------------------------------------------------
// backward of the fused input options (gate activation, q/k L2 norm, beta sigmoid): the
// chunked backward applies the options to the inputs it stages (in fp32, as the fused
// forward does), and the chain rule of each option is applied to its gradients after.
// ------------------------------------------------------------------------------------
struct PostParams {
    const void* q;           // raw inputs
    const void* k;
    const void* g;
    const void* beta;
    InputSpec in;
    int gate_bf16;
    const float* dq_hv;      // [rows][HV][K] per value head, from the chunked backward
    const float* dk_hv;
    const float* dg2;        // [rows][HV][K] with respect to the log2 gate
    const float* dba;        // [rows][HV] with respect to the activated beta
    void* dq;                // outputs
    void* dk;
    float* dg;
    void* dbeta;
    float* part;             // [NCmax][HV][K + 1]: ddt_bias and dA_log partial sums per chunk
    float* dA_log;
    float* ddt_bias;
    const int32_t* nchunks;
    const int2* table;
    int dense, NT, T, H, HV, NCmax;
};

// dq, dk: the sum over each q/k head's value heads, then the L2-norm backward
// r (dy - y (y . dy)); one wave per (row, head), per chunk
template <int K, typename TIn>
__global__ __launch_bounds__(256) void bwd_post_qk_kernel(PostParams p) {
    constexpr int NE = K / 64;
    const int c = blockIdx.x / p.H, h = blockIdx.x % p.H;
    if (!p.dense && c >= p.nchunks[0]) return;
    const int2 pos = chunk_pos(p.dense, p.NT, p.T, p.table, c);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = p.HV / p.H;
    for (int r = wave; r < pos.y; r += 4) {
        const size_t row = (size_t)(pos.x + r);
        for (int which = 0; which < 2; ++which) {
            const float* src = which ? p.dk_hv : p.dq_hv;
            const TIn* x_in = reinterpret_cast<const TIn*>(which ? p.k : p.q);
            TIn* out = reinterpret_cast<TIn*>(which ? p.dk : p.dq);
            const bool norm = which ? p.in.l2norm_k : p.in.l2norm_q;
            float dy[NE], y[NE];
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                const int d = lane + 64 * e;
                float acc = 0.f;
                for (int j = 0; j < grp; ++j) acc += src[(row * p.HV + h * grp + j) * K + d];
                dy[e] = acc;
                y[e] = to_f32(x_in[(row * p.H + h) * K + d]);
                ss = fmaf(y[e], y[e], ss);
            }
            if (norm) {
#pragma unroll
                for (int m = 1; m < 64; m <<= 1) ss += __shfl_xor(ss, m, 64);
                const float rn = l2norm_rstd(ss);
                float yd = 0.f;
#pragma unroll
                for (int e = 0; e < NE; ++e) { y[e] *= rn; yd = fmaf(y[e], dy[e], yd); }
#pragma unroll
                for (int m = 1; m < 64; m <<= 1) yd += __shfl_xor(yd, m, 64);
#pragma unroll
                for (int e = 0; e < NE; ++e) dy[e] = rn * (dy[e] - y[e] * yd);
            }
#pragma unroll
            for (int e = 0; e < NE; ++e) out[(row * p.H + h) * K + lane + 64 * e] = from_f32<TIn>(dy[e]);
        }
    }
}

// the raw gate's and beta's gradients per (chunk, value head), with this chunk's partial
// sums of ddt_bias (per channel) and dA_log
template <int K, typename TB>
__global__ __launch_bounds__(K) void bwd_post_gb_kernel(PostParams p) {
    const int c = blockIdx.x / p.HV, hv = blockIdx.x % p.HV;
    if (!p.dense && c >= p.nchunks[0]) return;
    const int2 pos = chunk_pos(p.dense, p.NT, p.T, p.table, c);
    const int d = threadIdx.x;
    const bool raw = p.in.gate_mode != GATE_LOG2;
    float sdt = 0.f, sA = 0.f;
    const float eA = raw ? expf(p.in.A_log[hv]) : 0.f;
    for (int r = 0; r < pos.y; ++r) {
        const size_t e = ((size_t)(pos.x + r) * p.HV + hv) * K + d;
        if (raw) {
            float x = p.gate_bf16 ? (float)static_cast<const __bf16*>(p.g)[e] : static_cast<const float*>(p.g)[e];
            if (p.in.dt_bias) x += p.in.dt_bias[(size_t)hv * K + d];
            const float sp = x > 15.f ? x : log1pf(expf(x));      // softplus
            const float gn = -eA * sp;                               // natural-log activation
            const bool clamped = p.in.has_lower_bound && gn < p.in.lower_bound;
            const float dgn = clamped ? 0.f : p.dg2[e] * LOG2E;      // d/dgn of the log2 value is 1/ln 2
            const float sig = 1.f / (1.f + expf(-x));
            const float dx = -eA * sig * dgn;
            p.dg[e] = dx;
            sdt += dx;
            sA = fmaf(dgn, gn, sA);
        }
        if (d == 0 && p.in.beta_sig != 0.f) {
            const size_t eb = (size_t)(pos.x + r) * p.HV + hv;
            const float b = to_f32(reinterpret_cast<const TB*>(p.beta)[eb]);
            const float sb = 1.f / (1.f + expf(-b));
            reinterpret_cast<TB*>(p.dbeta)[eb] = from_f32<TB>(p.dba[eb] * p.in.beta_sig * sb * (1.f - sb));
        }
    }
    if (raw) {
        float* pp = p.part + ((size_t)c * p.HV + hv) * (K + 1);
        pp[d] = sdt;
        // dA_log partial: the block's sum over channels
        __shared__ float red[K];
        red[d] = sA;
        __syncthreads();
        if (d == 0) {
            float t = 0.f;
            for (int i = 0; i < K; ++i) t += red[i];
            pp[K] = t;
        }
    }
}

// dA_log and ddt_bias: the chunk partials summed in chunk order (deterministic)
template <int K>
__global__ __launch_bounds__(K + 1) void bwd_gate_sum_kernel(PostParams p) {
    const int hv = blockIdx.x, j = threadIdx.x;
    const int nc = p.dense ? p.NCmax : p.nchunks[0];
    float t = 0.f;
    for (int c = 0; c < nc; ++c) t += p.part[((size_t)c * p.HV + hv) * (K + 1) + j];
    if (j < K) {
        if (p.ddt_bias) p.ddt_bias[(size_t)hv * K + j] = t;
    } else {
        p.dA_log[hv] = t;
    }
}

template <int K, typename TIn, typename TB>
hipError_t launch_bwd_ex_k(const ChunkBwdExArgs& x, const ChunkBwdExLayout& L) {
    const ChunkBwdArgs& a = x.core;
    char* ws = reinterpret_cast<char*>(a.workspace);
    hipError_t err;
    // the chunked backward with the options applied to its staged inputs, into fp32
    // gradients where a chain rule follows (dq, dk per value head; the log2 gate's and
    // the activated beta's gradients)
    ChunkBwdArgs c = a;
    c.in = x.in;
    const bool raw = x.in.gate_mode != GATE_LOG2, sig = x.in.beta_sig != 0.f;
    c.g = raw ? nullptr : a.g;
    c.dg = raw ? reinterpret_cast<float*>(ws + L.off_dg2) : a.dg;
    if (sig) {
        c.dbeta = ws + L.off_dba;
        c.dbeta_f32 = true;
    }
    c.skip_reduce = true;
    err = launch_chunk_bwd(c, L.core);
    if (err != hipSuccess || a.mode == BWD_FORWARD) return err;   // a training forward ends there

    PostParams q;
    q.q = a.q; q.k = a.k; q.g = x.g; q.beta = a.beta; q.in = x.in; q.gate_bf16 = x.gate_bf16;
    q.dq_hv = reinterpret_cast<const float*>(ws + L.core.off_dq);
    q.dk_hv = reinterpret_cast<const float*>(ws + L.core.off_dk);
    q.dg2 = reinterpret_cast<const float*>(ws + L.off_dg2);
    q.dba = reinterpret_cast<const float*>(ws + L.off_dba);
    q.dq = a.dq; q.dk = a.dk; q.dg = a.dg; q.dbeta = a.dbeta;
    q.part = reinterpret_cast<float*>(ws + L.off_part);
    q.dA_log = x.dA_log; q.ddt_bias = x.ddt_bias;
    const bool dense = a.cu_seqlens == nullptr;
    q.nchunks = dense ? nullptr : reinterpret_cast<const int32_t*>(ws) + 3 * a.N;
    q.table = dense ? nullptr : reinterpret_cast<const int2*>(ws + sched_table_offset(a.N));
    q.dense = dense; q.NT = (a.T + C - 1) / C; q.T = a.T; q.H = a.H; q.HV = a.HV; q.NCmax = L.core.fwd.NCmax;
    const long long nc = (long long)L.core.fwd.NCmax;
    if (nc > 0) {
        hipLaunchKernelGGL((bwd_post_qk_kernel<K, TIn>), dim3((unsigned)(nc * a.H)), dim3(256), 0, a.stream, q);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        if (raw || sig) {
            hipLaunchKernelGGL((bwd_post_gb_kernel<K, TB>), dim3((unsigned)(nc * a.HV)), dim3(K), 0, a.stream, q);
            if ((err = hipGetLastError()) != hipSuccess) return err;
        }
        if (raw) {
            hipLaunchKernelGGL((bwd_gate_sum_kernel<K>), dim3((unsigned)a.HV), dim3(K + 1), 0, a.stream, q);
            if ((err = hipGetLastError()) != hipSuccess) return err;
        }
    }
    return hipSuccess;
}

}  // namespace

bool chunk_bwd_layout(int B, int T, int HV, int K, int V, int N, bool packed, int qkv_dtype,
                      ChunkBwdLayout* out) {
    ChunkBwdLayout L{};
    if (!chunk_layout(B, T, HV, K, V, N, packed, qkv_dtype, &L.fwd, true)) return false;
    const size_t items = (size_t)HV * L.fwd.NCmax;
    const size_t rows = (size_t)B * T;
    size_t off = align256b(L.fwd.total);
    L.off_h = off;   off = align256b(off + items * K * V * 4);
    L.off_vn = off;  off = align256b(off + items * C * V * 4);
    L.off_mt = off;  off = align256b(off + items * (size_t)(2 * C * C) * 4);
    L.off_dh = off;  off = align256b(off + items * K * V * 4);
    L.off_dvn = off; off = align256b(off + items * C * V * 4);
    L.off_sops = off; off = align256b(off + items * (size_t)(2 * C * K + C * V + K * V) * 4);
    L.off_gs = off;  off = align256b(off + items * (size_t)(3 * C * K + C * C + K) * 4);
    L.off_wy = off;  off = align256b(off + items * (size_t)(C * K + C * C) * 4);
    L.off_dq = off;  off = align256b(off + rows * HV * K * 4);
    L.off_dk = off;  off = align256b(off + rows * HV * K * 4);
    L.total = off;
    *out = L;
    return true;
}

bool chunk_bwd_ex_layout(int B, int T, int H, int HV, int K, int V, int N, bool packed, int qkv_dtype,
                         ChunkBwdExLayout* out) {
    ChunkBwdExLayout L{};
    if (!chunk_bwd_layout(B, T, HV, K, V, N, packed, qkv_dtype, &L.core)) return false;
    const size_t rows = (size_t)B * T;
    size_t off = align256b(L.core.total);
    L.off_dg2 = off;  off = align256b(off + rows * HV * K * 4);
    L.off_dba = off;  off = align256b(off + rows * HV * 4);
    L.off_part = off; off = align256b(off + (size_t)L.core.fwd.NCmax * HV * (K + 1) * 4);
    L.total = off;
    *out = L;
    return true;
}

hipError_t launch_chunk_bwd_ex(const ChunkBwdExArgs& x, const ChunkBwdExLayout& L) {
    const ChunkBwdArgs& a = x.core;
    if (a.qkv_dtype == KDA_BF16) {
        if (a.beta_dtype == KDA_BF16)
            return a.K == 128 ? launch_bwd_ex_k<128, __bf16, __bf16>(x, L) : launch_bwd_ex_k<64, __bf16, __bf16>(x, L);
        return a.K == 128 ? launch_bwd_ex_k<128, __bf16, float>(x, L) : launch_bwd_ex_k<64, __bf16, float>(x, L);
    }
    if (a.beta_dtype == KDA_BF16)
        return a.K == 128 ? launch_bwd_ex_k<128, float, __bf16>(x, L) : launch_bwd_ex_k<64, float, __bf16>(x, L);
    return a.K == 128 ? launch_bwd_ex_k<128, float, float>(x, L) : launch_bwd_ex_k<64, float, float>(x, L);
}

hipError_t launch_chunk_bwd(const ChunkBwdArgs& a, const ChunkBwdLayout& L) {
    if (a.qkv_dtype == KDA_BF16)
        return a.beta_dtype == KDA_BF16 ? launch_bwd_t<__bf16, __bf16>(a, L) : launch_bwd_t<__bf16, float>(a, L);
    return a.beta_dtype == KDA_BF16 ? launch_bwd_t<float, __bf16>(a, L) : launch_bwd_t<float, float>(a, L);
}

}  // namespace kda
