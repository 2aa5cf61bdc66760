// Chunked KDA forward for gfx950: the chunk algebra of "kernel-fun 0.2.0.dev1 sdist",
// ALGORITHM.md, section Forward, in three kernels.
//
//  sched   (packed mode only, one block) validates the int32 offsets per slot and lays
//          out the chunks: each slot is cut into 64-row chunks starting at its first
//          row, the last one short.
//  intra   one block per (chunk, value head): Stage 1 (chunk-local cumsum of the log2
//          gate) and Stage 2 (Aqk, the WY inverse (I + L)^-1 with beta in L, and
//          w, u, qg, kg, 2^G), written as one record per (value head, chunk).
//  scan    one block per (sequence, value head, BV-column slice of V): Stage 3+4, the
//          serial walk over the sequence's chunks with the fp32 [K, BV] state held in
//          matrix-core accumulators; only o (and the final state) reach HBM.
//
// Numerics of Stage 2 (the page's sub-chunk rule). The gate sits inside the Aqk / L dot
// products, 2^(G_i - G_j) per channel, so it cannot be factored out of one product
// without a factor 2^(+G) that is unbounded. Rows are split into four 16-row blocks;
// block row I uses one anchor row m_I and the operands q_i 2^(G_i - G_m), k_i 2^(G_i -
// G_m) (rows of block I) and k_j 2^(G_m - G_j) (rows j of blocks 0..I). With m_I the
// middle row of block I, every factor that can exceed 1 spans at most 8 rows of decay;
// the kernel checks that bound per chunk and, when a block's half-spread exceeds
// 100 log2 units (2^100 stays far from fp32 overflow), switches that chunk to block-
// boundary anchors (all factors <= 1: safe at any gate magnitude) for the off-diagonal
// blocks and an exact one-sided 2^(G_i - G_j) per (i, j, channel) for the diagonal ones.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int C = 64;            // chunk rows
constexpr int NTHREADS = 256;
constexpr float SPREAD_LIMIT = 100.0f;

// byte offset of the chunk table inside the packed-mode schedule
inline size_t sched_table_offset(int N) { return ((size_t)(3 * (size_t)N + 1) * 4 + 15) / 16 * 16; }

__device__ __forceinline__ int xcd_remap(int b, int G) {
    // blocks are dealt round-robin to the 8 XCDs; give each XCD a contiguous run of
    // work items so neighbouring items (same chain, same chunk) share an L2
    if (G % 8 != 0) return b;
    return (b % 8) * (G / 8) + b / 8;
}

// ------------------------------------------------------------------------------------
// sched: per-slot validation, chunk offsets and the chunk table (packed mode)
// ------------------------------------------------------------------------------------
// Each slot is checked on its own (0 <= bos <= eos <= T, slot 0 starts at 0). Offsets that
// decrease always break some slot's check; the slots that pass may then overlap, so the
// chunk count is also capped at the table's capacity NCmax: a slot whose chunks would
// not fit is skipped and flagged like a malformed one. Entries past n_chunks are never
// read.
__global__ __launch_bounds__(1024) void sched_kernel(const int32_t* __restrict__ cu, int N,
                                                     int T, int NCmax,
                                                     int32_t* __restrict__ coff,
                                                     int32_t* __restrict__ cend,
                                                     int32_t* __restrict__ slot_ok,
                                                     int32_t* __restrict__ nchunks,
                                                     int2* __restrict__ table,
                                                     int32_t* dev_status) {
    __shared__ int scan[1024];
    __shared__ int used;
    const int tid = threadIdx.x;
    if (tid == 0) used = 0;
    long long carry = 0;
    for (int base = 0; base < N; base += 1024) {
        const int n = base + tid;
        int bos = 0, len = 0, cnt = 0, ok = 0;
        if (n < N) {
            bos = cu[n];
            const int eos = cu[n + 1];
            ok = bos >= 0 && bos <= eos && eos <= T && (n != 0 || bos == 0);
            if (ok) {
                len = eos - bos;
                cnt = (len + C - 1) / C;
            }
        }
        scan[tid] = cnt;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            const int x = tid >= off ? scan[tid - off] : 0;
            __syncthreads();
            scan[tid] += x;
            __syncthreads();
        }
        const int incl = scan[tid];
        const int total = scan[1023];
        __syncthreads();
        if (n < N) {
            const long long first = carry + incl - cnt;
            if (ok && first + cnt > NCmax) ok = 0;
            if (!ok && dev_status) atomicOr(dev_status, KDA_DEV_BAD_CU_SEQLENS);
            slot_ok[n] = ok;
            coff[n] = ok ? (int)first : 0;
            cend[n] = ok ? (int)(first + cnt) : 0;
            if (ok) {
                for (int i = 0; i < cnt; ++i) {
                    const int l = len - i * C < C ? len - i * C : C;
                    table[first + i] = make_int2(bos + i * C, l);
                }
                atomicMax(&used, (int)(first + cnt));
            }
        }
        carry += total;
        __syncthreads();
    }
    __syncthreads();
    if (tid == 0) nchunks[0] = used;
}

// ------------------------------------------------------------------------------------
// intra: Stage 1 + Stage 2 for one (chunk, value head)
// ------------------------------------------------------------------------------------
struct IntraParams {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const void* beta;
    const int32_t* nchunks;   // packed mode: device chunk count (else NULL)
    const int2* table;        // packed mode: chunk table
    char* rec;                // record base
    size_t rec_bytes, off_w, off_u, off_qg, off_kgT, off_aqk, off_eg;
    int T, H, HV, NT, NCmax;
    float scale;
};

template <int K, int V, typename TIn, typename TB>
__global__ __launch_bounds__(NTHREADS) void intra_kernel(IntraParams p) {
    typedef TIn TW;                        // intermediate / operand type
    constexpr int RG = NTHREADS / K;       // row groups of the elementwise mapping
    constexpr int RPT = C / RG;            // rows per thread (16 or 32)
    constexpr int RGV = NTHREADS / V;
    constexpr int RPTV = C / RGV;
    typedef Tile<TW, 16, K> TQ;            // one 16-row block of q-side / k-row operands
    typedef Tile<TW, C, K> TKC;            // k-column operands of a block row
    typedef Tile<TW, C, C> TB64;           // T beta
    typedef Tile<TW, K, C> TKD;            // (k 2^G)^T
    typedef Tile<TW, V, C> TVT;            // v^T
    constexpr int LD = C + 1;              // fp32 64x64 matrices, padded rows
    // bf16 operands carry a second "lo" tile holding what bf16 rounded away
    constexpr bool SPLIT = sizeof(TW) == 2;
    constexpr int NSPLIT = SPLIT ? 2 : 1;

    constexpr int P2_BYTES = NSPLIT * (2 * TQ::BYTES + TKC::BYTES);
    constexpr int P4_BYTES = TB64::BYTES + TKD::BYTES + TVT::BYTES;
    constexpr int GM_BYTES = C * K * 4;
    constexpr int XS_BYTES = 3 * 16 * 17 * 4;
    constexpr int U1 = P2_BYTES > P4_BYTES ? P2_BYTES : P4_BYTES;
    constexpr int U2 = U1 > GM_BYTES ? U1 : GM_BYTES;
    constexpr int UNION_BYTES = U2 > XS_BYTES ? U2 : XS_BYTES;

    __shared__ float gsum[4][128];
    __shared__ float anch[4][128];
    __shared__ float Lm[C * LD];
    __shared__ float Tm[C * LD];
    __shared__ float betas[C];
    __shared__ __attribute__((aligned(16))) char un[UNION_BYTES];

    TW* QH = reinterpret_cast<TW*>(un);
    TW* KR = reinterpret_cast<TW*>(un + TQ::BYTES);
    TW* KC = reinterpret_cast<TW*>(un + 2 * TQ::BYTES);
    TW* QHl = reinterpret_cast<TW*>(un + (2 * TQ::BYTES + TKC::BYTES));
    TW* KRl = reinterpret_cast<TW*>(un + (3 * TQ::BYTES + TKC::BYTES));
    TW* KCl = reinterpret_cast<TW*>(un + (4 * TQ::BYTES + TKC::BYTES));
    TW* TBs = reinterpret_cast<TW*>(un);
    TW* KDt = reinterpret_cast<TW*>(un + TB64::BYTES);
    TW* VTt = reinterpret_cast<TW*>(un + TB64::BYTES + TKD::BYTES);
    float* GM = reinterpret_cast<float*>(un);
    float* Xs = reinterpret_cast<float*>(un);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int G = p.NCmax * p.HV;
    const int item = xcd_remap(blockIdx.x, G);
    const int hv = item % p.HV;
    const int c = item / p.HV;
    const int h = hv / (p.HV / p.H);

    long long rs;   // first row of the chunk in the [B*T] row space
    int len;
    if (p.table) {
        if (c >= p.nchunks[0]) return;
        const int2 e = p.table[c];
        rs = e.x;
        len = e.y;
    } else {
        const int b = c / p.NT, ci = c % p.NT;
        rs = (long long)b * p.T + (long long)ci * C;
        len = p.T - ci * C < C ? p.T - ci * C : C;
    }
    const TIn* q = reinterpret_cast<const TIn*>(p.q);
    const TIn* k = reinterpret_cast<const TIn*>(p.k);
    const TIn* v = reinterpret_cast<const TIn*>(p.v);
    const TB* beta = reinterpret_cast<const TB*>(p.beta);
    char* rec = p.rec + ((size_t)hv * p.NCmax + c) * p.rec_bytes;
    TW* out_w = reinterpret_cast<TW*>(rec + p.off_w);
    float* out_u = reinterpret_cast<float*>(rec + p.off_u);
    TW* out_qg = reinterpret_cast<TW*>(rec + p.off_qg);
    TW* out_kgT = reinterpret_cast<TW*>(rec + p.off_kgT);
    TW* out_aqk = reinterpret_cast<TW*>(rec + p.off_aqk);
    TW* out_aqk_lo = out_aqk + C * C;             // residual tile (bf16 path)
    float* out_eg = reinterpret_cast<float*>(rec + p.off_eg);
    auto put_aqk = [&](int idx, float val) {
        const TW hi = from_f32<TW>(val);
        out_aqk[idx] = hi;
        if constexpr (SPLIT) out_aqk_lo[idx] = from_f32<TW>(val - to_f32(hi));
    };
    auto put_split = [&](TW* hi_t, TW* lo_t, int idx, float val) {
        const TW hi = from_f32<TW>(val);
        hi_t[idx] = hi;
        if constexpr (SPLIT) lo_t[idx] = from_f32<TW>(val - to_f32(hi));
    };

    // ---- phase 0: clear L and T, stage beta ----
    for (int i = tid; i < C * LD; i += NTHREADS) {
        Lm[i] = 0.f;
        Tm[i] = 0.f;
    }
    if (tid < C) betas[tid] = tid < len ? to_f32(beta[(size_t)(rs + tid) * p.HV + hv]) : 0.f;

    // ---- phase 1 (Stage 1): chunk-local cumsum of the log2 gate, column d per thread ----
    const int d = tid % K;
    const int rg = tid / K;
    const int i0 = rg * RPT;
    float gam[RPT], kk[RPT], qq[RPT];
#pragma unroll
    for (int ii = 0; ii < RPT; ++ii) {
        const int i = i0 + ii;
        float gv = 0.f, kv = 0.f, qv = 0.f;
        if (i < len) {
            const size_t r = (size_t)(rs + i);
            gv = p.g[(r * p.HV + hv) * K + d];
            kv = to_f32(k[(r * p.H + h) * K + d]);
            qv = to_f32(q[(r * p.H + h) * K + d]);
        }
        gam[ii] = gv;
        kk[ii] = kv;
        qq[ii] = qv;
    }
#pragma unroll
    for (int ii = 1; ii < RPT; ++ii) gam[ii] += gam[ii - 1];
    gsum[rg][d] = gam[RPT - 1];
    __syncthreads();
    float pre = 0.f, Gd = 0.f;
    for (int r2 = 0; r2 < RG; ++r2) {
        if (r2 < rg) pre += gsum[r2][d];
        Gd += gsum[r2][d];
    }
#pragma unroll
    for (int ii = 0; ii < RPT; ++ii) gam[ii] += pre;

    // anchors: midpoint of each 16-row block unless a half-block spans too much decay
    int wide = 0;
#pragma unroll
    for (int bl = 0; bl < RPT / 16; ++bl) {
        const float s0 = gam[bl * 16], sm = gam[bl * 16 + 8], s1 = gam[bl * 16 + 15];
        wide |= (s0 - sm > SPREAD_LIMIT) || (sm - s1 > SPREAD_LIMIT);
    }
    const bool exact_diag = block_any(wide) != 0;
#pragma unroll
    for (int bl = 0; bl < RPT / 16; ++bl) {
        const int I = (i0 >> 4) + bl;
        anch[I][d] = exact_diag ? gam[bl * 16] : gam[bl * 16 + 8];
    }
    __syncthreads();

    // ---- phase 2 (Stage 2, products): Aqk and L block rows ----
    const int lr = lane & 15;          // accumulator column
    const int lq = lane >> 4;          // accumulator row quad
    for (int I = 0; I < 4; ++I) {
        const float am = anch[I][d];
#pragma unroll
        for (int ii = 0; ii < RPT; ++ii) {
            const int i = i0 + ii;
            if ((i >> 4) == I) {
                const float f = exp2_fast(gam[ii] - am);
                put_split(QH, QHl, TQ::idx(i - 16 * I, d), qq[ii] * f);
                put_split(KR, KRl, TQ::idx(i - 16 * I, d), kk[ii] * f);
            }
            if ((i >> 4) <= I) {
                float kc = 0.f;
                if (!(exact_diag && (i >> 4) == I)) kc = kk[ii] * exp2_fast(am - gam[ii]);
                put_split(KC, KCl, TKC::idx(i, d), kc);
            }
        }
        __syncthreads();
        const int ntile = 2 * (I + 1);
        for (int tt = wave; tt < ntile; tt += 4) {
            const int J = tt >> 1;
            const bool is_qk = (tt & 1) == 0;
            if (exact_diag && J == I) continue;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = tile_mma<TW, TQ, TKC>(acc, is_qk ? QH : KR, 0, KC, 16 * J, 0, K, lane);
            if constexpr (SPLIT) {
                f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
                acc2 = tile_mma<TW, TQ, TKC>(acc2, is_qk ? QHl : KRl, 0, KC, 16 * J, 0, K, lane);
                acc2 = tile_mma<TW, TQ, TKC>(acc2, is_qk ? QH : KR, 0, KCl, 16 * J, 0, K, lane);
                acc += acc2;
            }
            const int j = 16 * J + lr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * I + 4 * lq + r;
                if (is_qk) {
                    const float val = i >= j ? p.scale * acc[r] : 0.f;
                    put_aqk(i * C + j, val);
                } else {
                    Lm[i * LD + j] = i > j ? betas[i] * acc[r] : 0.f;
                }
            }
        }
        __syncthreads();
    }
    // zero the upper blocks of Aqk
    for (int e = tid; e < 6 * 256; e += NTHREADS) {
        const int bi = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
        const int I = bi < 3 ? 0 : (bi < 5 ? 1 : 2);
        const int J = bi < 3 ? bi + 1 : (bi < 5 ? bi - 1 : 3);
        put_aqk((16 * I + rr) * C + 16 * J + cc, 0.f);
    }

    // ---- phase 2b: exact diagonal blocks when the decay is too steep for an anchor ----
    if (exact_diag) {
#pragma unroll
        for (int ii = 0; ii < RPT; ++ii) GM[(i0 + ii) * K + d] = gam[ii];
        __syncthreads();
        for (int e = tid; e < 4 * 256; e += NTHREADS) {
            const int I = e >> 8, ri = (e >> 4) & 15, rj = e & 15;
            const int i = 16 * I + ri, j = 16 * I + rj;
            if (rj > ri) {   // above the diagonal: Aqk is zero there
                put_aqk(i * C + j, 0.f);
                continue;
            }
            float aq = 0.f, ak = 0.f;
            if (i < len) {
                const size_t r_i = (size_t)(rs + i), r_j = (size_t)(rs + j);
                for (int dd = 0; dd < K; ++dd) {
                    const float f = exp2_fast(GM[i * K + dd] - GM[j * K + dd]);
                    const float kj = to_f32(k[(r_j * p.H + h) * K + dd]) * f;
                    aq = fmaf(to_f32(q[(r_i * p.H + h) * K + dd]), kj, aq);
                    ak = fmaf(to_f32(k[(r_i * p.H + h) * K + dd]), kj, ak);
                }
            }
            put_aqk(i * C + j, p.scale * aq);
            if (i > j) Lm[i * LD + j] = betas[i] * ak;
        }
        __syncthreads();
    }

    // ---- phase 3: T = (I + L)^-1 by blocks ----
    if (wave == 0) {
        const int I = lane >> 4, cc = lane & 15;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float s = (i == cc) ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < i; ++j) s = fmaf(-Lm[(16 * I + i) * LD + 16 * I + j], x[j], s);
            x[i] = s;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) Tm[(16 * I + i) * LD + 16 * I + cc] = x[i];
    }
    __syncthreads();
    for (int lev = 1; lev < 4; ++lev) {
        const int nb = 4 - lev;
        for (int e = tid; e < nb * 256; e += NTHREADS) {
            const int bi = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
            const int I = lev + bi, J = I - lev;
            float x = 0.f;
            for (int M = J; M < I; ++M)
#pragma unroll
                for (int m = 0; m < 16; ++m)
                    x = fmaf(Lm[(16 * I + rr) * LD + 16 * M + m], Tm[(16 * M + m) * LD + 16 * J + cc], x);
            Xs[(bi * 16 + rr) * 17 + cc] = x;
        }
        __syncthreads();
        for (int e = tid; e < nb * 256; e += NTHREADS) {
            const int bi = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
            const int I = lev + bi, J = I - lev;
            float t = 0.f;
#pragma unroll
            for (int m = 0; m < 16; ++m)
                t = fmaf(Tm[(16 * I + rr) * LD + 16 * I + m], Xs[(bi * 16 + m) * 17 + cc], t);
            Tm[(16 * I + rr) * LD + 16 * J + cc] = -t;
        }
        __syncthreads();
    }

    // ---- phase 4: operands of w and u, and the elementwise outputs ----
    for (int e = tid; e < C * C; e += NTHREADS) {
        const int i = e / C, j = e % C;
        TBs[TB64::idx(i, j)] = from_f32<TW>(Tm[i * LD + j] * betas[j]);
    }
#pragma unroll
    for (int ii = 0; ii < RPT; ++ii) {
        const int i = i0 + ii;
        const float e = exp2_fast(gam[ii]);
        KDt[TKD::idx(d, i)] = from_f32<TW>(kk[ii] * e);
        put_split(out_qg, out_qg + C * K, i * K + d, p.scale * qq[ii] * e);
        put_split(out_kgT, out_kgT + K * C, d * C + i, kk[ii] * exp2_fast(Gd - gam[ii]));
    }
    if (rg == 0) out_eg[d] = exp2_fast(Gd);
    {
        const int cv = tid % V;
        const int i1 = (tid / V) * RPTV;
#pragma unroll 4
        for (int ii = 0; ii < RPTV; ++ii) {
            const int i = i1 + ii;
            float vv = 0.f;
            if (i < len) vv = to_f32(v[((size_t)(rs + i) * p.HV + hv) * V + cv]);
            VTt[TVT::idx(cv, i)] = from_f32<TW>(vv);
        }
    }
    __syncthreads();

    // w = (T beta) (k 2^G)   [64 x K],   u = (T beta) v   [64 x V]
    constexpr int NTW = K / 16, NTU = V / 16;
    for (int tt = wave; tt < 4 * (NTW + NTU); tt += 4) {
        const int mt = tt % 4;
        const int nt = tt / 4;
        const int kend = (16 * mt + 16 + Mma<TW>::KS - 1) / Mma<TW>::KS * Mma<TW>::KS;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (nt < NTW) {
            acc = tile_mma<TW, TB64, TKD>(acc, TBs, 16 * mt, KDt, 16 * nt, 0, kend < C ? kend : C, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                out_w[(16 * mt + 4 * lq + r) * K + 16 * nt + lr] = from_f32<TW>(acc[r]);
        } else {
            const int nu = nt - NTW;
            acc = tile_mma<TW, TB64, TVT>(acc, TBs, 16 * mt, VTt, 16 * nu, 0, kend < C ? kend : C, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                out_u[(16 * mt + 4 * lq + r) * V + 16 * nu + lr] = acc[r];
        }
    }
}

// ------------------------------------------------------------------------------------
// scan: Stage 3+4 for one (sequence, value head, BV-column slice)
// ------------------------------------------------------------------------------------
struct ScanParams {
    const char* rec;
    size_t rec_bytes, off_w, off_u, off_qg, off_kgT, off_aqk, off_eg;
    const float* initial_state;
    float* final_state;
    void* o;
    const int32_t* coff;     // packed: first chunk of each slot [N]
    const int32_t* cend;     // packed: one past the last chunk of each slot [N]
    const int32_t* slot_ok;  // packed: slot validity
    const int2* table;       // packed: chunk table
    int N, T, HV, NT, NCmax;
};

// The chunk records stream through registers: the block issues the global loads of
// chunk c+1 right after chunk c's record is in LDS and only waits for them one step
// later, so HBM latency overlaps the serial matrix-core work.
template <int K, int V, int BV, typename TW>
struct RecordRegs {
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
    static constexpr bool SPLIT = sizeof(TW) == 2;
    static constexpr int NS = SPLIT ? 2 : 1;
    static constexpr int EPC = 16 / (int)sizeof(TW);
    static constexpr int CW = C * K / EPC / NTHREADS;        // 16-byte chunks per thread: w, qg, kgT
    static constexpr int CA = C * C / EPC / NTHREADS;        // Aqk
    static constexpr int CU = C * BV / 4 / NTHREADS;         // u slice (fp32, 4 per chunk)
    static_assert(CW * NTHREADS * EPC == C * K, "w tile must split evenly");
    static_assert(CA * NTHREADS * EPC == C * C, "Aqk tile must split evenly");
    static_assert(CU * NTHREADS * 4 == C * BV, "u slice must split evenly");
    u32x4 w[CW], q[NS][CW], g[NS][CW], a[NS][CA];
    f32x4 u[CU], e;
};

template <int K, int V, int BV, typename TW>
__device__ __forceinline__ void fetch_record(RecordRegs<K, V, BV, TW>& R, const char* rec,
                                             const ScanParams& p, int v0, int tid) {
    typedef RecordRegs<K, V, BV, TW> RR;
    typedef typename RR::u32x4 u32x4;
    const u32x4* gw = reinterpret_cast<const u32x4*>(rec + p.off_w);
    const u32x4* gq = reinterpret_cast<const u32x4*>(rec + p.off_qg);
    const u32x4* gg = reinterpret_cast<const u32x4*>(rec + p.off_kgT);
    const u32x4* ga = reinterpret_cast<const u32x4*>(rec + p.off_aqk);
#pragma unroll
    for (int j = 0; j < RR::CW; ++j) R.w[j] = gw[tid + j * NTHREADS];
#pragma unroll
    for (int sx = 0; sx < RR::NS; ++sx)
#pragma unroll
        for (int j = 0; j < RR::CW; ++j) {
            R.q[sx][j] = gq[sx * RR::CW * NTHREADS + tid + j * NTHREADS];
            R.g[sx][j] = gg[sx * RR::CW * NTHREADS + tid + j * NTHREADS];
        }
#pragma unroll
    for (int sx = 0; sx < RR::NS; ++sx)
#pragma unroll
        for (int j = 0; j < RR::CA; ++j) R.a[sx][j] = ga[sx * RR::CA * NTHREADS + tid + j * NTHREADS];
    const float* gu = reinterpret_cast<const float*>(rec + p.off_u);
#pragma unroll
    for (int j = 0; j < RR::CU; ++j) {
        const int e = tid + j * NTHREADS;
        const int row = e / (BV / 4), c4 = e % (BV / 4);
        R.u[j] = *reinterpret_cast<const f32x4*>(gu + row * V + v0 + 4 * c4);
    }
    if (tid < K / 4) R.e = reinterpret_cast<const f32x4*>(rec + p.off_eg)[tid];
}

template <int K, int V, int BV, typename TIn>
__global__ __launch_bounds__(NTHREADS) void scan_kernel(ScanParams p) {
    typedef TIn TW;
    typedef Tile<TW, C, K> TA;       // w, qg   [64][K]
    typedef Tile<TW, K, C> TG;       // kg^T    [K][64]
    typedef Tile<TW, C, C> TQK;      // Aqk     [64][64]
    typedef Tile<TW, BV, K> TS;      // S^T     [BV][K]
    typedef Tile<TW, BV, C> TV;      // v'^T    [BV][64]
    typedef RecordRegs<K, V, BV, TW> RR;
    typedef typename RR::u32x4 u32x4;
    // bf16 path: the state, v', qg, kg and Aqk operands are each a pair hi + lo of bf16
    // tiles, lo holding what rounding hi to bf16 lost; products use hi*hi + lo*hi + hi*lo.
    constexpr bool SPLIT = RR::SPLIT;
    constexpr int NS = RR::NS;
    constexpr int EPC = RR::EPC;
    constexpr int NVT = V / BV;
    constexpr int NNT = BV / 16;     // 16-column tiles of the slice
    constexpr int NDT = K / 64;      // 16-row state tiles per wave (K/16 tiles over 4 waves)

    __shared__ __attribute__((aligned(16))) TW Wt[TA::ELEMS];
    __shared__ __attribute__((aligned(16))) TW Qt[NS][TA::ELEMS];
    __shared__ __attribute__((aligned(16))) TW Gt[NS][TG::ELEMS];
    __shared__ __attribute__((aligned(16))) TW At[NS][TQK::ELEMS];
    __shared__ __attribute__((aligned(16))) TW St[2][NS][TS::ELEMS];
    __shared__ __attribute__((aligned(16))) TW Vt[NS][TV::ELEMS];
    __shared__ __attribute__((aligned(16))) float Ut[C][BV];
    __shared__ __attribute__((aligned(16))) float eG[K];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lr = lane & 15, lq = lane >> 4;
    const int G = p.N * p.HV * NVT;
    const int item = xcd_remap(blockIdx.x, G);
    const int vt = item % NVT;
    const int chain = item / NVT;
    const int hv = chain % p.HV;
    const int n = chain / p.HV;
    const int v0 = vt * BV;

    int c0, c1;
    if (p.table) {
        if (!p.slot_ok[n]) return;    // malformed offsets: leave this slot untouched
        c0 = p.coff[n];
        c1 = p.cend[n];
    } else {
        c0 = n * p.NT;
        c1 = c0 + p.NT;
    }
    auto record = [&](int c) { return p.rec + ((size_t)hv * p.NCmax + c) * p.rec_bytes; };

    // store an accumulator column block (4 rows) as hi (+ lo) into a pair of tiles
    auto put4 = [&](TW* hi, TW* lo, int col, int row0, f32x4 x, auto tile_tag) {
        typedef decltype(tile_tag) TT;
        const int base = TT::idx(col, row0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const TW h = from_f32<TW>(x[r]);
            hi[base + r] = h;
            if constexpr (SPLIT) lo[base + r] = from_f32<TW>(x[r] - to_f32(h));
        }
    };

    RR R;
    if (c0 < c1) fetch_record<K, V, BV, TW>(R, record(c0), p, v0, tid);

    // state tiles owned by this wave: dt = wave + 4 * a
    f32x4 S[NDT][NNT];
    const size_t sbase = ((size_t)n * p.HV + hv) * (size_t)K * V;
    if (p.initial_state) {
#pragma unroll
        for (int a = 0; a < NDT; ++a)
#pragma unroll
            for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int dd = 16 * (wave + 4 * a) + 4 * lq + r;
                    S[a][nt][r] = p.initial_state[sbase + (size_t)dd * V + v0 + 16 * nt + lr];
                }
    } else {
#pragma unroll
        for (int a = 0; a < NDT; ++a)
#pragma unroll
            for (int nt = 0; nt < NNT; ++nt) S[a][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    int cur = 0;
#pragma unroll
    for (int a = 0; a < NDT; ++a)
#pragma unroll
        for (int nt = 0; nt < NNT; ++nt)
            put4(St[0][0], St[0][NS - 1], 16 * nt + lr, 16 * (wave + 4 * a) + 4 * lq, S[a][nt], TS());

    TIn* o = reinterpret_cast<TIn*>(p.o);
    for (int c = c0; c < c1; ++c) {
        long long rs;
        int len;
        if (p.table) {
            const int2 e = p.table[c];
            rs = e.x;
            len = e.y;
        } else {
            const int ci = c - c0;
            rs = (long long)n * p.T + (long long)ci * C;
            len = p.T - ci * C < C ? p.T - ci * C : C;
        }
        // ---- commit the prefetched record of chunk c to LDS, start fetching c+1 ----
#pragma unroll
        for (int j = 0; j < RR::CW; ++j) {
            const int e = tid + j * NTHREADS;
            const int row = e / (K / EPC), col = (e % (K / EPC)) * EPC;
            *reinterpret_cast<u32x4*>(&Wt[TA::idx(row, col)]) = R.w[j];
#pragma unroll
            for (int sx = 0; sx < NS; ++sx)
                *reinterpret_cast<u32x4*>(&Qt[sx][TA::idx(row, col)]) = R.q[sx][j];
            const int grow = e / (C / EPC), gcol = (e % (C / EPC)) * EPC;
#pragma unroll
            for (int sx = 0; sx < NS; ++sx)
                *reinterpret_cast<u32x4*>(&Gt[sx][TG::idx(grow, gcol)]) = R.g[sx][j];
        }
#pragma unroll
        for (int j = 0; j < RR::CA; ++j) {
            const int e = tid + j * NTHREADS;
            const int row = e / (C / EPC), col = (e % (C / EPC)) * EPC;
#pragma unroll
            for (int sx = 0; sx < NS; ++sx)
                *reinterpret_cast<u32x4*>(&At[sx][TQK::idx(row, col)]) = R.a[sx][j];
        }
#pragma unroll
        for (int j = 0; j < RR::CU; ++j) {
            const int e = tid + j * NTHREADS;
            const int row = e / (BV / 4), c4 = e % (BV / 4);
            *reinterpret_cast<f32x4*>(&Ut[row][4 * c4]) = R.u[j];
        }
        if (tid < K / 4) *reinterpret_cast<f32x4*>(&eG[4 * tid]) = R.e;
        __syncthreads();
        if (c + 1 < c1) fetch_record<K, V, BV, TW>(R, record(c + 1), p, v0, tid);

        // ---- v' = u - w S ----
        const TW* Sh = St[cur][0];
        const TW* Sl = St[cur][NS - 1];
#pragma unroll
        for (int nt = 0; nt < NNT; ++nt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = tile_mma<TW, TA, TS>(acc, Wt, 16 * wave, Sh, 16 * nt, 0, K, lane);
            if constexpr (SPLIT) acc = tile_mma<TW, TA, TS>(acc, Wt, 16 * wave, Sl, 16 * nt, 0, K, lane);
            f32x4 vn;
#pragma unroll
            for (int r = 0; r < 4; ++r) vn[r] = Ut[16 * wave + 4 * lq + r][16 * nt + lr] - acc[r];
            put4(Vt[0], Vt[NS - 1], 16 * nt + lr, 16 * wave + 4 * lq, vn, TV());
        }
        __syncthreads();

        // ---- o = qg S + Aqk v'  (rows 16*wave ..) ----
        {
            const int kend = (16 * wave + 16 + Mma<TW>::KS - 1) / Mma<TW>::KS * Mma<TW>::KS;
            const int k1 = kend < C ? kend : C;
#pragma unroll
            for (int nt = 0; nt < NNT; ++nt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = tile_mma<TW, TA, TS>(acc, Qt[0], 16 * wave, Sh, 16 * nt, 0, K, lane);
                acc = tile_mma<TW, TQK, TV>(acc, At[0], 16 * wave, Vt[0], 16 * nt, 0, k1, lane);
                if constexpr (SPLIT) {
                    f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
                    acc2 = tile_mma<TW, TA, TS>(acc2, Qt[NS - 1], 16 * wave, Sh, 16 * nt, 0, K, lane);
                    acc2 = tile_mma<TW, TA, TS>(acc2, Qt[0], 16 * wave, Sl, 16 * nt, 0, K, lane);
                    acc2 = tile_mma<TW, TQK, TV>(acc2, At[NS - 1], 16 * wave, Vt[0], 16 * nt, 0, k1, lane);
                    acc2 = tile_mma<TW, TQK, TV>(acc2, At[0], 16 * wave, Vt[NS - 1], 16 * nt, 0, k1, lane);
                    acc += acc2;
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * wave + 4 * lq + r;
                    if (i < len)
                        o[((size_t)(rs + i) * p.HV + hv) * V + v0 + 16 * nt + lr] = from_f32<TIn>(acc[r]);
                }
            }
        }

        // ---- S = 2^G S + kg^T v' ----
        const int nxt = cur ^ 1;
#pragma unroll
        for (int a = 0; a < NDT; ++a) {
            const int dt = wave + 4 * a;
#pragma unroll
            for (int nt = 0; nt < NNT; ++nt) {
                f32x4 acc = S[a][nt];
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] *= eG[16 * dt + 4 * lq + r];
                acc = tile_mma<TW, TG, TV>(acc, Gt[0], 16 * dt, Vt[0], 16 * nt, 0, C, lane);
                if constexpr (SPLIT) {
                    f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
                    acc2 = tile_mma<TW, TG, TV>(acc2, Gt[NS - 1], 16 * dt, Vt[0], 16 * nt, 0, C, lane);
                    acc2 = tile_mma<TW, TG, TV>(acc2, Gt[0], 16 * dt, Vt[NS - 1], 16 * nt, 0, C, lane);
                    acc += acc2;
                }
                S[a][nt] = acc;
                put4(St[nxt][0], St[nxt][NS - 1], 16 * nt + lr, 16 * dt + 4 * lq, acc, TS());
            }
        }
        cur = nxt;
        __syncthreads();
    }

    if (p.final_state) {
#pragma unroll
        for (int a = 0; a < NDT; ++a)
#pragma unroll
            for (int nt = 0; nt < NNT; ++nt) {
                const int dt = wave + 4 * a;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int dd = 16 * dt + 4 * lq + r;
                    p.final_state[sbase + (size_t)dd * V + v0 + 16 * nt + lr] = S[a][nt][r];
                }
            }
    }
}

// ------------------------------------------------------------------------------------
// launch
// ------------------------------------------------------------------------------------
template <int K, int V, typename TIn>
hipError_t launch_scan(const ChunkArgs& a, const ScanParams& sp);

template <int K, int V, typename TIn, typename TB>
hipError_t launch_kv(const ChunkArgs& a, const ChunkLayout& L) {
    char* ws = reinterpret_cast<char*>(a.workspace);
    const bool packed = a.cu_seqlens != nullptr;
    const int NT = packed ? 0 : (a.T + C - 1) / C;
    int32_t *coff = nullptr, *cend = nullptr, *slot_ok = nullptr, *nch = nullptr;
    int2* table = nullptr;
    if (a.events) {
        hipError_t err = hipEventRecord(a.events[0], a.stream);
        if (err != hipSuccess) return err;
    }
    if (packed) {
        coff = reinterpret_cast<int32_t*>(ws);
        cend = coff + a.N;
        slot_ok = cend + a.N;
        nch = slot_ok + a.N;
        table = reinterpret_cast<int2*>(ws + sched_table_offset(a.N));
        hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(1024), 0, a.stream, a.cu_seqlens, a.N,
                           a.T, L.NCmax, coff, cend, slot_ok, nch, table, a.dev_status);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (a.events) {
        hipError_t err = hipEventRecord(a.events[1], a.stream);
        if (err != hipSuccess) return err;
    }
    char* recs = ws + L.sched_bytes;

    IntraParams ip;
    ip.q = a.q; ip.k = a.k; ip.v = a.v; ip.g = a.g; ip.beta = a.beta;
    ip.nchunks = nch; ip.table = table; ip.rec = recs;
    ip.rec_bytes = L.rec_bytes; ip.off_w = L.off_w; ip.off_u = L.off_u; ip.off_qg = L.off_qg;
    ip.off_kgT = L.off_kgT; ip.off_aqk = L.off_aqk; ip.off_eg = L.off_eg;
    ip.T = a.T; ip.H = a.H; ip.HV = a.HV; ip.NT = NT; ip.NCmax = L.NCmax;
    ip.scale = a.scale;
    const long long nintra = (long long)L.NCmax * a.HV;
    if (nintra > 0) {
        hipLaunchKernelGGL((intra_kernel<K, V, TIn, TB>), dim3((unsigned)nintra), dim3(NTHREADS), 0,
                           a.stream, ip);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }

    ScanParams sp;
    sp.rec = recs; sp.rec_bytes = L.rec_bytes; sp.off_w = L.off_w; sp.off_u = L.off_u;
    sp.off_qg = L.off_qg; sp.off_kgT = L.off_kgT; sp.off_aqk = L.off_aqk; sp.off_eg = L.off_eg;
    sp.initial_state = a.initial_state; sp.final_state = a.final_state; sp.o = a.o;
    sp.coff = coff; sp.cend = cend; sp.slot_ok = slot_ok; sp.table = table;
    sp.N = a.N; sp.T = a.T; sp.HV = a.HV; sp.NT = NT; sp.NCmax = L.NCmax;
    if (a.events) {
        hipError_t err = hipEventRecord(a.events[2], a.stream);
        if (err != hipSuccess) return err;
    }
    hipError_t err = launch_scan<K, V, TIn>(a, sp);
    if (err == hipSuccess && a.events) err = hipEventRecord(a.events[3], a.stream);
    return err;
}

template <int K, int V, typename TIn>
hipError_t launch_scan(const ChunkArgs& a, const ScanParams& sp) {
    const long long chains = (long long)a.N * a.HV;
    if (chains == 0) return hipSuccess;
    // pick the slice width: enough blocks to cover the chip, wide slices when chains abound
    // (the fp32 path keeps 16-column slices: its operand tiles take twice the LDS;
    //  the bf16 path's hi/lo pairs cap it at 32)
    int BV = 16;
    if (sizeof(TIn) == 2 && chains * (V / 32) >= 512) BV = 32;
    const unsigned nscan = (unsigned)(chains * (V / BV));
    if constexpr (sizeof(TIn) == 2) {
        if (BV == 32) {
            hipLaunchKernelGGL((scan_kernel<K, V, 32, TIn>), dim3(nscan), dim3(NTHREADS), 0, a.stream, sp);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((scan_kernel<K, V, 16, TIn>), dim3(nscan), dim3(NTHREADS), 0, a.stream, sp);
    return hipGetLastError();
}

template <typename TIn, typename TB>
hipError_t launch_t(const ChunkArgs& a, const ChunkLayout& L) {
    if (a.K == 128) return a.V == 128 ? launch_kv<128, 128, TIn, TB>(a, L) : launch_kv<128, 64, TIn, TB>(a, L);
    return a.V == 128 ? launch_kv<64, 128, TIn, TB>(a, L) : launch_kv<64, 64, TIn, TB>(a, L);
}

}  // namespace

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

bool chunk_layout(int B, int T, int HV, int K, int V, int N, bool packed, int qkv_dtype,
                  ChunkLayout* out) {
    ChunkLayout L{};
    if (packed) {
        L.NCmax = T / C + N;
    } else {
        L.NCmax = B * ((T + C - 1) / C);
    }
    L.elem = qkv_dtype == KDA_BF16 ? 2 : 4;
    // bf16 path: qg, kg^T and Aqk carry a second tile with their bf16 rounding residual
    const size_t ns = qkv_dtype == KDA_BF16 ? 2 : 1;
    size_t off = 0;
    L.off_w = off;   off += (size_t)C * K * L.elem;
    L.off_qg = off;  off += ns * C * K * L.elem;
    L.off_kgT = off; off += ns * K * C * L.elem;
    L.off_aqk = off; off += ns * C * C * L.elem;
    L.off_u = off;   off += (size_t)C * V * 4;        // u stays fp32 (used outside the MFMAs)
    L.off_eg = off;  off += (size_t)K * 4;
    L.rec_bytes = align256(off);
    L.sched_bytes = 0;
    if (packed) {
        size_t s = sched_table_offset(N);                      // coff, cend, slot_ok, n_chunks
        s += (size_t)L.NCmax * 8;                              // chunk table
        L.sched_bytes = align256(s);
    }
    L.total = L.sched_bytes + (size_t)HV * L.NCmax * L.rec_bytes;
    *out = L;
    return true;
}

hipError_t launch_chunk(const ChunkArgs& a, const ChunkLayout& L) {
    if (a.qkv_dtype == KDA_BF16)
        return a.beta_dtype == KDA_BF16 ? launch_t<__bf16, __bf16>(a, L) : launch_t<__bf16, float>(a, L);
    return a.beta_dtype == KDA_BF16 ? launch_t<float, __bf16>(a, L) : launch_t<float, float>(a, L);
}

}  // namespace kda
