// Per-token KDA recurrence (decode and token-by-token prefill) for gfx950.
//
// Contract: "Add fused recurrent_kda for decode and inference prefill" (attention-gym
// PR #317, description): the gate is the per-token log2 decay (or, optionally, formed
// from the raw gate input by the fused activation, with q / k normalisation and the beta
// sigmoid fused into the loads as in the chunked path), the scale is 1/sqrt(K),
// compute and state are fp32 whatever the input dtype, packed int32 offsets with empty
// slots passing their state through bitwise, one state per logical sequence. The update
// order (decay, delta-rule write, read of the updated state) is the one of KDA's chunk
// algebra in "kernel-fun 0.2.0.dev1 sdist", ALGORITHM.md, section Forward.
//
// Work decomposition. One wavefront owns one (sequence n, value head hv, BV-column slice
// of V) and walks its tokens in order. Its 64 lanes form CG = BV/4 column groups times
// RG = 64/CG row groups; lane l (column group cg = l % CG, row group rg = l / CG) holds
// the state block of the R = K/RG rows d(rg, i), i = 0 .. R-1, and the four columns
// c = v0 + 4 cg + j, j = 0 .. 3, in registers, so the state is read from HBM once and
// written once with 16-byte accesses. Per token the lane folds the decay into its block,
// forms partial sums of S~^T k and S~^T q over its rows (S~ = decayed state), and the row
// groups combine them with log2(RG) cross-lane exchanges. Then
//     delta = beta (v - S~^T k),   o = scale (S~^T q + delta (k . q)),   S = S~ + k delta^T
// which is o = scale S_t^T q without a second pass over the state.
//
// States stored [K][V] give each row group a contiguous run of rows, d = rg R + i: every
// access of the CG column-group lanes is then one contiguous run of a state row. States
// stored transposed ([V][K], fla's state_v_first) deal rows to the row groups four at a
// time, d = 4 RG (i / 4) + 4 rg + i % 4, so the RG row-group lanes of a column read one
// contiguous run of it. The two layouts thus sum rows in different orders, and their
// outputs agree to fp32 rounding, not bitwise.
//
// States stored [K][V]: BV = 64 (K = 128: 128 fp32 of state per lane, one wave per SIMD)
// when every sequence carries about one token: that launch is a pure state stream and
// the longer row runs keep it closest to a plain copy. Otherwise BV = 32 (half the
// registers, three waves per SIMD), which hides the per-token dependency chain of longer
// sequences. Transposed states: BV = 16 (16 row groups, four waves per SIMD), so each
// column access of a row-group set is one 256-byte run, the length of the [K][V] rows'.
//
// The grid is flat and 1-D (four wavefronts per 256-thread block), so N * HV * V/BV may
// exceed 65,535. The state layout and whether the state after every token is written
// out as well (fla's return_intermediate_states) are compile-time choices, so the plain
// decode kernel carries neither. Packed offsets are validated per slot on every call: a
// slot with bos < 0, bos > eos, eos > T, or slot 0 not starting at 0, is skipped and
// flagged.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

__device__ __forceinline__ void load4(const __bf16* p, float* out) {
    bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = (float)x[j];
}

__device__ __forceinline__ void load4(const float* p, float* out) {
    f32x4 x = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = x[j];
}

__device__ __forceinline__ void store4(__bf16* p, const float* x) {
    bf16x4 y;
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = (__bf16)x[j];
    *reinterpret_cast<bf16x4*>(p) = y;
}

__device__ __forceinline__ void store4(float* p, const float* x) {
    f32x4 y = {x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(p) = y;
}

// Sum over the row groups: lanes CG, 2 CG, ... apart hold the same columns.
template <int CG>
__device__ __forceinline__ float sum_row_groups(float x) {
#pragma unroll
    for (int off = CG; off < 64; off *= 2) x += __shfl_xor(x, off, 64);
    return x;
}

// Row i of a lane's block in row group rg of RG, R rows each: contiguous (rg R + i), or
// dealt four at a time (ILV) (see the work decomposition above). Rows i .. i+3, i a
// multiple of 4, are consecutive in both.
template <int RG, int R, bool ILV>
__device__ __forceinline__ int block_row(int rg, int i) {
    return ILV ? 4 * RG * (i >> 2) + 4 * rg + (i & 3) : rg * R + i;
}

// The lane's R entries of one K-vector (q, k, a gate row, dt_bias), in block-row order:
// 16-byte accesses of 8 (bf16) or 4 (fp32) elements where the rows are contiguous, else
// four consecutive elements at a time.
template <int RG, int R, bool ILV>
__device__ __forceinline__ void load_rows(const __bf16* p, int rg, float (&out)[R]) {
    if (!ILV) {
        p += rg * R;
#pragma unroll
        for (int i = 0; i < R; i += 8) {
            const bf16x8 x = *reinterpret_cast<const bf16x8*>(p + i);
#pragma unroll
            for (int e = 0; e < 8; ++e) out[i + e] = (float)x[e];
        }
    } else {
#pragma unroll
        for (int i = 0; i < R; i += 4) {
            const bf16x4 x = *reinterpret_cast<const bf16x4*>(p + block_row<RG, R, true>(rg, i));
#pragma unroll
            for (int e = 0; e < 4; ++e) out[i + e] = (float)x[e];
        }
    }
}

template <int RG, int R, bool ILV>
__device__ __forceinline__ void load_rows(const float* p, int rg, float (&out)[R]) {
#pragma unroll
    for (int i = 0; i < R; i += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(p + block_row<RG, R, ILV>(rg, i));
#pragma unroll
        for (int e = 0; e < 4; ++e) out[i + e] = x[e];
    }
}

// The lane's block of a state, columns c0 .. c0+3: [K][V] (row d at base + d V, rows
// contiguous per row group) or, with VK, [V][K] (column c at base + c K, rows dealt four
// at a time); 16-byte accesses in both.
template <int RG, int R, bool VK>
__device__ __forceinline__ void load_state(const float* base, int K, int V, int rg, int c0,
                                           f32x4 (&S)[R]) {
#pragma unroll
    for (int i = 0; i < R; i += 4) {
        const int d = block_row<RG, R, VK>(rg, i);
        if (!VK) {
#pragma unroll
            for (int e = 0; e < 4; ++e) S[i + e] = *reinterpret_cast<const f32x4*>(base + (size_t)(d + e) * V + c0);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(base + (size_t)(c0 + j) * K + d);
#pragma unroll
                for (int e = 0; e < 4; ++e) S[i + e][j] = x[e];
            }
        }
    }
}

template <int RG, int R, bool VK>
__device__ __forceinline__ void store_state(float* base, int K, int V, int rg, int c0,
                                            const f32x4 (&S)[R]) {
#pragma unroll
    for (int i = 0; i < R; i += 4) {
        const int d = block_row<RG, R, VK>(rg, i);
        if (!VK) {
#pragma unroll
            for (int e = 0; e < 4; ++e) *reinterpret_cast<f32x4*>(base + (size_t)(d + e) * V + c0) = S[i + e];
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<f32x4*>(base + (size_t)(c0 + j) * K + d) =
                    f32x4{S[i][j], S[i + 1][j], S[i + 2][j], S[i + 3][j]};
        }
    }
}

template <int CG, int R>
__device__ __forceinline__ void l2norm_rows(float (&x)[R]) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i) ss = fmaf(x[i], x[i], ss);
    const float rn = l2norm_rstd(sum_row_groups<CG>(ss));
#pragma unroll
    for (int i = 0; i < R; ++i) x[i] *= rn;
}

template <int K, int BV, typename TIn, typename TB, bool VK, bool INTER>
__global__ __launch_bounds__(256) void recurrent_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const float* __restrict__ g, const InputSpec in, const TB* __restrict__ beta,
    const float* initial_state, const int32_t* __restrict__ cu_seqlens,
    TIn* __restrict__ o, float* final_state, float* inter_states, int T, int H,
    int HV, int V, int nvt, long long n_items, float scale, int32_t* dev_status) {
    constexpr int CG = BV / 4;   // column groups: lanes along the wave's BV columns
    constexpr int RG = 64 / CG;  // row groups: lanes along K
    constexpr int R = K / RG;    // rows per lane
    const int lane = threadIdx.x & 63;
    const long long item = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= n_items) return;

    const int vt = (int)(item % nvt);
    const long long chain = item / nvt;
    const int hv = (int)(chain % HV);
    const int n = (int)(chain / HV);
    const int h = hv / (HV / H);
    const int cg = lane % CG;
    const int rg = lane / CG;
    const int c0 = vt * BV + 4 * cg;

    long long row0;
    int bos, eos;
    if (cu_seqlens) {
        bos = cu_seqlens[n];
        eos = cu_seqlens[n + 1];
        const bool ok = bos >= 0 && bos <= eos && eos <= T && (n != 0 || bos == 0);
        if (!ok) {
            if (lane == 0 && dev_status) atomicOr(dev_status, KDA_DEV_BAD_CU_SEQLENS);
            return;
        }
        row0 = 0;
    } else {
        bos = 0;
        eos = T;
        row0 = (long long)n * T;
    }

    const size_t sbase = ((size_t)n * HV + hv) * (size_t)K * V;
    f32x4 S[R];   // row i of the lane's block, columns c0 .. c0+3
    if (initial_state) {
        load_state<RG, R, VK>(initial_state + sbase, K, V, rg, c0, S);
    } else {
#pragma unroll
        for (int i = 0; i < R; ++i) S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const float amp = in.gate_mode != GATE_LOG2 ? -expf(in.A_log[hv]) : 0.f;
    const float lb2 = in.lower_bound * LOG2E;
    for (int t = bos; t < eos; ++t) {
        const long long r = row0 + t;
        float kk[R], qq[R], ee[R], vv[4];
        load_rows<RG, R, VK>(k + ((size_t)r * H + h) * K, rg, kk);
        load_rows<RG, R, VK>(q + ((size_t)r * H + h) * K, rg, qq);
        const size_t gofs = ((size_t)r * HV + hv) * K;
        if (in.gate_mode == GATE_LOG2) {
            load_rows<RG, R, VK>(g + gofs, rg, ee);
        } else {
            // the fused gate activation on the raw gate input
            if (in.gate_mode == GATE_RAW_BF16)
                load_rows<RG, R, VK>(static_cast<const __bf16*>(in.g_raw) + gofs, rg, ee);
            else
                load_rows<RG, R, VK>(static_cast<const float*>(in.g_raw) + gofs, rg, ee);
            if (in.dt_bias) {
                float db[R];
                load_rows<RG, R, VK>(in.dt_bias + (size_t)hv * K, rg, db);
#pragma unroll
                for (int i = 0; i < R; ++i) ee[i] += db[i];
            }
#pragma unroll
            for (int i = 0; i < R; ++i) ee[i] = gate_log2_from_raw(ee[i], amp, in.has_lower_bound, lb2);
        }
        load4(v + ((size_t)r * HV + hv) * V + c0, vv);
        float b = to_f32(beta[(size_t)r * HV + hv]);
        if (in.beta_sig != 0.f) b = beta_from_logit(b, in.beta_sig);
        // optional L2 normalisation of q / k (the four row groups hold a row between them)
        if (in.l2norm_q) l2norm_rows<CG>(qq);
        if (in.l2norm_k) l2norm_rows<CG>(kk);

        float p[4] = {0.f, 0.f, 0.f, 0.f};
        float rq[4] = {0.f, 0.f, 0.f, 0.f};
        float kq = 0.f;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const float e = exp2_fast(ee[i]);
            kq = fmaf(kk[i], qq[i], kq);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float s = S[i][j] * e;
                S[i][j] = s;
                p[j] = fmaf(kk[i], s, p[j]);
                rq[j] = fmaf(qq[i], s, rq[j]);
            }
        }
        kq = sum_row_groups<CG>(kq);
        float delta[4], out[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            p[j] = sum_row_groups<CG>(p[j]);
            rq[j] = sum_row_groups<CG>(rq[j]);
            delta[j] = b * (vv[j] - p[j]);
            out[j] = scale * fmaf(delta[j], kq, rq[j]);
        }
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) S[i][j] = fmaf(kk[i], delta[j], S[i][j]);
        if (rg == 0) store4(o + ((size_t)r * HV + hv) * V + c0, out);
        // the state after this token, in the states' layout
        if (INTER) store_state<RG, R, VK>(inter_states + ((size_t)r * HV + hv) * (size_t)K * V, K, V, rg, c0, S);
    }

    if (final_state) store_state<RG, R, VK>(final_state + sbase, K, V, rg, c0, S);
}

template <int K, int BV, typename TIn, typename TB, bool VK, bool INTER>
hipError_t launch_v(const RecurrentArgs& a) {
    const int nvt = a.V / BV;
    const long long n_items = (long long)a.N * a.HV * nvt;
    if (n_items == 0) return hipSuccess;
    const long long blocks = (n_items + 3) / 4;
    hipLaunchKernelGGL((recurrent_kernel<K, BV, TIn, TB, VK, INTER>), dim3((unsigned)blocks), dim3(256), 0,
                       a.stream, (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v, a.g, a.in,
                       (const TB*)a.beta, a.initial_state, a.cu_seqlens, (TIn*)a.o,
                       a.final_state, a.inter_states, a.T, a.H, a.HV, a.V, nvt, n_items, a.scale,
                       a.dev_status);
    return hipGetLastError();
}

template <int K, typename TIn, typename TB>
hipError_t launch_t(const RecurrentArgs& a) {
    if (a.state_vk)
        return a.inter_states ? launch_v<K, 16, TIn, TB, true, true>(a) : launch_v<K, 16, TIn, TB, true, false>(a);
    // about one token per sequence: B T rows over N sequences, at most 1.5 on average
    const bool one_token = 2LL * a.B * a.T <= 3LL * a.N;
    if (one_token)
        return a.inter_states ? launch_v<K, 64, TIn, TB, false, true>(a) : launch_v<K, 64, TIn, TB, false, false>(a);
    return a.inter_states ? launch_v<K, 32, TIn, TB, false, true>(a) : launch_v<K, 32, TIn, TB, false, false>(a);
}

template <int K>
hipError_t launch_k(const RecurrentArgs& a) {
    if (a.qkv_dtype == KDA_BF16) {
        return a.beta_dtype == KDA_BF16 ? launch_t<K, __bf16, __bf16>(a)
                                        : launch_t<K, __bf16, float>(a);
    }
    return a.beta_dtype == KDA_BF16 ? launch_t<K, float, __bf16>(a)
                                    : launch_t<K, float, float>(a);
}

}  // namespace

hipError_t launch_recurrent(const RecurrentArgs& a) {
    return a.K == 128 ? launch_k<128>(a) : launch_k<64>(a);
}

}  // namespace kda
