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
// Work decomposition. One wavefront owns one (sequence n, value head hv, 64-column
// slice of V) and walks its tokens in order. Lane l holds the state block
//     rows  d = (l / 16) * (K / 4) + i,   i = 0 .. K/4 - 1
//     cols  c = v0 + 4 * (l % 16) + j,    j = 0 .. 3
// in registers (K = 128: 32 x 4 fp32 per lane), so the state is read from HBM once and
// written once with 16-byte accesses. Per token the lane folds the decay into its block,
// forms partial sums of S~^T k and S~^T q over its rows (S~ = decayed state), and the
// four row groups combine them with two cross-lane exchanges. Then
//     delta = beta (v - S~^T k),   o = scale (S~^T q + delta (k . q)),   S = S~ + k delta^T
// which is o = scale S_t^T q without a second pass over the state.
//
// The grid is flat and 1-D (four wavefronts per 256-thread block), so N * HV * V/64 may
// exceed 65,535. States may be laid out [K][V] or transposed, [V][K] (fla's state_v_first);
// the state after every token can be written out as well (fla's
// return_intermediate_states). Packed offsets are validated per slot on every call: a slot with
// bos < 0, bos > eos, eos > T, or slot 0 not starting at 0, is skipped and flagged.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

__device__ __forceinline__ void load_row_block(const __bf16* p, float* out, int n) {
    // n consecutive bf16 values (n a multiple of 8, 16-byte aligned)
    for (int i = 0; i < n; i += 8) {
        bf16x8 x = *reinterpret_cast<const bf16x8*>(p + i);
#pragma unroll
        for (int j = 0; j < 8; ++j) out[i + j] = (float)x[j];
    }
}

__device__ __forceinline__ void load_row_block(const float* p, float* out, int n) {
    for (int i = 0; i < n; i += 4) {
        f32x4 x = *reinterpret_cast<const f32x4*>(p + i);
#pragma unroll
        for (int j = 0; j < 4; ++j) out[i + j] = x[j];
    }
}

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

__device__ __forceinline__ float sum_row_groups(float x) {
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}

// The lane's block of a state (rows d0 .. d0+R-1, columns c0 .. c0+3) in either layout:
// [K][V] (row d at base + d V) or, with vk, [V][K] (column c at base + c K); 16-byte
// accesses in both.
template <int R>
__device__ __forceinline__ void load_state(const float* base, int K, int V, bool vk, int d0, int c0,
                                           float (&S)[R][4]) {
    if (!vk) {
#pragma unroll
        for (int i = 0; i < R; ++i) load4(base + (size_t)(d0 + i) * V + c0, S[i]);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < R; i += 4) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(base + (size_t)(c0 + j) * K + d0 + i);
#pragma unroll
                for (int e = 0; e < 4; ++e) S[i + e][j] = x[e];
            }
    }
}

template <int R>
__device__ __forceinline__ void store_state(float* base, int K, int V, bool vk, int d0, int c0,
                                            const float (&S)[R][4]) {
    if (!vk) {
#pragma unroll
        for (int i = 0; i < R; ++i) store4(base + (size_t)(d0 + i) * V + c0, S[i]);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < R; i += 4)
                *reinterpret_cast<f32x4*>(base + (size_t)(c0 + j) * K + d0 + i) =
                    f32x4{S[i][j], S[i + 1][j], S[i + 2][j], S[i + 3][j]};
    }
}

template <int R>
__device__ __forceinline__ void l2norm_rows(float (&x)[R]) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i) ss = fmaf(x[i], x[i], ss);
    const float rn = l2norm_rstd(sum_row_groups(ss));
#pragma unroll
    for (int i = 0; i < R; ++i) x[i] *= rn;
}

template <int K, typename TIn, typename TB>
__global__ __launch_bounds__(256) void recurrent_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const float* __restrict__ g, const InputSpec in, const TB* __restrict__ beta,
    const float* initial_state, const int32_t* __restrict__ cu_seqlens,
    TIn* __restrict__ o, float* final_state, float* inter_states, int state_vk, int T, int H,
    int HV, int V, int nvt, long long n_items, float scale, int32_t* dev_status) {
    constexpr int R = K / 4;  // rows per lane
    const int lane = threadIdx.x & 63;
    const long long item = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= n_items) return;

    const int vt = (int)(item % nvt);
    const long long chain = item / nvt;
    const int hv = (int)(chain % HV);
    const int n = (int)(chain / HV);
    const int h = hv / (HV / H);
    const int cg = lane & 15;
    const int rg = lane >> 4;
    const int c0 = vt * 64 + 4 * cg;
    const int d0 = rg * R;

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
    float S[R][4];
    if (initial_state) {
        load_state<R>(initial_state + sbase, K, V, state_vk, d0, c0, S);
    } else {
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) S[i][j] = 0.0f;
    }

    const float amp = in.gate_mode != GATE_LOG2 ? -expf(in.A_log[hv]) : 0.f;
    const float lb2 = in.lower_bound * LOG2E;
    for (int t = bos; t < eos; ++t) {
        const long long r = row0 + t;
        float kk[R], qq[R], ee[R], vv[4];
        load_row_block(k + ((size_t)r * H + h) * K + d0, kk, R);
        load_row_block(q + ((size_t)r * H + h) * K + d0, qq, R);
        const size_t gofs = ((size_t)r * HV + hv) * K + d0;
        if (in.gate_mode == GATE_LOG2) {
            load_row_block(g + gofs, ee, R);
        } else {
            // the fused gate activation on the raw gate input
            if (in.gate_mode == GATE_RAW_BF16)
                load_row_block(static_cast<const __bf16*>(in.g_raw) + gofs, ee, R);
            else
                load_row_block(static_cast<const float*>(in.g_raw) + gofs, ee, R);
            if (in.dt_bias) {
                float db[R];
                load_row_block(in.dt_bias + (size_t)hv * K + d0, db, R);
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
        if (in.l2norm_q) l2norm_rows(qq);
        if (in.l2norm_k) l2norm_rows(kk);

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
        kq = sum_row_groups(kq);
        float delta[4], out[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            p[j] = sum_row_groups(p[j]);
            rq[j] = sum_row_groups(rq[j]);
            delta[j] = b * (vv[j] - p[j]);
            out[j] = scale * fmaf(delta[j], kq, rq[j]);
        }
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) S[i][j] = fmaf(kk[i], delta[j], S[i][j]);
        if (rg == 0) store4(o + ((size_t)r * HV + hv) * V + c0, out);
        // the state after this token, in the states' layout
        if (inter_states) store_state<R>(inter_states + ((size_t)r * HV + hv) * (size_t)K * V, K, V, state_vk, d0, c0, S);
    }

    if (final_state) store_state<R>(final_state + sbase, K, V, state_vk, d0, c0, S);
}

template <int K, typename TIn, typename TB>
hipError_t launch_t(const RecurrentArgs& a) {
    const int nvt = a.V / 64;
    const long long n_items = (long long)a.N * a.HV * nvt;
    if (n_items == 0) return hipSuccess;
    const long long blocks = (n_items + 3) / 4;
    hipLaunchKernelGGL((recurrent_kernel<K, TIn, TB>), dim3((unsigned)blocks), dim3(256), 0,
                       a.stream, (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v, a.g, a.in,
                       (const TB*)a.beta, a.initial_state, a.cu_seqlens, (TIn*)a.o,
                       a.final_state, a.inter_states, a.state_vk, a.T, a.H, a.HV, a.V, nvt, n_items, a.scale,
                       a.dev_status);
    return hipGetLastError();
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
