// Device-side building blocks shared by the KDA kernels (gfx950 / CDNA4).
//
//  * element types: inputs are fp32 or bf16 (__bf16, converted with the hardware
//    round-to-nearest-even instruction);
//  * 16x16 MFMA tiles: bf16 uses v_mfma_f32_16x16x32_bf16 (8 bf16 per lane, K step 32),
//    fp32 uses v_mfma_f32_16x16x4_f32 (1 fp32 per lane, K step 4). In both, lane l feeds
//    row/column (l % 16) at contraction offset (l / 16) * per_lane, and receives
//    D[4 * (l / 16) + r][l % 16] in accumulator register r;
//  * LDS tiles of 16-byte chunks whose chunk index is XOR-swizzled with (row & 7), so
//    that MFMA fragment reads (16 rows, same column) and transposed 4-row writes do not
//    pile onto the same banks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) float f32x8;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// 2^x with the hardware transcendental (v_exp_f32): results under 2^-126 flush to zero
// (below anything the outputs can resolve), large x gives +inf.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float LOG2E = 1.4426950408889634f;

// ---------------------------------------------------------------------------------
// Fusable input preprocessing (fp32, per element or per row)
// ---------------------------------------------------------------------------------

// The gate activation: log2 decay = -e^A softplus(x) / ln 2 = amp log2(1 + 2^(x log2 e))
// with amp = -e^A, and, when has_lb, the natural-log value clamped from below at the bound
// (lb2 = bound * log2 e, the bound in log2 units). For x > 15 the softplus is x to fp32
// precision. Where 1 + 2^(x log2 e) rounds to 1 (x below about -17) the result is 0
// instead of a value under 6e-8 e^A: a decay factor off by less than 4e-8 e^A per token.
__device__ __forceinline__ float gate_log2_from_raw(float x, float amp, bool has_lb, float lb2) {
    const float y = x * LOG2E;
    const float sp2 = x > 15.f ? y : __builtin_amdgcn_logf(1.f + exp2_fast(y));   // softplus / ln 2
    const float g2 = amp * sp2;
    return has_lb ? fmaxf(g2, lb2) : g2;
}

// beta from its pre-activation: bscale * sigmoid(b) = bscale / (1 + 2^(-b log2 e)); below
// b of about -88 the exponential overflows to +inf and beta is 0.
__device__ __forceinline__ float beta_from_logit(float b, float bscale) {
    return bscale / (1.f + exp2_fast(-LOG2E * b));
}

// Reciprocal norm of a row whose squares sum to ss: 1 / sqrt(ss + 1e-6) (v_rsq_f32).
constexpr float L2NORM_EPS = 1e-6f;
__device__ __forceinline__ float l2norm_rstd(float ss) { return __builtin_amdgcn_rsqf(ss + L2NORM_EPS); }

// ---------------------------------------------------------------------------------
// MFMA 16x16 tile products: C[16x16] += A[16 x Kc] * B[16 x Kc]^T, both operands with
// the contraction index contiguous.
// ---------------------------------------------------------------------------------
template <typename TW> struct Mma;

template <> struct Mma<__bf16> {
    static constexpr int KS = 32;   // contraction covered by one instruction
    static constexpr int KPL = 8;   // contraction elements held by one lane
    typedef bf16x8 frag;
    __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mma<float> {
    static constexpr int KS = 4;
    static constexpr int KPL = 1;
    typedef float frag;
    __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// ---------------------------------------------------------------------------------
// Swizzled LDS tile: ROWS x COLS elements of TW, 16-byte chunks, chunk ^= (row & 7).
// ---------------------------------------------------------------------------------
template <typename TW, int ROWS, int COLS> struct Tile {
    static constexpr int EPC = 16 / (int)sizeof(TW);   // elements per chunk
    static constexpr int NCH = COLS / EPC;             // chunks per row
    static_assert(COLS % EPC == 0, "row must be whole chunks");
    static_assert(NCH % 8 == 0, "swizzle needs at least 8 chunks per row");
    static constexpr int ELEMS = ROWS * COLS;
    static constexpr int BYTES = ELEMS * (int)sizeof(TW);

    __device__ __forceinline__ static int idx(int row, int col) {
        const int ch = col / EPC;
        return row * COLS + ((ch ^ (row & 7)) * EPC) + (col % EPC);
    }
    // MFMA operand fragment: row `row`, contraction offset kbase + (lane/16)*KPL
    __device__ __forceinline__ static typename Mma<TW>::frag frag(const TW* t, int row, int k) {
        return *reinterpret_cast<const typename Mma<TW>::frag*>(t + idx(row, k));
    }
};

// ---------------------------------------------------------------------------------
// Fragment-order tile in global memory: an R x KC matrix stored as 64-lane blocks, one
// per (16-row band b, contraction step s), band-major; lane l of block (b, s) holds row
// 16b + (l % 16), columns s*KS + (l / 16)*KPL .. +KPL contiguously. A wave reads one
// MFMA operand fragment of a band with one contiguous 64 x 16-byte (bf16) load.
// ---------------------------------------------------------------------------------
template <typename TW, int R, int KC> struct FragTile {
    typedef Mma<TW> M;
    static constexpr int NS = KC / M::KS;
    static constexpr int ELEMS = R * KC;
    static_assert(R % 16 == 0 && KC % M::KS == 0, "whole bands and steps");
    __device__ __forceinline__ static int idx(int row, int col) {
        const int b = row >> 4, st = col / M::KS;
        const int l = (row & 15) + 16 * ((col % M::KS) / M::KPL);
        return ((b * NS + st) * 64 + l) * M::KPL + (col % M::KPL);
    }
    __device__ __forceinline__ static int frag(int b, int st, int lane) {
        return ((b * NS + st) * 64 + lane) * M::KPL;
    }
};

// The fp8 residual (lo8_encode) of a bf16 FragTile<__bf16, R, KC>: the eight bytes of
// fragment lane (band b, step st, lane) at uint2 index frag(b, st, lane), in the same
// order as the bf16 tile, and per (band, lane) one 32-bit word whose byte st is that
// fragment's scale byte (at most four steps per band).
template <int R, int KC> struct Lo8Tile {
    static constexpr int NS = KC / 32, BANDS = R / 16;
    static_assert(R % 16 == 0 && KC % 32 == 0 && NS <= 4, "whole bands, at most 4 steps");
    static constexpr size_t LO_BYTES = (size_t)R * KC;
    static constexpr size_t SC_BYTES = (size_t)BANDS * 64 * 4;
    __device__ __forceinline__ static int frag(int b, int st, int lane) { return (b * NS + st) * 64 + lane; }
    __device__ __forceinline__ static int scale(int b, int lane) { return b * 64 + lane; }
};
// scale byte st of a word
__device__ __forceinline__ uint32_t lo8_byte(uint32_t word, int st) { return (word >> (8 * st)) & 0xFFu; }

// Accumulator-order tile of fp32 values [R][64] read back as four consecutive rows of
// one column: block (column tile ct = col/16, row band rb = row/16), lane
// l = (col % 16) + 16 * ((row % 16) / 4) holds rows 16rb + 4(l/16) .. +3 of column
// 16ct + (l % 16) -- the layout a 16x16 MFMA result has in its four accumulator registers.
struct AccTile {
    __device__ __forceinline__ static int quad(int col, int row) {   // offset of the 4-row group
        return (((col >> 4) * 4 + (row >> 4)) * 64 + (col & 15) + 16 * ((row & 15) >> 2)) * 4;
    }
};

// Product of a 16-row band of A (rows a_row0..+15) with a 16-row band of B (rows
// b_row0..+15) over contraction [k0, k1), accumulated into acc.
template <typename TW, typename TA, typename TB>
__device__ __forceinline__ f32x4 tile_mma(f32x4 acc, const TW* A, int a_row0, const TW* B,
                                          int b_row0, int k0, int k1, int lane) {
    const int r = lane & 15;
    const int ko = (lane >> 4) * Mma<TW>::KPL;
    for (int k = k0; k < k1; k += Mma<TW>::KS) {
        auto a = TA::frag(A, a_row0 + r, k + ko);
        auto b = TB::frag(B, b_row0 + r, k + ko);
        acc = Mma<TW>::mma(a, b, acc);
    }
    return acc;
}

// Two independent tile products over the same compile-time contraction [0, NK): all
// fragments of a step are loaded before its MFMAs, and the two accumulation chains
// interleave, so LDS latency and MFMA latency overlap. A2/B2 may alias A1/B1.
template <typename TW, typename TA, typename TB, int NK>
__device__ __forceinline__ void tile_mma2(f32x4& acc1, const TW* A1, int a1_row0, const TW* B1,
                                          int b1_row0, bool do1, f32x4& acc2, const TW* A2,
                                          int a2_row0, const TW* B2, int b2_row0, bool do2,
                                          int lane) {
    const int r = lane & 15;
    const int ko = (lane >> 4) * Mma<TW>::KPL;
#pragma unroll
    for (int k = 0; k < NK; k += Mma<TW>::KS) {
        if (do1) {
            auto a = TA::frag(A1, a1_row0 + r, k + ko);
            auto b = TB::frag(B1, b1_row0 + r, k + ko);
            acc1 = Mma<TW>::mma(a, b, acc1);
        }
        if (do2) {
            auto a = TA::frag(A2, a2_row0 + r, k + ko);
            auto b = TB::frag(B2, b2_row0 + r, k + ko);
            acc2 = Mma<TW>::mma(a, b, acc2);
        }
    }
}

// Single tile product over a compile-time contraction [0, NK).
template <typename TW, typename TA, typename TB, int NK>
__device__ __forceinline__ f32x4 tile_mma_n(f32x4 acc, const TW* A, int a_row0, const TW* B,
                                            int b_row0, int lane) {
    const int r = lane & 15;
    const int ko = (lane >> 4) * Mma<TW>::KPL;
#pragma unroll
    for (int k = 0; k < NK; k += Mma<TW>::KS) {
        auto a = TA::frag(A, a_row0 + r, k + ko);
        auto b = TB::frag(B, b_row0 + r, k + ko);
        acc = Mma<TW>::mma(a, b, acc);
    }
    return acc;
}

// Store N consecutive elements (converted from fp32) with one vector write; the
// destination must be aligned to N elements and not cross a 16-byte chunk.
template <typename TW, int N>
__device__ __forceinline__ void store_run(TW* dst, const float* x) {
    typedef __attribute__((ext_vector_type(N))) TW vec;
    vec v;
#pragma unroll
    for (int e = 0; e < N; ++e) v[e] = from_f32<TW>(x[e]);
    *reinterpret_cast<vec*>(dst) = v;
}

// Store 4 consecutive rows (row0..row0+3) of one column from accumulator registers into
// a transposed tile T[col][row0..row0+3] (row0 % 4 == 0).
template <typename TW, typename TT>
__device__ __forceinline__ void store_col4(TW* t, int col, int row0, f32x4 v) {
    TW* p = t + TT::idx(col, row0);
    p[0] = from_f32<TW>(v[0]);
    p[1] = from_f32<TW>(v[1]);
    p[2] = from_f32<TW>(v[2]);
    p[3] = from_f32<TW>(v[3]);
}

// ---------------------------------------------------------------------------------
// Cross-lane building blocks. A 64-lane wave is four DPP rows of 16 lanes.
// ---------------------------------------------------------------------------------
// x of lane (l - N) within this lane's 16-lane row; 0 for the first N lanes of the row
template <int N> __device__ __forceinline__ float row_shr(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 0x110 + N, 0xf, 0xf, true));
}
// x of lane N of this lane's 16-lane row (row_newbcast)
template <int N> __device__ __forceinline__ float row_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 0x150 + N, 0xf, 0xf, false));
}
// inclusive prefix sum over the 16 lanes of each row (Hillis-Steele, four steps)
__device__ __forceinline__ float row_scan(float x) {
    x += row_shr<1>(x);
    x += row_shr<2>(x);
    x += row_shr<4>(x);
    x += row_shr<8>(x);
    return x;
}

// Two 16x16 accumulator tiles X and Y (lane l holds M[4(l/16) + r][l % 16], r = 0..3) are
// the top and bottom halves of a 32 x 16 matrix Z = [X; Y]. Afterwards lane l holds the
// eight consecutive rows Z[8(l/16) + e][l % 16], e = 0..7: the operand-fragment layout of
// the 16 x 32 matrix Z^T. Two lane-swap steps per register, no LDS.
__device__ __forceinline__ void acc_pair_to_frag(f32x4 x, f32x4 y, float out[8]) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        // {X0 X1 Y0 Y1}, {X2 X3 Y2 Y3}  (Xg = rows 4g..4g+3 of X, one 16-lane row each)
        // (scalar copies: __builtin_bit_cast of a vector element reads element 0)
        const float xr = x[r], yr = y[r];
        const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(xr), __float_as_uint(yr), false, false);
        const unsigned s0 = s[0], s1 = s[1];
        // {X0 X2 Y0 Y2}, {X1 X3 Y1 Y3}
        const auto t = __builtin_amdgcn_permlane16_swap(s0, s1, false, false);
        const unsigned t0 = t[0], t1 = t[1];
        out[r] = __uint_as_float(t0);
        out[4 + r] = __uint_as_float(t1);
    }
}

// bf16 hi/lo split of 8 fp32 values: x = hi + lo to about 16 significant bits
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        hi[e] = (__bf16)x[e];
        lo[e] = (__bf16)(x[e] - (float)hi[e]);
    }
}
// Rounding residuals in fp8 (OCP e4m3: 4 significant bits, largest finite value 448) with
// one power-of-two scale per fragment lane: the lane's eight residuals r are stored as
// e4m3(r 2^s), s set from their largest magnitude m so that m 2^s lies in [128, 256)
// (nothing reaches 448, where the conversion would give NaN), and beside them the byte
// 127 - s, which is the exponent field of the decoding factor 2^-s. hi + lo then
// carries about 12 significant bits of each value, relative to the largest of its
// lane's eight; residuals of zero rows are stored as zeros.
__device__ __forceinline__ uint2 lo8_encode(const float* r, uint32_t& sbyte) {
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(r[e]));
    // m < 2^(eb - 126) for the biased exponent eb of m, so m 2^(134 - eb) < 256
    const int eb = (int)((__float_as_uint(m) >> 23) & 0xFFu);
    const int s = min(134 - eb, 126);
    const float mul = __uint_as_float((uint32_t)(127 + s) << 23);
    uint32_t w0 = 0, w1 = 0;
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(r[0] * mul, r[1] * mul, w0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(r[2] * mul, r[3] * mul, w0, true);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(r[4] * mul, r[5] * mul, w1, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(r[6] * mul, r[7] * mul, w1, true);
    sbyte = (uint32_t)(127 - s);
    return make_uint2(w0, w1);
}
// The inverse: eight e4m3 residuals times 2^(sbyte - 127), as a bf16 fragment (exact:
// a 4-bit significand times a power of two).
__device__ __forceinline__ bf16x8 lo8_decode(uint2 raw, uint32_t sbyte) {
    const float f = __uint_as_float(sbyte << 23);
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, f, true);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
// hi and the fp8 residual of eight fp32 values
__device__ __forceinline__ void split8_lo8(const float* x, bf16x8& hi, uint2& lo, uint32_t& sbyte) {
    float r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        hi[e] = (__bf16)x[e];
        r[e] = x[e] - (float)hi[e];
    }
    lo = lo8_encode(r, sbyte);
}

__device__ __forceinline__ void split4(f32x4 x, bf16x4& hi, bf16x4& lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        hi[e] = (__bf16)x[e];
        lo[e] = (__bf16)(x[e] - (float)hi[e]);
    }
}

// hi*hi + lo*hi + hi*lo on the 16x16x32 bf16 matrix cores (the lo*lo term is below fp32
// rounding of the result)
__device__ __forceinline__ f32x4 mma3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, c, 0, 0, 0);
}

// 16x16x16 bf16 product (lane l: row l % 16, contraction 4(l/16) .. +3), same split
typedef __attribute__((ext_vector_type(4))) short s16x4;
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16x3(f32x4 a, f32x4 b, f32x4 c) {
    bf16x4 ah, al, bh, bl;
    split4(a, ah, al);
    split4(b, bh, bl);
    c = mma16(ah, bl, c);
    c = mma16(al, bh, c);
    return mma16(ah, bh, c);
}

// B operand of a 16x16x32 product that selects contraction columns 16h .. 16h+15:
// B[n][k] = (k == n + 16h). With it, an A fragment (row m, eight consecutive columns per
// lane) comes out as A[m][16h + n] in accumulator layout -- four consecutive rows per lane.
// Exact: every product is x * 1 or x * 0.
__device__ __forceinline__ bf16x8 eye_frag(int lane, int h) {
    const int n = lane & 15, k0 = 8 * (lane >> 4);
    bf16x8 b;
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = (__bf16)((k0 + e == n + 16 * h) ? 1.f : 0.f);
    return b;
}

// Barrier for blocks that exchange data only through LDS: the fences are restricted to
// the LDS address space, so outstanding global loads (prefetches) and stores stay in
// flight across it (a full __syncthreads() must also drain global stores, and on gfx9
// one counter covers loads and stores, which would wait for every prefetch too).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Block-wide OR of a flag (256-thread blocks).
__device__ __forceinline__ int block_any(int pred) { return __syncthreads_or(pred); }

}  // namespace kda
