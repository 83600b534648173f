// Device-side helpers shared by the forward (ss_kernels.hip) and backward
// (ss_bwd.hip) kernels: work geometry, operand access, the step size and the
// pointwise functions.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "ss_internal.h"

namespace ssk {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int N = kDState;
constexpr int kWave = 64;
constexpr int kGroups = kScanWaves;  // waves per scan workgroup = state groups
constexpr int kNS = N / kGroups;  // state entries per wave
constexpr int kThreads = kWave * kGroups;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// fp32 -> bf16, round to nearest even (gfx950 converts in one instruction,
// v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

template <int DT>
struct Elem;
template <>
struct Elem<0> {  // fp32 operands
    using T = float;
    static __device__ __forceinline__ float load(const T* p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void store(T* p, int64_t i, float v) { p[i] = v; }
};
template <>
struct Elem<1> {  // bf16 operands, fp32 arithmetic
    using T = uint16_t;
    static __device__ __forceinline__ float load(const T* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
    static __device__ __forceinline__ void store(T* p, int64_t i, float v) { p[i] = f32_to_bf16_bits(v); }
};

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// silu(z) = z * sigmoid(z) = z / (1 + exp(-z))
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + exp2_hw(-z * kLog2e)); }

// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(t), t = e^-|v| in (0, 1]: no
// overflow.  log1p(t) = log(w) + log(1 + r/w) with w = 1 + t rounded and r the
// rounding error of w, which is exact (w - 1 is exact for w in [1, 2], and
// t - (w - 1) is exact because both are within a factor of two or w - 1 = 0).
// |r| <= 2^-24, so log(1 + r/w) = r/w to fp32 precision, and 2 - w stands in
// for 1/w within 12.5% (a relative 3e-9 on the result).  Where w rounds to 1
// the result is t itself.  Two hardware transcendentals (exp2, log2).
constexpr float kLn2 = 0.69314718f;
__device__ __forceinline__ float softplus(float v)
{
    const float t = exp2_hw(-fabsf(v) * kLog2e);
    const float w = 1.0f + t;
    const float r = t - (w - 1.0f);
    const float l1p = fmaf(__builtin_amdgcn_logf(w), kLn2, r * (2.0f - w));
    return fmaxf(v, 0.0f) + l1p;
}

// The step size of one (row, channel): the raw delta plus the channel's bias,
// through softplus when the call asks for it (LTI chapter, section 3.1.4.2:
// softplus of a per-channel parameter plus a projection of the input).
template <int MODE>
__device__ __forceinline__ float step_size(float raw, float bias)
{
    const float v = raw + bias;
    return (MODE & kOptSoftplus) ? softplus(v) : v;
}

// Zero-order hold (Mamba walk-through, section 2.2): Bbar = (dA)^-1 (e^{dA} - 1) dB,
// i.e. the Euler term delta*B times phi(x) = (e^x - 1)/x at x = delta*A.  Given
// x2 = x * log2 e, e = 2^x2 (already formed for Abar) and inv_x = 1/x: where
// e - 1 would cancel (|x| < 1/16) a degree-3 series;
// elsewhere (e - 1) * inv_x.  phi(0) = 1 comes from the series, so an infinite
// inv_x at delta = 0 or A = 0 is never used.  Worst case about 1e-6 relative:
// series truncation x^4/5! at the bound, or an ulp of e over |x| just above it.
constexpr float kZohSeriesBound = 0.090168440f;  // |x2| below which the series is used (|x| < 1/16)
__device__ __forceinline__ float zoh_phi(float x2, float e, float inv_x)
{
    constexpr float c1 = 0.34657359f;   // ln2 / 2!
    constexpr float c2 = 0.080075502f;  // ln2^2 / 3!
    constexpr float c3 = 0.013876027f;  // ln2^3 / 4!
    const float series = fmaf(x2, fmaf(x2, fmaf(x2, c3, c2), c1), 1.0f);
    const float direct = (e - 1.0f) * inv_x;
    return fabsf(x2) < kZohSeriesBound ? series : direct;
}

// The backward of the zero-order hold.  Its input coefficient beta = delta *
// phi(x) = (e^x - 1)/A has dbeta/ddelta = e^x and dbeta/dA = delta^2 psi(x),
// psi = phi' = (x e^x - e^x + 1)/x^2 = (e^x - phi)/x.  This returns
// dbeta/dA / delta: (e - phi) * inv_A, or, where e - phi would cancel
// (|x| < 1/4), delta times the degree-5 series sum_k (k+1) x^k / (k+2)!
// (truncation 1e-7 relative at the bound; the closed form just above it
// loses about 3e-6 to the rounding of e and phi).
constexpr float kZohPsiBound = 0.36067376f;  // |x2| below which psi's series is used (|x| < 1/4)
__device__ __forceinline__ float zoh_dbeta_dA_over_delta(float x2, float e, float phi, float inv_A, float delta)
{
    // (k+1) ln2^k / (k+2)!: the coefficients for x2 = x log2 e
    constexpr float c1 = 0.23104906f, c2 = 0.060056627f, c3 = 0.011100822f, c4 = 0.0016030215f,
                    c5 = 0.00019047940f;
    const float series = fmaf(x2, fmaf(x2, fmaf(x2, fmaf(x2, fmaf(x2, c5, c4), c3), c2), c1), 0.5f);
    return fabsf(x2) < kZohPsiBound ? delta * series : (e - phi) * inv_A;
}

// Scalar (wave-uniform) reads go through the constant address space so they
// are issued as scalar loads.
#define SS_CONST __attribute__((address_space(4)))

// Raw buffer access for the (B, L, D) row streams.  The resource is based at
// the chunk's first row; the lane's channel is the vector offset and the row a
// scalar offset.  Lanes past the last channel get an out-of-range vector
// offset: their loads read 0 and their stores are dropped by the range check.
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw (untyped) buffer, gfx9 family
constexpr uint32_t kIdleOffset = 0x80000000u;

template <int DT>
struct Buf;
template <>
struct Buf<0> {
    static constexpr uint32_t kBytes = 4;
    using Raw = uint32_t;
    static __device__ __forceinline__ Raw load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
    {
        return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
    }
    static __device__ __forceinline__ float widen(Raw v) { return __uint_as_float(v); }
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float v)
    {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);
    }
};
template <>
struct Buf<1> {
    static constexpr uint32_t kBytes = 2;
    using Raw = uint16_t;
    static __device__ __forceinline__ Raw load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
    {
        return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
    }
    static __device__ __forceinline__ float widen(Raw v) { return __uint_as_float(uint32_t(v) << 16); }
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float v)
    {
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(v), r, voff, soff, 0);
    }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), int(kRsrcWord3));
}

// Sixteen 32-bit words: one scalar load of a wave's B (or C) entries for
// 16 / kNS consecutive rows of the fp32 panel.
typedef uint32_t Words16 __attribute__((ext_vector_type(16)));

template <int V>
using Slot = std::integral_constant<int, V>;

// An empty asm statement that reads and rewrites a whole group of values: all of
// them are computed before it and nothing that consumes them moves above it.
template <int R, int C>
__device__ __forceinline__ void pin_rows(float (&v)[R][C])
{
    static_assert(C == 4 || C == 2 || C == 8, "row width");
#pragma unroll
    for (int r = 0; r + 1 < R; r += 2) {
        if constexpr (C == 4)
            __asm__ volatile("" : "+v"(v[r][0]), "+v"(v[r][1]), "+v"(v[r][2]), "+v"(v[r][3]), "+v"(v[r + 1][0]),
                             "+v"(v[r + 1][1]), "+v"(v[r + 1][2]), "+v"(v[r + 1][3]));
        else if constexpr (C == 2)
            __asm__ volatile("" : "+v"(v[r][0]), "+v"(v[r][1]), "+v"(v[r + 1][0]), "+v"(v[r + 1][1]));
        else
            __asm__ volatile("" : "+v"(v[r][0]), "+v"(v[r][1]), "+v"(v[r][2]), "+v"(v[r][3]), "+v"(v[r][4]),
                             "+v"(v[r][5]), "+v"(v[r][6]), "+v"(v[r][7]));
    }
}

template <int... I, typename F>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}

// f(std::integral_constant<int, 0>{}) ... f(std::integral_constant<int, N-1>{}), unrolled
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Value K of the lane's row of 16 lanes, broadcast across that row (DPP
// row_newbcast:K).  Used as the first operand of a multiply, the compiler folds
// it into the multiply itself (v_mul_f32_dpp).
constexpr int kDppRowNewBcast = 0x150;
template <int K>
__device__ __forceinline__ float row_bcast(float v)
{
    static_assert(K >= 0 && K < 16, "a row has 16 lanes");
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowNewBcast + K, 0xf, 0xf, false));
}

// acc[r] = C[r][0] * hh[r][0] + C[r][1] * hh[r][1] for the 8 rows of a tile,
// with C[r][i] value 2r + i of the lane's row of 16 lanes in cv (as row_bcast).
// The compiler does not fold a row broadcast into an fma, so the 16 products
// are written out: a multiply and an fma per row, each reading cv through
// DPP.  The leading s_nop gives the two wait states a DPP read needs after a
// vector write of its source register (cv comes from a load, but the
// compiler could have copied it).
__device__ __forceinline__ void contract_rows_bcast(float (&acc)[8], float cv, const float (&hh)[8][2])
{
    __asm__("s_nop 1\n\t"
                     "v_mul_f32_dpp %0, %8, %9 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
                     "v_fmac_f32_dpp %0, %8, %10 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
                     "v_mul_f32_dpp %1, %8, %11 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
                     "v_fmac_f32_dpp %1, %8, %12 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
                     "v_mul_f32_dpp %2, %8, %13 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
                     "v_fmac_f32_dpp %2, %8, %14 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
                     "v_mul_f32_dpp %3, %8, %15 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
                     "v_fmac_f32_dpp %3, %8, %16 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
                     "v_mul_f32_dpp %4, %8, %17 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
                     "v_fmac_f32_dpp %4, %8, %18 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
                     "v_mul_f32_dpp %5, %8, %19 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
                     "v_fmac_f32_dpp %5, %8, %20 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
                     "v_mul_f32_dpp %6, %8, %21 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
                     "v_fmac_f32_dpp %6, %8, %22 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
                     "v_mul_f32_dpp %7, %8, %23 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
                     "v_fmac_f32_dpp %7, %8, %24 row_newbcast:15 row_mask:0xf bank_mask:0xf"
            : "=&v"(acc[0]), "=&v"(acc[1]), "=&v"(acc[2]), "=&v"(acc[3]), "=&v"(acc[4]), "=&v"(acc[5]),
              "=&v"(acc[6]), "=&v"(acc[7])
            : "v"(cv), "v"(hh[0][0]), "v"(hh[0][1]), "v"(hh[1][0]), "v"(hh[1][1]), "v"(hh[2][0]), "v"(hh[2][1]),
              "v"(hh[3][0]), "v"(hh[3][1]), "v"(hh[4][0]), "v"(hh[4][1]), "v"(hh[5][0]), "v"(hh[5][1]),
              "v"(hh[6][0]), "v"(hh[6][1]), "v"(hh[7][0]), "v"(hh[7][1]));
}

// DPP controls: row shifts by 1/2/4/8 lanes within rows of 16, and the
// broadcasts of lane 15 (into rows 1 and 3) and lane 31 (into rows 2 and 3).
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

// v plus the value CTRL brings from another lane (a DPP row shift or row
// broadcast); lanes the shift or ROW_MASK leaves out add 0.  Chained over row
// shifts 1, 2, 4, 8 and the broadcasts of lanes 15 and 31 it forms an
// inclusive prefix sum across the wave.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float add_from(float v)
{
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

constexpr int kDppRowRor8 = 0x128, kDppRowHalfMirror = 0x141, kDppQuadSwap1 = 0xB1, kDppQuadSwap2 = 0x4E;

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Channel sums of 8 per-lane values at once: afterwards every lane l holds
// the sum over the wave's 64 lanes of v[l / 8].  A butterfly that halves the
// number of live vectors at each step, pairing vector p with vector p + m:
//   swap of the 32-lane halves (v_permlane32_swap): vector p holds value p in
//     lanes 0-31 and value p + 4 in lanes 32-63, each a sum over two lanes;
//   swap of odd and even 16-lane rows (v_permlane16_swap): value
//     p + 2*((l/16)&1) + 4*(l/32);
//   within each row, the two 8-lane halves (row rotation by 8): value l/8;
//   then a sum over each 8 lanes (half-row mirror, quad permutations 1,0,3,2
//   and 2,3,0,1).
// 18 instructions for 8 sums, where one DPP tree per value costs 6 each.
__device__ __forceinline__ float sum8_across_lanes(const float (&v)[8])
{
    const int lane = threadIdx.x & 63;
    float w[4], x[2];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[p]), __float_as_uint(v[p + 4]), false, false);
        w[p] = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(w[p]), __float_as_uint(w[p + 2]), false, false);
        x[p] = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    }
    const bool hi8 = (lane & 8) != 0;
    float z = (hi8 ? x[1] : x[0]) + dpp<kDppRowRor8>(hi8 ? x[0] : x[1]);
    z += dpp<kDppRowHalfMirror>(z);
    z += dpp<kDppQuadSwap1>(z);
    return z + dpp<kDppQuadSwap2>(z);
}

}  // namespace
}  // namespace ssk
