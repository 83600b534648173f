// gfx950 kernels of the selective scan (Mamba walk-through, section 3.3
// "selective_scan"; discrete recurrence of section 2.2; D skip and silu(z)
// gate of section 3.4) and of the single-token recurrent update.
//
// Work decomposition
//  * one lane owns one channel (b, d) and all 16 state entries h[n] in
//    registers; a wave covers 64 consecutive d of one batch row, so B[b,t,:]
//    and C[b,t,:] are wave-uniform (scalar loads) and u/delta/z/y rows are
//    read and written as 64 consecutive elements;
//  * the sequence is cut into chunks (LTI chapter 3.1, section 3.1.5.2: the
//    recurrence is a scan over an associative operator).  For K > 1 chunks:
//      1. scan_chunk_kernel<aggregate> runs chunks 0..K-2 from a zero state and
//         keeps only the chunk's end state S_c and its delta sum;
//      2. carry_kernel turns the per-chunk affine pairs (P_c, S_c), with
//         P_c = exp(A * sum_t delta_t), into carries by a wave-level
//         inclusive prefix combine over chunks (64 chunks per pass, the last
//         lane's value carried to the next pass);
//      3. scan_chunk_kernel<emit> reruns every chunk from its carry and writes y.
//    Only y, the chunk carries and h_last ever reach memory; the per-timestep
//    states and the discretised operands exp(delta*A), delta*B*u stay in
//    registers (the fused, state-in-fast-memory point of section 3.3 and of
//    LTI chapter section 3.1.5.3).
//  * exp(x) is evaluated as exp2(x * log2 e) on the hardware exp2 unit, with
//    A pre-scaled by log2 e once per lane.
#include <hip/hip_runtime.h>

#include "ss_internal.h"

namespace ssk {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int N = kDState;
constexpr int kWave = 64;

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

// B[b,t,:] and C[b,t,:] are the same for every lane of a wave: read them
// through the constant address space so they arrive as scalar loads, and
// widen bf16 on the scalar unit.
#define SS_CONST __attribute__((address_space(4)))

template <int DT>
struct Row;
template <>
struct Row<0> {  // 16 fp32 = 16 dwords per timestep
    static constexpr int kWords = 16;
    static __device__ __forceinline__ void widen(const uint32_t (&w)[kWords], float (&v)[N])
    {
#pragma unroll
        for (int n = 0; n < N; ++n) v[n] = __uint_as_float(w[n]);
    }
};
template <>
struct Row<1> {  // 16 bf16 = 8 dwords per timestep
    static constexpr int kWords = 8;
    static __device__ __forceinline__ void widen(const uint32_t (&w)[kWords], float (&v)[N])
    {
#pragma unroll
        for (int i = 0; i < kWords; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};

template <int W>
__device__ __forceinline__ void load_words(const SS_CONST uint32_t* p, uint32_t (&w)[W])
{
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = p[i];
}

// Raw buffer access for the (B, L, D) row streams.  The resource is based at
// the chunk's first row; the lane's channel is the vector offset and the row
// is a scalar offset, so moving along t costs no vector instruction.  Lanes
// past the last channel get an out-of-range vector offset: their loads read
// 0 and their stores are dropped by the hardware range check.
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

constexpr int kBlock = 8;  // timesteps per vector-prefetch block

// ---------------------------------------------------------------------------
// Chunk kernel.  grid = (ceil(dim/64), batch, chunks), block = 64.
// EMIT: start from the chunk's carry (or h0), write y and, for the last chunk,
//       h_last.
// !EMIT (aggregate): start from zero, write the chunk's end state into state
//       slot c+1 and its delta sum.
// Software pipeline: u/delta/z of the next kBlock timesteps are requested
// while the current block is computed (rows past the chunk end are clamped to
// its last row); the scalar B/C row of timestep t+1 is requested right after
// row t has been consumed (scalar loads may return out of order, so a wait
// always covers every one in flight).
// Host guarantees: chunk_len * dim * element size < 2^31.
// ---------------------------------------------------------------------------
template <int DT, bool EMIT, bool HAS_D, bool HAS_Z>
__global__ __launch_bounds__(kWave) void scan_chunk_kernel(ScanArgs a)
{
    using T = typename Elem<DT>::T;
    using R = Row<DT>;
    using V = Buf<DT>;
    using Raw = typename V::Raw;
    constexpr int W = R::kWords;

    const int64_t D = a.dim, L = a.seqlen, BD = a.batch * a.dim;
    const int64_t d_raw = int64_t(blockIdx.x) * kWave + threadIdx.x;
    const bool active = d_raw < D;
    const int64_t d = active ? d_raw : D - 1;  // idle lanes shadow the last channel
    const int64_t b = blockIdx.y;
    const int64_t c = blockIdx.z;
    const int64_t t0 = c * a.chunk_len;
    const int len = int(((t0 + a.chunk_len < L) ? t0 + a.chunk_len : L) - t0);
    const int64_t bd = b * D + d;
    const int64_t row0 = (b * L + t0) * D;  // first element of the chunk's first row

    const uint32_t row_bytes = uint32_t(D) * V::kBytes;
    const uint32_t span = uint32_t(len) * row_bytes;
    const uint32_t voff = active ? uint32_t(d_raw) * V::kBytes : kIdleOffset;
    const __amdgpu_buffer_rsrc_t r_u = make_rsrc(static_cast<const T*>(a.u) + row0, span);
    const __amdgpu_buffer_rsrc_t r_dl = make_rsrc(static_cast<const T*>(a.delta) + row0, span);
    const __amdgpu_buffer_rsrc_t r_z = make_rsrc(HAS_Z ? static_cast<const T*>(a.z) + row0 : nullptr, span);
    const __amdgpu_buffer_rsrc_t r_y = make_rsrc(EMIT ? static_cast<T*>(a.y) + row0 : nullptr, span);
    // address-space casts need the C cast form
    const SS_CONST uint32_t* pB = (const SS_CONST uint32_t*)(static_cast<const T*>(a.B) + (b * L + t0) * N);
    const SS_CONST uint32_t* pC = (const SS_CONST uint32_t*)(static_cast<const T*>(a.C) + (b * L + t0) * N);

    float A2[N];
#pragma unroll
    for (int n = 0; n < N; ++n) A2[n] = a.A[d * N + n] * kLog2e;

    float h[N];
    const bool from_ws = EMIT && a.n_chunks > 1;
    const bool from_h0 = EMIT && a.n_chunks == 1 && a.h0 != nullptr;
    if (from_ws || from_h0) {
        const float* init = from_ws ? a.ws_state + (c * BD + bd) * N : a.h0 + bd * N;
#pragma unroll
        for (int n = 0; n < N; ++n) h[n] = init[n];
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) h[n] = 0.0f;
    }

    const float dskip = (EMIT && HAS_D) ? a.Dskip[d] : 0.0f;
    float dsum = 0.0f;

    // row r of the chunk, clamped to the last one, as a scalar byte offset
    auto row_off = [&](int r) -> uint32_t { return uint32_t(r < len ? r : len - 1) * row_bytes; };

    Raw dl_c[kBlock], x_c[kBlock], z_c[kBlock];
#pragma unroll
    for (int j = 0; j < kBlock; ++j) {
        const uint32_t so = row_off(j);
        dl_c[j] = V::load(r_dl, voff, so);
        x_c[j] = V::load(r_u, voff, so);
        if (EMIT && HAS_Z) z_c[j] = V::load(r_z, voff, so);
    }
    uint32_t bw[W], cw[W];
    load_words(pB, bw);
    if (EMIT) load_words(pC, cw);

    for (int i0 = 0; i0 < len; i0 += kBlock) {
        Raw dl_n[kBlock], x_n[kBlock], z_n[kBlock];
#pragma unroll
        for (int j = 0; j < kBlock; ++j) {
            const uint32_t so = row_off(i0 + kBlock + j);
            dl_n[j] = V::load(r_dl, voff, so);
            x_n[j] = V::load(r_u, voff, so);
            if (EMIT && HAS_Z) z_n[j] = V::load(r_z, voff, so);
        }
#pragma unroll
        for (int j = 0; j < kBlock; ++j) {
            const int i = i0 + j;
            if (i >= len) break;
            float bv[N], cv[N];
            R::widen(bw, bv);
            if (EMIT) R::widen(cw, cv);
            // keep the next row's scalar loads behind this row's first use
            if (EMIT)
                __asm__ volatile("" ::"s"(bw[0]), "s"(cw[0]) : "memory");
            else
                __asm__ volatile("" ::"s"(bw[0]) : "memory");
            if (i + 1 < len) {
                load_words(pB + (i + 1) * W, bw);
                if (EMIT) load_words(pC + (i + 1) * W, cw);
            }
            const float dl = V::widen(dl_c[j]);
            const float x = V::widen(x_c[j]);
            const float xb = dl * x;
            float acc = 0.0f;
#pragma unroll
            for (int n = 0; n < N; ++n) {
                const float abar = exp2_hw(dl * A2[n]);
                h[n] = fmaf(abar, h[n], xb * bv[n]);
                if (EMIT) acc = fmaf(cv[n], h[n], acc);
            }
            if (EMIT) {
                if (HAS_D) acc = fmaf(dskip, x, acc);
                if (HAS_Z) acc *= silu(V::widen(z_c[j]));
                V::store(r_y, voff, uint32_t(i) * row_bytes, acc);
            } else {
                dsum += dl;
            }
        }
#pragma unroll
        for (int j = 0; j < kBlock; ++j) {
            dl_c[j] = dl_n[j];
            x_c[j] = x_n[j];
            if (EMIT && HAS_Z) z_c[j] = z_n[j];
        }
    }

    if (!active) return;
    if (EMIT) {
        if (c == a.n_chunks - 1 && a.h_last) {
#pragma unroll
            for (int n = 0; n < N; ++n) a.h_last[bd * N + n] = h[n];
        }
    } else {
        float* dst = a.ws_state + ((c + 1) * BD + bd) * N;
#pragma unroll
        for (int n = 0; n < N; ++n) dst[n] = h[n];
        a.ws_dsum[c * BD + bd] = dsum;
    }
}

// ---------------------------------------------------------------------------
// Carry kernel.  grid = batch*dim (one wave per channel), block = 64.
// Lane i of pass p owns chunk c = 64p + i and its affine pair
// (P_c, S_c) = (exp(A * sum delta over c), end state of c from zero).
// An inclusive Hillis-Steele combine over the lanes, earlier pair first,
//   (a1, b1) then (a2, b2) -> (a2*a1, a2*b1 + b2),
// gives each lane the composite map of chunks 0..c; applied to the incoming
// state it yields the carry H_c (state after chunk c), stored in slot c+1.
// Slot 0 receives the initial state.  Lanes past the last chunk hold the
// identity pair (1, 0), so lane 63 always ends with the pass's total.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kWave) void carry_kernel(ScanArgs a)
{
    const int64_t bd = blockIdx.x;
    const int64_t BD = a.batch * a.dim;
    const int64_t d = bd % a.dim;
    const int lane = threadIdx.x;
    const int64_t n_carry = a.n_chunks - 1;

    float A2[N], hin[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        A2[n] = a.A[d * N + n] * kLog2e;
        hin[n] = a.h0 ? a.h0[bd * N + n] : 0.0f;
    }
    if (lane < N) a.ws_state[bd * N + lane] = a.h0 ? a.h0[bd * N + lane] : 0.0f;

    for (int64_t base = 0; base < n_carry; base += kWave) {
        const int64_t c = base + lane;
        const bool valid = c < n_carry;
        const float dsum = valid ? a.ws_dsum[c * BD + bd] : 0.0f;
        float* slot = a.ws_state + ((c + 1) * BD + bd) * N;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            float P = valid ? exp2_hw(A2[n] * dsum) : 1.0f;
            float S = valid ? slot[n] : 0.0f;
#pragma unroll
            for (int k = 1; k < kWave; k <<= 1) {
                const float Pp = __shfl_up(P, k, kWave);
                const float Sp = __shfl_up(S, k, kWave);
                if (lane >= k) {
                    S = fmaf(P, Sp, S);
                    P *= Pp;
                }
            }
            const float H = fmaf(P, hin[n], S);
            if (valid) slot[n] = H;
            hin[n] = __shfl(H, kWave - 1, kWave);
        }
    }
}

// ---------------------------------------------------------------------------
// Recurrent step.  Four lanes per channel (b, d), each with 4 of the 16 state
// entries (16-byte loads/stores of h), the quad's partial C.h summed with two
// butterfly exchanges.  grid = ceil(batch*dim*4 / 256), block = 256.
// ---------------------------------------------------------------------------
template <int DT, bool HAS_D, bool HAS_Z>
__global__ __launch_bounds__(256) void step_kernel(StepArgs a)
{
    using E = Elem<DT>;
    using T = typename E::T;
    const T* __restrict__ u = static_cast<const T*>(a.u);
    const T* __restrict__ delta = static_cast<const T*>(a.delta);
    const T* __restrict__ Bm = static_cast<const T*>(a.B);
    const T* __restrict__ Cm = static_cast<const T*>(a.C);
    const T* __restrict__ z = static_cast<const T*>(a.z);
    T* __restrict__ y = static_cast<T*>(a.y);

    const int64_t total = a.batch * a.dim * 4;
    const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const bool active = gid < total;
    const int64_t g = active ? gid : total - 1;  // whole quads are idle together
    const int64_t bd = g >> 2;
    const int q = int(g & 3);
    const int64_t b = bd / a.dim, d = bd - b * a.dim;

    float4 hv = *reinterpret_cast<const float4*>(a.h + bd * N + q * 4);
    const float4 av = *reinterpret_cast<const float4*>(a.A + d * N + q * 4);
    const float dl = E::load(delta, bd);
    const float x = E::load(u, bd);
    const float xb = dl * x;
    const int64_t s0 = b * N + q * 4;

    float hs[4] = {hv.x, hv.y, hv.z, hv.w};
    const float as[4] = {av.x, av.y, av.z, av.w};
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float abar = exp2_hw(dl * (as[i] * kLog2e));
        hs[i] = fmaf(abar, hs[i], xb * E::load(Bm, s0 + i));
        part = fmaf(E::load(Cm, s0 + i), hs[i], part);
    }
    float acc = part + __shfl_xor(part, 1, 4);
    acc += __shfl_xor(acc, 2, 4);

    if (!active) return;
    *reinterpret_cast<float4*>(a.h + bd * N + q * 4) = make_float4(hs[0], hs[1], hs[2], hs[3]);
    if (q == 0) {
        if (HAS_D) acc = fmaf(a.Dskip[d], x, acc);
        if (HAS_Z) acc *= silu(E::load(z, bd));
        E::store(y, bd, acc);
    }
}

template <int DT, bool HAS_D, bool HAS_Z>
hipError_t launch_scan_t(const ScanArgs& a, hipStream_t s)
{
    const unsigned nblk = unsigned((a.dim + kWave - 1) / kWave);
    if (a.n_chunks > 1) {
        scan_chunk_kernel<DT, false, false, false>
            <<<dim3(nblk, unsigned(a.batch), unsigned(a.n_chunks - 1)), dim3(kWave), 0, s>>>(a);
        carry_kernel<<<dim3(unsigned(a.batch * a.dim)), dim3(kWave), 0, s>>>(a);
    }
    scan_chunk_kernel<DT, true, HAS_D, HAS_Z>
        <<<dim3(nblk, unsigned(a.batch), unsigned(a.n_chunks)), dim3(kWave), 0, s>>>(a);
    return hipGetLastError();
}

template <int DT, bool HAS_D, bool HAS_Z>
hipError_t launch_step_t(const StepArgs& a, hipStream_t s)
{
    const int64_t threads = a.batch * a.dim * 4;
    const unsigned blocks = unsigned((threads + 255) / 256);
    step_kernel<DT, HAS_D, HAS_Z><<<dim3(blocks), dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

template <int DT>
hipError_t dispatch_scan(const ScanArgs& a, hipStream_t s)
{
    const bool hd = a.Dskip != nullptr, hz = a.z != nullptr;
    if (hd && hz) return launch_scan_t<DT, true, true>(a, s);
    if (hd) return launch_scan_t<DT, true, false>(a, s);
    if (hz) return launch_scan_t<DT, false, true>(a, s);
    return launch_scan_t<DT, false, false>(a, s);
}

template <int DT>
hipError_t dispatch_step(const StepArgs& a, hipStream_t s)
{
    const bool hd = a.Dskip != nullptr, hz = a.z != nullptr;
    if (hd && hz) return launch_step_t<DT, true, true>(a, s);
    if (hd) return launch_step_t<DT, true, false>(a, s);
    if (hz) return launch_step_t<DT, false, true>(a, s);
    return launch_step_t<DT, false, false>(a, s);
}

}  // namespace

hipError_t launch_scan(const ScanArgs& a, int dtype, hipStream_t stream)
{
    (void)hipGetLastError();  // start from a clean per-thread error state
    return dtype == 0 ? dispatch_scan<0>(a, stream) : dispatch_scan<1>(a, stream);
}

hipError_t launch_step(const StepArgs& a, int dtype, hipStream_t stream)
{
    (void)hipGetLastError();
    return dtype == 0 ? dispatch_step<0>(a, stream) : dispatch_step<1>(a, stream);
}

}  // namespace ssk
