// gfx950 kernel of the multi-head state-space recurrence of Mamba-2 (Mamba
// walk-through, section 4.1: h_t = A_t h_{t-1} + B_t x_t, y_t = C_t h_t with a
// state per head, and its dual, a causal structured matrix applied to the
// inputs; section 5.2: heads of 64 channels, d_state 64-256).  Per batch row b
// and head h, with a scalar decay per head:
//   S_t = exp(dt_t A_h) S_{t-1} + dt_t B_t x_t^T        (S is dstate x 64)
//   y_t = S_t^T C_t + D_h x_t
//
// Here the intra-chunk work is a dense contraction, so it runs on the matrix
// cores (bf16 MFMA 32x32x16, fp32 accumulation).  One workgroup of 4 waves per
// (b, h) walks the sequence in chunks of 64 rows with the state in MFMA
// accumulator registers (fp32) -- it never reaches memory between chunks.  Per
// chunk, with cs_t = sum of dt_r A over the chunk's rows up to t:
//   G^T    = B C^T                                   (s x t, over dstate)
//   M[t,s] = G[t,s] exp(cs_t - cs_s) dt_s  for s <= t, else 0
//   Y^T    = X^T M^T + S_in^T C^T diag(exp(cs_t))  (+ D x)    (the dual form
//            inside the chunk, plus the carried state)
//   S_out  = exp(cs_end) S_in + B^T (w X),  w_s = exp(cs_end - cs_s) dt_s
// Every operand that is a product (M, w*x) or the fp32 state goes to the
// matrix cores as two bf16 parts, hi + lo (lo = the rounding error of hi), so
// each such product keeps ~16 more bits: rounding these operands once to bf16
// costs up to ~1% of y per operand on slowly decaying heads.
//
// Data movement.  Every LDS matrix is row-major and written with 8- or
// 16-byte stores: x and B as they arrive, M and the state copy straight from
// the accumulator layout.  An MFMA operand is 8 consecutive values along the
// contraction index: where that index runs along a row it is one 16-byte
// read, where it runs down a column (x over s, B over s) it comes
// from two LDS transpose reads; the state update's w*x operand is such a read
// of x scaled by w in registers.  Y is formed transposed (p x t), so each lane
// ends up with 4 consecutive channels of one row and stores them as 8 bytes.
// C goes from memory straight into registers in the operand layout.  The next
// chunk's x, B, C and dt are loaded into registers while the current chunk
// computes, through range-checked buffer loads: rows past the sequence read
// 0 and their y stores are dropped, so the ragged last chunk needs no
// branches.  Blocks above the diagonal of M are zero and skipped.
#include "ss_device.h"

namespace ssk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQ = 64;            // rows per chunk
constexpr int kP = 64;            // channels per head
constexpr int kSsdThreads = 256;  // 4 waves
constexpr int kPad = 8;           // bf16 padding per LDS row (keeps 16-byte alignment)
constexpr int kXP = kP + kPad;    // row pitch of x and M in LDS

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 8 bf16 along a row: one 16-byte LDS read
__device__ __forceinline__ bf16x8 lds_row8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// 8 bf16 down a column: operand[i] = Mx[8*(lane/32) + i][lane%32] of the
// row-major LDS block that starts at `base`, row pitch `pitch` elements.
// Within each group of 16 lanes the transpose read gives lane i, as its
// element k, element i%4 of the 4-vector that lane 4k + i/4 addresses.  So
// lane j of the group addresses row j/4, columns 4*(j%4).. of a 4 x 16 block
// and lane i receives rows 0..3 of column i; two reads cover the 8 rows.
__device__ __forceinline__ bf16x8 lds_col8(const uint16_t* base, int pitch, int lane)
{
    typedef __attribute__((address_space(3))) s16x4* lds_ptr;
    const int j = lane & 15, g = lane >> 4;
    const uint16_t* p = base + (8 * (g >> 1) + (j >> 2)) * pitch + 16 * (g & 1) + 4 * (j & 3);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(p + 4 * pitch));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// the bf16 in the low 16 bits of `bits`, widened
__device__ __forceinline__ float bf(uint32_t bits) { return __uint_as_float(bits << 16); }
// ... in the high 16 bits
__device__ __forceinline__ float bf_hi(uint32_t bits) { return __uint_as_float(bits & 0xffff0000u); }

// two values rounded to bf16 (nearest even) in one conversion: a in the low
// half, b in the high half
__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

// v = hi + lo with hi = bf16(v) and lo = bf16(v - hi), for four values, each
// part packed as 4 bf16 (8 bytes)
__device__ __forceinline__ void split4(const float (&v)[4], u32x2& hi, u32x2& lo)
{
    const uint32_t h01 = pack_bf16(v[0], v[1]), h23 = pack_bf16(v[2], v[3]);
    hi = u32x2{h01, h23};
    lo = u32x2{pack_bf16(v[0] - bf(h01), v[1] - bf_hi(h01)), pack_bf16(v[2] - bf(h23), v[3] - bf_hi(h23))};
}

// grid = (heads, batch), block = 256.  Host guarantees bf16 operands, headdim
// 64, dstate NS, 16-byte alignment of x, y, B, C, and byte extents of one
// batch row of x (seqlen*heads*128) and of B (seqlen*NS*2) below 2^31.
// SPLIT (dstate 2*NS) runs the kernel twice.  The state entries evolve
// independently and y sums over them (the intra-chunk G = B C^T too), so each
// launch runs the NS-entry recurrence on its half of B, C, h0 and h_last:
// SPLIT = 1 takes entries 0..NS-1 and writes its fp32 part of y, with the D
// term, to a.y_part; SPLIT = 2 takes entries NS..2NS-1, adds the first part to
// its own and writes y.  The host guarantees one batch row of y_part
// (seqlen*heads*256 bytes, with the rows a ragged last chunk reaches) below 2^31.
template <int NS, bool HAS_D, int SPLIT = 0>
__global__ __launch_bounds__(kSsdThreads) __attribute__((amdgpu_waves_per_eu(2))) void ssd_kernel(SsdArgs a)
{
    constexpr int kNB = NS / 32;                    // 32-row blocks of the state (index n)
    constexpr int kSPW = kNB * 2 / 4;               // state blocks (n block, p block) per wave
    constexpr int kBP = NS + kPad;                  // row pitch of B and of the state copy in LDS
    constexpr int kVB = kQ * NS / 8 / kSsdThreads;  // 16-byte pieces of B per thread and chunk
    constexpr int kVX = kQ * kP / 8 / kSsdThreads;  // ... of x
    constexpr int kKS = NS / 16;                    // MFMA steps over dstate
    static_assert(kSPW >= 1 && kVB >= 1 && kVX >= 1, "dstate 64 or 128");

    __shared__ __align__(16) uint16_t sB[kQ][kBP];     // B chunk (s, n)
    __shared__ __align__(16) uint16_t sX[kQ][kXP];     // x chunk (s, p)
    __shared__ __align__(16) uint16_t sU[2][kQ][kXP];  // M (t, s) hi/lo
    __shared__ __align__(16) uint16_t sS[2][kP][kBP];  // state^T (p, n) hi/lo
    __shared__ __align__(16) float s_cs[kQ];           // cs_t * log2 e
    __shared__ __align__(16) float s_lc[kQ];           // cs_s * log2 e - log2(dt_s)  (+inf where dt_s = 0)
    __shared__ __align__(16) float s_w[kQ];
    __shared__ float s_end;  // exp(cs_end)

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hl = lane >> 5;
    const int64_t h = blockIdx.x, b = blockIdx.y;
    const int64_t L = a.seqlen, H = a.heads;
    const float A2 = a.A[h] * kLog2e;
    // the state entries of this workgroup: n0 .. n0+NS-1 of NT
    constexpr int NT = SPLIT ? 2 * NS : NS;
    constexpr int n0 = SPLIT == 2 ? NS : 0;
    const float Dh = HAS_D ? a.D[h] : 0.0f;

    // range-checked views of this (b, h): row t of x and y at t*H*128 bytes, of
    // dt at t*H*2, of B and C at t*NT*2 (from entry n0).  All offsets go in the
    // vector operand.
    const uint32_t x_row = uint32_t(H) * kP * 2, dt_row = uint32_t(H) * 2, bc_row = NT * 2;
    const uint32_t x_ext = uint32_t(((L - 1) * H + 1) * kP * 2), dt_ext = uint32_t(((L - 1) * H + 1) * 2);
    const uint32_t bc_ext = uint32_t(L) * bc_row - uint32_t(n0) * 2;
    const __amdgpu_buffer_rsrc_t rX = make_rsrc(static_cast<const uint16_t*>(a.x) + (b * L * H + h) * kP, x_ext);
    const __amdgpu_buffer_rsrc_t rY = SPLIT == 1
                                          ? make_rsrc(a.y_part + (b * L * H + h) * kP, 2 * x_ext)
                                          : make_rsrc(static_cast<uint16_t*>(a.y) + (b * L * H + h) * kP, x_ext);
    // the first half's fp32 part of y (read by the second half)
    const __amdgpu_buffer_rsrc_t rP = make_rsrc(SPLIT == 2 ? a.y_part + (b * L * H + h) * kP : nullptr, 2 * x_ext);
    const __amdgpu_buffer_rsrc_t rDT = make_rsrc(static_cast<const uint16_t*>(a.dt) + b * L * H + h, dt_ext);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(static_cast<const uint16_t*>(a.B) + b * L * NT + n0, bc_ext);
    const __amdgpu_buffer_rsrc_t rC = make_rsrc(static_cast<const uint16_t*>(a.C) + b * L * NT + n0, bc_ext);

    // this wave's blocks: G^T block (s block gs, t block tb), Y^T block (p block
    // yp, t block tb), state blocks (n block, p block) number w*kSPW + j
    const int tb = w & 1, gs = w >> 1, yp = w >> 1;
    const bool has_g = gs <= tb;  // the G^T block with s > t throughout is zero

    // ---- operands of a chunk in flight (issued one chunk ahead) ----
    u32x4 pB[kVB], pX[kVX], pC[kKS];
    uint32_t pdt = 0;
    // Issue order matters: a wait for one load also waits for every older
    // one, so dt (needed first) goes out first and x/B last.
    auto issue = [&](uint32_t t0) {
        if (w == 0) pdt = __builtin_amdgcn_raw_buffer_load_b16(rDT, (t0 + lane) * dt_row, 0, 0);
        // C rows of this wave's t block in the MFMA operand layout (row l%32,
        // entries 16*ks + 8*(l/32) .. +8)
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks)
            pC[ks] = __builtin_amdgcn_raw_buffer_load_b128(rC, (t0 + 32 * tb + l32) * bc_row + (16 * ks + 8 * hl) * 2,
                                                           0, 0);
#pragma unroll
        for (int i = 0; i < kVB; ++i) {
            const int v = tid + kSsdThreads * i, r = v / (NS / 8), c8 = (v % (NS / 8)) * 8;
            pB[i] = __builtin_amdgcn_raw_buffer_load_b128(rB, (t0 + r) * bc_row + c8 * 2, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < kVX; ++i) {
            const int v = tid + kSsdThreads * i, s = v / (kP / 8), p8 = (v % (kP / 8)) * 8;
            pX[i] = __builtin_amdgcn_raw_buffer_load_b128(rX, (t0 + s) * x_row + p8 * 2, 0, 0);
        }
    };

    // ---- initial state: accumulators (n x p blocks) and the LDS copy ----
    f32x16 acc_s[kSPW];
#pragma unroll
    for (int j = 0; j < kSPW; ++j) {
        const int blk = w * kSPW + j, nb = blk % kNB, pb = blk / kNB;
        const int p = 32 * pb + l32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int n = 32 * nb + 8 * q + 4 * hl + e;
                v[e] = a.h0 ? a.h0[((b * H + h) * NT + n0 + n) * kP + p] : 0.0f;
                acc_s[j][4 * q + e] = v[e];
            }
            u32x2 hi, lo;
            split4(v, hi, lo);
            *reinterpret_cast<u32x2*>(&sS[0][p][32 * nb + 8 * q + 4 * hl]) = hi;
            *reinterpret_cast<u32x2*>(&sS[1][p][32 * nb + 8 * q + 4 * hl]) = lo;
        }
    }

    issue(0);
    const int64_t n_chunks = (L + kQ - 1) / kQ;
    for (int64_t c = 0; c < n_chunks; ++c) {
        const uint32_t t0 = uint32_t(c * kQ);

        // ---- A: stage the chunk, start the next one's loads ----
#pragma unroll
        for (int i = 0; i < kVB; ++i) {
            const int v = tid + kSsdThreads * i, r = v / (NS / 8), c8 = (v % (NS / 8)) * 8;
            *reinterpret_cast<u32x4*>(&sB[r][c8]) = pB[i];
        }
#pragma unroll
        for (int i = 0; i < kVX; ++i) {
            const int v = tid + kSsdThreads * i, s = v / (kP / 8), p8 = (v % (kP / 8)) * 8;
            *reinterpret_cast<u32x4*>(&sX[s][p8]) = pX[i];
        }
        bf16x8 ca[kKS];
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) ca[ks] = __builtin_bit_cast(bf16x8, pC[ks]);
        // dt*A prefix over the chunk (wave 0): inclusive scan across the 64
        // lanes, in log2 units; rows past the sequence have dt = 0
        if (w == 0) {
            const float dt = bf(pdt);
            float v = dt * A2;
            v = add_from<kDppRowShr1, 0xf>(v);
            v = add_from<kDppRowShr2, 0xf>(v);
            v = add_from<kDppRowShr4, 0xf>(v);
            v = add_from<kDppRowShr8, 0xf>(v);
            v = add_from<kDppRowBcast15, 0xa>(v);
            v = add_from<kDppRowBcast31, 0xc>(v);
            const float end = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kQ - 1));
            s_cs[lane] = v;
            s_lc[lane] = v - __builtin_amdgcn_logf(dt);
            s_w[lane] = exp2_hw(end - v) * dt;
            if (lane == 0) s_end = exp2_hw(end);
        }
        if (c + 1 < n_chunks) issue(t0 + kQ);
        __syncthreads();

        // ---- B: G^T = B C^T -> M (LDS); Y^T = S_in^T C^T, scaled by exp(cs_t) ----
        const int t = 32 * tb + l32;  // this lane's column of G^T and Y^T
        const float cs_t = s_cs[t];
        if (has_g) {
            f32x16 acc_g;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc_g[r] = 0.0f;
            bf16x8 gb[kKS];
#pragma unroll
            for (int ks = 0; ks < kKS; ++ks) gb[ks] = lds_row8(&sB[32 * gs + l32][16 * ks + 8 * hl]);
#pragma unroll
            for (int ks = 0; ks < kKS; ++ks) acc_g = mfma(gb[ks], ca[ks], acc_g);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int s0 = 32 * gs + 8 * q + 4 * hl;  // rows s0..s0+3 of G^T in this lane
                // exp(cs_t - cs_s) dt_s = exp2(cs_t*log2 e - s_lc[s])
                const float4 lc = *reinterpret_cast<const float4*>(&s_lc[s0]);
                const float lcv[4] = {lc.x, lc.y, lc.z, lc.w};
                // computed for every s and masked with a bitwise and (no
                // branches; above the diagonal the product may be inf or NaN)
                float m[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v = acc_g[4 * q + e] * exp2_hw(cs_t - lcv[e]);
                    m[e] = __uint_as_float(__float_as_uint(v) & (s0 + e <= t ? 0xffffffffu : 0u));
                }
                u32x2 hi, lo;
                split4(m, hi, lo);
                *reinterpret_cast<u32x2*>(&sU[0][t][s0]) = hi;
                *reinterpret_cast<u32x2*>(&sU[1][t][s0]) = lo;
            }
        }
        f32x16 acc_y, acc_l;  // the hi and lo parts of the state: two independent chains
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_y[r] = acc_l[r] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) {
            acc_y = mfma(lds_row8(&sS[0][32 * yp + l32][16 * ks + 8 * hl]), ca[ks], acc_y);
            acc_l = mfma(lds_row8(&sS[1][32 * yp + l32][16 * ks + 8 * hl]), ca[ks], acc_l);
        }
        {
            const float e_t = exp2_hw(cs_t);
#pragma unroll
            for (int r = 0; r < 16; ++r) acc_y[r] = (acc_y[r] + acc_l[r]) * e_t;
        }
        __syncthreads();

        // ---- C: Y^T += X^T M^T, + D x; store ----
        {
            // the second half adds the first half's part: loaded now, used at the store
            u32x4 part[4];
            if constexpr (SPLIT == 2) {
                const uint32_t prow = 2 * (t0 + 32 * tb + l32) * x_row;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    part[q] = __builtin_amdgcn_raw_buffer_load_b128(rP, prow + (32 * yp + 8 * q + 4 * hl) * 4, 0, 0);
            }
            const int ks_end = tb == 0 ? 2 : 4;  // M[t][s] = 0 for s > t
#pragma unroll
            for (int r = 0; r < 16; ++r) acc_l[r] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                if (ks < ks_end) {
                    const bf16x8 xa = lds_col8(&sX[16 * ks][32 * yp], kXP, lane);
                    acc_y = mfma(xa, lds_row8(&sU[0][t][16 * ks + 8 * hl]), acc_y);
                    acc_l = mfma(xa, lds_row8(&sU[1][t][16 * ks + 8 * hl]), acc_l);
                }
            }
            const uint32_t yrow = (t0 + t) * x_row;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int p0 = 32 * yp + 8 * q + 4 * hl;  // channels p0..p0+3 of row t in this lane
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc_y[4 * q + e] + acc_l[4 * q + e];
                if constexpr (SPLIT == 2) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] += __uint_as_float(part[q][e]);
                }
                if (HAS_D) {
                    const u32x2 xr = *reinterpret_cast<const u32x2*>(&sX[t][p0]);
                    v[0] = fmaf(Dh, bf(xr[0]), v[0]);
                    v[1] = fmaf(Dh, bf_hi(xr[0]), v[1]);
                    v[2] = fmaf(Dh, bf(xr[1]), v[2]);
                    v[3] = fmaf(Dh, bf_hi(xr[1]), v[3]);
                }
                if constexpr (SPLIT == 1) {
                    const u32x4 o = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                     __float_as_uint(v[3])};
                    __builtin_amdgcn_raw_buffer_store_b128(o, rY, 2 * yrow + p0 * 4, 0, 0);
                } else {
                    const u32x2 o = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
                    __builtin_amdgcn_raw_buffer_store_b64(o, rY, yrow + p0 * 2, 0, 0);
                }
            }
        }
        // ---- E: S = exp(cs_end) S + B^T (w x); new LDS copy of S^T ----
        // No barrier since phase C: this phase reads x, B and w (staged before
        // the first barrier) and writes the state copy, which C does not read.
        const float decay = s_end;
        // a wave's state blocks share their p block, so the w*x operands of a
        // step serve all of them
        const int spb = (w * kSPW) / kNB;
        static_assert(kNB % kSPW == 0, "a wave's state blocks lie in one p block");
        // the lo parts accumulate in chains of their own, added once at the end,
        // so that each block's MFMAs form two independent chains
        f32x16 acc_lo[kSPW];
#pragma unroll
        for (int j = 0; j < kSPW; ++j) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                acc_s[j][r] *= decay;
                acc_lo[j][r] = 0.0f;
            }
        }
#pragma unroll
        for (int ks = 0; ks < kQ / 16; ++ks) {
            // the w*x operand, formed in registers: rows s = 16ks + 8(l/32) + i
            // of x (a transpose read) times w_s, in two bf16 parts
            bf16x8 xh, xl;
            {
                const bf16x8 xv = lds_col8(&sX[16 * ks][32 * spb], kXP, lane);
                const float4 w0 = *reinterpret_cast<const float4*>(&s_w[16 * ks + 8 * hl]);
                const float4 w1 = *reinterpret_cast<const float4*>(&s_w[16 * ks + 8 * hl + 4]);
                const float first[4] = {w0.x * float(xv[0]), w0.y * float(xv[1]), w0.z * float(xv[2]),
                                        w0.w * float(xv[3])};
                const float second[4] = {w1.x * float(xv[4]), w1.y * float(xv[5]), w1.z * float(xv[6]),
                                         w1.w * float(xv[7])};
                u32x2 h0, l0, h1, l1;
                split4(first, h0, l0);
                split4(second, h1, l1);
                xh = __builtin_bit_cast(bf16x8, u32x4{h0[0], h0[1], h1[0], h1[1]});
                xl = __builtin_bit_cast(bf16x8, u32x4{l0[0], l0[1], l1[0], l1[1]});
            }
#pragma unroll
            for (int j = 0; j < kSPW; ++j) {
                const int nb = (w * kSPW + j) % kNB;
                const bf16x8 bt = lds_col8(&sB[16 * ks][32 * nb], kBP, lane);
                acc_s[j] = mfma(bt, xh, acc_s[j]);
                acc_lo[j] = mfma(bt, xl, acc_lo[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < kSPW; ++j) {
#pragma unroll
            for (int r = 0; r < 16; ++r) acc_s[j][r] += acc_lo[j][r];
        }
#pragma unroll
        for (int j = 0; j < kSPW; ++j) {
            const int nb = (w * kSPW + j) % kNB, pb = spb;
            const int p = 32 * pb + l32;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float v[4] = {acc_s[j][4 * q], acc_s[j][4 * q + 1], acc_s[j][4 * q + 2], acc_s[j][4 * q + 3]};
                u32x2 hi, lo;
                split4(v, hi, lo);
                *reinterpret_cast<u32x2*>(&sS[0][p][32 * nb + 8 * q + 4 * hl]) = hi;
                *reinterpret_cast<u32x2*>(&sS[1][p][32 * nb + 8 * q + 4 * hl]) = lo;
            }
        }
        __syncthreads();  // x and B consumed; the new state copy is complete
    }

    if (a.h_last) {
#pragma unroll
        for (int j = 0; j < kSPW; ++j) {
            const int blk = w * kSPW + j, nb = blk % kNB, pb = blk / kNB;
            const int p = 32 * pb + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int n = 32 * nb + 8 * (r >> 2) + 4 * hl + (r & 3);
                a.h_last[((b * H + h) * NT + n0 + n) * kP + p] = acc_s[j][r];
            }
        }
    }
}

template <int NS>
hipError_t launch_ssd_n(const SsdArgs& a, hipStream_t s)
{
    const dim3 grid(unsigned(a.heads), unsigned(a.batch));
    if (a.D)
        ssd_kernel<NS, true><<<grid, dim3(kSsdThreads), 0, s>>>(a);
    else
        ssd_kernel<NS, false><<<grid, dim3(kSsdThreads), 0, s>>>(a);
    return hipGetLastError();
}

// dstate 256: the first half, then the second, which adds the first's part of y
hipError_t launch_ssd_split(const SsdArgs& a, hipStream_t s)
{
    const dim3 grid(unsigned(a.heads), unsigned(a.batch));
    if (a.D)
        ssd_kernel<128, true, 1><<<grid, dim3(kSsdThreads), 0, s>>>(a);
    else
        ssd_kernel<128, false, 1><<<grid, dim3(kSsdThreads), 0, s>>>(a);
    ssd_kernel<128, false, 2><<<grid, dim3(kSsdThreads), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ssd(const SsdArgs& a, hipStream_t stream)
{
    (void)hipGetLastError();
    if (a.dstate == 256) return launch_ssd_split(a, stream);
    return a.dstate == 128 ? launch_ssd_n<128>(a, stream) : launch_ssd_n<64>(a, stream);
}

}  // namespace ssk
