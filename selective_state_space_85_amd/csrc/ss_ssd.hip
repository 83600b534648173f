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
//   G      = C B^T                                   (64 x 64, over dstate)
//   M[t,s] = G[t,s] exp(cs_t - cs_s) dt_s  for s <= t, else 0
//   Y      = M X + diag(exp(cs_t)) C S_in  (+ D x)   (the dual form inside the
//                                                     chunk, the carried state)
//   S_out^T = exp(cs_end) S_in^T + X^T diag(w) B,  w_s = exp(cs_end - cs_s) dt_s
// Every operand that is a product (M, w*B) or the fp32 state goes to the
// matrix cores as two bf16 parts, hi + lo (lo = the rounding error of hi), so
// each such product keeps ~16 more bits: rounding these operands once to bf16
// costs up to ~1% of y per operand on slowly decaying heads.
// C is loaded straight into registers in the MFMA operand layout; B by row
// (state index contiguous), x transposed (row index contiguous), M by row and
// the state's two bf16 parts transposed are staged in LDS.  Blocks above the
// diagonal of M are zero and skipped.
#include "ss_device.h"

namespace ssk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kQ = 64;            // rows per chunk
constexpr int kP = 64;            // channels per head
constexpr int kSsdThreads = 256;  // 4 waves
constexpr int kPad = 8;           // bf16 padding per LDS row (keeps 16-byte alignment)

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds_b128(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ float bf(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// Accumulator layout of a 32x32 MFMA block: lane l, register r holds row
// 8*(r/4) + 4*(l/32) + r%4 and column l%32.
__device__ __forceinline__ int acc_row(int lane, int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// v = hi + lo with hi = bf16(v) and lo = bf16(v - hi)
__device__ __forceinline__ void store_split(uint16_t& hi, uint16_t& lo, float v)
{
    const uint16_t h = f32_to_bf16_bits(v);
    hi = h;
    lo = f32_to_bf16_bits(v - __uint_as_float(uint32_t(h) << 16));
}

// M rows are 64 bf16 (128 bytes) with no padding; its 8-element groups are
// permuted per row (group g of row t at g ^ (t & 7)) so that the 32 rows a
// 16-byte operand read touches fall on different banks.
__device__ __forceinline__ int mcol(int t, int s) { return s ^ ((t & 7) << 3); }

// grid = (heads, batch), block = 256.  Host guarantees bf16 operands, headdim
// 64, dstate NS, 16-byte alignment of x, y, B, C.
template <int NS, bool HAS_D>
__global__ __launch_bounds__(kSsdThreads) void ssd_kernel(SsdArgs a)
{
    constexpr int kNB = NS / 32;               // 32-wide state blocks
    constexpr int kSB = (kP / 32) * kNB;       // state blocks of S^T (p x n)
    constexpr int kSPW = kSB / 4;              // state blocks per wave
    static_assert(kSPW >= 1, "dstate 64 or 128");

    __shared__ __align__(16) uint16_t sB[kQ][NS + kPad];   // B chunk (s, n)
    __shared__ __align__(16) uint16_t sXT[kP][kQ + kPad];  // x chunk transposed (p, s)
    __shared__ __align__(16) uint16_t sMh[kQ][kQ];         // masked decay matrix (t, s), hi part (swizzled)
    __shared__ __align__(16) uint16_t sMl[kQ][kQ];         // ... and lo part
    __shared__ __align__(16) uint16_t sSh[kP][NS + kPad];  // state transposed (p, n), hi part
    __shared__ __align__(16) uint16_t sSl[kP][NS + kPad];  // ... and lo part
    __shared__ float s_cs[kQ], s_dt[kQ], s_ecs[kQ], s_w[kQ];
    __shared__ float s_end;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t h = blockIdx.x, b = blockIdx.y;
    const int64_t L = a.seqlen, H = a.heads;
    const float Ah = a.A[h];
    const float Dh = HAS_D ? a.D[h] : 0.0f;
    const uint16_t* __restrict__ X = static_cast<const uint16_t*>(a.x);
    const uint16_t* __restrict__ DT = static_cast<const uint16_t*>(a.dt);
    const uint16_t* __restrict__ Bg = static_cast<const uint16_t*>(a.B);
    const uint16_t* __restrict__ Cg = static_cast<const uint16_t*>(a.C);
    uint16_t* __restrict__ Y = static_cast<uint16_t*>(a.y);

    // state blocks of this wave: block k -> (p block, n block)
    f32x16 acc_s[kSPW];
#pragma unroll
    for (int j = 0; j < kSPW; ++j) {
        const int blk = w * kSPW + j, pb = blk / kNB, nb = blk % kNB;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int p = 32 * pb + acc_row(lane, r), n = 32 * nb + (lane & 31);
            const float v = a.h0 ? a.h0[((b * H + h) * NS + n) * kP + p] : 0.0f;
            acc_s[j][r] = v;
            store_split(sSh[p][n], sSl[p][n], v);
        }
    }

    const int bm = w >> 1, bn = w & 1;  // this wave's 32x32 block of G, M and Y
    const int64_t n_chunks = (L + kQ - 1) / kQ;
    for (int64_t c = 0; c < n_chunks; ++c) {
        const int64_t t0 = c * kQ;
        const int rows = int(L - t0 < kQ ? L - t0 : kQ);

        // ---- stage the chunk ----
        // B and C: rows x NS bf16, 16-byte vectors
        constexpr int kVecRow = NS / 8;
#pragma unroll
        for (int i = 0; i < (kQ * kVecRow) / kSsdThreads; ++i) {
            const int v = tid + kSsdThreads * i, r = v / kVecRow, c8 = (v % kVecRow) * 8;
            uint4 qb = make_uint4(0, 0, 0, 0);
            if (r < rows) qb = *reinterpret_cast<const uint4*>(Bg + (b * L + t0 + r) * NS + c8);
            *reinterpret_cast<uint4*>(&sB[r][c8]) = qb;
        }
        // C: this wave's 32 rows, straight into the A-operand layout (row l%32,
        // entries 16*ks + 8*(l/32) .. +8)
        bf16x8 ca[NS / 16];
        {
            const int r = 32 * (w >> 1) + (lane & 31);
#pragma unroll
            for (int ks = 0; ks < NS / 16; ++ks) {
                uint4 q = make_uint4(0, 0, 0, 0);
                if (r < rows) q = *reinterpret_cast<const uint4*>(Cg + (b * L + t0 + r) * NS + 16 * ks + 8 * (lane >> 5));
                ca[ks] = __builtin_bit_cast(bf16x8, q);
            }
        }
        // x: rows x 64 bf16 (rows strided by H*64), written transposed
#pragma unroll
        for (int i = 0; i < (kQ * kP / 8) / kSsdThreads; ++i) {
            const int v = tid + kSsdThreads * i, s = v / (kP / 8), p8 = (v % (kP / 8)) * 8;
            uint4 q = make_uint4(0, 0, 0, 0);
            if (s < rows) q = *reinterpret_cast<const uint4*>(X + ((b * L + t0 + s) * H + h) * kP + p8);
            const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                sXT[p8 + 2 * k][s] = uint16_t(wd[k] & 0xffffu);
                sXT[p8 + 2 * k + 1][s] = uint16_t(wd[k] >> 16);
            }
        }
        // dt*A prefix over the chunk (wave 0): inclusive scan across the 64 lanes
        if (w == 0) {
            const float dt = lane < rows ? bf(DT[(b * L + t0 + lane) * H + h]) : 0.0f;
            float v = dt * Ah;
            v = add_from<kDppRowShr1, 0xf>(v);
            v = add_from<kDppRowShr2, 0xf>(v);
            v = add_from<kDppRowShr4, 0xf>(v);
            v = add_from<kDppRowShr8, 0xf>(v);
            v = add_from<kDppRowBcast15, 0xa>(v);
            v = add_from<kDppRowBcast31, 0xc>(v);
            const float end = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kQ - 1));
            s_cs[lane] = v;
            s_dt[lane] = dt;
            s_ecs[lane] = exp2_hw(v * kLog2e);
            s_w[lane] = exp2_hw((end - v) * kLog2e) * dt;
            if (lane == 0) s_end = exp2_hw(end * kLog2e);
        }
        __syncthreads();

        // ---- G = C B^T -> M (masked, decayed); Y = exp(cs_t) C S_in ----
        f32x16 acc_y;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_y[r] = 0.0f;
        {
            const bool upper = bm == 0 && bn == 1;  // t < 32 <= s: M is zero there
            f32x16 acc_g;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc_g[r] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < NS / 16; ++ks) {
                const int k0 = 16 * ks + 8 * (lane >> 5);
                if (!upper) acc_g = mfma(ca[ks], lds_b128(&sB[32 * bn + (lane & 31)][k0]), acc_g);
                acc_y = mfma(ca[ks], lds_b128(&sSh[32 * bn + (lane & 31)][k0]), acc_y);
                acc_y = mfma(ca[ks], lds_b128(&sSl[32 * bn + (lane & 31)][k0]), acc_y);
            }
            const int s = 32 * bn + (lane & 31);
            const float cs_s = s_cs[s], dt_s = s_dt[s];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int t = 32 * bm + acc_row(lane, r);
                const float m = (!upper && s <= t) ? acc_g[r] * exp2_hw((s_cs[t] - cs_s) * kLog2e) * dt_s : 0.0f;
                store_split(sMh[t][mcol(t, s)], sMl[t][mcol(t, s)], m);
                acc_y[r] *= s_ecs[t];
            }
        }
        __syncthreads();

        // ---- Y += M X, + D x; store ----
        {
            const int ks_end = bm == 0 ? 2 : 4;  // M[t][s] = 0 for s > t
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                if (ks < ks_end) {
                    const int k0 = 16 * ks + 8 * (lane >> 5);
                    const int t = 32 * bm + (lane & 31);
                    const bf16x8 xb = lds_b128(&sXT[32 * bn + (lane & 31)][k0]);
                    acc_y = mfma(lds_b128(&sMh[t][mcol(t, k0)]), xb, acc_y);
                    acc_y = mfma(lds_b128(&sMl[t][mcol(t, k0)]), xb, acc_y);
                }
            }
            const int p = 32 * bn + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int t = 32 * bm + acc_row(lane, r);
                float yv = acc_y[r];
                if (HAS_D) yv = fmaf(Dh, bf(sXT[p][t]), yv);
                if (t < rows) Y[((b * L + t0 + t) * H + h) * kP + p] = f32_to_bf16_bits(yv);
            }
        }
        // ---- S^T = exp(cs_end) S^T + X^T diag(w) B ----
        const float decay = s_end;
#pragma unroll
        for (int j = 0; j < kSPW; ++j) {
            const int blk = w * kSPW + j, pb = blk / kNB, nb = blk % kNB;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc_s[j][r] *= decay;
#pragma unroll
            for (int ks = 0; ks < kQ / 16; ++ks) {
                const int k0 = 16 * ks + 8 * (lane >> 5);
                const int n = 32 * nb + (lane & 31);
                // w*B in two bf16 parts (hi + lo): the state keeps ~16 more bits of it
                bf16x8 bw_hi, bw_lo;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float v = bf(sB[k0 + i][n]) * s_w[k0 + i];
                    bw_hi[i] = (__bf16)v;
                    bw_lo[i] = (__bf16)(v - (float)bw_hi[i]);
                }
                const bf16x8 xa = lds_b128(&sXT[32 * pb + (lane & 31)][k0]);
                acc_s[j] = mfma(xa, bw_hi, acc_s[j]);
                acc_s[j] = mfma(xa, bw_lo, acc_s[j]);
            }
        }
        __syncthreads();  // every wave is done with sB, sXT, sM and the old state parts
#pragma unroll
        for (int j = 0; j < kSPW; ++j) {
            const int blk = w * kSPW + j, pb = blk / kNB, nb = blk % kNB;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int p = 32 * pb + acc_row(lane, r), n = 32 * nb + (lane & 31);
                store_split(sSh[p][n], sSl[p][n], acc_s[j][r]);
            }
        }
        // the next chunk's staging writes sB/sXT (not the state parts) before its
        // first barrier, and the state parts are read only after that barrier
    }

    if (a.h_last) {
#pragma unroll
        for (int j = 0; j < kSPW; ++j) {
            const int blk = w * kSPW + j, pb = blk / kNB, nb = blk % kNB;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int p = 32 * pb + acc_row(lane, r), n = 32 * nb + (lane & 31);
                a.h_last[((b * H + h) * NS + n) * kP + p] = acc_s[j][r];
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

}  // namespace

hipError_t launch_ssd(const SsdArgs& a, hipStream_t stream)
{
    (void)hipGetLastError();
    return a.dstate == 128 ? launch_ssd_n<128>(a, stream) : launch_ssd_n<64>(a, stream);
}

}  // namespace ssk
