// gfx950 kernels of the selective scan's backward: the gradients of
// sum(dy * y) + sum(dh_last * h_last) with respect to u, delta (raw under
// softplus), A, B, C, D, z, the delta bias and h0.  The per-timestep states
// are never stored: they are recomputed from checkpoints (the backward of the
// Mamba walk-through's section 3.3 and of the LTI chapter's section 3.1.5.3,
// which recomputes the states from the inputs instead of reading them back).
//
// For a lane (b, d) and state n, with e_t = exp(delta_t A) and the adjoint g
// (the gradient with respect to h_t, accumulated from the last timestep down):
//   g += dy'_t C_t                         dy' = dy * silu(z) (the gated gradient)
//   dC_t += dy'_t h_t        (summed over channels d)
//   ddelta_t += g (A e_t h_{t-1} + B_t u_t),  dA += g delta_t e_t h_{t-1}
//   dB_t += g delta_t u_t    (summed over channels d),  du_t += g delta_t B_t
//   g *= e_t
// plus du_t += D dy'_t, dD += dy'_t u_t, dz_t = dy_t ypre_t silu'(z_t), the
// softplus derivative sigmoid(raw + bias) on ddelta, dbias += ddelta, dh0 = g.
// Under the zero-order hold (walk-through, section 2.2) the input term is
// beta B_t u_t with beta = delta_t phi(delta_t A), so delta_t becomes beta in
// dB and du, B_t u_t in ddelta is weighted by dbeta/ddelta = e_t, and dA gains
// g B_t u_t dbeta/dA (zoh_dbeta_dA_over_delta).
//
// Three launches after the B/C panel:
//  1. the checkpoint pass runs the recurrence once and stores the state every
//     kBwdSub rows (the checkpoints): the forward scan kernel's checkpoint-only
//     instantiation (ss_kernels.hip, launch_ckpt_pass), so the checkpoints are
//     bit for bit those a one-chunk ss_scan_fwd_ckpt writes.  It is skipped
//     when the caller passes the checkpoints of its forward pass, which reuses
//     the forward's states the way the chunked forward reuses its chunk
//     carries;
//  2. bwd_kernel walks the sub-blocks from the last to the first: it rebuilds
//     the sub-block's states in registers from its checkpoint, then runs the
//     adjoint down the sub-block, writing du, ddelta and dz and the
//     per-workgroup channel sums of dB and dC, and keeping dA, dD, dbias per
//     lane;
//  3. bwd_reduce_kernel adds the per-workgroup and per-batch-row partial sums
//     in a fixed order (the result does not depend on scheduling) and rounds
//     dB, dC to the operand type.
// The adjoint's workgroup shape is the forward's whole-wave one: 64 channels of
// one batch row, the 16 state entries split over 8 waves (2 per wave), B and C
// as scalar operands.
#include "ss_device.h"

namespace ssk {
namespace {

constexpr int kSub = kBwdSub;             // rows per sub-block (checkpoint spacing)
constexpr int kHalf = kSub / 2;           // the backward finishes a sub-block in two halves
static_assert(kSub == 2 * kTileRows, "a sub-block is two panel tiles");
static_assert(kHalf == kGroups, "each wave publishes and finishes one row of each half");
static_assert(kHalf * kNS == 16, "one 16-word scalar load holds a wave's entries of a half's rows");

__device__ __forceinline__ float sigmoid(float v) { return __builtin_amdgcn_rcpf(1.0f + exp2_hw(-v * kLog2e)); }

// The per-workgroup pieces both kernels share: channel, row streams, panel.
template <int DT>
struct Lane {
    using T = typename Elem<DT>::T;
    using V = Buf<DT>;
    int lane, w;
    bool active;
    int64_t d, b;  // d clamped to a real channel for idle lanes
    uint32_t row_bytes, voff;
    const SS_CONST char* pB;  // this wave's B plane of the batch row's panel
    const SS_CONST char* pC;

    __device__ Lane(const BwdArgs& a)
    {
        lane = threadIdx.x & (kWave - 1);
        w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
        const int64_t d_raw = int64_t(blockIdx.x) * kWave + lane;
        active = d_raw < a.dim;
        d = active ? d_raw : a.dim - 1;
        b = blockIdx.y;
        row_bytes = uint32_t(a.dim) * V::kBytes;
        voff = active ? uint32_t(d_raw) * V::kBytes : kIdleOffset;
        const int64_t plane = a.panel_rows * kNS;
        pB = (const SS_CONST char*)(a.panel + (b * kGroups + w) * 2 * plane);
        pC = pB + plane * 4;
    }
    // a (B, L, D) stream of this batch row
    __device__ __amdgpu_buffer_rsrc_t rsrc(const void* base, const BwdArgs& a) const
    {
        return make_rsrc(static_cast<const T*>(base) + b * a.seqlen * a.dim, uint32_t(a.seqlen) * row_bytes);
    }
    // this wave's B (or C) entries of the 8 rows of half `half` of sub-block j
    __device__ Words16 words_B(int j, int half) const
    {
        return *(const SS_CONST Words16*)(pB + uint32_t(j * kSub + half * kHalf) * uint32_t(kNS * 4));
    }
    __device__ Words16 words_C(int j, int half) const
    {
        return *(const SS_CONST Words16*)(pC + uint32_t(j * kSub + half * kHalf) * uint32_t(kNS * 4));
    }
};

// entry i of row rr (0..7) of a half, from its 16 words
__device__ __forceinline__ float word(const Words16& wv, int rr, int i) { return __uint_as_float(wv[rr * kNS + i]); }

// The rows a wave publishes (and, in the backward, finishes) in a sub-block:
// row w of the first half and row w of the second.
__device__ __forceinline__ int row_of(int w, int k) { return w + k * kHalf; }

// Raw operand rows of a sub-block in flight, and the widened values a wave
// keeps for its own rows.
template <int DT>
struct Rows {
    using V = Buf<DT>;
    typename V::Raw dl[2], x[2], dy[2], z[2];

    template <bool HAS_Z>
    __device__ void issue(const Lane<DT>& ln, int64_t L, int j, __amdgpu_buffer_rsrc_t r_dl,
                          __amdgpu_buffer_rsrc_t r_u, __amdgpu_buffer_rsrc_t r_dy, __amdgpu_buffer_rsrc_t r_z)
    {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int64_t t = int64_t(j) * kSub + row_of(ln.w, k);
            const uint32_t so = uint32_t(t < L ? t : L - 1) * ln.row_bytes;
            dl[k] = V::load(r_dl, ln.voff, so);
            x[k] = V::load(r_u, ln.voff, so);
            dy[k] = V::load(r_dy, ln.voff, so);
            if (HAS_Z) z[k] = V::load(r_z, ln.voff, so);
        }
    }
};

// ---------------------------------------------------------------------------
// bwd_kernel: the adjoint, sub-block by sub-block from the last.  grid =
// (ceil(dim/64), batch), block = 64 * kGroups.  Per sub-block: publish the
// rows, rebuild the states from the checkpoint, then for each half (last
// first) run the adjoint down its rows -- per-wave partial sums over the
// wave's state entries of g.B and g.h_{t-1}.e.A go to LDS, the channel sums
// of g*delta*u (dB) to the partial buffer -- then, from the rebuilt states,
// the channel sums of dy'*h_t (dC) and, with a gate, the per-wave partial
// C.h_t; and finish one row per wave: du, ddelta, dz, and the per-lane dD and
// dbias terms.
// ---------------------------------------------------------------------------
template <int DT, bool HAS_D, bool HAS_Z, int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu((MODE & kOptZoh) ? 2 : 4))) void bwd_kernel(
    BwdArgs a)
{
    constexpr bool ZOH = (MODE & kOptZoh) != 0;
    using V = Buf<DT>;
    __shared__ float4 s_row[kSub][kWave];        // (delta, delta*u, dy', 1/delta under the zero-order hold)
    // per wave (sum g.B, sum g.h.e.A) of one half; under the zero-order hold (sum g.phi.B, ...)
    __shared__ float2 s_par[kGroups][kHalf][kWave];
    __shared__ float s_yp[HAS_Z ? kGroups : 1][kHalf][kWave];  // per wave C.h_t of one half (for dz)
    __shared__ float s_ge[ZOH ? kGroups : 1][kHalf][kWave];    // per wave sum g.e.B (zero-order hold)
    // the rebuild's phi per row, wave and lane (its two entries), for the adjoint (zero-order
    // hold: the kernel runs one workgroup per CU, so this 64 KB replaces 8 VALU per element)
    __shared__ float2 s_phi[ZOH ? kSub : 1][ZOH ? kGroups : 1][kWave];

    const Lane<DT> ln(a);
    const int lane = ln.lane, w = ln.w;
    const int64_t D = a.dim, L = a.seqlen, NB = a.batch, blk = blockIdx.x;
    const auto r_u = ln.rsrc(a.u, a), r_dl = ln.rsrc(a.delta, a), r_dy = ln.rsrc(a.dy, a);
    const auto r_z = ln.rsrc(HAS_Z ? a.z : a.u, a);
    const auto r_du = ln.rsrc(a.du, a), r_ddl = ln.rsrc(a.ddelta, a);
    const auto r_dz = ln.rsrc(HAS_Z ? a.dz : a.du, a);

    float A2[kNS], Av[kNS], iA[kNS], g[kNS], dA_acc[kNS];
#pragma unroll
    for (int i = 0; i < kNS; ++i) {
        Av[i] = a.A[ln.d * N + w * kNS + i];
        A2[i] = Av[i] * kLog2e;
        iA[i] = ZOH ? 1.0f / Av[i] : 0.0f;
        g[i] = (a.dh_last && ln.active) ? a.dh_last[(ln.b * D + ln.d) * N + w * kNS + i] : 0.0f;
        dA_acc[i] = 0.0f;
    }
    const float bias = a.delta_bias ? a.delta_bias[ln.d] : 0.0f;
    const float dskip = HAS_D ? a.Dskip[ln.d] : 0.0f;
    float dD_acc = 0.0f, dbias_acc = 0.0f;

    Rows<DT> rows;
    rows.template issue<HAS_Z>(ln, L, int(a.n_sub) - 1, r_dl, r_u, r_dy, r_z);
    float xf[2], dlf[2], sgf[2], dypf[2], dzf[2];  // dzf: dy * silu'(z), dz without ypre

    for (int j = int(a.n_sub) - 1; j >= 0; --j) {
        float hprev[kNS];
#pragma unroll
        for (int i = 0; i < kNS; ++i)
            hprev[i] = ln.active ? a.ckpt[((int64_t(j) * NB + ln.b) * N + w * kNS + i) * D + ln.d] : 0.0f;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int r = row_of(w, k);
            const bool in = ln.active && int64_t(j) * kSub + r < L;
            const float v = V::widen(rows.dl[k]) + bias;
            const float dl = in ? ((MODE & kOptSoftplus) ? softplus(v) : v) : 0.0f;
            const float x = V::widen(rows.x[k]);
            const float dyv = in ? V::widen(rows.dy[k]) : 0.0f;
            const float zv = HAS_Z ? V::widen(rows.z[k]) : 0.0f;
            const float dyp = HAS_Z ? dyv * silu(zv) : dyv;
            s_row[r][lane] = make_float4(dl, dl * x, dyp, ZOH ? __builtin_amdgcn_rcpf(dl) : 0.0f);
            xf[k] = x;
            dlf[k] = dl;
            sgf[k] = (MODE & kOptSoftplus) ? sigmoid(v) : 1.0f;
            dypf[k] = dyp;
            if (HAS_Z) {
                const float sz = sigmoid(zv);
                dzf[k] = dyv * sz * fmaf(zv, 1.0f - sz, 1.0f);
            }
        }
        if (j > 0) rows.template issue<HAS_Z>(ln, L, j - 1, r_dl, r_u, r_dy, r_z);
        __syncthreads();

        // the sub-block's states, rebuilt from its checkpoint
        float hh[kSub][kNS];
        // Euler: the second half's decays e_t, kept for its adjoint, which runs right after
        // the rebuild (the first half's would not fit beside the states: 29 values spill)
        float ee[kHalf][kNS];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const Words16 bw = ln.words_B(j, half);
#pragma unroll
            for (int rr = 0; rr < kHalf; ++rr) {
                const int r = half * kHalf + rr;
                const float4 rv = s_row[r][lane];
                float ph[kNS] = {};
#pragma unroll
                for (int i = 0; i < kNS; ++i) {
                    const float x2 = rv.x * A2[i], e = exp2_hw(x2);
                    if (!ZOH && half == 1) ee[rr][i] = e;
                    float in_term = rv.y * word(bw, rr, i);
                    if constexpr (ZOH) {
                        ph[i] = zoh_phi(x2, e, iA[i] * rv.w);
                        in_term *= ph[i];
                    }
                    hh[r][i] = fmaf(e, r ? hh[r - 1][i] : hprev[i], in_term);
                }
                static_assert(kNS == 2, "two entries per lane");
                if constexpr (ZOH) s_phi[ZOH ? r : 0][ZOH ? w : 0][lane] = make_float2(ph[0], ph[1]);
            }
        }

#pragma unroll
        for (int half = 1; half >= 0; --half) {
            const Words16 bw = ln.words_B(j, half), cw = ln.words_C(j, half);
            // the half's rows in two quarters of 4, last first: per quarter the
            // channel sums of g*delta*u (dB) and dy'*h_t (dC) over its 8
            // (row, state) values, taken as soon as the quarter is done so that
            // few of them and of the states are live at once
#pragma unroll
            for (int qt = 1; qt >= 0; --qt) {
                float db[8], dc[8];
#pragma unroll
                for (int rq = 3; rq >= 0; --rq) {
                    const int rr = 4 * qt + rq, r = half * kHalf + rr;
                    const float4 rv = s_row[r][lane];
                    const float2 phr = ZOH ? s_phi[ZOH ? r : 0][ZOH ? w : 0][lane] : make_float2(0.0f, 0.0f);
                    float s1 = 0.0f, s2 = 0.0f, s3 = 0.0f, yp = 0.0f;
#pragma unroll
                    for (int i = 0; i < kNS; ++i) {
                        // h_t is last needed here: dC, and C.h_t for dz
                        dc[rq * kNS + i] = rv.z * hh[r][i];
                        if (HAS_Z) yp = fmaf(word(cw, rr, i), hh[r][i], yp);
                        g[i] = fmaf(rv.z, word(cw, rr, i), g[i]);
                        const float hp = r ? hh[r - 1][i] : hprev[i];
                        // g e is both a factor of g h_{t-1} e and the next row's g
                        const float x2 = rv.x * A2[i], e = (!ZOH && half == 1) ? ee[rr][i] : exp2_hw(x2);
                        const float ge = g[i] * e;
                        const float t1 = ge * hp;
                        dA_acc[i] = fmaf(t1, rv.x, dA_acc[i]);
                        s2 = fmaf(t1, Av[i], s2);
                        const float bv = word(bw, rr, i);
                        if constexpr (ZOH) {
                            // beta = delta phi: g phi feeds du (times delta) and dB (times delta u)
                            const float ph = i ? phr.y : phr.x;
                            const float gp = g[i] * ph;
                            s1 = fmaf(gp, bv, s1);
                            s3 = fmaf(ge, bv, s3);
                            db[rq * kNS + i] = gp * rv.y;
                            const float gbx = g[i] * bv * rv.y;  // g B delta u
                            dA_acc[i] = fmaf(gbx, zoh_dbeta_dA_over_delta(x2, e, ph, iA[i], rv.x), dA_acc[i]);
                        } else {
                            s1 = fmaf(g[i], bv, s1);
                            db[rq * kNS + i] = g[i] * rv.y;
                        }
                        g[i] = ge;
                    }
                    s_par[w][rr][lane] = make_float2(s1, s2);
                    if (HAS_Z) s_yp[w][rr][lane] = yp;
                    if (ZOH) s_ge[ZOH ? w : 0][rr][lane] = s3;
                }
                // lane l holds the sums of value l/8 = (row, state) of the quarter
                const float tb = sum8_across_lanes(db), tc = sum8_across_lanes(dc);
                const int k = lane >> 3;
                const int64_t t = int64_t(j) * kSub + half * kHalf + 4 * qt + (k >> 1);
                if ((lane & 7) == 0 && t < L) {
                    const int64_t at = ((blk * NB + ln.b) * L + t) * N + w * kNS + (k & 1);
                    a.part_dB[at] = tb;
                    a.part_dC[at] = tc;
                }
            }
            __syncthreads();
            {
                const int r = row_of(w, half);
                const int64_t t = int64_t(j) * kSub + r;
                if (ln.active && t < L) {
                    float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
                    for (int q = 0; q < kGroups; ++q) {
                        const float2 p = s_par[q][w][lane];
                        s1 += p.x;
                        s2 += p.y;
                    }
                    float du = dlf[half] * s1;
                    if (HAS_D) {
                        du = fmaf(dskip, dypf[half], du);
                        dD_acc = fmaf(dypf[half], xf[half], dD_acc);
                    }
                    // the input path of ddelta: u sum g B (Euler), u sum g e B (zero-order hold)
                    float s_in = s1;
                    if constexpr (ZOH) {
                        s_in = s_ge[0][w][lane];
#pragma unroll
                        for (int q = 1; q < kGroups; ++q) s_in += s_ge[ZOH ? q : 0][w][lane];
                    }
                    const float ddl = fmaf(xf[half], s_in, s2) * sgf[half];
                    dbias_acc += ddl;
                    V::store(r_du, ln.voff, uint32_t(t) * ln.row_bytes, du);
                    V::store(r_ddl, ln.voff, uint32_t(t) * ln.row_bytes, ddl);
                    if constexpr (HAS_Z) {
                        // dz = dy * ypre * silu'(z), ypre = C.h_t + D u
                        float y = s_yp[0][w][lane];
#pragma unroll
                        for (int q = 1; q < kGroups; ++q) y += s_yp[q][w][lane];
                        if (HAS_D) y = fmaf(dskip, xf[half], y);
                        V::store(r_dz, ln.voff, uint32_t(t) * ln.row_bytes, dzf[half] * y);
                    }
                }
            }
            __syncthreads();
        }
    }

    const int64_t bd = ln.b * D + ln.d;
    if (ln.active) {
#pragma unroll
        for (int i = 0; i < kNS; ++i) {
            if (a.dh0) a.dh0[bd * N + w * kNS + i] = g[i];
            a.part_dA[bd * N + w * kNS + i] = dA_acc[i];
        }
    }
    // dD and dbias: the eight waves' per-lane terms, added in wave order
    s_par[w][0][lane] = make_float2(dD_acc, dbias_acc);
    __syncthreads();
    if (w == 0 && ln.active) {
        float sd = 0.0f, sb = 0.0f;
#pragma unroll
        for (int q = 0; q < kGroups; ++q) {
            const float2 p = s_par[q][0][lane];
            sd += p.x;
            sb += p.y;
        }
        a.part_dD[bd] = sd;
        a.part_dbias[bd] = sb;
    }
}

// ---------------------------------------------------------------------------
// bwd_reduce_kernel: fixed-order sums of the partials.  blockIdx.y selects the
// job: 0 = dB, dC over the channel blocks (rounded to the operand type);
// 1 = dA over batch rows; 2 = dD and dbias over batch rows.  block = 256.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs a)
{
    using E = Elem<DT>;
    using T = typename E::T;
    const int64_t k = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t BLN = a.batch * a.seqlen * N;
    if (blockIdx.y == 0) {
        if (k >= BLN) return;
        // in block order; eight blocks' loads in flight at a time
        constexpr int U = 8;
        float sb = 0.0f, sc = 0.0f;
        int64_t q = 0;
        for (; q + U <= a.nblk; q += U) {
            float vb[U], vc[U];
#pragma unroll
            for (int j = 0; j < U; ++j) {
                vb[j] = a.part_dB[(q + j) * BLN + k];
                vc[j] = a.part_dC[(q + j) * BLN + k];
            }
#pragma unroll
            for (int j = 0; j < U; ++j) {
                sb += vb[j];
                sc += vc[j];
            }
        }
        for (; q < a.nblk; ++q) {
            sb += a.part_dB[q * BLN + k];
            sc += a.part_dC[q * BLN + k];
        }
        E::store(static_cast<T*>(a.dB), k, sb);
        E::store(static_cast<T*>(a.dC), k, sc);
    } else if (blockIdx.y == 1) {
        const int64_t DN = a.dim * N;
        if (k >= DN) return;
        float s = 0.0f;
        for (int64_t q = 0; q < a.batch; ++q) s += a.part_dA[q * DN + k];
        a.dA[k] = s;
    } else {
        if (k >= a.dim) return;
        float sd = 0.0f, sb = 0.0f;
        for (int64_t q = 0; q < a.batch; ++q) {
            sd += a.part_dD[q * a.dim + k];
            sb += a.part_dbias[q * a.dim + k];
        }
        if (a.Dskip) a.dD[k] = sd;
        if (a.delta_bias) a.ddelta_bias[k] = sb;
    }
}

template <int DT, bool HAS_D, bool HAS_Z, int MODE>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s)
{
    const dim3 grid(unsigned(a.nblk), unsigned(a.batch));
    bwd_kernel<DT, HAS_D, HAS_Z, MODE><<<grid, dim3(kThreads), 0, s>>>(a);
    int64_t most = a.batch * a.seqlen * N;
    if (a.dim * N > most) most = a.dim * N;
    bwd_reduce_kernel<DT><<<dim3(unsigned((most + 255) / 256), 3), dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

template <int DT, int MODE>
hipError_t dispatch_bwd_mode(const BwdArgs& a, hipStream_t s)
{
    const bool hd = a.Dskip != nullptr, hz = a.z != nullptr;
    if (hd && hz) return launch_bwd_t<DT, true, true, MODE>(a, s);
    if (hd) return launch_bwd_t<DT, true, false, MODE>(a, s);
    if (hz) return launch_bwd_t<DT, false, true, MODE>(a, s);
    return launch_bwd_t<DT, false, false, MODE>(a, s);
}

template <int DT>
hipError_t dispatch_bwd(const BwdArgs& a, hipStream_t s)
{
    switch (a.options & kOptAll) {
        case 0: return dispatch_bwd_mode<DT, 0>(a, s);
        case kOptSoftplus: return dispatch_bwd_mode<DT, kOptSoftplus>(a, s);
        case kOptZoh: return dispatch_bwd_mode<DT, kOptZoh>(a, s);
        default: return dispatch_bwd_mode<DT, kOptSoftplus | kOptZoh>(a, s);
    }
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int dtype, hipStream_t stream)
{
    (void)hipGetLastError();
    return dtype == 0 ? dispatch_bwd<0>(a, stream) : dispatch_bwd<1>(a, stream);
}

}  // namespace ssk
