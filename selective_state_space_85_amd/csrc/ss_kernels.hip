// gfx950 kernels of the selective scan (Mamba walk-through, section 3.3
// "selective_scan"; discrete recurrence of section 2.2; D skip and silu(z)
// gate of section 3.4) and of the single-token recurrent update.
//
// Scan work decomposition
//  * A workgroup of kGroups waves (8) owns 64 consecutive channels d of one
//    batch row b (lane = channel) and one chunk of the sequence.  Wave w holds
//    state entries n = kNS*w .. kNS*w+kNS-1 of every channel in registers, so
//    B[b,t,n] and C[b,t,n] are the same for all lanes of a wave: they are
//    scalar operands.  Per element the wave issues one multiply (delta*A), one
//    exp2, one multiply (delta*u*B), one fma (state) and one fma (C.h) -- no
//    MFMA: nothing here is a dense contraction.
//  * B and C reach the waves through a panel: a pre-pass (panel_kernel) copies
//    them to fp32 in the workspace, grouped per wave so that a wave's entries
//    of consecutive rows are contiguous, zero-padded past the chunk end.  A
//    tile of rows then costs one 16-word scalar load for B and one for C, with
//    no widening or row clamping on the scalar unit.
//  * The sequence is processed in tiles of kTileRows rows.  Per tile, each wave
//    widens its share of the rows' u and delta once and publishes
//    (delta, delta*u) in LDS for the other waves; each wave leaves its partial
//    C.h per row in LDS; each wave then finishes its share of rows (sum of the
//    partials, D skip, silu(z) gate, rounding, store).  LDS buffers alternate
//    between even and odd tiles, so one barrier per tile suffices.
//  * Prefetch: u/delta/z rows three tiles ahead (raw buffer loads, the channel
//    as vector offset and the row as scalar offset, so stepping in t costs no
//    vector instruction); the wave's B/C words one tile ahead, issued right
//    after the tile's LDS reads have landed so that no LDS wait drains them.
//  * The sequence can be cut into chunks (LTI chapter 3.1, section 3.1.5.2:
//    the recurrence is a scan over an associative operator).  For K > 1:
//      1. scan_kernel<aggregate> runs chunks 0..K-2 from a zero state and
//         keeps only each chunk's end state S_c and its delta sum;
//      2. carry_kernel combines the affine pairs (P_c, S_c),
//         P_c = exp(A * sum_t delta_t), with a wave-level inclusive prefix over
//         chunks (64 chunks per pass) into the carry of every chunk;
//      3. scan_kernel<emit> reruns every chunk from its carry and writes y.
//    Only y, the chunk carries and h_last reach memory: the per-timestep
//    states and the discretised operands exp(delta*A), delta*B*u never do (the
//    fused, state-in-fast-memory point of section 3.3 and of LTI chapter
//    section 3.1.5.3).
//  * exp(x) is evaluated as exp2(x * log2 e) on the hardware exp2 unit, with
//    A pre-scaled by log2 e once per lane.
#include "ss_device.h"

namespace ssk {
namespace {

// ---------------------------------------------------------------------------
// Panel kernel: the fp32 B/C panel of every (batch row, chunk),
//   panel[b][c][w][part][p][i] = (part ? C : B)[b, c*chunk_len + p, w*kNS + i]
// for rows p inside the chunk and 0 for the rest of the chunk's panel_rows.
// One thread per panel word; grid = ceil(words / 256), block = 256.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(256) void panel_kernel(ScanArgs a)
{
    using E = Elem<DT>;
    using T = typename E::T;
    const int64_t P = a.panel_rows;
    const int64_t total = a.batch * a.n_chunks * kGroups * 2 * P * kNS;
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= total) return;
    const int i = int(idx % kNS);
    int64_t rest = idx / kNS;
    const int64_t p = rest % P;
    rest /= P;
    const int part = int(rest % 2);
    rest /= 2;
    const int g = int(rest % kGroups);
    rest /= kGroups;
    const int64_t c = rest % a.n_chunks;
    const int64_t b = rest / a.n_chunks;
    const int64_t t0 = c * a.chunk_len;
    const int64_t len = (a.seqlen - t0 < a.chunk_len) ? a.seqlen - t0 : a.chunk_len;
    float v = 0.0f;
    if (p < len) v = E::load(static_cast<const T*>(part ? a.C : a.B), (b * a.seqlen + t0 + p) * N + g * kNS + i);
    a.ws_panel[idx] = v;
}

// ---------------------------------------------------------------------------
// Scan kernel.  grid = (ceil(dim/64), batch, chunks), block = 64 * kGroups.
// EMIT: start from the chunk's carry (or h0), write y and, for the last chunk,
//       h_last.
// !EMIT (aggregate): start from zero, write the chunk's end state into state
//       slot c+1 and its delta sum.
// Host guarantees: chunk_len * dim * element size < 2^31.
// ---------------------------------------------------------------------------
// The zero-order hold's extra arithmetic would take the kernel just past 80
// VGPRs, which leaves room for two 8-wave workgroups per CU instead of three;
// it is held to 80 (six waves per SIMD).
template <int DT, bool EMIT, bool HAS_D, bool HAS_Z, int MODE, bool CKPT = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu((MODE & kOptZoh) ? 6 : 2))) void scan_kernel(
    ScanArgs a)
{
    constexpr bool ZOH = (MODE & kOptZoh) != 0;
    using T = typename Elem<DT>::T;
    using V = Buf<DT>;
    using Raw = typename V::Raw;
    constexpr int TT = kTileRows;
    constexpr int RPW = TT / kGroups;     // rows each wave widens and finishes per tile
    constexpr int PW = TT * kNS / 16;     // 16-word panel loads per tile and plane

    __shared__ float2 s_xd[2][TT][kWave];                       // (delta, delta*u) per row and channel
    __shared__ float s_iv[ZOH ? 2 : 1][TT][kWave];              // 1/delta per row and channel (ZOH)
    __shared__ float s_part[EMIT ? 2 : 1][kGroups][TT][kWave];  // partial C.h per wave

    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t D = a.dim, L = a.seqlen, BD = a.batch * a.dim;
    const int64_t d_raw = int64_t(blockIdx.x) * kWave + lane;
    const bool active = d_raw < D;
    const int64_t d = active ? d_raw : D - 1;  // idle lanes shadow the last channel
    const int64_t b = blockIdx.y;
    const int64_t c = blockIdx.z;
    const int64_t t0 = c * a.chunk_len;
    const int len = int(((t0 + a.chunk_len < L) ? t0 + a.chunk_len : L) - t0);
    // an even number of tiles; rows past the chunk end are neutral (see publish_rows)
    const int ntiles = (((len + TT - 1) / TT) + 1) & ~1;
    const int64_t bd = b * D + d;
    const int64_t row0 = (b * L + t0) * D;  // first element of the chunk's first row

    const uint32_t row_bytes = uint32_t(D) * V::kBytes;
    const uint32_t span = uint32_t(len) * row_bytes;
    const uint32_t voff = active ? uint32_t(d_raw) * V::kBytes : kIdleOffset;
    const __amdgpu_buffer_rsrc_t r_u = make_rsrc(static_cast<const T*>(a.u) + row0, span);
    const __amdgpu_buffer_rsrc_t r_dl = make_rsrc(static_cast<const T*>(a.delta) + row0, span);
    const __amdgpu_buffer_rsrc_t r_z = make_rsrc(HAS_Z ? static_cast<const T*>(a.z) + row0 : nullptr, span);
    const __amdgpu_buffer_rsrc_t r_y = make_rsrc(EMIT ? static_cast<T*>(a.y) + row0 : nullptr, span);
    // the wave's B and C planes of the chunk's panel (address-space casts need the C cast form)
    const int64_t plane = a.panel_rows * kNS;
    const SS_CONST char* pB =
        (const SS_CONST char*)(a.ws_panel + ((b * a.n_chunks + c) * kGroups + w) * 2 * plane);
    const SS_CONST char* pC = pB + plane * 4;

    const int64_t sbase = bd * N + w * kNS;  // this lane's entries in a (B, D, N) state array
    float A2[kNS], iA[kNS];  // A * log2 e, and 1/A for the zero-order hold
#pragma unroll
    for (int i = 0; i < kNS; ++i) {
        const float av = a.A[d * N + w * kNS + i];
        A2[i] = av * kLog2e;
        iA[i] = ZOH ? 1.0f / av : 0.0f;
    }
    const float bias = a.delta_bias ? a.delta_bias[d] : 0.0f;

    float h[kNS];
    const bool from_ws = EMIT && a.n_chunks > 1;
    const bool from_h0 = EMIT && a.n_chunks == 1 && a.h0 != nullptr;
    if (from_ws || from_h0) {
        const float* init = from_ws ? a.ws_state + c * BD * N + sbase : a.h0 + sbase;
#pragma unroll
        for (int i = 0; i < kNS; ++i) h[i] = init[i];
    } else {
#pragma unroll
        for (int i = 0; i < kNS; ++i) h[i] = 0.0f;
    }
    const float dskip = (EMIT && HAS_D) ? a.Dskip[d] : 0.0f;
    float dsum = 0.0f;

    Raw rdl[2][RPW], ru[2][RPW], rz[2][RPW];  // raw rows in flight, by tile parity
    float xf[2][RPW], zf[2][RPW];             // widened u, z kept for the epilogue
    Words16 bw[2][PW], cw[2][PW];             // the tile's panel words, by tile parity

    // row r of the chunk, clamped to the last one
    auto clamp_row = [&](int r) { return r < len ? r : len - 1; };

    auto issue_rows = [&](int tile, auto slot) {
        constexpr int S = decltype(slot)::value;
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
            const uint32_t so = uint32_t(clamp_row(tile * TT + w * RPW + j)) * row_bytes;
            rdl[S][j] = V::load(r_dl, voff, so);
            ru[S][j] = V::load(r_u, voff, so);
            if (EMIT && HAS_Z) rz[S][j] = V::load(r_z, voff, so);
        }
    };
    // widen this wave's rows of a tile and publish (delta, delta*u).  Rows past
    // the chunk end are published as (0, 0): exp2(0) = 1 and 0*B = 0 leave the
    // state bit-unchanged, so the last tiles need no row-count branches.
    auto publish_rows = [&](int tile, auto slot) {
        constexpr int S = decltype(slot)::value;
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
            const bool in = tile * TT + w * RPW + j < len;
            const float dl = in ? step_size<MODE>(V::widen(rdl[S][j]), bias) : 0.0f;
            const float x = V::widen(ru[S][j]);
            s_xd[S][w * RPW + j][lane] = make_float2(dl, dl * x);
            if constexpr (ZOH) s_iv[S][w * RPW + j][lane] = __builtin_amdgcn_rcpf(dl);
            if (EMIT) {
                xf[S][j] = x;
                if (HAS_Z) {
                    // widen z now: a raw value kept to the epilogue would outlive
                    // its prefetch slot and force a wait on every row load in flight
                    zf[S][j] = V::widen(rz[S][j]);
                    __asm__ volatile("" : "+v"(zf[S][j]));
                }
            }
        }
    };
    // a tile's panel rows are contiguous: 16-word scalar loads at a 32-bit
    // byte offset from the plane's 64-bit base, no clamping (the panel holds
    // zero rows past the chunk end and one spare tile)
    auto issue_words = [&](int tile, auto slot) {
        constexpr int S = decltype(slot)::value;
        const uint32_t off = uint32_t(tile) * uint32_t(TT * kNS * 4);
        const SS_CONST Words16* qb = (const SS_CONST Words16*)(pB + off);
        const SS_CONST Words16* qc = (const SS_CONST Words16*)(pC + off);
#pragma unroll
        for (int q = 0; q < PW; ++q) {
            bw[S][q] = qb[q];
            if (EMIT) cw[S][q] = qc[q];
        }
    };
    // entry i of row r of a tile, from its panel words
    auto word = [&](const Words16 (&wv)[PW], int r, int i) {
        const int k = r * kNS + i;
        return __uint_as_float(wv[k / 16][k % 16]);
    };
    // finish this wave's rows of a tile: sum the partials, skip, gate, store
    auto finish_rows = [&](int tile, auto slot) {
        constexpr int S = decltype(slot)::value;
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
            const int r = w * RPW + j;
            const int t = tile * TT + r;
            if (t < len) {
                float acc = s_part[S][0][r][lane];
#pragma unroll
                for (int g = 1; g < kGroups; ++g) acc += s_part[S][g][r][lane];
                if (HAS_D) acc = fmaf(dskip, xf[S][j], acc);
                if (HAS_Z) acc *= silu(zf[S][j]);
                V::store(r_y, voff, uint32_t(t) * row_bytes, acc);
            }
        }
    };
    // the recurrence over one tile for this wave's state entries
    auto scan_rows = [&](int tile, auto slot) {
        constexpr int S = decltype(slot)::value;
        float2 xd[TT];
#pragma unroll
        for (int r = 0; r < TT; ++r) xd[r] = s_xd[S][r][lane];
        // the next tile's scalar loads go out only after all of this tile's LDS
        // reads have landed (LDS and scalar loads share one counter, and scalar
        // loads return out of order: a later LDS wait would drain them too)
        static_assert(TT == 8, "the wait below names eight rows");
        float iv[TT];  // 1/delta per row (zero-order hold only)
#pragma unroll
        for (int r = 0; r < TT; ++r) iv[r] = ZOH ? s_iv[ZOH ? S : 0][r][lane] : 0.0f;
        __asm__ volatile("" ::"v"(xd[0].x), "v"(xd[0].y), "v"(xd[1].x), "v"(xd[1].y), "v"(xd[2].x), "v"(xd[2].y),
                         "v"(xd[3].x), "v"(xd[3].y), "v"(xd[4].x), "v"(xd[4].y), "v"(xd[5].x), "v"(xd[5].y),
                         "v"(xd[6].x), "v"(xd[6].y), "v"(xd[7].x), "v"(xd[7].y)
                         : "memory");
        if constexpr (ZOH)
            __asm__ volatile("" ::"v"(iv[0]), "v"(iv[1]), "v"(iv[2]), "v"(iv[3]), "v"(iv[4]), "v"(iv[5]), "v"(iv[6]),
                             "v"(iv[7])
                             : "memory");
        issue_words(tile + 1, Slot<1 - S>{});
        // All delta*A products of the tile are formed before the first exp2 is
        // issued (the empty asm statements pin them in registers), so every
        // exp2 reads an operand produced many instructions earlier instead of
        // waiting on the multiply right before it.
        float x2[TT][kNS], e[TT][kNS];
#pragma unroll
        for (int r = 0; r < TT; ++r) {
#pragma unroll
            for (int i = 0; i < kNS; ++i) x2[r][i] = xd[r].x * A2[i];
        }
        pin_rows(x2);
#pragma unroll
        for (int r = 0; r < TT; ++r) {
#pragma unroll
            for (int i = 0; i < kNS; ++i) e[r][i] = exp2_hw(x2[r][i]);
        }
#pragma unroll
        for (int r = 0; r < TT; ++r) {
            const float xb = xd[r].y;
#pragma unroll
            for (int i = 0; i < kNS; ++i) {
                float in_term = xb * word(bw[S], r, i);  // delta*B*u (Euler)
                if constexpr (ZOH) in_term *= zoh_phi(x2[r][i], e[r][i], iA[i] * iv[r]);
                h[i] = fmaf(e[r][i], h[i], in_term);
            }
            if constexpr (EMIT) {
                float acc = 0.0f;
#pragma unroll
                for (int i = 0; i < kNS; ++i) acc = fmaf(word(cw[S], r, i), h[i], acc);
                s_part[S][w][r][lane] = acc;
            } else {
                dsum += xd[r].x;
            }
        }
    };

    // one tile step: finish tile k-1, publish tile k+1, scan tile k
    // every load below is clamped to a valid row, so all of it runs unconditionally
    auto step = [&](int k, auto slot) {
        constexpr int S = decltype(slot)::value;
        if constexpr (EMIT) {
            if (k >= 1) finish_rows(k - 1, Slot<1 - S>{});
        }
        publish_rows(k + 1, Slot<1 - S>{});
        issue_rows(k + 3, Slot<1 - S>{});
        scan_rows(k, Slot<S>{});
        __syncthreads();
    };

    issue_rows(0, Slot<0>{});
    issue_rows(1, Slot<1>{});
    publish_rows(0, Slot<0>{});
    issue_rows(2, Slot<0>{});
    issue_words(0, Slot<0>{});
    __syncthreads();

    // Two or three workgroups share a CU, and the wave arbiter favours older
    // waves: left alone, the first workgroup finishes far ahead of the last and
    // the CU ends its run with a single latency-bound workgroup.  Lowering a
    // wave's priority at each quarter of the chunk lets the laggards catch up,
    // so the workgroups of a CU stay within a quarter of each other.
    static_assert(2 * kTileRows == kBwdSub, "checkpoints fall at the start of every tile pair");
    // checkpoints (a separate instantiation: the plain kernel has no scalar
    // registers to spare): this lane's entries of the one at row t0 + k*TT,
    // advanced by one checkpoint per tile pair
    float* ck_row = nullptr;
    int64_t ck_step = 0;
    if constexpr (CKPT) {
        ck_row = a.ckpt + ((t0 / kBwdSub * a.batch + b) * N + w * kNS) * D + d;
        ck_step = a.batch * N * D;
    }
    const int quarter = (ntiles / 4) & ~1;
    __builtin_amdgcn_s_setprio(3);
    for (int k = 0; k < ntiles; k += 2) {
        if (quarter > 0) {
            if (k == quarter) __builtin_amdgcn_s_setprio(2);
            else if (k == 2 * quarter) __builtin_amdgcn_s_setprio(1);
            else if (k == 3 * quarter) __builtin_amdgcn_s_setprio(0);
        }
        if constexpr (CKPT) {
            // the state entering row t0 + k*TT, a multiple of kBwdSub (k is even)
            if (active && k * TT < len) {
#pragma unroll
                for (int i = 0; i < kNS; ++i) ck_row[int64_t(i) * D] = h[i];
            }
            ck_row += ck_step;
        }
        step(k, Slot<0>{});
        step(k + 1, Slot<1>{});
    }
    if constexpr (EMIT) finish_rows(ntiles - 1, Slot<1>{});

    if (!active) return;
    if (EMIT) {
        if (c == a.n_chunks - 1 && a.h_last) {
#pragma unroll
            for (int i = 0; i < kNS; ++i) a.h_last[sbase + i] = h[i];
        }
    } else {
        float* dst = a.ws_state + (c + 1) * BD * N + sbase;
#pragma unroll
        for (int i = 0; i < kNS; ++i) dst[i] = h[i];
        if (w == 0) a.ws_dsum[c * BD + bd] = dsum;
    }
}

// ---------------------------------------------------------------------------
// Carry kernel.  Each chunk c < K-1 has its affine pair
// (P_c, S_c) = (exp(A * sum of delta over chunk c), end state of c from zero).
// An inclusive Hillis-Steele combine over lanes, earlier pair first,
//   (a1, b1) then (a2, b2) -> (a2*a1, a2*b1 + b2),
// gives each lane the composite map of chunks 0..c; applied to the incoming
// state it yields the carry H_c (state after chunk c), stored in slot c+1.
// Slot 0 receives the initial state.
// One wave per channel.  It holds R = 4..64 consecutive chunks (R the power
// of two covering the K-1 aggregated chunks, 64 and passes of 64 beyond that)
// for each of 64/R state entries at a time: lane l takes chunk base + l%R of
// entry n0 + l/R, so that with few chunks the lanes are not left idle, and the
// wave covers the 16 entries in 64/R groups (the entries of a slot share
// cache lines, so they stay with one wave).  The combine is a scan within
// each row of 16 lanes (DPP row shifts 1, 2, 4, 8, masked at the edges of
// groups narrower than a row), then, for R = 32 and 64, the broadcasts of lane
// 15 into rows 1 and 3 and of lane 31 into rows 2 and 3.  Lanes past the last
// chunk hold the identity (1, 0), so a group's last lane ends with the pass's
// total.  grid = batch*dim, block = 64.
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void combine_from(float& P, float& S, bool take = true)
{
    // a source outside the row (or a row left out by ROW_MASK) reads the identity (1, 0)
    float Pp = __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(P), CTRL, ROW_MASK, 0xf, false));
    float Sp = __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(0.0f), __float_as_int(S), CTRL, ROW_MASK, 0xf, false));
    if (!take) {  // the source is another group's chunk
        Pp = 1.0f;
        Sp = 0.0f;
    }
    S = fmaf(P, Sp, S);
    P *= Pp;
}

template <int R>
__global__ __launch_bounds__(kWave) void carry_kernel(ScanArgs a)
{
    static_assert(R >= 4 && R <= kWave && (R & (R - 1)) == 0, "R: 4..64, a power of two");
    constexpr int G = kWave / R;  // state entries per wave
    const int64_t bd = blockIdx.x;
    const int64_t BD = a.batch * a.dim;
    const int64_t d = bd % a.dim;
    const int lane = threadIdx.x;
    const int i = lane % R;  // chunk within the pass
    const int64_t n_carry = a.n_chunks - 1;

    // the wave's entries: n = q*G + lane/R for q < N/G, all advanced together so
    // that their loads and combines overlap
    constexpr int NG = N / G;
    float A2[NG], hin[NG];
#pragma unroll
    for (int q = 0; q < NG; ++q) {
        const int n = q * G + lane / R;
        A2[q] = a.A[d * N + n] * kLog2e;
        hin[q] = a.h0 ? a.h0[bd * N + n] : 0.0f;
        if (i == 0) a.ws_state[bd * N + n] = hin[q];
    }

    for (int64_t base = 0; base < n_carry; base += R) {
        const int64_t c = base + i;
        const bool valid = c < n_carry;
        const float dsum = valid ? a.ws_dsum[c * BD + bd] : 0.0f;
        float* slot = a.ws_state + ((c + 1) * BD + bd) * N + lane / R;
        float S[NG];
#pragma unroll
        for (int q = 0; q < NG; ++q) S[q] = valid ? slot[q * G] : 0.0f;
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            float P = valid ? exp2_hw(A2[q] * dsum) : 1.0f;
            float Sq = S[q];
            combine_from<kDppRowShr1, 0xf>(P, Sq, R >= 16 || i >= 1);
            combine_from<kDppRowShr2, 0xf>(P, Sq, R >= 16 || i >= 2);
            if constexpr (R >= 8) combine_from<kDppRowShr4, 0xf>(P, Sq, R >= 16 || i >= 4);
            if constexpr (R >= 16) combine_from<kDppRowShr8, 0xf>(P, Sq);
            if constexpr (R >= 32) combine_from<kDppRowBcast15, 0xa>(P, Sq);
            if constexpr (R >= 64) combine_from<kDppRowBcast31, 0xc>(P, Sq);
            const float H = fmaf(P, hin[q], Sq);
            if (valid) slot[q * G] = H;
            // the next pass (only when R = 64) starts from this pass's total
            if constexpr (R == kWave) hin[q] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(H), kWave - 1));
        }
    }
}

template <int R>
void launch_carry(const ScanArgs& a, hipStream_t s)
{
    carry_kernel<R><<<dim3(unsigned(a.batch * a.dim)), dim3(kWave), 0, s>>>(a);
}

// ---------------------------------------------------------------------------
// Recurrent step.  Four lanes per channel (b, d), each with 4 of the 16 state
// entries (16-byte loads/stores of h), the quad's partial C.h summed with two
// butterfly exchanges.  grid = ceil(batch*dim*4 / 256), block = 256.
// ---------------------------------------------------------------------------
template <int DT, bool HAS_D, bool HAS_Z, int MODE>
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
    const float dl = step_size<MODE>(E::load(delta, bd), a.delta_bias ? a.delta_bias[d] : 0.0f);
    const float x = E::load(u, bd);
    const float xb = dl * x;
    const float inv_dl = (MODE & kOptZoh) ? __builtin_amdgcn_rcpf(dl) : 0.0f;
    const int64_t s0 = b * N + q * 4;

    float hs[4] = {hv.x, hv.y, hv.z, hv.w};
    const float as[4] = {av.x, av.y, av.z, av.w};
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float x2 = dl * (as[i] * kLog2e);
        const float abar = exp2_hw(x2);
        float in_term = xb * E::load(Bm, s0 + i);
        if constexpr ((MODE & kOptZoh) != 0) in_term *= zoh_phi(x2, abar, (1.0f / as[i]) * inv_dl);
        hs[i] = fmaf(abar, hs[i], in_term);
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

template <int DT, bool HAS_D, bool HAS_Z, int MODE>
hipError_t launch_scan_t(const ScanArgs& a, hipStream_t s)
{
    const unsigned nblk = unsigned((a.dim + kWave - 1) / kWave);
    const int64_t words = a.batch * a.n_chunks * 2 * a.panel_rows * N;
    panel_kernel<DT><<<dim3(unsigned((words + 255) / 256)), dim3(256), 0, s>>>(a);
    if (a.n_chunks > 1) {
        scan_kernel<DT, false, false, false, MODE>
            <<<dim3(nblk, unsigned(a.batch), unsigned(a.n_chunks - 1)), dim3(kThreads), 0, s>>>(a);
        // R lanes per state entry: the power of two covering the K-1 aggregated chunks, 4..64
        const int64_t n_carry = a.n_chunks - 1;
        if (n_carry <= 4)
            launch_carry<4>(a, s);
        else if (n_carry <= 8)
            launch_carry<8>(a, s);
        else if (n_carry <= 16)
            launch_carry<16>(a, s);
        else if (n_carry <= 32)
            launch_carry<32>(a, s);
        else
            launch_carry<64>(a, s);
    }
    const dim3 grid(nblk, unsigned(a.batch), unsigned(a.n_chunks));
    if (a.ckpt)
        scan_kernel<DT, true, HAS_D, HAS_Z, MODE, true><<<grid, dim3(kThreads), 0, s>>>(a);
    else
        scan_kernel<DT, true, HAS_D, HAS_Z, MODE><<<grid, dim3(kThreads), 0, s>>>(a);
    return hipGetLastError();
}

template <int DT, bool HAS_D, bool HAS_Z, int MODE>
hipError_t launch_step_t(const StepArgs& a, hipStream_t s)
{
    const int64_t threads = a.batch * a.dim * 4;
    const unsigned blocks = unsigned((threads + 255) / 256);
    step_kernel<DT, HAS_D, HAS_Z, MODE><<<dim3(blocks), dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

template <int DT, int MODE>
hipError_t dispatch_scan_mode(const ScanArgs& a, hipStream_t s)
{
    const bool hd = a.Dskip != nullptr, hz = a.z != nullptr;
    if (hd && hz) return launch_scan_t<DT, true, true, MODE>(a, s);
    if (hd) return launch_scan_t<DT, true, false, MODE>(a, s);
    if (hz) return launch_scan_t<DT, false, true, MODE>(a, s);
    return launch_scan_t<DT, false, false, MODE>(a, s);
}

template <int DT>
hipError_t dispatch_scan(const ScanArgs& a, hipStream_t s)
{
    switch (a.options & kOptAll) {
        case 0: return dispatch_scan_mode<DT, 0>(a, s);
        case kOptSoftplus: return dispatch_scan_mode<DT, kOptSoftplus>(a, s);
        case kOptZoh: return dispatch_scan_mode<DT, kOptZoh>(a, s);
        default: return dispatch_scan_mode<DT, kOptSoftplus | kOptZoh>(a, s);
    }
}

template <int DT, int MODE>
hipError_t dispatch_step_mode(const StepArgs& a, hipStream_t s)
{
    const bool hd = a.Dskip != nullptr, hz = a.z != nullptr;
    if (hd && hz) return launch_step_t<DT, true, true, MODE>(a, s);
    if (hd) return launch_step_t<DT, true, false, MODE>(a, s);
    if (hz) return launch_step_t<DT, false, true, MODE>(a, s);
    return launch_step_t<DT, false, false, MODE>(a, s);
}

template <int DT>
hipError_t dispatch_step(const StepArgs& a, hipStream_t s)
{
    switch (a.options & kOptAll) {
        case 0: return dispatch_step_mode<DT, 0>(a, s);
        case kOptSoftplus: return dispatch_step_mode<DT, kOptSoftplus>(a, s);
        case kOptZoh: return dispatch_step_mode<DT, kOptZoh>(a, s);
        default: return dispatch_step_mode<DT, kOptSoftplus | kOptZoh>(a, s);
    }
}

}  // namespace

hipError_t launch_scan(const ScanArgs& a, int dtype, hipStream_t stream)
{
    (void)hipGetLastError();  // start from a clean per-thread error state
    return dtype == 0 ? dispatch_scan<0>(a, stream) : dispatch_scan<1>(a, stream);
}

hipError_t launch_panel(const ScanArgs& a, int dtype, hipStream_t stream)
{
    (void)hipGetLastError();
    const int64_t words = a.batch * a.n_chunks * 2 * a.panel_rows * N;
    const dim3 grid(unsigned((words + 255) / 256));
    if (dtype == 0)
        panel_kernel<0><<<grid, dim3(256), 0, stream>>>(a);
    else
        panel_kernel<1><<<grid, dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_step(const StepArgs& a, int dtype, hipStream_t stream)
{
    (void)hipGetLastError();
    return dtype == 0 ? dispatch_step<0>(a, stream) : dispatch_step<1>(a, stream);
}

}  // namespace ssk
