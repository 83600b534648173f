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
//    the recurrence is a scan over an associative operator).  For K > 1 and
//    chunks shorter than 1024 rows:
//      1. scan_kernel<aggregate> runs chunks 0..K-2 from a zero state and
//         keeps only each chunk's end state S_c and its delta sum;
//      2. carry_kernel combines the affine pairs (P_c, S_c),
//         P_c = exp(A * sum_t delta_t), with a wave-level inclusive prefix over
//         chunks (64 chunks per pass) into the carry of every chunk;
//      3. scan_kernel<emit> reruns every chunk from its carry and writes y.
//    For chunks of 1024 rows or more (emit first, CORR):
//      1. scan_kernel<emit, CORR> pass 1 runs every chunk from its own start
//         (h0 for chunk 0, zero for the others), writes y and keeps S_c and the
//         delta sum, as the aggregate pass would;
//      2. carry_kernel as above;
//      3. pass 2 reruns each chunk c >= 1 from its carry over its first rows
//         only, rewriting y there.  The carry's share of the state decays as
//         exp(A * sum of delta); once it is below fp32 resolution of the state
//         the first pass's y is already right.  A workgroup where that does not
//         hold (or with A > 0 or a negative step size) reruns the whole chunk.
//    Only y, the chunk carries and h_last reach memory: the per-timestep
//    states and the discretised operands exp(delta*A), delta*B*u never do (the
//    fused, state-in-fast-memory point of section 3.3 and of LTI chapter
//    section 3.1.5.3).
//  * exp(x) is evaluated as exp2(x * log2 e) on the hardware exp2 unit, with
//    A pre-scaled by log2 e once per lane.
#include <atomic>
#include <mutex>

#include "ss_device.h"

// The workspace of ss_scan_fwd_noalloc: one array per GPU (each device holds
// its own copy of a __device__ variable), alive until the process ends.  Host
// code never uses the name itself as an address -- on the host it is only a
// stand-in for the symbol -- but the device address that scratch_pointer looks
// up for the current device.
static __device__ __align__(256) unsigned char scratch[ssk::kScratchBytes];

namespace ssk {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;
}  // namespace

hipError_t scratch_pointer(void** ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

namespace {

// ---------------------------------------------------------------------------
// Panel kernel: the fp32 B/C panel of every (batch row, chunk),
//   panel[b][c][w][part][p][i] = (part ? C : B)[b, c*chunk_len + p, w*kNS + i]
// for rows p inside the chunk and 0 for the rest of the chunk's panel_rows.
// One thread per panel word; grid = (ceil(panel_rows * kNS / 256), kGroups * 2,
// the launch's (batch row, chunk) pairs from bc0 on), block = 256.  The word's
// place comes from the grid and a shift (one flat index split by 64-bit
// divisions took the long context's panel 14.9 -> 18.2 us).
template <int DT>
__global__ __launch_bounds__(256) void panel_kernel(ScanArgs a, int64_t bc0)
{
    using E = Elem<DT>;
    using T = typename E::T;
    const int64_t P = a.panel_rows;
    const int64_t k = int64_t(blockIdx.x) * 256 + threadIdx.x;  // word within the plane: row k/kNS
    if (k >= P * kNS) return;
    const int64_t bc = bc0 + blockIdx.z;  // b * n_chunks + c
    const int64_t b = bc / a.n_chunks;     // uniform: a scalar division per wave
    const int64_t c = bc - b * a.n_chunks;
    const int g = int(blockIdx.y >> 1), part = int(blockIdx.y & 1);
    const int64_t p = k / kNS;
    const int i = int(k % kNS);
    const int64_t t0 = c * a.chunk_len;
    const int64_t len = (a.seqlen - t0 < a.chunk_len) ? a.seqlen - t0 : a.chunk_len;
    float v = 0.0f;
    if (p < len) v = E::load(static_cast<const T*>(part ? a.C : a.B), (b * a.seqlen + t0 + p) * N + g * kNS + i);
    a.ws_panel[((bc * kGroups + g) * 2 + part) * P * kNS + k] = v;
}

template <int DT>
void launch_panel_t(const ScanArgs& a, hipStream_t s)
{
    const int64_t bcs = a.batch * a.n_chunks;
    const unsigned gx = unsigned((a.panel_rows * kNS + 255) / 256);
    constexpr int64_t kMaxZ = 65535;
    for (int64_t bc0 = 0; bc0 < bcs; bc0 += kMaxZ) {
        const dim3 grid(gx, unsigned(kGroups * 2), unsigned(bcs - bc0 < kMaxZ ? bcs - bc0 : kMaxZ));
        panel_kernel<DT><<<grid, dim3(256), 0, s>>>(a, bc0);
    }
}

// ---------------------------------------------------------------------------
// Scan kernel.  Two layouts of the same work, both with the 16 state entries
// of a channel split into 8 groups of 2 (one group per 64 lanes of state):
//  * whole-wave (HALF = false): a workgroup of 8 waves owns 64 channels of one
//    batch row and chunk; wave w holds group w of every channel (lane =
//    channel), so B and C are wave-uniform scalar operands.
//    grid = (ceil(dim/64), batch, chunks), block = 512.
//  * half-wave (HALF = true): a workgroup of 4 waves owns 32 channels; the two
//    32-lane halves of wave w hold groups 2w and 2w+1 (lane = channel within
//    a half).  B and C then differ between the halves: each wave loads a
//    tile's 16 values of its two groups into one register (lane 16q + k holds
//    value k of the group of its half: row k/2, entry k%2) and every use takes
//    value k by a broadcast within the lane's row of 16 lanes (DPP
//    row_newbcast, folded into the multiply or the fma).  Twice as many
//    workgroups of half the size: the large layer's 640 whole-wave blocks on
//    256 CUs leave half of the CUs with three and half with two, its 1280
//    half-wave blocks give every CU five.  RAW (the aggregate and emit passes
//    of the short-chunk scheme, without checkpoints) loads that register from
//    the (B, L, N) arrays themselves, widening bf16 with a shift, so the call
//    needs no panel pass: one launch fewer, where the launches are a large
//    part of a short call, for one or two more vector instructions per tile.
//    grid = (ceil(dim/32), batch, chunks), block = 256.
// In both, each (row, channel) of a tile is widened and published by one lane
// and finished by the same lane.
// EMIT: start from the chunk's carry (or h0), write y and, for the last chunk,
//       h_last.
// !EMIT (aggregate): start from zero, write the chunk's end state into state
//       slot c+1 and its delta sum.
// CKPT: also store the state entering every second tile (every kBwdSub rows)
//       in a.ckpt.  With !EMIT (the backward's checkpoint pass, one chunk,
//       half-wave) that is all it writes: it starts from h0 and keeps no end
//       state or delta sum.
// Host guarantees: chunk_len * dim * element size < 2^31.
// ---------------------------------------------------------------------------
// The zero-order hold's extra arithmetic would take the whole-wave kernel just
// past 80 VGPRs, which leaves room for two 8-wave workgroups per CU instead of
// three; it is held to 80 (six waves per SIMD).  The half-wave emit-first pass
// 1 (every chunk of a long sequence) is held to 64 (eight workgroups per CU, as
// its LDS allows, instead of seven): a handful of values spill, outside the tile
// loop, and the long context took 0.94 against 0.955 ms, B=4 L=16384 D=2048 0.499
// against 0.511 ms.  (Holding the whole-wave emit-first passes to 64, four
// workgroups per CU instead of three, made the long context 23% slower.)
template <bool HALF>
struct ScanShape {
    static constexpr int kWaves = HALF ? 4 : kGroups;  // waves per workgroup
    static constexpr int kCh = HALF ? 32 : kWave;      // channels per workgroup
};

template <bool HALF>
constexpr int scan_threads()
{
    return HALF ? 4 * kWave : kGroups * kWave;
}
template <int MODE, int CORR, bool HALF>
constexpr int scan_waves_per_eu()
{
    return (MODE & kOptZoh) ? 6 : (CORR == 1 && HALF ? 8 : 2);
}

template <int DT, bool EMIT, bool HAS_D, bool HAS_Z, int MODE, bool CKPT = false, bool HALF = false,
          int CORR = 0, bool RAW = false>
__global__ __launch_bounds__(scan_threads<HALF>())
    __attribute__((amdgpu_waves_per_eu(scan_waves_per_eu<MODE, CORR, HALF>()))) void scan_kernel(ScanArgs a)
{
    static_assert(CORR == 0 || (EMIT && !CKPT), "the emit-first passes are emit passes without checkpoints");
    static_assert(!RAW || (HALF && CORR == 0 && !CKPT), "B and C unpanelled: the half-wave aggregate scheme only");
    constexpr bool ZOH = (MODE & kOptZoh) != 0;
    using T = typename Elem<DT>::T;
    using V = Buf<DT>;
    using Raw = typename V::Raw;
    constexpr int TT = kTileRows;
    constexpr int CH = ScanShape<HALF>::kCh;
    // rows each lane widens and finishes per tile: one in the half-wave layout
    // (wave w, half h: row 2w + h); TT / kGroups in the whole-wave one
    constexpr int RPW = HALF ? 1 : TT / kGroups;
    constexpr int PW = TT * kNS / 16;  // 16-word panel loads per tile and plane (whole-wave)
    static_assert(!HALF || (TT == 8 && kNS == 2 && kGroups == 8),
                  "half-wave layout: 8-row tiles, a tile's 16 values of a group in one register");

    __shared__ float2 s_xd[2][TT][CH];                       // (delta, delta*u) per row and channel
    __shared__ float s_iv[ZOH ? 2 : 1][TT][CH];              // 1/delta per row and channel (ZOH)
    __shared__ float s_part[EMIT ? 2 : 1][kGroups][TT][CH];  // partial C.h per state group

    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int half = HALF ? (lane >> 5) : 0;
    const int ch = HALF ? (lane & 31) : lane;  // channel within the workgroup's block
    const int g = HALF ? 2 * w + half : w;     // state group: entries kNS*g .. kNS*g+kNS-1
    const int64_t D = a.dim, L = a.seqlen, BD = a.batch * a.dim;
    // The workgroup's channel block.  Workgroups are dealt to the 8 XCDs in turn
    // (linear id mod 8), each with its own L2.  Half-wave blocks 2p and 2p+1 share
    // the 128-byte lines of every bf16 row, so they are given ids 8 apart (the same
    // XCD): otherwise both XCDs fetch each line.  Needs the grid's x extent to be a
    // multiple of 16 (then linear id mod 8 = x mod 8); otherwise blocks stay in order.
    const int blk = [&] {
        const int x = int(blockIdx.x);
        if (!HALF || (gridDim.x & 15) != 0) return x;
        return (x & ~15) + 2 * (x & 7) + ((x >> 3) & 1);
    }();
    const int64_t d_raw = int64_t(blk) * CH + ch;
    const bool active = d_raw < D;
    const int64_t d = active ? d_raw : D - 1;  // idle lanes shadow the last channel
    const int64_t b = blockIdx.y;
    const int64_t c = blockIdx.z + (CORR == 2 ? 1 : 0);  // the correction pass skips chunk 0
    const int64_t t0 = c * a.chunk_len;
    const int len = int(((t0 + a.chunk_len < L) ? t0 + a.chunk_len : L) - t0);
    // an even number of tiles; rows past the chunk end are neutral (see publish_rows)
    const int ntiles = (((len + TT - 1) / TT) + 1) & ~1;
    const int64_t bd = b * D + d;
    const int64_t row0 = (b * L + t0) * D;  // first element of the chunk's first row

    const uint32_t row_bytes = uint32_t(D) * V::kBytes;
    const uint32_t span = uint32_t(len) * row_bytes;
    // vector offsets: the lane's channel, plus (half-wave) one row for the odd half.  The
    // row goes into the vector offset too in the half-wave layout, because the range
    // check covers the vector offset only: loads of rows past the chunk end then read 0
    // and stores to them are dropped, with no clamping or branch per row (offsets stay
    // below 2^32: the chunk span is below 2^31 and the prefetch runs at most 4 tiles
    // past it).  The whole-wave layout's rows are wave-uniform: a clamped scalar
    // offset, a mask and a scalar branch cost it no vector instruction.  Idle lanes
    // shadow the last channel throughout: they load its rows, compute its values bit
    // for bit and store the same y the lane that owns it stores; their state stores
    // are skipped.
    const uint32_t voff_lo = uint32_t(d) * V::kBytes;
    const uint32_t voff_hi = voff_lo + (half ? row_bytes : 0u);
    // half-wave: rows past the chunk end read a zero step size; only a bias or the
    // softplus can turn that into a non-zero one, so only then are they masked
    const bool mask_rows = (MODE & kOptSoftplus) != 0 || a.delta_bias != nullptr;
    const __amdgpu_buffer_rsrc_t r_u = make_rsrc(static_cast<const T*>(a.u) + row0, span);
    const __amdgpu_buffer_rsrc_t r_dl = make_rsrc(static_cast<const T*>(a.delta) + row0, span);
    const __amdgpu_buffer_rsrc_t r_z = make_rsrc(HAS_Z ? static_cast<const T*>(a.z) + row0 : nullptr, span);
    const __amdgpu_buffer_rsrc_t r_y = make_rsrc(EMIT ? static_cast<T*>(a.y) + row0 : nullptr, span);
    // the B and C planes of the chunk's panel
    const int64_t plane = a.panel_rows * kNS;
    const SS_CONST char* pB =
        (const SS_CONST char*)(a.ws_panel + ((b * a.n_chunks + c) * kGroups + g) * 2 * plane);
    const SS_CONST char* pC = pB + plane * 4;
    // half-wave: the chunk's panel block as a buffer; lane 16q + k reads word k of a
    // tile of its group's planes
    const __amdgpu_buffer_rsrc_t r_pan =
        make_rsrc(a.ws_panel + (b * a.n_chunks + c) * kGroups * 2 * plane, uint32_t(kGroups * 2 * plane * 4));
    const uint32_t voff_pan = uint32_t((g * 2 * plane + (lane & 15)) * 4);
    // RAW: no panel; the same values read from the (B, L, N) arrays themselves.  Lane
    // 16q + k reads row k/2, entry k%2 of its group; the tile goes into the vector
    // offset too, so rows past the chunk end read 0 (the range covers the chunk's rows)
    const uint32_t raw_span = RAW ? uint32_t(len * N) * V::kBytes : 0u;
    const __amdgpu_buffer_rsrc_t r_Braw =
        make_rsrc(RAW ? static_cast<const T*>(a.B) + (b * L + t0) * N : nullptr, raw_span);
    const __amdgpu_buffer_rsrc_t r_Craw =
        make_rsrc((RAW && EMIT) ? static_cast<const T*>(a.C) + (b * L + t0) * N : nullptr, raw_span);
    const uint32_t voff_raw = uint32_t((((lane & 15) >> 1) * N + g * kNS + (lane & 1)) * V::kBytes);

    const int64_t sbase = bd * N + g * kNS;  // this lane's entries in a (B, D, N) state array
    float A2[kNS], iA[kNS];  // A * log2 e, and 1/A for the zero-order hold
#pragma unroll
    for (int i = 0; i < kNS; ++i) {
        const float av = a.A[d * N + g * kNS + i];
        A2[i] = av * kLog2e;
        iA[i] = ZOH ? 1.0f / av : 0.0f;
    }
    const float bias = a.delta_bias ? a.delta_bias[d] : 0.0f;

    float h[kNS];
    // whole sequence, or the emit after an aggregate pass: from h0 or the carry;
    // emit first (pass 1): chunk 0 from h0, the others from zero; correction
    // (pass 2): from the carry
    const bool first = CORR == 1;
    const bool from_ws = EMIT && a.n_chunks > 1 && !first;
    const bool from_h0 = (EMIT || CKPT) && a.h0 != nullptr && (a.n_chunks == 1 || (first && c == 0));
    const bool fused = CORR == 0 && from_ws && a.fuse_carry != 0;
    // fused carry: run() forms h with this once the first tiles' loads are in flight
    auto fuse_carry_init = [&]() {
        // the carry into chunk c: the initial state through the affine maps of chunks
        // 0..c-1, (P_j, S_j) with P_j = exp(A * sum of delta over chunk j) and S_j the
        // chunk's end state from zero, applied earlier chunk first.  The loads are
        // independent, so all are issued before the first combine.
        float sv[kFuseMaxChunks - 1][kNS], dj[kFuseMaxChunks - 1];
#pragma unroll
        for (int j = 0; j < kFuseMaxChunks - 1; ++j) {
            if (j < c) {
                const float* src = a.ws_agg + int64_t(j) * BD * N + sbase;
#pragma unroll
                for (int i = 0; i < kNS; ++i) sv[j][i] = src[i];
                dj[j] = a.ws_dsum[int64_t(j) * BD + bd];
            }
        }
#pragma unroll
        for (int i = 0; i < kNS; ++i) h[i] = a.h0 ? a.h0[sbase + i] : 0.0f;
#pragma unroll
        for (int j = 0; j < kFuseMaxChunks - 1; ++j) {
            if (j < c) {
#pragma unroll
                for (int i = 0; i < kNS; ++i) h[i] = fmaf(exp2_hw(A2[i] * dj[j]), h[i], sv[j][i]);
            }
        }
        if (active) {
            // the carry, kept in the chunk's slot as the carry pass would
            float* dst = a.ws_state + c * BD * N + sbase;
#pragma unroll
            for (int i = 0; i < kNS; ++i) dst[i] = h[i];
        }
    };
    if (fused) {
#pragma unroll
        for (int i = 0; i < kNS; ++i) h[i] = 0.0f;  // set by fuse_carry_init before the first tile
    } else if (from_ws || from_h0) {
        const float* init = from_ws ? a.ws_state + c * BD * N + sbase : a.h0 + sbase;
#pragma unroll
        for (int i = 0; i < kNS; ++i) h[i] = init[i];
    } else {
#pragma unroll
        for (int i = 0; i < kNS; ++i) h[i] = 0.0f;
    }
    const float dskip = (EMIT && HAS_D) ? a.Dskip[d] : 0.0f;
    float dsum = 0.0f;
    float dmin = __builtin_inff();  // emit first: the smallest step size of the chunk

    Raw rdl[2][RPW], ru[2][RPW], rz[2][RPW];  // raw rows in flight, by tile parity
    float xf[2][RPW], zf[2][RPW];             // widened u, z kept for the epilogue
    Words16 bw[2][HALF ? 1 : PW], cw[2][HALF ? 1 : PW];  // whole-wave: the tile's panel words
    float bv[2], cv[2];                                  // half-wave: the tile's B, C values

    // first row (within the chunk) a lane's wave widens in a tile: its rows are that
    // row + j (whole-wave) or that row + its half (half-wave)
    auto wave_row = [&](int tile) { return tile * TT + (HALF ? 2 * w : w * RPW); };
    // the row a lane widens and finishes
    auto lane_row = [&](int tile, int j) { return wave_row(tile) + (HALF ? half : j); };
    // a lane's vector offset of row r of the chunk (see voff_lo)
    // (the row is wave-uniform: readfirstlane keeps its offset in a scalar register)
    auto row_voff = [&](uint32_t base, int r) {
        return base + __builtin_amdgcn_readfirstlane(uint32_t(r) * row_bytes);
    };

    auto issue_rows = [&](int tile, auto slot) {
        constexpr int S = decltype(slot)::value;
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
            if constexpr (HALF) {
                // voff_hi carries the odd half's row; past the chunk end the loads read 0
                const uint32_t vo = row_voff(voff_hi, wave_row(tile));
                rdl[S][j] = V::load(r_dl, vo, 0);
                ru[S][j] = V::load(r_u, vo, 0);
                if (EMIT && HAS_Z) rz[S][j] = V::load(r_z, vo, 0);
            } else {
                // whole-wave: the row is uniform, so it stays a clamped scalar offset
                // (no vector instruction) and publish_rows masks rows past the end
                const int r = lane_row(tile, j);
                const uint32_t so = uint32_t(r < len ? r : len - 1) * row_bytes;
                rdl[S][j] = V::load(r_dl, voff_lo, so);
                ru[S][j] = V::load(r_u, voff_lo, so);
                if (EMIT && HAS_Z) rz[S][j] = V::load(r_z, voff_lo, so);
            }
        }
    };
    // widen this lane's rows of a tile and publish (delta, delta*u).  Rows past
    // the chunk end are published as (0, 0): exp2(0) = 1 and 0*B = 0 leave the
    // state bit-unchanged, so the last tiles need no row-count branches.
    auto publish_rows = [&](int tile, auto slot) {
        constexpr int S = decltype(slot)::value;
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
            const int r = lane_row(tile, j) - tile * TT;
            float dl = V::widen(rdl[S][j]);
            if (!HALF || mask_rows) {
                // a uniform branch: the empty asm keeps the compiler from computing this
                // path everywhere and selecting
                __asm__ volatile("" ::: "memory");
                dl = lane_row(tile, j) < len ? step_size<MODE>(dl, bias) : 0.0f;
            }
            const float x = V::widen(ru[S][j]);
            s_xd[S][r][ch] = make_float2(dl, dl * x);
            if constexpr (ZOH) s_iv[S][r][ch] = __builtin_amdgcn_rcpf(dl);
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
    // a tile's panel rows are contiguous: whole-wave, 16-word scalar loads at a
    // 32-bit byte offset from the plane's 64-bit base; half-wave, one word per
    // lane.  No clamping: the panel holds zero rows past the chunk end and one
    // spare tile.
    auto issue_words = [&](int tile, auto slot) {
        constexpr int S = decltype(slot)::value;
        const uint32_t off = uint32_t(tile) * uint32_t(TT * kNS * 4);
        if constexpr (RAW) {
            const uint32_t vo = voff_raw + __builtin_amdgcn_readfirstlane(uint32_t(tile) * uint32_t(TT * N * V::kBytes));
            bv[S] = V::widen(V::load(r_Braw, vo, 0));
            if (EMIT) cv[S] = V::widen(V::load(r_Craw, vo, 0));
        } else if constexpr (HALF) {
            bv[S] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_pan, voff_pan, off, 0));
            if (EMIT)
                cv[S] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_pan, voff_pan + uint32_t(plane * 4),
                                                                             off, 0));
        } else {
            const SS_CONST Words16* qb = (const SS_CONST Words16*)(pB + off);
            const SS_CONST Words16* qc = (const SS_CONST Words16*)(pC + off);
#pragma unroll
            for (int q = 0; q < PW; ++q) {
                bw[S][q] = qb[q];
                if (EMIT) cw[S][q] = qc[q];
            }
        }
    };
    // entry i of row r of a tile, from its panel words (whole-wave)
    auto word = [&](const Words16 (&wv)[HALF ? 1 : PW], int r, int i) {
        const int k = r * kNS + i;
        return __uint_as_float(wv[k / 16][k % 16]);
    };
    // finish this lane's rows of a tile: sum the partials, skip, gate, store
    auto finish_rows = [&](int tile, auto slot) {
        constexpr int S = decltype(slot)::value;
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
            const int t = lane_row(tile, j);
            const int r = t - tile * TT;
            // half-wave: the range check drops stores past the chunk end; whole-wave:
            // the row is uniform, a scalar branch
            if (HALF || t < len) {
                float acc = s_part[S][0][r][ch];
#pragma unroll
                for (int q = 1; q < kGroups; ++q) acc += s_part[S][q][r][ch];
                if (HAS_D) acc = fmaf(dskip, xf[S][j], acc);
                if (HAS_Z) acc *= silu(zf[S][j]);
                if constexpr (HALF)
                    V::store(r_y, row_voff(voff_hi, wave_row(tile)), 0, acc);
                else
                    V::store(r_y, voff_lo, uint32_t(t) * row_bytes, acc);
            }
        }
    };
    // the recurrence over one tile for this lane's state entries
    auto scan_rows = [&](int tile, auto slot) {
        constexpr int S = decltype(slot)::value;
        float2 xd[TT];
#pragma unroll
        for (int r = 0; r < TT; ++r) xd[r] = s_xd[S][r][ch];
        // whole-wave: the next tile's scalar loads go out only after all of this
        // tile's LDS reads have landed (LDS and scalar loads share one counter, and
        // scalar loads return out of order: a later LDS wait would drain them too)
        static_assert(TT == 8, "the wait below names eight rows");
        float iv[TT];  // 1/delta per row (zero-order hold only)
#pragma unroll
        for (int r = 0; r < TT; ++r) iv[r] = ZOH ? s_iv[ZOH ? S : 0][r][ch] : 0.0f;
        __asm__ volatile("" ::"v"(xd[0].x), "v"(xd[0].y), "v"(xd[1].x), "v"(xd[1].y), "v"(xd[2].x), "v"(xd[2].y),
                         "v"(xd[3].x), "v"(xd[3].y), "v"(xd[4].x), "v"(xd[4].y), "v"(xd[5].x), "v"(xd[5].y),
                         "v"(xd[6].x), "v"(xd[6].y), "v"(xd[7].x), "v"(xd[7].y)
                         : "memory");
        if constexpr (ZOH)
            __asm__ volatile("" ::"v"(iv[0]), "v"(iv[1]), "v"(iv[2]), "v"(iv[3]), "v"(iv[4]), "v"(iv[5]), "v"(iv[6]),
                             "v"(iv[7])
                             : "memory");
        issue_words(tile + 1, Slot<1 - S>{});
        // rows past the chunk end are published with delta = 0: no effect on the sum or
        // the minimum
        if constexpr (CORR == 2) {
            // the correction: every lane checks the decay with the sum over its rows
#pragma unroll
            for (int r = 0; r < TT; ++r) dsum += xd[r].x;
        } else if constexpr (CORR == 1) {
            // pass 1: only wave 0's sum and minimum are used (it stores the delta sums of
            // the workgroup's channels, and its vote on a negative step size covers all of
            // them), so the other waves skip them (long context 958 -> 920 us; the same in
            // the aggregate pass of the short chunks made it slower, 43.7 -> 45.9 us: wave
            // 0 then lags at every barrier).  A uniform branch: the empty asm keeps the
            // compiler from computing this everywhere and selecting
            if (w == 0) {
                __asm__ volatile("" ::: "memory");
#pragma unroll
                for (int r = 0; r < TT; ++r) {
                    dsum += xd[r].x;
                    dmin = fminf(dmin, xd[r].x);
                }
            }
        }
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
        if constexpr (HALF) {
            float hh[TT][kNS];  // the state after each row, for the C contraction
            static_for<TT>([&](auto rc) {
                constexpr int r = decltype(rc)::value;
                const float xb = xd[r].y;
                static_for<kNS>([&](auto ic) {
                    constexpr int i = decltype(ic)::value;
                    float in_term = xb * row_bcast<r * kNS + i>(bv[S]);  // delta*B*u (Euler)
                    // Without the emit path the compiler would otherwise form half of the
                    // broadcasts above the barrier, apart from their multiplies, as moves
                    // of their own (32 more vector instructions per tile pair); held
                    // here, each folds into its multiply
                    if constexpr (!EMIT) __asm__ volatile("" : "+v"(in_term));
                    if constexpr (ZOH) in_term *= zoh_phi(x2[r][i], e[r][i], iA[i] * iv[r]);
                    h[i] = fmaf(e[r][i], h[i], in_term);
                    hh[r][i] = h[i];
                });
                if constexpr (!EMIT && !CKPT) dsum += xd[r].x;
            });
            if constexpr (EMIT) {
                float acc[TT];
                contract_rows_bcast(acc, cv[S], hh);
#pragma unroll
                for (int r = 0; r < TT; ++r) s_part[S][g][r][ch] = acc[r];
            }
        } else {
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
                    s_part[S][g][r][ch] = acc;
                } else if constexpr (!CKPT) {
                    dsum += xd[r].x;
                }
            }
        }
    };

    // one tile step: finish tile k-1, publish tile k+1, scan tile k
    // every load below is of a valid row (whole-wave: clamped) or range-checked (half-wave:
    // rows past the chunk end read 0), so all of it runs unconditionally
    // k0: the first tile of the current run (the tile before it is finished already)
    auto step = [&](int k, int k0, auto slot) {
        constexpr int S = decltype(slot)::value;
        if constexpr (EMIT) {
            if (k > k0) finish_rows(k - 1, Slot<1 - S>{});
        }
        publish_rows(k + 1, Slot<1 - S>{});
        issue_rows(k + 3, Slot<1 - S>{});
        scan_rows(k, Slot<S>{});
        __syncthreads();
    };

    // Two or three workgroups share a CU, and the wave arbiter favours older
    // waves: left alone, the first workgroup finishes far ahead of the last and
    // the CU ends its run with a single latency-bound workgroup.  Lowering a
    // wave's priority at each quarter of the chunk lets the laggards catch up,
    // so the workgroups of a CU stay within a quarter of each other.
    static_assert(2 * kTileRows == kBwdSub, "checkpoints fall at the start of every tile pair");
    constexpr float kCorrTol = 5.9604645e-8f;  // 2^-24
    // checkpoints (a separate instantiation: the plain kernel has no scalar
    // registers to spare): this lane's entries of the one at row t0 + k*TT,
    // advanced by one checkpoint per tile pair.  Stored nontemporal: nothing
    // reads them before the backward, and the large layer's 335 MB would only
    // push the rows in flight out of the caches (checkpointing forward 0.347 ->
    // 0.334 ms)
    float* ck_row = nullptr;
    int64_t ck_step = 0;
    if constexpr (CKPT) {
        ck_row = a.ckpt + ((t0 / kBwdSub * a.batch + b) * N + g * kNS) * D + d;
        ck_step = a.batch * N * D;
    }
    // tiles [k0, k1) (both even) of the chunk, with the prefetch pipeline primed at
    // k0.  stop(n) is asked after every tile pair (n tiles run so far) and ends the
    // run early when it returns true; it must return the same for every wave.
    // Returns the tile the run ended before.
    auto run = [&](int k0, int k1, auto stop) {
        issue_rows(k0, Slot<0>{});
        issue_rows(k0 + 1, Slot<1>{});
        // its loads go out after the first two tiles', so their latencies overlap
        if (fused && k0 == 0) fuse_carry_init();
        publish_rows(k0, Slot<0>{});
        issue_rows(k0 + 2, Slot<0>{});
        issue_words(k0, Slot<0>{});
        __syncthreads();
        const int quarter = ((k1 - k0) / 4) & ~1;
        __builtin_amdgcn_s_setprio(3);
        int k = k0;
        while (k < k1) {
            if (quarter > 0) {
                if (k - k0 == quarter) __builtin_amdgcn_s_setprio(2);
                else if (k - k0 == 2 * quarter) __builtin_amdgcn_s_setprio(1);
                else if (k - k0 == 3 * quarter) __builtin_amdgcn_s_setprio(0);
            }
            if constexpr (CKPT) {
                // the state entering row t0 + k*TT, a multiple of kBwdSub (k is even)
                if (active && k * TT < len) {
#pragma unroll
                    for (int i = 0; i < kNS; ++i) __builtin_nontemporal_store(h[i], &ck_row[int64_t(i) * D]);
                }
                ck_row += ck_step;
            }
            step(k, k0, Slot<0>{});
            step(k + 1, k0, Slot<1>{});
            k += 2;
            if (stop(k - k0)) break;
        }
        // the rows, loads and publication of tiles past k are left unused
        if constexpr (EMIT) finish_rows(k - 1, Slot<1>{});
        return k;
    };
    const auto never = [](int) { return false; };
    // emit first: whether p holds for any lane of the workgroup.  Every wave calls
    // it at the same point, right after a tile pair, where the even tiles' partial
    // sums are finished and not yet rewritten: each wave leaves its ballot in a
    // word of that buffer, a barrier, every wave reads them all, and a second
    // barrier before the buffer is written again.  (__syncthreads_or would add
    // LDS of its own: a quarter of the CU's LDS is exactly what the whole-wave
    // kernel uses, so four workgroups per CU would no longer fit.)
    auto wg_any = [&](bool p) {
        const bool any = __builtin_amdgcn_ballot_w64(p) != 0;
        if (lane == 0) s_part[0][0][0][w] = any ? 1.0f : 0.0f;
        __syncthreads();
        bool r = false;
#pragma unroll
        for (int q = 0; q < ScanShape<HALF>::kWaves; ++q) r = r || s_part[0][0][0][q] != 0.0f;
        __syncthreads();
        return r;
    };

    if constexpr (CORR == 2) {
        // Correction of chunk c >= 1 after the emit-first pass, which ran it from
        // a zero state: rerun from the carry H.  After rows [0, r) the state
        // differs from the zero-start one by P * H, P = exp(A * sum of delta over
        // those rows); where the chunk's step sizes are all >= 0 and A <= 0 that
        // difference only decays, so the first pass's later rows are right to
        // fp32 resolution once P*|H| <= 2^-24 of the lane's largest |state|.
        // That is checked after corr_head_tiles tiles and then every
        // kCorrEveryTiles; the rerun stops at the first check every lane of the
        // workgroup passes, else runs to the chunk's end.
        float H[kNS];
#pragma unroll
        for (int i = 0; i < kNS; ++i) H[i] = h[i];
        const int64_t n32 = (D + 31) / 32;
        const int64_t fl = (c * a.batch + b) * n32 + int64_t(blk) * (CH / 32);
        // a negative step size anywhere in the chunk (first pass): no early stop
        const bool can_stop = a.ws_neg[fl] == 0u;
        const int first = a.corr_head_tiles;
        auto decayed = [&](int n) {
            if (!can_stop || n < first || (n - first) % kCorrEveryTiles != 0) return false;
            float smax = 0.0f;
#pragma unroll
            for (int i = 0; i < kNS; ++i) smax = fmaxf(smax, fabsf(h[i]));
            bool ok = true;
#pragma unroll
            for (int i = 0; i < kNS; ++i)
                ok = ok && A2[i] <= 0.0f && exp2_hw(A2[i] * dsum) * fabsf(H[i]) <= kCorrTol * smax;
            ok = ok || !active;  // idle lanes have no say
            return !wg_any(!ok);
        };
        const bool whole = run(0, ntiles, decayed) >= ntiles;
        if (threadIdx.x == 0) {
            // one flag per 32-channel block (a whole-wave workgroup holds two)
            uint32_t* f = a.ws_whole + ((c - 1) * a.batch + b) * n32 + int64_t(blk) * (CH / 32);
            f[0] = whole ? 1u : 0u;
            if (CH == 64 && int64_t(blk) * 2 + 1 < n32) f[1] = whole ? 1u : 0u;
        }
        if (!active || c != a.n_chunks - 1 || !a.h_last) return;
        if (whole) {
#pragma unroll
            for (int i = 0; i < kNS; ++i) a.h_last[sbase + i] = h[i];
        } else {
            // the first pass's end state from zero, plus the carry decayed over
            // the whole chunk
            const float dtot = a.ws_dsum[c * BD + bd];
#pragma unroll
            for (int i = 0; i < kNS; ++i)
                a.h_last[sbase + i] = fmaf(exp2_hw(A2[i] * dtot), H[i], a.h_last[sbase + i]);
        }
    } else {
        run(0, ntiles, never);
        if constexpr (CORR == 1) {
            // emit first: whether any step size of the chunk is negative, per workgroup
            const bool neg = wg_any(dmin < 0.0f);
            if (threadIdx.x == 0) {
                const int64_t n32 = (D + 31) / 32;
                uint32_t* f = a.ws_neg + (c * a.batch + b) * n32 + int64_t(blk) * (CH / 32);
                f[0] = neg ? 1u : 0u;
                if (CH == 64 && int64_t(blk) * 2 + 1 < n32) f[1] = neg ? 1u : 0u;
            }
        }

        if (!active) return;
        if constexpr (EMIT) {
            if (c == a.n_chunks - 1 && a.h_last) {
#pragma unroll
                for (int i = 0; i < kNS; ++i) a.h_last[sbase + i] = h[i];
            }
            if constexpr (CORR == 1) {
                // emit first: the end state from the chunk's own start (h0 for chunk 0,
                // zero for the others) and the chunk's delta sum, for the carry pass
                if (c < a.n_chunks - 1) {
                    float* dst = a.ws_agg + c * BD * N + sbase;
#pragma unroll
                    for (int i = 0; i < kNS; ++i) dst[i] = h[i];
                }
                if (g == 0) a.ws_dsum[c * BD + bd] = dsum;
            }
        } else if constexpr (!CKPT) {
            float* dst = a.ws_agg + c * BD * N + sbase;
#pragma unroll
            for (int i = 0; i < kNS; ++i) dst[i] = h[i];
            if (g == 0) a.ws_dsum[c * BD + bd] = dsum;
        }
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

// R lanes per state entry: the power of two covering the K-1 aggregated chunks, 4..64
void launch_carry_for(const ScanArgs& a, hipStream_t s)
{
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

// ---------------------------------------------------------------------------
typedef float F32x4 __attribute__((ext_vector_type(4)));
// Recurrent step.  Q lanes per channel (b, d), each with S = 16/Q of the 16
// state entries: S/4 16-byte loads and stores of h and of A, and (VEC, when
// the host has checked B and C for 16-byte alignment) B and C as 16-byte
// loads too; the partial C.h of the Q lanes summed with log2(Q) butterfly
// exchanges.  grid = (ceil(dim*Q / 256), ceil(batch rows of the launch / CPL)),
// block = 256: each lane steps CPL batch rows of one channel, so A is read
// once for them, and its channel is found with a shift, never a 64-bit
// division.
// The state is loaded and stored nontemporally.  In a model a layer's state
// comes back after every other layer has run, out of every cache; timed that
// way (the 256 MB last-level cache flushed before each token) at B=256 D=5120
// the step took 38.5 us against 42.8 us with ordinary accesses, and 32.5
// against 27.6 us when the same state is stepped again at once.
// ---------------------------------------------------------------------------
template <int DT, int S, bool VEC>
__device__ __forceinline__ void load_row(const typename Elem<DT>::T* p, float (&out)[S])
{
    if constexpr (VEC && DT == 1 && S == 4) {
        // bf16: 4 values per 8 bytes
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        out[0] = __uint_as_float(v.x << 16);
        out[1] = __uint_as_float(v.x & 0xffff0000u);
        out[2] = __uint_as_float(v.y << 16);
        out[3] = __uint_as_float(v.y & 0xffff0000u);
    } else if constexpr (VEC && DT == 1 && S >= 8) {
        // bf16: 8 values per 16 bytes
#pragma unroll
        for (int k = 0; k < S / 8; ++k) {
            const uint4 v = reinterpret_cast<const uint4*>(p)[k];
            const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                out[8 * k + 2 * j] = __uint_as_float(wv[j] << 16);
                out[8 * k + 2 * j + 1] = __uint_as_float(wv[j] & 0xffff0000u);
            }
        }
    } else if constexpr (VEC && DT == 0) {
#pragma unroll
        for (int k = 0; k < S / 4; ++k) {
            const float4 v = reinterpret_cast<const float4*>(p)[k];
            out[4 * k] = v.x;
            out[4 * k + 1] = v.y;
            out[4 * k + 2] = v.z;
            out[4 * k + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < S; ++i) out[i] = Elem<DT>::load(p, i);
    }
}

template <int DT, bool HAS_D, bool HAS_Z, int MODE, int Q, bool VEC, int CPL>
__global__ __launch_bounds__(256) void step_kernel(StepArgs a)
{
    constexpr int S = N / Q;  // state entries per lane
    static_assert(Q == 1 || Q == 2 || Q == 4, "1, 2 or 4 lanes per channel");
    using E = Elem<DT>;
    using T = typename E::T;
    const T* __restrict__ u = static_cast<const T*>(a.u);
    const T* __restrict__ delta = static_cast<const T*>(a.delta);
    const T* __restrict__ Bm = static_cast<const T*>(a.B);
    const T* __restrict__ Cm = static_cast<const T*>(a.C);
    const T* __restrict__ z = static_cast<const T*>(a.z);
    T* __restrict__ y = static_cast<T*>(a.y);

    // One channel per lane (Q lanes per channel), CPL batch rows ceil(rows/CPL) apart
    // (grid row r: rows b0 + r + j * ceil(rows/CPL)): A is read once for all of them,
    // every load is issued before the first is used, and the channel comes from a
    // shift, never a 64-bit division.
    const int64_t rows = (a.rows + CPL - 1) / CPL;  // grid rows between a lane's rows
    const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    // the lane's state entries (q) and channel; a channel's lanes are idle together, and
    // idle lanes read the last channel's entries q
    const int q = int(gid & (Q - 1));
    const bool in_dim = gid / Q < a.dim;
    const int64_t d = in_dim ? gid / Q : a.dim - 1;
    bool active[CPL];
    int64_t bd[CPL], b[CPL];
    float hs[CPL][S], as[S], bs[CPL][S], cs[CPL][S], dl[CPL], x[CPL], zv[CPL];
#pragma unroll
    for (int k = 0; k < S / 4; ++k) {
        const float4 av = reinterpret_cast<const float4*>(a.A + d * N + q * S)[k];
        as[4 * k] = av.x;
        as[4 * k + 1] = av.y;
        as[4 * k + 2] = av.z;
        as[4 * k + 3] = av.w;
    }
    const float bias = a.delta_bias ? a.delta_bias[d] : 0.0f;
    const float dsk = HAS_D ? a.Dskip[d] : 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int64_t rj = int64_t(blockIdx.y) + j * rows;
        active[j] = in_dim && rj < a.rows;
        b[j] = a.b0 + (rj < a.rows ? rj : a.rows - 1);
        bd[j] = b[j] * a.dim + d;
#pragma unroll
        for (int k = 0; k < S / 4; ++k) {
            const F32x4 hv = __builtin_nontemporal_load(reinterpret_cast<const F32x4*>(a.h + bd[j] * N + q * S) + k);
            hs[j][4 * k] = hv.x;
            hs[j][4 * k + 1] = hv.y;
            hs[j][4 * k + 2] = hv.z;
            hs[j][4 * k + 3] = hv.w;
        }
        load_row<DT, S, VEC>(Bm + b[j] * N + q * S, bs[j]);
        load_row<DT, S, VEC>(Cm + b[j] * N + q * S, cs[j]);
        dl[j] = step_size<MODE>(E::load(delta, bd[j]), bias);
        x[j] = E::load(u, bd[j]);
        zv[j] = HAS_Z ? E::load(z, bd[j]) : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const float xb = dl[j] * x[j];
        const float inv_dl = (MODE & kOptZoh) ? __builtin_amdgcn_rcpf(dl[j]) : 0.0f;
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < S; ++i) {
            const float x2 = dl[j] * (as[i] * kLog2e);
            const float abar = exp2_hw(x2);
            float in_term = xb * bs[j][i];
            if constexpr ((MODE & kOptZoh) != 0) in_term *= zoh_phi(x2, abar, (1.0f / as[i]) * inv_dl);
            hs[j][i] = fmaf(abar, hs[j][i], in_term);
            part = fmaf(cs[j][i], hs[j][i], part);
        }
        float acc = part;
        if constexpr (Q >= 2) acc += __shfl_xor(acc, 1, Q);
        if constexpr (Q >= 4) acc += __shfl_xor(acc, 2, Q);
        if (active[j]) {
#pragma unroll
            for (int k = 0; k < S / 4; ++k) {
                const F32x4 hv = {hs[j][4 * k], hs[j][4 * k + 1], hs[j][4 * k + 2], hs[j][4 * k + 3]};
                __builtin_nontemporal_store(hv, reinterpret_cast<F32x4*>(a.h + bd[j] * N + q * S) + k);
            }
            if (q == 0) {
                if (HAS_D) acc = fmaf(dsk, x[j], acc);
                if (HAS_Z) acc *= silu(zv[j]);
                E::store(y, bd[j], acc);
            }
        }
    }
}

template <int DT, bool HAS_D, bool HAS_Z, int MODE, bool HALF>
hipError_t launch_scan_layout(const ScanArgs& a, hipStream_t s)
{
    constexpr int CH = ScanShape<HALF>::kCh;
    const dim3 block(ScanShape<HALF>::kWaves * kWave);
    const unsigned nblk = unsigned((a.dim + CH - 1) / CH);
    if constexpr (HALF) {
        if (a.raw_bc) {
            // the short-chunk scheme's passes read B and C as they are: no panel pass
            scan_kernel<DT, false, false, false, MODE, false, true, 0, true>
                <<<dim3(nblk, unsigned(a.batch), unsigned(a.n_chunks - 1)), block, 0, s>>>(a);
            if (!a.fuse_carry) launch_carry_for(a, s);
            scan_kernel<DT, true, HAS_D, HAS_Z, MODE, false, true, 0, true>
                <<<dim3(nblk, unsigned(a.batch), unsigned(a.n_chunks)), block, 0, s>>>(a);
            return hipGetLastError();
        }
    }
    launch_panel_t<DT>(a, s);
    if (a.n_chunks > 1 && a.corr_head_tiles > 0 && !a.ckpt) {
        // emit first: every chunk from its own start (h0 or zero), writing y and its
        // end state; the carries; then chunks 1..K-1 corrected from their carries
        scan_kernel<DT, true, HAS_D, HAS_Z, MODE, false, HALF, 1>
            <<<dim3(nblk, unsigned(a.batch), unsigned(a.n_chunks)), block, 0, s>>>(a);
        ScanArgs cc = a;
        cc.h0 = nullptr;  // chunk 0's end state already starts from h0
        launch_carry_for(cc, s);
        scan_kernel<DT, true, HAS_D, HAS_Z, MODE, false, HALF, 2>
            <<<dim3(nblk, unsigned(a.batch), unsigned(a.n_chunks - 1)), block, 0, s>>>(a);
        return hipGetLastError();
    }
    if (a.n_chunks > 1) {
        scan_kernel<DT, false, false, false, MODE, false, HALF>
            <<<dim3(nblk, unsigned(a.batch), unsigned(a.n_chunks - 1)), block, 0, s>>>(a);
        if (!a.fuse_carry) launch_carry_for(a, s);
    }
    const dim3 grid(nblk, unsigned(a.batch), unsigned(a.n_chunks));
    if (a.ckpt)
        scan_kernel<DT, true, HAS_D, HAS_Z, MODE, true, HALF><<<grid, block, 0, s>>>(a);
    else
        scan_kernel<DT, true, HAS_D, HAS_Z, MODE, false, HALF><<<grid, block, 0, s>>>(a);
    return hipGetLastError();
}

template <int DT, bool HAS_D, bool HAS_Z, int MODE>
hipError_t launch_scan_t(const ScanArgs& a, hipStream_t s)
{
    return a.half ? launch_scan_layout<DT, HAS_D, HAS_Z, MODE, true>(a, s)
                  : launch_scan_layout<DT, HAS_D, HAS_Z, MODE, false>(a, s);
}

#ifndef SS_STEP_LANES
#define SS_STEP_LANES 4
#endif
#ifndef SS_STEP_CPL
#define SS_STEP_CPL 2
#endif
template <int DT, bool HAS_D, bool HAS_Z, int MODE>
hipError_t launch_step_t(const StepArgs& a, hipStream_t s)
{
    constexpr int Q = SS_STEP_LANES, CPL = SS_STEP_CPL;
    const unsigned blocks = unsigned((a.dim * Q + 255) / 256);
    // batch rows per launch: a grid row covers CPL of them
    constexpr int64_t kMaxRows = 65535 * int64_t(CPL);
    for (int64_t b0 = 0; b0 < a.batch; b0 += kMaxRows) {
        StepArgs p = a;
        p.b0 = b0;
        p.rows = a.batch - b0 < kMaxRows ? a.batch - b0 : kMaxRows;
        const dim3 grid(blocks, unsigned((p.rows + CPL - 1) / CPL));
        if (a.vec_bc)
            step_kernel<DT, HAS_D, HAS_Z, MODE, Q, true, CPL><<<grid, dim3(256), 0, s>>>(p);
        else
            step_kernel<DT, HAS_D, HAS_Z, MODE, Q, false, CPL><<<grid, dim3(256), 0, s>>>(p);
    }
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

// The backward's checkpoint pass: the recurrence once over the whole sequence (one
// chunk), from h0, keeping only the state entering every kBwdSub-th row in a.ckpt.
// The half-wave scan kernel without its contraction and epilogue: the same states,
// bit for bit, as the checkpoints a one-chunk ss_scan_fwd_ckpt writes.
template <int DT, int MODE>
hipError_t launch_ckpt_pass_t(const ScanArgs& a, hipStream_t s)
{
    constexpr int CH = ScanShape<true>::kCh;
    const dim3 grid(unsigned((a.dim + CH - 1) / CH), unsigned(a.batch), 1u);
    scan_kernel<DT, false, false, false, MODE, true, true><<<grid, dim3(scan_threads<true>()), 0, s>>>(a);
    return hipGetLastError();
}

template <int DT>
hipError_t dispatch_ckpt_pass(const ScanArgs& a, hipStream_t s)
{
    switch (a.options & kOptAll) {
        case 0: return launch_ckpt_pass_t<DT, 0>(a, s);
        case kOptSoftplus: return launch_ckpt_pass_t<DT, kOptSoftplus>(a, s);
        case kOptZoh: return launch_ckpt_pass_t<DT, kOptZoh>(a, s);
        default: return launch_ckpt_pass_t<DT, kOptSoftplus | kOptZoh>(a, s);
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
    if (dtype == 0)
        launch_panel_t<0>(a, stream);
    else
        launch_panel_t<1>(a, stream);
    return hipGetLastError();
}

hipError_t launch_ckpt_pass(const ScanArgs& a, int dtype, hipStream_t stream)
{
    (void)hipGetLastError();
    return dtype == 0 ? dispatch_ckpt_pass<0>(a, stream) : dispatch_ckpt_pass<1>(a, stream);
}

hipError_t launch_step(const StepArgs& a, int dtype, hipStream_t stream)
{
    (void)hipGetLastError();
    return dtype == 0 ? dispatch_step<0>(a, stream) : dispatch_step<1>(a, stream);
}

}  // namespace ssk
