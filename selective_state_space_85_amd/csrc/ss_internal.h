// Internal interface between the C-ABI layer (ss_api.cpp) and the gfx950
// kernels (ss_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace ssk {

constexpr int kDState = 16;  // the state width the kernels are built for

// Option bits of a scan or step call (the same values as the C ABI's).
constexpr uint32_t kOptSoftplus = 1u;  // step size = softplus(delta + bias[d])
constexpr uint32_t kOptZoh = 2u;       // zero-order-hold input term
constexpr uint32_t kOptAll = kOptSoftplus | kOptZoh;

// Waves per scan workgroup; the 16 state entries are split evenly across them.
#ifndef SS_SCAN_WAVES
#define SS_SCAN_WAVES 8
#endif
constexpr int kScanWaves = SS_SCAN_WAVES;
static_assert(kScanWaves == 2 || kScanWaves == 4 || kScanWaves == 8, "state split must divide 16");
constexpr int kGroupStates = kDState / kScanWaves;  // state entries per wave

// Rows of the sequence per scan tile (one LDS barrier per tile).
#ifndef SS_TILE_ROWS
#define SS_TILE_ROWS 8
#endif
constexpr int kTileRows = SS_TILE_ROWS;
static_assert(kTileRows % kScanWaves == 0, "tile rows must split evenly across the waves");
static_assert((kTileRows * kGroupStates) % 16 == 0, "a wave's tile of B (or C) is loaded 16 words at a time");

// Rows of one chunk in the fp32 B/C panel: the chunk's tiles rounded up to an
// even count (the scan loop runs tiles in pairs) plus one tile that the last
// tile's prefetch reads.  Rows past the chunk end hold zeros.
inline int64_t panel_rows(int64_t chunk_rows)
{
    int64_t tiles = (chunk_rows + kTileRows - 1) / kTileRows;
    tiles = (tiles + 1) & ~int64_t(1);
    return (tiles + 1) * kTileRows;
}

struct ScanArgs {
    const void* u;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* Dskip;  // nullable
    const void* z;       // nullable
    const float* h0;     // nullable
    const float* delta_bias;  // (dim,), nullable
    uint32_t options;         // kOpt* bits
    void* y;
    float* h_last;       // nullable
    float* ws_state;     // (K, batch, dim, N) state slots, nullable when K == 1
    float* ws_dsum;      // (K, batch, dim) per-chunk delta sums
    // end states of chunks 0..K-2 from a zero start, (K-1, batch, dim, N):
    // the aggregate pass and the emit-first pass write them here; when the
    // carry is fused (fuse_carry) a region of its own, else slots 1..K-1
    float* ws_agg;
    // short-chunk plans with few chunks: the emit pass forms each chunk's carry
    // from the initial state and the end states and delta sums of the chunks
    // before it, and writes it to the chunk's slot; no carry pass
    int fuse_carry;
    // (K-1, batch, ceil(dim/32)), emit first: 1 where the correction pass reran
    // the whole chunk c+1, 0 where only its head
    uint32_t* ws_whole;
    // (batch, K, waves, {B, C}, panel_rows, kGroupStates) fp32 copy of B and C,
    // regrouped so that a wave's entries of consecutive rows are contiguous
    float* ws_panel;
    int64_t panel_rows;
    // (ceil(seqlen / kBwdSub), batch, N, dim) fp32: the state entering every
    // kBwdSub-th row, written when not null by the emit pass (chunk_len is then
    // a multiple of kBwdSub or n_chunks is 1) or by the backward's
    // checkpoint-only pass (launch_ckpt_pass)
    float* ckpt;
    int64_t batch, seqlen, dim;
    int64_t chunk_len, n_chunks;
    // the half-wave layout (32 channels per 4-wave workgroup) instead of the
    // whole-wave one (64 channels per 8-wave workgroup)
    bool half;
    // half-wave layout, chunks shorter than the emit-first threshold, no checkpoints:
    // the aggregate and emit passes read B and C from their arrays (no panel pass)
    int raw_bc;
    // > 0 (with K > 1 and no checkpoints): emit first, then correct.  Pass 1
    // runs every chunk from its own start and writes y; the carry pass follows;
    // pass 2 reruns chunks 1..K-1 from their carries until the carry's effect
    // has decayed below fp32 resolution, checked after corr_head_tiles tiles
    // (even) and then every kCorrEveryTiles, or to the chunk's end
    int corr_head_tiles;
    uint32_t* ws_neg;  // (K, batch, ceil(dim/32)): pass 1 met a negative step size
};

struct StepArgs {
    float* h;
    const void* u;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* Dskip;  // nullable
    const void* z;       // nullable
    const float* delta_bias;  // (dim,), nullable
    uint32_t options;         // kOpt* bits
    void* y;
    int64_t batch, dim;
    int64_t b0, rows;  // the batch rows [b0, b0 + rows) this launch covers
    bool vec_bc;  // B and C are 16-byte aligned: their rows are read 16 bytes at a time
};

// Backward: rows per sub-block, which is also the spacing of the state
// checkpoints the backward recomputes from.
constexpr int kBwdSub = 16;
// emit first, then correct: the correction pass checks whether the carry has
// decayed every kCorrEveryTiles tiles after its first check
constexpr int kCorrEveryTiles = 8;
// the most chunks for which the emit pass forms the carries itself
constexpr int kFuseMaxChunks = 16;

struct BwdArgs {
    // forward inputs
    const void* u;
    const void* delta;
    const float* A;
    const float* Dskip;       // nullable
    const void* z;            // nullable
    const float* h0;          // nullable
    const float* delta_bias;  // nullable
    uint32_t options;         // kOptSoftplus only
    // incoming gradients
    const void* dy;           // (batch, seqlen, dim), dtype
    const float* dh_last;     // (batch, dim, N), nullable
    // gradients
    void* du;
    void* ddelta;
    void* dz;                 // written when z is given
    float* dh0;               // nullable
    void* dB;
    void* dC;
    float* dA;
    float* dD;                // written when Dskip is given
    float* ddelta_bias;       // written when delta_bias is given
    // workspace
    const float* panel;       // the fp32 B/C panel, one chunk per batch row
    int64_t panel_rows;
    float* ckpt;              // (n_sub, batch, N, dim): state entering row kBwdSub*j
    float* part_dB;           // (nblk, batch, seqlen, N): per-workgroup sums over its channels
    float* part_dC;
    float* part_dA;           // (batch, dim, N): per-batch-row sums over time
    float* part_dD;           // (batch, dim)
    float* part_dbias;        // (batch, dim)
    int64_t batch, seqlen, dim, n_sub, nblk;
};

// Causal depthwise convolution + SiLU: rows of output per thread run.
constexpr int64_t kConvRows = 64;

struct ConvArgs {
    const void* x;     // rows of x_stride elements
    int64_t x_stride;
    const float* w;    // (dim, width)
    const float* bias; // (dim,), nullable
    void* u;           // (batch, seqlen, dim)
    int64_t batch, seqlen, dim, width;
};

// Multi-head state-space recurrence (bf16 operands, 64 channels per head).
struct SsdArgs {
    const void* x;     // (batch, seqlen, heads, 64)
    const void* dt;    // (batch, seqlen, heads)
    const float* A;    // (heads,)
    const void* B;     // (batch, seqlen, dstate)
    const void* C;     // (batch, seqlen, dstate)
    const float* D;    // (heads,), nullable
    const float* h0;   // (batch, heads, dstate, 64), nullable
    void* y;           // (batch, seqlen, heads, 64)
    float* h_last;     // (batch, heads, dstate, 64), nullable
    int64_t batch, seqlen, heads, dstate;
    // dstate 256: the first half of the state entries' fp32 part of y (batch,
    // seqlen, heads, 64), which the launch for the second half adds to its own
    float* y_part;
};

// The allocation-free scan entry point's workspace: a static device array of
// kScratchBytes per GPU.  scratch_pointer looks up its address on the current
// device (once per device; later calls return the kept address).
constexpr size_t kScratchBytes = size_t(32) << 20;
hipError_t scratch_pointer(void** ptr);

// Each returns the hipError_t of its launches (hipSuccess when all were enqueued).
hipError_t launch_scan(const ScanArgs& a, int dtype, hipStream_t stream);
hipError_t launch_step(const StepArgs& a, int dtype, hipStream_t stream);
// the B/C panel alone (a.B, a.C, a.ws_panel, a.panel_rows, a.batch, a.seqlen,
// a.chunk_len, a.n_chunks)
hipError_t launch_panel(const ScanArgs& a, int dtype, hipStream_t stream);
// the backward's checkpoint pass over one chunk of the whole sequence (a.u, a.delta,
// a.A, a.h0, a.delta_bias, a.options, a.ws_panel (filled), a.panel_rows, a.ckpt,
// a.batch, a.seqlen, a.dim, a.chunk_len = seqlen, a.n_chunks = 1)
hipError_t launch_ckpt_pass(const ScanArgs& a, int dtype, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, int dtype, hipStream_t stream);
// vec: channels per thread, 1, or 4 (bf16) / 2 (fp32) when the host has checked alignment
hipError_t launch_conv(const ConvArgs& a, int dtype, int vec, hipStream_t stream);
hipError_t launch_ssd(const SsdArgs& a, hipStream_t stream);

}  // namespace ssk
