// C ABI of libssscan.so: argument validation, the chunk plan, workspace
// sizing and kernel dispatch.  Validation runs on the host before anything is
// enqueued, so every rejection path works without a GPU.
#include <stdint.h>
#include <string.h>

#include "ss_internal.h"
#include "ss_scan.h"

static_assert(ssk::kScratchBytes == SS_NOALLOC_MAX_WORKSPACE_BYTES, "the header states the scratch size");

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kWave = 64;
constexpr int64_t kMinAutoChunk = 64;  // the automatic plan never cuts finer
// The automatic plan, in scan workgroups (64 channels of one batch row and one
// chunk each) against the 256 CUs of an MI355X.  Cutting the sequence costs an
// extra aggregate pass over all but the last chunk, so a shape whose one-chunk
// launch already has kSingleChunkBlocks workgroups (about 0.8 per CU) stays
// whole; below that the chunk length halves until the emit launch has
// kTargetBlocks (three per CU).  Measured at L = 2048 (one chunk against the
// best cut): 128 workgroups 180 against 125 us, 160: 196 / 157, 192: 185 / 171,
// 240: 201 / 226, 480: 256 / 376, 640 (the large layer): 380 / 475; the
// small-model layer (48) at 8 / 16 / 32 chunks 73 / 59 / 69 us.
constexpr int64_t kSingleChunkBlocks = 208;
constexpr int64_t kTargetBlocks = 768;
// (Chunks of 1024 rows or more take the emit-first scheme, whose extra cost is
// a correction per chunk, not an aggregate pass: there more chunks only add
// work.  An earlier rule halved such chunks on up to 2048 workgroups; dropping
// it, B=4 L=16384 D=2048 went from 0.59 to 0.54 ms (T 1024 -> 2048) and the
// long context from 1.03 to 1.01 ms (T 2048 -> 4096), half-wave layout.)
constexpr int64_t kMaxGridYZ = 65535;
// A chunk's (B, L, D) slab is addressed with 32-bit buffer offsets, and idle
// lanes use offsets at and above 2^31: one chunk of rows must stay below 2^31
// bytes at 4 bytes per element.
constexpr int64_t kMaxChunkBytes = int64_t(1) << 31;

bool mul(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

int64_t ceil_div(int64_t a, int64_t b) { return a / b + (a % b != 0); }

struct Range {
    uintptr_t lo, hi;  // [lo, hi); empty when the pointer is NULL
};

Range span(const void* p, int64_t bytes)
{
    if (!p) return {0, 0};
    return {reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + static_cast<uintptr_t>(bytes)};
}

bool overlap(Range a, Range b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

bool aligned(const void* p, uintptr_t al) { return (reinterpret_cast<uintptr_t>(p) % al) == 0; }

struct Sizes {
    int64_t rows;    // batch*seqlen*dim
    int64_t srows;   // batch*seqlen*dstate
    int64_t states;  // batch*dim*dstate
    int64_t an;      // dim*dstate
};

// Element counts and their fp32 byte sizes must fit in int64.
bool shape_sizes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, Sizes* s)
{
    if (batch <= 0 || seqlen <= 0 || dim <= 0 || dstate <= 0) return false;
    int64_t bl, tmp;
    if (!mul(batch, seqlen, &bl)) return false;
    if (!mul(bl, dim, &s->rows) || !mul(s->rows, 4, &tmp)) return false;
    if (!mul(bl, dstate, &s->srows) || !mul(s->srows, 4, &tmp)) return false;
    if (!mul(batch, dim, &tmp) || !mul(tmp, dstate, &s->states) || !mul(s->states, 4, &tmp)) return false;
    if (!mul(dim, dstate, &s->an) || !mul(s->an, 4, &tmp)) return false;
    return true;
}

// Plan: chunk length and count.  Automatic plans start from one chunk; a
// shape with fewer than kSingleChunkBlocks workgroups then halves the chunk
// length (staying a power of two, never below kMinAutoChunk) until the emit
// launch has at least kTargetBlocks workgroups.
bool plan(int64_t batch, int64_t seqlen, int64_t dim, int64_t request, int64_t* T, int64_t* K)
{
    if (request < 0) return false;
    int64_t t = request;
    if (t == 0) {
        t = 1;
        while (t < seqlen) t <<= 1;
        int64_t blocks;  // workgroups of a one-chunk launch
        if (!mul(batch, ceil_div(dim, kWave), &blocks)) blocks = INT64_MAX;
        if (blocks < kSingleChunkBlocks) {
            while (t > kMinAutoChunk) {
                int64_t launched;
                if (!mul(blocks, ceil_div(seqlen, t), &launched)) break;
                if (launched >= kTargetBlocks) break;
                t >>= 1;
            }
        }
        int64_t bytes;
        while (t > 1 && (!mul(t, dim, &bytes) || !mul(bytes, 4, &bytes) || bytes >= kMaxChunkBytes)) t >>= 1;
    }
    *T = t;
    *K = ceil_div(seqlen, t);
    return true;
}

// Scan layout: whole-wave workgroups (8 waves, 64 channels) or half-wave ones
// (4 waves, 32 channels), for the same work.  The CUs run their workgroups
// side by side and the call ends with the most loaded CU, so the layout whose
// busiest CU holds less work wins: ceil(wg / 256) workgroups of 64 channels
// against ceil(2 * wg / 256) of 32.  On a tie the whole-wave layout stays (its
// B and C are scalar operands), except for the emit-first scheme (emit_first):
// there the half-wave one was faster on every shape measured, 1.5-6% (the long
// context 1.013 against 1.044 ms at T = 4096; B=4 L=16384 D=2048 0.540 against
// 0.572 ms at T = 2048), and for the short-chunk scheme without checkpoints
// (raw_ok), where the half-wave passes read B and C from their arrays and the
// panel pass goes: B=2 L=2048 D=1536 47.6 -> 45.8 us, B=1 L=2048 D=1024 28.7 ->
// 25.8 us, B=4 L=1024 D=2048 59.9 -> 57.5 us, B=3 L=2048 D=4096 145 -> 144 us
// (B=2 L=4096 D=1536 without skip or gate 78.0 against 79.2 us).
// SS_SCAN_LAYOUT forces a layout at build time (1 whole-wave, 2 half-wave) and
// SS_RAW_BC=0 keeps the panel pass, for measurements.
#ifndef SS_SCAN_LAYOUT
#define SS_SCAN_LAYOUT 0
#endif
#ifndef SS_RAW_BC
#define SS_RAW_BC 1
#endif
constexpr int64_t kCUs = 256;
bool half_layout(int64_t batch, int64_t dim, int64_t K, bool emit_first, bool raw_ok)
{
    if (SS_SCAN_LAYOUT == 1) return false;
    if (SS_SCAN_LAYOUT == 2) return true;
    if (emit_first || (raw_ok && SS_RAW_BC)) return true;
    const int64_t whole = batch * ceil_div(dim, kWave) * K;
    const int64_t halves = batch * ceil_div(dim, kWave / 2) * K;
    return ceil_div(halves, kCUs) < 2 * ceil_div(whole, kCUs);
}

// Emit first, then correct: for chunks of kCorrMinChunk rows or more (a
// multiple of two 8-row tiles) every chunk is first run from its own start,
// and chunks 1..K-1 are then rerun from their carries until the carry's effect
// has decayed below fp32 resolution: checked first after kCorrHead rows, then
// every kCorrEveryTiles tiles.  Shorter chunks take the aggregate pass instead.
// Not with checkpoints.  Returns the first check in tiles, or 0.
#ifndef SS_CORR_MIN_CHUNK
#define SS_CORR_MIN_CHUNK 1024
#endif
constexpr int64_t kCorrMinChunk = SS_CORR_MIN_CHUNK, kCorrHead = 128;
int corr_head_tiles(int64_t T, int64_t K)
{
    if (K < 2 || T < kCorrMinChunk || T % (2 * ssk::kTileRows) != 0) return 0;
    return int(kCorrHead / ssk::kTileRows);
}

// Short-chunk plans with at most kFuseMaxChunks chunks: the emit pass forms each
// chunk's carry itself from the aggregate pass's end states and delta sums (a
// sequential combine of at most 15 affine maps per lane), so there is no carry
// launch.  The small-model layer (16 chunks of 128 rows) had its carry pass at
// 7 us of 57.
bool fuse_carry(int64_t T, int64_t K)
{
    return K > 1 && K <= ssk::kFuseMaxChunks && corr_head_tiles(T, K) == 0;
}

// Workspace layout for K chunks of T rows (fp32 words):
//   K > 1: K state slots of batch*dim*dstate, then (K-1)*batch*dim delta sums;
//   then, at the next multiple of 256 bytes, the B/C panel of
//   batch*K*2*panel_rows(min(T, seqlen))*dstate words.
struct WsLayout {
    int64_t flags_offset = 0;  // bytes (K > 1, emit first): "whole chunk rerun" flags
    int64_t neg_offset = 0;    // bytes: "negative step size" flags
    int64_t agg_offset = 0;    // bytes (fused carry): chunk end states from zero
    int64_t panel_offset;  // bytes
    int64_t panel_words;
    int64_t panel_rows;
    int64_t total;  // bytes
};

bool ws_layout(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int64_t T, int64_t K, WsLayout* w)
{
    int64_t front = 0;
    if (K > 1) {
        int64_t bd, slots, dsums, flags = 0, agg = 0;
        if (!mul(batch, dim, &bd)) return false;
        if (!mul(bd, dstate, &slots) || !mul(slots, K, &slots)) return false;
        if (!mul(bd, K, &dsums)) return false;
        // emit first: (K-1) "whole chunk rerun" and K "negative step" flags per block
        if (corr_head_tiles(T, K) > 0 && !mul(batch * ceil_div(dim, 32), 2 * K - 1, &flags)) return false;
        // fused carry: the K-1 end states from zero, apart from the slots
        if (fuse_carry(T, K) && !mul(slots / K, K - 1, &agg)) return false;
        w->flags_offset = (slots + dsums) * 4;
        w->neg_offset = w->flags_offset + batch * ceil_div(dim, 32) * (K - 1) * 4;
        w->agg_offset = (slots + dsums) * 4;
        if (__builtin_add_overflow(slots, dsums, &front) || __builtin_add_overflow(front, flags, &front) ||
            __builtin_add_overflow(front, agg, &front) || !mul(front, 4, &front))
            return false;
    }
    if (__builtin_add_overflow(front, int64_t(255), &front)) return false;
    w->panel_offset = front & ~int64_t(255);
    w->panel_rows = ssk::panel_rows(T < seqlen ? T : seqlen);
    int64_t words, bytes;
    if (!mul(batch, K, &words) || !mul(words, 2 * w->panel_rows, &words) || !mul(words, dstate, &words))
        return false;
    w->panel_words = words;
    if (!mul(words, 4, &bytes) || __builtin_add_overflow(w->panel_offset, bytes, &w->total)) return false;
    return true;
}

// Backward workspace (fp32 words), each region from a 256-byte boundary:
//   B/C panel (one chunk per batch row), checkpoints (J, B, N, D) with
//   J = ceil(L / kBwdSub), dB and dC partials (nblk, B, L, N) each, dA
//   partials (B, D, N), dD and dbias partials (B, D) each.
struct BwdLayout {
    int64_t panel_rows, n_sub, nblk;
    int64_t off_panel, off_ckpt, off_pdB, off_pdC, off_pdA, off_pdD, off_pdbias;  // bytes
    int64_t total;                                                               // bytes
};

// ckpt_region: false when the caller supplies the checkpoints (the region is
// then empty).
bool bwd_layout(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, BwdLayout* w, bool ckpt_region = true)
{
    w->panel_rows = ssk::panel_rows(seqlen);
    w->n_sub = ceil_div(seqlen, ssk::kBwdSub);
    w->nblk = ceil_div(dim, kWave);
    int64_t words[7];
    int64_t bl, tmp;
    if (!mul(batch, seqlen, &bl)) return false;
    if (!mul(batch, 2 * w->panel_rows, &tmp) || !mul(tmp, dstate, &words[0])) return false;
    if (!mul(w->n_sub, batch, &tmp) || !mul(tmp, dstate, &tmp) || !mul(tmp, dim, &words[1])) return false;
    if (!ckpt_region) words[1] = 0;
    if (!mul(w->nblk, bl, &tmp) || !mul(tmp, dstate, &words[2])) return false;
    words[3] = words[2];
    if (!mul(batch, dim, &tmp) || !mul(tmp, dstate, &words[4])) return false;
    if (!mul(batch, dim, &words[5])) return false;
    words[6] = words[5];
    int64_t* offs[7] = {&w->off_panel, &w->off_ckpt, &w->off_pdB, &w->off_pdC, &w->off_pdA, &w->off_pdD,
                        &w->off_pdbias};
    int64_t at = 0;
    for (int i = 0; i < 7; ++i) {
        int64_t bytes;
        if (__builtin_add_overflow(at, int64_t(255), &at)) return false;
        at &= ~int64_t(255);
        *offs[i] = at;
        if (!mul(words[i], 4, &bytes) || __builtin_add_overflow(at, bytes, &at)) return false;
    }
    w->total = at;
    return true;
}

ss_status hip_fail(hipError_t e)
{
    g_last_hip_error = static_cast<int>(e);
    return SS_ERR_HIP;
}

// ss_scan_bwd with optional caller checkpoints (see ss_scan_bwd_ckpt)
ss_status scan_bwd_impl(const void* u, const void* delta, const float* A, const void* B, const void* C,
                        const float* Dskip, const void* z, const float* h0, const float* delta_bias,
                        uint32_t options, const void* dy, const float* dh_last, void* du, void* ddelta, float* dA,
                        void* dB, void* dC, float* dD, void* dz, float* ddelta_bias, float* dh0, const float* ckpt,
                        void* workspace, size_t workspace_bytes, int64_t batch, int64_t seqlen, int64_t dim,
                        int64_t dstate, ss_dtype dtype, hipStream_t stream);

// ss_scan_fwd_ex with an optional checkpoint output (see ss_scan_fwd_ckpt);
// with use_scratch the workspace arguments are ignored and the library's
// static per-GPU array is used instead (see ss_scan_fwd_noalloc)
ss_status scan_fwd_impl(const void* u, const void* delta, const float* A, const void* B, const void* C,
                        const float* Dskip, const void* z, const float* h0, const float* delta_bias,
                        uint32_t options, void* y, float* h_last, float* ckpt, void* workspace,
                        size_t workspace_bytes, int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                        int64_t chunk_len_request, ss_dtype dtype, hipStream_t stream, bool use_scratch = false);

}  // namespace

extern "C" {

ss_status ss_scan_plan_ex(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int64_t chunk_len_request,
                          int64_t* chunk_len_T, int64_t* n_chunks_K)
{
    Sizes s;
    if (!shape_sizes(batch, seqlen, dim, dstate, &s)) return SS_ERR_INVALID_ARG;
    int64_t T, K;
    if (!plan(batch, seqlen, dim, chunk_len_request, &T, &K)) return SS_ERR_INVALID_ARG;
    if (chunk_len_T) *chunk_len_T = T;
    if (n_chunks_K) *n_chunks_K = K;
    return SS_OK;
}

ss_status ss_scan_plan(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int64_t* chunk_len_T,
                       int64_t* n_chunks_K)
{
    return ss_scan_plan_ex(batch, seqlen, dim, dstate, 0, chunk_len_T, n_chunks_K);
}

size_t ss_scan_workspace_bytes_ex(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                  int64_t chunk_len_request)
{
    Sizes s;
    int64_t T, K;
    WsLayout wl;
    if (!shape_sizes(batch, seqlen, dim, dstate, &s)) return static_cast<size_t>(-1);
    if (!plan(batch, seqlen, dim, chunk_len_request, &T, &K)) return static_cast<size_t>(-1);
    if (!ws_layout(batch, seqlen, dim, dstate, T, K, &wl)) return static_cast<size_t>(-1);
    return static_cast<size_t>(wl.total);
}

size_t ss_scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate)
{
    return ss_scan_workspace_bytes_ex(batch, seqlen, dim, dstate, 0);
}

ss_status ss_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                      const float* Dskip, const void* z, const float* h0, void* y, float* h_last,
                      void* workspace, size_t workspace_bytes, int64_t batch, int64_t seqlen, int64_t dim,
                      int64_t dstate, ss_dtype dtype, hipStream_t stream)
{
    return ss_scan_fwd_ex(u, delta, A, B, C, Dskip, z, h0, nullptr, 0u, y, h_last, workspace, workspace_bytes,
                          batch, seqlen, dim, dstate, 0, dtype, stream);
}

ss_status ss_scan_fwd_ex(const void* u, const void* delta, const float* A, const void* B, const void* C,
                         const float* Dskip, const void* z, const float* h0, const float* delta_bias,
                         uint32_t options, void* y, float* h_last, void* workspace, size_t workspace_bytes,
                         int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int64_t chunk_len_request,
                         ss_dtype dtype, hipStream_t stream)
{
    return scan_fwd_impl(u, delta, A, B, C, Dskip, z, h0, delta_bias, options, y, h_last, nullptr, workspace,
                         workspace_bytes, batch, seqlen, dim, dstate, chunk_len_request, dtype, stream);
}

ss_status ss_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B, const void* C,
                              const float* Dskip, const void* z, const float* h0, void* y, float* h_last,
                              int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, ss_dtype dtype,
                              hipStream_t stream)
{
    return scan_fwd_impl(u, delta, A, B, C, Dskip, z, h0, nullptr, 0u, y, h_last, nullptr, nullptr, 0, batch,
                         seqlen, dim, dstate, 0, dtype, stream, true);
}

size_t ss_scan_ckpt_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate)
{
    Sizes s;
    int64_t bytes;
    if (!shape_sizes(batch, seqlen, dim, dstate, &s)) return static_cast<size_t>(-1);
    if (!mul(ceil_div(seqlen, ssk::kBwdSub), s.states, &bytes) || !mul(bytes, 4, &bytes))
        return static_cast<size_t>(-1);
    return static_cast<size_t>(bytes);
}

ss_status ss_scan_fwd_ckpt(const void* u, const void* delta, const float* A, const void* B, const void* C,
                           const float* Dskip, const void* z, const float* h0, const float* delta_bias,
                           uint32_t options, void* y, float* h_last, float* ckpt, void* workspace,
                           size_t workspace_bytes, int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                           int64_t chunk_len_request, ss_dtype dtype, hipStream_t stream)
{
    if (!ckpt) return SS_ERR_INVALID_ARG;
    return scan_fwd_impl(u, delta, A, B, C, Dskip, z, h0, delta_bias, options, y, h_last, ckpt, workspace,
                         workspace_bytes, batch, seqlen, dim, dstate, chunk_len_request, dtype, stream);
}

}  // extern "C"

namespace {

ss_status scan_fwd_impl(const void* u, const void* delta, const float* A, const void* B, const void* C,
                        const float* Dskip, const void* z, const float* h0, const float* delta_bias,
                        uint32_t options, void* y, float* h_last, float* ckpt, void* workspace,
                        size_t workspace_bytes, int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                        int64_t chunk_len_request, ss_dtype dtype, hipStream_t stream, bool use_scratch)
{
    if (!u || !delta || !A || !B || !C || !y) return SS_ERR_INVALID_ARG;
    Sizes s;
    if (!shape_sizes(batch, seqlen, dim, dstate, &s)) return SS_ERR_INVALID_ARG;
    int64_t T, K;
    if (!plan(batch, seqlen, dim, chunk_len_request, &T, &K)) return SS_ERR_INVALID_ARG;
    if (dtype != SS_F32 && dtype != SS_BF16) return SS_ERR_UNSUPPORTED;
    if (dstate != ssk::kDState) return SS_ERR_UNSUPPORTED;
    if (options & ~ssk::kOptAll) return SS_ERR_UNSUPPORTED;
    if (batch > kMaxGridYZ || K > kMaxGridYZ || batch * dim > INT32_MAX) return SS_ERR_UNSUPPORTED;
    // checkpoints fall every kBwdSub rows: every chunk must start on one
    if (ckpt && K > 1 && T % ssk::kBwdSub != 0) return SS_ERR_UNSUPPORTED;
    WsLayout wl;
    if (!ws_layout(batch, seqlen, dim, dstate, T, K, &wl)) return SS_ERR_INVALID_ARG;
    // the panel kernel runs one thread per word in a one-dimensional grid
    if (ceil_div(wl.panel_words, 256) > int64_t(UINT32_MAX)) return SS_ERR_UNSUPPORTED;
    const int64_t need = wl.total;

    const uintptr_t es = dtype == SS_F32 ? 4 : 2;
    int64_t chunk_bytes;
    if (!mul(T < seqlen ? T : seqlen, dim, &chunk_bytes) || !mul(chunk_bytes, int64_t(es), &chunk_bytes) ||
        chunk_bytes >= kMaxChunkBytes)
        return SS_ERR_UNSUPPORTED;
    const void* elem_ptrs[] = {u, delta, B, C, z, y};
    for (const void* p : elem_ptrs)
        if (p && !aligned(p, es)) return SS_ERR_INVALID_ARG;
    const void* vec_ptrs[] = {A, h0, h_last};
    for (const void* p : vec_ptrs)
        if (p && !aligned(p, 16)) return SS_ERR_INVALID_ARG;
    if (Dskip && !aligned(Dskip, 4)) return SS_ERR_INVALID_ARG;
    if (delta_bias && !aligned(delta_bias, 4)) return SS_ERR_INVALID_ARG;

    const int64_t e = static_cast<int64_t>(es);
    const Range r_u = span(u, s.rows * e), r_dl = span(delta, s.rows * e), r_z = span(z, s.rows * e);
    const Range r_B = span(B, s.srows * e), r_C = span(C, s.srows * e);
    const Range r_A = span(A, s.an * 4), r_D = span(Dskip, dim * 4), r_bias = span(delta_bias, dim * 4);
    const Range r_h0 = span(h0, s.states * 4), r_hl = span(h_last, s.states * 4);
    const Range r_y = span(y, s.rows * e);
    const Range inputs[] = {r_u, r_dl, r_z, r_B, r_C, r_A, r_D, r_bias, r_h0};
    constexpr int kH0 = 8;  // index of h0 in inputs
    for (const Range& r : inputs)
        if (overlap(r_y, r)) return SS_ERR_INVALID_ARG;
    if (overlap(r_y, r_hl)) return SS_ERR_INVALID_ARG;
    Range r_ck = span(nullptr, 0);
    if (ckpt) {
        if (!aligned(ckpt, 16)) return SS_ERR_INVALID_ARG;
        r_ck = span(ckpt, static_cast<int64_t>(ss_scan_ckpt_bytes(batch, seqlen, dim, dstate)));
        for (const Range& r : inputs)
            if (overlap(r_ck, r)) return SS_ERR_INVALID_ARG;
        if (overlap(r_ck, r_y) || overlap(r_ck, r_hl)) return SS_ERR_INVALID_ARG;
    }
    for (const Range& r : inputs) {
        if (&r == &inputs[kH0] && h_last == h0) continue;  // exact in-place continuation is allowed
        if (overlap(r_hl, r)) return SS_ERR_INVALID_ARG;
    }

    if (use_scratch) {
        // every argument is checked above, on the host; the first HIP call comes only now
        if (static_cast<size_t>(need) > ssk::kScratchBytes) return SS_ERR_WORKSPACE;
        const hipError_t se = ssk::scratch_pointer(&workspace);
        if (se != hipSuccess) return hip_fail(se);
        workspace_bytes = ssk::kScratchBytes;
    }
    if (!workspace || workspace_bytes < static_cast<size_t>(need)) return SS_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return SS_ERR_INVALID_ARG;
    const Range r_ws = span(workspace, need);
    for (const Range& r : inputs)
        if (overlap(r_ws, r)) return SS_ERR_INVALID_ARG;
    if (overlap(r_ws, r_y) || overlap(r_ws, r_hl) || overlap(r_ws, r_ck)) return SS_ERR_INVALID_ARG;

    ssk::ScanArgs a;
    a.u = u;
    a.delta = delta;
    a.A = A;
    a.B = B;
    a.C = C;
    a.Dskip = Dskip;
    a.z = z;
    a.h0 = h0;
    a.delta_bias = delta_bias;
    a.options = options;
    a.y = y;
    a.h_last = h_last;
    a.ws_state = K > 1 ? static_cast<float*>(workspace) : nullptr;
    a.ws_dsum = K > 1 ? static_cast<float*>(workspace) + K * batch * dim * dstate : nullptr;
    a.ws_whole = K > 1 ? reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + wl.flags_offset) : nullptr;
    a.ws_neg = K > 1 ? reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + wl.neg_offset) : nullptr;
    a.fuse_carry = fuse_carry(T, K) ? 1 : 0;
    a.ws_agg = K <= 1 ? nullptr
               : a.fuse_carry ? reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.agg_offset)
                              : a.ws_state + batch * dim * dstate;
    a.ws_panel = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.panel_offset);
    a.panel_rows = wl.panel_rows;
    a.ckpt = ckpt;
    a.batch = batch;
    a.seqlen = seqlen;
    a.dim = dim;
    a.chunk_len = T;
    a.n_chunks = K;
    a.corr_head_tiles = ckpt ? 0 : corr_head_tiles(T, K);
    // the short-chunk scheme without checkpoints reads B and C unpanelled
    const bool raw_ok = K > 1 && a.corr_head_tiles == 0 && !ckpt;
    a.half = half_layout(batch, dim, K, a.corr_head_tiles > 0, raw_ok);
    a.raw_bc = (SS_RAW_BC && a.half && raw_ok) ? 1 : 0;
    const hipError_t err = ssk::launch_scan(a, dtype == SS_F32 ? 0 : 1, stream);
    if (err != hipSuccess) return hip_fail(err);
    return SS_OK;
}

}  // namespace

extern "C" {

ss_status ss_step(float* h, const void* u, const void* delta, const float* A, const void* B, const void* C,
                  const float* Dskip, const void* z, void* y, int64_t batch, int64_t dim, int64_t dstate,
                  ss_dtype dtype, hipStream_t stream)
{
    return ss_step_ex(h, u, delta, A, B, C, Dskip, z, nullptr, 0u, y, batch, dim, dstate, dtype, stream);
}

ss_status ss_step_ex(float* h, const void* u, const void* delta, const float* A, const void* B, const void* C,
                     const float* Dskip, const void* z, const float* delta_bias, uint32_t options, void* y,
                     int64_t batch, int64_t dim, int64_t dstate, ss_dtype dtype, hipStream_t stream)
{
    if (!h || !u || !delta || !A || !B || !C || !y) return SS_ERR_INVALID_ARG;
    Sizes s;
    if (!shape_sizes(batch, 1, dim, dstate, &s)) return SS_ERR_INVALID_ARG;
    if (dtype != SS_F32 && dtype != SS_BF16) return SS_ERR_UNSUPPORTED;
    if (dstate != ssk::kDState) return SS_ERR_UNSUPPORTED;
    if (options & ~ssk::kOptAll) return SS_ERR_UNSUPPORTED;
    int64_t threads;
    if (!mul(s.rows, 4, &threads) || ceil_div(threads, 256) > INT32_MAX) return SS_ERR_UNSUPPORTED;

    const uintptr_t es = dtype == SS_F32 ? 4 : 2;
    const void* elem_ptrs[] = {u, delta, B, C, z, y};
    for (const void* p : elem_ptrs)
        if (p && !aligned(p, es)) return SS_ERR_INVALID_ARG;
    if (!aligned(h, 16) || !aligned(A, 16)) return SS_ERR_INVALID_ARG;
    if (Dskip && !aligned(Dskip, 4)) return SS_ERR_INVALID_ARG;
    if (delta_bias && !aligned(delta_bias, 4)) return SS_ERR_INVALID_ARG;

    const int64_t e = static_cast<int64_t>(es);
    const Range r_h = span(h, s.states * 4), r_y = span(y, s.rows * e);
    const Range inputs[] = {span(u, s.rows * e), span(delta, s.rows * e), span(z, s.rows * e),
                            span(B, s.srows * e), span(C, s.srows * e), span(A, s.an * 4),
                            span(Dskip, dim * 4), span(delta_bias, dim * 4)};
    if (overlap(r_h, r_y)) return SS_ERR_INVALID_ARG;
    for (const Range& r : inputs)
        if (overlap(r_h, r) || overlap(r_y, r)) return SS_ERR_INVALID_ARG;

    ssk::StepArgs a;
    a.h = h;
    a.u = u;
    a.delta = delta;
    a.A = A;
    a.B = B;
    a.C = C;
    a.Dskip = Dskip;
    a.z = z;
    a.delta_bias = delta_bias;
    a.options = options;
    a.y = y;
    a.batch = batch;
    a.dim = dim;
    a.vec_bc = aligned(B, 16) && aligned(C, 16);
    const hipError_t err = ssk::launch_step(a, dtype == SS_F32 ? 0 : 1, stream);
    if (err != hipSuccess) return hip_fail(err);
    return SS_OK;
}

size_t ss_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate)
{
    Sizes s;
    BwdLayout wl;
    if (!shape_sizes(batch, seqlen, dim, dstate, &s)) return static_cast<size_t>(-1);
    if (!bwd_layout(batch, seqlen, dim, dstate, &wl)) return static_cast<size_t>(-1);
    return static_cast<size_t>(wl.total);
}

size_t ss_scan_bwd_ckpt_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate)
{
    Sizes s;
    BwdLayout wl;
    if (!shape_sizes(batch, seqlen, dim, dstate, &s)) return static_cast<size_t>(-1);
    if (!bwd_layout(batch, seqlen, dim, dstate, &wl, false)) return static_cast<size_t>(-1);
    return static_cast<size_t>(wl.total);
}

ss_status ss_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                      const float* Dskip, const void* z, const float* h0, const float* delta_bias,
                      uint32_t options, const void* dy, const float* dh_last, void* du, void* ddelta, float* dA,
                      void* dB, void* dC, float* dD, void* dz, float* ddelta_bias, float* dh0, void* workspace,
                      size_t workspace_bytes, int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                      ss_dtype dtype, hipStream_t stream)
{
    return scan_bwd_impl(u, delta, A, B, C, Dskip, z, h0, delta_bias, options, dy, dh_last, du, ddelta, dA, dB,
                         dC, dD, dz, ddelta_bias, dh0, nullptr, workspace, workspace_bytes, batch, seqlen, dim,
                         dstate, dtype, stream);
}

ss_status ss_scan_bwd_ckpt(const void* u, const void* delta, const float* A, const void* B, const void* C,
                           const float* Dskip, const void* z, const float* h0, const float* delta_bias,
                           uint32_t options, const void* dy, const float* dh_last, const float* ckpt, void* du,
                           void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz, float* ddelta_bias,
                           float* dh0, void* workspace, size_t workspace_bytes, int64_t batch, int64_t seqlen,
                           int64_t dim, int64_t dstate, ss_dtype dtype, hipStream_t stream)
{
    if (!ckpt) return SS_ERR_INVALID_ARG;
    return scan_bwd_impl(u, delta, A, B, C, Dskip, z, h0, delta_bias, options, dy, dh_last, du, ddelta, dA, dB,
                         dC, dD, dz, ddelta_bias, dh0, ckpt, workspace, workspace_bytes, batch, seqlen, dim,
                         dstate, dtype, stream);
}

}  // extern "C"

namespace {

ss_status scan_bwd_impl(const void* u, const void* delta, const float* A, const void* B, const void* C,
                        const float* Dskip, const void* z, const float* h0, const float* delta_bias,
                        uint32_t options, const void* dy, const float* dh_last, void* du, void* ddelta, float* dA,
                        void* dB, void* dC, float* dD, void* dz, float* ddelta_bias, float* dh0, const float* ckpt,
                        void* workspace, size_t workspace_bytes, int64_t batch, int64_t seqlen, int64_t dim,
                        int64_t dstate, ss_dtype dtype, hipStream_t stream)
{
    if (!u || !delta || !A || !B || !C || !dy || !du || !ddelta || !dA || !dB || !dC) return SS_ERR_INVALID_ARG;
    if ((Dskip && !dD) || (z && !dz) || (delta_bias && !ddelta_bias)) return SS_ERR_INVALID_ARG;
    Sizes s;
    if (!shape_sizes(batch, seqlen, dim, dstate, &s)) return SS_ERR_INVALID_ARG;
    if (dtype != SS_F32 && dtype != SS_BF16) return SS_ERR_UNSUPPORTED;
    if (dstate != ssk::kDState) return SS_ERR_UNSUPPORTED;
    if (options & ~ssk::kOptAll) return SS_ERR_UNSUPPORTED;
    if (batch > kMaxGridYZ || batch * dim > INT32_MAX) return SS_ERR_UNSUPPORTED;
    BwdLayout wl;
    if (!bwd_layout(batch, seqlen, dim, dstate, &wl, ckpt == nullptr)) return SS_ERR_INVALID_ARG;
    const uintptr_t es = dtype == SS_F32 ? 4 : 2;
    int64_t row_bytes_all;  // one batch row's (L, D) slab is addressed with 32-bit buffer offsets
    if (!mul(seqlen, dim, &row_bytes_all) || !mul(row_bytes_all, int64_t(es), &row_bytes_all) ||
        row_bytes_all >= kMaxChunkBytes)
        return SS_ERR_UNSUPPORTED;

    const void* elem_ptrs[] = {u, delta, B, C, z, dy, du, ddelta, dB, dC, dz};
    for (const void* p : elem_ptrs)
        if (p && !aligned(p, es)) return SS_ERR_INVALID_ARG;
    if (!aligned(A, 16)) return SS_ERR_INVALID_ARG;
    const void* f32_ptrs[] = {Dskip, h0, delta_bias, dh_last, dA, dD, ddelta_bias, dh0};
    for (const void* p : f32_ptrs)
        if (p && !aligned(p, 4)) return SS_ERR_INVALID_ARG;

    const int64_t e = static_cast<int64_t>(es);
    if (ckpt && !aligned(ckpt, 16)) return SS_ERR_INVALID_ARG;
    const int64_t ckpt_bytes = ckpt ? static_cast<int64_t>(ss_scan_ckpt_bytes(batch, seqlen, dim, dstate)) : 0;
    const Range inputs[] = {span(u, s.rows * e), span(delta, s.rows * e), span(z, s.rows * e),
                            span(B, s.srows * e), span(C, s.srows * e), span(A, s.an * 4), span(Dskip, dim * 4),
                            span(h0, s.states * 4), span(delta_bias, dim * 4), span(dy, s.rows * e),
                            span(dh_last, s.states * 4), span(ckpt, ckpt_bytes)};
    const Range outputs[] = {span(du, s.rows * e), span(ddelta, s.rows * e), span(dz, s.rows * e),
                             span(dB, s.srows * e), span(dC, s.srows * e), span(dA, s.an * 4),
                             span(dD, dim * 4), span(ddelta_bias, dim * 4), span(dh0, s.states * 4)};
    // outputs overlap neither the inputs nor each other
    for (size_t i = 0; i < sizeof(outputs) / sizeof(outputs[0]); ++i) {
        for (const Range& r : inputs)
            if (overlap(outputs[i], r)) return SS_ERR_INVALID_ARG;
        for (size_t k = i + 1; k < sizeof(outputs) / sizeof(outputs[0]); ++k)
            if (overlap(outputs[i], outputs[k])) return SS_ERR_INVALID_ARG;
    }
    if (!workspace || workspace_bytes < static_cast<size_t>(wl.total)) return SS_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return SS_ERR_INVALID_ARG;
    const Range r_ws = span(workspace, wl.total);
    for (const Range& r : inputs)
        if (overlap(r_ws, r)) return SS_ERR_INVALID_ARG;
    for (const Range& r : outputs)
        if (overlap(r_ws, r)) return SS_ERR_INVALID_ARG;
    if (ceil_div(int64_t(batch) * 2 * wl.panel_rows * dstate, 256) > int64_t(UINT32_MAX)) return SS_ERR_UNSUPPORTED;

    char* ws = static_cast<char*>(workspace);
    ssk::ScanArgs pa{};
    pa.B = B;
    pa.C = C;
    pa.ws_panel = reinterpret_cast<float*>(ws + wl.off_panel);
    pa.panel_rows = wl.panel_rows;
    pa.batch = batch;
    pa.seqlen = seqlen;
    pa.dim = dim;
    pa.chunk_len = seqlen;
    pa.n_chunks = 1;
    hipError_t err = ssk::launch_panel(pa, dtype == SS_F32 ? 0 : 1, stream);
    if (err != hipSuccess) return hip_fail(err);
    if (!ckpt) {
        // the checkpoints: the half-wave scan kernel's checkpoint-only pass (1280
        // workgroups for the large layer, five per CU; a pass of its own in the
        // adjoint's whole-wave shape ran 640 as 2.5 per CU: 329 against ~250 us)
        ssk::ScanArgs ca = pa;
        ca.u = u;
        ca.delta = delta;
        ca.A = A;
        ca.h0 = h0;
        ca.delta_bias = delta_bias;
        ca.options = options;
        ca.ckpt = reinterpret_cast<float*>(ws + wl.off_ckpt);
        ca.half = 1;
        err = ssk::launch_ckpt_pass(ca, dtype == SS_F32 ? 0 : 1, stream);
        if (err != hipSuccess) return hip_fail(err);
    }

    ssk::BwdArgs a{};
    a.u = u;
    a.delta = delta;
    a.A = A;
    a.Dskip = Dskip;
    a.z = z;
    a.h0 = h0;
    a.delta_bias = delta_bias;
    a.options = options;
    a.dy = dy;
    a.dh_last = dh_last;
    a.du = du;
    a.ddelta = ddelta;
    a.dz = dz;
    a.dh0 = dh0;
    a.dB = dB;
    a.dC = dC;
    a.dA = dA;
    a.dD = dD;
    a.ddelta_bias = ddelta_bias;
    a.panel = pa.ws_panel;
    a.panel_rows = wl.panel_rows;
    // the adjoint only reads the checkpoints (the caller's, or the pass above wrote them)
    a.ckpt = ckpt ? const_cast<float*>(ckpt) : reinterpret_cast<float*>(ws + wl.off_ckpt);
    a.part_dB = reinterpret_cast<float*>(ws + wl.off_pdB);
    a.part_dC = reinterpret_cast<float*>(ws + wl.off_pdC);
    a.part_dA = reinterpret_cast<float*>(ws + wl.off_pdA);
    a.part_dD = reinterpret_cast<float*>(ws + wl.off_pdD);
    a.part_dbias = reinterpret_cast<float*>(ws + wl.off_pdbias);
    a.batch = batch;
    a.seqlen = seqlen;
    a.dim = dim;
    a.n_sub = wl.n_sub;
    a.nblk = wl.nblk;
    err = ssk::launch_bwd(a, dtype == SS_F32 ? 0 : 1, stream);
    if (err != hipSuccess) return hip_fail(err);
    return SS_OK;
}

}  // namespace

extern "C" {

ss_status ss_conv1d_silu(const void* x, int64_t x_row_stride, const float* weight, const float* bias, void* u,
                         int64_t batch, int64_t seqlen, int64_t dim, int64_t width, ss_dtype dtype,
                         hipStream_t stream)
{
    if (!x || !weight || !u) return SS_ERR_INVALID_ARG;
    if (batch <= 0 || seqlen <= 0 || dim <= 0 || width <= 0 || x_row_stride < dim) return SS_ERR_INVALID_ARG;
    if (dtype != SS_F32 && dtype != SS_BF16) return SS_ERR_UNSUPPORTED;
    if (width < 2 || width > 4) return SS_ERR_UNSUPPORTED;
    const int64_t es = dtype == SS_F32 ? 4 : 2;
    int64_t bl, u_elems, x_elems, u_bytes, x_bytes;
    if (!mul(batch, seqlen, &bl) || !mul(bl, dim, &u_elems) || !mul(u_elems, es, &u_bytes)) return SS_ERR_INVALID_ARG;
    // x spans (batch*seqlen - 1) strides plus one row of dim elements
    if (!mul(bl - 1, x_row_stride, &x_elems) || __builtin_add_overflow(x_elems, dim, &x_elems) ||
        !mul(x_elems, es, &x_bytes))
        return SS_ERR_INVALID_ARG;
    if (batch > kMaxGridYZ || ceil_div(seqlen, ssk::kConvRows) > kMaxGridYZ) return SS_ERR_UNSUPPORTED;
    if (!aligned(x, uintptr_t(es)) || !aligned(u, uintptr_t(es))) return SS_ERR_INVALID_ARG;
    if (!aligned(weight, 4) || (bias && !aligned(bias, 4))) return SS_ERR_INVALID_ARG;
    const Range r_u = span(u, u_bytes);
    if (overlap(r_u, span(x, x_bytes)) || overlap(r_u, span(weight, dim * width * 4)) ||
        overlap(r_u, span(bias, dim * 4)))
        return SS_ERR_INVALID_ARG;
    // 8-byte accesses when every row start is 8-byte aligned
    const int vec = int(8 / es);
    const bool vec_ok = dim % vec == 0 && x_row_stride % vec == 0 && aligned(x, 8) && aligned(u, 8);
    ssk::ConvArgs a{x, x_row_stride, weight, bias, u, batch, seqlen, dim, width};
    const hipError_t err = ssk::launch_conv(a, dtype == SS_F32 ? 0 : 1, vec_ok ? vec : 1, stream);
    if (err != hipSuccess) return hip_fail(err);
    return SS_OK;
}

size_t ss_ssd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t heads, int64_t headdim, int64_t dstate)
{
    if (batch <= 0 || seqlen <= 0 || heads <= 0 || headdim <= 0 || dstate <= 0) return static_cast<size_t>(-1);
    int64_t n;
    if (!mul(batch, seqlen, &n) || !mul(n, heads, &n) || !mul(n, headdim, &n) || !mul(n, 4, &n))
        return static_cast<size_t>(-1);
    return dstate == 256 ? static_cast<size_t>(n) : 0;  // the first half's fp32 part of y at dstate 256
}

ss_status ss_ssd_fwd(const void* x, const void* dt, const float* A, const void* B, const void* C, const float* D,
                     const float* h0, void* y, float* h_last, int64_t batch, int64_t seqlen, int64_t heads,
                     int64_t headdim, int64_t dstate, ss_dtype dtype, hipStream_t stream)
{
    return ss_ssd_fwd_ex(x, dt, A, B, C, D, h0, y, h_last, nullptr, 0, batch, seqlen, heads, headdim, dstate, dtype,
                         stream);
}

ss_status ss_ssd_fwd_ex(const void* x, const void* dt, const float* A, const void* B, const void* C, const float* D,
                        const float* h0, void* y, float* h_last, void* workspace, size_t workspace_bytes,
                        int64_t batch, int64_t seqlen, int64_t heads, int64_t headdim, int64_t dstate, ss_dtype dtype,
                        hipStream_t stream)
{
    if (!x || !dt || !A || !B || !C || !y) return SS_ERR_INVALID_ARG;
    if (batch <= 0 || seqlen <= 0 || heads <= 0 || headdim <= 0 || dstate <= 0) return SS_ERR_INVALID_ARG;
    if (dtype != SS_BF16 && dtype != SS_F32) return SS_ERR_UNSUPPORTED;
    if (dtype != SS_BF16 || headdim != 64 || (dstate != 64 && dstate != 128 && dstate != 256))
        return SS_ERR_UNSUPPORTED;
    if (batch > kMaxGridYZ || heads > INT32_MAX) return SS_ERR_UNSUPPORTED;
    // the kernel addresses one batch row of x, y (and B, C) with 32-bit byte offsets
    const int64_t row_bytes = 2 * (heads * headdim > dstate ? heads * headdim : dstate);
    if (seqlen > (int64_t(1) << 31) / row_bytes - 1) return SS_ERR_UNSUPPORTED;
    // at dstate 256 also one batch row of the fp32 parts of y, with the rows a ragged
    // last chunk reaches past the sequence
    if (dstate == 256 && seqlen + 64 > (int64_t(1) << 31) / (heads * headdim * 2)) return SS_ERR_UNSUPPORTED;
    int64_t bl, xe, se, he, hs;
    if (!mul(batch, seqlen, &bl) || !mul(bl, heads, &he) || !mul(he, headdim, &xe) || !mul(xe, 2, &xe))
        return SS_ERR_INVALID_ARG;
    if (!mul(bl, dstate, &se) || !mul(se, 2, &se) || !mul(he, 2, &he)) return SS_ERR_INVALID_ARG;
    if (!mul(batch, heads, &hs) || !mul(hs, dstate, &hs) || !mul(hs, headdim, &hs) || !mul(hs, 4, &hs))
        return SS_ERR_INVALID_ARG;
    const void* v16[] = {x, B, C, y};
    for (const void* p : v16)
        if (!aligned(p, 16)) return SS_ERR_INVALID_ARG;
    if (!aligned(dt, 2)) return SS_ERR_INVALID_ARG;
    const void* f32[] = {A, D, h0, h_last};
    for (const void* p : f32)
        if (p && !aligned(p, 4)) return SS_ERR_INVALID_ARG;
    const Range inputs[] = {span(x, xe), span(dt, he), span(A, heads * 4), span(B, se), span(C, se),
                            span(D, heads * 4), span(h0, hs)};
    const Range r_y = span(y, xe), r_hl = span(h_last, hs);
    if (overlap(r_y, r_hl)) return SS_ERR_INVALID_ARG;
    for (const Range& r : inputs)
        if (overlap(r_y, r) || overlap(r_hl, r)) return SS_ERR_INVALID_ARG;
    const size_t need = ss_ssd_workspace_bytes(batch, seqlen, heads, headdim, dstate);
    if (need == static_cast<size_t>(-1)) return SS_ERR_INVALID_ARG;
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return SS_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return SS_ERR_INVALID_ARG;
        const Range r_ws = span(workspace, static_cast<int64_t>(need));
        if (overlap(r_ws, r_y) || overlap(r_ws, r_hl)) return SS_ERR_INVALID_ARG;
        for (const Range& r : inputs)
            if (overlap(r_ws, r)) return SS_ERR_INVALID_ARG;
    }
    ssk::SsdArgs a{x, dt, A, B, C, D, h0, y, h_last, batch, seqlen, heads, dstate,
                   need > 0 ? static_cast<float*>(workspace) : nullptr};
    const hipError_t err = ssk::launch_ssd(a, stream);
    if (err != hipSuccess) return hip_fail(err);
    return SS_OK;
}

const char* ss_status_string(ss_status st)
{
    switch (st) {
        case SS_OK: return "SS_OK";
        case SS_ERR_INVALID_ARG: return "SS_ERR_INVALID_ARG: invalid argument";
        case SS_ERR_UNSUPPORTED: return "SS_ERR_UNSUPPORTED: unsupported dstate, dtype or size";
        case SS_ERR_WORKSPACE: return "SS_ERR_WORKSPACE: workspace missing or too small";
        case SS_ERR_HIP: return "SS_ERR_HIP: a HIP launch or call failed";
    }
    return "unknown status";
}

int ss_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
