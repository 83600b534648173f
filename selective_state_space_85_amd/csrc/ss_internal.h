// Internal interface between the C-ABI layer (ss_api.cpp) and the gfx950
// kernels (ss_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace ssk {

constexpr int kDState = 16;  // the state width the kernels are built for

// Waves per scan workgroup; the 16 state entries are split evenly across them.
#ifndef SS_SCAN_WAVES
#define SS_SCAN_WAVES 8
#endif
constexpr int kScanWaves = SS_SCAN_WAVES;
static_assert(kScanWaves == 2 || kScanWaves == 4 || kScanWaves == 8, "state split must divide 16");

struct ScanArgs {
    const void* u;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* Dskip;  // nullable
    const void* z;       // nullable
    const float* h0;     // nullable
    void* y;
    float* h_last;       // nullable
    float* ws_state;     // (K, batch, dim, N) state slots, nullable when K == 1
    float* ws_dsum;      // (K-1, batch, dim) per-chunk delta sums
    int64_t batch, seqlen, dim;
    int64_t chunk_len, n_chunks;
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
    void* y;
    int64_t batch, dim;
};

// Each returns the hipError_t of its launches (hipSuccess when all were enqueued).
hipError_t launch_scan(const ScanArgs& a, int dtype, hipStream_t stream);
hipError_t launch_step(const StepArgs& a, int dtype, hipStream_t stream);

}  // namespace ssk
