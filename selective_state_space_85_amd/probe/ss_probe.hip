// Measurement kernels for gfx950 (see ss_probe.h): a read:write stream and a
// vector-ALU issue probe.  They give the two ceilings of a memory-streaming
// pass with one transcendental per element: the HBM stream rate the chip
// sustains for that traffic mix, and the issue cost of v_exp_f32 next to
// ordinary fp32 arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ss_probe.h"

namespace {

// out[i] = in0[i] ^ in1[i] ^ in2[i] over 16-byte words, grid-stride.
template <int NREAD>
__global__ __launch_bounds__(256) void stream_kernel(const uint4* __restrict__ a, const uint4* __restrict__ b,
                                                     const uint4* __restrict__ c, uint4* __restrict__ out,
                                                     int64_t n)
{
    const int64_t stride = int64_t(gridDim.x) * 256;
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride) {
        uint4 v = a[i];
        if constexpr (NREAD == 3) {
            const uint4 p = b[i], q = c[i];
            v.x ^= p.x ^ q.x;
            v.y ^= p.y ^ q.y;
            v.z ^= p.z ^ q.z;
            v.w ^= p.w ^ q.w;
        }
        out[i] = v;
    }
}

// KIND 0: 16 independent fma chains per lane, v = fma(v, s, t).  KIND 1: 16
// independent exp2 chains, v = exp2(-v) (converges to a fixed point in (0, 1),
// no overflow).  KIND 2: the scan's element, for 8 rows r per loop trip and 16
// state registers i: x = d[r] * a[i] (mul), e = exp2(x), in = xb[r] * b[i]
// (mul), v[i] = fma(e, v[i], in), acc[r] = fma(c[i], v[i], acc[r]) -- four
// vector operations and one v_exp_f32 per element, as in the recurrence.
// KIND 3: one dependent fma chain of 16 per trip (latency).  KIND 4: one
// dependent exp2 chain of 16 per trip (latency).  The empty asm statements
// keep the compiler from hoisting loop-invariant products or merging
// iterations.  Each wave records its shader-clock (s_memtime) and 100 MHz
// reference-clock (s_memrealtime) cycles.
template <int KIND>
__global__ __launch_bounds__(1024) void alu_kernel(int iters, uint64_t* __restrict__ cycles, float* __restrict__ sink)
{
    float v[16];
    const float s = 0.999f, t = 1.0e-3f * float(threadIdx.x & 7);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = 0.25f + 0.01f * float(i) + 1.0e-4f * float(threadIdx.x);
    float d[8], xb[8], acc[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        d[r] = 0.01f * float(r + 1);
        xb[r] = 0.001f * float(r + 1);
        acc[r] = 0.0f;
    }
    __syncthreads();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int k = 0; k < iters; ++k) {
        if constexpr (KIND == 2) {
#pragma unroll
            for (int r = 0; r < 8; ++r) __asm__ volatile("" : "+v"(d[r]), "+v"(xb[r]));
#pragma unroll
            for (int r = 0; r < 8; ++r) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float x = d[r] * (-0.0625f * float(i + 1));
                    const float e = __builtin_amdgcn_exp2f(x);
                    const float in = xb[r] * (0.5f + 0.03125f * float(i));
                    v[i] = fmaf(e, v[i], in);
                    acc[r] = fmaf(0.125f + 0.0078125f * float(i), v[i], acc[r]);
                }
            }
        } else if constexpr (KIND == 5) {
            // the scan element without its exp2: e = x
#pragma unroll
            for (int r = 0; r < 8; ++r) __asm__ volatile("" : "+v"(d[r]), "+v"(xb[r]));
#pragma unroll
            for (int r = 0; r < 8; ++r) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float e = d[r] * (-0.0625f * float(i + 1));
                    const float in = xb[r] * (0.5f + 0.03125f * float(i));
                    v[i] = fmaf(e, v[i], in);
                    acc[r] = fmaf(0.125f + 0.0078125f * float(i), v[i], acc[r]);
                }
            }
        } else if constexpr (KIND == 6 || KIND == 8) {
            // the scan element with its exp2s issued as a batch: per pair of rows all 32
            // products, then all 32 exp2, then the 32 (mul, fma, fma) groups
#pragma unroll
            for (int r = 0; r < 8; ++r) __asm__ volatile("" : "+v"(d[r]), "+v"(xb[r]));
#pragma unroll
            for (int r = 0; r < 8; r += 2) {
                float e[2][16];
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int i = 0; i < 16; ++i) e[q][i] = d[r + q] * (-0.0625f * float(i + 1));
#pragma unroll
                for (int q = 0; q < 2; ++q)
                    __asm__ volatile("" : "+v"(e[q][0]), "+v"(e[q][1]), "+v"(e[q][2]), "+v"(e[q][3]), "+v"(e[q][4]),
                                     "+v"(e[q][5]), "+v"(e[q][6]), "+v"(e[q][7]), "+v"(e[q][8]), "+v"(e[q][9]),
                                     "+v"(e[q][10]), "+v"(e[q][11]), "+v"(e[q][12]), "+v"(e[q][13]), "+v"(e[q][14]),
                                     "+v"(e[q][15]));
                if constexpr (KIND == 8) __syncthreads();
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int i = 0; i < 16; ++i) e[q][i] = __builtin_amdgcn_exp2f(e[q][i]);
                if constexpr (KIND == 8) __syncthreads();
#pragma unroll
                for (int q = 0; q < 2; ++q)
                    __asm__ volatile("" : "+v"(e[q][0]), "+v"(e[q][1]), "+v"(e[q][2]), "+v"(e[q][3]), "+v"(e[q][4]),
                                     "+v"(e[q][5]), "+v"(e[q][6]), "+v"(e[q][7]), "+v"(e[q][8]), "+v"(e[q][9]),
                                     "+v"(e[q][10]), "+v"(e[q][11]), "+v"(e[q][12]), "+v"(e[q][13]), "+v"(e[q][14]),
                                     "+v"(e[q][15]));
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const float in = xb[r + q] * (0.5f + 0.03125f * float(i));
                        v[i] = fmaf(e[q][i], v[i], in);
                        acc[r + q] = fmaf(0.125f + 0.0078125f * float(i), v[i], acc[r + q]);
                    }
            }
        } else if constexpr (KIND == 7) {
            // waves of even workgroups run kind 0's fma chains, those of odd ones kind
            // 1's exp2 chains (a SIMD holds waves of several workgroups): whether the two
            // kinds of instruction overlap on one SIMD
            const bool odd = blockIdx.x & 1;
            if (odd) {
#pragma unroll
                for (int i = 0; i < 16; ++i) v[i] = __builtin_amdgcn_exp2f(-v[i]);
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) v[i] = fmaf(v[i], s, t);
            }
        } else if constexpr (KIND >= 9 && KIND <= 11) {
            // one exp2 (its own chain) beside 2, 4 or 8 independent fma (their own chains):
            // whether a transcendental overlaps ordinary vector work
            constexpr int NF = KIND == 9 ? 2 : (KIND == 10 ? 4 : 8);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                v[i] = __builtin_amdgcn_exp2f(-v[i]);
#pragma unroll
                for (int j = 0; j < NF; ++j) acc[j] = fmaf(acc[j], s, t);
            }
        } else if constexpr (KIND == 3) {
#pragma unroll
            for (int i = 0; i < 16; ++i) v[0] = fmaf(v[0], s, t);
        } else if constexpr (KIND == 4) {
#pragma unroll
            for (int i = 0; i < 16; ++i) v[0] = __builtin_amdgcn_exp2f(-v[0]);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if constexpr (KIND == 0)
                    v[i] = fmaf(v[i], s, t);
                else
                    v[i] = __builtin_amdgcn_exp2f(-v[i]);
            }
        }
        __asm__ volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]),
                         "+v"(v[7]));
        __asm__ volatile("" : "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]),
                         "+v"(v[14]), "+v"(v[15]));
        if constexpr (KIND >= 9)
            __asm__ volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]),
                             "+v"(acc[6]), "+v"(acc[7]));
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    float r = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) r += v[i];
#pragma unroll
    for (int j = 0; j < 8; ++j) r += acc[j];
    sink[int64_t(blockIdx.x) * blockDim.x + threadIdx.x] = r;
    if ((threadIdx.x & 63) == 0) {
        const int64_t wv = int64_t(blockIdx.x) * (blockDim.x / 64) + threadIdx.x / 64;
        cycles[2 * wv] = t1 - t0;
        cycles[2 * wv + 1] = r1 - r0;
    }
}

}  // namespace

extern "C" int ss_probe_stream(const void* in0, const void* in1, const void* in2, void* out, size_t bytes,
                               int n_read, int blocks, hipStream_t stream)
{
    if (!in0 || !out || bytes % 16 != 0 || blocks <= 0 || (n_read != 1 && n_read != 3)) return int(hipErrorInvalidValue);
    if (n_read == 3 && (!in1 || !in2)) return int(hipErrorInvalidValue);
    const int64_t n = int64_t(bytes / 16);
    (void)hipGetLastError();
    if (n_read == 1)
        stream_kernel<1><<<dim3(blocks), dim3(256), 0, stream>>>(static_cast<const uint4*>(in0), nullptr, nullptr,
                                                                  static_cast<uint4*>(out), n);
    else
        stream_kernel<3><<<dim3(blocks), dim3(256), 0, stream>>>(static_cast<const uint4*>(in0),
                                                                  static_cast<const uint4*>(in1),
                                                                  static_cast<const uint4*>(in2),
                                                                  static_cast<uint4*>(out), n);
    return int(hipGetLastError());
}

extern "C" int ss_probe_alu(int kind, int iters, int blocks, uint64_t* cycles, float* sink, hipStream_t stream)
{
    return ss_probe_alu_wg(kind, iters, blocks, 256, cycles, sink, stream);
}

extern "C" int ss_probe_alu_wg(int kind, int iters, int blocks, int threads, uint64_t* cycles, float* sink,
                               hipStream_t stream)
{
    if (!cycles || !sink || iters <= 0 || blocks <= 0 || kind < 0 || kind > 11) return int(hipErrorInvalidValue);
    if (threads != 256 && threads != 512 && threads != 1024) return int(hipErrorInvalidValue);
    (void)hipGetLastError();
    const dim3 g(blocks), b(threads);
    switch (kind) {
        case 0: alu_kernel<0><<<g, b, 0, stream>>>(iters, cycles, sink); break;
        case 1: alu_kernel<1><<<g, b, 0, stream>>>(iters, cycles, sink); break;
        case 2: alu_kernel<2><<<g, b, 0, stream>>>(iters, cycles, sink); break;
        case 3: alu_kernel<3><<<g, b, 0, stream>>>(iters, cycles, sink); break;
        case 4: alu_kernel<4><<<g, b, 0, stream>>>(iters, cycles, sink); break;
        case 5: alu_kernel<5><<<g, b, 0, stream>>>(iters, cycles, sink); break;
        case 6: alu_kernel<6><<<g, b, 0, stream>>>(iters, cycles, sink); break;
        case 7: alu_kernel<7><<<g, b, 0, stream>>>(iters, cycles, sink); break;
        case 8: alu_kernel<8><<<g, b, 0, stream>>>(iters, cycles, sink); break;
        case 9: alu_kernel<9><<<g, b, 0, stream>>>(iters, cycles, sink); break;
        case 10: alu_kernel<10><<<g, b, 0, stream>>>(iters, cycles, sink); break;
        default: alu_kernel<11><<<g, b, 0, stream>>>(iters, cycles, sink); break;
    }
    return int(hipGetLastError());
}
