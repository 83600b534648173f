/*
 * ss_probe.h -- C ABI of libssprobe.so: two measurement kernels for gfx950 that
 * give the ceilings the scan is measured against.  Not part of the scan
 * library; only the bench calls them.
 *
 *  ss_probe_stream : a plain stream with n_read input arrays and one output
 *                    array of `bytes` each (out = in0 ^ in1 ^ ... on 16-byte
 *                    words), the read:write mix of a memory-bound pass.  With
 *                    n_read = 3 it is the scan's mix (u, delta, z read, y
 *                    written); with n_read = 1 a copy.  Pointers are device
 *                    pointers, 16-byte aligned, bytes a multiple of 16;
 *                    in1/in2 may be NULL when n_read is 1.
 *  ss_probe_alu    : a vector-ALU issue probe.  Every lane runs `iters`
 *                    iterations of a fixed instruction group; each wave
 *                    records the shader-clock cycles (s_memtime) and the
 *                    100 MHz reference-clock ticks (s_memrealtime) it took in
 *                    cycles[2*wave] and cycles[2*wave+1].  kind 0: 16
 *                    independent fp32 fma chains, one fma each per iteration;
 *                    kind 1: 16 independent v_exp_f32 chains; kind 2: the
 *                    scan's per-element group (four fp32 multiply/fma plus one
 *                    v_exp_f32) for 8 rows x 16 states per iteration (128
 *                    groups); kind 3: one dependent chain of 16 fma per
 *                    iteration; kind 4: one dependent chain of 16 v_exp_f32;
 *                    kind 5: kind 2 without its v_exp_f32; kind 6: kind 2
 *                    with each pair of rows' 32 exp2 issued as one batch;
 *                    kind 7: waves of even workgroups kind 0, of odd ones kind 1;
 *                    kind 8: kind 6 with a workgroup barrier before and after
 *                    each batch of exp2 (the waves of a workgroup change phase
 *                    together); kinds 9, 10, 11: one v_exp_f32 beside 2, 4
 *                    or 8 independent fp32 fma, 8 groups per iteration.
 *                    Launch: `blocks` workgroups of 256 lanes (four waves);
 *                    cycles holds blocks*8 entries (uint64), sink blocks*256
 *                    floats.
 * Both return 0, or the hipError_t of the launch.
 */
#ifndef SS_PROBE_H
#define SS_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

int ss_probe_stream(const void* in0, const void* in1, const void* in2, void* out, size_t bytes, int n_read,
                    int blocks, hipStream_t stream);

int ss_probe_alu(int kind, int iters, int blocks, uint64_t* cycles, float* sink, hipStream_t stream);

/* ss_probe_alu with workgroups of `threads` lanes (256, 512 or 1024: 1, 2 or 4 waves per
 * SIMD from one workgroup); cycles holds blocks*threads/64*2 entries, sink blocks*threads. */
int ss_probe_alu_wg(int kind, int iters, int blocks, int threads, uint64_t* cycles, float* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SS_PROBE_H */
