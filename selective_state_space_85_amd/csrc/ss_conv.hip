// gfx950 kernel of the Mamba block's causal depthwise convolution + SiLU
// that produces the scan's input (Mamba walk-through, section 3.4: a Conv1d
// with one filter of `width` taps per channel, padding width-1 with only the
// first L outputs kept, then silu):
//   u[b,t,d] = silu(bias[d] + sum_k w[d,k] * x[b, t-width+1+k, d]),  x = 0 before t = 0.
//
// Memory-bound: every x element is read once (plus a halo of width-1 rows per
// run of kConvRows rows) and every u element written once.  A thread owns VEC
// adjacent channels (8-byte accesses where alignment allows) and a run of
// rows; the previous width-1 rows of its channels stay in registers as a
// sliding window, so no row is fetched twice within a run.  Rows are loaded
// in groups of kConvBatch to keep several loads in flight per thread.  x rows
// may be strided, so the x half of the in-projection (B, L, 2D) is read in
// place.
#include "ss_device.h"

namespace ssk {
namespace {

constexpr int kConvThreads = 256;
constexpr int kConvBatch = 8;  // rows loaded together

template <int DT, int VEC>
struct VecIO;
template <int VEC>
struct VecIO<0, VEC> {  // fp32
    static __device__ __forceinline__ void load(const void* base, int64_t i, float (&v)[VEC])
    {
        const float* p = static_cast<const float*>(base) + i;
        if constexpr (VEC == 2) {
            const float2 q = *reinterpret_cast<const float2*>(p);
            v[0] = q.x;
            v[1] = q.y;
        } else {
            v[0] = p[0];
        }
    }
    static __device__ __forceinline__ void store(void* base, int64_t i, const float (&v)[VEC])
    {
        float* p = static_cast<float*>(base) + i;
        if constexpr (VEC == 2)
            *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
        else
            p[0] = v[0];
    }
};
template <int VEC>
struct VecIO<1, VEC> {  // bf16
    static __device__ __forceinline__ void load(const void* base, int64_t i, float (&v)[VEC])
    {
        const uint16_t* p = static_cast<const uint16_t*>(base) + i;
        if constexpr (VEC == 4) {
            const uint2 q = *reinterpret_cast<const uint2*>(p);
            v[0] = __uint_as_float(q.x << 16);
            v[1] = __uint_as_float(q.x & 0xffff0000u);
            v[2] = __uint_as_float(q.y << 16);
            v[3] = __uint_as_float(q.y & 0xffff0000u);
        } else {
            v[0] = bf16_bits_to_f32(p[0]);
        }
    }
    static __device__ __forceinline__ void store(void* base, int64_t i, const float (&v)[VEC])
    {
        uint16_t* p = static_cast<uint16_t*>(base) + i;
        if constexpr (VEC == 4) {
            const uint2 q = make_uint2(uint32_t(f32_to_bf16_bits(v[0])) | (uint32_t(f32_to_bf16_bits(v[1])) << 16),
                                       uint32_t(f32_to_bf16_bits(v[2])) | (uint32_t(f32_to_bf16_bits(v[3])) << 16));
            *reinterpret_cast<uint2*>(p) = q;
        } else {
            p[0] = f32_to_bf16_bits(v[0]);
        }
    }
};

// grid = (ceil(dim / (256 * VEC)), ceil(seqlen / kConvRows), batch), block = 256.
// Host guarantees dim % VEC == 0, x_stride % VEC == 0 and VEC-element alignment
// of x and u.
template <int DT, int VEC, int W>
__global__ __launch_bounds__(kConvThreads) void conv_kernel(ConvArgs a)
{
    using IO = VecIO<DT, VEC>;
    const int64_t d0 = (int64_t(blockIdx.x) * kConvThreads + threadIdx.x) * VEC;
    if (d0 >= a.dim) return;
    const int64_t L = a.seqlen;
    const int64_t t0 = int64_t(blockIdx.y) * kConvRows;
    const int64_t b = blockIdx.z;
    const int64_t xrow0 = b * L;  // first row of this batch row in x (units of rows)

    float w[VEC][W], bias[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
#pragma unroll
        for (int k = 0; k < W; ++k) w[v][k] = a.w[(d0 + v) * W + k];
        bias[v] = a.bias ? a.bias[d0 + v] : 0.0f;
    }
    // window[k] = x row t - (W-1) + k for the next output row t, k < W-1
    float win[W > 1 ? W - 1 : 1][VEC];
#pragma unroll
    for (int k = 0; k < W - 1; ++k) {
        const int64_t s = t0 - (W - 1) + k;
        if (s >= 0) {
            IO::load(a.x, (xrow0 + s) * a.x_stride + d0, win[k]);
        } else {
#pragma unroll
            for (int v = 0; v < VEC; ++v) win[k][v] = 0.0f;
        }
    }
    const int64_t t_end = (t0 + kConvRows < L) ? t0 + kConvRows : L;
    for (int64_t tb = t0; tb < t_end; tb += kConvBatch) {
        float xr[kConvBatch][VEC];
#pragma unroll
        for (int r = 0; r < kConvBatch; ++r) {
            const int64_t t = tb + r;
            const int64_t tc = t < t_end ? t : t_end - 1;  // stay inside the run (values unused)
            IO::load(a.x, (xrow0 + tc) * a.x_stride + d0, xr[r]);
        }
#pragma unroll
        for (int r = 0; r < kConvBatch; ++r) {
            const int64_t t = tb + r;
            if (t >= t_end) break;
            float out[VEC];
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                float acc = bias[v];
#pragma unroll
                for (int k = 0; k < W - 1; ++k) acc = fmaf(w[v][k], win[k][v], acc);
                acc = fmaf(w[v][W - 1], xr[r][v], acc);
                out[v] = silu(acc);
            }
            IO::store(a.u, (b * L + t) * a.dim + d0, out);
#pragma unroll
            for (int k = 0; k + 1 < W - 1; ++k) {
#pragma unroll
                for (int v = 0; v < VEC; ++v) win[k][v] = win[k + 1][v];
            }
            if constexpr (W > 1) {
#pragma unroll
                for (int v = 0; v < VEC; ++v) win[W - 2][v] = xr[r][v];
            }
        }
    }
}

template <int DT, int VEC>
hipError_t launch_conv_v(const ConvArgs& a, hipStream_t s)
{
    const dim3 grid(unsigned((a.dim + kConvThreads * VEC - 1) / (kConvThreads * VEC)),
                    unsigned((a.seqlen + kConvRows - 1) / kConvRows), unsigned(a.batch));
    switch (a.width) {
        case 2: conv_kernel<DT, VEC, 2><<<grid, dim3(kConvThreads), 0, s>>>(a); break;
        case 3: conv_kernel<DT, VEC, 3><<<grid, dim3(kConvThreads), 0, s>>>(a); break;
        default: conv_kernel<DT, VEC, 4><<<grid, dim3(kConvThreads), 0, s>>>(a); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv(const ConvArgs& a, int dtype, int vec, hipStream_t stream)
{
    (void)hipGetLastError();
    if (dtype == 0) return vec == 2 ? launch_conv_v<0, 2>(a, stream) : launch_conv_v<0, 1>(a, stream);
    return vec == 4 ? launch_conv_v<1, 4>(a, stream) : launch_conv_v<1, 1>(a, stream);
}

}  // namespace ssk
