// prefill_f32.hip -- causal Parallax prefill in fp32 on the vector ALUs (small head dims).
//
// One thread owns one query row and walks its visible keys 0..i in order, keeping the
// streaming state of both branches: one running max m (log2 domain), normaliser l,
// beta = sum w t, A1 = sum w v and A2 = sum w t v; the output is
// o = (A1/l)(1 + beta/l) - A2/l  [Parallax (paper.rainbus.top summary), method steps 2-6
// and the streaming sentences; agihunt review, hardware paragraph]. Keys and values are
// staged through LDS 64 rows at a time and read by every thread of the block (broadcast).
#include "plx_device.hpp"
#include "plx_kernels.hpp"

namespace plx {
namespace {

constexpr int kRows = 64;  // query rows per block == key rows per LDS tile

template <int D>
__global__ __launch_bounds__(kRows) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ rho, float* __restrict__ o, int H, int T, float c) {
    __shared__ float Ks[kRows][D];
    __shared__ float Vs[kRows][D];
    const int tid = threadIdx.x;
    const int i = blockIdx.x * kRows + tid;
    const size_t slice = ((size_t)blockIdx.z * H + blockIdx.y) * (size_t)T;
    const bool valid = i < T;

    float qi[D], ri[D], a1[D], a2[D];
#pragma unroll
    for (int e = 0; e < D; ++e) {
        qi[e] = valid ? q[(slice + i) * D + e] : 0.f;
        ri[e] = valid && rho ? rho[(slice + i) * D + e] : 0.f;  // no rho: the softmax-only case
        a1[e] = 0.f;
        a2[e] = 0.f;
    }
    float m = -INFINITY, l = 0.f, beta = 0.f;

    const int kend = min(T, (int)blockIdx.x * kRows + kRows);
    for (int k0 = 0; k0 < kend; k0 += kRows) {
        __syncthreads();
        for (int idx = tid; idx < kRows * D; idx += kRows) {
            const int r = idx / D, e = idx % D;
            const int key = k0 + r;
            Ks[r][e] = key < T ? k[(slice + key) * D + e] : 0.f;
            Vs[r][e] = key < T ? v[(slice + key) * D + e] : 0.f;
        }
        __syncthreads();
        if (!valid) continue;
        const int jn = min(kRows, i - k0 + 1);  // keys k0 .. i of this tile
        for (int j = 0; j < jn; ++j) {
            float s = 0.f, t = 0.f;
#pragma unroll
            for (int e = 0; e < D; ++e) {
                s = fmaf(qi[e], Ks[j][e], s);
                t = fmaf(ri[e], Ks[j][e], t);
            }
            const float sc = s * c;
            if (sc > m) {  // one rescale factor for both branches
                const float alpha = exp2_fast(m - sc);
                l *= alpha;
                beta *= alpha;
#pragma unroll
                for (int e = 0; e < D; ++e) {
                    a1[e] *= alpha;
                    a2[e] *= alpha;
                }
                m = sc;
            }
            const float w = exp2_fast(sc - m);
            const float wt = w * t;
            l += w;
            beta += wt;
#pragma unroll
            for (int e = 0; e < D; ++e) {
                a1[e] = fmaf(w, Vs[j][e], a1[e]);
                a2[e] = fmaf(wt, Vs[j][e], a2[e]);
            }
        }
    }
    if (!valid) return;
    const float inv = 1.f / l;
    const float one_tb = 1.f + beta * inv;
#pragma unroll
    for (int e = 0; e < D; ++e) o[(slice + i) * D + e] = inv * (a1[e] * one_tb - a2[e]);
}

template <int D>
hipError_t launch(const PrefillArgs& a, hipStream_t stream) {
    dim3 grid((a.T + kRows - 1) / kRows, a.H, a.B);
    hipLaunchKernelGGL(prefill_f32_kernel<D>, grid, dim3(kRows), 0, stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v,
                       (const float*)a.rho, (float*)a.o, a.H, a.T, a.scale * kLog2e);
    return hipGetLastError();
}

}  // namespace

bool prefill_f32_supported(int d) { return d == 16 || d == 32 || d == 64; }

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) {
    switch (a.d) {
        case 16: return launch<16>(a, stream);
        case 32: return launch<32>(a, stream);
        case 64: return launch<64>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace plx
