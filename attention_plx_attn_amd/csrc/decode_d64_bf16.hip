// decode_d64_bf16.hip -- the combine of split decode records at head dim 64, gfx950.
//
// The decode at head dim 64 (the compute-matched head dim of the agihunt review's pretraining
// table: halving d makes the four products per cached row cost what softmax attention's two
// cost at d = 128) runs the grouped-head kernel with d = 64 (decode_gqa_bf16.hip; one query
// head per cache head unless grouped). With more than one chunk per (b, h) its partials go to
// records of 2 * 64 + 4 floats, which this kernel merges: o = (A1/l)(1 + beta/l) - A2/l after
// rescaling every record to the largest running max [Parallax (paper.rainbus.top summary),
// method step 6].
#include "plx_device.hpp"
#include "plx_kernels.hpp"

namespace plx {
namespace {

constexpr int D = 64;
constexpr int REC = 2 * D + 4;  // record: A1[D], A2[D], m, l, beta, pad

// o = (A1/l)(1 + beta/l) - A2/l; an empty range (l == 0) gives 0.
__device__ __forceinline__ float combine_out(float a1, float a2, float l, float beta) {
    if (!(l > 0.f)) return 0.f;
    const float inv = 1.f / l;
    return inv * (a1 * (1.f + beta * inv) - a2);
}

// Online merge state of one wave; lane owns dim lane.
struct Merge {
    float m = -INFINITY, l = 0.f, beta = 0.f, a1 = 0.f, a2 = 0.f;
};

// Fold records rec_at(0 .. n-1) into st, issuing the loads of a batch of BATCH records before
// using any of them (one memory round trip per batch). An empty record has m = -inf.
template <int BATCH, class RecAt>
__device__ __forceinline__ void fold_records(Merge& st, int n, RecAt rec_at, int lane) {
    for (int u0 = 0; u0 < n; u0 += BATCH) {
        float ms[BATCH], ls[BATCH], bs[BATCH], x1[BATCH], x2[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const float* rec = rec_at(min(u0 + u, n - 1));
            ms[u] = u0 + u < n ? rec[2 * D] : -INFINITY;
            ls[u] = rec[2 * D + 1];
            bs[u] = rec[2 * D + 2];
            x1[u] = rec[lane];
            x2[u] = rec[D + lane];
        }
        float mb = st.m;
#pragma unroll
        for (int u = 0; u < BATCH; ++u) mb = fmaxf(mb, ms[u]);
        if (mb == -INFINITY) continue;  // nothing non-empty yet (wave-uniform)
        const float fo = st.m > -INFINITY ? exp2_fast(st.m - mb) : 0.f;
        st.l *= fo;
        st.beta *= fo;
        st.a1 *= fo;
        st.a2 *= fo;
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const float f = ms[u] > -INFINITY ? exp2_fast(ms[u] - mb) : 0.f;
            st.l = fmaf(f, ls[u], st.l);
            st.beta = fmaf(f, bs[u], st.beta);
            st.a1 = fmaf(f, x1[u], st.a1);
            st.a2 = fmaf(f, x2[u], st.a2);
        }
        st.m = mb;
    }
}

// One wave per (b, h): lane owns dim lane and folds the S records in batches of 16 (all loads
// of a batch in flight together; one batch for up to 16 splits).
__global__ __launch_bounds__(64) void decode_combine_d64_kernel(const float* __restrict__ ws,
                                                               __bf16* __restrict__ o, int S) {
    const int lane = threadIdx.x;
    const size_t bh = blockIdx.x;
    const float* base = ws + bh * (size_t)S * REC;
    Merge st;
    fold_records<16>(st, S, [&](int u) { return base + (size_t)u * REC; }, lane);
    o[bh * D + lane] = (__bf16)combine_out(st.a1, st.a2, st.l, st.beta);
}

}  // namespace

hipError_t launch_decode_combine_d64(const DecodeArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(decode_combine_d64_kernel, dim3(a.B * a.H), dim3(64), 0, stream,
                       (const float*)a.ws, (__bf16*)a.o, a.splits);
    return hipGetLastError();
}

}  // namespace plx
