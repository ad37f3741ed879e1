// decode_d64_bf16.hip -- one Parallax decode step at head dim 64 (the compute-matched head dim
// of the agihunt review's pretraining table: halving d makes the four products per cached row
// cost what softmax attention's two cost at d = 128), bf16 in/out, gfx950. Split-KV
// partials plus a combine, as at d = 128.
//
// The per-wave step follows the d = 128 decode [agihunt review, hardware paragraph: the probe
// products ride in accumulator rows a single query row leaves idle]:
//  * scores: each 16-row key tile is one v_mfma_f32_16x16x32_bf16 per 32 dims (two here) with
//    the keys as rows and the columns [q, rho, 0 ... 0], so column 0 holds q.k and column 1
//    the probe products t = rho.k;
//  * online softmax with a wave-uniform running max; the weights w and w*t stay fp32 (the
//    value products run on the VALU) and l, beta are summed from them [Parallax
//    (paper.rainbus.top summary), method steps 2-6];
//  * values: a 64-dim row is 8 lanes of 16 bytes, so the 64 lanes take 8 row groups: lane
//    (col, g) accumulates A1 = sum w v and A2 = sum w t v for dims 8 (col & 7) .. +7 over the
//    8 rows 8 (2 g + (col >> 3)) .. +7 of each 64-row step.
// A step covers 64 rows, so that a wave has as many bytes in flight per step as the d = 128
// decode's 32-row steps.
// Loads use raw buffer resources: rows at or beyond the resource's range read as zero.
#include "plx_device.hpp"
#include "plx_kernels.hpp"

namespace plx {
namespace {

constexpr int D = 64;
constexpr int KB = 64;       // keys per wave step (16 KB of K and V, as a d = 128 step)
constexpr int KT = KB / 16;  // score tiles per step
constexpr int VR = KB / 8;   // value rows per lane per step (8 row groups)
constexpr int NW = 4;        // waves per workgroup
constexpr int NT = 64 * NW;
constexpr int REC = 2 * D + 4;  // record: A1[D], A2[D], m, l, beta, pad
constexpr uint32_t ROWB = 2 * D;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int clamp_len(int n, int L_max) {
    return n < 0 ? 0 : (n > L_max ? L_max : n);
}

// o = (A1/l)(1 + beta/l) - A2/l; an empty range (l == 0) gives 0.
__device__ __forceinline__ float combine_out(float a1, float a2, float l, float beta) {
    if (!(l > 0.f)) return 0.f;
    const float inv = 1.f / l;
    return inv * (a1 * (1.f + beta * inv) - a2);
}

struct Frag {
    u32x4 k[KT][2];  // K rows 16 t + col, dims 32 st + 8 g .. +7
    u32x4 v[VR];     // V rows VR (2 g + (col >> 3)) + r, dims 8 (col & 7) .. +7
};

struct Acc {
    float m_run, rsum, a1[8], a2[8];
    __device__ __forceinline__ void reset() {
        m_run = -INFINITY;
        rsum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a1[e] = a2[e] = 0.f;
    }
};

__device__ __forceinline__ void load_step(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                          int kb0, int col, int g, Frag& f) {
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int st = 0; st < 2; ++st)
            f.k[t][st] = load16_nt(rk, (uint32_t)(kb0 + 16 * t + col) * ROWB + 64u * st + 16u * g);
    const int vg = 2 * g + (col >> 3);
#pragma unroll
    for (int r = 0; r < VR; ++r)
        f.v[r] = load16_nt(rv, (uint32_t)(kb0 + VR * vg + r) * ROWB + 16u * (col & 7));
}

template <bool PROBE>
__device__ __forceinline__ void consume(Acc& s, const Frag& f, const bf16x8 (&bqr)[2], int kb0,
                                        int je, float c, float (*ush)[KB], int col, int g) {
    f32x4 sc[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) {
        sc[t] = f32x4{};
#pragma unroll
        for (int st = 0; st < 2; ++st) sc[t] = mfma16(as_bf16x8(f.k[t][st]), bqr[st], sc[t]);
    }
    // Lane (col, g) register i holds key kb0 + 16 t + 4 g + i.
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            mx = fmaxf(mx, (col == 0 && kb0 + 16 * t + 4 * g + i < je) ? sc[t][i] * c : -INFINITY);
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float mb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), 0));
    if (mb > s.m_run) {  // wave-uniform
        const float alpha = exp2_fast(s.m_run - mb);
        s.rsum *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            s.a1[e] *= alpha;
            if constexpr (PROBE) s.a2[e] *= alpha;
        }
        s.m_run = mb;
    }
#pragma unroll
    for (int t = 0; t < KT; ++t) {
        float u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float own = sc[t][i];
            const float partner = swap_adjacent(own);  // every lane active
            const float score = col == 1 ? partner : own;
            const bool valid = kb0 + 16 * t + 4 * g + i < je;
            const float wgt = valid ? exp2_fast(fmaf(score, c, -s.m_run)) : 0.f;
            u[i] = col == 0 ? wgt : (col == 1 ? wgt * own : 0.f);
        }
        // The value products run on the VALU in fp32, so w and w t stay fp32 and l, beta
        // are summed from exactly the weights that multiply the values.
        s.rsum += (u[0] + u[1]) + (u[2] + u[3]);
        if (col < 2) *(f32x4*)&ush[col][16 * t + 4 * g] = f32x4{u[0], u[1], u[2], u[3]};
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    const int vg = 2 * g + (col >> 3);
#pragma unroll
    for (int r4 = 0; r4 < VR / 4; ++r4) {
        const f32x4 u0 = *(const f32x4*)&ush[0][VR * vg + 4 * r4];
        const f32x4 u1 = PROBE ? *(const f32x4*)&ush[1][VR * vg + 4 * r4] : f32x4{};
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const u32x4 x = f.v[4 * r4 + rr];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float vlo = bf16_lo(x[p]), vhi = bf16_hi(x[p]);
                s.a1[2 * p] = fmaf(u0[rr], vlo, s.a1[2 * p]);
                s.a1[2 * p + 1] = fmaf(u0[rr], vhi, s.a1[2 * p + 1]);
                if constexpr (PROBE) {
                    s.a2[2 * p] = fmaf(u1[rr], vlo, s.a2[2 * p]);
                    s.a2[2 * p + 1] = fmaf(u1[rr], vhi, s.a2[2 * p + 1]);
                }
            }
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Split mode: workgroup (s, h, b) takes chunk s of sequence b's rows for head h; its 4 waves
// stride through the chunk in 64-row steps (loads of the next step issued before the current
// one is consumed) and merge their states through LDS. S == 1 writes o, else a record.
template <bool PROBE>
__global__ __launch_bounds__(NT, 2) void decode_split_bf16_d64_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ rho, const __bf16* __restrict__ kc,
    const __bf16* __restrict__ vc, const int32_t* __restrict__ seqlens, __bf16* __restrict__ o,
    float* __restrict__ ws, int H, int L_max, int S, float c) {
    __shared__ __attribute__((aligned(16))) float ush[NW][2][KB];
    __shared__ __attribute__((aligned(16))) float red[NW][REC];

    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int col = lane & 15, g = lane >> 4;

    const int nb_keys = clamp_len(seqlens[b], L_max);
    const int chunk = (((nb_keys + S - 1) / S) + KB - 1) / KB * KB;
    const int j0 = s * chunk;
    const int j1 = min(j0 + chunk, nb_keys);
    const size_t bh = (size_t)b * H + h;
    const uint32_t range = j1 > 0 ? (uint32_t)j1 * ROWB : 0u;
    const auto rk = make_rsrc(kc + bh * (size_t)L_max * D, range);
    const auto rv = make_rsrc(vc + bh * (size_t)L_max * D, range);

    // B operand [q | rho | 0 ...]: lane (col, g) holds dims 32 st + 8 g .. +7 of column col;
    // other columns read past the 128-byte ranges and get zeros.
    bf16x8 bqr[2];
    {
        const auto rq = make_rsrc(q + bh * D, ROWB);
        const auto rr = make_rsrc(PROBE ? rho + bh * D : q, PROBE ? ROWB : 0u);
        const uint32_t oq = col == 0 ? 16u * g : 1024u, orr = col == 1 ? 16u * g : 1024u;
#pragma unroll
        for (int st = 0; st < 2; ++st)
            bqr[st] = as_bf16x8(load16(rq, oq + 64u * st) | load16(rr, orr + 64u * st));
    }

    Acc acc;
    acc.reset();
    constexpr int STEP = KB * NW;
    Frag fa, fb;
    int kb0 = j0 + KB * w;
    if (kb0 < j1) load_step(rk, rv, kb0, col, g, fa);
    for (; kb0 < j1; kb0 += 2 * STEP) {
        load_step(rk, rv, kb0 + STEP, col, g, fb);
        consume<PROBE>(acc, fa, bqr, kb0, j1, c, ush[w], col, g);
        if (kb0 + STEP >= j1) break;
        load_step(rk, rv, kb0 + 2 * STEP, col, g, fa);
        consume<PROBE>(acc, fb, bqr, kb0 + STEP, j1, c, ush[w], col, g);
    }

    // Wave totals: values over the 8 row groups (lanes 0..7 then hold dims 8 lane .. +7),
    // l in lane 0 and beta in lane 1.
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        acc.a1[e] += shfl_xor(acc.a1[e], 8);
        acc.a1[e] += shfl_xor(acc.a1[e], 16);
        acc.a1[e] += shfl_xor(acc.a1[e], 32);
        if constexpr (PROBE) {
            acc.a2[e] += shfl_xor(acc.a2[e], 8);
            acc.a2[e] += shfl_xor(acc.a2[e], 16);
            acc.a2[e] += shfl_xor(acc.a2[e], 32);
        }
    }
    acc.rsum += shfl_xor(acc.rsum, 16);
    acc.rsum += shfl_xor(acc.rsum, 32);
    if (lane < 8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            red[w][8 * lane + e] = acc.a1[e];
            red[w][D + 8 * lane + e] = acc.a2[e];
        }
    }
    if (lane == 0) {
        red[w][2 * D] = acc.m_run;
        red[w][2 * D + 1] = acc.rsum;
    }
    if (lane == 1) red[w][2 * D + 2] = acc.rsum;
    __syncthreads();

    // Merge the 4 wave states; thread tid < 64 owns dim tid.
    if (tid < D) {
        float M = -INFINITY;
#pragma unroll
        for (int i = 0; i < NW; ++i) M = fmaxf(M, red[i][2 * D]);
        float l = 0.f, beta = 0.f, A1 = 0.f, A2 = 0.f;
        if (M > -INFINITY) {
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                const float mi = red[i][2 * D];
                const float f = mi > -INFINITY ? exp2_fast(mi - M) : 0.f;
                l = fmaf(f, red[i][2 * D + 1], l);
                beta = fmaf(f, red[i][2 * D + 2], beta);
                A1 = fmaf(f, red[i][tid], A1);
                A2 = fmaf(f, red[i][D + tid], A2);
            }
        }
        if (S == 1) {
            o[bh * D + tid] = (__bf16)combine_out(A1, A2, l, beta);
        } else {
            float* rec = ws + (bh * (size_t)S + s) * REC;
            rec[tid] = A1;
            rec[D + tid] = A2;
            if (tid == 0) {
                rec[2 * D] = M;
                rec[2 * D + 1] = l;
                rec[2 * D + 2] = beta;
                rec[2 * D + 3] = 0.f;
            }
        }
    }
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

hipError_t launch_decode_bf16_d64(const DecodeArgs& a, hipStream_t stream) {
    if (a.waves > 0 || a.table) return hipErrorInvalidValue;  // split mode, contiguous cache
    const dim3 grid(a.splits, a.H, a.B);
    const float c = a.scale * kLog2e;
    if (a.rho)
        hipLaunchKernelGGL(decode_split_bf16_d64_kernel<true>, grid, dim3(NT), 0, stream,
                           (const __bf16*)a.q, (const __bf16*)a.rho, (const __bf16*)a.k,
                           (const __bf16*)a.v, a.seqlens, (__bf16*)a.o, a.ws, a.H, a.L_max,
                           a.splits, c);
    else
        hipLaunchKernelGGL(decode_split_bf16_d64_kernel<false>, grid, dim3(NT), 0, stream,
                           (const __bf16*)a.q, (const __bf16*)a.q, (const __bf16*)a.k,
                           (const __bf16*)a.v, a.seqlens, (__bf16*)a.o, a.ws, a.H, a.L_max,
                           a.splits, c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    return launch_decode_combine_d64(a, stream);
}

hipError_t launch_decode_combine_d64(const DecodeArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(decode_combine_d64_kernel, dim3(a.B * a.H), dim3(64), 0, stream,
                       (const float*)a.ws, (__bf16*)a.o, a.splits);
    return hipGetLastError();
}

}  // namespace plx
