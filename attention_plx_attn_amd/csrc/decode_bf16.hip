// decode_bf16.hip -- one Parallax decode step over a contiguous per-sequence KV cache,
// bf16 in/out, d_qk = d_v = 128, gfx950.
//
// Design points taken from the pages and re-made for CDNA4:
//  * QK and RK in one matrix instruction [agihunt review, hardware paragraph: a decode step
//    has one query row, so most accumulator rows of a matrix instruction sit idle; Parallax
//    puts the probe products in the same instruction]. Here each 16-key tile is one
//    v_mfma_f32_16x16x32_bf16 per 32 dims with the cache keys as the 16 rows and the
//    columns [q, rho, 0 ... 0]: column 0 yields the scores, column 1 the probe products t,
//    at no extra instruction cost.
//  * Persistent KV-loop splitting with a reduction of the partials [Parallax
//    (paper.rainbus.top summary), reproducibility section: the decode kernel's optimisations
//    are instruction sharing, KV-loop splitting and the reduction of the split partials].
//    Each workgroup streams one chunk of one (b, h) and writes its partial state
//    (m, l, beta, A1 = sum w v, A2 = sum w t v); a second kernel merges the partials with
//    one rescale each and applies o = (A1/l)(1 + beta/l) - A2/l. With one chunk per (b, h)
//    the first kernel writes o directly.
//  * Decode is bound by HBM bandwidth: the cache is read once with non-temporal 16-byte
//    buffer loads (every K load is a contiguous 64-byte row segment per 4 lanes, every V
//    load a 256-byte row per 16 lanes). A wave step covers 32 keys (16 KiB) and the loads
//    of the next step are issued before the current one is consumed, so each wave keeps
//    up to 32 KiB in flight; the split heuristic aims at one such 4-wave workgroup per
//    compute unit, which measured best on MI355X. The buffer range ends at the chunk's
//    last valid row, so rows at or beyond seqlens are never read (they come back as zeros
//    and get zero weight).
// Softmax weights and weight*probe products are rounded to bf16 and the sums l and beta are
// taken from the rounded values, as in the prefill kernel.
#include "plx_device.hpp"
#include "plx_kernels.hpp"

namespace plx {
namespace {

constexpr int D = 128;
constexpr int NT = 256;  // 4 waves
constexpr int NW = 4;
constexpr int REC = kDecodeRecord;
#ifndef PLX_DECODE_KB
#define PLX_DECODE_KB 32
#endif

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// KB: keys per wave per step (a multiple of 16); KT = KB / 16 score tiles per step; each
// lane group of 16 lanes accumulates KB / 4 value rows per step.
template <int KB>
__global__ __launch_bounds__(NT, KB <= 32 ? 2 : 1) void decode_split_bf16_d128_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ rho, const __bf16* __restrict__ kc,
    const __bf16* __restrict__ vc, const int32_t* __restrict__ seqlens, __bf16* __restrict__ o,
    float* __restrict__ ws, int H, int L_max, int S, float c) {
    __shared__ __attribute__((aligned(16))) float ush[NW][2][KB];  // rounded w and w t per key
    __shared__ __attribute__((aligned(16))) float red[NW][2 * D + 4];

    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int col = lane & 15;  // column of the score tile (0: q, 1: rho); V: dims 8 col ..
    const int g = lane >> 4;    // row group of the score tile; V: key sub-range

    int nb_keys = seqlens[b];
    nb_keys = nb_keys < 0 ? 0 : (nb_keys > L_max ? L_max : nb_keys);
    // The S chunks of this sequence split its own length (not L_max) evenly, in whole wave
    // steps, so that ragged batches keep every split busy; trailing chunks may be empty.
    const int chunk = (((nb_keys + S - 1) / S) + KB - 1) / KB * KB;
    const int j0 = s * chunk;
    const int j1 = min(j0 + chunk, nb_keys);
    const size_t bh = (size_t)b * H + h;
    const __bf16* kbase = kc + bh * (size_t)L_max * D;
    const __bf16* vbase = vc + bh * (size_t)L_max * D;
    const uint32_t range = j1 > 0 ? (uint32_t)j1 * 256u : 0u;
    const auto rk = make_rsrc(kbase, range);
    const auto rv = make_rsrc(vbase, range);

    // B operand [q | rho | 0...]: lane holds dims 32 st + 8 g .. +7 of column `col`.
    bf16x8 bqr[4];
    {
        const auto rq = make_rsrc(q + bh * D, 256u);
        const auto rr = make_rsrc(rho + bh * D, 256u);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const u32x4 xq = load16(rq, 64u * st + 16u * g);
            const u32x4 xr = load16(rr, 64u * st + 16u * g);
            bqr[st] = as_bf16x8(col == 0 ? xq : (col == 1 ? xr : u32x4{}));
        }
    }

    float m_run = -INFINITY;
    float rsum = 0.f;  // sum of rounded weights: l in column-0 lanes, beta in column-1 lanes
    float a1[8], a2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) a1[e] = a2[e] = 0.f;

    // Software pipeline over this wave's steps: the loads of step n + 1 are issued before
    // step n is consumed (two register sets, so the loop is unrolled by two). A prefetch
    // past the chunk reads beyond the buffer range and returns zeros without touching memory.
    constexpr int KT = KB / 16, VR = KB / 4;
    auto load_step = [&](int kb0, u32x4 (&kf)[KT][4], u32x4 (&vf)[VR]) {
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int st = 0; st < 4; ++st)
                kf[t][st] = load16_nt(rk, (uint32_t)(kb0 + 16 * t + col) * 256u + 64u * st + 16u * g);
#pragma unroll
        for (int r = 0; r < VR; ++r)
            vf[r] = load16_nt(rv, (uint32_t)(kb0 + VR * g + r) * 256u + 16u * col);
    };
    auto consume = [&](int kb0, const u32x4 (&kf)[KT][4], const u32x4 (&vf)[VR]) {
        // Score tile: row = key (16 per tile), column 0 = q.k, column 1 = rho.k.
        f32x4 sc[KT];
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            sc[t] = f32x4{};
#pragma unroll
            for (int st = 0; st < 4; ++st) sc[t] = mfma16(as_bf16x8(kf[t][st]), bqr[st], sc[t]);
        }
        // Lane (col, g) register i holds key kb0 + 16 t + 4 g + i.
        float mx = -INFINITY;
        if (col == 0) {
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (kb0 + 16 * t + 4 * g + i < j1) mx = fmaxf(mx, sc[t][i] * c);
        }
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const float mb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), 0));
        if (mb > m_run) {  // wave-uniform
            const float alpha = exp2_fast(m_run - mb);
            rsum *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                a1[e] *= alpha;
                a2[e] *= alpha;
            }
            m_run = mb;
        }

        // Column 0 lanes: w; column 1 lanes: w t (score from the adjacent column-0 lane).
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            float u[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float own = sc[t][i];
                // DPP must run with every lane active: take the neighbour's value first.
                const float partner = swap_adjacent(own);
                const float score = col == 1 ? partner : own;
                const bool valid = kb0 + 16 * t + 4 * g + i < j1;
                const float wgt = valid ? exp2_fast(fmaf(score, c, -m_run)) : 0.f;
                u[i] = col == 0 ? wgt : (col == 1 ? wgt * own : 0.f);
            }
            const uint32_t p01 = pack_bf16x2(u[0], u[1]);
            const uint32_t p23 = pack_bf16x2(u[2], u[3]);
            rsum = add_bf16x2(p23, add_bf16x2(p01, rsum));
            if (col < 2)
                *(f32x4*)&ush[w][col][16 * t + 4 * g] =
                    f32x4{bf16_lo(p01), bf16_hi(p01), bf16_lo(p23), bf16_hi(p23)};
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // Value accumulation: lane (col, g) takes keys kb0 + VR g .. +VR-1, dims 8 col .. +7.
#pragma unroll
        for (int r4 = 0; r4 < VR / 4; ++r4) {
            const f32x4 u0 = *(const f32x4*)&ush[w][0][VR * g + 4 * r4];
            const f32x4 u1 = *(const f32x4*)&ush[w][1][VR * g + 4 * r4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const u32x4 x = vf[4 * r4 + rr];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const float vlo = bf16_lo(x[p]), vhi = bf16_hi(x[p]);
                    a1[2 * p] = fmaf(u0[rr], vlo, a1[2 * p]);
                    a1[2 * p + 1] = fmaf(u0[rr], vhi, a1[2 * p + 1]);
                    a2[2 * p] = fmaf(u1[rr], vlo, a2[2 * p]);
                    a2[2 * p + 1] = fmaf(u1[rr], vhi, a2[2 * p + 1]);
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    constexpr int STEP = KB * NW;
    u32x4 kfA[KT][4], vfA[VR], kfB[KT][4], vfB[VR];
    int kb0 = j0 + KB * w;
    if (kb0 < j1) load_step(kb0, kfA, vfA);
    for (; kb0 < j1; kb0 += 2 * STEP) {
        load_step(kb0 + STEP, kfB, vfB);
        consume(kb0, kfA, vfA);
        if (kb0 + STEP >= j1) break;
        load_step(kb0 + 2 * STEP, kfA, vfA);
        consume(kb0 + STEP, kfB, vfB);
    }

    // Wave totals: values over the 4 key sub-ranges; l and beta over the 4 row groups.
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a1[e] += shfl_xor(a1[e], 16);
        a1[e] += shfl_xor(a1[e], 32);
        a2[e] += shfl_xor(a2[e], 16);
        a2[e] += shfl_xor(a2[e], 32);
    }
    rsum += shfl_xor(rsum, 16);
    rsum += shfl_xor(rsum, 32);
    if (lane < 16) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            red[w][8 * lane + e] = a1[e];
            red[w][D + 8 * lane + e] = a2[e];
        }
    }
    if (lane == 0) {
        red[w][2 * D] = m_run;
        red[w][2 * D + 1] = rsum;
    }
    if (lane == 1) red[w][2 * D + 2] = rsum;
    __syncthreads();

    // Merge the 4 wave states (one rescale each); thread tid < 128 owns dim tid.
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
            float y = 0.f;
            if (l > 0.f) {
                const float inv = 1.f / l;
                y = inv * (A1 * (1.f + beta * inv) - A2);
            }
            o[bh * D + tid] = (__bf16)y;
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

// One workgroup per (b, h). Wave w folds the partials s = w, w + 4, ... with an online
// max/rescale, issuing the loads of a batch of 8 partials before using any of them (one
// memory round trip per batch); lane owns dims 2 lane, 2 lane + 1. The four wave states are
// then merged through LDS with one rescale each.
__global__ __launch_bounds__(NT) void decode_combine_kernel(const float* __restrict__ ws,
                                                            __bf16* __restrict__ o, int S) {
    constexpr int BATCH = 8;
    __shared__ __attribute__((aligned(16))) float reds[NW][2 * D + 4];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const size_t bh = blockIdx.x;
    const float* base = ws + bh * (size_t)S * REC;

    float m = -INFINITY, l = 0.f, beta = 0.f, a1x = 0.f, a1y = 0.f, a2x = 0.f, a2y = 0.f;
    for (int s0 = w; s0 < S; s0 += NW * BATCH) {
        float ms[BATCH], ls[BATCH], bs[BATCH];
        float2 x1[BATCH], x2[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int s = s0 + NW * u;
            const float* rec = base + (size_t)min(s, S - 1) * REC;
            ms[u] = s < S ? rec[2 * D] : -INFINITY;
            ls[u] = rec[2 * D + 1];
            bs[u] = rec[2 * D + 2];
            x1[u] = *(const float2*)(rec + 2 * lane);
            x2[u] = *(const float2*)(rec + D + 2 * lane);
        }
        float mb = m;
#pragma unroll
        for (int u = 0; u < BATCH; ++u) mb = fmaxf(mb, ms[u]);
        if (mb == -INFINITY) continue;  // nothing non-empty yet (wave-uniform)
        const float fo = m > -INFINITY ? exp2_fast(m - mb) : 0.f;
        l *= fo;
        beta *= fo;
        a1x *= fo;
        a1y *= fo;
        a2x *= fo;
        a2y *= fo;
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const float f = ms[u] > -INFINITY ? exp2_fast(ms[u] - mb) : 0.f;  // empty: 0
            l = fmaf(f, ls[u], l);
            beta = fmaf(f, bs[u], beta);
            a1x = fmaf(f, x1[u].x, a1x);
            a1y = fmaf(f, x1[u].y, a1y);
            a2x = fmaf(f, x2[u].x, a2x);
            a2y = fmaf(f, x2[u].y, a2y);
        }
        m = mb;
    }
    *(float2*)&reds[w][2 * lane] = float2{a1x, a1y};
    *(float2*)&reds[w][D + 2 * lane] = float2{a2x, a2y};
    if (lane == 0) {
        reds[w][2 * D] = m;
        reds[w][2 * D + 1] = l;
        reds[w][2 * D + 2] = beta;
    }
    __syncthreads();
    if (w == 0) {
        float M = -INFINITY;
#pragma unroll
        for (int i = 0; i < NW; ++i) M = fmaxf(M, reds[i][2 * D]);
        float L = 0.f, Bt = 0.f, A1x = 0.f, A1y = 0.f, A2x = 0.f, A2y = 0.f;
        if (M > -INFINITY) {
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                const float mi = reds[i][2 * D];
                const float f = mi > -INFINITY ? exp2_fast(mi - M) : 0.f;
                L = fmaf(f, reds[i][2 * D + 1], L);
                Bt = fmaf(f, reds[i][2 * D + 2], Bt);
                A1x = fmaf(f, reds[i][2 * lane], A1x);
                A1y = fmaf(f, reds[i][2 * lane + 1], A1y);
                A2x = fmaf(f, reds[i][D + 2 * lane], A2x);
                A2y = fmaf(f, reds[i][D + 2 * lane + 1], A2y);
            }
        }
        float yx = 0.f, yy = 0.f;
        if (L > 0.f) {
            const float inv = 1.f / L;
            const float one_tb = 1.f + Bt * inv;
            yx = inv * (A1x * one_tb - A2x);
            yy = inv * (A1y * one_tb - A2y);
        }
        *(uint32_t*)(o + bh * D + 2 * lane) = pack_bf16x2(yx, yy);
    }
}

}  // namespace

hipError_t launch_decode_bf16_d128(const DecodeArgs& a, hipStream_t stream) {
    dim3 grid(a.splits, a.H, a.B);
    hipLaunchKernelGGL(decode_split_bf16_d128_kernel<PLX_DECODE_KB>, grid, dim3(NT), 0, stream,
                       (const __bf16*)a.q, (const __bf16*)a.rho, (const __bf16*)a.k,
                       (const __bf16*)a.v, a.seqlens, (__bf16*)a.o, a.ws, a.H, a.L_max, a.splits,
                       a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    const int BH = a.B * a.H;
    hipLaunchKernelGGL(decode_combine_kernel, dim3(BH), dim3(NT), 0, stream, (const float*)a.ws,
                       (__bf16*)a.o, a.splits);
    return hipGetLastError();
}

}  // namespace plx
