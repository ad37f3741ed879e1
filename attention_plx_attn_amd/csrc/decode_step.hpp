// decode_step.hpp -- the per-wave streaming step shared by the Parallax decode kernels
// (bf16 in, d_qk = d_v = 128, gfx950).
//
// One wave consumes KB = 32 cache rows of one (b, h) per step:
//  * scores: each 16-row key tile is one v_mfma_f32_16x16x32_bf16 per 32 dims with the keys as
//    the 16 rows and the columns [q, rho, 0 ... 0], so column 0 holds q.k and column 1 the
//    probe products t = rho.k [agihunt review, hardware paragraph: a decode step has one
//    query row, so Parallax puts the probe products into accumulator rows that would
//    otherwise sit idle];
//  * online softmax with a wave-uniform running max (one rescale when it grows);
//  * the weights w and w*t stay fp32 (the value products run on the VALU), are summed into
//    l and beta, and are handed through LDS to the value layout, where each lane accumulates
//    A1 = sum w v and A2 = sum w t v for 8 dims over 8 of the step's rows.
// Loads use raw buffer resources: rows at or beyond the resource's range read as zero
// without touching memory, which masks sequence ends and empty prefetches.
#pragma once

#include "plx_device.hpp"

namespace plx {
namespace decode {

constexpr int D = 128;
constexpr int KB = 32;      // keys per wave step
constexpr int KT = KB / 16; // score tiles per step
constexpr int VR = KB / 4;  // value rows per lane per step
constexpr int NW = 4;       // waves per workgroup
constexpr int NT = 64 * NW;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Registers of one step in flight.
struct Frag {
    u32x4 k[KT][4];  // K rows 16 t + col, dims 32 st + 8 g .. +7 (A operand of the score tile)
    u32x4 v[VR];     // V rows VR g + r, dims 8 col .. +7
};

// Running state of one wave over one piece of a (b, h) key range.
struct Acc {
    float m_run;  // running max of the log2-domain scores
    float rsum;   // sum of the weights: l in column-0 lanes, beta in column-1 lanes
    float a1[8], a2[8];

    __device__ __forceinline__ void reset() {
        m_run = -INFINITY;
        rsum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a1[e] = a2[e] = 0.f;
    }
};

// Issue the loads of rows [kb0, kb0 + KB): lane (col, g) fetches 64-byte K row segments
// (4 lanes per 256-byte row) and 16-byte V row pieces (16 lanes per row).
__device__ __forceinline__ void load_step(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                          int kb0, int col, int g, Frag& f) {
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int st = 0; st < 4; ++st)
            f.k[t][st] =
                load16_nt(rk, (uint32_t)(kb0 + 16 * t + col) * 256u + 64u * st + 16u * g);
#pragma unroll
    for (int r = 0; r < VR; ++r)
        f.v[r] = load16_nt(rv, (uint32_t)(kb0 + VR * g + r) * 256u + 16u * col);
}

// B operand [q | rho | 0 ...]: lane (col, g) holds dims 32 st + 8 g .. +7 of column col.
// Lanes of other columns read past the 256-byte ranges and get zeros.
__device__ __forceinline__ void load_qr(__amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rr,
                                        int col, int g, bf16x8 (&bqr)[4]) {
    const uint32_t oq = col == 0 ? 16u * g : 1024u;
    const uint32_t orr = col == 1 ? 16u * g : 1024u;
#pragma unroll
    for (int st = 0; st < 4; ++st)
        bqr[st] = as_bf16x8(load16(rq, oq + 64u * st) | load16(rr, orr + 64u * st));
}

// Consume the step whose loads are in f: rows kb0 + ... count while below je.
// ush: this wave's [2][KB] LDS exchange area (fp32 w and w t per row).
// PROBE = false is the softmax-only specialisation (rho = 0 exactly, column 1 of bqr zero):
// A2 stays 0 and is not accumulated; every other value is computed as with PROBE and rho = 0.
template <bool PROBE>
__device__ __forceinline__ void consume(Acc& s, const Frag& f, const bf16x8 (&bqr)[4], int kb0,
                                        int je, float c, float (*ush)[KB], int col, int g) {
    // Score tile: row = key (16 per tile), column 0 = q.k, column 1 = rho.k.
    f32x4 sc[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) {
        sc[t] = f32x4{};
#pragma unroll
        for (int st = 0; st < 4; ++st) sc[t] = mfma16(as_bf16x8(f.k[t][st]), bqr[st], sc[t]);
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

    // Value accumulation: lane (col, g) takes rows kb0 + VR g .. +VR-1, dims 8 col .. +7.
#pragma unroll
    for (int r4 = 0; r4 < VR / 4; ++r4) {
        const f32x4 u0 = *(const f32x4*)&ush[0][VR * g + 4 * r4];
        const f32x4 u1 = PROBE ? *(const f32x4*)&ush[1][VR * g + 4 * r4] : f32x4{};
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

// Wave totals: values over the 4 row groups (lanes 0..15 then hold dims 8 col .. +7), l in
// lane 0 and beta in lane 1.
template <bool PROBE>
__device__ __forceinline__ void wave_totals(Acc& s) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        s.a1[e] += shfl_xor(s.a1[e], 16);
        s.a1[e] += shfl_xor(s.a1[e], 32);
        if constexpr (PROBE) {
            s.a2[e] += shfl_xor(s.a2[e], 16);
            s.a2[e] += shfl_xor(s.a2[e], 32);
        }
    }
    s.rsum += shfl_xor(s.rsum, 16);
    s.rsum += shfl_xor(s.rsum, 32);
}

}  // namespace decode
}  // namespace plx
