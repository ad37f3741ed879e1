// decode_gqa_bf16.hip -- one Parallax decode step with grouped query heads: G = H_q / H_kv
// query heads share each cache head; bf16 in/out, d_qk = d_v = 128, gfx950.
//
// A decode step has one query row per head, so most rows of a matrix instruction would sit
// idle; Parallax fills them with the probe products [agihunt review, hardware paragraph].
// With grouped heads there are more rows to fill: one v_mfma_f32_16x16x32_bf16 per 16 keys x
// 32 dims takes the cache keys as its 16 rows and the columns [q_0, rho_0, q_1, rho_1, ...,
// q_{G-1}, rho_{G-1}, 0 ...], so the scores and probe products of all G heads cost the same
// instructions as one head (G <= 8).
//
// The value products run on the matrix cores too: O[c][dim] += sum_k P[c][k] V[k][dim] with
// the 16 columns c as the MFMA rows. The k index of a matrix instruction is a sum index, so its
// order is free: k-slot (g, e) of lane group g stands for key 4 g + e (e < 4) or 16 + 4 g + e - 4
// (e >= 4) of the 32-key step, which is exactly what the score accumulators of lane (c, g)
// hold. The weights therefore become the A operand in place, as two bf16 terms (hi and the
// rounding remainder lo, one matrix instruction each), with no lane exchange. V is loaded in the same key order (lane (c, g) loads the 8 keys of its k-slots, 8
// dims each), transposed in registers and stored in LDS as V^T[dim][slot], so each B operand
// read is one 16-byte LDS load.
//
// Per (b, h_kv, chunk) a workgroup of 4 waves streams its keys in 32-key steps (next step's
// loads in flight); each column keeps its own running max (lazy update by 2^8) and the fp32
// sums l = sum w, beta = sum w t. The 4 wave states merge through LDS; with
// one chunk per (b, h_kv) the kernel writes o, otherwise per-query-head partials (the record
// of the split decode) that the split decode's combine kernel merges. The PAGED instance reads
// the cache from a pool of blocks through a per-sequence block table.
#include <type_traits>

#include "plx_device.hpp"
#include "plx_kernels.hpp"

namespace plx {
namespace {

constexpr int NT = 256;
constexpr int NW = 4;
constexpr int KB = 32;       // keys per wave step
constexpr int VTS = KB + 8;  // LDS row stride of V^T (bf16): 80 bytes, conflict-free reads
constexpr float kLazyTau = 8.0f;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// key of k-slot e of lane group g in a 32-key step
__device__ __forceinline__ int slot_key(int g, int e) { return e < 4 ? 4 * g + e : 12 + 4 * g + e; }

// PAGED: the caches are pools of blocks [num_blocks, Hkv, 2^bs_log2, d] and table[b][i] names
// the block of rows i 2^bs_log2 .. of sequence b (blocks of at least 32 rows, so a 32-row step
// never crosses a block). Only blocks holding rows below the chunk end are looked up, one step
// ahead of their loads; an entry outside [0, num_blocks) is never dereferenced and its steps
// are skipped (its rows get no weight).
// D = 128 or 64. At d = 64 a row is 8 chunks of 16 bytes: lanes col < 8 load the V rows of
// k-slots 0..3 of their group and lanes col >= 8 those of k-slots 4..7, chunk col & 7 each.
// DEEP: each wave keeps its next step's loads in flight while it consumes the current one
// (two register sets, two waves per SIMD); without it one step per pass with one register set,
// for chunks of at most one step per wave, where the second set is never used: five waves per
// SIMD at d = 64, three at d = 128 (where the per-wave V^T buffers, 40 KB per workgroup, allow
// three workgroups per compute unit). Same steps in the same order: bit-identical outputs.
template <int D, int G, bool PAGED, bool DEEP>
__global__ __launch_bounds__(NT, DEEP ? 2 : (D == 128 ? 3 : 4)) void decode_gqa_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ rho, const __bf16* __restrict__ kc,
    const __bf16* __restrict__ vc, const int32_t* __restrict__ seqlens, __bf16* __restrict__ o,
    float* __restrict__ ws, int Hkv, int L_max, int S, float c, const int32_t* __restrict__ table,
    int max_blocks, int bs_log2, int num_blocks) {
    static_assert(G >= 1 && G <= 8, "up to 8 query heads per cache head");
    static_assert(D == 128 || D == 64, "head dim");
    constexpr int NS = D / 32;              // 32-dim steps of the scores
    constexpr int NDB = D / 16;             // 16-dim blocks of the value products
    constexpr int NV = D / 16;              // 16-byte V loads per lane and step
    constexpr uint32_t ROWB = 2 * D;        // bytes per cache row
    constexpr int REC = 2 * D + 4;          // split record: A1[D], A2[D], m, l, beta, pad
    __shared__ __attribute__((aligned(16))) __bf16 vt[NW][D * VTS];            // 40 KB at 128
    static_assert(NW * 16 * D * 4 <= (int)sizeof(vt), "merge area");
    __shared__ __attribute__((aligned(16))) float st_m[NW][16], st_l[NW][16];  // per column

    const int s = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, g = lane >> 4;
    const int Hq = Hkv * G;

    int nb = seqlens[b];
    nb = nb < 0 ? 0 : (nb > L_max ? L_max : nb);
    const int chunk = (((nb + S - 1) / S) + KB - 1) / KB * KB;
    const int j0 = s * chunk, j1 = min(j0 + chunk, nb);
    const size_t bk = (size_t)b * Hkv + hk;
    const uint32_t range = j1 > 0 ? (uint32_t)j1 * ROWB : 0u;
    const auto rk = make_rsrc(kc + bk * (size_t)L_max * D, range);
    const auto rv = make_rsrc(vc + bk * (size_t)L_max * D, range);

    // B operand of the scores: column col = 2 gq (q of query head hk G + gq) or 2 gq + 1 (its
    // rho); lane holds dims 32 st + 8 g .. +7. Columns from 2 G on, and rho when absent, are 0.
    bf16x8 bqr[NS];
    {
        const int gq = col >> 1;
        const bool live = gq < G && (!(col & 1) || rho != nullptr);
        const __bf16* src = (col & 1) ? rho : q;
        const auto r = make_rsrc(live ? src + ((size_t)b * Hq + (size_t)hk * G + gq) * D : q,
                                 live ? ROWB : 0u);
#pragma unroll
        for (int st = 0; st < NS; ++st) bqr[st] = as_bf16x8(load16(r, 64u * st + 16u * g));
    }

    f32x4 acc[NDB];  // acc[blk][i]: column 4 g + i, dim 16 blk + col
#pragma unroll
    for (int blk = 0; blk < NDB; ++blk) acc[blk] = f32x4{};
    float m_run = -INFINITY;  // running max of this lane's column's head
    float rsum = 0.f;         // this lane's share of sum w (even columns) or sum w t (odd)

    struct Frag {
        u32x4 k[2][NS];
        u32x4 v[NV];
    };
    // The V rows and the chunk a lane loads: k-slot vslot(e) of its group, chunk vchunk.
    const int vhalf = D == 128 ? 0 : 4 * (col >> 3);
    const int vchunk = D == 128 ? col : (col & 7);
    // Loads of the 32 rows from row r of the resources ck, cv.
    auto load_rows = [&](__amdgpu_buffer_rsrc_t ck, __amdgpu_buffer_rsrc_t cv, int r, Frag& f) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int st = 0; st < NS; ++st)
                f.k[t][st] =
                    load16_nt(ck, (uint32_t)(r + 16 * t + col) * ROWB + 64u * st + 16u * g);
#pragma unroll
        for (int e = 0; e < NV; ++e)
            f.v[e] = load16_nt(cv, (uint32_t)(r + slot_key(g, vhalf + e)) * ROWB + 16u * vchunk);
    };
    // Block of the step at row kb0 (paged caches), or -1 past the chunk.
    auto lookup = [&](int kb0) -> int {
        if constexpr (!PAGED) return 0;
        return kb0 < j1 ? __builtin_amdgcn_readfirstlane(
                              table[(size_t)b * max_blocks + (kb0 >> bs_log2)])
                        : -1;
    };
    // Loads of the step at row kb0: the contiguous cache, or the block that holds it.
    auto load = [&](int kb0, int phys, Frag& f) {
        if constexpr (!PAGED) {
            load_rows(rk, rv, kb0, f);
        } else {
            // The resources span the step's block up to the block's or the chunk's end,
            // whichever comes first.
            uint32_t bytes = 0;
            size_t base = 0;
            const int rel = kb0 & ((1 << bs_log2) - 1);
            if (kb0 < j1 && (unsigned)phys < (unsigned)num_blocks) {
                base = (((size_t)phys * Hkv + hk) << bs_log2) * D;
                bytes = (uint32_t)min(1 << bs_log2, j1 - (kb0 - rel)) * ROWB;
            }
            load_rows(make_rsrc(kc + base, bytes), make_rsrc(vc + base, bytes), rel, f);
        }
    };
    // Whether a step's rows take part: always, or when its block is in the pool (a step of 32
    // rows lies in one block; a step with no weight leaves every sum unchanged).
    auto in_pool = [&](int phys) { return !PAGED || (unsigned)phys < (unsigned)num_blocks; };
    __bf16* vtw = vt[w];
    auto consume = [&](int kb0, const Frag& f) {
        // V^T: lane (col, g) holds dims 8 vchunk .. +7 of its slot keys (slots vhalf ..
        // vhalf + NV - 1 of its group); row 8 vchunk + d gets them at columns 8 g + vhalf ..
        // (two bf16 per dword: slots 2 p, 2 p + 1).
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) {
            uint32_t lo[NV / 2], hi[NV / 2];  // dims 8 vchunk + 2 dd (low halves), + 1 (high)
#pragma unroll
            for (int p = 0; p < NV / 2; ++p) {
                lo[p] = __builtin_amdgcn_perm(f.v[2 * p + 1][dd], f.v[2 * p][dd], 0x05040100u);
                hi[p] = __builtin_amdgcn_perm(f.v[2 * p + 1][dd], f.v[2 * p][dd], 0x07060302u);
            }
            __bf16* r0 = vtw + (8 * vchunk + 2 * dd) * VTS + 8 * g + vhalf;
            if constexpr (NV == 8) {
                *(u32x4*)r0 = u32x4{lo[0], lo[1], lo[2], lo[3]};
                *(u32x4*)(r0 + VTS) = u32x4{hi[0], hi[1], hi[2], hi[3]};
            } else {
                *(u32x2*)r0 = u32x2{lo[0], lo[1]};
                *(u32x2*)(r0 + VTS) = u32x2{hi[0], hi[1]};
            }
        }
        // Scores and probe products: sc[t][i] = key 16 t + 4 g + i, column col.
        f32x4 sc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            sc[t] = f32x4{};
#pragma unroll
            for (int st = 0; st < NS; ++st) sc[t] = mfma16(as_bf16x8(f.k[t][st]), bqr[st], sc[t]);
        }
        // Column max of the scores; odd columns take their head's score column's max.
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                mx = fmaxf(mx, kb0 + 16 * t + 4 * g + i < j1 ? sc[t][i] * c : -INFINITY);
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const float mpart = swap_adjacent(mx);
        const float ms = (col & 1) ? mpart : mx;
        const bool need = ms > m_run + kLazyTau;
        if (wave_any(need)) {
            const float mn = need ? ms : m_run;
            const float alpha = exp2_fast(m_run - mn);
            rsum *= alpha;
            m_run = mn;
            // accumulator register i holds column 4 g + i: its alpha lives in lane 4 g + i
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ai = shfl_xor(alpha, lane ^ (4 * g + i));
#pragma unroll
                for (int blk = 0; blk < NDB; ++blk) acc[blk][i] *= ai;
            }
        }
        // Weights: even columns w = exp2(s c - m), odd columns w t; 0 past the range and for
        // columns beyond the group. Packed in k-slot order: slots e < 4 are tile 0, e >= 4
        // tile 1.
        // Each weight u enters the value products as two bf16 terms, hi = bf16(u) and
        // lo = bf16(u - hi), so the products see u to about 2^-17 relative, and l, beta are
        // the fp32 sums of u itself.
        const bool live_col = col < 2 * G;
        uint32_t pk[4], pl[4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            float u[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float own = sc[t][i];
                const float partner = swap_adjacent(own);
                const float score = (col & 1) ? partner : own;
                const bool valid = live_col && kb0 + 16 * t + 4 * g + i < j1;
                const float wgt = valid ? exp2_fast(fmaf(score, c, -m_run)) : 0.f;
                u[i] = (col & 1) ? wgt * own : wgt;
            }
            rsum += (u[0] + u[1]) + (u[2] + u[3]);
            pk[2 * t] = pack_bf16x2(u[0], u[1]);
            pk[2 * t + 1] = pack_bf16x2(u[2], u[3]);
            pl[2 * t] = pack_bf16x2(u[0] - bf16_lo(pk[2 * t]), u[1] - bf16_hi(pk[2 * t]));
            pl[2 * t + 1] =
                pack_bf16x2(u[2] - bf16_lo(pk[2 * t + 1]), u[3] - bf16_hi(pk[2 * t + 1]));
        }
        const bf16x8 pa = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
        const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pl[0], pl[1], pl[2], pl[3]});
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // O[c][dim] += P[c][slots] V^T[dim][slots]: B operand lane (col = dim, g) reads
        // V^T[16 blk + col][8 g .. 8 g + 7].
#pragma unroll
        for (int blk = 0; blk < NDB; ++blk) {
            const bf16x8 vb = *(const bf16x8*)(vtw + (16 * blk + col) * VTS + 8 * g);
            acc[blk] = mfma16(pa, vb, acc[blk]);
            acc[blk] = mfma16(pb, vb, acc[blk]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    constexpr int STEP = KB * NW;
    Frag fa, fb;
    int kb0 = j0 + KB * w;
    if constexpr (!DEEP) {
        for (; kb0 < j1; kb0 += STEP) {
            const int ph = lookup(kb0);
            load(kb0, ph, fa);
            if (in_pool(ph)) consume(kb0, fa);
        }
    } else {
        int pha = lookup(kb0);
        if (kb0 < j1) load(kb0, pha, fa);
        int ph1 = lookup(kb0 + STEP);
        for (; kb0 < j1; kb0 += 2 * STEP) {
            load(kb0 + STEP, ph1, fb);
            const int phb = ph1;
            const int ph2 = lookup(kb0 + 2 * STEP);
            if (in_pool(pha)) consume(kb0, fa);
            if (kb0 + STEP >= j1) break;
            load(kb0 + 2 * STEP, ph2, fa);
            pha = ph2;
            ph1 = lookup(kb0 + 3 * STEP);
            if (in_pool(phb)) consume(kb0 + STEP, fb);
        }
    }

    // Column totals of the weights (over the 4 row groups).
    rsum += shfl_xor(rsum, 16);
    rsum += shfl_xor(rsum, 32);
    if (g == 0) {
        st_m[w][col] = m_run;
        st_l[w][col] = rsum;
    }
    __syncthreads();
    // Merge the 4 wave states into wave 0's LDS area, reusing the V^T buffers:
    // O[w][c][dim] as floats (16 x 128 per wave = 8 KB).
    float* ow = reinterpret_cast<float*>(&vt[0][0]);  // [NW][16][D]
    __syncthreads();
#pragma unroll
    for (int blk = 0; blk < NDB; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) ow[(w * 16 + 4 * g + i) * D + 16 * blk + col] = acc[blk][i];
    __syncthreads();
    // Thread tid handles dims 2 (tid % TPH) .. +1 of query heads tid / TPH, + NT / TPH, ...
    constexpr int TPH = D / 2;  // threads per query head
    for (int gq = tid / TPH; gq < G; gq += NT / TPH) {
        const int d0 = 2 * (tid % TPH);
        float M = -INFINITY;
#pragma unroll
        for (int v = 0; v < NW; ++v) M = fmaxf(M, st_m[v][2 * gq]);
        float l = 0.f, beta = 0.f, a1x = 0.f, a1y = 0.f, a2x = 0.f, a2y = 0.f;
        if (M > -INFINITY) {
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                const float mv = st_m[v][2 * gq];
                const float f = mv > -INFINITY ? exp2_fast(mv - M) : 0.f;
                l = fmaf(f, st_l[v][2 * gq], l);
                beta = fmaf(f, st_l[v][2 * gq + 1], beta);
                const float* o1 = ow + (v * 16 + 2 * gq) * D + d0;
                const float* o2 = ow + (v * 16 + 2 * gq + 1) * D + d0;
                a1x = fmaf(f, o1[0], a1x);
                a1y = fmaf(f, o1[1], a1y);
                a2x = fmaf(f, o2[0], a2x);
                a2y = fmaf(f, o2[1], a2y);
            }
        }
        const size_t bh = (size_t)b * Hq + (size_t)hk * G + gq;
        if (S == 1) {
            float yx = 0.f, yy = 0.f;
            if (l > 0.f) {
                const float inv = 1.f / l;
                yx = inv * (a1x * (1.f + beta * inv) - a2x);
                yy = inv * (a1y * (1.f + beta * inv) - a2y);
            }
            *(uint32_t*)(o + bh * D + d0) = pack_bf16x2(yx, yy);
        } else {
            float* rec = ws + (bh * (size_t)S + s) * REC;
            *(float2*)(rec + d0) = float2{a1x, a1y};
            *(float2*)(rec + D + d0) = float2{a2x, a2y};
            if (d0 == 0) *(f32x4*)(rec + 2 * D) = f32x4{M, l, beta, 0.f};
        }
    }
}

}  // namespace

hipError_t launch_decode_gqa_bf16(const DecodeArgs& a, int Hkv, hipStream_t stream) {
    const int G = a.H / Hkv;
    dim3 grid(a.splits, Hkv, a.B);
    const float c = a.scale * kLog2e;
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, grid, dim3(NT), 0, stream, (const __bf16*)a.q,
                           (const __bf16*)a.rho, (const __bf16*)a.k, (const __bf16*)a.v,
                           a.seqlens, (__bf16*)a.o, a.ws, Hkv, a.L_max, a.splits, c, a.table,
                           a.max_blocks, a.block_log2, a.num_blocks);
    };
    // Chunks of at most one step per wave run the one-register-set instance (the kernel's
    // chunk of a sequence is at most that of L_max).
    const bool deep = ((a.L_max + a.splits - 1) / a.splits + KB - 1) / KB * KB > KB * NW;
    auto pick = [&](auto d_tag, auto g_tag) {
        constexpr int DD = decltype(d_tag)::value, GG = decltype(g_tag)::value;
        if (a.table)
            deep ? go(decode_gqa_bf16_kernel<DD, GG, true, true>)
                 : go(decode_gqa_bf16_kernel<DD, GG, true, false>);
        else
            deep ? go(decode_gqa_bf16_kernel<DD, GG, false, true>)
                 : go(decode_gqa_bf16_kernel<DD, GG, false, false>);
    };
    auto by_g = [&](auto d_tag) {
        switch (G) {
            case 1: pick(d_tag, std::integral_constant<int, 1>{}); return true;
            case 2: pick(d_tag, std::integral_constant<int, 2>{}); return true;
            case 4: pick(d_tag, std::integral_constant<int, 4>{}); return true;
            case 8: pick(d_tag, std::integral_constant<int, 8>{}); return true;
            default: return false;
        }
    };
    bool ok = false;
    if (a.d == 128) ok = by_g(std::integral_constant<int, 128>{});
    else if (a.d == 64) ok = by_g(std::integral_constant<int, 64>{});
    if (!ok) return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    return a.d == 64 ? launch_decode_combine_d64(a, stream) : launch_decode_combine(a, stream);
}

}  // namespace plx
