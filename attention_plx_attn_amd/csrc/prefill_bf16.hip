// prefill_bf16.hip -- causal Parallax prefill, bf16 in/out, d_qk = d_v = 128, gfx950.
//
// Method [Parallax (paper.rainbus.top summary), "方法步骤详情": per KV block compute the
// scores S1 = Q K^T and the probe products S2 = R K^T sharing one matrix instruction's
// operand, then P1 = exp(S1 - m) and P2 = P1 * S2, and accumulate O1 += P1 V and O2 += P2 V
// in parallel; agihunt review, hardware paragraph: both branches share one KV stream, one
// running max and one rescale factor]. Final combine o = (1 + tbar) O1 - O2 with
// tbar = sum P2 / sum P1 (method step 6).
//
// Work decomposition (one workgroup = 4 waves = 128 query rows of one (b, h)):
//   * every wave owns 32 query rows; its Q and R fragments stay in registers as the
//     B operand of v_mfma_f32_32x32x16_bf16, so the product tile is S^T = K [Q|R]^T with
//     keys on the 32 rows and the wave's queries on the 32 lanes of each half-wave;
//   * K and V tiles of 64 keys are staged in LDS, double-buffered: K row-major (rows stored
//     in a permuted order, below), V transposed (d rows x 64 keys) so that a value operand
//     is one 16-byte LDS read. In the transposed tile the 16-byte key chunk of dim row d is
//     XOR-swizzled with bits 4..6 of d: the transposing 8-byte stores of 16 lanes (16 dims
//     8 apart) would otherwise all hit one bank pair. gfx950's LDS serves 16 lanes of a
//     16-byte access per clock over 64 banks; with the 144-byte row pitch and this swizzle
//     both the stores and the operand reads are conflict-free;
//   * the score tile's accumulator layout is reused directly as the P operand of the value
//     products O^T += V^T P^T: storing key rows with bits 2 and 3 of the row index swapped
//     makes each lane's eight consecutive accumulator registers hold eight consecutive
//     keys, exactly the operand layout, so no cross-lane traffic is needed;
//   * lane <-> query throughout, so max, rescale and normaliser stay lane-local except one
//     exchange with the other half-wave per tile (the two halves hold the two key halves);
//   * P1 and P2 are rounded to bf16 and the sums l = sum P1, beta = sum P2 are taken from
//     the rounded values, so the effective corrected weights sum to exactly one;
//   * the running max is updated lazily (only when a row's tile max exceeds it by more than
//     2^8); the result is the same exact expression, with far fewer rescales.
// Workgroups are issued longest query block first; with B*H a multiple of 8 all blocks of
// one (b, h) land on the same XCD (dispatch is round-robin over the 8 XCDs), so its K/V
// stay in that XCD's L2.
#include <type_traits>

#include "plx_device.hpp"
#include "plx_kernels.hpp"

namespace plx {
namespace {

constexpr int D = 128;
constexpr int BR = 128;  // query rows per workgroup
constexpr int BC = 64;   // keys per LDS tile
constexpr int NT = 256;  // threads per workgroup (4 waves)
constexpr int KS = D + 8;               // LDS row stride of the K tile (bf16 elements)
constexpr int VS = BC + 8;              // LDS row stride of the transposed V tile
constexpr int K_ELEMS = BC * KS;        // 8704
constexpr int V_ELEMS = D * VS;         // 9216
constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
constexpr float kLazyTau = 8.0f;        // log2 headroom before the running max moves

// Row order inside each 32-key half of a K tile: bits 2 and 3 swapped (an involution).
__device__ __forceinline__ int perm_row(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(NT, 1) void prefill_bf16_d128_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ rho, __bf16* __restrict__ o, int BH, int T, int nqb, float c) {
    __shared__ __attribute__((aligned(16))) __bf16 lds[2 * BUF_ELEMS];

    const int wid = blockIdx.x;
    const int bh = wid % BH;
    const int qb = nqb - 1 - wid / BH;  // longest query blocks first
    const int q0 = qb * BR;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int n = lane & 31;  // query within the wave's 32 rows
    const int h = lane >> 5;  // half-wave: which 8-element k-slice of an operand

    const size_t slice = (size_t)bh * (size_t)T * D;
    const uint32_t slice_bytes = (uint32_t)T * D * 2u;
    const auto rq = make_rsrc(q + slice, slice_bytes);
    const auto rr = make_rsrc(rho + slice, slice_bytes);
    const auto rk = make_rsrc(k + slice, slice_bytes);
    const auto rv = make_rsrc(v + slice, slice_bytes);

    // Q and R fragments: B operand, lane holds dims 16 s + 8 h .. +7 of its query row.
    const int qrow = q0 + 32 * w + n;
    bf16x8 qf[8], rf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const uint32_t off = (uint32_t)qrow * 256u + 32u * s + 16u * h;
        qf[s] = as_bf16x8(load16(rq, off));
        rf[s] = as_bf16x8(load16(rr, off));
    }

    const int kend = min(q0 + BR, T);
    const int ntiles = (kend + BC - 1) / BC;

    f32x16 acc1[4], acc2[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        acc1[nb] = f32x16{};
        acc2[nb] = f32x16{};
    }
    float m_run = -INFINITY, lsum = 0.f, bsum = 0.f;

    // ---- global -> registers -> LDS staging of one 64-key tile
    u32x4 kst[4], vst[4];
    const int vdc = tid & 15;  // V: dims 8 vdc .. +7
    const int vkg = tid >> 4;  // V: keys 4 vkg .. +3
    auto gload = [&](int kt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int chunk = tid + NT * j;
            const int row = chunk >> 4, col = chunk & 15;
            kst[j] = load16(rk, (uint32_t)(kt * BC + row) * 256u + 16u * col);
            vst[j] = load16(rv, (uint32_t)(kt * BC + 4 * vkg + j) * 256u + 16u * vdc);
        }
    };
    auto lstore = [&](int buf) {
        __bf16* Kl = lds + buf * BUF_ELEMS;
        __bf16* Vl = Kl + K_ELEMS;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int chunk = tid + NT * j;
            const int row = chunk >> 4, col = chunk & 15;
            const int prow = (row & 32) | perm_row(row & 31);
            *(u32x4*)(Kl + prow * KS + col * 8) = kst[j];
        }
        // Transpose 4 keys x 8 dims into 8 dims x 4 keys (byte permutes), 8-byte stores.
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t lo01 = __builtin_amdgcn_perm(vst[1][p], vst[0][p], 0x05040100u);
            const uint32_t lo23 = __builtin_amdgcn_perm(vst[3][p], vst[2][p], 0x05040100u);
            const uint32_t hi01 = __builtin_amdgcn_perm(vst[1][p], vst[0][p], 0x07060302u);
            const uint32_t hi23 = __builtin_amdgcn_perm(vst[3][p], vst[2][p], 0x07060302u);
            const int d0 = 8 * vdc + 2 * p;  // d0 and d0 + 1 share bits 4..6 (= vdc >> 1)
            const int cs = 8 * ((vkg >> 1) ^ ((vdc >> 1) & 7)) + 4 * (vkg & 1);
            *(u32x2*)(Vl + d0 * VS + cs) = u32x2{lo01, lo23};
            *(u32x2*)(Vl + (d0 + 1) * VS + cs) = u32x2{hi01, hi23};
        }
    };

    const int qi = q0 + 32 * w + n;

    // One 64-key tile: scores on the shared K operand, online softmax with the lazy
    // running max, value products on the shared V operand. DIAG: the tile reaches past
    // some row of the block, so keys after the row are masked (weight exactly 0).
    auto tile = [&](int kt, auto diag_tag) {
        constexpr bool DIAG = decltype(diag_tag)::value;
        const __bf16* Kl = lds + (kt & 1) * BUF_ELEMS;
        const __bf16* Vl = Kl + K_ELEMS;
#pragma unroll
        for (int hc = 0; hc < 2; ++hc) {
            f32x16 S = f32x16{}, Tt = f32x16{};
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const bf16x8 kf = *(const bf16x8*)(Kl + (32 * hc + n) * KS + 16 * s + 8 * h);
                S = mfma32(kf, qf[s], S);
                Tt = mfma32(kf, rf[s], Tt);
            }
            // Register i of this half-wave holds key 64 kt + 32 hc + perm_row(8 (i/4) + 4 h + i%4).
            if constexpr (DIAG) {
                const int lim = qi - (kt * BC + 32 * hc);
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (perm_row(8 * (i >> 2) + 4 * h + (i & 3)) > lim) S[i] = -INFINITY;
            }
            float mt = S[0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mt = fmaxf(mt, S[i]);
            mt = fmaxf(mt, shfl_xor(mt, 32));
            const float ms = mt > -INFINITY ? mt * c : -INFINITY;

            const bool need = ms > m_run + kLazyTau;
            if (wave_any(need)) {
                const float mn = need ? ms : m_run;
                const float alpha = exp2_fast(m_run - mn);
                lsum *= alpha;
                bsum *= alpha;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    acc1[nb] *= alpha;
                    acc2[nb] *= alpha;
                }
                m_run = mn;
            }

            // P1 = exp2(S c - m), P2 = P1 * T, rounded to bf16 (row sums from the rounded
            // values), then O1^T += V^T P1^T and O2^T += V^T P2^T on a shared V operand.
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                float wv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    wv[e] = exp2_fast(fmaf(S[8 * r + e], c, -m_run));
                    if constexpr (DIAG) wv[e] = S[8 * r + e] == -INFINITY ? 0.f : wv[e];
                }
                u32x4 pw, p2w;
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    pw[e >> 1] = pack_bf16x2(wv[e], wv[e + 1]);
                    p2w[e >> 1] = pack_bf16x2(wv[e] * Tt[8 * r + e], wv[e + 1] * Tt[8 * r + e + 1]);
                    lsum = add_bf16x2(pw[e >> 1], lsum);
                    bsum = add_bf16x2(p2w[e >> 1], bsum);
                }
                const bf16x8 pf = as_bf16x8(pw), p2f = as_bf16x8(p2w);
                const int ks = 2 * hc + r;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    const int vr = 32 * nb + n;
                    const bf16x8 vf =
                        *(const bf16x8*)(Vl + vr * VS + 8 * ((2 * ks + h) ^ ((vr >> 4) & 7)));
                    acc1[nb] = mfma32(vf, pf, acc1[nb]);
                    acc2[nb] = mfma32(vf, p2f, acc2[nb]);
                }
            }
        }
        // Stage the next tile (prefetched into registers at the top of the iteration).
        lstore((kt & 1) ^ 1);
        __syncthreads();
    };

    gload(0);
    lstore(0);
    __syncthreads();
    // Tiles entirely below the block's first row need no mask; the last one or two do.
    // The next tile is prefetched unconditionally: after the last tile this reads one
    // tile past the block (zeros past T through the buffer range) into an LDS buffer
    // nobody reads again, which keeps branches out of the loop body.
    const int nfull = min(ntiles, q0 / BC);
    for (int kt = 0; kt < nfull; ++kt) {
        gload(kt + 1);
        tile(kt, std::false_type{});
    }
    for (int kt = nfull; kt < ntiles; ++kt) {
        gload(kt + 1);
        tile(kt, std::true_type{});
    }

    // Epilogue: combine the half-waves' sums, o = (A1/l)(1 + beta/l) - A2/l, RNE to bf16.
    lsum += shfl_xor(lsum, 32);
    bsum += shfl_xor(bsum, 32);
    if (qi < T) {
        const float inv = 1.f / lsum;
        const float one_tb = 1.f + bsum * inv;
        __bf16* orow = o + slice + (size_t)qi * D;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float y[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    y[r] = inv * (acc1[nb][4 * g + r] * one_tb - acc2[nb][4 * g + r]);
                const int d0 = 32 * nb + 8 * g + 4 * h;
                *(u32x2*)(orow + d0) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
            }
        }
    }
}

}  // namespace

hipError_t launch_prefill_bf16_d128(const PrefillArgs& a, hipStream_t stream) {
    const int BH = a.B * a.H;
    const int nqb = (a.T + BR - 1) / BR;
    const long long nblocks = (long long)BH * nqb;
    if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(prefill_bf16_d128_kernel, dim3((unsigned)nblocks), dim3(NT), 0, stream,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                       (const __bf16*)a.rho, (__bf16*)a.o, BH, a.T, nqb, a.scale * kLog2e);
    return hipGetLastError();
}

}  // namespace plx
