// prefill_bf16.hip -- causal Parallax prefill, bf16 in/out, d_qk = d_v = 128, gfx950.
//
// Method [Parallax (paper.rainbus.top summary), "方法步骤详情": per KV block compute the
// scores S1 = Q K^T and the probe products S2 = R K^T, then P1 = exp(S1 - m) and
// P2 = P1 * S2, and accumulate O1 += P1 V and O2 += P2 V in parallel; agihunt review,
// hardware paragraph: both branches share one KV stream, one running max and one rescale
// factor]. Final combine o = (1 + tbar) O1 - O2 with tbar = sum P2 / sum P1 (step 6).
//
// Work decomposition: one workgroup = 128 query rows of one (b, h) = 4 query groups of 32
// rows, and 8 waves, two per SIMD. For query group g, wave g runs the softmax branch
// (Q K^T, running max, P1, O1 += P1 V) and wave g + 4, on the same SIMD, runs the probe
// branch (R K^T, P2 = P1 * T, O2 += P2 V) one tile behind, reading the softmax wave's
// rounded weights and rescale factors from LDS. Both waves issue the same number of
// matrix instructions, and the probe wave is shifted by half a tile (it computes T one
// iteration ahead and does its vector work first), so each SIMD's matrix pipe alternates
// between the two instruction streams instead of both waves computing and then both
// waiting at the same time. Details:
//   * a wave's Q (or R) fragments stay in registers as the B operand of
//     v_mfma_f32_32x32x16_bf16, so the product tile is S^T = K Q^T (or T^T = K R^T) with
//     keys on the 32 rows and the group's queries on the 32 lanes of each half-wave;
//   * K and V tiles of 64 keys are staged in LDS by the softmax waves, three buffers each
//     (while tile t + 1 is stored, the softmax waves read tile t and the probe waves tile
//     t - 1): K row-major with rows stored in a permuted order, V transposed (d rows x 64
//     keys) so a value operand is one 16-byte LDS read; the 16-byte key chunks of dim row d
//     are XOR-swizzled with bits 4..6 of d, which keeps the operand reads conflict-free on
//     gfx950's 64-bank LDS and spreads the transposing 8-byte stores;
//   * the score tile's accumulator layout is reused directly as the P operand of the value
//     products O^T += V^T P^T: storing key rows with bits 2 and 3 of the row index swapped
//     makes each lane's eight consecutive accumulator registers hold eight consecutive
//     keys, exactly the operand layout, so no cross-lane traffic is needed;
//   * P1 and P2 are rounded to bf16 and l = sum P1, beta = sum P2 are taken from the rounded
//     values, so the effective corrected weights sum to exactly one; the probe wave forms
//     P2 from the rounded P1 the softmax wave hands over and keeps both sums;
//   * the running max is updated lazily (only when a row's tile max exceeds it by more than
//     2^8); the result is the same exact expression, with far fewer rescales.
// Persistent launch: one workgroup per compute unit, each working through a static list of
// items (128 query rows of one (b, h)), longest first in snake order so that every
// workgroup gets the same number of tiles. The items of one workgroup form a single stream
// of K/V tiles: an item's last slot already stages the next item's first tile and
// requests its Q and R fragments, so there is no per-item launch, prologue load latency or
// drain of the workgroup. With B*H a multiple of 8, workgroup x (dispatched to XCD x % 8)
// serves only the heads with bh % 8 == x % 8, so each head's K and V are read through one
// XCD's L2.
#include <type_traits>

#include "plx_device.hpp"
#include "plx_kernels.hpp"

namespace plx {
namespace {

constexpr int D = 128;
constexpr int BR = 128;  // query rows per workgroup
constexpr int BC = 64;   // keys per LDS tile
constexpr int NT = 512;  // threads per workgroup (8 waves)
constexpr int KS = D + 8;         // LDS row stride of a K tile (bf16 elements)
constexpr int VS = BC + 8;        // LDS row stride of a transposed V tile
constexpr int K_ELEMS = BC * KS;  // 8704 bf16
constexpr int V_ELEMS = D * VS;   // 9216 bf16
constexpr int NBUF = 3;
constexpr int W_BYTES = 4 * 4 * 64 * 16;  // rounded P1 of one tile: 4 groups x 4 k-steps x 64 lanes
// LDS byte layout: K buffers | V buffers | 2 x P1 hand-over | 2 x rescale factors
constexpr int OFF_V = NBUF * K_ELEMS * 2;
constexpr int OFF_W = OFF_V + NBUF * V_ELEMS * 2;
constexpr int OFF_A = OFF_W + 2 * W_BYTES;
constexpr int LDS_BYTES = OFF_A + 2 * 4 * 32 * 4;
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
static_assert(4 * 64 * 64 * 4 <= OFF_W, "epilogue hand-over must fit in the K/V buffers");
constexpr float kLazyTau = 8.0f;  // log2 headroom before the running max moves

// Row order inside each 32-key half of a K tile: bits 2 and 3 swapped (an involution).
__device__ __forceinline__ int perm_row(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Position of a workgroup's kk-th item in its class's list (sorted by descending length):
// snake order over the class's Wc workers, so that long and short items pair up.
__device__ __forceinline__ int item_position(int kk, int j, int Wc) {
    return kk * Wc + ((kk & 1) ? Wc - 1 - j : j);
}

// One work item: 128 query rows (query block qb) of one (b, h).
struct Item {
    int bh, q0, ntiles, nfull;
};

__device__ __forceinline__ Item item_at(int pos, int cls, int ncls, int nbh_c, int nqb, int T) {
    Item it;
    const int qb = nqb - 1 - pos / nbh_c;  // longest query blocks first
    it.bh = cls + ncls * (pos % nbh_c);
    it.q0 = qb * BR;
    const int kend = min(it.q0 + BR, T);
    it.ntiles = (kend + BC - 1) / BC;
    it.nfull = min(it.ntiles, it.q0 / BC);  // tiles entirely below the block's first row
    return it;
}

__global__ __launch_bounds__(NT, 1) void prefill_bf16_d128_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ rho, __bf16* __restrict__ o, int BH, int T, int nqb, float c,
    int ncls) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // The two roles run separate instantiations of the whole item loop, so that neither keeps
    // the other's loop-invariant values live. Both pass the same barriers in the same order.
    auto run = [&](auto role) {
        constexpr bool probe = decltype(role)::value;
        const int g = w & 3;        // query group
        const int n = lane & 31;    // query within the group
        const int h = lane >> 5;    // half-wave: which 8-element k-slice of an operand
        const uint32_t slice_bytes = (uint32_t)T * D * 2u;
        auto slice_of = [&](int bh) { return (size_t)bh * (size_t)T * D; };

        // ---- static schedule. With ncls = 8, workgroup x (on XCD x % 8) serves the (b, h) with
        // bh % 8 == x % 8, so each head's K and V are read through one XCD's L2.
        const int cls = blockIdx.x % ncls;
        const int jw = blockIdx.x / ncls;
        const int Wc = gridDim.x / ncls;
        const int nbh_c = BH / ncls;
        const int nit_c = nbh_c * nqb;

        auto kbuf = [&](int t) { return (__bf16*)(lds + (t % NBUF) * K_ELEMS * 2); };
        auto vbuf = [&](int t) { return (__bf16*)(lds + OFF_V + (t % NBUF) * V_ELEMS * 2); };
        auto wbuf = [&](int t) { return (u32x4*)(lds + OFF_W + (t & 1) * W_BYTES) + g * 256; };
        auto abuf = [&](int t) { return (float*)(lds + OFF_A) + ((t & 1) * 4 + g) * 32; };

        // Q (softmax waves) or R (probe waves) fragments of an item: B operand, lane holds dims
        // 16 s + 8 h .. +7 of its query row (rows past T read as zeros).
        bf16x8 xf[8];
        auto load_x = [&](const Item& it) {
            const auto rx = make_rsrc((probe ? rho : q) + slice_of(it.bh), slice_bytes);
            const uint32_t qi = (uint32_t)(it.q0 + 32 * g + n);
#pragma unroll
            for (int s = 0; s < 8; ++s)
                xf[s] = as_bf16x8(load16(rx, qi * 256u + 32u * s + 16u * h));
        };

        f32x16 acc[4];
        float rsum = 0.f;  // probe waves: beta = sum P2
        float lsum = 0.f;  // probe waves: l = sum P1 (from the rounded P1 they receive)

        // ---- staging: the softmax waves (threads 0..255) load and store both the K and the V
        // tile; the probe waves have the longer dependency chain per slot (P2 = P1 * T and
        // their products), so they stage nothing. The buffer resource starts at the tile, so
        // every tile uses the same per-lane offsets.
        const int st = tid & 255;
        const uint32_t koff = (uint32_t)(st >> 4) * 256u + 16u * (st & 15);  // + 4096 j
        const uint32_t voff = (uint32_t)(4 * (st >> 4)) * 256u + 16u * (st & 15);  // + 256 j
        u32x4 stg[8];  // K chunks 0..3, V chunks 4..7
        auto gload = [&](int bh, int kt) {
            if (probe) return;
            const size_t base = slice_of(bh) + (size_t)kt * BC * D;
            const uint32_t bytes = slice_bytes - (uint32_t)kt * BC * 256u;  // kt * BC < T
            const auto rk = make_rsrc(k + base, bytes);
#pragma unroll
            for (int j = 0; j < 4; ++j) stg[j] = load16(rk, koff + 4096u * j);
            // dims 8 (st & 15) .. +7 of keys 4 (st >> 4) .. +3
            const auto rv = make_rsrc(v + base, bytes);
#pragma unroll
            for (int j = 0; j < 4; ++j) stg[4 + j] = load16(rv, voff + 256u * j);
        };
        auto lstore = [&](int t) {
            if (probe) return;
            __bf16* Kl = kbuf(t);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int chunk = st + 256 * j;
                const int row = chunk >> 4, col = chunk & 15;
                const int prow = (row & 32) | perm_row(row & 31);
                *(u32x4*)(Kl + prow * KS + col * 8) = stg[j];
            }
            __bf16* Vl = vbuf(t);
            const int vdc = st & 15, vkg = st >> 4;
            // Transpose 4 keys x 8 dims into 8 dims x 4 keys (byte permutes), 8-byte stores.
            const u32x4* sv = stg + 4;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t lo01 = __builtin_amdgcn_perm(sv[1][p], sv[0][p], 0x05040100u);
                const uint32_t lo23 = __builtin_amdgcn_perm(sv[3][p], sv[2][p], 0x05040100u);
                const uint32_t hi01 = __builtin_amdgcn_perm(sv[1][p], sv[0][p], 0x07060302u);
                const uint32_t hi23 = __builtin_amdgcn_perm(sv[3][p], sv[2][p], 0x07060302u);
                const int d0 = 8 * vdc + 2 * p;  // d0 and d0 + 1 share bits 4..6 (= vdc >> 1)
                const int cs = 8 * ((vkg >> 1) ^ ((vdc >> 1) & 7)) + 4 * (vkg & 1);
                *(u32x2*)(Vl + d0 * VS + cs) = u32x2{lo01, lo23};
                *(u32x2*)(Vl + (d0 + 1) * VS + cs) = u32x2{hi01, hi23};
            }
        };

        // Product tile for one 32-key half (hc) of the K tile in buffer slot t.
        auto scores = [&](int t, int hc) {
            const __bf16* Kl = kbuf(t) + (32 * hc + n) * KS + 8 * h;
            f32x16 S = f32x16{};
#pragma unroll
            for (int s = 0; s < 8; ++s) S = mfma32(*(const bf16x8*)(Kl + 16 * s), xf[s], S);
            __builtin_amdgcn_iglp_opt(0);  // interleave the operand reads with the matrix ops
            return S;
        };
        // O^T += V^T P^T for k-step ks (keys 16 ks .. +15) of the V tile in slot t. Lane (n, h) of
        // block nb reads dim row vr = 32 nb + n, chunk (2 ks + h) ^ ((vr >> 4) & 7) =
        // 2 (ks ^ nb) + (h ^ (n >> 4)): a per-lane base plus a constant per (nb, ks), so every read
        // uses the immediate offset.
        const int vlane = (n * VS + 8 * (h ^ (n >> 4))) * 2;
        auto value_products = [&](int t, int ks, bf16x8 pf) {
            const unsigned char* Vl = (const unsigned char*)vbuf(t) + vlane;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const bf16x8 vf = *(const bf16x8*)(Vl + 32 * nb * VS * 2 + 32 * (ks ^ nb));
                acc[nb] = mfma32(vf, pf, acc[nb]);
            }
            __builtin_amdgcn_iglp_opt(0);
        };

        // ---- softmax branch: local tile kt of the current item, held in buffer slot t. When
        // `next` is set, the next item's Q fragments are requested as soon as the scores no
        // longer need the current ones.
        float m_run = -INFINITY;
        auto softmax_tile = [&](int t, int kt, int qi, auto diag_tag, bool next, const Item& nx) {
            constexpr bool DIAG = decltype(diag_tag)::value;
            f32x16 S[2];
            S[0] = scores(t, 0);
            S[1] = scores(t, 1);
            if constexpr (DIAG) {
                if (next) load_x(nx);
            }
            // Register i of half hc holds key 64 kt + 32 hc + perm_row(8 (i/4) + 4 h + i%4).
            if constexpr (DIAG) {
#pragma unroll
                for (int hc = 0; hc < 2; ++hc) {
                    const int lim = qi - (kt * BC + 32 * hc);
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (perm_row(8 * (i >> 2) + 4 * h + (i & 3)) > lim) S[hc][i] = -INFINITY;
                }
            }
            float mt = max3(S[0][0], S[1][0], S[0][1]);
            mt = max3(mt, S[1][1], S[0][2]);
#pragma unroll
            for (int i = 2; i < 15; ++i) mt = max3(mt, S[1][i], S[0][i + 1]);
            mt = max3(mt, S[1][15], S[1][15]);
            mt = max_with_other_half(mt);
            const float ms = mt > -INFINITY ? mt * c : -INFINITY;
            const bool need = ms > m_run + kLazyTau;
            float alpha = 1.f;
            if (wave_any(need)) {
                const float mn = need ? ms : m_run;
                alpha = exp2_fast(m_run - mn);
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) acc[nb] *= alpha;
                m_run = mn;
            }
            if (h == 0) abuf(t)[n] = alpha;  // the probe wave applies the same rescale
            u32x4* wout = wbuf(t);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int hc = ks >> 1, r = ks & 1;
                u32x4 pw;
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    float w0 = exp2_fast(fmaf(S[hc][8 * r + e], c, -m_run));
                    float w1 = exp2_fast(fmaf(S[hc][8 * r + e + 1], c, -m_run));
                    if constexpr (DIAG) {  // masked keys: weight exactly 0 (also when c == 0)
                        w0 = S[hc][8 * r + e] == -INFINITY ? 0.f : w0;
                        w1 = S[hc][8 * r + e + 1] == -INFINITY ? 0.f : w1;
                    }
                    pw[e >> 1] = pack_bf16x2(w0, w1);
                }
                wout[ks * 64 + lane] = pw;
                value_products(t, ks, as_bf16x8(pw));
            }
        };

        // ---- probe branch, finishing the tile in slot t: its products T were computed in the
        // previous slot (so that this vector work overlaps the softmax wave's score products).
        auto probe_finish = [&](int t, const f32x16 (&Tt)[2]) {
            const float alpha = abuf(t)[n];
            if (wave_any(alpha != 1.f)) {
                rsum *= alpha;
                lsum *= alpha;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) acc[nb] *= alpha;
            }
            const u32x4* win = wbuf(t);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int hc = ks >> 1, r = ks & 1;
                const u32x4 pw = win[ks * 64 + lane];
                u32x4 p2w;
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const uint32_t x = pw[e >> 1];
                    p2w[e >> 1] = pack_bf16x2(bf16_lo(x) * Tt[hc][8 * r + e],
                                              bf16_hi(x) * Tt[hc][8 * r + e + 1]);
                    rsum = add_bf16x2(p2w[e >> 1], rsum);
                    lsum = add_bf16x2(x, lsum);
                }
                value_products(t, ks, as_bf16x8(p2w));
            }
        };

        // ---- pipeline. The workgroup's items form one stream of K/V tiles; stream tile t sits in
        // buffer t % 3. In the slot where the softmax waves process stream tile t (and the probe
        // waves finish t - 1 and compute the products of t), tile t + 1 is loaded into registers
        // at the top and stored at the bottom, before the one barrier per slot; its buffer last
        // held t - 2, read by the softmax waves two slots and the probe waves one slot before.
        // Each item ends with a drain slot (the probe waves finish its last tile; nothing is
        // staged) and a two-round epilogue that uses only the weight and rescale hand-over
        // areas, so the next item's first tile, staged in the item's last slot, stays intact.
        int kk = 0;
        int pos = item_position(0, jw, Wc);
        if (pos >= nit_c) return;  // more workgroups than items in this class
        Item cur = item_at(pos, cls, ncls, nbh_c, nqb, T);
        load_x(cur);
        gload(cur.bh, 0);
        lstore(0);
        __syncthreads();
        int t0 = 0;  // stream index of the current item's tile 0
        for (;;) {
            const int pos_n = item_position(kk + 1, jw, Wc);
            const bool has_next = pos_n < nit_c;
            const Item nx = item_at(has_next ? pos_n : pos, cls, ncls, nbh_c, nqb, T);
            const int nt = cur.ntiles;
            // Staging of the slot that processes local tile kt: the item's next tile, or the next
            // item's first tile. Returns whether anything was loaded.
            auto stage = [&](int kt) {
                const bool inside = kt + 1 < nt;
                if (probe || (!inside && !has_next)) return false;
                gload(inside ? cur.bh : nx.bh, inside ? kt + 1 : 0);
                return true;
            };
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x16{};
            const int qi = cur.q0 + 32 * g + n;
            if (!probe) {
                m_run = -INFINITY;
                for (int kt = 0; kt < cur.nfull; ++kt) {
                    const bool staged = stage(kt);
                    softmax_tile(t0 + kt, kt, qi, std::false_type{}, false, nx);
                    if (staged) lstore(t0 + kt + 1);
                    __syncthreads();
                }
                for (int kt = cur.nfull; kt < nt - 1; ++kt) {
                    const bool staged = stage(kt);
                    softmax_tile(t0 + kt, kt, qi, std::true_type{}, false, nx);
                    if (staged) lstore(t0 + kt + 1);
                    __syncthreads();
                }
                {  // the last tile (always diagonal), peeled so that no loop issues the next
                   // item's fragment loads
                    const int kt = nt - 1;
                    const bool staged = stage(kt);
                    softmax_tile(t0 + kt, kt, qi, std::true_type{}, has_next, nx);
                    if (staged) lstore(t0 + kt + 1);
                    __syncthreads();
                }
                __syncthreads();  // drain slot
            } else {
                rsum = 0.f;
                lsum = 0.f;
                f32x16 Tt[2];
                {
                    const bool staged = stage(0);
                    Tt[0] = scores(t0, 0);
                    Tt[1] = scores(t0, 1);
                    if (staged) lstore(t0 + 1);
                    __syncthreads();
                }
                for (int kt = 1; kt < nt - 1; ++kt) {
                    const bool staged = stage(kt);
                    probe_finish(t0 + kt - 1, Tt);
                    Tt[0] = scores(t0 + kt, 0);
                    Tt[1] = scores(t0 + kt, 1);
                    if (staged) lstore(t0 + kt + 1);
                    __syncthreads();
                }
                if (nt > 1) {  // the last tile's products, peeled like the softmax waves' last tile
                    const int kt = nt - 1;
                    const bool staged = stage(kt);
                    probe_finish(t0 + kt - 1, Tt);
                    Tt[0] = scores(t0 + kt, 0);
                    Tt[1] = scores(t0 + kt, 1);
                    if (has_next) load_x(nx);
                    if (staged) lstore(t0 + kt + 1);
                    __syncthreads();
                }
                probe_finish(t0 + nt - 1, Tt);  // drain slot
                if (has_next && nt == 1) load_x(nx);  // single-tile item: no earlier point
                __syncthreads();
            }

            // ---- epilogue, two rounds of 32 dims x 2 blocks: the probe waves hand O2 (and l,
            // beta) over through their group's weight and rescale areas; the softmax waves
            // combine o = (A1/l)(1 + beta/l) - A2/l and round to bf16. Group g only touches its own
            // areas, so a softmax wave may start the next item's first slot right after reading.
            // The next item's Q or R fragments, requested a slot and a half ago, have arrived
            // by now; waiting for them here (vmcnt 0, nothing else is in flight) tells the
            // compiler so, instead of it waiting on every vector load the next item's slots
            // issue.
            __builtin_amdgcn_s_waitcnt(0x0F70);
            u32x4* hand0 = (u32x4*)(lds + OFF_W) + g * 256;            // 4 KB
            u32x4* hand1 = (u32x4*)(lds + OFF_W + W_BYTES) + g * 256;  // 4 KB
            float* bhand0 = (float*)(lds + OFF_A) + g * 32;            // l
            float* bhand1 = (float*)(lds + OFF_A) + (4 + g) * 32;      // beta
            __bf16* orow = o + slice_of(cur.bh) + (size_t)qi * D;
#pragma unroll
            for (int round = 0; round < 2; ++round) {
                if (probe) {
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const f32x16& a = acc[2 * round + i];
                            (i ? hand1 : hand0)[j * 64 + lane] = __builtin_bit_cast(
                                u32x4, f32x4{a[4 * j], a[4 * j + 1], a[4 * j + 2], a[4 * j + 3]});
                        }
                    if (round == 0) {
                        rsum += shfl_xor(rsum, 32);  // both key halves of each row
                        lsum += shfl_xor(lsum, 32);
                        if (h == 0) {
                            bhand0[n] = lsum;
                            bhand1[n] = rsum;
                        }
                    }
                }
                __syncthreads();
                if (!probe && qi < T) {
                    const float inv = 1.f / bhand0[n];
                    const float one_tb = 1.f + bhand1[n] * inv;
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const int nb = 2 * round + i;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const f32x4 a2 =
                                __builtin_bit_cast(f32x4, (i ? hand1 : hand0)[j * 64 + lane]);
                            float y[4];
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                y[r] = inv * (acc[nb][4 * j + r] * one_tb - a2[r]);
                            // register 4 j + r holds dim 32 nb + 8 j + 4 h + r
                            const int d0 = 32 * nb + 8 * j + 4 * h;
                            *(u32x2*)(orow + d0) =
                                u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
                        }
                    }
                }
                if (round == 0) __syncthreads();
            }
            if (!has_next) break;
            t0 += nt;
            cur = nx;
            pos = pos_n;
            ++kk;
        }
    };
    if (w >= 4)
        run(std::true_type{});
    else
        run(std::false_type{});
}

}  // namespace

hipError_t launch_prefill_bf16_d128(const PrefillArgs& a, hipStream_t stream) {
    const int BH = a.B * a.H;
    const int nqb = (a.T + BR - 1) / BR;
    const long long nitems = (long long)BH * nqb;
    // One resident workgroup per compute unit (the LDS footprint allows one), each working
    // through a static list of items; at most one workgroup per item.
    long long grid = nitems < a.workers ? nitems : a.workers;
    int ncls = 1;
    if (BH % 8 == 0 && grid >= 8) {
        ncls = 8;
        grid -= grid % 8;
    }
    if (grid < 1 || grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(prefill_bf16_d128_kernel, dim3((unsigned)grid), dim3(NT), 0, stream,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                       (const __bf16*)a.rho, (__bf16*)a.o, BH, a.T, nqb, a.scale * kLog2e, ncls);
    return hipGetLastError();
}

}  // namespace plx
