// prefill_bf16.hip -- causal Parallax prefill, bf16 in/out, d_qk = d_v = 128 or 64, gfx950.
//
// Method [Parallax (paper.rainbus.top summary), "方法步骤详情": per KV block compute the
// scores S1 = Q K^T and the probe products S2 = R K^T, then P1 = exp(S1 - m) and
// P2 = P1 * S2, and accumulate O1 += P1 V and O2 += P2 V in parallel; agihunt review,
// hardware paragraph: the softmax and correction branches read the keys and values once
// between them and are rescaled together from a single row maximum]. Final combine
// o = (1 + tbar) O1 - O2 with tbar = sum P2 / sum P1 (step 6).
//
// Work decomposition: a work item is 128 query rows of one (b, h); a workgroup has 8 waves
// (two per SIMD) of 16 query rows each, and every wave runs both branches for its rows on
// v_mfma_f32_16x16x32_bf16:
//   * the Q and R fragments of the wave's 16 queries stay in registers as the B operand, so
//     the product tiles are S^T = K Q^T and T^T = K R^T with keys on the rows; one K operand
//     read from LDS feeds both products, and one V operand read feeds both O1^T += V^T P1^T
//     and O2^T += V^T P2^T;
//   * K rows are stored in LDS in an order (key 8 q + 4 b + i of each 32-key group at row
//     16 b + 4 q + i) that makes each lane's accumulator registers of two score blocks hold
//     the 8 consecutive keys of its value-product operand: no cross-lane traffic;
//   * the V tiles arrive in LDS row-major, by direct-to-LDS loads (all but the split-weights
//     instances at d = 64), and each value operand (8 consecutive keys of one dim) is two
//     transposing LDS reads (ds_read_b64_tr_b16); otherwise the V stagers store V transposed
//     (d rows x BC keys, 16-byte key chunks XOR-swizzled with bits 4..6 of d), so a value
//     operand is one 16-byte LDS read whose address is a per-lane base plus a constant;
//   * P1 and P2 are rounded to bf16 and l = sum P1, beta = sum P2 are taken from the rounded
//     values, so the effective corrected weights sum to exactly one; the sums run on the
//     matrix cores as one more value product each, against a block of ones; P2 = P1 * T is
//     formed from the unrounded P1 (or, in the SPLIT instances, both go in as hi + lo bf16
//     terms and l, beta are fp32 sums of the unrounded weights);
//   * the running max is updated lazily (only when a row's tile max exceeds it by more than
//     2^8); the result is the same exact expression, with far fewer rescales.
// A tile holds BC = 64 keys at d = 128 and BC = 128 keys at d = 64 (the same bytes).
// Waves 0-3 stage the K tiles and waves 4-7 the V tiles; the V stagers issue at a higher
// priority, which balances the two waves of a SIMD (the hardware otherwise favours the older
// wave for the matrix pipe).
// Persistent launch: one workgroup per compute unit, each working through a static list of
// items, longest first in snake order so that every workgroup gets the same number of tiles.
// The items of one workgroup form a single stream of K/V tiles in a ring of four LDS
// buffers; tile s + 2 is staged while tile s is processed, so the workgroup synchronizes only
// after every second tile, and an item's last tiles already stage the next item's first ones.
// The Q and R fragments of the next item are requested right after the products of an item's
// last tile. With B*H a multiple of 8, workgroup x (dispatched to XCD x % 8) serves only
// the heads with bh % 8 == x % 8, so each head's K and V are read through one XCD's L2.
#include <type_traits>

#include "plx_device.hpp"
#include "plx_kernels.hpp"
#include "prefill_sched.hpp"

namespace plx {
namespace {

using prefill::BR;
using prefill::Item;
using prefill::item_at;
using prefill::item_position;
using prefill::krow;
using prefill::krow_inv;
constexpr int NT = 512;  // threads per workgroup (8 waves x 16 query rows)
constexpr int NBUF = 4;  // stream tiles s + 2 is staged while s is processed

// Sizes that follow from the head dim D (d_qk = d_v = D, a multiple of 32, at most 128) and
// from how the K tiles are staged.
template <int D, bool KDMA_>
struct Geo {
    // Keys per LDS tile: 64 at d = 128; 128 at d = 64, so that a tile holds the same bytes,
    // the stagers move the same number of chunks and the per-tile softmax and barrier cost
    // is spread over as much matrix work as possible.
    static constexpr int BC = D == 64 ? 128 : 64;
    static constexpr int NKB = BC / 16;      // 16-key score blocks per tile
    static constexpr int NG = BC / 32;       // 32-key value steps per tile
    static constexpr int VS = BC + 8;        // LDS row stride of a transposed V tile
    // KDMA (all but the split-weights instances at d = 64): the K tiles are staged by
    // direct-to-LDS loads into unpadded rows whose 16-byte chunks are XOR-swizzled by the row
    // (kswz), which keeps the operand reads conflict-free without padding; the V tiles the same
    // way, row-major with their own chunk swizzle (vswz), read back transposed. Otherwise the
    // stagers store through registers: K into rows padded by 16 bytes, V transposed (d rows of
    // BC keys, stride VS).
    static constexpr bool KDMA = KDMA_;
    static constexpr int KS = KDMA ? D : D + 8;  // LDS row stride of a K tile (bf16 elements)
    static constexpr int K_ELEMS = BC * KS;      // 8192 bf16 at D = 128
    static constexpr int V_ELEMS = KDMA ? BC * D : D * VS;
    static constexpr int OFF_V = NBUF * K_ELEMS * 2;
    static constexpr int LDS_BYTES = OFF_V + NBUF * V_ELEMS * 2;
    static constexpr int NS = D / 32;    // 32-dim steps of a q.k product
    static constexpr int NDB = D / 16;   // 16-dim blocks of a value product
    static constexpr int CPR = D / 8;    // 16-byte chunks per row
    static constexpr int CPR_LOG = D == 128 ? 4 : 3;
    static constexpr int KCH = BC * CPR / 256;  // chunks per K stager thread
    static constexpr int VST = BC / 4 * CPR;    // V stager threads (4 keys x one chunk each)
    static constexpr uint32_t ROWB = 2 * D;     // bytes per row
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};
constexpr float kLazyTau = 8.0f;  // log2 headroom before the running max moves

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane 4 a + b receives
// element b of the 4 consecutive 16-bit elements that lanes 4 j + a (j = 0..3) address.
__device__ __forceinline__ i16x4_t lds_read_tr(const unsigned char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4_t*)(__attribute__((address_space(3))) unsigned char*)p);
}

// Chunk swizzles of the direct-to-LDS tiles: chunk c of row r sits at position c ^ kswz(r)
// in a K tile and c ^ vswz(r) in a V tile (rows of 16 chunks at d = 128, 8 at d = 64, so two
// d = 64 rows share one 256-byte line of the 64 banks).
//  * K: a score operand read touches rows 16 kb + 0..15 at one chunk: the 16 rows get 16
//    distinct positions in the banks (d = 64: the 8 rows of either parity 8 distinct ones).
//  * V: the value operand reads of one half-wave touch rows 8 g + j (+ 4, + 32 G) for g = 0, 1
//    and j = 0..3, 32 bytes (a chunk pair) each: vswz is even, so pairs stay together, and
//    it gives these 8 rows 8 distinct 32-byte spans of the banks.
template <int D>
__device__ __forceinline__ int kswz(int r) {
    return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int vswz(int r) {
    return D == 128 ? 2 * ((r & 3) | (((r >> 3) & 1) << 2))
                    : 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1));
}

__device__ __forceinline__ float max_across_row_groups(float x) {
    // max over the four lanes l, l ^ 16, l ^ 32, l ^ 48
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F)));
    return max_with_other_half(x);
}

// PROBE = false: the softmax-only specialisation (rho = 0 exactly): no R K^T products, no P2,
// no O2 and no beta, so o = O1 / l. With rho = 0 the full kernel computes the same values in
// the same order (P2 = 0, beta = 0, o = O1 (1 + 0) / l - 0), so both give identical bits.
//
// STATS = true also writes, per query row, vbar = O1 / l (the softmax-weighted mean of the
// values, rounded to bf16) and (lse, tbar) in fp32, with lse the natural log of the softmax
// normaliser of scale * q.k; the backward pass starts from these. lse and tbar come from
// extra fp32 sums of the unrounded weights and weight * probe products, so that they agree
// with the weights and probe products the backward recomputes (with a large probe, |t| ~ 10,
// the bf16-rounded beta / l would differ from them by ~2^-9 |t|).
//
// SPLIT = true passes each weight u (P1 and P2) to the value products as two bf16 terms,
// hi = bf16(u) and lo = bf16(u - hi), one matrix instruction each, and sums l and beta from
// the fp32 weights: the products then see the weights to about 2^-17 relative instead of
// 2^-9. The output's sensitivity to the weights grows with |t - tbar| (the correction's
// size), so a unit-RMS probe (|t| ~ 10) needs this to stay within 1e-2 of the exact result.
template <int D, bool PROBE, bool STATS, bool SPLIT>
__global__ __launch_bounds__(NT, 1) void prefill_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ rho, __bf16* __restrict__ o, __bf16* __restrict__ vbar,
    float* __restrict__ stats, int BH, int T, int nqb, float c, int ncls) {
    static_assert(!(STATS && SPLIT), "the statistics instances keep single bf16 weights");
    // Direct-to-LDS K and V staging where it fits the register budget: everywhere but the
    // split instances at d = 64 (there the role-specialised tile loops would spill).
    constexpr bool KDMA = !SPLIT || D == 128;
    using G_ = Geo<D, KDMA>;
    constexpr int KS = G_::KS, K_ELEMS = G_::K_ELEMS, V_ELEMS = G_::V_ELEMS, OFF_V = G_::OFF_V;
    constexpr int BC = G_::BC, NKB = G_::NKB, NG = G_::NG, VS = G_::VS;
    constexpr int NS = G_::NS, NDB = G_::NDB, CPR = G_::CPR, CPR_LOG = G_::CPR_LOG;
    constexpr int KCH = G_::KCH;
    constexpr uint32_t ROWB = G_::ROWB;
    constexpr int RPL = 1024 / (int)ROWB;  // LDS rows per 1 KB direct-to-LDS load
    __shared__ __attribute__((aligned(16))) unsigned char lds[G_::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;  // query of the wave (score column)
    const int gq = lane >> 4;   // row group: keys 8 gq .. +7 of a 32-key step; dims 4 gq .. +3
    const uint32_t slice_bytes = (uint32_t)T * D * 2u;
    auto slice_of = [&](int bh) { return (size_t)bh * (size_t)T * D; };

    const int cls = blockIdx.x % ncls;
    const int jw = blockIdx.x / ncls;
    const int Wc = gridDim.x / ncls;
    const int nbh_c = BH / ncls;
    const int nit_c = nbh_c * nqb;

    auto kbuf = [&](int t) { return lds + (t % NBUF) * K_ELEMS * 2; };
    auto vbuf = [&](int t) { return lds + OFF_V + (t % NBUF) * V_ELEMS * 2; };

    // Q and R fragments (B operand of S^T = K Q^T): lane holds dims 32 st + 8 gq .. +7 of
    // query `col`.
    bf16x8 xq[NS], xr[NS];
    auto load_x = [&](const Item& it) {
        const auto rq = make_rsrc(q + slice_of(it.bh), slice_bytes);
        const auto rr = make_rsrc(rho + slice_of(it.bh), slice_bytes);
        const uint32_t qoff = (uint32_t)(it.q0 + 16 * w + col) * ROWB + 16u * gq;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            xq[st] = as_bf16x8(load16(rq, qoff + 64u * st));
            if constexpr (PROBE) xr[st] = as_bf16x8(load16(rr, qoff + 64u * st));
        }
    };

    f32x4 a1[NDB], a2[NDB];  // O1^T, O2^T: dim block db (16 dims), lane: dims 16 db + 4 gq + i
    float lsum = 0.f, bsum = 0.f;
    // Single bf16 weights: l and beta are summed on the matrix cores, as the value products of
    // a block of ones (every row of the accumulator holds the column sums of P1^T and P2^T);
    // each lane then holds the full sums of its query. The split instances sum fp32 weights.
    f32x4 al = {}, ab = {};
    bf16x8 ones;
#pragma unroll
    for (int i = 0; i < 8; ++i) ones[i] = (__bf16)1.0f;
    float lsx = 0.f, bsx = 0.f;  // STATS: the same sums of the unrounded weights and products
    float m_run = -INFINITY;

    // ---- staging: waves 0-3 load and store the K tile, waves 4-7 the V tile. K stager st
    // moves chunks st + 256 j (key chunk / CPR, dims 8 (chunk % CPR) ..); V stager st moves
    // keys 4 (st / CPR) .. +3 of dim chunk st % CPR (all of waves 4-7 at D = 128, the first
    // 2 D of them otherwise). CPR (16-byte chunks per row) is a power of two.
    const bool kstager = w < 4;
    const int st = tid & 255;
    const bool vactive = G_::VST >= 256 || st < G_::VST;
    const uint32_t koff = (uint32_t)(st >> CPR_LOG) * ROWB + 16u * (st & (CPR - 1));  // + 4096 j
    const uint32_t voff =
        (uint32_t)(4 * (st >> CPR_LOG)) * ROWB + 16u * (st & (CPR - 1));  // + ROWB j
    u32x4 stg[4];
    // Loads of tile kt of head bh, bound for ring slot t: direct-to-LDS for K and V at d = 128
    // (the LDS destination must be known now), into registers otherwise (stored by lstore).
    // In the KDMA instances the staging role is a template argument of the tile loop (the
    // loop is compiled once per role, behind a wave-uniform branch): measured 3% faster than
    // one loop that branches on the role at each staging point.
    // role: std::true_type / std::false_type (K / V stager) in the KDMA instances; elsewhere
    // the runtime role `kstager` decides and the argument is ignored.
    auto is_k = [&](auto role) {
        if constexpr (KDMA) return decltype(role)::value;
        else return kstager;
    };
    auto gload = [&](auto role, int bh, int kt, int t) {
        const size_t base = slice_of(bh) + (size_t)kt * BC * D;
        const uint32_t bytes = slice_bytes - (uint32_t)kt * BC * ROWB;  // kt * BC < T
        if (is_k(role)) {
            const auto rk = make_rsrc(k + base, bytes);
            if constexpr (KDMA) {
                // Load j of K-stager wave w fills the RPL rows from LDS row RPL (4 j + w) on
                // (1 KB, 16 bytes per lane in lane order; RPL = 1024 / ROWB): lane (row r,
                // position p) fetches chunk p ^ kswz(r) of key krow_inv(r). Rows past T read
                // as zero.
                unsigned char* Kl = kbuf(t);
                const int p = lane & (CPR - 1);
#pragma unroll
                for (int j = 0; j < KCH; ++j) {
                    const int r = RPL * (4 * j + w) + (lane >> CPR_LOG);
                    const uint32_t src =
                        (uint32_t)krow_inv(r) * ROWB + 16u * (p ^ kswz<D>(r));
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rk, (__attribute__((address_space(3))) void*)(Kl + RPL * (4 * j + w) * ROWB),
                        16, src, 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int j = 0; j < KCH; ++j) stg[j] = load16(rk, koff + 4096u * j);
            }
        } else if (vactive) {
            const auto rv = make_rsrc(v + base, bytes);
            if constexpr (KDMA) {
                // Load j of V-stager wave w fills the RPL rows from LDS row RPL (4 j + w - 4)
                // on in lane order: lane (row r, position p) fetches chunk p ^ vswz(r) of key r.
                unsigned char* Vl = vbuf(t);
                const int p = lane & (CPR - 1), wv = w - 4;
#pragma unroll
                for (int j = 0; j < KCH; ++j) {
                    const int r = RPL * (4 * j + wv) + (lane >> CPR_LOG);
                    const uint32_t src = (uint32_t)r * ROWB + 16u * (p ^ vswz<D>(r));
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rv, (__attribute__((address_space(3))) void*)(Vl + RPL * (4 * j + wv) * ROWB),
                        16, src, 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) stg[j] = load16(rv, voff + ROWB * j);
            }
        }
    };
    auto lstore = [&](auto role, int t) {
        if constexpr (KDMA) return;  // K and V are already in LDS
        if (is_k(role)) {
            unsigned char* Kl = kbuf(t);
#pragma unroll
            for (int j = 0; j < KCH; ++j) {
                const int chunk = st + 256 * j;
                const int key = chunk >> CPR_LOG, cc = chunk & (CPR - 1);
                *(u32x4*)(Kl + krow(key) * KS * 2 + cc * 16) = stg[j];
            }
        } else if (vactive) {
            __bf16* Vl = (__bf16*)vbuf(t);
            const int vdc = st & (CPR - 1), vkg = st >> CPR_LOG;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t lo01 = __builtin_amdgcn_perm(stg[1][p], stg[0][p], 0x05040100u);
                const uint32_t lo23 = __builtin_amdgcn_perm(stg[3][p], stg[2][p], 0x05040100u);
                const uint32_t hi01 = __builtin_amdgcn_perm(stg[1][p], stg[0][p], 0x07060302u);
                const uint32_t hi23 = __builtin_amdgcn_perm(stg[3][p], stg[2][p], 0x07060302u);
                const int d0 = 8 * vdc + 2 * p;
                const int cs = 8 * ((vkg >> 1) ^ ((vdc >> 1) & 7)) + 4 * (vkg & 1);
                *(u32x2*)(Vl + d0 * VS + cs) = u32x2{lo01, lo23};
                *(u32x2*)(Vl + (d0 + 1) * VS + cs) = u32x2{hi01, hi23};
            }
        }
    };

    // Scores and probe products of K tile t: block kb covers LDS rows 16 kb .. +15.
    // Lane (col, gq) register i of block kb holds key 32 (kb >> 1) + 8 gq + 4 (kb & 1) + i.
    // The operand of lane (col, gq) for dim step s is chunk 4 s + gq of row 16 kb + col; in the
    // swizzled d = 128 layout it sits at position (4 s + gq) ^ col = 4 (s ^ (col >> 2)) +
    // (gq ^ (col & 3)), one lane offset per s.
    int klane[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s)
        klane[s] = KDMA ? col * KS * 2 + 16 * ((4 * s + gq) ^ kswz<D>(col))
                        : col * KS * 2 + 16 * gq;  // + 64 s as an immediate offset below
    auto products = [&](int t, f32x4 (&S)[NKB], f32x4 (&Tp)[NKB]) {
        const unsigned char* Kl = kbuf(t);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            S[kb] = f32x4{};
            Tp[kb] = f32x4{};
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const bf16x8 kf = *(const bf16x8*)(Kl + (KDMA ? klane[s] : klane[0] + 64 * s) +
                                                   16 * kb * KS * 2);
                S[kb] = mfma16(kf, xq[s], S[kb]);
                if constexpr (PROBE) Tp[kb] = mfma16(kf, xr[s], Tp[kb]);
            }
        }
        __builtin_amdgcn_iglp_opt(1);
    };
    // Value products of 32-key step G of V tile t: lane (col, gq) of dim block db reads dim
    // row 16 db + col, keys 32 G + 8 gq .. +7, stored at chunk (4 G + gq) ^ db.
    int vlane[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) vlane[x] = col * VS * 2 + 16 * (gq ^ x);
    // KDMA: the operand of dim block db, step G is two transposing reads (keys 32 G + 8 gq +
    // 0..3 and + 4..7); lane 4 j + a of a 16-lane group addresses row 32 G + 8 gq + j (+ 4),
    // dims 16 db + 4 a .. +3, i.e. bytes 8 a of 32-byte span db ^ s at s = vswz(row) / 2.
    int vtr[KDMA ? NDB : 1];
    if constexpr (KDMA) {
        const int j = col >> 2, sw = vswz<D>(8 * gq + j) / 2;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            vtr[db] = (8 * gq + j) * (int)ROWB + 32 * (db ^ sw) + 8 * (col & 3);
    }
    // SPLIT: q1, q2 are the lo terms of p1, p2 (same V operand, two more products).
    auto values = [&](int t, int G, bf16x8 p1, bf16x8 p2, bf16x8 q1, bf16x8 q2) {
        const unsigned char* Vl = vbuf(t);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            bf16x8 vf;
            if constexpr (KDMA) {
                const unsigned char* p = Vl + vtr[db] + 32 * G * ROWB;
                const i16x4_t lo = lds_read_tr(p), hi = lds_read_tr(p + 4 * ROWB);
                vf = __builtin_bit_cast(bf16x8,
                                        __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            } else {
                vf = *(const bf16x8*)(Vl + vlane[db & 3] + 16 * db * VS * 2 +
                                      64 * (G ^ (db >> 2)));
            }
            a1[db] = mfma16(vf, p1, a1[db]);
            if constexpr (PROBE) a2[db] = mfma16(vf, p2, a2[db]);
            if constexpr (SPLIT) {
                a1[db] = mfma16(vf, q1, a1[db]);
                if constexpr (PROBE) a2[db] = mfma16(vf, q2, a2[db]);
            }
        }
        if constexpr (!SPLIT) {
            al = mfma16(ones, p1, al);
            if constexpr (PROBE) ab = mfma16(ones, p2, ab);
        }
        __builtin_amdgcn_iglp_opt(1);
    };

    // Weights and value products of tile t (local index kt) from its products S, Tp.
    auto finish = [&](int t, int kt, int qi, auto diag_tag, f32x4 (&S)[NKB],
                      const f32x4 (&Tp)[NKB]) {
        constexpr bool DIAG = decltype(diag_tag)::value;
        if constexpr (DIAG) {
            // key kt * BC + 8 gq + (32 (kb >> 1) + 4 (kb & 1) + i) is visible iff the constant
            // part is at most lim
            const int lim = qi - kt * BC - 8 * gq;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (32 * (kb >> 1) + 4 * (kb & 1) + i > lim) S[kb][i] = -INFINITY;
        }
        float mt = max3(S[0][0], S[0][1], S[0][2]);
        mt = max3(mt, S[0][3], S[1][0]);
        mt = max3(mt, S[1][1], S[1][2]);
        mt = max3(mt, S[1][3], S[2][0]);
        mt = max3(mt, S[2][1], S[2][2]);
        mt = max3(mt, S[2][3], S[3][0]);
        mt = max3(mt, S[3][1], S[3][2]);
        mt = max3(mt, S[3][3], S[3][3]);
#pragma unroll
        for (int kb = 4; kb < NKB; kb += 2) {
            mt = max3(mt, S[kb][0], S[kb][1]);
            mt = max3(mt, S[kb][2], S[kb][3]);
            mt = max3(mt, S[kb + 1][0], S[kb + 1][1]);
            mt = max3(mt, S[kb + 1][2], S[kb + 1][3]);
        }
        // The running max moves only when some score of the row exceeds it by more than tau:
        // each lane tests its own keys, and the max across the row's four lanes is formed
        // only when some lane of the wave passes (the same decisions as testing the row max).
        const bool need_lane = (mt > -INFINITY ? mt * c : -INFINITY) > m_run + kLazyTau;
        if (wave_any(need_lane)) {
            mt = max_across_row_groups(mt);
            const float ms = mt > -INFINITY ? mt * c : -INFINITY;
            const bool need = ms > m_run + kLazyTau;
            const float mn = need ? ms : m_run;
            const float alpha = exp2_fast(m_run - mn);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                a1[db] *= alpha;
                if constexpr (PROBE) a2[db] *= alpha;
            }
            if constexpr (SPLIT) {
                lsum *= alpha;
                if constexpr (PROBE) bsum *= alpha;
            } else {
                al *= alpha;
                if constexpr (PROBE) ab *= alpha;
            }
            if constexpr (STATS) {
                lsx *= alpha;
                bsx *= alpha;
            }
            m_run = mn;
        }
#pragma unroll
        for (int G = 0; G < NG; ++G) {
            uint32_t p1[4], p2[4], q1[4] = {}, q2[4] = {};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int kb = 2 * G + (e >> 1), i0 = 2 * (e & 1);
                float w0 = exp2_fast(fmaf(S[kb][i0], c, -m_run));
                float w1 = exp2_fast(fmaf(S[kb][i0 + 1], c, -m_run));
                if constexpr (DIAG) {
                    w0 = S[kb][i0] == -INFINITY ? 0.f : w0;
                    w1 = S[kb][i0 + 1] == -INFINITY ? 0.f : w1;
                }
                p1[e] = pack_bf16x2(w0, w1);
                if constexpr (SPLIT) {
                    q1[e] = pack_bf16x2(w0 - bf16_lo(p1[e]), w1 - bf16_hi(p1[e]));
                    lsum += w0 + w1;
                }
                if constexpr (STATS) {
                    lsx += w0 + w1;
                    if constexpr (PROBE) bsx = fmaf(w1, Tp[kb][i0 + 1], fmaf(w0, Tp[kb][i0], bsx));
                }
                if constexpr (PROBE) {
                    const float u0 = w0 * Tp[kb][i0], u1 = w1 * Tp[kb][i0 + 1];
                    p2[e] = pack_bf16x2(u0, u1);
                    if constexpr (SPLIT) {
                        q2[e] = pack_bf16x2(u0 - bf16_lo(p2[e]), u1 - bf16_hi(p2[e]));
                        bsum += u0 + u1;
                    }
                } else {
                    p2[e] = 0u;
                }
            }
            values(t, G, __builtin_bit_cast(bf16x8, u32x4{p1[0], p1[1], p1[2], p1[3]}),
                   __builtin_bit_cast(bf16x8, u32x4{p2[0], p2[1], p2[2], p2[3]}),
                   __builtin_bit_cast(bf16x8, u32x4{q1[0], q1[1], q1[2], q1[3]}),
                   __builtin_bit_cast(bf16x8, u32x4{q2[0], q2[1], q2[2], q2[3]}));
        }
    };

    if (w >= 4) __builtin_amdgcn_s_setprio(2);  // the V stagers carry the longer slot
    // Stream tile s + 2 is staged while tile s is processed (four buffers), so a barrier is
    // needed only after every second tile: between the step that last reads a buffer (s - 2)
    // and the one that refills it (s) lies a barrier, and so does between that refill and the
    // step that reads it (s + 2).
    int kk = 0;
    int pos = item_position(0, jw, Wc);
    if (pos >= nit_c) return;
    Item cur = item_at<BC>(pos, cls, ncls, nbh_c, nqb, T);
    // Source of the tile `ahead` tiles after local tile kt of item a, given the next two items.
    auto source = [&](const Item& a, int kt, int ahead, bool h1, const Item& n1, bool h2,
                      const Item& n2, int* bh, int* tile) {
        int r = kt + ahead;
        if (r < a.ntiles) { *bh = a.bh; *tile = r; return true; }
        r -= a.ntiles;
        if (!h1) return false;
        if (r < n1.ntiles) { *bh = n1.bh; *tile = r; return true; }
        r -= n1.ntiles;
        if (!h2 || r >= n2.ntiles) return false;
        *bh = n2.bh; *tile = r;
        return true;
    };
    load_x(cur);
    {
        const int p1 = item_position(1, jw, Wc), p2 = item_position(2, jw, Wc);
        const bool h1 = p1 < nit_c, h2 = p2 < nit_c;
        const Item n1 = item_at<BC>(h1 ? p1 : pos, cls, ncls, nbh_c, nqb, T);
        const Item n2 = item_at<BC>(h2 ? p2 : pos, cls, ncls, nbh_c, nqb, T);
        auto first_two = [&](auto role) {
            gload(role, cur.bh, 0, 0);
            lstore(role, 0);
            int sbh = 0, stile = 0;
            if (source(cur, 0, 1, h1, n1, h2, n2, &sbh, &stile)) {
                gload(role, sbh, stile, 1);
                lstore(role, 1);
            }
        };
        if constexpr (KDMA) {
            if (kstager) first_two(std::true_type{});
            else first_two(std::false_type{});
        } else {
            first_two(std::false_type{});
        }
    }
    __syncthreads();
    __builtin_amdgcn_s_waitcnt(0x0F70);  // the fragments have arrived (see the epilogue)
    int t0 = 0;
    auto tile_loop = [&](auto role) {
    for (;;) {
        const int pos_n = item_position(kk + 1, jw, Wc);
        const bool has_next = pos_n < nit_c;
        const Item nx = item_at<BC>(has_next ? pos_n : pos, cls, ncls, nbh_c, nqb, T);
        const int pos_n2 = item_position(kk + 2, jw, Wc);
        const bool has_next2 = has_next && pos_n2 < nit_c;
        const Item nx2 = item_at<BC>(has_next2 ? pos_n2 : pos, cls, ncls, nbh_c, nqb, T);
        const int nt = cur.ntiles;
        auto stage = [&](int kt) {
            int sbh = 0, stile = 0;
            if (!source(cur, kt, 2, has_next, nx, has_next2, nx2, &sbh, &stile)) return false;
            gload(role, sbh, stile, t0 + kt + 2);
            return true;
        };
        auto slot_end = [&](int kt) {
            if ((t0 + kt) & 1) __syncthreads();
        };
#pragma unroll
        for (int db = 0; db < NDB; ++db) a1[db] = a2[db] = f32x4{};  // a2 stays 0 without PROBE
        lsum = bsum = 0.f;
        al = ab = f32x4{};
        lsx = bsx = 0.f;
        m_run = -INFINITY;
        const int qi = cur.q0 + 16 * w + col;
        f32x4 S[NKB], Tp[NKB];
        for (int kt = 0; kt < cur.nfull; ++kt) {
            const bool staged = stage(kt);
            products(t0 + kt, S, Tp);
            finish(t0 + kt, kt, qi, std::false_type{}, S, Tp);
            if (staged) lstore(role, t0 + kt + 2);
            slot_end(kt);
        }
        for (int kt = cur.nfull; kt < nt - 1; ++kt) {
            const bool staged = stage(kt);
            products(t0 + kt, S, Tp);
            finish(t0 + kt, kt, qi, std::true_type{}, S, Tp);
            if (staged) lstore(role, t0 + kt + 2);
            slot_end(kt);
        }
        {
            const int kt = nt - 1;
            const bool staged = stage(kt);
            // When every key of the tile lies after every row of the wave (waves 0-3 in a full
            // item's last tile) the wave has nothing to add; skipping leaves the SIMD's matrix
            // pipe to the other wave for this slot.
            const bool skip = kt * BC > cur.q0 + 16 * w + 15;
            if (!skip) products(t0 + kt, S, Tp);
            if (has_next) load_x(nx);
            if (!skip) finish(t0 + kt, kt, qi, std::true_type{}, S, Tp);
            if (staged) lstore(role, t0 + kt + 2);
            slot_end(kt);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);
        // ---- epilogue: l and beta (split instances: over the four lanes of each query);
        // o = (A1/l)(1 + beta/l) - A2/l, rounded to bf16.
        if constexpr (!SPLIT) {
            lsum = al[0];
            bsum = PROBE ? ab[0] : 0.f;
        } else {
            lsum += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(lsum), 0x401F));
            const auto r1 = __builtin_amdgcn_permlane32_swap(__float_as_int(lsum),
                                                             __float_as_int(lsum), false, false);
            lsum = __int_as_float(r1[0]) + __int_as_float(r1[1]);
        }
        if constexpr (PROBE && SPLIT) {
            bsum += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(bsum), 0x401F));
            const auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_int(bsum),
                                                             __float_as_int(bsum), false, false);
            bsum = __int_as_float(r2[0]) + __int_as_float(r2[1]);
        }
        if (qi < T) {
            const float inv = 1.f / lsum;
            const float one_tb = 1.f + bsum * inv;
            __bf16* orow = o + slice_of(cur.bh) + (size_t)qi * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                float y[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    y[i] = PROBE ? inv * (a1[db][i] * one_tb - a2[db][i]) : inv * a1[db][i];
                *(u32x2*)(orow + 16 * db + 4 * gq) =
                    u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
            }
            if constexpr (STATS) {
                __bf16* vrow = vbar + slice_of(cur.bh) + (size_t)qi * D;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    *(u32x2*)(vrow + 16 * db + 4 * gq) =
                        u32x2{pack_bf16x2(inv * a1[db][0], inv * a1[db][1]),
                              pack_bf16x2(inv * a1[db][2], inv * a1[db][3])};
                // lse and tbar from the unrounded weights: sum_j exp2(c s_ij) = lsx 2^m_run, so
                // lse = (m_run + log2 lsx) ln 2, and tbar = bsx / lsx
                lsx += shfl_xor(lsx, 16);
                lsx += shfl_xor(lsx, 32);
                bsx += shfl_xor(bsx, 16);
                bsx += shfl_xor(bsx, 32);
                if (gq == 0) {
                    const float lse = (m_run + __builtin_log2f(lsx)) * 0.6931471805599453f;
                    *(float2*)(stats + 2 * ((size_t)cur.bh * T + qi)) =
                        float2{lse, PROBE ? bsx / lsx : 0.f};
                }
            }
        }
        if (!has_next) break;
        t0 += nt;
        cur = nx;
        pos = pos_n;
        ++kk;
    }
    };
    if constexpr (KDMA) {
        if (kstager) tile_loop(std::true_type{});
        else tile_loop(std::false_type{});
    } else {
        tile_loop(std::false_type{});
    }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
    const int BH = a.B * a.H;
    const int nqb = (a.T + BR - 1) / BR;
    const long long nitems = (long long)BH * nqb;
    long long grid = nitems < a.workers ? nitems : a.workers;
    int ncls = 1;
    if (BH % 8 == 0 && grid >= 8) {
        ncls = 8;
        grid -= grid % 8;
    }
    if (grid < 1 || grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const __bf16* qp = (const __bf16*)a.q;
    const __bf16* rp = a.rho ? (const __bf16*)a.rho : qp;  // unread without the probe branch
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(NT), 0, stream, qp,
                           (const __bf16*)a.k, (const __bf16*)a.v, rp, (__bf16*)a.o,
                           (__bf16*)a.vbar, a.stats, BH, a.T, nqb, a.scale * kLog2e, ncls);
    };
    if (a.stats && a.split) return hipErrorInvalidValue;
    auto pick = [&](auto d_tag) {
        constexpr int D = decltype(d_tag)::value;
        if (a.stats) {
            if (a.rho) go(prefill_bf16_kernel<D, true, true, false>);
            else go(prefill_bf16_kernel<D, false, true, false>);
        } else if (a.split) {
            if (a.rho) go(prefill_bf16_kernel<D, true, false, true>);
            else go(prefill_bf16_kernel<D, false, false, true>);
        } else {
            if (a.rho) go(prefill_bf16_kernel<D, true, false, false>);
            else go(prefill_bf16_kernel<D, false, false, false>);
        }
    };
    if (a.d == 64) {
        pick(std::integral_constant<int, 64>{});
    } else if (a.d == 128) {
        pick(std::integral_constant<int, 128>{});
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace plx
