// decode_bf16.hip -- one Parallax decode step over a contiguous per-sequence KV cache,
// bf16 in/out, d_qk = d_v = 128, gfx950.
//
// The per-step arithmetic (one matrix instruction yields the scores and the probe products;
// see decode_step.hpp) is shared by two ways of dividing the cache among waves:
//
//  * Split mode: persistent KV-loop splitting with a reduction of the partials [Parallax
//    (paper.rainbus.top summary), reproducibility section: the decode kernel's optimisations
//    are instruction sharing, KV-loop splitting and the reduction of the split partials].
//    Workgroup (s, h, b) streams chunk s of the (b, h) range (the S chunks split that
//    sequence's own length evenly), its 4 waves interleaving 32-row steps, and writes the
//    partial state (m, l, beta, A1 = sum w v, A2 = sum w t v); a second kernel merges the S
//    partials of each (b, h) with one rescale each and applies o = (A1/l)(1 + beta/l) - A2/l.
//    With S = 1 the first kernel writes o directly. Suits few long sequences.
//
//  * Wave-range mode: the (b, h) key ranges, laid end to end (sequence-major, head-minor),
//    form one flat range of W = H * sum_b n_b rows, and wave g of G streams the slice
//    [g W / G, (g + 1) W / G). Every wave therefore gets the same number of rows whatever the
//    mix of sequence lengths, and it prefetches across (b, h) boundaries, so short sequences
//    cost no pipeline restart. Each workgroup first forms the prefix sums of the clamped
//    lengths in LDS; a wave finds its first (b, h) with a 64-way search. A (b, h) that lies
//    inside one slice is finished by its wave (o written); one cut by slice boundaries leaves
//    a partial per piece, and a combine kernel (one wave per slice boundary) merges them.
//    With the boundaries moved to the next (b, h) start ("whole" plans, chosen from 2 (b, h)
//    per wave) nothing is cut and no combine runs. Suits many short sequences.
//
// Both stream the cache once with non-temporal 16-byte buffer loads in 32-row steps (16 KiB);
// split mode keeps two steps in flight per wave, wave-range mode one step per wave with 16
// waves per compute unit. Buffer ranges end at the last valid row, so rows at or beyond
// seqlens are never read.
#include "decode_step.hpp"
#include "plx_kernels.hpp"

namespace plx {
namespace {

using decode::Acc;
using decode::D;
using decode::Frag;
using decode::KB;
using decode::NT;
using decode::NW;
constexpr int REC = kDecodeRecord;

__device__ __forceinline__ int rfl(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ int clamp_len(int n, int L_max) {
    return n < 0 ? 0 : (n > L_max ? L_max : n);
}

// o = (A1/l)(1 + beta/l) - A2/l; an empty range (l == 0) gives 0.
__device__ __forceinline__ float combine_out(float a1, float a2, float l, float beta) {
    if (!(l > 0.f)) return 0.f;
    const float inv = 1.f / l;
    return inv * (a1 * (1.f + beta * inv) - a2);
}

// ------------------------------------------------------------------------- partial merging
// Online merge of partial records by one wave; lane owns dims 2 lane, 2 lane + 1.
struct Merge {
    float m = -INFINITY, l = 0.f, beta = 0.f, a1x = 0.f, a1y = 0.f, a2x = 0.f, a2y = 0.f;
};

// Fold records rec_at(0 .. n-1) into st, issuing the loads of a batch of 8 records before
// using any of them (one memory round trip per batch). An empty record has m = -inf.
template <int BATCH = 8, class RecAt>
__device__ __forceinline__ void fold_records(Merge& st, int n, RecAt rec_at, int lane) {
    for (int u0 = 0; u0 < n; u0 += BATCH) {
        float ms[BATCH], ls[BATCH], bs[BATCH];
        float2 x1[BATCH], x2[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const float* rec = rec_at(min(u0 + u, n - 1));
            ms[u] = u0 + u < n ? rec[2 * D] : -INFINITY;
            ls[u] = rec[2 * D + 1];
            bs[u] = rec[2 * D + 2];
            x1[u] = *(const float2*)(rec + 2 * lane);
            x2[u] = *(const float2*)(rec + D + 2 * lane);
        }
        float mb = st.m;
#pragma unroll
        for (int u = 0; u < BATCH; ++u) mb = fmaxf(mb, ms[u]);
        if (mb == -INFINITY) continue;  // nothing non-empty yet (wave-uniform)
        const float fo = st.m > -INFINITY ? exp2_fast(st.m - mb) : 0.f;
        st.l *= fo;
        st.beta *= fo;
        st.a1x *= fo;
        st.a1y *= fo;
        st.a2x *= fo;
        st.a2y *= fo;
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const float f = ms[u] > -INFINITY ? exp2_fast(ms[u] - mb) : 0.f;  // empty: 0
            st.l = fmaf(f, ls[u], st.l);
            st.beta = fmaf(f, bs[u], st.beta);
            st.a1x = fmaf(f, x1[u].x, st.a1x);
            st.a1y = fmaf(f, x1[u].y, st.a1y);
            st.a2x = fmaf(f, x2[u].x, st.a2x);
            st.a2y = fmaf(f, x2[u].y, st.a2y);
        }
        st.m = mb;
    }
}

__device__ __forceinline__ void store_merged(const Merge& st, __bf16* o_bh, int lane) {
    *(uint32_t*)(o_bh + 2 * lane) = pack_bf16x2(combine_out(st.a1x, st.a2x, st.l, st.beta),
                                                combine_out(st.a1y, st.a2y, st.l, st.beta));
}

// ------------------------------------------------------------------------------ split mode
// PROBE = false (rho == NULL at the boundary): the softmax-only specialisation, see consume().
// PAGED: the cache is a pool of blocks [num_blocks, H, 2^bs_log2, d] and block_table[b][i]
// names the block of rows i 2^bs_log2 .. of sequence b (blocks of at least 32 rows, so a step
// never crosses a block). Only blocks holding rows below the chunk end are looked up; an entry
// outside [0, num_blocks) is never dereferenced and its rows get no weight (skipped).
// DEEP: each wave keeps its next step's loads in flight while it consumes the current one
// (two register sets, two waves per SIMD). Without it each wave holds one step (one register
// set, four waves per SIMD): for chunks of at most one step per wave (short contexts) the
// second set is never used, and the doubled occupancy keeps twice the workgroups resident.
// Both consume the same steps in the same order, so their outputs are bit-identical.
template <bool PROBE, bool PAGED, bool DEEP>
__global__ __launch_bounds__(NT, DEEP ? 2 : 4) void decode_split_bf16_d128_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ rho, const __bf16* __restrict__ kc,
    const __bf16* __restrict__ vc, const int32_t* __restrict__ seqlens, __bf16* __restrict__ o,
    float* __restrict__ ws, int H, int L_max, int S, float c, const int32_t* __restrict__ table,
    int max_blocks, int bs_log2, int num_blocks) {
    __shared__ __attribute__((aligned(16))) float ush[NW][2][KB];  // fp32 w and w t per key
    __shared__ __attribute__((aligned(16))) float red[NW][2 * D + 4];

    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    // The paged instance needs the wave index (and with it each step's block) wave-uniform,
    // so that the block's buffer resource lives in scalar registers.
    const int w = PAGED ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
    const int col = lane & 15;  // column of the score tile (0: q, 1: rho); V: dims 8 col ..
    const int g = lane >> 4;    // row group of the score tile; V: key sub-range

    const int nb_keys = clamp_len(seqlens[b], L_max);
    // The S chunks of this sequence split its own length (not L_max) evenly, in whole wave
    // steps, so that ragged batches keep every split busy; trailing chunks may be empty.
    const int chunk = (((nb_keys + S - 1) / S) + KB - 1) / KB * KB;
    const int j0 = s * chunk;
    const int j1 = min(j0 + chunk, nb_keys);
    const size_t bh = (size_t)b * H + h;
    const uint32_t range = j1 > 0 ? (uint32_t)j1 * 256u : 0u;
    const auto rk = make_rsrc(kc + bh * (size_t)L_max * D, range);  // contiguous cache
    const auto rv = make_rsrc(vc + bh * (size_t)L_max * D, range);
    // Block of the step at row kb0 (paged cache; looked up a step before its loads are
    // issued, so that the table read is not on the way to them).
    auto lookup = [&](int kb0) -> int {
        if constexpr (!PAGED) return 0;
        return kb0 < j1 ? __builtin_amdgcn_readfirstlane(
                              table[(size_t)b * max_blocks + (kb0 >> bs_log2)])
                        : -1;
    };
    // Loads of the step at row kb0: the contiguous cache, or the block that holds it.
    auto load_at = [&](int kb0, int phys, Frag& f) {
        if constexpr (!PAGED) {
            decode::load_step(rk, rv, kb0, col, g, f);
        } else {
            int rel = 0;
            uint32_t bytes = 0;
            size_t base = 0;
            if (kb0 < j1) {
                const int blk = kb0 >> bs_log2, r0 = blk << bs_log2;
                if (phys >= 0 && phys < num_blocks) {
                    base = (((size_t)phys * H + h) << bs_log2) * D;
                    bytes = (uint32_t)min(1 << bs_log2, j1 - r0) * 256u;
                }
                rel = kb0 - r0;
            }
            decode::load_step(make_rsrc(kc + base, bytes), make_rsrc(vc + base, bytes), rel, col,
                              g, f);
        }
    };

    bf16x8 bqr[4];
    decode::load_qr(make_rsrc(q + bh * D, 256u), make_rsrc(PROBE ? rho + bh * D : q, PROBE ? 256u : 0u),
                    col, g, bqr);

    Acc acc;
    acc.reset();

    // Software pipeline over this wave's steps (rows j0 + KB w + n STEP): the loads of step
    // n + 1 are issued before step n is consumed. A prefetch past the chunk reads beyond the
    // buffer range and returns zeros without touching memory.
    constexpr int STEP = KB * NW;
    Frag fa, fb;
    int kb0 = j0 + KB * w;
    if constexpr (!DEEP) {
        // One step per pass; a step whose table entry lies outside [0, num_blocks) reads
        // zeros and gets no weight (its row limit is its own first row).
        for (; kb0 < j1; kb0 += STEP) {
            const int ph = lookup(kb0);
            load_at(kb0, ph, fa);
            const int lim = PAGED && (unsigned)ph >= (unsigned)num_blocks ? kb0 : j1;
            decode::consume<PROBE>(acc, fa, bqr, kb0, lim, c, ush[w], col, g);
        }
    } else if constexpr (PAGED) {
        // A step whose table entry lies outside [0, num_blocks) has no rows: its loads read
        // zeros and its row limit is its own first row, so none of its rows gets a weight.
        auto limit = [&](int phys, int at) {
            return (unsigned)phys < (unsigned)num_blocks ? j1 : at;
        };
        int pha = lookup(kb0);
        if (kb0 < j1) load_at(kb0, pha, fa);
        int ph1 = lookup(kb0 + STEP);
        for (; kb0 < j1; kb0 += 2 * STEP) {
            load_at(kb0 + STEP, ph1, fb);
            const int phb = ph1;
            const int ph2 = lookup(kb0 + 2 * STEP);
            decode::consume<PROBE>(acc, fa, bqr, kb0, limit(pha, kb0), c, ush[w], col, g);
            if (kb0 + STEP >= j1) break;
            load_at(kb0 + 2 * STEP, ph2, fa);
            pha = ph2;
            ph1 = lookup(kb0 + 3 * STEP);
            decode::consume<PROBE>(acc, fb, bqr, kb0 + STEP, limit(phb, kb0 + STEP), c, ush[w],
                                   col, g);
        }
    } else {
        if (kb0 < j1) decode::load_step(rk, rv, kb0, col, g, fa);
        for (; kb0 < j1; kb0 += 2 * STEP) {
            decode::load_step(rk, rv, kb0 + STEP, col, g, fb);
            decode::consume<PROBE>(acc, fa, bqr, kb0, j1, c, ush[w], col, g);
            if (kb0 + STEP >= j1) break;
            decode::load_step(rk, rv, kb0 + 2 * STEP, col, g, fa);
            decode::consume<PROBE>(acc, fb, bqr, kb0 + STEP, j1, c, ush[w], col, g);
        }
    }

    decode::wave_totals<PROBE>(acc);
    if (lane < 16) {
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

// One wave per (b, h): lane owns dims 2 lane, 2 lane + 1 and folds the S records in batches of
// 16 (all loads of a batch in flight together; one batch for up to 16 splits).
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ ws,
                                                            __bf16* __restrict__ o, int S) {
    const int lane = threadIdx.x;
    const size_t bh = blockIdx.x;
    const float* base = ws + bh * (size_t)S * REC;
    Merge st;
    fold_records<16>(st, S, [&](int u) { return base + (size_t)u * REC; }, lane);
    store_merged(st, o + bh * D, lane);
}

// ------------------------------------------------------------------------ wave-range mode
// P[0..B]: prefix sums of the clamped sequence lengths, formed by the whole workgroup:
// thread t sums the block of per = ceil(B / 256) <= 32 sequences from t per (all loads
// issued before any is used; reads past B return 0), a wave scan and the 4 wave totals give
// the block offsets. Ends with a workgroup barrier.
__device__ __forceinline__ void seq_prefix(const int32_t* __restrict__ seqlens, int B, int L_max, int* P) {
    constexpr int MAXPER = (kDecodeRangeMaxB + NT - 1) / NT;
    __shared__ int wsum[NW];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int per = (B + NT - 1) / NT;
    const auto rs = make_rsrc(seqlens, (uint32_t)B * 4u);
    int n[MAXPER];
#pragma unroll
    for (int i = 0; i < MAXPER; ++i)
        n[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(
            rs, i < per ? (uint32_t)(tid * per + i) * 4u : 0x7FFFFFF0u, 0, 0);
    int sum = 0;
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
        n[i] = clamp_len(n[i], L_max);
        sum += n[i];
    }
    int x = sum;  // inclusive scan over the wave
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int run = x - sum;
    for (int i = 0; i < w; ++i) run += wsum[i];
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
        run += n[i];
        const int b = tid * per + i;
        if (i < per && b < B) P[b + 1] = run;
    }
    if (tid == 0) P[0] = 0;
    __syncthreads();
}

// First sequence b in [0, B] with H P[b] >= x (requires H P[B] >= x). Each round the 64 lanes
// test 64 evenly spaced candidates and a ballot keeps the interval holding the answer, so
// B <= 8192 needs at most 3 rounds. Wave-uniform.
__device__ __forceinline__ int first_seq_from(const int* P, int B, int H, int x) {
    const int lane = __lane_id();
    int lo = 0, hi = B;
    while (lo < hi) {
        const int stride = (hi - lo + 62) / 63;  // lane 63 tests hi
        const bool p = H * P[min(lo + lane * stride, hi)] >= x;
        const int l = __builtin_ctzll(__builtin_amdgcn_ballot_w64(p));
        if (l == 0) break;  // the answer is lo
        const int t_hit = min(lo + l * stride, hi);
        lo = rfl(lo + (l - 1) * stride + 1);
        hi = rfl(t_hit);
    }
    return lo;
}

// Position x of the flat range: the (b, h) holding row x, its start F and length n, and the
// offset j = x - F; when x is a (b, h) start (j = 0) it is the first such (b, h), which may
// be empty. b == B means x == W with no (b, h) left.
struct Loc {
    int b, h, F, n, j;
};
__device__ __forceinline__ Loc locate(const int* P, int B, int H, int x) {
    const int b = first_seq_from(P, B, H, x);
    const int Pb = rfl(P[b]);
    Loc L;
    if (H * Pb == x) {
        L.b = b;
        L.h = 0;
        L.F = x;
        L.j = 0;
        L.n = b < B ? rfl(P[b + 1]) - Pb : 0;
        return L;
    }
    const int Pp = rfl(P[b - 1]);  // H P[b-1] < x < H P[b]: sequence b - 1 is not empty
    L.b = b - 1;
    L.n = Pb - Pp;
    L.h = (x - H * Pp) / L.n;
    L.F = H * Pp + L.h * L.n;
    L.j = x - L.F;
    return L;
}

// Slice boundary g of G over W rows; "whole" plans move it to the next (b, h) start.
template <bool WHOLE>
__device__ __forceinline__ int boundary(const int* P, int B, int H, int W, int g, int G) {
    const int x = (int)((long long)g * W / G);
    if (!WHOLE) return x;
    const Loc L = locate(P, B, H, x);
    return L.j > 0 ? L.F + L.n : x;
}

template <bool WHOLE, bool PROBE>
__global__ __launch_bounds__(NT, 4) void decode_range_bf16_d128_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ rho, const __bf16* __restrict__ kc,
    const __bf16* __restrict__ vc, const int32_t* __restrict__ seqlens, __bf16* __restrict__ o,
    float* __restrict__ ws, int B, int H, int L_max, float c) {
    extern __shared__ int P[];  // B + 1 prefix sums
    __shared__ __attribute__((aligned(16))) float ush[NW][2][KB];
    seq_prefix(seqlens, B, L_max, P);

    const int lane = threadIdx.x & 63;
    const int w = rfl(threadIdx.x >> 6);
    const int col = lane & 15, g = lane >> 4;
    const int G = gridDim.x * NW, gw = blockIdx.x * NW + w;
    const bool last = gw == G - 1;  // also takes empty (b, h) at the very end
    const int W = H * rfl(P[B]);
    const int r0 = boundary<WHOLE>(P, B, H, W, gw, G);
    const int r1 = boundary<WHOLE>(P, B, H, W, gw + 1, G);

    // Cursor over this slice: (b, h) with start F and length n; the piece [j, je) of it.
    const Loc L = locate(P, B, H, r0);
    int b = L.b, h = L.h, F = L.F, n = L.n, j = L.j, js = L.j;
    bool more = b < B && (j > 0 || F < r1 || last);
    int je = last ? n : min(n, r1 - F);

    struct Step {
        int it, kb0, je, js, n;
        bool valid, last;
    };
    // Next step of KB rows; a piece with no rows (an empty (b, h), or an empty slice inside
    // a (b, h)) still takes one step so that its output or partial gets written.
    auto next = [&]() {
        Step s;
        s.valid = more;
        s.it = b * H + h;
        s.kb0 = j;
        s.je = je;
        s.js = js;
        s.n = n;
        s.last = j + KB >= je;
        if (!s.last) {
            j += KB;
            return s;
        }
        F += n;
        if (++h == H) {
            h = 0;
            ++b;
            n = b < B ? rfl(P[b + 1]) - rfl(P[b]) : 0;
        }
        more = b < B && (F < r1 || last);
        j = js = 0;
        je = last ? n : min(n, r1 - F);
        return s;
    };
    Acc acc;
    acc.reset();
    // End of a piece: the whole (b, h) range writes o, a cut piece writes its partial to
    // slot 0 (piece starts inside the (b, h)) or 1 (piece starts at the (b, h) start).
    auto finish = [&](const Step& s) {
        decode::wave_totals<PROBE>(acc);
        const float l = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc.rsum), 0));
        const float beta = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc.rsum), 1));
        if (s.js == 0 && s.je == s.n) {
            if (lane < 16) {
                uint32_t pk[4];
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    pk[p] = pack_bf16x2(combine_out(acc.a1[2 * p], acc.a2[2 * p], l, beta),
                                        combine_out(acc.a1[2 * p + 1], acc.a2[2 * p + 1], l, beta));
                *(u32x4*)(o + (size_t)s.it * D + 8 * lane) = u32x4{pk[0], pk[1], pk[2], pk[3]};
            }
        } else {
            float* rec = ws + ((size_t)gw * 2 + (s.js > 0 ? 0 : 1)) * REC;
            if (lane < 16) {
                *(f32x4*)(rec + 8 * lane) = f32x4{acc.a1[0], acc.a1[1], acc.a1[2], acc.a1[3]};
                *(f32x4*)(rec + 8 * lane + 4) = f32x4{acc.a1[4], acc.a1[5], acc.a1[6], acc.a1[7]};
                *(f32x4*)(rec + D + 8 * lane) = f32x4{acc.a2[0], acc.a2[1], acc.a2[2], acc.a2[3]};
                *(f32x4*)(rec + D + 8 * lane + 4) =
                    f32x4{acc.a2[4], acc.a2[5], acc.a2[6], acc.a2[7]};
            }
            if (lane == 0) *(f32x4*)(rec + 2 * D) = f32x4{acc.m_run, l, beta, 0.f};
        }
        acc.reset();
    };

    // One step in flight per wave; latency is hidden by the other waves of the compute unit
    // (16 at this kernel's register count).
    Frag f;
    bf16x8 bqr[4];
    while (more) {
        const Step s = next();
        // q and rho of the step's (b, h), reloaded every step (cache hits after the first):
        // lane (col, g) reads column col's dims 32 st + 8 g .. +7 and keeps them for col < 2.
        const __bf16* qr_src = (PROBE && col == 1 ? rho : q) + (size_t)s.it * D + 8 * g;
        u32x4 xq[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) xq[st] = *(const u32x4*)(qr_src + 32 * st);
        const size_t row0 = (size_t)s.it * L_max;
        const uint32_t range = (uint32_t)s.je * 256u;
        decode::load_step(make_rsrc(kc + row0 * D, range), make_rsrc(vc + row0 * D, range),
                          s.kb0, col, g, f);
        __builtin_amdgcn_sched_barrier(0);  // every load of the step is issued before any wait
#pragma unroll
        for (int st = 0; st < 4; ++st)
            bqr[st] = as_bf16x8(col == 0 || (PROBE && col == 1) ? xq[st] : u32x4{});
        decode::consume<PROBE>(acc, f, bqr, s.kb0, s.je, c, ush[w], col, g);
        if (s.last) finish(s);
    }
}

// Merges the pieces of every (b, h) that slice boundaries cut: wave g (1 <= g < G) looks at
// boundary g; if it is the first boundary inside a (b, h), the pieces are wave g-1's slot 1
// and slot 0 of waves g, g+1, ... whose slices start inside that (b, h).
__global__ __launch_bounds__(NT) void decode_range_combine_kernel(
    const float* __restrict__ ws, __bf16* __restrict__ o, const int32_t* __restrict__ seqlens,
    int B, int H, int L_max, int G) {
    extern __shared__ int P[];
    seq_prefix(seqlens, B, L_max, P);
    const int lane = threadIdx.x & 63;
    const int gb = blockIdx.x * NW + rfl(threadIdx.x >> 6) + 1;
    if (gb >= G) return;
    const int W = H * rfl(P[B]);
    auto R = [&](int k) { return (int)((long long)k * W / G); };
    const Loc L = locate(P, B, H, R(gb));
    if (L.b >= B || L.j == 0 || R(gb - 1) > L.F) return;
    const int E = L.F + L.n;
    int np = 1;
    while (gb + np - 1 < G && R(gb + np - 1) < E) ++np;
    Merge st;
    fold_records(st, np,
                 [&](int u) {
                     return u == 0 ? ws + ((size_t)(gb - 1) * 2 + 1) * REC
                                   : ws + ((size_t)(gb + u - 1) * 2) * REC;
                 },
                 lane);
    store_merged(st, o + ((size_t)L.b * H + L.h) * D, lane);
}


template <bool PROBE>
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    const float c = a.scale * kLog2e;
    const __bf16* rho = PROBE ? (const __bf16*)a.rho : (const __bf16*)a.q;
    if (a.waves > 0) {
        const int grid = a.waves / NW;
        const size_t lds = (size_t)(a.B + 1) * sizeof(int);
        if (a.whole)
            hipLaunchKernelGGL((decode_range_bf16_d128_kernel<true, PROBE>), dim3(grid), dim3(NT),
                               lds, stream, (const __bf16*)a.q, rho, (const __bf16*)a.k,
                               (const __bf16*)a.v, a.seqlens, (__bf16*)a.o, a.ws, a.B, a.H,
                               a.L_max, c);
        else
            hipLaunchKernelGGL((decode_range_bf16_d128_kernel<false, PROBE>), dim3(grid),
                               dim3(NT), lds, stream, (const __bf16*)a.q, rho,
                               (const __bf16*)a.k, (const __bf16*)a.v, a.seqlens, (__bf16*)a.o,
                               a.ws, a.B, a.H, a.L_max, c);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || a.whole || a.waves == 1) return e;
        hipLaunchKernelGGL(decode_range_combine_kernel, dim3((a.waves - 1 + NW - 1) / NW),
                           dim3(NT), lds, stream, (const float*)a.ws, (__bf16*)a.o, a.seqlens,
                           a.B, a.H, a.L_max, a.waves);
        return hipGetLastError();
    }
    const int BH = a.B * a.H;
    dim3 grid(a.splits, a.H, a.B);
    // Chunks of at most one step per wave run the one-register-set instance (the kernel's
    // chunk of a sequence is at most that of L_max).
    const bool deep = ((a.L_max + a.splits - 1) / a.splits + KB - 1) / KB * KB > KB * NW;
    auto split = [&](auto kern, const int32_t* table) {
        hipLaunchKernelGGL(kern, grid, dim3(NT), 0, stream, (const __bf16*)a.q, rho,
                           (const __bf16*)a.k, (const __bf16*)a.v, a.seqlens, (__bf16*)a.o, a.ws,
                           a.H, a.L_max, a.splits, c, table, table ? a.max_blocks : 0,
                           table ? a.block_log2 : 0, table ? a.num_blocks : 0);
    };
    if (a.table)
        deep ? split(decode_split_bf16_d128_kernel<PROBE, true, true>, a.table)
             : split(decode_split_bf16_d128_kernel<PROBE, true, false>, a.table);
    else
        deep ? split(decode_split_bf16_d128_kernel<PROBE, false, true>, nullptr)
             : split(decode_split_bf16_d128_kernel<PROBE, false, false>, nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    hipLaunchKernelGGL(decode_combine_kernel, dim3(BH), dim3(64), 0, stream, (const float*)a.ws,
                       (__bf16*)a.o, a.splits);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16_d128(const DecodeArgs& a, hipStream_t stream) {
    return a.rho ? launch_decode<true>(a, stream) : launch_decode<false>(a, stream);
}

hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(decode_combine_kernel, dim3(a.B * a.H), dim3(64), 0, stream,
                       (const float*)a.ws, (__bf16*)a.o, a.splits);
    return hipGetLastError();
}

}  // namespace plx
