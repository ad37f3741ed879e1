// probe_bf16.hip -- the probe producer: rho = gate_h * RoPE(gamma * RMSNorm_head(x W_R^T)),
// bf16 in/out, d = 128, gfx950.
//
// The probe is one matrix product from the layer input followed by its own RMSNorm, with RoPE
// on it as an option [agihunt review, method paragraph: a learned projection W_R gives
// rho = W_R x; rho gets its own RMSNorm, and RoPE on it helps; gist.science summary (Spanish),
// method section: rho_i = W_R x_i from the layer input]. A learned sigmoid gate on the probe
// appears in the review's mechanism-analysis paragraph; here it is a per-head multiplier, the
// sigmoid left to the caller.
//
// A workgroup computes a block of tokens x the 128 dims of HG heads as Y^T = W_R X^T on
// v_mfma_f32_16x16x32_bf16, each wave UG groups of 16 tokens. Narrow inputs: 4 waves; per
// 32-wide K step the head's W_R slice (128 rows padded by 16 bytes, so the operand reads are
// free of bank conflicts) is staged in LDS, double-buffered, and the B operand (x rows) is
// read straight from global memory. Wide inputs: 8 waves, 256 tokens; per 64-wide K step both
// the W_R slice and the x rows arrive by direct-to-LDS loads into a three-stage ring, two
// steps ahead, in unpadded chunk-swizzled rows.
// Narrow calls are bound by the per-token vector work of the epilogue, so there the RoPE
// frequencies come from a per-workgroup table, gamma from LDS, the gate is folded into the
// norm's scale, and with one K step two heads share each token's sines and cosines.
// Each lane then holds 32 dims (4 consecutive dims of each 16-dim block) of one token per
// group, so the RMSNorm sum of squares needs only 4 lanes, the RoPE pairs (i, i + 64) sit in
// the same lane, and rho is written with 8-byte row pieces in the [B, H, T, d] layout the
// attention kernels read. RoPE angles are reduced to a fraction of a turn with the product's
// rounding error (fma) added back, then fed to the hardware sine and cosine (which take
// turns).
#include "plx_device.hpp"
#include "plx_kernels.hpp"

namespace plx {
namespace {

constexpr int D = 128;
constexpr int kProbeNarrowC = 64;  // inputs up to this width take one token group per wave

// gamma of a call that passes none (RMSNorm without a learned scale)
__constant__ float kOnes[D] = {
    1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f,
    1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f,
    1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f,
    1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f,
    1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f,
    1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f,
    1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f,
    1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 raw_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xFFFFu), (int)bytes, 0x00020000};
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Six 16-byte direct-to-LDS loads of one K step of the wide instance: byte offsets w0, w1 of
// raw buffer rw into LDS bytes lw + 1024 i + 16 lane (i = 0, 1), and x0 .. x3 of rx into
// lx + 1024 i + 16 lane (bounds-checked: offsets past a buffer write zeros). One asm block, so
// that the compiler's wait accounting does not track them (it would make every LDS read after
// them wait); the caller waits (vmcnt) before the barrier that publishes the stage. M0 is
// restored on exit; the leading s_nop covers a VALU write of the resources' SGPRs just before.
__device__ __forceinline__ void dma_step(i32x4 rw, i32x4 rx, uint32_t lw, uint32_t lx,
                                         uint32_t w0, uint32_t w1, uint32_t x0, uint32_t x1,
                                         uint32_t x2, uint32_t x3) {
    uint32_t saved;
    asm volatile(
        "s_nop 4\n\t"
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %5, %3, 0 offen lds\n\t"
        "s_add_u32 m0, %1, 0x400\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %6, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %7, %4, 0 offen lds\n\t"
        "s_add_u32 m0, %2, 0x400\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %8, %4, 0 offen lds\n\t"
        "s_add_u32 m0, %2, 0x800\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %9, %4, 0 offen lds\n\t"
        "s_add_u32 m0, %2, 0xc00\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %10, %4, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lw), "s"(lx), "s"(rw), "s"(rx), "v"(w0), "v"(w1), "v"(x0), "v"(x1), "v"(x2),
          "v"(x3)
        : "memory", "scc");
}

// Sequence b and position t of token n = b T + t. Token indices fit 31 bits (the host checks
// B T C 2 < 2^31), so 32-bit division serves (a 64-bit one is a long instruction sequence).
__device__ __forceinline__ void seq_pos(int n, int T, int& b, int& t) {
    b = (int)((unsigned)n / (unsigned)T);
    t = n - b * T;
}

// UG groups of 16 tokens per wave: UG = 2 lets every W_R operand read feed two products (wide
// inputs, matrix-bound; 8 waves, 256 tokens per workgroup); UG = 1 halves the accumulators so
// that more waves are resident (narrow inputs; 4 waves, 64 tokens). HG heads per workgroup,
// one after the other: for inputs of at most 32 (one K step) both heads' W_R slices are staged
// at once, and the RoPE sines and cosines, which depend on the token and not on the head, are
// evaluated once for both (narrow calls are bound by this per-token vector work).
template <int UG, int HG>
__global__ __launch_bounds__(UG == 2 ? 512 : 256, UG == 1 ? 4 : 2) void probe_bf16_d128_kernel(
    const __bf16* __restrict__ x, const __bf16* __restrict__ wr, const float* __restrict__ gamma,
    const float* __restrict__ gate, const int32_t* __restrict__ positions, __bf16* __restrict__ rho,
    int B, int T, int C, int H, float eps, float log2_base) {
    constexpr uint32_t OOB = 0xFFFFFFF0u;  // past every resource: reads as zeros
    // WIDE (UG = 2): K steps of 64; both operands of each step (the head's W_R slice, 128 rows,
    // and the workgroup's 256 x rows, 128 bytes each) arrive by direct-to-LDS loads into a ring
    // of three stages, two steps ahead; rows unpadded, chunk c of row r at c ^ ((r >> 1) & 7)
    // (the 16 rows of an operand read, two per 256-byte line of the banks, hit 16 distinct
    // bank positions). The output rows reuse the ring after the K loop.
    // Narrow (UG = 1): K steps of 32, the W_R slice staged through registers into rows padded
    // to 80 bytes (free of bank conflicts), double-buffered; x rows read straight from global
    // memory as the B operand.
    constexpr bool WIDE = UG == 2;
    constexpr int NTK = WIDE ? 512 : 256;
    constexpr int NW = NTK / 64;
    constexpr int KS = WIDE ? 64 : 32;
    constexpr int WR = KS + 8;  // narrow: LDS row stride of the W_R slice (bf16)
    constexpr int TOK = NW * 16 * UG;  // tokens per workgroup
    constexpr int X_OFF = D * KS * 2;  // wide: bytes of a stage's W_R slice
    constexpr int STAGE = X_OFF + TOK * KS * 2;
    constexpr int WL_BYTES = WIDE ? 3 * STAGE : 2 * D * WR * 2;
    constexpr int OT_BYTES = NW * 16 * (D + 8) * 2;
    constexpr int SMEM = WIDE ? (WL_BYTES > OT_BYTES ? WL_BYTES : OT_BYTES) : WL_BYTES + OT_BYTES;
    __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
    __bf16* const wl = (__bf16*)smem;  // narrow: slices b = 0, 1 at wl + b D WR
    __bf16 (*const ot)[16][D + 8] =    // output rows
        reinterpret_cast<__bf16 (*)[16][D + 8]>(smem + (WIDE ? 0 : WL_BYTES));
    __shared__ __attribute__((aligned(16))) float turn_tab[D / 2];  // turns per position, per pair
    __shared__ __attribute__((aligned(16))) float gam[D];           // gamma (ones if none)
    static_assert(HG == 1 || HG == 2, "heads per workgroup");
    static_assert(!WIDE || HG == 1, "the wide instance takes one head per workgroup");
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c16 = lane & 15, g = lane >> 4;
    const int h0 = blockIdx.y * HG;
    const long long N = (long long)B * T;
    long long tok[UG];
    bool tok_ok[UG];
    uint32_t xrow[UG];
#pragma unroll
    for (int u = 0; u < UG; ++u) {
        tok[u] = (long long)blockIdx.x * TOK + 16 * UG * w + 16 * u + c16;
        tok_ok[u] = tok[u] < N;
        xrow[u] = tok_ok[u] ? (uint32_t)(tok[u] * C) * 2u : OOB;
    }
    const auto rx = make_rsrc(x, (uint32_t)(N * C * 2));  // < 2^31 (checked on the host)
    auto rw_of = [&](int h) { return make_rsrc(wr + (size_t)h * D * C, (uint32_t)D * C * 2u); };
    const auto rw = rw_of(h0);

    // Staging: thread tid copies 16-byte piece tid % PR (PR = KS / 8 pieces per row) of rows
    // tid / PR + (256 / PR) r, r = 0 .. NR - 1.
    constexpr int PR = KS / 8, NR = 2 * PR / 4;
    const int sr = tid / PR, sp = tid % PR;
    auto stage = [&](int k0, u32x4 (&st)[NR]) {
        const int kc = k0 + 8 * sp;
#pragma unroll
        for (int r = 0; r < NR; ++r)
            st[r] = load16(rw, kc < C ? (uint32_t)((sr + (256 / PR) * r) * C + kc) * 2u : OOB);
    };
    auto put = [&](int buf, const u32x4 (&st)[NR]) {
#pragma unroll
        for (int r = 0; r < NR; ++r)
            *(u32x4*)&wl[buf * D * WR + (sr + (256 / PR) * r) * WR + 8 * sp] = st[r];
    };

    // Everything the workgroup reads from memory besides the later K steps is requested up
    // front, so that the W_R slice, the first x rows, gamma, the gate and the positions arrive
    // in one round trip instead of one after another.
    // x rows of one K step: lane (token c16, g) holds k-slots 32 h + 8 g .. +7, h < KS / 32.
    constexpr int KH = KS / 32;
    auto load_x = [&](int k0, bf16x8 (&bx)[UG][KH]) {
#pragma unroll
        for (int h = 0; h < KH; ++h) {
            const int kc = k0 + 32 * h + 8 * g;
#pragma unroll
            for (int u = 0; u < UG; ++u)
                bx[u][h] = as_bf16x8(load16(rx, tok_ok[u] && kc < C ? xrow[u] + 2u * kc : OOB));
        }
    };
    bf16x8 bx[UG][KH];
    // Wide: lane (row r, position p) of load i fetches chunk p ^ ((r >> 1) & 7) of its row:
    // W_R rows 16 w + 8 i + (lane >> 3) (i < 2), x rows 32 w + 8 i + (lane >> 3) (i < 4).
    const int nst = (C + KS - 1) / KS;
    const auto rwd = raw_rsrc(wr + (size_t)h0 * D * C, (uint32_t)D * C * 2u);
    const auto rxd = raw_rsrc(x, (uint32_t)(N * C * 2));
    auto dma = [&](int k, int stg) {
        const int k0 = k * KS;
        const int l3 = lane >> 3, sw = (lane & 7) ^ (l3 >> 1);
        uint32_t o[6];
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            const int kc = k0 + 8 * (i < 2 ? (sw ^ (4 * i & 7)) : (sw ^ (4 * (i - 2) & 7)));
            if (i < 2) {
                const int r = 16 * w + 8 * i + l3;
                o[i] = kc < C ? (uint32_t)(r * C + kc) * 2u : OOB;
            } else {
                const long long t = (long long)blockIdx.x * TOK + 32 * w + 8 * (i - 2) + l3;
                o[i] = t < N && kc < C ? (uint32_t)(t * C + kc) * 2u : OOB;
            }
        }
        const uint32_t base = lds_addr(smem + stg * STAGE);
        dma_step(rwd, rxd, base + 16 * w * 128, base + X_OFF + 32 * w * 128, o[0], o[1], o[2],
                 o[3], o[4], o[5]);
    };
    if constexpr (WIDE) {
        dma(0, 0);
        if (nst > 1) dma(1, 1);
    } else {
        load_x(0, bx);
    }
    if (tid < D) gam[tid] = (gamma ? gamma : kOnes)[tid];  // published by the K loop's barriers
    // Token group u (16 consecutive tokens from tg0[u]) usually lies in one sequence (b0, from
    // position t0): then a lane's position and the group's output rows follow by addition.
    int tg0[UG], b0[UG], t0[UG];
    bool one_seq[UG];
    int pos0[UG];
#pragma unroll
    for (int u = 0; u < UG; ++u) {
        tg0[u] = (int)((long long)blockIdx.x * TOK + 16 * UG * w + 16 * u);
        seq_pos(tg0[u] < N ? tg0[u] : 0, T, b0[u], t0[u]);
        one_seq[u] = tg0[u] + 15 < N && t0[u] + 15 < T;
        int bl = b0[u];
        if (!one_seq[u]) {
            int tl;
            seq_pos(tok_ok[u] ? (int)tok[u] : 0, T, bl, tl);
        }
        pos0[u] = positions ? positions[bl] : 0;
    }
    // Turns per position of rotation pair p (dims p and p + 64): base^(-2 p / d) / (2 pi),
    // the same for every token and head: formed once per workgroup.
    if (tid < D / 2)
        turn_tab[tid] = log2_base > 0.f
                            ? exp2f(-(2.f * tid / D) * log2_base) * 0.15915494309189535f
                            : 0.f;

    f32x4 acc[UG][8];
    u32x4 st[NR];
    if constexpr (!WIDE) stage(0, st);
    if constexpr (HG == 2) {  // C <= 32: the second head's slice goes to the other buffer
        const int kc = 8 * sp;
        const auto rw1 = rw_of(h0 + 1);
        u32x4 st1[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r)
            st1[r] = load16(rw1, kc < C ? (uint32_t)((sr + 64 * r) * C + kc) * 2u : OOB);
        put(1, st1);
    }
    if constexpr (WIDE) {
        if (nst > 1) __builtin_amdgcn_s_waitcnt(0x0F76);  // vmcnt(6): step 0 is in LDS
        else __builtin_amdgcn_s_waitcnt(0x0F70);
    } else {
        put(0, st);
    }
    __syncthreads();
    // One K step; the first starts the accumulators from zero. Narrow inputs (one or two
    // steps) request each step's data in the step before.
    auto products = [&](int b, const bf16x8 (&x)[UG][KH], bool first) {
#pragma unroll
        for (int h = 0; h < KH; ++h)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const bf16x8 a =
                    *(const bf16x8*)&wl[b * D * WR + (16 * j + c16) * WR + 32 * h + 8 * g];
#pragma unroll
                for (int u = 0; u < UG; ++u)
                    acc[u][j] = mfma16(a, x[u][h], first && h == 0 ? f32x4{} : acc[u][j]);
            }
    };
    if constexpr (HG == 1 && UG == 1) {
        int buf = 0;
        for (int k0 = 0; k0 < C; k0 += KS) {
            const bool more = k0 + KS < C;
            if (more) stage(k0 + KS, st);
            if (k0 > 0) load_x(k0, bx);
            products(buf, bx, k0 == 0);
            if (more) put(buf ^ 1, st);
            __syncthreads();
            buf ^= 1;
        }
    } else {
        // Wide: step k reads stage k % 3 while the loads of step k + 2 fill stage (k + 2) % 3
        // (read in step k - 1, which ended with a barrier). Before the barrier that ends step
        // k, each wave waits for its own loads of step k + 1 (leaving those of step k + 2 in
        // flight), so that after it step k + 1 is in LDS. Operand reads: W_R row 16 j + c16
        // and x row 32 w + 16 u + c16, chunk 4 h + g at position (4 h + g) ^ ((c16 >> 1) & 7).
        int aoff[KH];
#pragma unroll
        for (int h = 0; h < KH; ++h) aoff[h] = c16 * 128 + 16 * ((4 * h + g) ^ ((c16 >> 1) & 7));
        int sk = 0, sk2 = 2;  // stages of steps k and k + 2
        for (int k = 0; k < nst; ++k) {
            const bool ahead = k + 2 < nst;
            if (ahead) dma(k + 2, sk2);
            const unsigned char* S = smem + sk * STAGE;
#pragma unroll
            for (int h = 0; h < KH; ++h) {
                bf16x8 b[UG];
#pragma unroll
                for (int u = 0; u < UG; ++u)
                    b[u] = *(const bf16x8*)(S + X_OFF + 32 * w * 128 + 2048 * u + aoff[h]);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const bf16x8 a = *(const bf16x8*)(S + 2048 * j + aoff[h]);
#pragma unroll
                    for (int u = 0; u < UG; ++u)
                        acc[u][j] = mfma16(a, b[u], k == 0 && h == 0 ? f32x4{} : acc[u][j]);
                }
            }
            // interleave the step's LDS reads with its products (measured: 73.7 -> 69.5 us at
            // C = 2048)
            __builtin_amdgcn_iglp_opt(0);
            if (ahead) __builtin_amdgcn_s_waitcnt(0x0F76);  // vmcnt(6)
            else __builtin_amdgcn_s_waitcnt(0x0F70);        // vmcnt(0)
            __syncthreads();
            sk = sk == 2 ? 0 : sk + 1;
            sk2 = sk2 == 2 ? 0 : sk2 + 1;
        }
    }

    // acc[u][j][i]: dim 16 j + 4 g + i of token tok[u]. The lane's 16 rotation pairs are
    // p = 16 j + 4 g + i, j < 4 (the table was published by the K loop's barriers).
    f32x4 turns[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) turns[j] = *(const f32x4*)&turn_tab[16 * j + 4 * g];
    float rc[UG][4][4], rs[UG][4][4];  // cosine and sine of the lane's 16 rotation angles
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
        const int h = h0 + hh;
        if constexpr (HG == 2) {  // the one K step of this head, from its staged slice
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const bf16x8 a = *(const bf16x8*)&wl[hh * D * WR + (16 * j + c16) * WR + 8 * g];
#pragma unroll
                for (int u = 0; u < UG; ++u) acc[u][j] = mfma16(a, bx[u][0], f32x4{});
            }
        }
        const float gh = gate ? gate[h] : 1.f;
#pragma unroll
        for (int u = 0; u < UG; ++u) {
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) ss = fmaf(acc[u][j][i], acc[u][j][i], ss);
            ss += shfl_xor(ss, 16);
            ss += shfl_xor(ss, 32);
            // the gate is a scalar, so it commutes with the rotation: fold it into the norm
            const float sc = gh * __builtin_amdgcn_rsqf(ss * (1.f / D) + eps);
            int t = t0[u] + c16;
            if (!one_seq[u]) {
                int b;
                seq_pos(tok_ok[u] ? (int)tok[u] : 0, T, b, t);
            }
            float n[8][4];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const f32x4 gmv = *(const f32x4*)&gam[16 * j + 4 * g];
#pragma unroll
                for (int i = 0; i < 4; ++i) n[j][i] = gmv[i] * acc[u][j][i] * sc;
            }
            if (log2_base > 0.f) {
                if (hh == 0) {
                    const float pos = (float)(pos0[u] + t);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            // fraction of a turn: p + e = pos * turns exactly (e from the fma),
                            // less the nearest whole number of turns
                            const float p = pos * turns[j][i];
                            const float e = fmaf(pos, turns[j][i], -p);
                            const float fr = (p - rintf(p)) + e;
                            rs[u][j][i] = __builtin_amdgcn_sinf(fr);
                            rc[u][j][i] = __builtin_amdgcn_cosf(fr);
                        }
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float lo = n[j][i], hi = n[j + 4][i];
                        n[j][i] = lo * rc[u][j][i] - hi * rs[u][j][i];
                        n[j + 4][i] = hi * rc[u][j][i] + lo * rs[u][j][i];
                    }
            }
            // The group's 16 rows go through LDS so that each store writes whole 256-byte rows:
            // lane (c16, g) then stores 16-byte piece c16 of rows 4 r + g, r = 0..3.
#pragma unroll
            for (int j = 0; j < 8; ++j)
                *(u32x2*)&ot[w][c16][16 * j + 4 * g] = u32x2{pack_bf16x2(n[j][0], n[j][1]),
                                                          pack_bf16x2(n[j][2], n[j][3])};
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            __bf16* const row0 = rho + (((size_t)b0[u] * H + h) * T + t0[u]) * D + 8 * c16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * r + g;
                const int tr = tg0[u] + row;
                const u32x4 val = *(const u32x4*)&ot[w][row][8 * c16];
                if (one_seq[u]) {
                    *(u32x4*)(row0 + (size_t)row * D) = val;
                } else if (tr < N) {
                    int br, trr;
                    seq_pos(tr, T, br, trr);
                    *(u32x4*)(rho + (((size_t)br * H + h) * T + trr) * D + 8 * c16) = val;
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }
}

}  // namespace

hipError_t launch_probe_bf16_d128(const ProbeArgs& a, hipStream_t stream) {
    const long long N = (long long)a.B * a.T;
    const float lb = a.rope_base > 0.f ? log2f(a.rope_base) : 0.f;
    auto go = [&](auto kernel, int tok, int hg, int nt) {
        const long long nblk = (N + tok - 1) / tok;
        if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(kernel, dim3((unsigned)nblk, a.H / hg), dim3(nt), 0, stream,
                           (const __bf16*)a.x, (const __bf16*)a.w_r, a.gamma, a.gate,
                           a.positions, (__bf16*)a.rho, a.B, a.T, a.C, a.H, a.eps, lb);
        return hipGetLastError();
    };
    // Narrow inputs (one K step or two): one token group per wave; with one K step and an even
    // head count, two heads per workgroup. Measured at 4 x 2048 tokens, H = 16: see the probe
    // producer's profile.
    if (a.C <= 32 && a.H % 2 == 0) return go(probe_bf16_d128_kernel<1, 2>, 64, 2, 256);
    if (a.C <= kProbeNarrowC) return go(probe_bf16_d128_kernel<1, 1>, 64, 1, 256);
    return go(probe_bf16_d128_kernel<2, 1>, 256, 1, 512);
}

}  // namespace plx
