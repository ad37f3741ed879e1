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
// One workgroup (4 waves) computes 64 UG tokens x the 128 dims of one head as
// Y^T = W_R X^T on v_mfma_f32_16x16x32_bf16: per 32-wide K step the workgroup stages the
// head's W_R slice (128 rows x 64 bytes, rows padded to 80 bytes so the operand reads are
// free of bank conflicts) in LDS, double-buffered, and every wave reads its A operand blocks
// there; the B operand is UG 16-token groups of x rows read straight from global memory.
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
constexpr int NT = 256;
constexpr int WROW = 40;     // LDS row stride of the W_R slice (bf16): 80 bytes
constexpr int WBUF = D * WROW;
constexpr int kProbeNarrowC = 64;  // inputs up to this width take one token group per wave

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Sequence b and position t of token n = b T + t. Token indices fit 31 bits (the host checks
// B T C 2 < 2^31), so 32-bit division serves (a 64-bit one is a long instruction sequence).
__device__ __forceinline__ void seq_pos(int n, int T, int& b, int& t) {
    b = (int)((unsigned)n / (unsigned)T);
    t = n - b * T;
}

// UG groups of 16 tokens per wave, 64 UG tokens per workgroup: UG = 2 lets every W_R operand
// read feed two products (wide inputs, matrix-bound); UG = 1 halves the accumulators so that
// more waves are resident (narrow inputs, where the call is bound by latency and the writes).
template <int UG>
__global__ __launch_bounds__(NT) void probe_bf16_d128_kernel(
    const __bf16* __restrict__ x, const __bf16* __restrict__ wr, const float* __restrict__ gamma,
    const float* __restrict__ gate, const int32_t* __restrict__ positions, __bf16* __restrict__ rho,
    int B, int T, int C, int H, float eps, float log2_base) {
    constexpr uint32_t OOB = 0xFFFFFFF0u;  // past every resource: reads as zeros
    __shared__ __attribute__((aligned(16))) __bf16 wl[2][WBUF];
    __shared__ __attribute__((aligned(16))) __bf16 ot[NT / 64][16][D + 8];  // output rows
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c16 = lane & 15, g = lane >> 4;
    constexpr int TOK = 64 * UG;  // tokens per workgroup
    const int h = blockIdx.y;
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
    const auto rw = make_rsrc(wr + (size_t)h * D * C, (uint32_t)D * C * 2u);

    // Staging: thread tid copies 16-byte pieces (tid & 3) of rows tid >> 2 and 64 + (tid >> 2).
    const int sr = tid >> 2, sp = tid & 3;
    auto stage = [&](int k0, u32x4 (&st)[2]) {
        const int kc = k0 + 8 * sp;
#pragma unroll
        for (int r = 0; r < 2; ++r)
            st[r] = load16(rw, kc < C ? (uint32_t)((sr + 64 * r) * C + kc) * 2u : OOB);
    };
    auto put = [&](int buf, const u32x4 (&st)[2]) {
#pragma unroll
        for (int r = 0; r < 2; ++r) *(u32x4*)&wl[buf][(sr + 64 * r) * WROW + 8 * sp] = st[r];
    };

    // Everything the workgroup reads from memory besides the later K steps is requested up
    // front, so that the W_R slice, the first x rows, gamma, the gate and the positions arrive
    // in one round trip instead of one after another.
    auto load_x = [&](int k0, bf16x8 (&bx)[UG]) {
        const int kc = k0 + 8 * g;
#pragma unroll
        for (int u = 0; u < UG; ++u)
            bx[u] = as_bf16x8(load16(rx, tok_ok[u] && kc < C ? xrow[u] + 2u * kc : OOB));
    };
    bf16x8 bx[UG];
    load_x(0, bx);
    f32x4 gmv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        gmv[j] = gamma ? *(const f32x4*)(gamma + 16 * j + 4 * g) : f32x4{1.f, 1.f, 1.f, 1.f};
    const float gh = gate ? gate[h] : 1.f;
    int pos0[UG];
#pragma unroll
    for (int u = 0; u < UG; ++u) {
        const int tk = tok_ok[u] ? (int)tok[u] : 0;
        pos0[u] = positions ? positions[(unsigned)tk / (unsigned)T] : 0;
    }

    f32x4 acc[UG][8];
#pragma unroll
    for (int u = 0; u < UG; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[u][j] = f32x4{};
    u32x4 st[2];
    stage(0, st);
    put(0, st);
    __syncthreads();
    int buf = 0;
    for (int k0 = 0; k0 < C; k0 += 32) {
        const bool more = k0 + 32 < C;
        if (more) stage(k0 + 32, st);
        if (k0 > 0) load_x(k0, bx);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bf16x8 a = *(const bf16x8*)&wl[buf][(16 * j + c16) * WROW + 8 * g];
#pragma unroll
            for (int u = 0; u < UG; ++u) acc[u][j] = mfma16(a, bx[u], acc[u][j]);
        }
        if (more) put(buf ^ 1, st);
        __syncthreads();
        buf ^= 1;
    }

    // acc[u][j][i]: dim 16 j + 4 g + i of token tok[u].
    // Turns per position of the 16 rotation pairs this lane holds: base^(-2 di / d) / (2 pi).
    float turns[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            turns[j][i] = exp2f(-(2.f * (16 * j + 4 * g + i) / D) * log2_base) *
                          0.15915494309189535f;
#pragma unroll
    for (int u = 0; u < UG; ++u) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) ss = fmaf(acc[u][j][i], acc[u][j][i], ss);
        ss += shfl_xor(ss, 16);
        ss += shfl_xor(ss, 32);
        const float inv = 1.f / sqrtf(ss * (1.f / D) + eps);
        int b, t;
        seq_pos(tok_ok[u] ? (int)tok[u] : 0, T, b, t);
        float n[8][4];
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) n[j][i] = gmv[j][i] * acc[u][j][i] * inv;
        if (log2_base > 0.f) {
            const float pos = (float)(pos0[u] + t);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // fraction of a turn: p + e = pos * turns exactly (e from the fma), less
                    // the nearest whole number of turns
                    const float p = pos * turns[j][i];
                    const float e = fmaf(pos, turns[j][i], -p);
                    const float fr = (p - rintf(p)) + e;
                    const float sn = __builtin_amdgcn_sinf(fr), cs = __builtin_amdgcn_cosf(fr);
                    const float lo = n[j][i], hi = n[j + 4][i];
                    n[j][i] = lo * cs - hi * sn;
                    n[j + 4][i] = hi * cs + lo * sn;
                }
        }
        // The group's 16 rows go through LDS so that each store writes whole 256-byte rows:
        // lane (c16, g) then stores 16-byte piece c16 of rows 4 r + g, r = 0..3.
#pragma unroll
        for (int j = 0; j < 8; ++j)
            *(u32x2*)&ot[w][c16][16 * j + 4 * g] = u32x2{pack_bf16x2(gh * n[j][0], gh * n[j][1]),
                                                      pack_bf16x2(gh * n[j][2], gh * n[j][3])};
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 4 * r + g;
            const long long tr = (long long)blockIdx.x * TOK + 16 * UG * w + 16 * u + row;
            if (tr < N) {
                int br, trr;
                seq_pos((int)tr, T, br, trr);
                *(u32x4*)(rho + (((size_t)br * H + h) * T + trr) * D + 8 * c16) =
                    *(const u32x4*)&ot[w][row][8 * c16];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

}  // namespace

hipError_t launch_probe_bf16_d128(const ProbeArgs& a, hipStream_t stream) {
    const long long N = (long long)a.B * a.T;
    const float lb = a.rope_base > 0.f ? log2f(a.rope_base) : 0.f;
    auto go = [&](auto kernel, int tok) {
        const long long nblk = (N + tok - 1) / tok;
        if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(kernel, dim3((unsigned)nblk, a.H), dim3(NT), 0, stream,
                           (const __bf16*)a.x, (const __bf16*)a.w_r, a.gamma, a.gate,
                           a.positions, (__bf16*)a.rho, a.B, a.T, a.C, a.H, a.eps, lb);
        return hipGetLastError();
    };
    // Narrow inputs (one K step or two): one token group per wave. Measured at 4 x 2048 tokens,
    // H = 16: see the probe producer's profile.
    if (a.C <= kProbeNarrowC) return go(probe_bf16_d128_kernel<1>, 64);
    return go(probe_bf16_d128_kernel<2>, 128);
}

}  // namespace plx
