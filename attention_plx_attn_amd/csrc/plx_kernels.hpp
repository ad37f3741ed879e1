// plx_kernels.hpp -- host-side launch interface of the Parallax kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace plx {

struct PrefillArgs {
    int B, H, T, d;
    const void* q;
    const void* k;
    const void* v;
    const void* rho;
    void* o;
    float scale;
    int workers;  // resident workgroups of a persistent launch (the device's compute units)
    void* vbar = nullptr;    // O1 / l per row [B, H, T, d] (bf16), or nullptr
    float* stats = nullptr;  // with vbar: (lse, tbar) per row [B, H, T, 2]
    bool split = false;      // weights as hi + lo bf16 terms (bf16 path, without stats)
};

// Backward of the causal prefill (bf16, d = 64 or 128). All tensors [B, H, T, d] except
// stats [B, H, T, 2] (lse, tbar from the forward) and ws [B, H, T] x 4 floats (per-row records
// the dq kernel writes for the dk kernel).
struct PrefillBwdArgs {
    int B, H, T, d;
    const void *q, *k, *v, *rho, *o, *vbar;
    const float* stats;
    const void* dout;
    void *dq, *dk, *dv, *drho;
    float* ws;
    float scale;
};

struct DecodeArgs {
    int B, H, L_max, d;
    const void* q;
    const void* rho;
    const void* k;
    const void* v;
    const int32_t* seqlens;
    void* o;
    float scale;
    int splits;  // split mode: chunks per (b, h) actually launched
    int chunk;   // keys per chunk of the L_max plan (the kernel splits each sequence evenly)
    float* ws;   // partials: split mode [B*H*splits][kDecodeRecord] floats (unused if
                 // splits == 1); wave-range mode [waves][2][kDecodeRecord] (unused if whole)
    int waves;   // > 0: wave-range mode with this many waves (a multiple of 4); 0: split mode
    int whole;   // wave-range mode: slices end at (b, h) boundaries, no partials
    // Paged cache (split mode only): k, v are pools [num_blocks, H, 2^block_log2, d] and
    // table [B][max_blocks] names each sequence's blocks; L_max = max_blocks 2^block_log2.
    const int32_t* table = nullptr;
    int max_blocks = 0, block_log2 = 0, num_blocks = 0;
};

constexpr int kDecodeRecord = 2 * 128 + 4;  // A1[128], A2[128], m, l, beta, pad
constexpr int kDecodeRangeMaxB = 8192;      // wave-range mode keeps B + 1 prefix sums in LDS
constexpr int kDecodeRangeMaxWaves = 1 << 16;

struct ProbeArgs {
    int B, T, C, H;            // tokens [B, T], input width C, heads H (d = 128)
    const void* x;             // [B, T, C]
    const void* w_r;           // [H * d, C]
    const float* gamma;        // [d] RMSNorm weight or nullptr (1)
    const float* gate;         // [H] per-head multiplier or nullptr (1)
    const int32_t* positions;  // [B] position of token 0 of each sequence, or nullptr (0)
    void* rho;                 // [B, H, T, d]
    float eps, rope_base;      // rope_base 0: no rotation
};

bool prefill_f32_supported(int d);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);
// bf16 prefill, d = 64 or 128 (with vbar and stats: the statistics the backward starts from).
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_bwd_bf16(const PrefillBwdArgs& a, hipStream_t stream);
hipError_t launch_decode_bf16_d128(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_probe_bf16_d128(const ProbeArgs& a, hipStream_t stream);
// Grouped query heads: a.H query heads over Hkv cache heads (a.H / Hkv in {1, 2, 4, 8}), a.d
// 128 or 64, split mode with a.splits chunks; partials in the split decode's record layout
// of that head dim, per query head; a paged cache when a.table is set.
hipError_t launch_decode_gqa_bf16(const DecodeArgs& a, int Hkv, hipStream_t stream);
// The split decode's combines: merge a.splits records per (b, query head) into o (d = 128,
// d = 64).
hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_combine_d64(const DecodeArgs& a, hipStream_t stream);

}  // namespace plx
