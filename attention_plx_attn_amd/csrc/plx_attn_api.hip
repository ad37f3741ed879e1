// plx_attn_api.hip -- the exported C ABI: argument validation, dispatch, split planning.
//
// Every entry point validates on the host before touching the HIP runtime, so an invalid
// call enqueues nothing. The only device query is the compute-unit count (cached per
// device) used by the decode split heuristic.
#include <atomic>
#include <climits>
#include <cmath>
#include <mutex>

#include "plx_attn.h"
#include "plx_kernels.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

// Compute units of the current device, queried once per device.
plx_status_t current_cu_count(int* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PLX_ERR_HIP;
    if (dev >= 0 && dev < kMaxDevices) {
        const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
        if (cached > 0) {
            *out = cached;
            return PLX_OK;
        }
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        return PLX_ERR_HIP;
    if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(cus, std::memory_order_relaxed);
    *out = cus;
    return PLX_OK;
}

constexpr int kDecodeWaveKeys = 64;      // chunk granularity (keys)
constexpr int kDecodeMinChunk = 256;     // at least one step per wave of a 4-wave workgroup
constexpr int kDecodeMaxSplits = 4096;
constexpr int kDecodeWgPerCu = 1;        // one streaming workgroup per compute unit (measured best)
// Ragged batches: with one chunk per (b, h) the longest sequences set the time. Long contexts
// are therefore split further, up to kDecodeBalanceWgPerCu workgroups per compute unit in all
// (enough for the dispatcher to even out the lengths as workgroups finish) and at most one
// chunk per kDecodeBalanceRows rows of L_max (shorter chunks cost more in per-workgroup
// overhead than they gain in balance). Measured on the decode grid (seqlens ~ U[ctx/2, ctx]):
// 16 x 32768 555 -> 474 us at 16 chunks, 128 x 32768 4154 -> 3794 us at 2, 16 x 4096 76 -> 72
// us at 2; contexts up to 2048 rows, and B H >= 32 CUs, keep one chunk.
constexpr int kDecodeBalanceWgPerCu = 32;
constexpr int kDecodeBalanceRows = 2048;
// Wave-range mode: slices end at (b, h) starts once there are 2 (b, h) per wave; it runs only
// when asked for (num_splits < 0). Short contexts use split mode with one chunk per (b, h):
// chunks of at most one step per wave run the one-register-set split kernel (four waves per
// SIMD), which measured ahead of wave-range mode on MI355X (B x ctx = 128 x 128: 23.1 vs
// 36.8 us; 512 x 128: 67.4 vs 76.6 us; 2048 x 128: 258.8 vs 280.0 us).
constexpr int kRangeWholeBhPerWave = 2;

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// Keys per chunk for a requested split count (a multiple of 64) and the chunks that result.
void chunk_plan(int L_max, int splits, int* chunk, int* launched) {
    int c = ceil_div(L_max, splits);
    c = ceil_div(c, kDecodeWaveKeys) * kDecodeWaveKeys;
    *chunk = c;
    *launched = ceil_div(L_max, c);
}

// How a decode call divides the cache: split mode (splits chunks of each (b, h)) or
// wave-range mode (waves equal slices of all (b, h) laid end to end).
struct DecodePlan {
    int splits = 1, chunk = 0;  // split mode
    int waves = 0;              // > 0: wave-range mode
    bool whole = false;         // wave-range slices end at (b, h) starts
    size_t ws_bytes = 0;
    int reported() const { return waves > 0 ? -waves : splits; }
};

bool range_mode_fits(int B, int H, int L_max) {
    return B <= plx::kDecodeRangeMaxB && (long long)B * H * L_max < (1LL << 31);
}

plx_status_t plan_decode(int B, int H, int L_max, int d_v, int num_splits, DecodePlan* p) {
    if (num_splits > kDecodeMaxSplits || num_splits < -plx::kDecodeRangeMaxWaves)
        return PLX_ERR_INVALID_ARG;
    *p = DecodePlan{};
    const long long bh = (long long)B * H;
    const size_t rec_bytes = (size_t)(2 * d_v + 4) * sizeof(float);
    const bool range_built = d_v == 128;  // wave-range mode exists at d = 128 only
    int waves = 0, splits = num_splits;
    if (num_splits < 0) {
        if (!range_built || !range_mode_fits(B, H, L_max)) return PLX_ERR_UNSUPPORTED;
        waves = ceil_div(-(long long)num_splits, 4) * 4;
    } else if (num_splits == 0) {
        int cus = 0;
        const plx_status_t st = current_cu_count(&cus);
        if (st != PLX_OK) return st;
        // split mode: fill the chip once with (b, h, chunk) workgroups
        long long s = (kDecodeWgPerCu * (long long)cus + bh - 1) / bh;
        long long s_bal = (kDecodeBalanceWgPerCu * (long long)cus + bh - 1) / bh;
        if (s_bal > L_max / kDecodeBalanceRows) s_bal = L_max / kDecodeBalanceRows;
        if (s < s_bal) s = s_bal;
        const long long smax = (L_max + kDecodeMinChunk - 1) / kDecodeMinChunk;
        if (s > smax) s = smax;
        if (s < 1) s = 1;
        if (s > kDecodeMaxSplits) s = kDecodeMaxSplits;
        splits = (int)s;
    }
    if (waves > 0) {
        p->waves = waves;
        p->whole = bh >= (long long)kRangeWholeBhPerWave * waves;
        p->ws_bytes = p->whole ? 0 : (size_t)waves * 2 * rec_bytes;
        return PLX_OK;
    }
    chunk_plan(L_max, splits, &p->chunk, &p->splits);
    p->ws_bytes = p->splits > 1 ? (size_t)bh * p->splits * rec_bytes : 0;
    return PLX_OK;
}

plx_status_t check_decode_shape(int B, int H, int L_max, int d_v) {
    if (B < 1 || H < 1 || L_max < 1 || d_v < 1) return PLX_ERR_INVALID_SHAPE;
    if ((long long)B * H > INT_MAX / 4) return PLX_ERR_INVALID_SHAPE;
    if ((long long)L_max * 256 >= (1LL << 31)) return PLX_ERR_INVALID_SHAPE;
    if (B > 65535 || H > 65535) return PLX_ERR_INVALID_SHAPE;  // grid y/z limits
    return PLX_OK;
}

// Shapes of the forward-with-statistics and the backward: bf16, d_qk = d_v in {64, 128}.
plx_status_t check_bwd_shape(plx_dtype_t dtype, int B, int H, int T, int d_qk, int d_v,
                             float scale) {
    if (B < 1 || H < 1 || T < 1 || d_qk < 1 || d_v < 1) return PLX_ERR_INVALID_SHAPE;
    if (!std::isfinite(scale) || scale < 0.f) return PLX_ERR_INVALID_ARG;
    if (dtype != PLX_BF16 || d_qk != d_v || (d_qk != 128 && d_qk != 64))
        return PLX_ERR_UNSUPPORTED;
    if ((long long)T * d_qk * 2 >= (1LL << 31)) return PLX_ERR_INVALID_SHAPE;
    if ((long long)B * H * ((T + 127) / 128) > INT_MAX) return PLX_ERR_INVALID_SHAPE;
    return PLX_OK;
}

// ---------------------------------------------------------------- no-allocation decode
// Scratch of plx_attn_decode_noalloc: the split partial records of a decode call, in a
// file-scope device array (one copy per GPU, held until the process ends). Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for the symbol): the
// device address of each GPU's copy is looked up once per device with hipGetSymbolAddress
// and kept here.
constexpr size_t kScratchBytes = PLX_DECODE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of the current device's `scratch`, looked up on the first call on a device
// (with that device current) and cached.
plx_status_t scratch_of_current_device(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PLX_ERR_HIP;
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (ptr == nullptr) {
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
                return PLX_ERR_HIP;
            g_scratch_ptr[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return PLX_OK;
}

plx_status_t decode_call(plx_dtype_t dtype, int32_t B, int32_t H, int32_t L_max, int32_t d_qk,
                         int32_t d_v, const void* q, const void* rho, const void* k_cache,
                         const void* v_cache, const int32_t* seqlens, void* o,
                         float softmax_scale, int32_t num_splits, void* workspace,
                         size_t workspace_bytes, void* stream, bool use_scratch);

}  // namespace

extern "C" {

const char* plx_status_string(plx_status_t s) {
    switch (s) {
        case PLX_OK: return "ok";
        case PLX_ERR_NULL_POINTER: return "a required pointer is NULL";
        case PLX_ERR_INVALID_SHAPE: return "invalid or too large shape";
        case PLX_ERR_INVALID_ARG: return "invalid argument (dtype, scale or split count)";
        case PLX_ERR_UNSUPPORTED: return "unsupported dtype / head-dim combination";
        case PLX_ERR_MISALIGNED: return "pointer not 16-byte aligned";
        case PLX_ERR_WORKSPACE_TOO_SMALL: return "decode workspace too small";
        case PLX_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

plx_status_t plx_attn_prefill(plx_dtype_t dtype, int32_t B, int32_t H, int32_t T,
                              int32_t d_qk, int32_t d_v, const void* q, const void* k,
                              const void* v, const void* rho, void* o, float softmax_scale,
                              void* stream) {
    return plx_attn_prefill_ex(dtype, B, H, T, d_qk, d_v, q, k, v, rho, o, softmax_scale, 0u,
                               stream);
}

plx_status_t plx_attn_prefill_ex(plx_dtype_t dtype, int32_t B, int32_t H, int32_t T,
                                 int32_t d_qk, int32_t d_v, const void* q, const void* k,
                                 const void* v, const void* rho, void* o, float softmax_scale,
                                 uint32_t flags, void* stream) {
    if (dtype != PLX_F32 && dtype != PLX_BF16) return PLX_ERR_INVALID_ARG;
    if (flags & ~(uint32_t)PLX_PREFILL_SPLIT_WEIGHTS) return PLX_ERR_INVALID_ARG;
    if (!q || !k || !v || !o) return PLX_ERR_NULL_POINTER;  // rho == NULL: softmax only
    if (B < 1 || H < 1 || T < 1 || d_qk < 1 || d_v < 1) return PLX_ERR_INVALID_SHAPE;
    if (!std::isfinite(softmax_scale) || softmax_scale < 0.f) return PLX_ERR_INVALID_ARG;
    const long long esize = dtype == PLX_BF16 ? 2 : 4;
    if ((long long)T * d_qk * esize >= (1LL << 31) || (long long)T * d_v * esize >= (1LL << 31))
        return PLX_ERR_INVALID_SHAPE;
    if ((long long)B * H > INT_MAX / 2) return PLX_ERR_INVALID_SHAPE;
    if (d_qk != d_v) return PLX_ERR_UNSUPPORTED;
    const bool ok = (dtype == PLX_BF16 && (d_qk == 128 || d_qk == 64)) ||
                    (dtype == PLX_F32 && plx::prefill_f32_supported(d_qk));
    if (!ok) return PLX_ERR_UNSUPPORTED;
    if (dtype == PLX_F32 && (B > 65535 || H > 65535)) return PLX_ERR_INVALID_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(rho) || !aligned16(o))
        return PLX_ERR_MISALIGNED;  // aligned16(NULL) holds

    int cus = 1;
    if (dtype == PLX_BF16) {
        const plx_status_t s = current_cu_count(&cus);
        if (s != PLX_OK) return s;
    }
    plx::PrefillArgs a{B, H, T, d_qk, q, k, v, rho, o, softmax_scale, cus};
    a.split = (flags & PLX_PREFILL_SPLIT_WEIGHTS) != 0;  // no rounding to split on fp32
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t e = dtype == PLX_BF16 ? plx::launch_prefill_bf16(a, st)
                                           : plx::launch_prefill_f32(a, st);
    return e == hipSuccess ? PLX_OK : PLX_ERR_HIP;
}

plx_status_t plx_attn_prefill_fwd(plx_dtype_t dtype, int32_t B, int32_t H, int32_t T,
                                  int32_t d_qk, int32_t d_v, const void* q, const void* k,
                                  const void* v, const void* rho, void* o, void* vbar,
                                  float* stats, float softmax_scale, void* stream) {
    if (dtype != PLX_F32 && dtype != PLX_BF16) return PLX_ERR_INVALID_ARG;
    if (!q || !k || !v || !o || !vbar || !stats) return PLX_ERR_NULL_POINTER;
    const plx_status_t s = check_bwd_shape(dtype, B, H, T, d_qk, d_v, softmax_scale);
    if (s != PLX_OK) return s;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(rho) || !aligned16(o) ||
        !aligned16(vbar) || !aligned16(stats))
        return PLX_ERR_MISALIGNED;
    int cus = 1;
    const plx_status_t sc = current_cu_count(&cus);
    if (sc != PLX_OK) return sc;
    plx::PrefillArgs a{B, H, T, d_qk, q, k, v, rho, o, softmax_scale, cus};
    a.vbar = vbar;
    a.stats = stats;
    const hipError_t e = plx::launch_prefill_bf16(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PLX_OK : PLX_ERR_HIP;
}

plx_status_t plx_attn_prefill_bwd_workspace_size(int32_t B, int32_t H, int32_t T,
                                                 size_t* bytes_out) {
    if (!bytes_out) return PLX_ERR_NULL_POINTER;
    if (B < 1 || H < 1 || T < 1) return PLX_ERR_INVALID_SHAPE;
    *bytes_out = (size_t)B * H * T * 4 * sizeof(float);
    return PLX_OK;
}

plx_status_t plx_attn_prefill_bwd(plx_dtype_t dtype, int32_t B, int32_t H, int32_t T,
                                  int32_t d_qk, int32_t d_v, const void* q, const void* k,
                                  const void* v, const void* rho, const void* o,
                                  const void* vbar, const float* stats, const void* d_o,
                                  void* dq, void* dk, void* dv, void* drho, void* workspace,
                                  size_t workspace_bytes, float softmax_scale, void* stream) {
    if (dtype != PLX_F32 && dtype != PLX_BF16) return PLX_ERR_INVALID_ARG;
    if (!q || !k || !v || !rho || !o || !vbar || !stats || !d_o || !dq || !dk || !dv ||
        !drho || !workspace)
        return PLX_ERR_NULL_POINTER;
    const plx_status_t s = check_bwd_shape(dtype, B, H, T, d_qk, d_v, softmax_scale);
    if (s != PLX_OK) return s;
    const void* ptrs[] = {q, k, v, rho, o, vbar, stats, d_o, dq, dk, dv, drho, workspace};
    for (const void* p : ptrs)
        if (!aligned16(p)) return PLX_ERR_MISALIGNED;
    size_t need = 0;
    plx_attn_prefill_bwd_workspace_size(B, H, T, &need);
    if (workspace_bytes < need) return PLX_ERR_WORKSPACE_TOO_SMALL;
    plx::PrefillBwdArgs a{B, H, T, d_qk, q, k, v, rho, o, vbar, stats, d_o, dq, dk, dv, drho,
                          static_cast<float*>(workspace), softmax_scale};
    const hipError_t e = plx::launch_prefill_bwd_bf16(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PLX_OK : PLX_ERR_HIP;
}

plx_status_t plx_attn_decode_num_splits(int32_t B, int32_t H, int32_t L_max,
                                        int32_t num_splits, int32_t* splits_out) {
    if (!splits_out) return PLX_ERR_NULL_POINTER;
    plx_status_t st = check_decode_shape(B, H, L_max, 1);
    if (st != PLX_OK) return st;
    DecodePlan p;
    st = plan_decode(B, H, L_max, 128, num_splits, &p);
    if (st != PLX_OK) return st;
    *splits_out = p.reported();
    return PLX_OK;
}

plx_status_t plx_attn_decode_workspace_size(int32_t B, int32_t H, int32_t L_max,
                                            int32_t d_v, int32_t num_splits,
                                            size_t* bytes_out) {
    if (!bytes_out) return PLX_ERR_NULL_POINTER;
    plx_status_t st = check_decode_shape(B, H, L_max, d_v);
    if (st != PLX_OK) return st;
    DecodePlan p;
    st = plan_decode(B, H, L_max, d_v, num_splits, &p);
    if (st != PLX_OK) return st;
    *bytes_out = p.ws_bytes;
    return PLX_OK;
}

plx_status_t plx_attn_decode(plx_dtype_t dtype, int32_t B, int32_t H, int32_t L_max,
                             int32_t d_qk, int32_t d_v, const void* q, const void* rho,
                             const void* k_cache, const void* v_cache,
                             const int32_t* seqlens, void* o, float softmax_scale,
                             int32_t num_splits, void* workspace, size_t workspace_bytes,
                             void* stream) {
    return decode_call(dtype, B, H, L_max, d_qk, d_v, q, rho, k_cache, v_cache, seqlens, o,
                       softmax_scale, num_splits, workspace, workspace_bytes, stream, false);
}

plx_status_t plx_attn_decode_noalloc(plx_dtype_t dtype, int32_t B, int32_t H, int32_t L_max,
                                     int32_t d_qk, int32_t d_v, const void* q, const void* rho,
                                     const void* k_cache, const void* v_cache,
                                     const int32_t* seqlens, void* o, float softmax_scale,
                                     int32_t num_splits, void* stream) {
    return decode_call(dtype, B, H, L_max, d_qk, d_v, q, rho, k_cache, v_cache, seqlens, o,
                       softmax_scale, num_splits, nullptr, kScratchBytes, stream, true);
}

}  // extern "C"

namespace {

// One decode step (the body of plx_attn_decode). With use_scratch, the split records go to
// this GPU's copy of `scratch` (workspace is ignored, workspace_bytes is the array's size).
plx_status_t decode_call(plx_dtype_t dtype, int32_t B, int32_t H, int32_t L_max, int32_t d_qk,
                         int32_t d_v, const void* q, const void* rho, const void* k_cache,
                         const void* v_cache, const int32_t* seqlens, void* o,
                         float softmax_scale, int32_t num_splits, void* workspace,
                         size_t workspace_bytes, void* stream, bool use_scratch) {
    if (dtype != PLX_F32 && dtype != PLX_BF16) return PLX_ERR_INVALID_ARG;
    if (!q || !k_cache || !v_cache || !seqlens || !o) return PLX_ERR_NULL_POINTER;
    plx_status_t st = check_decode_shape(B, H, L_max, d_v);
    if (st != PLX_OK) return st;
    if (d_qk < 1) return PLX_ERR_INVALID_SHAPE;
    if (!std::isfinite(softmax_scale) || softmax_scale < 0.f) return PLX_ERR_INVALID_ARG;
    if (num_splits > kDecodeMaxSplits || num_splits < -plx::kDecodeRangeMaxWaves)
        return PLX_ERR_INVALID_ARG;
    if (!(dtype == PLX_BF16 && d_qk == d_v && (d_qk == 128 || d_qk == 64)))
        return PLX_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(rho) || !aligned16(k_cache) || !aligned16(v_cache) ||
        !aligned16(o) || (reinterpret_cast<uintptr_t>(seqlens) & 3u) != 0)
        return PLX_ERR_MISALIGNED;

    DecodePlan p;
    st = plan_decode(B, H, L_max, d_v, num_splits, &p);
    if (st != PLX_OK) return st;
    if (use_scratch) {
        if (p.ws_bytes > kScratchBytes) return PLX_ERR_WORKSPACE_TOO_SMALL;
        st = scratch_of_current_device(&workspace);
        if (st != PLX_OK) return st;
    }
    if (p.ws_bytes > 0) {
        if (!workspace) return PLX_ERR_NULL_POINTER;
        if (workspace_bytes < p.ws_bytes) return PLX_ERR_WORKSPACE_TOO_SMALL;
        if (!aligned16(workspace)) return PLX_ERR_MISALIGNED;
    }
    plx::DecodeArgs a{B, H, L_max, d_qk, q, rho, k_cache, v_cache, seqlens, o, softmax_scale,
                      p.splits, p.chunk, static_cast<float*>(workspace), p.waves,
                      p.whole ? 1 : 0};
    // d = 64 (split mode): the grouped-head kernel with one query head per cache head
    const hipError_t e =
        d_qk == 64 ? plx::launch_decode_gqa_bf16(a, H, static_cast<hipStream_t>(stream))
                   : plx::launch_decode_bf16_d128(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PLX_OK : PLX_ERR_HIP;
}

// Paged decode, one query head per cache head (the split decode kernel at d = 128) or grouped
// query heads (the grouped kernel, also for one head per cache head when `grouped` or at
// d = 64).
plx_status_t paged_call(plx_dtype_t dtype, int32_t B, int32_t H_q, int32_t H_kv,
                        int32_t block_size, int32_t max_blocks, int32_t num_blocks, int32_t d_qk,
                        int32_t d_v, const void* q, const void* rho, const void* k_pool,
                        const void* v_pool, const int32_t* block_table, const int32_t* seqlens,
                        void* o, float softmax_scale, int32_t num_splits, void* workspace,
                        size_t workspace_bytes, void* stream, bool grouped);

}  // namespace

extern "C" {

plx_status_t plx_attn_decode_gqa_plan(int32_t B, int32_t H_q, int32_t H_kv, int32_t L_max,
                                     int32_t d_v, int32_t num_splits, int32_t* splits_out,
                                     size_t* workspace_bytes_out) {
    if (!splits_out || !workspace_bytes_out) return PLX_ERR_NULL_POINTER;
    plx_status_t st = check_decode_shape(B, H_q, L_max, d_v);
    if (st != PLX_OK) return st;
    if (H_kv < 1 || H_q % H_kv != 0) return PLX_ERR_INVALID_SHAPE;
    const int G = H_q / H_kv;
    if (G != 1 && G != 2 && G != 4 && G != 8) return PLX_ERR_UNSUPPORTED;
    if (num_splits < 0) return PLX_ERR_INVALID_ARG;  // split mode only
    DecodePlan p;
    st = plan_decode(B, H_kv, L_max, d_v, num_splits == 0 ? 0 : num_splits, &p);
    if (st != PLX_OK) return st;
    *splits_out = p.splits;
    *workspace_bytes_out = p.splits > 1 ? (size_t)B * H_q * p.splits *
                                              (size_t)(2 * d_v + 4) * sizeof(float)
                                        : 0;
    return PLX_OK;
}

plx_status_t plx_attn_decode_gqa(plx_dtype_t dtype, int32_t B, int32_t H_q, int32_t H_kv,
                                 int32_t L_max, int32_t d_qk, int32_t d_v, const void* q,
                                 const void* rho, const void* k_cache, const void* v_cache,
                                 const int32_t* seqlens, void* o, float softmax_scale,
                                 int32_t num_splits, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    if (dtype != PLX_F32 && dtype != PLX_BF16) return PLX_ERR_INVALID_ARG;
    if (!q || !k_cache || !v_cache || !seqlens || !o) return PLX_ERR_NULL_POINTER;
    plx_status_t st = check_decode_shape(B, H_q, L_max, d_v);
    if (st != PLX_OK) return st;
    if (d_qk < 1 || H_kv < 1 || H_q % H_kv != 0) return PLX_ERR_INVALID_SHAPE;
    if (!std::isfinite(softmax_scale) || softmax_scale < 0.f) return PLX_ERR_INVALID_ARG;
    if (num_splits < 0 || num_splits > kDecodeMaxSplits) return PLX_ERR_INVALID_ARG;
    const int G = H_q / H_kv;
    if (!(dtype == PLX_BF16 && d_qk == d_v && (d_qk == 128 || d_qk == 64)) ||
        (G != 1 && G != 2 && G != 4 && G != 8))
        return PLX_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(rho) || !aligned16(k_cache) || !aligned16(v_cache) ||
        !aligned16(o) || (reinterpret_cast<uintptr_t>(seqlens) & 3u) != 0)
        return PLX_ERR_MISALIGNED;
    int splits = 0;
    size_t need = 0;
    st = plx_attn_decode_gqa_plan(B, H_q, H_kv, L_max, d_v, num_splits, &splits, &need);
    if (st != PLX_OK) return st;
    if (need > 0) {
        if (!workspace) return PLX_ERR_NULL_POINTER;
        if (workspace_bytes < need) return PLX_ERR_WORKSPACE_TOO_SMALL;
        if (!aligned16(workspace)) return PLX_ERR_MISALIGNED;
    }
    plx::DecodeArgs a{B, H_q, L_max, d_qk, q, rho, k_cache, v_cache, seqlens, o, softmax_scale,
                      splits, 0, static_cast<float*>(workspace), 0, 0};
    const hipError_t e = plx::launch_decode_gqa_bf16(a, H_kv, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PLX_OK : PLX_ERR_HIP;
}

plx_status_t plx_attn_decode_paged(plx_dtype_t dtype, int32_t B, int32_t H, int32_t block_size,
                                   int32_t max_blocks, int32_t num_blocks, int32_t d_qk,
                                   int32_t d_v, const void* q, const void* rho,
                                   const void* k_pool, const void* v_pool,
                                   const int32_t* block_table, const int32_t* seqlens, void* o,
                                   float softmax_scale, int32_t num_splits, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    return paged_call(dtype, B, H, H, block_size, max_blocks, num_blocks, d_qk, d_v, q, rho,
                      k_pool, v_pool, block_table, seqlens, o, softmax_scale, num_splits,
                      workspace, workspace_bytes, stream, false);
}

plx_status_t plx_attn_decode_paged_gqa(plx_dtype_t dtype, int32_t B, int32_t H_q, int32_t H_kv,
                                       int32_t block_size, int32_t max_blocks,
                                       int32_t num_blocks, int32_t d_qk, int32_t d_v,
                                       const void* q, const void* rho, const void* k_pool,
                                       const void* v_pool, const int32_t* block_table,
                                       const int32_t* seqlens, void* o, float softmax_scale,
                                       int32_t num_splits, void* workspace,
                                       size_t workspace_bytes, void* stream) {
    return paged_call(dtype, B, H_q, H_kv, block_size, max_blocks, num_blocks, d_qk, d_v, q, rho,
                      k_pool, v_pool, block_table, seqlens, o, softmax_scale, num_splits,
                      workspace, workspace_bytes, stream, true);
}

plx_status_t plx_attn_probe(plx_dtype_t dtype, int32_t B, int32_t T, int32_t C, int32_t H,
                            int32_t d, const void* x, const void* w_r, const float* gamma,
                            const float* gate, const int32_t* positions, float eps,
                            float rope_base, void* rho, void* stream) {
    if (dtype != PLX_F32 && dtype != PLX_BF16) return PLX_ERR_INVALID_ARG;
    if (!x || !w_r || !rho) return PLX_ERR_NULL_POINTER;
    if (B < 1 || T < 1 || C < 1 || H < 1 || d < 1) return PLX_ERR_INVALID_SHAPE;
    if ((long long)B * T * C * 2 >= (1LL << 31) || (long long)d * C * 2 >= (1LL << 31) ||
        H > 65535 || (long long)B * T > (1LL << 36))
        return PLX_ERR_INVALID_SHAPE;
    if (!std::isfinite(eps) || eps < 0.f || !std::isfinite(rope_base) ||
        (rope_base != 0.f && !(rope_base > 1.f)))
        return PLX_ERR_INVALID_ARG;
    if (!(dtype == PLX_BF16 && d == 128) || C % 8 != 0) return PLX_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(w_r) || !aligned16(rho) || !aligned16(gamma) ||
        (reinterpret_cast<uintptr_t>(gate) & 3u) ||
        (reinterpret_cast<uintptr_t>(positions) & 3u))
        return PLX_ERR_MISALIGNED;
    plx::ProbeArgs a{B, T, C, H, x, w_r, gamma, gate, positions, rho, eps, rope_base};
    const hipError_t e = plx::launch_probe_bf16_d128(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PLX_OK : PLX_ERR_HIP;
}

}  // extern "C"

namespace {

plx_status_t paged_call(plx_dtype_t dtype, int32_t B, int32_t H_q, int32_t H_kv,
                        int32_t block_size, int32_t max_blocks, int32_t num_blocks, int32_t d_qk,
                        int32_t d_v, const void* q, const void* rho, const void* k_pool,
                        const void* v_pool, const int32_t* block_table, const int32_t* seqlens,
                        void* o, float softmax_scale, int32_t num_splits, void* workspace,
                        size_t workspace_bytes, void* stream, bool grouped) {
    if (dtype != PLX_F32 && dtype != PLX_BF16) return PLX_ERR_INVALID_ARG;
    if (!q || !k_pool || !v_pool || !block_table || !seqlens || !o) return PLX_ERR_NULL_POINTER;
    if (block_size < 32 || (block_size & (block_size - 1)) != 0 || max_blocks < 1 ||
        num_blocks < 1)
        return PLX_ERR_INVALID_SHAPE;
    if ((long long)max_blocks * block_size > INT_MAX) return PLX_ERR_INVALID_SHAPE;
    const int L_max = max_blocks * block_size;
    plx_status_t st = check_decode_shape(B, H_q, L_max, d_v);
    if (st != PLX_OK) return st;
    if (d_qk < 1 || H_kv < 1 || H_q % H_kv != 0) return PLX_ERR_INVALID_SHAPE;
    if (!std::isfinite(softmax_scale) || softmax_scale < 0.f) return PLX_ERR_INVALID_ARG;
    if (num_splits < 0 || num_splits > kDecodeMaxSplits) return PLX_ERR_INVALID_ARG;
    const int G = H_q / H_kv;
    if (!(dtype == PLX_BF16 && d_qk == d_v && (d_qk == 128 || d_qk == 64)) ||
        (G != 1 && G != 2 && G != 4 && G != 8))
        return PLX_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(rho) || !aligned16(k_pool) || !aligned16(v_pool) ||
        !aligned16(o) || (reinterpret_cast<uintptr_t>(seqlens) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(block_table) & 3u) != 0)
        return PLX_ERR_MISALIGNED;
    int splits = 0;
    size_t need = 0;
    st = plx_attn_decode_gqa_plan(B, H_q, H_kv, L_max, d_v, num_splits, &splits, &need);
    if (st != PLX_OK) return st;
    if (need > 0) {
        if (!workspace) return PLX_ERR_NULL_POINTER;
        if (workspace_bytes < need) return PLX_ERR_WORKSPACE_TOO_SMALL;
        if (!aligned16(workspace)) return PLX_ERR_MISALIGNED;
    }
    int log2 = 0;
    while ((1 << log2) < block_size) ++log2;
    plx::DecodeArgs a{B, H_q, L_max, d_qk, q, rho, k_pool, v_pool, seqlens, o, softmax_scale,
                      splits, 0, static_cast<float*>(workspace), 0, 0,
                      block_table, max_blocks, log2, num_blocks};
    // d = 64 runs the grouped kernel also with one query head per cache head
    const hipError_t e =
        grouped || d_qk == 64
            ? plx::launch_decode_gqa_bf16(a, H_kv, static_cast<hipStream_t>(stream))
            : plx::launch_decode_bf16_d128(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PLX_OK : PLX_ERR_HIP;
}

}  // namespace
