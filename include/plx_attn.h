/*
 * plx_attn.h -- C ABI of the Parallax attention forward on AMD Instinct MI355X (gfx950).
 *
 * Parallax adds a covariance-correction branch to causal softmax attention. For query i
 * over its visible keys j, with softmax weights p_ij of the scores a_ij = scale <q_i, k_j>:
 *
 *     o_i = o_SA_i - Sigma_KV^(i) rho_i                                        (1)
 *
 * where o_SA_i = sum_j p_ij v_j is the softmax-attention output and Sigma_KV^(i) is the
 * softmax-weighted covariance of the values against the keys, applied to the per-query
 * probe rho_i (the row of the extra R matrix). Equation (1) is the central equation of the
 * method [Resumen Tecnico: Parallax - Atencion Lineal Local Parametrizada para Modelado de
 * Lenguaje, section "Mecanismo Central"]; the covariance is the softmax-weighted KV
 * covariance [Parallax: Parameterized Local Linear Attention for Language Modeling,
 * agihunt.info review, method paragraph]. Expanded, (1) is the corrected-weight sum
 *
 *     o_i = sum_j p_ij (1 - (t_ij - tbar_i)) v_j,  t_ij = <rho_i, k_j>,  tbar_i = sum_j p_ij t_ij
 *
 * [Parallax (paper.rainbus.top summary), section "方法步骤详情" (method steps 2-6)], which
 * the kernels evaluate in streaming form: one pass over the keys with one running max and
 * one rescale factor shared by both branches, accumulating sum w v, sum w t v, sum w and
 * sum w t together (same section's streaming sentences; agihunt review, hardware paragraph).
 * The boundary-amplification factor of exact local linear attention is fixed at zero.
 * The probe rho is an input: its projection W_R x and normalisation happen before the call.
 *
 * Conventions shared by every entry point
 *   - All tensors are device pointers to contiguous, row-major arrays, 16-byte aligned.
 *   - The caller allocates and owns every buffer, including the decode workspace; the
 *     library allocates nothing and keeps no per-call state. It caches the device's
 *     compute-unit count on first use.
 *   - Calls are asynchronous: work is enqueued on `stream` (a hipStream_t passed as
 *     void*; NULL = the default stream). Buffers must stay valid until the stream reaches
 *     the work. The output must not alias any input.
 *   - Arguments are validated on the host first; an invalid call returns its status code
 *     without enqueuing anything. A launch failure returns PLX_ERR_HIP. No exception
 *     crosses the ABI and the library never aborts.
 *   - Arithmetic: bf16 inputs are multiplied on the matrix cores with fp32 accumulation.
 *     Prefill rounds the softmax weights and the weight*probe products to bf16 (RNE) before
 *     the value products and takes the row sums from the same rounded values, unless
 *     plx_attn_prefill_ex is asked to split them (hi + lo bf16 terms, fp32 row sums). The
 *     decode paths keep the weights in fp32 (vector-ALU value products) or split them (the
 *     grouped-head decode's matrix-core value products). Output is rounded to the input
 *     dtype (RNE). fp32 inputs use fp32 throughout.
 *   - softmax_scale multiplies q.k only (t is unscaled); it must be finite and >= 0
 *     (0 gives uniform weights).
 */
#ifndef PLX_ATTN_H
#define PLX_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PLX_OK = 0,
    PLX_ERR_NULL_POINTER = 1,        /* a required pointer is NULL */
    PLX_ERR_INVALID_SHAPE = 2,       /* a size is < 1 or too large for 32-bit slice offsets */
    PLX_ERR_INVALID_ARG = 3,         /* scale not finite or negative; bad split count; bad dtype */
    PLX_ERR_UNSUPPORTED = 4,         /* (dtype, d_qk, d_v) combination not built */
    PLX_ERR_MISALIGNED = 5,          /* a pointer is not 16-byte aligned */
    PLX_ERR_WORKSPACE_TOO_SMALL = 6, /* decode workspace smaller than required */
    PLX_ERR_HIP = 7                  /* a HIP runtime call or kernel launch failed */
} plx_status_t;

typedef enum { PLX_F32 = 0, PLX_BF16 = 1 } plx_dtype_t;

/*
 * Causal prefill: every query row of every (batch, head) against keys 0..i.
 *
 *   q, k, rho : [B, H, T, d_qk]   v, o : [B, H, T, d_v]   (dtype for all five)
 *   Key j is visible to query i iff j <= i (top-left aligned, T_q = T_k = T).
 *   rho == NULL means rho = 0 exactly: plain softmax attention, computed by a specialisation
 *   without the probe branch; its output is bit-identical to a call with an all-zero rho.
 *
 * Built combinations: (PLX_BF16, d_qk = d_v in {64, 128}) on the matrix cores (d = 64 is
 * the compute-matched head dim of the pages' control: a Parallax layer with the head dim
 * halved does the FLOPs of softmax attention at the full head dim [agihunt review,
 * pretraining table and the paragraph after it; gist.science summary (Spanish), results
 * section, controls item]); (PLX_F32, d_qk = d_v in {16, 32, 64}) on the vector ALUs.
 * Limits: B*H <= 2^31-1 and T * d * sizeof(dtype) < 2^31 (one (b,h) slice per buffer).
 */
plx_status_t plx_attn_prefill(plx_dtype_t dtype, int32_t B, int32_t H, int32_t T,
                              int32_t d_qk, int32_t d_v, const void* q, const void* k,
                              const void* v, const void* rho, void* o, float softmax_scale,
                              void* stream);

/* Flags of plx_attn_prefill_ex. */
#define PLX_PREFILL_SPLIT_WEIGHTS 1u

/*
 * plx_attn_prefill with a flags word (plx_attn_prefill is this call with flags = 0). Same
 * arguments, layouts, ownership and errors; flags other than those defined here give
 * PLX_ERR_INVALID_ARG.
 *
 * PLX_PREFILL_SPLIT_WEIGHTS (bf16 path): each softmax weight w and each weight*probe product
 * w*t enters the value products as two bf16 terms, hi = bf16(u) and lo = bf16(u - hi), and
 * the row sums l, beta are fp32 sums of the unrounded values. The corrected output
 * o = sum_j p_j (1 - (t_j - tbar)) v_j [paper.rainbus.top summary, method steps 2-6] moves
 * by about sum_j p_j |1 + tbar - t_j| |v_j - vbar| times the relative error of the weights,
 * which bf16 weights (2^-9) keep under 1e-2 only while |t| stays small (probe RMS ~0.1 at
 * d = 128); a unit-RMS probe (|t| ~ 10, a probe normalised as the method prescribes
 * [agihunt review, method paragraph]) needs the split, whose weights reach ~2^-17. It costs
 * two more matrix products per value operand. No effect on the fp32 path (fp32 weights).
 */
plx_status_t plx_attn_prefill_ex(plx_dtype_t dtype, int32_t B, int32_t H, int32_t T,
                                 int32_t d_qk, int32_t d_v, const void* q, const void* k,
                                 const void* v, const void* rho, void* o, float softmax_scale,
                                 uint32_t flags, void* stream);

/*
 * The plan a decode call with these arguments will use at d = 128, written to *splits_out in
 * the encoding of num_splits: S > 0 for split mode with S chunks per (b, h), or -G for
 * wave-range mode with G waves. num_splits > 0 and < 0 are taken as given (a negative count
 * is rounded up to a multiple of 4); 0 picks a split-mode plan from B*H, L_max and the current
 * device's compute-unit count. At d = 64 only split mode exists: 0 then picks the split count the
 * split heuristic gives (plx_attn_decode_workspace_size, which takes d_v, sizes it).
 */
plx_status_t plx_attn_decode_num_splits(int32_t B, int32_t H, int32_t L_max,
                                        int32_t num_splits, int32_t* splits_out);

/*
 * Bytes of fp32 workspace plx_attn_decode needs for the same (B, H, L_max, d_v,
 * num_splits): split mode B*H*S*(2*d_v + 4)*4 for S > 1 chunks (0 when S == 1);
 * wave-range mode G*2*(2*d_v + 4)*4 for G waves, or 0 when its slices hold whole (b, h).
 */
plx_status_t plx_attn_decode_workspace_size(int32_t B, int32_t H, int32_t L_max,
                                            int32_t d_v, int32_t num_splits,
                                            size_t* bytes_out);

/*
 * One decode step over a contiguous per-sequence KV cache: equation (1) for the one new query
 * row of each (b, h) against its cached keys. The score and probe products of a cache row
 * share one matrix instruction (the probe fills accumulator rows the single query leaves idle
 * [agihunt review, hardware paragraph]), and the key loop is split across workgroups whose
 * partial states are then reduced [Parallax (paper.rainbus.top summary), reproducibility
 * section: the decode kernel is optimised by instruction sharing, splitting the KV loop and
 * reducing the split partials].
 *
 *   q, rho   : [B, H, d_qk]            k_cache : [B, H, L_max, d_qk]
 *   v_cache  : [B, H, L_max, d_v]      o       : [B, H, d_v]
 *   rho == NULL means rho = 0 exactly (plain softmax attention, a specialisation without
 *              the probe accumulations; bit-identical to a call with an all-zero rho).
 *   seqlens  : device int32 [B]; query b attends to cache rows [0, n_b) with
 *              n_b = min(max(seqlens[b], 0), L_max); n_b == 0 gives o[b] = 0.
 *              Rows at or beyond n_b are never read, so they may hold anything.
 *   num_splits : how the cache is divided among waves; 0 = heuristic.
 *              > 0: split mode, that many KV chunks per (b, h) (each sequence's own length
 *              split evenly); each chunk's partial state (running max, normaliser, sum w t,
 *              sum w v, sum w t v) goes to the workspace and a second kernel merges them.
 *              < 0: wave-range mode with -num_splits waves (rounded up to a multiple of 4):
 *              the (b, h) ranges are laid end to end (sequence-major, head-minor) and each
 *              wave streams an equal slice, whatever the mix of lengths; a (b, h) cut by
 *              slice ends leaves partials that a second kernel merges. With at least 2
 *              (b, h) per wave the slices end at (b, h) starts instead and nothing is merged.
 *              Needs B <= 8192 and B*H*L_max < 2^31 (else PLX_ERR_UNSUPPORTED).
 *   workspace  : device buffer of at least plx_attn_decode_workspace_size() bytes
 *              (may be NULL when that size is 0).
 *
 * Built combinations: (PLX_BF16, d_qk = d_v = 128), both modes; (PLX_BF16, d_qk = d_v = 64),
 * split mode (num_splits >= 0; a negative count returns PLX_ERR_UNSUPPORTED).
 * Limits: L_max * d * 2 < 2^31; -65536 <= num_splits <= 4096.
 */
plx_status_t plx_attn_decode(plx_dtype_t dtype, int32_t B, int32_t H, int32_t L_max,
                             int32_t d_qk, int32_t d_v, const void* q, const void* rho,
                             const void* k_cache, const void* v_cache,
                             const int32_t* seqlens, void* o, float softmax_scale,
                             int32_t num_splits, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Bytes of the per-GPU scratch array of plx_attn_decode_noalloc. */
#define PLX_DECODE_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * plx_attn_decode for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same step with the
 * same arguments, plan, kernels and results, except that the split partial records go to a
 * fixed scratch array the library holds on each GPU it runs on (PLX_DECODE_NOALLOC_SCRATCH_BYTES,
 * 16 MiB, kept until the process ends) instead of a caller workspace. The caller still passes
 * the inputs and the output. The call allocates nothing: no hipMalloc, no hipFree, no
 * allocating library routine. The scratch's device address is looked up on the first call on
 * each device (with that device current) and cached.
 *
 * A plan whose workspace (plx_attn_decode_workspace_size) exceeds the scratch returns
 * PLX_ERR_WORKSPACE_TOO_SMALL without enqueuing anything; pass a smaller num_splits.
 * All calls on one GPU share its scratch: calls that overlap on one GPU (on different streams,
 * or from several threads) race and must be serialised by the caller. Nothing in the scratch
 * needs to start at zero (every record a call reads, that call has written).
 */
plx_status_t plx_attn_decode_noalloc(plx_dtype_t dtype, int32_t B, int32_t H, int32_t L_max,
                                     int32_t d_qk, int32_t d_v, const void* q, const void* rho,
                                     const void* k_cache, const void* v_cache,
                                     const int32_t* seqlens, void* o, float softmax_scale,
                                     int32_t num_splits, void* stream);

/*
 * Decode with grouped query heads: H_q query heads over H_kv cache heads, G = H_q / H_kv in
 * {1, 2, 4, 8}; query head h reads cache head h / G. Same conventions as plx_attn_decode, with
 *   q, rho  : [B, H_q, d_qk]      k_cache : [B, H_kv, L_max, d_qk]
 *   v_cache : [B, H_kv, L_max, d_v]   o : [B, H_q, d_v]
 * One matrix instruction per 16 cache rows yields the scores and probe products of all G
 * heads (columns q_0, rho_0, ..., q_{G-1}, rho_{G-1}; agihunt review, hardware paragraph: the
 * idle rows of a decode step's matrix instructions carry extra work), and the value products
 * run on the matrix cores as well. Split mode only: num_splits 0 (heuristic) or > 0 chunks per
 * (b, h_kv); rho may be NULL (rho = 0).
 * Built combinations: (PLX_BF16, d_qk = d_v in {64, 128}, G in {1, 2, 4, 8}).
 * plx_attn_decode_gqa_plan writes the split count and the workspace bytes a call with the
 * same arguments needs (B*H_q*S*(2*d_v + 4)*4 for S > 1, else 0).
 */
plx_status_t plx_attn_decode_gqa_plan(int32_t B, int32_t H_q, int32_t H_kv, int32_t L_max,
                                     int32_t d_v, int32_t num_splits, int32_t* splits_out,
                                     size_t* workspace_bytes_out);
plx_status_t plx_attn_decode_gqa(plx_dtype_t dtype, int32_t B, int32_t H_q, int32_t H_kv,
                                 int32_t L_max, int32_t d_qk, int32_t d_v, const void* q,
                                 const void* rho, const void* k_cache, const void* v_cache,
                                 const int32_t* seqlens, void* o, float softmax_scale,
                                 int32_t num_splits, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * One decode step over a paged KV cache: the cache is a pool of blocks and each sequence lists
 * its blocks in a table. Same conventions and split plan as plx_attn_decode_gqa with
 * H_q = H_kv = H and L_max = max_blocks * block_size, with
 *   k_pool, v_pool : [num_blocks, H, block_size, d] (dtype)
 *   block_table    : device int32 [B, max_blocks]; rows i*block_size .. (i+1)*block_size - 1
 *                    of sequence b are block block_table[b][i] of the pool
 *   block_size     : a power of two, at least 32
 * Only the blocks that hold rows below n_b are read. A table entry outside [0, num_blocks) is
 * never dereferenced: the rows it would hold are skipped (they get no softmax weight, as if
 * they were not part of the sequence), so a sequence with such an entry below n_b attends to
 * its other rows only.
 * Built combinations: (PLX_BF16, d_qk = d_v in {64, 128}); rho may be NULL (rho = 0). At
 * d = 128 the result is bitwise that of plx_attn_decode (split mode) over the cache the table
 * describes, with the same split count; at d = 64 that of plx_attn_decode_gqa with H_q = H_kv.
 */
plx_status_t plx_attn_decode_paged(plx_dtype_t dtype, int32_t B, int32_t H, int32_t block_size,
                                   int32_t max_blocks, int32_t num_blocks, int32_t d_qk,
                                   int32_t d_v, const void* q, const void* rho,
                                   const void* k_pool, const void* v_pool,
                                   const int32_t* block_table, const int32_t* seqlens, void* o,
                                   float softmax_scale, int32_t num_splits, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * Paged decode with grouped query heads: plx_attn_decode_paged's pool and table over H_kv
 * cache heads, read by H_q = G H_kv query heads as in plx_attn_decode_gqa (query head h reads
 * cache head h / G; same split plan, plx_attn_decode_gqa_plan with L_max = max_blocks *
 * block_size, and same workspace), with
 *   q, rho         : [B, H_q, d_qk]          o : [B, H_q, d_v]
 *   k_pool, v_pool : [num_blocks, H_kv, block_size, d] (dtype)
 *   block_table    : device int32 [B, max_blocks], as for plx_attn_decode_paged
 * A table entry outside [0, num_blocks) below n_b is never dereferenced and its rows get no
 * weight, as for plx_attn_decode_paged. With the same plan the result is bitwise that of
 * plx_attn_decode_gqa over the cache the table describes.
 * Built combinations: (PLX_BF16, d_qk = d_v in {64, 128}, G in {1, 2, 4, 8}); rho may be NULL.
 */
plx_status_t plx_attn_decode_paged_gqa(plx_dtype_t dtype, int32_t B, int32_t H_q, int32_t H_kv,
                                       int32_t block_size, int32_t max_blocks,
                                       int32_t num_blocks, int32_t d_qk, int32_t d_v,
                                       const void* q, const void* rho, const void* k_pool,
                                       const void* v_pool, const int32_t* block_table,
                                       const int32_t* seqlens, void* o, float softmax_scale,
                                       int32_t num_splits, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * The probe producer: rho = gate_h * RoPE(gamma (.) RMSNorm_head(x W_R^T)), written in the
 * layout plx_attn_prefill / plx_attn_decode read (agihunt review, method paragraph: rho is one
 * matrix product W_R x from the layer input, with its own RMSNorm and, optionally, RoPE; the
 * mechanism-analysis paragraph of the same review mentions a learned gate on the probe).
 *
 *   x   : [B, T, C] tokens of the layer input (dtype)     w_r : [H*d, C] (dtype), row-major
 *   rho : [B, H, T, d] (dtype), written
 *   gamma     : device float[d] (16-byte aligned), the RMSNorm weight, or NULL for 1
 *   gate      : device float[H], a per-head multiplier (e.g. a sigmoid gate's value), or NULL
 *   positions : device int32[B], position of token 0 of sequence b (token t has position
 *               positions[b] + t; for one decode token, seqlens[b] - 1), or NULL for 0
 *   eps       : RMSNorm epsilon (>= 0): y / sqrt(mean over the head's d dims of y^2 + eps)
 *   rope_base : 0 for no rotation; else > 1, the rotate-half RoPE: dims (i, i + d/2) of each
 *               head turned by position * rope_base^(-2i/d), i < d/2
 * Order: y = x W_R^T; per (token, head): RMSNorm, times gamma, RoPE, times gate.
 * Arithmetic: bf16 products with fp32 accumulation on the matrix cores; normalisation and
 * rotation in fp32; output rounded to bf16 (RNE).
 * Built combination: (PLX_BF16, d = 128) with C a multiple of 8. Limits: B*T*C*2 < 2^31.
 * Errors as for the other entry points; nothing is enqueued on a validation failure.
 */
plx_status_t plx_attn_probe(plx_dtype_t dtype, int32_t B, int32_t T, int32_t C, int32_t H,
                            int32_t d, const void* x, const void* w_r, const float* gamma,
                            const float* gate, const int32_t* positions, float eps,
                            float rope_base, void* rho, void* stream);

/*
 * Training support: the causal prefill with saved statistics, and its backward.
 *
 * The layer is trained from scratch (0.6B and 1.7B language models pretrained with it:
 * Parallax (paper.rainbus.top summary), sections "实验结果" and "复现评估"), but the pages give
 * no backward; the gradients below are the chain rule of the forward (1) in its
 * corrected-weight form. For each visible pair (i, j), with s_ij = p_ij (1 - t_ij +
 * tbar_i), g_ij = <dO_i, v_j>, G_i = <dO_i, vbar_i>, D_i = <dO_i, o_i> + tbar_i G_i:
 *     dt_ij = p_ij (G_i - g_ij)        da_ij = p_ij ((1 - t_ij + tbar_i) g_ij + t_ij G_i - D_i)
 *     dv_j = sum_i s_ij dO_i           dk_j = scale sum_i da_ij q_i + sum_i dt_ij rho_i
 *     dq_i = scale sum_j da_ij k_j     drho_i = sum_j dt_ij k_j
 *
 * plx_attn_prefill_fwd: as plx_attn_prefill (same o, bit for bit), and also writes
 *   vbar  : [B, H, T, d] (dtype) the softmax-weighted mean of the values, O1 / l, per row
 *   stats : [B, H, T, 2] float, per row (lse, tbar): lse = ln sum_j exp(scale <q_i, k_j>)
 *           over the visible keys, tbar = sum_j p_ij t_ij (0 when rho == NULL)
 *
 * plx_attn_prefill_bwd: gradients of sum(d_o * o) with respect to q, k, v and rho, given the
 *   forward's inputs, its o, vbar and stats, and d_o [B, H, T, d]. rho must not be NULL (pass
 *   zeros for plain softmax attention; drho is still the gradient at rho = 0).
 *   dq, dk, dv, drho : [B, H, T, d] (dtype), written; none may alias an input
 *   workspace        : device buffer of plx_attn_prefill_bwd_workspace_size() bytes (per-row
 *                      records passed between the two kernels of the call)
 * Arithmetic: products on the matrix cores (bf16 operands, fp32 accumulation); the pair
 * quantities s, scale * da and dt are rounded to bf16 before the accumulating products; p is
 * recomputed as exp(scale <q_i, k_j> - lse_i). Output rounded to bf16 (RNE).
 * Built combinations (both calls): (PLX_BF16, d_qk = d_v in {64, 128}). Limits:
 * T * d * 2 < 2^31.
 * Errors as for the other entry points; PLX_ERR_WORKSPACE_TOO_SMALL for a short workspace.
 */
plx_status_t plx_attn_prefill_fwd(plx_dtype_t dtype, int32_t B, int32_t H, int32_t T,
                                  int32_t d_qk, int32_t d_v, const void* q, const void* k,
                                  const void* v, const void* rho, void* o, void* vbar,
                                  float* stats, float softmax_scale, void* stream);
plx_status_t plx_attn_prefill_bwd_workspace_size(int32_t B, int32_t H, int32_t T,
                                                 size_t* bytes_out);
plx_status_t plx_attn_prefill_bwd(plx_dtype_t dtype, int32_t B, int32_t H, int32_t T,
                                  int32_t d_qk, int32_t d_v, const void* q, const void* k,
                                  const void* v, const void* rho, const void* o,
                                  const void* vbar, const float* stats, const void* d_o,
                                  void* dq, void* dk, void* dv, void* drho, void* workspace,
                                  size_t workspace_bytes, float softmax_scale, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* plx_status_string(plx_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* PLX_ATTN_H */
