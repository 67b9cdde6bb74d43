/*
 * qgguf.h -- C ABI of libqgguf.so: dequantize-fused quantized-weight GEMV and
 * small-batch / prefill matrix products on AMD Instinct MI355X (gfx950).
 *
 * Weights are GGUF Q8_0, Q4_K or Q6_K blocks, dotted against activations
 * quantized to Q8_1 blocks.  The pages this library follows name these types
 * as the ones with dedicated integer-dot GPU kernels (blazr README, "Model
 * Formats > GGUF"), describe in-shader dequantization feeding an integer mmq
 * path (infr page, "models"), and MoE expert calls (infr page, "Per-op device
 * profiling": the expert_gateup role; "Paged experts").  They give no byte
 * layout; the layouts below are GGUF's published ones, little-endian:
 *
 *   Q8_0 (32 values, 34 B):  fp16 d | int8 qs[32]               w = d*qs[i]
 *   Q8_1 (32 values, 36 B):  fp16 d | fp16 s | int8 qs[32]      x = d*qs[i],
 *                            s = d*sum(qs) (informational; not read by dots)
 *   Q4_K (256 values, 144 B): fp16 d | fp16 dmin | u8 scales[12] | u8 qs[128]
 *        sub-block j = i/32 has 6-bit scale sc_j and min m_j packed in
 *        scales[]; w = d*sc_j*q - dmin*m_j with q the 4-bit code.
 *   Q6_K (256 values, 210 B): u8 ql[128] | u8 qh[64] | int8 scales[16] | fp16 d
 *        w = d*scales[i/16]*(q - 32) with q the 6-bit code.
 *
 * Conventions for every call:
 *   - Matrices are row-major.  A weight matrix of n rows and k columns is n
 *     rows of k/block_elems blocks, rows contiguous.
 *   - All pointers are DEVICE pointers owned by the caller.  The library
 *     allocates and frees nothing.  Block buffers (weights, Q8_1) and float
 *     inputs must be 16-byte aligned; float / int32 outputs 4-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls enqueue work
 *     and return; they never synchronize.  Launch errors are reported from
 *     hipGetLastError right after the enqueue; device faults surface at the
 *     caller's next synchronization.
 *   - Arguments are validated before any HIP call.  On any error nothing is
 *     launched and nothing is written.  Outputs are overwritten, not
 *     accumulated.  Empty problems (n == 0 or m == 0) return QG_OK and launch
 *     nothing; k == 0 writes zeros.
 *   - Devices other than gfx950 are refused with QG_ERR_ARCH.
 *   - Calls on one stream are ordered; calls on different streams that write
 *     the same buffers race, as for any HIP kernel.
 */
#ifndef QGGUF_H
#define QGGUF_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QG_OK = 0,
    QG_ERR_NULL = 1,      /* a required pointer is NULL */
    QG_ERR_SHAPE = 2,     /* negative size, k not a multiple of the block, size too large */
    QG_ERR_ALIGN = 3,     /* a pointer is not aligned as required */
    QG_ERR_WORKSPACE = 4, /* MoE workspace smaller than moe_qgemv_q4_k_workspace_size() */
    QG_ERR_NO_DEVICE = 5, /* no HIP device is visible */
    QG_ERR_ARCH = 6,      /* the current device is not gfx950 */
    QG_ERR_LAUNCH = 7     /* the kernel launch failed */
} qg_status;

/* Static description of a status code (never NULL). */
const char *qg_status_str(qg_status s);

/*
 * quantize_q8_1 -- activations f32 -> Q8_1 (the activation side of every dot).
 * Defining passage: the integer-dot kernels the blazr README names ("Model
 * Formats > GGUF": dp4a kernels for Q4_K, Q6_K and Q8_0) take 8-bit codes on
 * both sides, so the activation is quantized to GGUF's 32-value Q8_1 block;
 * the pages name the integer dot, not the block, and this is the reading.
 * Per block of 32 values: amax = max|x|; d = amax/127 (fp32, correctly
 * rounded); q = round-half-away-from-zero(x/d), computed from the fp32 d and
 * clamped to [-127, 127]; s = d*sum(q) as an fp32 product.  d and s are stored
 * rounded once to fp16 (round to nearest even, subnormals kept).  A block whose
 * values are all zero stores d = s = 0 and q = 0.
 *   x   : f32 [rows][k], 16-byte aligned
 *   xq  : Q8_1 [rows][k/32] (36 B each), 16-byte aligned, written
 *   k   : multiple of 32, <= 2^30;  rows * k <= 2^40
 */
qg_status quantize_q8_1(const float *x, void *xq, int64_t rows, int64_t k, hipStream_t stream);

/*
 * qgemv_q8_0 / qgemv_q4_k / qgemv_q6_k -- batch-1 decode GEMV, y = W . x^.
 * Defining passages: blazr README, "Model Formats > GGUF" (the three weight
 * types with dedicated dp4a dot kernels on the GPU); infr page, "Benchmarks
 * you can compare" and "Per-op device profiling" (decode time is spent in the
 * GEMV buckets, reported per kernel and per shape).
 * y[r] = sum_j w^[r][j] * x^[j] with w^ dequantized from the weight blocks and
 * x^ from the Q8_1 activation.  Computed from exact per-block int32 dots
 * (Q8_0 and Q4_K: per 32 values; Q6_K: per 16 values) scaled in fp32.
 *   w   : weight blocks [n][k/block_elems]
 *   xq  : Q8_1 [k/32] (one activation row)
 *   y   : f32 [n], written
 *   k   : multiple of 32 (Q8_0) or 256 (Q4_K, Q6_K), <= 2^24;  n <= 2^31 - 1
 */
qg_status qgemv_q8_0(const void *w, const void *xq, float *y, int64_t n, int64_t k, hipStream_t stream);
qg_status qgemv_q4_k(const void *w, const void *xq, float *y, int64_t n, int64_t k, hipStream_t stream);
qg_status qgemv_q6_k(const void *w, const void *xq, float *y, int64_t n, int64_t k, hipStream_t stream);

/*
 * qgemv_q5_k -- the same decode GEMV for Q5_K weights, one of the GGUF types
 * the blazr README ("Model Formats > GGUF") runs beyond the three with
 * dedicated dot kernels.  Block (176 bytes): fp16 d, fp16 dmin, 12 bytes of
 * six-bit scales/mins packed as Q4_K's, qh[32], qs[128]; element 32j + l of a
 * superblock has the 4-bit code Q4_K's qs rule gives plus bit j of qh[l] as
 * its fifth bit, w = d*sc_j*q - dmin*m_j.  Same arguments, limits and errors
 * as qgemv_q4_k (w: Q5_K [n][k/256]).
 */
qg_status qgemv_q5_k(const void *w, const void *xq, float *y, int64_t n, int64_t k, hipStream_t stream);

/*
 * qgemv_q4_0 / qgemv_q5_0 -- the same decode GEMV for the 32-value GGUF types
 * Q4_0 and Q5_0, two more of the types the blazr README ("Model Formats >
 * GGUF") runs beyond the three with dedicated dot kernels.
 *   Q4_0 block (18 bytes): fp16 d, qs[16]; byte j of qs holds the 4-bit codes
 *        of elements j (low nibble) and 16 + j (high nibble); w = d*(q - 8).
 *   Q5_0 block (22 bytes): fp16 d, qh (4 bytes), qs[16] as Q4_0; bit i of the
 *        little-endian 32-bit qh is element i's fifth bit; w = d*(q - 16).
 * The per-block dot is the exact integer sum of (q - 8)*qa (q - 16 for Q5_0),
 * scaled in fp32 by d*d_a.  Same arguments and errors as qgemv_q8_0
 * (w: [n][k/32] blocks, 16-byte aligned), except that k must be a multiple of
 * 64 (the kernel reads block pairs).
 */
qg_status qgemv_q4_0(const void *w, const void *xq, float *y, int64_t n, int64_t k, hipStream_t stream);
qg_status qgemv_q5_0(const void *w, const void *xq, float *y, int64_t n, int64_t k, hipStream_t stream);

/*
 * qgemv_q8_0_batch / qgemv_q4_k_batch / qgemv_q6_k_batch -- small-batch GEMV,
 * b activation rows against one read of the weights (the decode step of b
 * concurrent sequences: infr page, "Concurrent slots, many models").
 * y[i][r] = sum_j w^[r][j] * x^_i[j] for i < b, each row computed like the
 * batch-1 GEMV above from exact per-block int32 dots scaled in fp32 (the fp32
 * rounding order may differ from qgemv_*, the value is the same to 1e-3).
 *   w   : weight blocks [n][k/block_elems]
 *   xq  : Q8_1 [b][k/32], the b rows back to back, 16-byte aligned
 *   y   : f32 [b][n] row-major, written
 *   b   : 0..8 (0 and n = 0 do nothing);  b * n <= 2^31 - 1
 *   k   : multiple of 32 (Q8_0) or 256 (Q4_K, Q6_K), <= 2^24; k = 0 writes y = 0
 */
qg_status qgemv_q8_0_batch(const void *w, const void *xq, float *y, int64_t b, int64_t n, int64_t k,
                           hipStream_t stream);
qg_status qgemv_q4_k_batch(const void *w, const void *xq, float *y, int64_t b, int64_t n, int64_t k,
                           hipStream_t stream);
qg_status qgemv_q6_k_batch(const void *w, const void *xq, float *y, int64_t b, int64_t n, int64_t k,
                           hipStream_t stream);

/*
 * rmsnorm_quantize_q8_1 -- the activation prologue of a projection in the
 * model families the infr page runs ("models": Llama, Qwen, Gemma): per row,
 *   r = 1 / sqrt(sum(x^2) / k + eps)     (fp32; the sum in a fixed order)
 *   xq = Q8_1((x * r) * gamma)           (fp32 products, then quantize_q8_1's rule)
 *   x     : f32 [rows][k];  gamma : f32 [k];  both 16-byte aligned
 *   xq    : Q8_1 [rows][k/32], written;  r_out : f32 [rows] or NULL
 *   k     : multiple of 32, <= 2^24;  eps >= 0 and finite
 * rows = 0 or k = 0 writes nothing.
 */
qg_status rmsnorm_quantize_q8_1(const float *x, const float *gamma, float eps, void *xq, float *r_out,
                                int64_t rows, int64_t k, hipStream_t stream);

/*
 * qgemm_q4_k_mmq -- prefill product on int8 matrix cores.
 * Defining passages: infr page, "models" (in-shader dequantization feeding an
 * integer-dot mmq) and "Vulkan-first, Metal too" (cooperative-matrix matmul on
 * AMD); infr page, "llama.cpp-compatible refs" (Q4_K_M, the default quant,
 * whose bulk is Q4_K weights).
 * c[i][r] = sum_j a^[i][j] * w^[r][j]: each 32-wide slice of k is one int8
 * 32x32x32 MFMA tile of exact per-block dots, rescaled in fp32 by d*sc_j*d_a
 * with the min term -dmin*m_j*d_a*sum(qa) of that Q8_1 block.
 *   w   : Q4_K [n][k/256]
 *   aq  : Q8_1 [m][k/32] (m activation rows, e.g. tokens)
 *   c   : f32 [m][n] row-major, written
 *   k   : multiple of 256, <= 2^24;  m, n <= 2^31 - 1
 */
qg_status qgemm_q4_k_mmq(const void *w, const void *aq, float *c, int64_t m, int64_t n, int64_t k,
                         hipStream_t stream);

/*
 * qgemm_q6_k_mmq / qgemm_q8_0_mmq / qgemm_q5_k_mmq -- the same prefill product
 * for the other two integer-dot weight types the blazr README ("Model Formats
 * > GGUF") names, and for Q5_K (see qgemv_q5_k for its block).
 *   Q6_K: each 16-wide sub-block is one int8 32x32x16 MFMA tile of exact dots
 *         of (q - 32) and qa, rescaled in fp32 by d*scales_j*d_a.
 *   Q8_0: each 32-wide block is one int8 32x32x32 MFMA tile of exact dots,
 *         rescaled in fp32 by d_w*d_a.
 *   Q5_K: as Q4_K with the 5-bit codes.
 *   w   : Q6_K or Q5_K [n][k/256], or Q8_0 [n][k/32]
 *   aq  : Q8_1 [m][k/32];  c : f32 [m][n] row-major, written
 *   k   : multiple of 256 (Q6_K, Q5_K) or 32 (Q8_0), <= 2^24;  m, n <= 2^31 - 1
 * Same errors and conventions as qgemm_q4_k_mmq.
 */
qg_status qgemm_q6_k_mmq(const void *w, const void *aq, float *c, int64_t m, int64_t n, int64_t k,
                         hipStream_t stream);
qg_status qgemm_q8_0_mmq(const void *w, const void *aq, float *c, int64_t m, int64_t n, int64_t k,
                         hipStream_t stream);
qg_status qgemm_q5_k_mmq(const void *w, const void *aq, float *c, int64_t m, int64_t n, int64_t k,
                         hipStream_t stream);

/*
 * qgemm_q4_0_mmq / qgemm_q5_0_mmq -- the prefill product for Q4_0 and Q5_0
 * weights (blocks as in qgemv_q4_0 / qgemv_q5_0): each 32-wide block is one
 * int8 32x32x32 MFMA tile of exact dots of (q - 8) (or q - 16) and qa,
 * rescaled in fp32 by d_w*d_a.  Arguments, errors and conventions as
 * qgemm_q8_0_mmq (w: [n][k/32]; k a multiple of 32, <= 2^24).
 */
qg_status qgemm_q4_0_mmq(const void *w, const void *aq, float *c, int64_t m, int64_t n, int64_t k,
                         hipStream_t stream);
qg_status qgemm_q5_0_mmq(const void *w, const void *aq, float *c, int64_t m, int64_t n, int64_t k,
                         hipStream_t stream);

/*
 * moe_qgemv_q4_k_workspace_size / moe_qgemv_q4_k -- MoE expert FFN with Q4_K
 * experts (the expert_gateup + down calls of an MoE layer).  Defining
 * passages: infr page, "Per-op device profiling" (expert_gateup, a dispatch
 * role of its own), "Paged experts, spillable KV" (MoE experts streamed from
 * VRAM) and "install" (a Qwen3-30B-A3B Q4_K_M MoE model).  The pages do not
 * write the FFN out; the reading is the gated-SiLU expert FFN of those MoE
 * models.  For token t and each routed slot i with expert e = ids[t][i]:
 *   g = Wgu[e][0:n_ff] . x^_t, u = Wgu[e][n_ff:2n_ff] . x^_t       (fp32)
 *   h = silu(g) * u, silu(g) = g / (1 + exp(-g))                   (fp32)
 *   h^ = Q8_1(h) exactly as quantize_q8_1
 *   out[t] = sum_i weights[t][i] * (Wdown[e] . h^)                  (fp32)
 * The routing table is an input; ids outside [0, n_expert) contribute nothing.
 * Each touched expert's weights are read once for all of its tokens.
 *   w_gate_up : Q4_K [n_expert][2*n_ff][n_embd/256]; rows 0..n_ff-1 gate,
 *               n_ff..2n_ff-1 up
 *   w_down    : Q4_K [n_expert][n_embd][n_ff/256]
 *   xq        : Q8_1 [n_tok][n_embd/32]
 *   ids       : int32 [n_tok][top_k];  weights : f32 [n_tok][top_k]
 *   out       : f32 [n_tok][n_embd], written
 *   workspace : device scratch of at least moe_qgemv_q4_k_workspace_size()
 *               bytes, 256-byte aligned, owned by the caller.  Layout, for
 *               P = n_tok*top_k pairs p = t*top_k + i:
 *                 [0, P*(n_ff/32)*36)            h^ per pair, Q8_1
 *                 then f32 [P][2*n_ff]           g | u per pair
 *                 then f32 [P][n_embd]           weights[p] * (Wdown . h^)
 *                                                (four-kernel path only)
 *               each region starting on a 256-byte boundary.  Every byte the
 *               call reads it has written first in the same call.
 * Small routing tables (n_tok*top_k <= 256 over <= 256 experts, n_embd <=
 * 4096, n_ff/64 a power of two in 4..64 times 1, 2 or 3, top_k*n_ff*1.25 <=
 * 32 KiB) run two kernels: gate/up, then a token-major down that forms h^
 * first and sums the slots itself; other shapes run four (gate/up,
 * activation, down, routed sum).
 *   n_embd, n_ff : multiples of 256, <= 2^20;  top_k in [1, 64];
 *   n_tok * top_k <= 2^20;  n_expert in [1, 2^16]
 */
size_t moe_qgemv_q4_k_workspace_size(int64_t n_tok, int64_t top_k, int64_t n_expert, int64_t n_ff,
                                     int64_t n_embd);

/*
 * moe_router_topk -- the router that makes the routing table moe_qgemv_q4_k
 * takes: two launches on `stream` (the logits, then the selection).  Per
 * token t:
 *   logits[t][e] = sum_h w_router[e][h] * x[t][h]           (fp32)
 *   ids[t][0..top_k-1]: the top_k experts by logit, larger first, equal
 *                       logits in increasing expert order
 *   weights[t][i] = exp(l_i - l_0) / sum_j exp(l_j - l_0) over the selected
 * (the softmax of the selected logits, as the MoE models the infr page runs
 * use; "models").  The router matrix is f32, as in their Q4_K_M files.
 *   w_router : f32 [n_expert][n_embd];  x : f32 [n_tok][n_embd] (16-byte aligned)
 *   ids      : int32 [n_tok][top_k], weights : f32 [n_tok][top_k], written
 *   logits   : f32 [n_tok][n_expert], written (the selection reads them back);
 *              each logit is summed in an order that depends on n_embd alone
 *   n_expert in [1, 256];  top_k in [1, min(64, n_expert)];
 *   n_embd a multiple of 4 in [4, 65536];  n_tok = 0 does nothing (x, ids,
 *   weights and logits may then be NULL)
 * NaN logits are not defined.
 */
qg_status moe_router_topk(const float *w_router, const float *x, int32_t *ids, float *weights, float *logits,
                          int64_t n_tok, int64_t n_expert, int64_t n_embd, int64_t top_k, hipStream_t stream);
qg_status moe_qgemv_q4_k(const void *w_gate_up, const void *w_down, const void *xq, const int32_t *ids,
                         const float *weights, float *out, int64_t n_tok, int64_t top_k, int64_t n_expert,
                         int64_t n_ff, int64_t n_embd, void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * moe_qgemv_q4_k_noalloc -- moe_qgemv_q4_k without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  It allocates
 * nothing: the workspace is a device array of the library, one copy per GPU,
 * moe_qgemv_q4_k_noalloc_max_workspace() bytes (32 MiB), held until the
 * process ends.  Same computation, arguments, limits and errors as
 * moe_qgemv_q4_k (its kernels are the same), except:
 *   - a call whose moe_qgemv_q4_k_workspace_size() exceeds the maximum
 *     returns QG_ERR_WORKSPACE and launches nothing;
 *   - all calls on one GPU share that GPU's array: calls that overlap on one
 *     GPU (streams with no ordering between them) race.  Calls ordered on a
 *     stream do not: every workspace byte a call reads it has written first.
 */
size_t moe_qgemv_q4_k_noalloc_max_workspace(void);
qg_status moe_qgemv_q4_k_noalloc(const void *w_gate_up, const void *w_down, const void *xq, const int32_t *ids,
                                 const float *weights, float *out, int64_t n_tok, int64_t top_k, int64_t n_expert,
                                 int64_t n_ff, int64_t n_embd, hipStream_t stream);

/*
 * Test access to the exact per-block int32 dots, computed by the same device
 * unpack and dot code the products above run (not for production use).
 *   qg_blockdots_q8_0 : D int32 [n][k/32],  D[r][b] = sum_i qw*qa over block b
 *   qg_blockdots_q4_k : D int32 [n][k/32] (4-bit codes times qa per 32 values),
 *                       S int32 [k/32] = sum of qa per activation block
 *   qg_blockdots_q5_k : as qg_blockdots_q4_k, with the 5-bit Q5_K codes
 *   qg_blockdots_q6_k : D int32 [n][k/16],  sum over 16 values of (q-32)*qa
 *   qg_blockdots_q4_0, qg_blockdots_q5_0 : D int32 [n][k/32], sum over the
 *                       block of (q-8)*qa or (q-16)*qa
 *   qg_blockdots_q4_k_mmq : D int32 [m][n][k/32] from the int8 MFMA tiles of
 *                       qgemm_q4_k_mmq; m*n*(k/32) <= 2^28
 *   qg_blockdots_q8_0_mmq, qg_blockdots_q5_k_mmq, qg_blockdots_q4_0_mmq,
 *   qg_blockdots_q5_0_mmq : the same for qgemm_q8_0_mmq, qgemm_q5_k_mmq,
 *                       qgemm_q4_0_mmq and qgemm_q5_0_mmq
 *   qg_blockdots_q6_k_mmq : D int32 [m][n][k/16] per 16-value sub-block, from
 *                       qgemm_q6_k_mmq; m*n*(k/16) <= 2^28
 *   qg_blockdots_q8_0_batch, qg_blockdots_q4_k_batch, qg_blockdots_q6_k_batch :
 *                       D int32 [b][n][k/32] (Q6_K: [b][n][k/16] per 16-value
 *                       sub-block) from the kernel qgemv_*_batch runs for b
 *                       rows (v_dot4 or matrix cores), on its launch grid;
 *                       b*n*(k/32) (Q6_K: b*n*(k/16)) <= 2^29
 * The GEMV and small-batch dumps run on the grid the product call of the same
 * shape uses, so a dump walks the rows exactly as that launch does.
 * Same validation rules and limits as the corresponding products.
 */
qg_status qg_blockdots_q8_0(const void *w, const void *xq, int32_t *D, int64_t n, int64_t k, hipStream_t stream);
qg_status qg_blockdots_q4_k(const void *w, const void *xq, int32_t *D, int32_t *S, int64_t n, int64_t k,
                            hipStream_t stream);
qg_status qg_blockdots_q5_k(const void *w, const void *xq, int32_t *D, int32_t *S, int64_t n, int64_t k,
                            hipStream_t stream);
qg_status qg_blockdots_q6_k(const void *w, const void *xq, int32_t *D, int64_t n, int64_t k, hipStream_t stream);
qg_status qg_blockdots_q4_k_mmq(const void *w, const void *aq, int32_t *D, int64_t m, int64_t n, int64_t k,
                                hipStream_t stream);
qg_status qg_blockdots_q8_0_mmq(const void *w, const void *aq, int32_t *D, int64_t m, int64_t n, int64_t k,
                                hipStream_t stream);
qg_status qg_blockdots_q6_k_mmq(const void *w, const void *aq, int32_t *D, int64_t m, int64_t n, int64_t k,
                                hipStream_t stream);
qg_status qg_blockdots_q5_k_mmq(const void *w, const void *aq, int32_t *D, int64_t m, int64_t n, int64_t k,
                                hipStream_t stream);
qg_status qg_blockdots_q4_0(const void *w, const void *xq, int32_t *D, int64_t n, int64_t k, hipStream_t stream);
qg_status qg_blockdots_q5_0(const void *w, const void *xq, int32_t *D, int64_t n, int64_t k, hipStream_t stream);
qg_status qg_blockdots_q4_0_mmq(const void *w, const void *aq, int32_t *D, int64_t m, int64_t n, int64_t k,
                                hipStream_t stream);
qg_status qg_blockdots_q5_0_mmq(const void *w, const void *aq, int32_t *D, int64_t m, int64_t n, int64_t k,
                                hipStream_t stream);
qg_status qg_blockdots_q8_0_batch(const void *w, const void *xq, int32_t *D, int64_t b, int64_t n, int64_t k,
                                  hipStream_t stream);
qg_status qg_blockdots_q4_k_batch(const void *w, const void *xq, int32_t *D, int64_t b, int64_t n, int64_t k,
                                  hipStream_t stream);
qg_status qg_blockdots_q6_k_batch(const void *w, const void *xq, int32_t *D, int64_t b, int64_t n, int64_t k,
                                  hipStream_t stream);
/*
 * qg_blockdots_moe_q4_k : the exact dots of moe_qgemv_q4_k's expert GEMVs,
 *                       from their dump instances on the product's grids:
 *                       D_gu int32 [P][2*n_ff][n_embd/32] (gate/up rows
 *                       against the token's Q8_1 row) and D_dn int32
 *                       [P][n_embd][n_ff/32] (down rows against the pair's
 *                       h^, which the call leaves in the workspace as the
 *                       product does); rows of pairs with an out-of-range id
 *                       are not written.  out is not written.  Same arguments
 *                       and errors as moe_qgemv_q4_k; P*2*n_ff*(n_embd/32) and
 *                       P*n_embd*(n_ff/32) <= 2^29.
 * qg_moe_q4_k_launches : kernel launches moe_qgemv_q4_k makes for a shape
 *                       (2 or 4; 0 for an invalid shape).
 */
qg_status qg_blockdots_moe_q4_k(const void *w_gate_up, const void *w_down, const void *xq, const int32_t *ids,
                                const float *weights, int64_t n_tok, int64_t top_k, int64_t n_expert, int64_t n_ff,
                                int64_t n_embd, void *workspace, size_t workspace_bytes, int32_t *D_gu,
                                int32_t *D_dn, hipStream_t stream);
int qg_moe_q4_k_launches(int64_t n_tok, int64_t top_k, int64_t n_expert, int64_t n_ff, int64_t n_embd);

/*
 * Measurement references (for the roofline fractions the benchmark reports;
 * the per-kernel accounting of infr page, "Per-op device profiling").  They
 * compute nothing of the products above.
 *   qg_peak_read : reads every 16-byte word of src (bytes, a multiple of 16,
 *                  16-byte aligned) once, with grid workgroups of threads
 *                  (64..1024, a multiple of 64) keeping loads (4 or 8) loads
 *                  in flight per thread, non-temporal if nontemporal != 0.
 *                  sink: uint32 [sink_entries >= grid], practically never
 *                  written (it only keeps the loads from being dropped).
 *   qg_peak_mfma_i8 : iters (1..2^24) rounds of four independent
 *                  v_mfma_i32_32x32x32_i8 per wave, eight 4-wave workgroups
 *                  per CU; *ops (host pointer) receives the int8 operation
 *                  count of the launch (2*32*32*32 per MFMA).  sink: int32
 *                  [sink_entries >= 8 * CUs].
 * Same validation and error rules as the products.
 */
qg_status qg_peak_read(const void *src, int64_t bytes, uint32_t *sink, int64_t sink_entries, int32_t grid,
                       int32_t threads, int32_t loads, int32_t nontemporal, hipStream_t stream);
qg_status qg_peak_mfma_i8(int32_t *sink, int64_t sink_entries, int64_t iters, int64_t *ops, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QGGUF_H */
