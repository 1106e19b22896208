/*
 * vq.h -- C ABI of the block-quantized matmul library for AMD Instinct MI355X
 * (gfx950).
 *
 * Y = X * W^T with block-quantized weights (Q4_K, Q5_K, Q6_K, Q8_0) and activations
 * quantized on the device to Q8_K (paired with the K-quants) or Q8_1 (paired
 * with Q8_0): decode GEMV, prefill GEMM and the routed-expert grouped GEMM
 * with the weighted expert sum.
 *
 * Pages this contract follows (by title and section):
 *  - vllm.cpp PR #2890 "fuse silu-mul with Q8_K quant epilogue": commit
 *    "kROCM keep-quant provider" (Y = X*W^T on block weights; unsupported
 *    dtypes are an error naming the dtype, never a silent fallback; outputs
 *    fully overwritten, so a poisoned output buffer is a valid input), commit
 *    "grouped Q8_0 delegation" (capability query; Q8_0 dots a 32-block
 *    activation, the K-quants dot Q8_K super-blocks), commit "T4a
 *    VT_GEMV_MMVQ" (decode GEMV with the activation quantizer folded into its
 *    prologue), commit "QuantizeQ8KKWarpCoop" (the Q8_K quantizer), commit
 *    "Lever-C norm-quant epilogue" (a matmul that is handed pre-quantized
 *    activations skips its own quantizer).
 *  - strix-llama.cpp PR #18 "Optimize ROCM Prefill and Decode": commits
 *    "mul_mat_vec_q_fq" (fused Q8_1 quantizer, amax / IEEE division / roundf),
 *    "mul_mat_vec_q_fq generic" (Q8_1 block sum in butterfly order),
 *    "routed-compact" (MUL_MAT_ID tiles sized from rows per expert) and
 *    "weighted expert sum" (slot-ordered multiply then add, no FMA).
 *
 * Conventions for every entry point:
 *  - Pointers named W, X, x, Xq, Y, y, ids, route_w, ws are DEVICE memory
 *    owned by the caller; the library never allocates, frees or keeps them.
 *  - Every call is asynchronous on the given stream (0 = the null stream) and
 *    may be called from several host threads.
 *  - Arguments are validated on the host before anything is launched; a
 *    failed check returns a status, launches nothing, and sets a per-thread
 *    message (vq_last_error) naming the offending type or size.  There is no
 *    host fallback: the only compute path is the gfx950 kernels.
 *  - Outputs are fully overwritten (no accumulation into Y).
 *  - Block weight buffers and quantized-activation buffers must be 16-byte
 *    aligned; fp32 buffers 4-byte aligned (16-byte for vq_weighted_sum).
 */
#ifndef VQ_H
#define VQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------------- */
/* Types and block layouts.                                                */
/*                                                                         */
/* The pages name the fields of each format but give no bit positions; the */
/* layouts below are this library's own.                                    */
/*                                                                         */
/* VQ_Q4_K  weights, 144 bytes per 256 values, little endian:              */
/*   [0,2) d (binary16)  [2,4) dmin (binary16)  [4,16) scales  [16,144) qs  */
/*   scales byte j (j<8): bits 0-5 = sc_j, bits 6-7 = bits 0-1 of m_j       */
/*   scales byte 8+(j>>1), nibble (j&1) = bits 2-5 of m_j                   */
/*   qs byte 32c+l (c<4, l<32): low nibble = element 64c+l,                 */
/*                              high nibble = element 64c+32+l              */
/*   value_i = d*sc_(i/32)*q_i - dmin*m_(i/32)                              */
/* VQ_Q6_K  weights, 210 bytes per 256 values:                             */
/*   [0,128) ql  [128,192) qh  [192,208) int8 sc[16]  [208,210) d (binary16) */
/*   element e, h=e/128, r=e%128: low 4 bits = nibble r/64 of               */
/*   ql[64h + r%64]; high 2 bits = bit pair r/32 of qh[32h + r%32]          */
/*   value_e = d*sc_(e/16)*(q_e - 32), q_e in 0..63                         */
/* VQ_Q8_0  weights, 34 bytes per 32 values: [0,2) d (binary16), [2,34)     */
/*   int8 q; value_i = d*q_i                                                */
/* VQ_Q5_K  weights, 176 bytes per 256 values (the pages name Q5_K without  */
/*   a layout): [0,16) d, dmin and scales exactly as Q4_K; [16,48) qh, bit */
/*   j of byte 16+l = bit 4 of element 32j+l; [48,176) the Q4_K nibbles;    */
/*   q_i = nibble_i | qhbit_i << 4 in 0..31; value_i = d*sc*q_i - dmin*m    */
/* Weight matrices [N][K] are stored row-major: row n is K/QK consecutive   */
/* blocks with no padding.  Grouped weights are [E][N][K/QK] blocks.        */
/*                                                                         */
/* VQ_Q8_K  activations (device layout, planar), for M rows of K values:   */
/*   qs    int8   [M][K]       at offset 0                                 */
/*   d     fp32   [M][K/256]   at offset align256(M*K)                     */
/*   bsums int16  [M][K/16]    after d, 256-byte aligned                   */
/*   value = d*qs; bsums[m][j] = sum of qs[m][16j .. 16j+15]               */
/* VQ_Q8_1  activations (device layout, planar):                          */
/*   qs    int8     [M][K]     at offset 0                                 */
/*   d     binary16 [M][K/32]  at offset align256(M*K)                     */
/*   s     binary16 [M][K/32]  after d, 256-byte aligned                   */
/*   value = d*qs; s = binary16 of the block's binary32 butterfly sum of x  */
/* ---------------------------------------------------------------------- */
typedef enum {
    VQ_Q4_K = 0,
    VQ_Q6_K = 1,
    VQ_Q8_0 = 2,
    VQ_Q8_K = 3,
    VQ_Q8_1 = 4,
    VQ_Q5_K = 5
} vq_type;

typedef enum {
    VQ_OK = 0,
    VQ_ERR_INVALID_ARG = 1,      /* null / misaligned pointer, negative size */
    VQ_ERR_UNSUPPORTED_TYPE = 2, /* the type cannot be used in this role */
    VQ_ERR_TYPE_PAIR = 3,        /* weight/activation types do not pair */
    VQ_ERR_SHAPE = 4,            /* K not a multiple of the block length, size limits */
    VQ_ERR_ALIAS = 5,            /* an output overlaps an input */
    VQ_ERR_WORKSPACE = 6,        /* workspace missing or too small */
    VQ_ERR_HIP = 7,              /* a HIP runtime call failed (launch, attribute) */
    VQ_ERR_DEVICE = 8            /* a kernel reported a failure (vq_device_status) */
} vq_status;

/* Operations for vq_is_supported. */
typedef enum {
    VQ_OP_GEMV = 0,
    VQ_OP_GEMM = 1,
    VQ_OP_GEMM_GROUPED = 2
} vq_op;

/* Static string for a status code. */
const char* vq_status_string(vq_status s);

/* Message of the last failed call on this host thread ("" if none). */
const char* vq_last_error(void);

/* Static name of a type ("Q4_K", ...), or "unknown". */
const char* vq_type_name(int t);

/* 1 if weights of type w with activations of type act are supported by op,
 * else 0 (the pages' keep-quant capability query).  Q4_K and Q6_K pair with
 * Q8_K; Q8_0 pairs with Q8_1; every op supports every pair. */
int vq_is_supported(int w, int act, int op);

/* Values per block (256 or 32) and bytes per block; 0 for an unknown type. */
int vq_block_values(int t);
size_t vq_block_bytes(int t);

/* Bytes of an [N][K] block weight matrix; 0 if K is not a multiple of the
 * block length or the type is not a weight type. */
size_t vq_weight_bytes(int w, int64_t N, int64_t K);

/* Bytes of the planar activation buffer for M rows of K values (layout
 * above); 0 on a bad type or K. */
size_t vq_act_bytes(int act, int64_t M, int64_t K);

/* Byte offsets of the d plane and of the bsums (Q8_K) / s (Q8_1) plane. */
size_t vq_act_d_offset(int act, int64_t M, int64_t K);
size_t vq_act_aux_offset(int act, int64_t M, int64_t K);

/* ---------------------------------------------------------------------- */
/* Activation quantizer.                                                   */
/*   Q8_K (QuantizeQ8KKWarpCoop): per row and 256-value super-block, the     */
/*   first value of largest magnitude mx (ascending scan, strict compare, a */
/*   NaN is never chosen); all-zero or all-NaN blocks give the zero block; */
/*   iscale = -127/mx (IEEE division); q = min(127, rint(iscale*x)) with    */
/*   ties to even; d = 1/iscale; bsums = sums of 16 quants.                */
/*   Q8_1 (mul_mat_vec_q_fq): per 32-block amax, d = amax/127, q =          */
/*   roundf(x/d) (IEEE division, halves away from zero; 0 when amax = 0),  */
/*   s = binary32 butterfly sum (xor 16, 8, 4, 2, 1); d and s stored as     */
/*   binary16, nearest even.                                               */
/* X: fp32 [M][ldx] (ldx >= K); Xq: vq_act_bytes(act, M, K) bytes, written   */
/* completely.  Blocks holding Inf, or NaN mixed with numbers, are outside  */
/* the contract (their bytes are unspecified but nothing faults).           */
/* ---------------------------------------------------------------------- */
vq_status vq_quantize_act(int act, const float* X, int64_t M, int64_t K, int64_t ldx,
                          void* Xq, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Weight encoder (data preparation, not on the matmul path): fp32 W        */
/* [N][K] -> blocks.  Per 32-value sub-block (Q4_K): lo = min(0, min w),    */
/* hi = max w, s = (hi-lo)/15, o = -lo; d = f16(max s/63), dmin =            */
/* f16(max o/63); sc = clamp(rint(s/d),0,63); m = clamp(rint(o/dmin),0,63); */
/* q = clamp(rint((w + dmin*m)/(d*sc)),0,15).  Q6_K (16-value sub-blocks):  */
/* s = max|w|/31, d = f16(max s/127), sc = clamp(rint(s/d),0,127), q =       */
/* clamp(rint(w/(d*sc)),-32,31)+32.  Q8_0: d = amax/127, q =                */
/* clamp(roundf(w/d),-127,127), d stored as binary16.  A zero divisor gives */
/* a zero quant (stored 32 for Q6_K).  All arithmetic binary32, no FMA.     */
/* ---------------------------------------------------------------------- */
vq_status vq_quantize_weights(int w, const float* W, int64_t N, int64_t K, void* Wq,
                              hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Producers with the activation quantizer as their epilogue (vllm.cpp PR   */
/* #2890, commits "Norm epilogue" and "SiLU-mul quant"): one launch writes   */
/* the producer's binary32 output Y (optional) and its quantized blocks Xq, */
/* which are byte-identical to vq_quantize_act applied to that Y.  Xq then  */
/* goes to vq_gemm (any M, including the decode case M = 1) or the grouped  */
/* calls in place of a separate quantizer launch.                           */
/*   vq_rmsnorm_quant: Y = X * r * gamma per row, r = 1/sqrt(sum(x^2)/K +    */
/*     eps) (binary32; the sum's order is the kernel's own).  gamma fp32 [K]. */
/*   vq_silu_mul_quant: Y = silu(G) * U = G / (1 + exp(-G)) * U (binary32).  */
/*     G and U share the row stride ldx (a [M][2K] gate|up buffer works with */
/*     U = G + K, ldx = 2K).                                                 */
/* act: VQ_Q8_K or VQ_Q8_1 (K a multiple of its block); X, G, U:             */
/* fp32 [M][ldx]; Y: NULL or fp32 [M][ldy]; Xq: vq_act_bytes(act, M, K)     */
/* bytes.  Y and Xq must not overlap the inputs or each other.             */
/* ---------------------------------------------------------------------- */
vq_status vq_rmsnorm_quant(int act, const float* X, const float* gamma, int64_t M, int64_t K, int64_t ldx,
                           float eps, float* Y, int64_t ldy, void* Xq, hipStream_t stream);
vq_status vq_silu_mul_quant(int act, const float* G, const float* U, int64_t M, int64_t K, int64_t ldx,
                            float* Y, int64_t ldy, void* Xq, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Decode GEMV (M = 1), activation quantizer fused into the prologue:       */
/*   y[n] = sum over blocks b ascending of c_b, binary32, where for Q4_K     */
/*   c = da*(d*S - dmin*Mn) with S = sum_j sc_j*I_j, Mn = sum_j m_j*bsum32_j */
/*   (I_j the exact int32 sub-block dot), for Q6_K c = da*(d*S) with         */
/*   S = sum_j sc_j*I_j over (q-32), for Q8_0 c = (dw*da)*I.  The result is  */
/*   bit-identical to that fixed-order definition.                         */
/* W: [N][K] blocks of type w; x: fp32 [K]; y: fp32 [N]; xq_out: NULL or      */
/* vq_act_bytes(act, 1, K) bytes that receive the fused quantizer's          */
/* activation bytes (identical to vq_quantize_act's).  One weight row and  */
/* the quantized activation must fit the 160 KiB LDS: K up to about 90K     */
/* (Q4_K), 84K (Q5_K), 78K (Q6_K), 32K (Q8_0); longer K is VQ_ERR_SHAPE.    */
/* ---------------------------------------------------------------------- */
vq_status vq_gemv(int w, const void* W, int64_t N, int64_t K, const float* x, float* y,
                  void* xq_out, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Prefill GEMM: Y[m][n] = sum_k deq(Xq)[m][k]*deq(W)[n][k] for m < M,       */
/* n < N, through exact int32 sub-block sums and binary32 scale combines.   */
/* Xq is the planar activation buffer of type act (Q8_K for Q4_K/Q6_K/Q5_K, */
/* Q8_1 for Q8_0) holding M rows; Y fp32 with row stride ldy >= N.          */
/* Small batches, M <= vq_small_batch_max(w), run on the decode GEMV kernel */
/* over the pre-quantized rows (the weights streamed once for all rows, in  */
/* groups of 4 rows above 8), larger M on the int8 MFMA GEMM.               */
/* Numerics: the int32 sub-block sums are exact; the binary32 combine and   */
/* accumulation order is the kernel's own (fused multiply-adds), fixed for  */
/* given arguments, so two calls with the same arguments (including         */
/* ws_bytes) give bitwise equal Y; Y meets the pages' tolerance (NMSE <=    */
/* 1e-6 against the fixed-order binary32 definition, relative error <= 5e-4 */
/* against the fp64 dequantized product).                                  */
/* ws: NULL or a device workspace of at least vq_gemm_workspace(w, M, N, K) */
/* bytes, 256-byte aligned, ZERO-FILLED BEFORE ITS FIRST USE; the MFMA GEMM */
/* splits K across workgroups when its tiles cannot fill the chip (a grid  */
/* of at most one tile per CU into up to eight parts, one or two           */
/* workgroups per CU; up to two tiles per CU with K >= 4096 in two or      */
/* three), keeps per-tile arrival counters in the first 64 KiB of the      */
/* workspace (the same place for every shape) and the fp32 partial tiles   */
/* after them, and leaves the counters zero when the call completes, so    */
/* one workspace serves calls of any shape.  A smaller workspace (or NULL) */
/* gives fewer splits (or none): the result stays within the tolerance    */
/* but its fp32 rounding may differ.  Calls that share a workspace must    */
/* not run concurrently (same stream, or ordered streams).                 */
/* ---------------------------------------------------------------------- */
vq_status vq_gemm(int w, const void* W, int64_t N, int64_t K, int act, const void* Xq,
                  int64_t M, float* Y, int64_t ldy, void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes vq_gemm wants for this shape (0: none needed). */
size_t vq_gemm_workspace(int w, int64_t M, int64_t N, int64_t K);

/* ---------------------------------------------------------------------- */
/* The GEMV <-> GEMM crossover of vq_gemm (vllm.cpp PR #2890, "lever-B1":  */
/* the fold crossover made tunable at run time): vq_gemm with weight type w */
/* runs M <= max_m on the GEMV kernel.  max_m in [0, 64] (0: never), -1     */
/* restores the default (Q4_K 8, Q5_K 8, Q6_K 8, Q8_0 32, measured on      */
/* the decode shapes).  Per calling thread: other threads keep their own. */
/* vq_small_batch_max returns the current value (-1 for a non-weight type). */
/* ---------------------------------------------------------------------- */
vq_status vq_set_small_batch_max(int w, int64_t max_m);
int64_t vq_small_batch_max(int w);

/* ---------------------------------------------------------------------- */
/* Failures seen on the device.  Kernels never fault or hang on purpose:   */
/* the decode GEMV's loader waves wait for each other a bounded number of  */
/* polls, and a workgroup whose wait gives up writes its rows as NaN and   */
/* sets bit 1 of the GPU's device error word.  In debug mode the grouped    */
/* calls also check the expert ids on the device (bit 2: an id outside      */
/* [0, E), bit 4: an id repeated within a token; such pairs are skipped or  */
/* computed as documented above, never read out of bounds).                 */
/* vq_device_status(stream): waits for `stream`, then returns VQ_OK, or     */
/* VQ_ERR_DEVICE with the bits named in vq_last_error, and clears the word. */
/* vq_set_debug(flags, wait_polls), per calling thread: VQ_DEBUG_SYNC makes */
/* vq_gemv, vq_gemm and the grouped calls wait for their launches and      */
/* return VQ_ERR_DEVICE themselves; VQ_DEBUG_CHECK_IDS turns on the id      */
/* check; wait_polls bounds the GEMV loaders' wait (0: the default 2^20;    */
/* a tiny bound makes the wait give up, for tests of this reporting).       */
/* ---------------------------------------------------------------------- */
#define VQ_DEBUG_SYNC 1
#define VQ_DEBUG_CHECK_IDS 2
vq_status vq_set_debug(int flags, int64_t wait_polls);
vq_status vq_device_status(hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Measurement: the streaming floor of a decode GEMV launch.  Reads the     */
/* weight bytes that vq_gemv(w, W, N, K, ...) reads, with the GEMV's grid    */
/* and workgroup size, each workgroup its own rows' bytes once, and does    */
/* nothing else; its time is what this launch shape needs just to stream    */
/* the weights from memory ([P3] "mul_mat_vec_q_fq": the decode GEMV keeps  */
/* the weight stream in flight while it computes, so the stream bounds it). */
/* W: the weights as for vq_gemv (16-byte aligned); sink: device memory of  */
/* at least 4*N bytes, 4-byte aligned, that the probe may write (it writes  */
/* nothing in practice).  Shapes and errors as vq_gemv.                    */
/* ---------------------------------------------------------------------- */
vq_status vq_stream_probe(int w, const void* W, int64_t N, int64_t K, void* sink, size_t sink_bytes,
                          hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Measurement: the int8 MFMA ceiling, the secondary reference beside the   */
/* 5.0 POP/s spec for the GEMMs' fractions.  Two workgroups of four waves   */
/* per CU, each wave running eight independent chains of                    */
/* v_mfma_i32_32x32x32_i8 on register operands for `iters` rounds and      */
/* nothing else: the rate the matrix cores sustain at this part's clocks    */
/* under load.  iters in [1, 2^24]; sink: device memory of at least 4       */
/* bytes, 4-byte aligned (stored to only if the accumulators reach a value  */
/* the probe never produces in practice); ops_out (host, may be NULL): the  */
/* int8 operations of the launch (2*32*32*32 per MFMA).                     */
/* ---------------------------------------------------------------------- */
vq_status vq_mfma_probe(int64_t iters, void* sink, size_t sink_bytes, int64_t* ops_out, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Row blocks of the MFMA arm of vq_gemm.  The GEMM kernel addresses the    */
/* activation bytes of one launch with 32-bit offsets, so vq_gemm launches  */
/* it once per block of at most floor(2^31 / K) rows (rounded down to the   */
/* tile height), which is one launch for every practical shape; the Q8_0   */
/* grouped GEMM likewise launches once per 32768 routed tiles.  rows > 0    */
/* caps the block at that many rows (any value; for tests of the blocking)  */
/* and the Q8_0 grouped launches at max(1, rows / 96) routed tiles of 96    */
/* rows; 0 restores the default.  The K-quant results stay within the     */
/* GEMM's tolerance under any blocking (a block's K splits depend on its   */
/* rows); Q8_0 results do not depend on it.  Per calling thread: other     */
/* threads keep their own.  rows < 0: VQ_ERR_INVALID_ARG.                  */
/* ---------------------------------------------------------------------- */
vq_status vq_set_gemm_row_block(int64_t rows);

/* ---------------------------------------------------------------------- */
/* Routed-expert grouped GEMM (MUL_MAT_ID, broadcast arm) with the weighted  */
/* expert sum ([P3] "routed-compact J rule" and "weighted expert sum";     */
/* [P2] "grouped Q8_0 delegation": every weight type, Q8_0 paired with a    */
/* 32-block activation):                                                   */
/*   Y[t][s][:] = W_(ids[t][s]) . x_t  for t < T, s < top_k                 */
/*   Ysum[t][n] = (((w0*y0 + w1*y1) + w2*y2) + ...), slots ascending, each  */
/*                product and sum rounded on its own (skipped if Ysum NULL) */
/* w: Q4_K, Q5_K, Q6_K (act Q8_K) or Q8_0 (act Q8_1).  W: [E][N][K/QK] blocks; */
/* Xq: planar activation buffer of T rows; ids int32 [T][top_k], each in    */
/* [0,E) and distinct within a token (a precondition, not checked on the    */
/* device; a pair whose id is outside [0,E) is not computed: its Y row keeps */
/* what it held, and Ysum adds that row like any other, so such ids must    */
/* not be used with Ysum); route_w fp32 [T][top_k] (required when Ysum is   */
/* given); Y fp32 [T][top_k][N]; Ysum fp32 [T][N] or NULL.                  */
/* ws: workspace of vq_grouped_workspace_bytes(E, T, top_k) bytes; after the */
/* call it holds, at offset 0, int32 counts[E], then int32 offsets[E+1],     */
/* then int32 list[T*top_k] (pair indices t*top_k+s grouped per expert in   */
/* ascending order), each section 256-byte aligned.                         */
/* Tiles: the pairs of each expert are cut into routed tiles whose height   */
/* comes from the mean rows per expert r = T*top_k/E ([P3] "routed-compact  */
/* J rule"): the smallest of 32, 64, 96 rows holding r + 3 sqrt(r), and 96 */
/* above that, so nearly every expert is one tile or a few (Q8_0: 96 rows). */
/* Numerics: routing and Ysum (of the Y written) are exact; the K-quant Y   */
/* meets the tolerance of vq_gemm and two identical calls are bitwise      */
/* equal; the Q8_0 Y is the fixed-order binary32 definition.               */
/* Limits: E <= 1024, top_k <= 16, N % 16 == 0.                              */
/* ---------------------------------------------------------------------- */
size_t vq_grouped_workspace_bytes(int64_t E, int64_t T, int64_t top_k);

vq_status vq_gemm_grouped(int w, const void* W, int64_t E, int64_t N, int64_t K, int act,
                          const void* Xq, int64_t T, const int32_t* ids, int64_t top_k,
                          const float* route_w, float* Y, float* Ysum, void* ws,
                          size_t ws_bytes, hipStream_t stream);

/* Per-row arm of the same operation ([P2] "kROCM keep-quant provider": the  */
/* grouped towers have a broadcast and a per-row arm), e.g. an MoE down     */
/* projection whose input differs per (token, slot):                       */
/*   Y[t][s][:] = W_(ids[t][s]) . x_(t*top_k+s)                              */
/* Xq holds T*top_k rows; every other argument, the workspace, limits and    */
/* errors are those of vq_gemm_grouped.                                     */
vq_status vq_gemm_grouped_rows(int w, const void* W, int64_t E, int64_t N, int64_t K, int act,
                               const void* Xq, int64_t T, const int32_t* ids, int64_t top_k,
                               const float* route_w, float* Y, float* Ysum, void* ws,
                               size_t ws_bytes, hipStream_t stream);

/* vq_gemm_grouped without the ws argument, for callers that cannot allocate */
/* device memory (code under HIP graph capture, tight serving loops,        */
/* harnesses that forbid hipMalloc).  The routing workspace comes from a    */
/* static device array of VQ_GROUPED_NOALLOC_SCRATCH_BYTES bytes, one per   */
/* GPU, held until the process ends; the call itself allocates nothing.    */
/* The caller still passes every input and output.  Outputs, limits and     */
/* errors are those of vq_gemm_grouped; a call whose routing workspace,     */
/* vq_grouped_workspace_bytes(E, T, top_k), exceeds the array (T*top_k of   */
/* about 410k pairs at E = 256) fails with VQ_ERR_WORKSPACE before any      */
/* launch.  Every call on one GPU uses that GPU's one array: calls that     */
/* overlap on one GPU (different streams, or threads without ordering)      */
/* race and must not be issued; calls ordered on one stream are fine.  The  */
/* current device must be the one the stream belongs to.                    */
#define VQ_GROUPED_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
vq_status vq_gemm_grouped_noalloc(int w, const void* W, int64_t E, int64_t N, int64_t K, int act,
                                  const void* Xq, int64_t T, const int32_t* ids, int64_t top_k,
                                  const float* route_w, float* Y, float* Ysum, hipStream_t stream);

/* Weighted expert sum alone (same definition as in vq_gemm_grouped):
 * Y fp32 [T][top_k][N], route_w fp32 [T][top_k], Ysum fp32 [T][N]; N % 4 == 0. */
vq_status vq_weighted_sum(const float* Y, const float* route_w, int64_t T, int64_t top_k,
                          int64_t N, float* Ysum, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Dispatch witness: launch counters per kernel variant since the last      */
/* reset (host-side, atomic).  Tests use them to prove which kernel ran.    */
/* ---------------------------------------------------------------------- */
typedef struct {
    uint64_t quantize_q8k;
    uint64_t quantize_q8_1;
    uint64_t quantize_weights;
    uint64_t gemv_q4k;
    uint64_t gemv_q6k;
    uint64_t gemv_q8_0;
    uint64_t gemm_q4k;
    uint64_t gemm_q6k;
    uint64_t gemm_q8_0;
    uint64_t route;
    uint64_t gemm_grouped_q4k;
    uint64_t weighted_sum;
    uint64_t gemm_grouped_q6k;
    uint64_t gemm_grouped_q8_0;
    uint64_t gemm_grouped_rows;  /* calls of the per-row arm (also counted per type) */
    uint64_t gemm_skinny;        /* vq_gemm calls with M <= 8 run on the GEMV kernel (also counted per type) */
    uint64_t gemv_q5k, gemm_q5k, gemm_grouped_q5k;  /* Q5_K calls of vq_gemv, vq_gemm, grouped calls */
    uint64_t rmsnorm_quant;      /* vq_rmsnorm_quant calls */
    uint64_t silu_mul_quant;     /* vq_silu_mul_quant calls */
} vq_stats;

void vq_get_stats(vq_stats* out);
void vq_reset_stats(void);

/* Library version string. */
const char* vq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VQ_H */
