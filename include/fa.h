/*
 * fa.h -- C ABI of the MI355X (gfx950) fused exact-attention library.
 *
 * The library computes exact attention,
 *
 *     O = softmax(scale * Q K^T + mask) V
 *
 * ("Vanilla Attention", displayed equation, mrodiduger.github.io page; the
 * scale and mask are caller parameters), with the IO-aware method the pages
 * describe: inputs are tiled into on-chip blocks, the softmax is formed
 * online with a running row maximum and normaliser, and only O and one
 * log-sum-exp per row are written back to HBM (interviewsvector.com page,
 * "Architecture, step by step", steps 1-4; chipfoundryservices.com page,
 * "FlashAttention Key Insight").  The backward recomputes the scores and
 * probabilities from the stored statistics ("Recomputation",
 * mrodiduger.github.io page) and returns dQ, dK and dV.  Masking and dropout
 * are fused into both passes (same page, "Vanilla Attention" and
 * "Experimental Results").
 *
 * Conventions shared by every entry point:
 *   - Tensors are contiguous [B, H, N, d] in the element type `dtype`
 *     (row-major, d fastest); lse and the backward's row statistics are
 *     contiguous [B, H, N] float32 (natural logarithm).
 *   - Every pointer argument is a DEVICE pointer, allocated and owned by the
 *     caller; it must be 16-byte aligned.  Outputs must not alias inputs.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream)
 *     and the call returns without synchronising.  The library never
 *     allocates device memory; the backward's scratch is the caller's
 *     `workspace`.
 *   - Arguments are validated before any HIP call: FA_EINVAL for a bad value
 *     or pointer, FA_EUNSUPPORTED for a well-formed request the library does
 *     not implement.  FA_EHIP reports a failed launch; faults of enqueued work
 *     surface at the caller's next synchronisation.  fa_last_error() returns
 *     a message for the calling thread's last non-OK status.
 *   - Calls are stateless and reentrant; concurrent calls on different
 *     streams are independent.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
    FA_OK = 0,
    FA_EINVAL = 1,        /* invalid argument (null/misaligned pointer, bad size or value) */
    FA_EUNSUPPORTED = 2,  /* valid but not implemented (head dim, dtype) */
    FA_EHIP = 3           /* a HIP launch or runtime call failed */
} fa_status_t;

typedef enum fa_dtype {
    FA_F32 = 0,           /* float32 inputs, fp32 matrix-core products */
    FA_BF16 = 1,          /* bfloat16 inputs, fp32 accumulation */
    FA_F16 = 2,           /* float16 inputs, fp32 accumulation */
    FA_FP8_E4M3 = 3       /* OCP e4m3 inputs with per-head descale factors (fa_fwd_fp8 only) */
} fa_dtype_t;

/*
 * Problem description (64 bytes, no implicit padding).
 *   B, H, N, d : batch, heads, sequence length, head dimension.  B, H, N >= 0
 *                (a zero extent is an empty problem: FA_OK, nothing
 *                launched); N < 2^31; d in {32, 64, 96, 128} for every
 *                dtype and also 256 for FA_BF16 / FA_F16 (other values:
 *                FA_EUNSUPPORTED).  16-bit inputs run the tuned kernels at
 *                every head dimension; fp32 inputs run the generic ones.
 *   dtype      : fa_dtype_t of q, k, v (and dout in the backward).
 *   causal     : 0 or 1.  With 1, key j is masked for query i when j > i
 *                (the diagonal is kept); masked probabilities are exactly 0.
 *   scale      : finite and > 0; scores are scale * q.k (callers usually
 *                pass 1/sqrt(d)).
 *   dropout_p  : 0 <= p < 1.  Inverted dropout on the normalised
 *                probabilities: kept entries are multiplied by
 *                c = (float)(1/(1-p)); the row statistics are not affected.
 *                The keep bit of (b, h, row, col) is lane (col & 7) of the
 *                Philox-4x32-10 block (Salmon et al., SC'11) with counter
 *                (col >> 3, row, h, b) and key (seed low 32, seed high 32);
 *                lane 2w is the low and lane 2w+1 the high half of output
 *                word w; kept iff lane >= round(p * 65536).  A p > 0 that
 *                rounds to a zero threshold (p < 2^-17) is FA_EUNSUPPORTED.
 *   seed       : dropout seed (ignored when dropout_p == 0).
 *   out_f32    : 0 -> outputs (o, dq, dk, dv) in `dtype`; 1 -> float32.
 *   Nk         : keys (and values) per head for the forward; 0 means N
 *                (self-attention).  With Nk != N the queries are the last N
 *                positions of a sequence of Nk keys (decoding) or attend to
 *                another sequence (cross attention): when causal, key j is
 *                visible to query i iff j <= i + (Nk - N), so the last query
 *                sees every key; a query with no visible key gets O = 0 and
 *                LSE = -inf.  Dropout counters use the query's own row i.
 *                The backward takes the same Nk: dk, dv are [B,H,Nk,d].
 *                One head of any operand (q, k, v, o, dout or an output)
 *                must stay below 2 GiB (else FA_EUNSUPPORTED): the kernels
 *                address a head with signed 32-bit byte offsets.
 */
typedef struct fa_params {
    int64_t B, H, N, d;
    int32_t dtype;
    int32_t causal;
    float scale;
    float dropout_p;
    uint64_t seed;
    int32_t out_f32;
    int32_t Nk;           /* keys per head; 0 = N */
} fa_params_t;

/*
 * Forward.  Reads q [B,H,N,d] and k, v [B,H,Nk,d]; writes o [B,H,N,d]
 * (dtype, or float32 with out_f32) and lse [B,H,N] float32 with
 * lse_i = ln sum_j exp(s_ij) over the visible keys of row i.  Nothing else
 * is written to device memory.
 */
fa_status_t fa_fwd(const fa_params_t *p, const void *q, const void *k, const void *v,
                   void *o, float *lse, void *stream);

/*
 * Forward with FP8 inputs (the FP8 precision of the "FlashAttention-3
 * (2024)" section of the chipfoundryservices.com page).  q, k, v are
 * [B,H,N,d] / [B,H,Nk,d] OCP e4m3 bytes (1 sign, 4 exponent bits with bias
 * 7, 3 mantissa bits; no infinities) with p->dtype = FA_FP8_E4M3; the
 * attention inputs are q * descale_q[b*H + h] (and k, v likewise):
 * descale_q, descale_k, descale_v are device arrays of B*H positive finite
 * float32 factors.  Writes o [B,H,N,d] (bfloat16, or float32 with out_f32)
 * and lse [B,H,N] float32 as fa_fwd does for the dequantized inputs.  Both
 * products run on the FP8 matrix cores with fp32 accumulation; the
 * probabilities enter the second product rounded to e4m3 (after scaling by
 * 2^6), while the row sums and lse use them unrounded, so
 *     |o - o_exact| <= (2^-4 + n 2^-16) max_j |v_j| (+ output rounding)
 * per element, n the number of keys the row sees.  d = 128 only and
 * dropout_p = 0 only (else FA_EUNSUPPORTED); causal, Nk and out_f32 as in
 * fa_fwd.
 */
fa_status_t fa_fwd_fp8(const fa_params_t *p, const void *q, const void *k, const void *v,
                       const float *descale_q, const float *descale_k, const float *descale_v,
                       void *o, float *lse, void *stream);

/*
 * Forward with the keys of every (b, h, block of query rows) split into up
 * to num_splits contiguous chunks (of a multiple of 64 keys) processed by
 * separate workgroups, for problems with few query rows (decoding, short
 * queries over long keys) that would otherwise leave most of the GPU idle:
 * the parallelism across the sequence dimension of the "FlashAttention-2
 * Improvements" section of the chipfoundryservices.com page, applied to the
 * keys.  Each chunk writes its O,
 * normalised over its own keys, and its log-sum-exp to `workspace` (fp32);
 * a second kernel merges them per row with the online-softmax rescaling
 * (LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s).  Same
 * arguments and results as fa_fwd (up to fp32 rounding order).
 * 1 <= num_splits <= 256 (else FA_EINVAL).  `workspace` must hold
 * fa_fwd_splitkv_workspace_bytes(p, num_splits) bytes (0 when fewer than
 * two chunks result: then the plain forward runs and workspace may be
 * NULL); its contents on entry are ignored.
 */
size_t fa_fwd_splitkv_workspace_bytes(const fa_params_t *p, int32_t num_splits);
fa_status_t fa_fwd_splitkv(const fa_params_t *p, const void *q, const void *k, const void *v,
                           void *o, float *lse, int32_t num_splits, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace fa_bwd needs for `p` (0 for an empty problem,
 * (size_t)-1 for invalid parameters): two fp32 arrays of B*H*N row
 * statistics (see fa_bwd_prepare), each rounded up to 256 bytes.
 */
size_t fa_bwd_workspace_bytes(const fa_params_t *p);

/*
 * Backward.  Reads q and dout [B,H,N,d], k and v [B,H,Nk,d] in dtype, o
 * (the forward's output, in the forward's output type: dtype, or float32
 * when out_f32) and lse (from fa_fwd); writes dq [B,H,N,d] and dk, dv
 * [B,H,Nk,d] (dtype, or float32 with out_f32).  `workspace` must hold at least
 * fa_bwd_workspace_bytes(p) bytes; its contents on entry are ignored.  The
 * same p (scale, causal, dropout_p, seed) as the forward must be passed.
 */
fa_status_t fa_bwd(const fa_params_t *p, const void *q, const void *k, const void *v,
                   const void *o, const float *lse, const void *dout,
                   void *dq, void *dk, void *dv, void *workspace, size_t workspace_bytes,
                   void *stream);

/*
 * The backward as three stages, in the order fa_bwd enqueues them (all on
 * one stream; later stages read the D_i the first one leaves in
 * `workspace`):
 *   fa_bwd_prepare  per query row i, in fp32 into the workspace: D_i / c
 *                   (D_i = dO_i . O_i, c = 1/(1-dropout_p), 1 without
 *                   dropout) and -lse_i log2(e); the later stages fold c
 *                   into their outputs;
 *   fa_bwd_dkdv     recomputes S and P tile by tile per key block and writes
 *                   dK and dV;
 *   fa_bwd_dq       recomputes S and P tile by tile per query block and
 *                   writes dQ (no atomics: results are deterministic).
 * Arguments mean the same as in fa_bwd; each stage validates its own.
 */
fa_status_t fa_bwd_prepare(const fa_params_t *p, const void *o, const float *lse, const void *dout,
                           void *workspace, size_t workspace_bytes, void *stream);
fa_status_t fa_bwd_dkdv(const fa_params_t *p, const void *q, const void *k, const void *v,
                        const float *lse, const void *dout, void *dk, void *dv,
                        const void *workspace, size_t workspace_bytes, void *stream);
fa_status_t fa_bwd_dq(const fa_params_t *p, const void *q, const void *k, const void *v,
                      const float *lse, const void *dout, void *dq, const void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * The backward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, kernels and results as fa_bwd, but the row statistics
 * live in a static device array of fa_bwd_noalloc_max_workspace_bytes()
 * bytes (32 MiB: B*H*N <= 4,194,304 query rows), one copy per device, held
 * until the process ends.  The array's device address is looked up on the
 * first call on each device (with that device current); no call allocates
 * or frees memory.  A larger problem is refused with FA_EINVAL (use fa_bwd
 * with a workspace).  Every call on a device shares that device's array,
 * so calls that overlap on one device (other streams, other threads) race;
 * nothing in it needs clearing between calls.
 */
size_t fa_bwd_noalloc_max_workspace_bytes(void);
fa_status_t fa_bwd_noalloc(const fa_params_t *p, const void *q, const void *k, const void *v,
                           const void *o, const float *lse, const void *dout,
                           void *dq, void *dk, void *dv, void *stream);

/*
 * Test hook: writes the dropout keep mask of plane (b, h) -- mask[row*N +
 * col] = 1 when kept, 0 when dropped -- using the same device generator as
 * the attention kernels.  Only B, H, N, dropout_p and seed of p are read
 * (d and dtype are not checked).  mask is an N*N byte device buffer.
 */
fa_status_t fa_dropout_mask(const fa_params_t *p, int64_t b, int64_t h, uint8_t *mask,
                            void *stream);

/*
 * Test hook (host only, no HIP call): the order in which the kernels take
 * their work units.  A kernel's grid has one workgroup per unit, BH heads
 * times nb blocks per head; workgroup u is dispatched to XCD u % 8, and
 * unit_of (fa_kernels.hpp) assigns it the head bh[u] and the block rank
 * rank[u] (rank 0 = the longest block of a causal head), so that each XCD
 * works through a contiguous range of an order that takes the heads in
 * groups of `group` and, within a group, blocks rank by rank.  bh and rank
 * are host arrays of BH * nb entries.  FA_EINVAL for BH, nb or group < 1 or
 * BH * nb or group * nb >= 2^31.
 */
fa_status_t fa_unit_order(int64_t BH, int64_t nb, int32_t group, uint32_t *bh, uint32_t *rank);

/* Static description of a status code. */
const char *fa_status_str(fa_status_t s);

/* Message for the calling thread's most recent non-OK status ("" if none). */
const char *fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
