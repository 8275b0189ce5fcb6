/*
 * attn.h -- C ABI of the exact fused attention library (libattn.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is exact scaled-dot-product attention
 *     O = softmax(scale * Q K^T) V
 * computed one tile at a time with an online softmax, so that the N x N
 * score matrix S and probability matrix P never reach device memory
 * ("13% more FLOPs, 5.7x faster: how FlashAttention's online softmax keeps
 * the NxN matrix out of HBM", sections "Softmax is the anti-tiling
 * operation" and "FlashAttention's move: rescale the output, too";
 * "FlashAttention" explainer, Steps 3-4 and "What is FlashAttention?").
 * The forward saves only O and one statistic per row, and the backward
 * rebuilds S and P from Q, K, V and that statistic (same blog post,
 * section "The backward pass: recompute instead of read").
 *
 * Conventions shared by every entry point
 *  - Tensors q, k, v, o, dO, dq, dk, dv are device pointers to contiguous
 *    row-major [B, H, N, d] arrays (d fastest): q, k, v, dO of element type
 *    `dtype`, o, dq, dk, dv of element type `out_dtype`.
 *    lse is a device pointer to a contiguous [B, H, N] float array.  Every
 *    pointer must be 16-byte aligned.
 *  - d is 64 or 128.  B, H, N >= 0; if any of them is 0 the call does
 *    nothing and returns ATTN_OK (pointers are then not examined).
 *    N * d must stay below 2^30 elements per head.
 *  - scale is any finite float (usually 1/sqrt(d)).  causal is 0 (every key
 *    visible) or 1 (query i sees keys 0..i; Q and K have the same length so
 *    the mask is the lower triangle).
 *  - The caller owns all memory.  The library allocates nothing, frees
 *    nothing and does not synchronise: work is enqueued on `stream` (a
 *    hipStream_t; NULL is the default stream) and the call returns once it
 *    is enqueued.  Outputs are overwritten entirely (never accumulated into)
 *    and must not overlap any input.
 *  - Arguments are validated before anything is enqueued: a negative
 *    status means nothing was launched and no output was touched, except
 *    ATTN_ERR_LAUNCH, which reports a failed kernel launch
 *    (hipGetLastError) after enqueueing.
 *  - There is no global mutable state apart from attn_bwd_noalloc's fixed
 *    per-GPU workspace (see there); every other call is thread-safe.
 */
#ifndef EXACT_ATTN_H
#define EXACT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  `dtype` (the inputs q, k, v, dO) is ATTN_F16 or ATTN_BF16.
 * `out_dtype` (the forward's o, which attn_bwd reads back, and the gradients
 * dq, dk, dv) is either the same as `dtype` or ATTN_F32.  Products are
 * accumulated in fp32 on the matrix cores; a 16-bit output is rounded once,
 * to nearest even, from the fp32 result an ATTN_F32 output would hold. */
typedef enum attn_dtype {
    ATTN_F16 = 0,  /* IEEE binary16 */
    ATTN_BF16 = 1, /* bfloat16 */
    ATTN_F32 = 2   /* IEEE binary32 (outputs only) */
} attn_dtype_t;

/* Status codes (0 = success). */
enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL = -1,      /* a required pointer is NULL */
    ATTN_ERR_SHAPE = -2,     /* B, H or N negative, or N*d too large */
    ATTN_ERR_HEAD_DIM = -3,  /* d is not 64 or 128 */
    ATTN_ERR_DTYPE = -4,     /* bad dtype, or out_dtype neither dtype nor ATTN_F32 */
    ATTN_ERR_ALIGN = -5,     /* a pointer is not 16-byte aligned */
    ATTN_ERR_WORKSPACE = -6, /* backward workspace missing or too small */
    ATTN_ERR_LAUNCH = -7,    /* the HIP runtime rejected a kernel launch */
    ATTN_ERR_SCALE = -8,     /* scale is NaN or infinite (or a bad descale factor) */
    ATTN_ERR_CAUSAL = -9,    /* causal is neither 0 nor 1 */
    ATTN_ERR_ALIAS = -10,    /* an output overlaps an input or another output */
    ATTN_ERR_SPLIT = -11,    /* nsplit outside 1 .. ATTN_MAX_SPLIT */
    ATTN_ERR_DROPOUT = -12   /* dropout_p not finite, negative, or round(256 p) > 255 */
};

/* Largest number of K/V chunks attn_fwd_split accepts. */
#define ATTN_MAX_SPLIT 64

/*
 * attn_fwd -- forward pass.
 *
 * For every (b, h) and query row i, with A(i) = {0..N-1}, or {0..i} when
 * causal:
 *     s_ij   = scale * q_i . k_j                    (j in A(i))
 *     o_i    = sum_j exp(s_ij - m_i) v_j / l_i
 *     lse_i  = m_i + ln(l_i)
 * where m_i = max_j s_ij and l_i = sum_j exp(s_ij - m_i): the running
 * maximum and normaliser of the online softmax ("Softmax is the anti-tiling
 * operation"), saved in logsumexp form as the per-row statistic the
 * backward needs ("The backward pass: recompute instead of read").
 *
 *   q, k, v : inputs, [B, H, N, d] of `dtype`
 *   o       : output, [B, H, N, d] of `out_dtype`
 *   lse     : output, [B, H, N] float (natural-log logsumexp of the scaled,
 *             masked scores of each row)
 *   stream  : hipStream_t to enqueue on
 * Returns ATTN_OK or a negative attn_status.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
             int dtype, int out_dtype, void* stream);

/*
 * attn_fwd_split_workspace_size -- bytes of device workspace attn_fwd_split
 * needs: nsplit partial outputs and partial lse, fp32,
 * nsplit * B * H * N * (d + 1) * 4.  Returns 0 when there is nothing to do
 * and for invalid arguments (attn_fwd_split validates them).
 */
size_t attn_fwd_split_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d, int nsplit);

/*
 * attn_fwd_split -- the forward pass with each query block's K/V tiles split
 * into nsplit chunks processed by separate workgroups (Flash-Decoding:
 * explainer "Common questions"), for shapes whose query blocks alone do not
 * fill the GPU.  Each chunk c yields, for every row, its own softmax over
 * the chunk's keys: a partial output O_c (normalised by the chunk's sum) and
 * a partial lse_c (-inf when the row sees no key of the chunk).  A second
 * kernel merges them with the rescale rule of the online softmax ("FlashAttention's
 * move: rescale the output, too") in logsumexp form:
 *     lse = log sum_c exp(lse_c),   o = sum_c exp(lse_c - lse) O_c.
 * The result is the same o and lse as attn_fwd up to rounding.
 *
 *   q, k, v, o, lse, B, H, N, d, scale, causal, dtype, out_dtype, stream :
 *             as for attn_fwd
 *   workspace, workspace_bytes : caller-owned device memory of at least
 *             attn_fwd_split_workspace_size(B, H, N, d, nsplit) bytes,
 *             16-byte aligned, overlapping no input or output; its contents
 *             on entry do not matter and on return are unspecified
 *   nsplit  : number of chunks, 1 .. ATTN_MAX_SPLIT (chunks past a query
 *             block's last tile are empty)
 * Returns ATTN_OK or a negative attn_status (ATTN_ERR_SPLIT for nsplit out
 * of range, ATTN_ERR_WORKSPACE for a missing or short workspace).
 */
int attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                   void* workspace, size_t workspace_bytes, int64_t B, int64_t H, int64_t N,
                   int64_t d, float scale, int causal, int dtype, int out_dtype, int nsplit,
                   void* stream);

/*
 * attn_fwd_decode -- the split K/V forward for Nq query rows against Nk keys
 * per head, the shape Flash-Decoding is for: a few new queries against a
 * long key/value cache, whose keys are split over many workgroups
 * (explainer "Common questions").  For every (b, h) and query row i, with
 * A(i) = {0..Nk-1}, or under the causal mask {0 .. i + Nk - Nq} (the queries
 * are the last Nq positions of the sequence; i's own key is Nk - Nq + i):
 *     o_i = sum_{j in A(i)} exp(s_ij - m_i) v_j / l_i,  lse_i = m_i + ln(l_i)
 * as for attn_fwd; a row with A(i) empty (causal, Nq > Nk) gets o_i = 0 and
 * lse_i = -inf.  With Nq = Nk this is attn_fwd_split.
 *
 *   q, o    : [B, H, Nq, d] (q of `dtype`, o of `out_dtype`)
 *   k, v    : [B, H, Nk, d] of `dtype`
 *   lse     : [B, H, Nq] float
 *   workspace, workspace_bytes : at least
 *             attn_fwd_split_workspace_size(B, H, Nq, d, nsplit) bytes,
 *             16-byte aligned, overlapping no input or output
 *   nsplit  : chunks of each query block's keys, 1 .. ATTN_MAX_SPLIT
 *   the rest: as for attn_fwd; Nq, Nk >= 0 (Nq = 0 does nothing),
 *             Nq * d and Nk * d below 2^30
 * Returns ATTN_OK or a negative attn_status.
 */
int attn_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                    void* workspace, size_t workspace_bytes, int64_t B, int64_t H, int64_t Nq,
                    int64_t Nk, int64_t d, float scale, int causal, int dtype, int out_dtype,
                    int nsplit, void* stream);

/*
 * attn_bwd_workspace_size -- bytes of device workspace attn_bwd needs for
 * these sizes (0 when there is nothing to do; otherwise a multiple of 256).
 * Returns 0 for invalid arguments as well; attn_bwd validates them.
 */
size_t attn_bwd_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d, int dtype);

/*
 * attn_bwd -- backward pass with recomputation.
 *
 * Gradients of L = sum(O * dO) with respect to q, k, v.  S and P are
 * recomputed tile by tile from q, k and the saved lse ("The backward pass:
 * recompute instead of read"; explainer Step 5 "IO Savings"):
 *     P_ij  = exp(s_ij - lse_i)  (0 for masked j)
 *     D_i   = dO_i . o_i
 *     dv_j  = sum_i P_ij dO_i
 *     dS_ij = P_ij (dO_i . v_j - D_i)
 *     dq_i  = scale * sum_j dS_ij k_j
 *     dk_j  = scale * sum_i dS_ij q_i
 *
 *   q, k, v   : the forward's inputs
 *   o, lse    : the forward's outputs (from attn_fwd with the same scale,
 *               causal flag and out_dtype); o is [B, H, N, d] of `out_dtype`
 *   dO        : upstream gradient, [B, H, N, d] of `dtype`
 *   dq, dk, dv: outputs, [B, H, N, d] of `out_dtype`
 *   workspace : device scratch of at least attn_bwd_workspace_size(...)
 *               bytes, 16-byte aligned; its contents on entry do not matter
 *               and are undefined on return
 * Returns ATTN_OK or a negative attn_status.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
             const float* lse, void* dq, void* dk, void* dv,
             void* workspace, size_t workspace_bytes,
             int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
             int dtype, int out_dtype, void* stream);

/*
 * attn_bwd_noalloc -- attn_bwd without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Arguments, results and
 * kernels are those of attn_bwd; the workspace is a fixed array the library
 * holds in every GPU's memory (ATTN_BWD_SCRATCH_BYTES, 16 MiB) until the
 * process ends, so the call allocates and frees nothing.
 *  - attn_bwd_workspace_size(B, H, N, d, dtype) must not exceed
 *    ATTN_BWD_SCRATCH_BYTES (B * H * ceil(N / 64) * 64 <= 2^21 rows), else
 *    ATTN_ERR_WORKSPACE and nothing is launched.
 *  - The array is looked up on the current device (hipGetDevice) at the
 *    first call there; `stream` must belong to that device.
 *  - Every call on one GPU uses the same array: calls that overlap in time
 *    on one GPU (on two streams, or from two threads without ordering) race
 *    and give wrong gradients.  Calls on one stream are ordered and safe.
 *    Nothing in the array needs clearing between calls: each call writes the
 *    rows it reads.
 */
#define ATTN_BWD_SCRATCH_BYTES (16u << 20)
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                     const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H,
                     int64_t N, int64_t d, float scale, int causal, int dtype, int out_dtype,
                     void* stream);

/*
 * attn_bwd_dq, attn_bwd_dkdv -- the two halves of attn_bwd, callable on
 * their own.  attn_bwd is exactly attn_bwd_dq followed by attn_bwd_dkdv on
 * the same stream with the same arguments.
 *
 * attn_bwd_dq computes dq and fills `workspace` with two values per query
 * row (-D_i, D_i = dO_i . o_i, and lse_i log2(e)); it reads q, k, v, o, dO, lse and
 * writes dq and the workspace.  attn_bwd_dkdv computes dk and dv; it reads
 * q, k, v, dO and a workspace filled by attn_bwd_dq for the same inputs,
 * sizes and flags (enqueued earlier on the same stream, or otherwise
 * complete), and writes dk and dv.  It does not read o or lse.  Argument
 * meanings, layouts and validation are those of attn_bwd; pointers a call
 * does not use may be NULL.
 */
int attn_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dO,
                const float* lse, void* dq, void* workspace, size_t workspace_bytes,
                int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                int dtype, int out_dtype, void* stream);
int attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                  void* dk, void* dv, const void* workspace, size_t workspace_bytes,
                  int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                  int dtype, int out_dtype, void* stream);

/*
 * attn_fwd_dropout, attn_bwd_dropout -- forward and backward with dropout on
 * the attention probabilities, fused into the kernels; the forward keeps only
 * the generator state (seed, offset), from which the backward regenerates
 * the same mask ("13% more FLOPs, 5.7x faster", section "The backward pass:
 * recompute instead of read"; explainer Step 3 "Tiling": matmul, mask,
 * softmax, dropout and matmul in one kernel).
 *
 * With t = floor(256 dropout_p + 1/2) (dropout_p is used as t / 256) and
 * r = 256 / (256 - t), for every (b, h), query row i and visible key j:
 *     keep_ij = [R_ij >= t]
 *     o_i     = sum_j keep_ij r exp(s_ij - m_i) / l_i  v_j
 *     lse_i   = m_i + ln(l_i)        (the undropped softmax's statistic)
 * where R_ij is byte (j mod 4) of output word floor((j mod 32) / 8) of
 * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
 * easy as 1, 2, 3", SC 2011) with key (seed mod 2^32, floor(seed / 2^32))
 * and counter (i, 2 floor(j / 32) + (floor(j / 4) mod 2), b H + h, offset).
 * The backward returns the gradients of L = sum(O * dO) through the dropped
 * weights W_ij = keep_ij r P_ij: dv_j = sum_i W_ij dO_i, and dS_ij =
 * P_ij (keep_ij r dO_i . v_j - D_i) with D_i = dO_i . o_i, dq and dk from dS
 * as in attn_bwd.  dropout_p = 0 gives the results of attn_fwd / attn_bwd.
 *
 *   dropout_p : probability of dropping an element: finite, >= 0, and
 *               floor(256 dropout_p + 1/2) <= 255
 *   seed      : generator key (64 bits)
 *   offset    : counter word distinguishing calls that share a seed
 *   the rest  : as for attn_fwd and attn_bwd; attn_bwd_dropout takes the o
 *               and lse of attn_fwd_dropout with the same dropout_p, seed,
 *               offset, scale, causal flag and out_dtype
 * Return ATTN_OK or a negative attn_status (ATTN_ERR_DROPOUT for a bad
 * dropout_p).
 */
int attn_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                     int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                     float dropout_p, uint64_t seed, uint32_t offset,
                     int dtype, int out_dtype, void* stream);
int attn_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dO,
                     const float* lse, void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes,
                     int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                     float dropout_p, uint64_t seed, uint32_t offset,
                     int dtype, int out_dtype, void* stream);

/*
 * attn_fwd_fp8 -- the forward with 8-bit inputs: q, k, v hold E4M3 codes
 * (the OCP 8-bit floating-point format: sign, 4 exponent bits with bias 7,
 * 3 mantissa bits, no infinity, largest value 448; one byte per element,
 * [B, H, N, d] as above), each tensor with one descale factor, so that code
 * x stands for decode(x) * descale.  The low-precision forward is the one the
 * pages name for FlashAttention-3 ("FlashAttention" explainer, "Common
 * questions" and its references); they fix no details, so the operation is
 * the exact attention of attn_fwd on those values, with scores
 * scale * q_descale * k_descale * (Q K^T) and o scaled by v_descale.  The
 * probabilities enter the P.V product rounded to nearest even E4M3 (each
 * within 2^-4 of its value, or 2^-10 of a row's largest below E4M3's normal
 * range); the row sums and lse use them in fp32.
 *
 *   q, k, v     : device pointers, E4M3 codes, [B, H, N, d], 16-byte aligned
 *   o, lse      : outputs as for attn_fwd, o of `out_dtype`
 *                 (ATTN_F16, ATTN_BF16 or ATTN_F32)
 *   d           : 128
 *   q_descale, k_descale, v_descale : finite and > 0
 *   the rest    : as for attn_fwd
 * Returns ATTN_OK or a negative attn_status (ATTN_ERR_HEAD_DIM for d != 128,
 * ATTN_ERR_SCALE for a descale factor that is not finite and positive, or a
 * score scale that overflows).
 */
int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                 int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                 float q_descale, float k_descale, float v_descale, int causal,
                 int out_dtype, void* stream);

/*
 * attn_fwd_decode_fp8 -- attn_fwd_decode with 8-bit inputs: Nq queries
 * against Nk keys per (batch, head) (causal query i sees keys 0 ..
 * i + Nk - Nq), each query block's keys split in nsplit chunks and merged,
 * with q, k, v as E4M3 codes and their descale factors as for attn_fwd_fp8
 * (a key/value cache held in 8 bits; q quantised by the caller).  The
 * chunks' partial outputs obey the same element-wise error statement as
 * attn_fwd_fp8, and the merge's exact weights keep it for the result.
 *
 *   q, o       : [B, H, Nq, d]; k, v : [B, H, Nk, d]; lse : [B, H, Nq]
 *   workspace  : attn_fwd_split_workspace_size(B, H, Nq, d, nsplit) bytes
 *   d          : 128; out_dtype : ATTN_F16, ATTN_BF16 or ATTN_F32
 *   the rest   : as for attn_fwd_decode and attn_fwd_fp8
 * Returns ATTN_OK or a negative attn_status.
 */
int attn_fwd_decode_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                        void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                        int64_t Nq, int64_t Nk, int64_t d, float scale, float q_descale,
                        float k_descale, float v_descale, int causal, int out_dtype, int nsplit,
                        void* stream);

/*
 * Materialised standard attention -- the unfused baseline the pages measure
 * the fused kernel against ("FlashAttention" explainer, Step 2 "Standard
 * Attention": S = Q K^T written to HBM, read back for P = softmax(S), P
 * written and read back for O = P V; "13% more FLOPs, 5.7x faster",
 * introduction).  Same result as attn_fwd up to rounding, but S and P are
 * real [B, H, N, N] arrays in device memory: 4 N^2 elements of traffic per
 * head beside the 4 N d of Q, K, V and O.  It exists to measure that
 * traffic; attn_fwd is the path to use.
 *
 * Conventions as above, plus: N <= ATTN_STD_MAX_N, and the caller provides
 * the N x N arrays.
 *   s : [B, H, N, N] float, s_ij = scale * q_i . k_j for every i, j (the mask
 *       is not applied to s)
 *   p : [B, H, N, N] of `dtype`, p_ij = exp(s_ij - m_i) / l_i over j in A(i),
 *       0 for masked j, normalised in fp32 and rounded once to nearest even
 *   lse : [B, H, N] float, m_i + ln(l_i), as attn_fwd writes it
 */
#define ATTN_STD_MAX_N 32768

/* Bytes of the workspace attn_std_fwd takes: s (fp32) and then p (`dtype`),
 * B * H * N * N * 6 (s rounded up to a multiple of 256 bytes).  0 for
 * invalid arguments or when there is nothing to do. */
size_t attn_std_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d, int dtype);

/* The three passes in order, with s and p in `workspace` (s at its start, p
 * after it); o and lse as for attn_fwd.  The workspace holds s and p
 * afterwards. */
int attn_std_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 void* workspace, size_t workspace_bytes, int64_t B, int64_t H, int64_t N,
                 int64_t d, float scale, int causal, int dtype, int out_dtype, void* stream);

/* Pass 1: s = scale * q k^T for every (i, j), fp32, on the matrix cores. */
int attn_std_scores(const void* q, const void* k, float* s, int64_t B, int64_t H, int64_t N,
                    int64_t d, float scale, int dtype, void* stream);

/* Pass 2: p and lse from s, row by row (the mask applied here). */
int attn_std_softmax(const float* s, void* p, float* lse, int64_t B, int64_t H, int64_t N,
                     int causal, int dtype, void* stream);

/* Pass 3: o = p v over every key, fp32 accumulation on the matrix cores,
 * o of `out_dtype` (`dtype` or ATTN_F32) rounded once. */
int attn_std_pv(const void* p, const void* v, void* o, int64_t B, int64_t H, int64_t N,
                int64_t d, int dtype, int out_dtype, void* stream);

/*
 * attn_probe_mfma -- a measurement aid, not part of the method: the rate the
 * matrix cores sustain on this device, against which the kernels'
 * utilisation is stated beside the published peak (the pages rate attention
 * kernels by the fraction of the hardware's peak they reach: "FlashAttention"
 * explainer, Step 6, "IO-optimal is not occupancy-optimal").  Launches
 * `workgroups` workgroups of 256 threads (four waves); every wave runs
 * `rounds` rounds of 16 v_mfma_f32_32x32x16_bf16 products (32768 FLOP each)
 * in four chains: in step s = 0..3 of a round, chain j multiplies A operand
 * j by B operand (j + s) mod 4, so consecutive products change operands.
 * Element e of lane l's A operand j holds the bf16 bits h(64 (8 j + e) + l),
 * of B operand j h(64 (8 (j + 4) + e) + l), where h(x) mixes x with the
 * MurmurHash3 finaliser and keeps bit 15 (sign), bits 0..6 (mantissa) and
 * bit 8 as the exponent's low bit (exponent 126 or 127): values of either
 * sign in [0.5, 2), as random as attention's operands.  Every thread stores
 * the sum of its 64 accumulators to out[workgroup * 256 + thread].  The
 * caller times the launch (e.g. with HIP events): FLOP per launch =
 * workgroups * 4 * 16 * rounds * 32768.
 *   out        : device float array of workgroups * 256 elements (written)
 *   workgroups : 1 .. 2^20 (two per compute unit fill the device)
 *   rounds     : 1 .. 2^24
 * Returns ATTN_OK, ATTN_ERR_SHAPE, ATTN_ERR_NULL, ATTN_ERR_ALIGN or
 * ATTN_ERR_LAUNCH.
 */
int attn_probe_mfma(float* out, int64_t workgroups, int64_t rounds, void* stream);

/*
 * attn_probe_hbm -- a measurement aid, not part of the method: the rate at
 * which this device streams a buffer from HBM, against which memory-bound
 * kernels (the decode step reads its key/value cache once) are stated beside
 * the published 8 TB/s (the pages measure such kernels by the bytes they
 * move: "13% more FLOPs, 5.7x faster", "The takeaway that outlives the
 * kernel").  Launches `workgroups` workgroups of 256 threads (four waves).
 * `buf` is cut into 1 KiB chunks (chunk c = bytes 1024 c .. 1024 c + 1023);
 * workgroup b takes chunks b C .. min((b + 1) C, chunks) - 1, C =
 * ceil(chunks / workgroups), and its wave w the chunks w, w + 4, w + 8, ...
 * of that range, copied into LDS with the kernels' non-temporal
 * direct-to-LDS copy, eight in flight.  Thread 64 (4 b + w) + l stores to
 * out[256 b + 64 w + l] the sum, modulo 2^32, of the four 32-bit words at
 * bytes 1024 c + 16 l of every chunk c its wave copied (bytes past the end
 * of `buf` count as 0).  Every byte of `buf` is read once; the caller times
 * the launch.
 *   buf        : device buffer, 16-byte aligned, `bytes` long (read only)
 *   bytes      : 16 .. 2^42, a multiple of 16
 *   out        : device array of workgroups * 256 unsigned ints (written),
 *                16-byte aligned, not overlapping buf
 *   workgroups : 1 .. 2^20
 * Returns ATTN_OK, ATTN_ERR_SHAPE, ATTN_ERR_NULL, ATTN_ERR_ALIGN,
 * ATTN_ERR_ALIAS or ATTN_ERR_LAUNCH.
 */
int attn_probe_hbm(const void* buf, int64_t bytes, unsigned* out, int64_t workgroups, void* stream);

/* attn_status_str -- static, human-readable name of a status code. */
const char* attn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTN_H */
