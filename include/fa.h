/*
 * fa.h — C ABI of the MI355X (gfx950) exact tiled attention library (libfa.so).
 *
 * Computes exact scaled-dot-product attention
 *
 *     O = softmax(Q K^T * scale + mask) V,     LSE = log(sum_j exp(S_ij))
 *
 * tile by tile with the online-softmax recurrence (running row max m, running
 * sum of exponentials l, rescale of the accumulated output by exp(m_old - m_new)),
 * so the Nq x Nk score and probability matrices never reach device memory.
 *   - The operation: "Flash Attention Optimization", section "Attention is not
 *     slow because of arithmetic" (S = QK^T/sqrt(d), P = softmax(S), O = PV), and
 *     "Explain FlashAttention. Why is it called IO-aware, and what does it actually
 *     save?", section "Keep only the state needed for the final weighted average"
 *     (scale, then mask, then softmax; running state m, l, o).
 *   - The recurrence and why it is exact: "FlashAttention: Attention Is Limited by
 *     Memory, Not Math", section "How tiling and online softmax stay exact".
 *   - Split-KV decode with a merge of partial (m, l, o) states: same page, section
 *     "Where it helps, and where it does not" (Flash-Decoding), with the two-sided
 *     merge of "Flash Attention Optimization", section "The fix: tile the
 *     computation, never materialize the full matrix".
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller. The library
 *     never allocates, frees or synchronises; it launches asynchronously on
 *     `stream` (a hipStream_t; NULL = the default stream) and returns.
 *   - Layout: contiguous row-major [B][H][N][d] (d innermost) for q, k, v and o;
 *     [B][H][Nq] for lse. q, k, v and o must be 16-byte aligned.
 *   - q, k, v hold FA_BF16 (bfloat16) or FA_F32 (IEEE float32) elements; o and
 *     lse are always float32.
 *   - Causal masking uses absolute positions ("Explain FlashAttention ...",
 *     section "Executable recurrence, with an empty-state policy": masks use global
 *     positions, not tile-local ones). `causal` = 1 aligns the query block to the
 *     END of the key sequence: query i (0-based) sits at position i + (Nk - Nq) and
 *     sees key j iff j <= i + (Nk - Nq). `causal` = 2 aligns it to the START: query i
 *     sees key j iff j <= i. For Nq == Nk both are j <= i; 0 means no mask.
 *   - A query row that sees no key (only possible when causal = 1 and Nq > Nk) gets
 *     O = 0 and LSE = -inf (the empty-row policy of the same section).
 *   - LSE is the natural-log log-sum-exp of the scaled, masked scores of the row.
 *   - Arguments are validated before any HIP call; a rejected call launches
 *     nothing and writes nothing. There is no silent fallback: unsupported
 *     shapes return FA_ERR_UNSUPPORTED. NaN/Inf in q, k or v is outside the
 *     contract (not scanned for).
 *   - Stateless and thread-safe.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,         /* a required pointer is NULL                          */
  FA_ERR_SHAPE = -2,        /* a size is < 1, or sizes overflow the index range    */
  FA_ERR_UNSUPPORTED = -3,  /* valid but not implemented: head dim, dtype, size    */
  FA_ERR_WORKSPACE = -4,    /* workspace NULL or smaller than required             */
  FA_ERR_HIP = -5,          /* the HIP runtime reported an error at launch         */
  FA_ERR_VALUE = -6,        /* scale not finite and > 0, causal not 0/1/2, ...     */
  FA_ERR_ALIGN = -7         /* a tensor pointer or bias stride is not aligned      */
} fa_status;

typedef enum { FA_BF16 = 0, FA_F32 = 1 } fa_dtype;

/*
 * fa_fwd — attention forward (prefill): every query row of every (b, h).
 *   q   [B][H][Nq][d]  dtype          k, v [B][H][Nk][d]  dtype
 *   o   [B][H][Nq][d]  float32 (written)
 *   lse [B][H][Nq]     float32 (written) or NULL to skip it
 *   d in {64, 128}; B, H, Nq, Nk >= 1 (ragged sizes allowed); Nk * d <= 2^30.
 *   scale: finite and > 0 (1/sqrt(d) for standard attention).
 *   causal: 0, 1 (bottom-right) or 2 (top-left).
 * bf16 inputs use bf16 MFMA with float32 accumulation; float32 inputs use
 * float32 MFMA and never round to a narrower type.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, float* o, float* lse,
                 int B, int H, int Nq, int Nk, int d, float scale, int causal,
                 fa_dtype dtype, void* stream);

/*
 * fa_fwd_bias — fa_fwd with an additive bias on the scaled scores ("Explain
 * FlashAttention ...", section "Keep only the state needed for the final weighted average":
 * the scores are scaled, then the intended mask or bias is added, then the softmax):
 *     S[b][h][i][j] = scale * q_i . k_j + bias[b*stride_b + h*stride_h + i*stride_q + j]
 *   bias: dtype elements (bfloat16 or float32, like q, k, v), keys contiguous; strides in
 *   elements, each >= 0 (0 repeats the same values along that dimension, e.g. one [Nq][Nk]
 *   bias for every (b, h), or a [B][Nk] key-padding bias with stride_h = stride_q = 0).
 *   The bias is not multiplied by scale. A key hidden by the causal mask stays hidden
 *   whatever its bias; a bias of -inf hides a key (a row whose keys are all hidden gets
 *   O = 0 and LSE = -inf); +inf and NaN are outside the contract. LSE is that of the
 *   scaled, biased, masked scores.
 *   FA_BF16: the bias pointer must be 16-byte aligned and the three strides multiples of
 *   8; each bias row is read in 16-byte pieces, so its first Nk elements rounded up to a
 *   multiple of 8 must be readable (pad the key dimension of the allocation to a multiple
 *   of 8). The bias of rows and keys that are masked may be read but never matters.
 *   FA_F32: 4-byte alignment; only the first Nk elements of each row are read.
 *   stride_q * 64 < 2^31. Other arguments, sizes and errors as in fa_fwd.
 */
fa_status fa_fwd_bias(const void* q, const void* k, const void* v, const void* bias,
                      long long bias_stride_b, long long bias_stride_h, long long bias_stride_q,
                      float* o, float* lse, int B, int H, int Nq, int Nk, int d, float scale,
                      int causal, fa_dtype dtype, void* stream);

/*
 * fa_fwd_fp8 — fa_fwd with 8-bit floating-point inputs on the FP8 matrix cores ("FlashAttention:
 * Attention Is Limited by Memory, Not Math", section "FlashAttention 1, 2 and 3": FP8 is one
 * of FlashAttention-3's additions).
 *   q [B][H][Nq][d], k, v [B][H][Nk][d]: OCP E4M3 bytes (1 sign, 4 exponent bits with bias
 *   7, 3 mantissa bits, no infinities); the real inputs are q * q_descale, k * k_descale,
 *   v * v_descale (finite, > 0).
 *   o [B][H][Nq][d] float32; lse [B][H][Nq] float32 or NULL.
 *   d = 128; scale, causal and the empty-row policy as in fa_fwd.
 * Scores are float32 (the q.k products and their sums are exact up to float32 rounding);
 * the probabilities enter the second product as E4M3(256 * exp(s - m)), rounded to nearest
 * even with the row's largest weight exact; the normaliser sums the float32 weights.
 */
fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, float* o, float* lse,
                     int B, int H, int Nq, int Nk, int d, float scale, float q_descale,
                     float k_descale, float v_descale, int causal, void* stream);

/*
 * fa_fwd_varlen — fa_fwd over a packed batch of variable-length sequences (no padding).
 *   q [total_q][H][d], k, v [total_k][H][d]  FA_BF16     o [total_q][H][d] float32
 *   lse [H][total_q] float32 or NULL
 *   cu_seqlens_q, cu_seqlens_k [B+1] int32 (device): sequence b owns query rows
 *   cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key rows cu_seqlens_k[b] ..
 *   cu_seqlens_k[b+1]-1; both start at 0, never decrease and end at total_q / total_k.
 *   A sequence's queries see only its own keys; the causal mask uses positions inside the
 *   sequence, aligned as in fa_fwd (causal = 1: query i of nq sees key j of nk iff
 *   j <= i + nk - nq; causal = 2: iff j <= i); a row that sees no key gets O = 0 and
 *   LSE = -inf.
 *   max_seqlen_q: an upper bound on every sequence's query count (rows past it are not
 *   computed). Offsets outside [0, total] are clamped on the device, so malformed ones
 *   cannot read or write outside the tensors.
 *   d in {64, 128}; H*d*256 < 2^31; scale finite and > 0; causal 0, 1 or 2. The
 *   cu_seqlens arrays need 4-byte alignment, the tensors 16-byte.
 */
fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, float* o, float* lse,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int H,
                        int total_q, int total_k, int max_seqlen_q, int d, float scale,
                        int causal, fa_dtype dtype, void* stream);

/*
 * fa_decode_workspace_bytes — bytes of device workspace fa_decode_splitkv needs:
 * B*H*num_splits*(d+2)*4. Returns 0 if an argument is < 1 or the size overflows.
 */
size_t fa_decode_workspace_bytes(int B, int H, int d, int num_splits);

/*
 * fa_decode_splitkv — one query per (b, h) against a long key/value cache
 * (Flash-Decoding). The Nk keys are cut into num_splits chunks of
 * C = ceil(Nk / num_splits) keys (trailing chunks may be short or empty); one
 * pass computes each chunk's partial state (m, l, o) relative to the chunk's own
 * max, and a second pass merges the partials in fixed order (deterministic).
 *   q [B][H][1][d]  dtype        k, v [B][H][Nk][d]  dtype
 *   o [B][H][1][d]  float32      lse [B][H][1] float32 or NULL
 *   workspace: device memory of at least fa_decode_workspace_bytes(B, H, d,
 *   num_splits) bytes, 16-byte aligned, owned by the caller; its contents on
 *   entry are ignored and on return are unspecified. Not causal (a single query
 *   at the end of the sequence sees every key).
 *   d = 128 (FA_BF16 or FA_F32) or d = 64; 1 <= num_splits <= 1024; Nk >= 1.
 */
fa_status fa_decode_splitkv(const void* q, const void* k, const void* v, float* o, float* lse,
                            int B, int H, int Nk, int d, float scale, int num_splits,
                            void* workspace, size_t workspace_bytes, fa_dtype dtype,
                            void* stream);

/*
 * fa_decode_splitkv_noalloc — fa_decode_splitkv for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels, with the partial states kept in a fixed array that the
 * library holds on every GPU it runs on (FA_NOALLOC_SCRATCH_BYTES bytes per GPU, held until
 * the process ends) instead of in a caller's workspace. The call allocates nothing; the
 * caller still owns q, k, v, o and lse. Arguments, results and errors as in
 * fa_decode_splitkv, plus:
 *   - FA_ERR_WORKSPACE when fa_decode_workspace_bytes(B, H, d, num_splits) exceeds
 *     FA_NOALLOC_SCRATCH_BYTES (at d = 128: when B*H*num_splits > 64,527);
 *   - FA_ERR_HIP when the array's address cannot be obtained on the stream's device.
 * The array is looked up on the stream's device (the current device for the null stream)
 * at the first call there. All calls on one GPU share its array: calls that overlap in
 * time on one GPU (on different streams, or from threads without ordering) race on it and
 * must not be issued; calls ordered on one stream are safe. Nothing in the array needs to
 * start at zero (every partial state a call reads, it wrote).
 */
#define FA_NOALLOC_SCRATCH_BYTES (32u << 20)
fa_status fa_decode_splitkv_noalloc(const void* q, const void* k, const void* v, float* o,
                                    float* lse, int B, int H, int Nk, int d, float scale,
                                    int num_splits, fa_dtype dtype, void* stream);

/*
 * fa_decode_paged — fa_decode_splitkv over a paged key/value cache with per-sequence
 * lengths: the page indirection that serving engines pair with split-KV decoding
 * ("FlashAttention: Attention Is Limited by Memory, Not Math", section "Where it helps,
 * and where it does not").
 *   q        [B][H][1][d]                         dtype
 *   k_cache, v_cache [num_pages][page_size][H][d] dtype  (a shared pool of pages)
 *   block_table [B][max_pages_per_seq] int32 (device): key t of sequence b is row
 *            t % page_size of page block_table[b][t / page_size].
 *   seq_lens [B] int32 (device): keys of sequence b (clamped to [0, max_pages_per_seq *
 *            page_size]); the single query sees all of them (it sits at the end).
 *   o [B][H][1][d] float32, lse [B][H][1] float32 or NULL. A sequence with no key gets
 *   O = 0 and LSE = -inf.
 *   Each sequence's keys are cut into num_splits chunks of ceil(seq_lens[b] / num_splits);
 *   partials merge as in fa_decode_splitkv (same workspace size:
 *   fa_decode_workspace_bytes(B, H, d, num_splits)).
 *   page_size: a power of two; num_pages, max_pages_per_seq >= 1. A block-table entry
 *   outside [0, num_pages) is never read through: the keys it would hold are skipped.
 *   block_table and seq_lens need 4-byte alignment, the other pointers 16-byte.
 *   d in {64, 128}; FA_BF16 or FA_F32; 1 <= num_splits <= 1024.
 */
fa_status fa_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                          const int* block_table, const int* seq_lens, float* o, float* lse,
                          int B, int H, int d, int page_size, int num_pages, int max_pages_per_seq,
                          float scale, int num_splits, void* workspace, size_t workspace_bytes,
                          fa_dtype dtype, void* stream);

/*
 * fa_bwd_workspace_bytes — bytes of device workspace fa_bwd needs:
 * B*H*ceil(Nq/128)*128*8 (two float32 statistics per query row, rows padded to a whole
 * number of 128-row tiles). Returns 0 if an argument is < 1 or the size overflows.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int Nq);

/*
 * fa_bwd — attention backward: the gradients of a loss L with respect to q, k and v, given
 * do = dL/dO and the o and lse that fa_fwd returned for the same q, k, v, scale and causal.
 * The probabilities are recomputed tile by tile from lse rather than stored ("Flash
 * Attention Optimization", section "Sizing a tile, and why the backward pass recomputes
 * instead of storing"; "Explain FlashAttention ...", section "Exact attention, finite
 * precision and backward"); with P = softmax(S) as in fa_fwd, the chain rule gives
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(dO * O)),
 *   dQ = scale dS K,  dK = scale dS^T Q        (masked pairs contribute nothing).
 *   q, do [B][H][Nq][d]  dtype         k, v [B][H][Nk][d]  dtype
 *   o     [B][H][Nq][d]  float32       lse  [B][H][Nq] float32 (as written by fa_fwd;
 *                                      a row with LSE = -inf contributes nothing)
 *   dq    [B][H][Nq][d]  float32, dk, dv [B][H][Nk][d] float32 (written; every element)
 *   workspace: device memory of at least fa_bwd_workspace_bytes(B, H, Nq) bytes, 16-byte
 *   aligned, owned by the caller; contents on entry are ignored, on return unspecified.
 *   dtype: FA_BF16 or FA_F32 (q, k, v and do share it). d in {64, 128}; B, H, Nq, Nk >= 1;
 *   Nq * d, Nk * d <= 2^30. scale finite and > 0; causal 0, 1 or 2 (the alignments of
 *   fa_fwd). lse only needs 4-byte alignment. Three kernels run in order on `stream`;
 *   every output element is written exactly once (deterministic, no atomics). FA_BF16: P
 *   and dS are rounded to bfloat16 as MFMA operands, everything else is float32. FA_F32:
 *   float32 MFMA throughout, nothing is rounded below float32.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const float* o, const float* lse,
                 const void* dout, float* dq, float* dk, float* dv, int B, int H, int Nq, int Nk,
                 int d, float scale, int causal, void* workspace, size_t workspace_bytes,
                 fa_dtype dtype, void* stream);

/*
 * fa_bwd_varlen — fa_bwd for a packed batch of variable-length sequences: the gradients of
 * a loss L with respect to q, k and v, given do = dL/dO and the o and lse that
 * fa_fwd_varlen returned for the same inputs, offsets, scale and causal. Sequences share
 * no scores, so each sequence's gradients are those of fa_bwd on its own rows ("Explain
 * FlashAttention ...", section "Exact attention, finite precision and backward": the
 * backward covers the masks and awkward dimensions the forward supports).
 *   q, do [total_q][H][d]  FA_BF16     k, v [total_k][H][d]  FA_BF16
 *   o     [total_q][H][d]  float32     lse  [H][total_q] float32 (as fa_fwd_varlen writes it)
 *   dq    [total_q][H][d]  float32, dk, dv [total_k][H][d] float32 (written; every row of a
 *   sequence within the caps below, zero where a row attends to nothing or is attended by
 *   nothing)
 *   cu_seqlens_q, cu_seqlens_k [B+1] int32 (device), causal 0, 1 or 2: as in fa_fwd_varlen.
 *   max_seqlen_q, max_seqlen_k: upper bounds on every sequence's query and key counts (rows
 *   past them are neither read nor written). Offsets outside [0, total] are clamped on the
 *   device, so malformed ones cannot read or write outside the tensors.
 *   workspace: at least fa_bwd_workspace_bytes(B, H, max_seqlen_q) bytes, 16-byte aligned,
 *   owned by the caller; contents on entry are ignored, on return unspecified.
 *   d in {64, 128}; H*d*256 < 2^31; scale finite and > 0. FA_F32 returns
 *   FA_ERR_UNSUPPORTED. Three kernels on `stream`, every output element written once, as in
 *   fa_bwd (deterministic).
 */
fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const float* o,
                        const float* lse, const void* dout, float* dq, float* dk, float* dv,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int H,
                        int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int d,
                        float scale, int causal, void* workspace, size_t workspace_bytes,
                        fa_dtype dtype, void* stream);

/*
 * fa_bwd_bias — fa_bwd for the attention of fa_fwd_bias (S = scale * Q K^T + bias): the
 * gradients with respect to q, k and v of a loss L, given do = dL/dO and the o and lse
 * that fa_fwd_bias returned for the same q, k, v, bias, scale and causal; optionally also
 * the gradient with respect to a full bias. The bias enters each score with weight 1, so
 * dL/dbias_ij = dS_ij = P_ij (dP_ij - rowsum(dO * O)_i) ("Explain FlashAttention ...",
 * section "Exact attention, finite precision and backward": the backward covers the masks
 * and biases the forward supports).
 *   bias, bias_stride_b/h/q: as in fa_fwd_bias (FA_BF16 rules: 16-byte aligned, strides
 *   multiples of 8, each row readable to its first Nk elements rounded up to 8);
 *   bias_stride_q * 128 < 2^31.
 *   dbias: NULL, or float32 [B][H][Nq][Nk] (16-byte aligned), written in full: dS for every
 *   (query, key) pair, 0 where the mask or a -inf bias hides the pair. It is the gradient of
 *   a full bias; the gradient of a bias that is shared along some dimensions (a stride of 0)
 *   is its sum over those dimensions, which the caller forms.
 *   Other arguments, layouts, workspace and errors as in fa_bwd; dtype FA_BF16 only
 *   (FA_F32 returns FA_ERR_UNSUPPORTED).
 */
fa_status fa_bwd_bias(const void* q, const void* k, const void* v, const void* bias,
                      long long bias_stride_b, long long bias_stride_h, long long bias_stride_q,
                      const float* o, const float* lse, const void* dout, float* dq, float* dk,
                      float* dv, float* dbias, int B, int H, int Nq, int Nk, int d, float scale,
                      int causal, void* workspace, size_t workspace_bytes, fa_dtype dtype,
                      void* stream);

/*
 * fa_probe_mfma — measurement aid, not part of the attention method: launches `blocks`
 * workgroups of 256 threads in which every wave issues 4 * iters back-to-back
 * v_mfma_f32_32x32x16_bf16 (32768 FLOP each) on register operands, with no memory traffic,
 * and writes one float per thread to `sink` (device memory of at least blocks * 1024 bytes,
 * 4-byte aligned; its values are meaningless). Timing the launch gives the practical
 * dense bf16 MFMA rate of the device at its current clock, the context for the attention
 * kernels' own rate. Errors: FA_ERR_NULL, FA_ERR_SHAPE (blocks or iters < 1),
 * FA_ERR_WORKSPACE (sink too small), FA_ERR_ALIGN, FA_ERR_HIP.
 */
fa_status fa_probe_mfma(float* sink, size_t sink_bytes, int blocks, int iters, void* stream);

/* fa_status_str — static English description of a status code (never NULL). */
const char* fa_status_str(fa_status s);

/*
 * fa_last_hip_error — the hipError_t (as int) behind the most recent FA_ERR_HIP returned
 * on the calling thread; 0 (hipSuccess) if there was none. fa_last_hip_error_str gives
 * the HIP runtime's name for it (never NULL).
 */
int fa_last_hip_error(void);
const char* fa_last_hip_error_str(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
