/*
 * parallax.h - C ABI of libparallax: the MI355X (gfx950) Parallax attention
 * (decode, causal prefill, chunked prefill, the prefill backward) and the
 * fused q, k, v, rho projection that feeds it.
 *
 * Parallax ("Parallax: Parameterized Local Linear Attention for Language
 * Modeling", paper page, "Abstract"; explainer blog "Parallax: Breaking the
 * Boundary Bias with Parameterized Local Linear Attention", section "The Core
 * Insight: Covariance Correction", output equation) computes, for each query,
 * softmax attention minus the key/value covariance applied to a learned
 * per-head probe rho:
 *
 *     w_i   = softmax_i(scale * q . k_i)
 *     mu_v  = sum_i w_i v_i,   mu_k = sum_i w_i k_i
 *     S_KV  = sum_i w_i (v_i - mu_v)(k_i - mu_k)^T      (value rows, key columns)
 *     out   = mu_v - S_KV rho
 *
 * The blog's "Hardware Efficiency" section describes a decode kernel that
 * fuses the softmax and covariance branches into one pass over the KV stream;
 * these entry points do that on CDNA4. Readings of points the pages leave
 * open: rho is in key space and is not multiplied by `scale`; the covariance
 * is centred at the softmax-weighted means and uses the softmax weights
 * (summing to one); GQA groups are contiguous (query head h reads KV head
 * h / (H_q / H_kv)); a query that sees no key outputs zeros.
 *
 * Conventions shared by every call:
 *  - Tensor pointers are DEVICE pointers to dense row-major arrays (last
 *    dimension contiguous) on the current HIP device; they must be 16-byte
 *    aligned. The caller owns every buffer; the library never allocates or
 *    frees memory, never synchronises, and keeps no mutable global state
 *    besides a lazily filled, thread-safe cache of per-device compute-unit
 *    counts and the per-device scratch of parallax_decode_noalloc.
 *  - Inputs are read only. Outputs are written in full (every element), except
 *    the K/V caches of parallax_qkvr_projection, of which only the projected
 *    rows are written.
 *  - `dtype` is the storage type of q, rho, K and V (bf16 or fp32; fp32 for
 *    decode only); all accumulation is fp32 and attention outputs and
 *    gradients are fp32.
 *  - `seq_lens` is a device int32 array [B]. Its values cannot be checked on
 *    the host without a synchronisation, so kernels clamp them to [0, S_max]
 *    (for prefill, rows t >= seq_lens[b] are written as zeros). Keys at or past
 *    a sequence's length are never read into the result (NaN padding there is
 *    harmless).
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL means the null
 *    stream). Every argument check happens on the host before any launch: on
 *    an error status nothing has been launched and no buffer was touched.
 *    Launch failures return PARALLAX_ERR_HIP. No call throws.
 *  - Supported: head dim d in {64, 128}; any integral G = H_q / H_kv (up
 *    to 4 query heads, or up to 8 when G > 4, share one pass over their KV
 *    head; G > 8 re-reads K and V once per further group of 8); each
 *    (b, h_kv) slice of K or V must be smaller than 2 GiB.
 */
#ifndef PARALLAX_H
#define PARALLAX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PARALLAX_ABI_VERSION 7

typedef enum {
  PARALLAX_OK = 0,
  PARALLAX_ERR_NULL_POINTER = 1, /* a required pointer is NULL */
  PARALLAX_ERR_BAD_SHAPE = 2,    /* a size <= 0, H_q % H_kv != 0, T > S_max, scale not finite, ... */
  PARALLAX_ERR_UNSUPPORTED = 3,  /* d, G, dtype or size outside what is built */
  PARALLAX_ERR_MISALIGNED = 4,   /* a tensor pointer is not 16-byte aligned */
  PARALLAX_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than required */
  PARALLAX_ERR_HIP = 6,          /* a HIP runtime call or kernel launch failed */
  PARALLAX_ERR_TOO_LARGE = 7     /* beyond the built-in scratch of parallax_decode_noalloc */
} parallax_status_t;

typedef enum {
  PARALLAX_BF16 = 0,
  PARALLAX_F32 = 1,
  /* not dtypes: they give the type the range of int, so that any int a
     caller passes is a value of it (and is refused as unsupported) */
  PARALLAX_DTYPE_RANGE_MIN_ = -0x7fffffff - 1,
  PARALLAX_DTYPE_RANGE_MAX_ = 0x7fffffff
} parallax_dtype_t;

/* PARALLAX_ABI_VERSION of the built library. */
int parallax_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* parallax_status_string(parallax_status_t s);

/*
 * Split-KV plan for decode (passage: the single pass over the KV stream of
 * the blog "Parallax: Breaking the Boundary Bias with Parameterized Local
 * Linear Attention", "Hardware Efficiency: Faster than Flash?"; the split
 * and its merge are this library's). Each (b, KV head, group of <= 4 query
 * heads, or <= 8 when the KV head serves more than 4) is cut into
 * `num_splits` contiguous key ranges of `chunk` keys (a multiple of 128),
 * processed by separate workgroups whose partial softmax states are merged
 * by the combine step. `requested` = 0 picks a plan from the device's
 * compute-unit count (about one workgroup per compute unit; a workgroup
 * has 8 waves for bf16 at d = 64, whose rows are half as long, else 4);
 * a positive
 * value asks for that many splits (rounded so that chunk is a multiple of
 * 128). Writes the plan to *num_splits and *chunk (either may be NULL).
 * Returns PARALLAX_ERR_BAD_SHAPE for sizes <= 0 or H_q % H_kv != 0,
 * PARALLAX_ERR_UNSUPPORTED for d not in {64, 128} or S_max > INT_MAX - 128,
 * PARALLAX_ERR_HIP if the device cannot be queried.
 */
parallax_status_t parallax_decode_plan(int B, int H_q, int H_kv, int d, int S_max,
                                       int requested, int* num_splits, int* chunk);

/*
 * Workspace bytes needed by parallax_decode / parallax_decode_partial for the
 * plan `num_splits` (as returned by parallax_decode_plan): one fp32 record of
 * (2 d + 4) values (running max, weight sum, probe sum, probe reference, and
 * two d-vectors) per (b, h_q, split), followed by B * H_q 32-bit arrival
 * counters (rounded up to 16 bytes). 0 if num_splits == 1 (the kernel then
 * finalises directly), on a bad shape, or when the workspace would reach
 * 2^62 bytes (every call refuses such a plan with PARALLAX_ERR_UNSUPPORTED).
 *
 * The counters are used by parallax_decode only. They must be zero before the
 * first parallax_decode call on a workspace (allocate it zeroed, or clear the
 * whole workspace once); every call returns them to zero. Calls that share a
 * workspace must be ordered (same stream or synchronised): overlapping calls
 * on one workspace race.
 */
size_t parallax_decode_workspace_size(int B, int H_q, int d, int num_splits);

/*
 * Decode: one new query per (b, h_q) against the first seq_lens[b] cached keys.
 *   q, rho    [B, H_q, d]          dtype
 *   k_cache   [B, H_kv, S_max, d]  dtype
 *   v_cache   [B, H_kv, S_max, d]  dtype
 *   seq_lens  [B]                  int32 (device)
 *   out       [B, H_q, d]          fp32, written in full
 *   scale     softmax scale applied to q . k only (never to rho . k); any finite
 *             value (negative and zero included)
 *   num_splits 0 = automatic plan, else the requested split count
 *   workspace  device scratch of at least parallax_decode_workspace_size()
 *              bytes for the resolved plan (may be NULL when that is 0)
 * One kernel launch: each workgroup streams its key range once; with several
 * splits, the last workgroup to finish for each (b, KV head, group of query
 * heads) merges the partial states (same result as parallax_decode_partial
 * followed by parallax_decode_combine, up to rounding). With several splits
 * the workspace's counters must be zero on entry (see
 * parallax_decode_workspace_size); they are zero again on exit.
 * Passage: the output equation of the blog "Parallax: Breaking the Boundary
 * Bias with Parameterized Local Linear Attention", "The Core Insight:
 * Covariance Correction" (out = mu_v - S_KV rho), with rho the per-token
 * learned probe of the paper page "Parallax: Parameterized Local Linear
 * Attention for Language Modeling", "Abstract", computed in the single pass
 * over the KV stream of the blog's "Hardware Efficiency: Faster than Flash?"
 * (streaming form: out = (A (1 + Bs / l) - C) / l over l = sum w, A = sum w v,
 * Bs = sum w r, C = sum w r v, r = rho . k, softmax weights w).
 * Errors: PARALLAX_ERR_NULL_POINTER (q, rho, a cache, seq_lens or out NULL);
 * PARALLAX_ERR_BAD_SHAPE (a size <= 0, H_q % H_kv != 0, num_splits < 0, scale
 * not finite); PARALLAX_ERR_UNSUPPORTED (d not in {64, 128}, dtype not bf16
 * or fp32, B > 65535, a (b, h_kv) slice or one sequence's [H_q, d] queries
 * of 2 GiB or more, more than 65535 splits, a workspace of 2^62 bytes or
 * more); PARALLAX_ERR_MISALIGNED (a tensor or the workspace not 16-byte
 * aligned, seq_lens not 4-byte aligned); PARALLAX_ERR_WORKSPACE (workspace
 * NULL or smaller than parallax_decode_workspace_size for the plan);
 * PARALLAX_ERR_HIP (device query or launch failed).
 */
parallax_status_t parallax_decode(const void* q, const void* rho, const void* k_cache,
                                  const void* v_cache, const int32_t* seq_lens, float* out,
                                  int B, int H_q, int H_kv, int d, int S_max, float scale,
                                  parallax_dtype_t dtype, int num_splits, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Bytes of the scratch array parallax_decode_noalloc keeps on each device,
 * and the part of it that holds the arrival counters. */
#define PARALLAX_NOALLOC_SCRATCH_BYTES (32u << 20)
#define PARALLAX_NOALLOC_COUNTER_BYTES (256u << 10)

/*
 * Allocation-free decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): parallax_decode (same arguments, checks, result and single
 * fused launch, minus the workspace) with the partial records and arrival
 * counters in a scratch array the library holds on each device it runs on,
 * from the library's load until the process ends:
 * PARALLAX_NOALLOC_SCRATCH_BYTES (32 MiB), of which
 * PARALLAX_NOALLOC_COUNTER_BYTES (256 KiB) hold the counters.
 *  - Limit: the resolved plan's records, B * H_q * num_splits * (2 d + 4) * 4
 *    bytes, within the scratch past the counters (33,292,288 bytes; this
 *    also keeps B * H_q within the 65,536 counters). Beyond it,
 *    PARALLAX_ERR_TOO_LARGE and nothing is launched. A one-split plan (no
 *    records, no counters) has no limit and does not touch the scratch.
 *  - The first call on a device (that device current) looks up the array's
 *    address and clears its counters with a small kernel on `stream`; every
 *    call returns them to zero.
 *  - Every call on one device shares that device's array: calls that
 *    overlap on a device (different streams without ordering, or several
 *    host threads) race and give wrong results. Order them.
 *  - Nothing is allocated: no hipMalloc, hipFree or allocating library call.
 */
parallax_status_t parallax_decode_noalloc(const void* q, const void* rho, const void* k_cache,
                                          const void* v_cache, const int32_t* seq_lens,
                                          float* out, int B, int H_q, int H_kv, int d, int S_max,
                                          float scale, parallax_dtype_t dtype, int num_splits,
                                          void* stream);

/*
 * First phase of decode: streams every valid K/V row once and writes one
 * partial state per (b, h_q, split) to `workspace` (or, when the resolved
 * plan has one split, finalises straight into `out`, which may otherwise be
 * NULL). Arguments, passage and errors as parallax_decode (out may be NULL
 * unless the plan has one split). Does not use the workspace counters.
 * Record of (b, h_q, split) (fp32, 2 d + 4 values): running max m of the
 * scaled scores (log2 units), l, Bs and the probe reference c of the
 * streaming form (Bs and C relative to c), then A and C, each a d-vector
 * relative to the weights 2^(s - m).
 */
parallax_status_t parallax_decode_partial(const void* q, const void* rho, const void* k_cache,
                                          const void* v_cache, const int32_t* seq_lens,
                                          float* out, int B, int H_q, int H_kv, int d,
                                          int S_max, float scale, parallax_dtype_t dtype,
                                          int num_splits, void* workspace,
                                          size_t workspace_bytes, void* stream);

/*
 * Second phase of decode: merges the partial states written by
 * parallax_decode_partial with the same (B, H_q, H_kv, d, S_max, num_splits)
 * and writes out [B, H_q, d] fp32. Splits that start at or past seq_lens[b]
 * are skipped (never read). A no-op returning PARALLAX_OK when the resolved
 * plan has one split. Passage as parallax_decode: the merge rescales each
 * record to the common max and moves it to the common probe reference
 * (Bs -> Bs + (c_s - c) l_s, C -> C + (c_s - c) A_s, exact) before the
 * streaming form's final step.
 * Errors: PARALLAX_ERR_NULL_POINTER (seq_lens or out NULL);
 * PARALLAX_ERR_BAD_SHAPE and PARALLAX_ERR_UNSUPPORTED as parallax_decode for
 * the sizes and d; PARALLAX_ERR_MISALIGNED (out or the workspace not 16-byte
 * aligned); PARALLAX_ERR_WORKSPACE (workspace NULL or too small);
 * PARALLAX_ERR_HIP.
 */
parallax_status_t parallax_decode_combine(const int32_t* seq_lens, float* out, int B, int H_q,
                                          int H_kv, int d, int S_max, int num_splits,
                                          const void* workspace, size_t workspace_bytes,
                                          void* stream);

/*
 * Causal prefill: query row t of sequence b sees keys 0..t (no past offset).
 *   q, rho    [B, H_q, T, d]       dtype (rho is per token)
 *   k, v      [B, H_kv, S_max, d]  dtype, T <= S_max
 *   seq_lens  [B]                  int32 (device); rows t >= seq_lens[b] -> 0
 *   out       [B, H_q, T, d]       fp32, written in full
 * Needs no workspace. Only dtype PARALLAX_BF16 is built for prefill.
 * Passage: the output equation of the blog "Parallax: Breaking the Boundary
 * Bias with Parameterized Local Linear Attention", "The Core Insight:
 * Covariance Correction", for every query row of a causal sequence, with the
 * per-token probe of the paper page "Parallax: Parameterized Local Linear
 * Attention for Language Modeling", "Abstract" (the pages' pretraining
 * setting), computed per row in the streaming form given for
 * parallax_decode.
 * Precision: the softmax weights w and the products w (r - c) enter the
 * value contraction rounded once to fp16 (toward zero, with l and Bs summed
 * from the same rounded values) and V is staged as fp16, exact for bf16
 * values of magnitude 2^-14 .. 65504; smaller magnitudes lose low bits (fp16
 * subnormals) and larger ones are not representable. Measured per-row error
 * against an fp64 evaluation: a few 1e-4 at unit-scale inputs, up to about
 * 1.3e-3 with probes 20 times stronger and a sharp softmax.
 * Errors: PARALLAX_ERR_NULL_POINTER (any pointer NULL); PARALLAX_ERR_BAD_SHAPE
 * (a size <= 0, H_q % H_kv != 0, T > S_max, scale not finite);
 * PARALLAX_ERR_UNSUPPORTED (dtype not bf16, d not in {64, 128}, B or H_q
 * above 65535, a (b, h_kv) slice or a (b, h_q) block of 2 GiB or more);
 * PARALLAX_ERR_MISALIGNED (a tensor not 16-byte aligned, seq_lens not 4-byte
 * aligned); PARALLAX_ERR_HIP (launch failed).
 */
parallax_status_t parallax_prefill(const void* q, const void* rho, const void* k,
                                   const void* v, const int32_t* seq_lens, float* out, int B,
                                   int H_q, int H_kv, int d, int T, int S_max, float scale,
                                   parallax_dtype_t dtype, void* stream);

/*
 * Chunked causal prefill against an existing cache (also multi-token decode):
 * row t of sequence b sits at position past_lens[b] + t and sees keys
 * 0 .. past_lens[b] + t of the cache. The cache must already hold the
 * chunk's own keys and values at positions past_lens[b] .. past_lens[b] +
 * chunk_lens[b] - 1 (append first, then attend). With every past length 0 this
 * is parallax_prefill.
 *   q, rho      [B, H_q, T, d]       dtype (rho is per token)
 *   k_cache,
 *   v_cache     [B, H_kv, S_max, d]  dtype, T <= S_max
 *   past_lens   [B]                  int32 (device), clamped to [0, S_max]
 *   chunk_lens  [B]                  int32 (device), valid rows of the chunk,
 *                                    clamped to [0, min(T, S_max - past)];
 *                                    rows t >= chunk_lens[b] are written as 0
 *   out         [B, H_q, T, d]       fp32, written in full
 * Only dtype PARALLAX_BF16 is built. Passage and precision as
 * parallax_prefill, with the chunk's rows placed after the cached tokens
 * (the causal reading of continuing a sequence). Chunks of at most 256 rows
 * split each row block's keys into 4 ranges (up to 64 rows) or 2 ranges
 * whose partial states are merged exactly (rescaled to a common max and moved
 * to a common probe reference).
 * Errors as parallax_prefill, plus PARALLAX_ERR_NULL_POINTER for a NULL
 * past_lens and PARALLAX_ERR_MISALIGNED for a past_lens not 4-byte aligned.
 */
parallax_status_t parallax_prefill_chunked(const void* q, const void* rho, const void* k_cache,
                                           const void* v_cache, const int32_t* past_lens,
                                           const int32_t* chunk_lens, float* out, int B, int H_q,
                                           int H_kv, int d, int T, int S_max, float scale,
                                           parallax_dtype_t dtype, void* stream);

/*
 * Multi-token decode: the result of parallax_prefill_chunked (same arguments,
 * layouts and clamping of past_lens and chunk_lens), computed by the split-KV
 * decode kernel for the few new tokens per sequence of speculative decoding.
 * Each (query head, token) pair is one decode query: token t of sequence b
 * attends keys 0 .. past_lens[b] + t, rows t >= chunk_lens[b] are written as
 * 0, and every KV head is streamed once per group of 8 (query head, token)
 * pairs (of 4 when there are at most 4). Passage: the same as
 * parallax_decode (one pass over the KV stream, [blog] "Hardware
 * Efficiency"), with the causal reading of the chunk.
 * Choice against parallax_prefill_chunked: each further group of 8 pairs
 * reads K and V again, so this call wins for short chunks only. At 8
 * sequences of 4096 keys, 16 query heads on 8 KV heads and d = 128, it took
 * 29, 47 and 77 us for 4, 8 and 16 new tokens, against 92 us for the chunked
 * prefill; at 32 tokens it took 148 us against 97 us.
 *   dtype       PARALLAX_BF16 or PARALLAX_F32
 *   num_splits, workspace, workspace_bytes as parallax_decode, for
 *               H_q * T queries: the plan is parallax_decode_plan(B, H_q * T,
 *               H_kv, d, S_max, num_splits) and the size
 *               parallax_decode_workspace_size(B, H_q * T, d, num_splits);
 *               the same zeroed-counter rule applies.
 * Errors as parallax_decode (any number (H_q / H_kv) * T of (head, token)
 * pairs per KV head is supported), plus
 * PARALLAX_ERR_NULL_POINTER for a NULL past_lens or chunk_lens and
 * PARALLAX_ERR_BAD_SHAPE for T <= 0 or T > S_max.
 */
parallax_status_t parallax_decode_tokens(const void* q, const void* rho, const void* k_cache,
                                         const void* v_cache, const int32_t* past_lens,
                                         const int32_t* chunk_lens, float* out, int B, int H_q,
                                         int H_kv, int d, int T, int S_max, float scale,
                                         parallax_dtype_t dtype, int num_splits,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* Causal prefill for training: parallax_prefill plus what the backward
 * needs. Besides `out` it writes
 *   mu_v   [B, H_q, T, d] fp32: the softmax-attention part sum_j w_j v_j;
 *   stats  [B, H_q, T, 4] fp32: per row (log2 of sum_j 2^(scale log2(e) q.k_j),
 *          c = rho . k_0, rbar - c, 0), where rbar = sum_j w_j rho . k_j.
 * Rows t >= seq_lens[b] get zeros in all three. The gradients are those of
 * the output of the blog "Parallax: Breaking the Boundary Bias with
 * Parameterized Local Linear Attention", "The Core Insight: Covariance
 * Correction", output equation, with the learned probe of the paper page
 * "Parallax: Parameterized Local Linear Attention for Language Modeling",
 * "Abstract". Arguments, errors and semantics otherwise as parallax_prefill;
 * mu_v and stats must be 16-byte aligned device pointers. */
parallax_status_t parallax_prefill_train(const void* q, const void* rho, const void* k,
                                         const void* v, const int32_t* seq_lens, float* out,
                                         float* mu_v, float* stats, int B, int H_q, int H_kv,
                                         int d, int T, int S_max, float scale,
                                         parallax_dtype_t dtype, void* stream);

/* Bytes of workspace parallax_prefill_backward needs: dO split into bf16
 * high and low parts (2 x B H_q T d x 2 bytes) and two floats per row,
 * rounded to 16 bytes; 0 for a shape parallax_prefill_backward refuses
 * (sizes <= 0, d not in {64, 128}, B or H_q above 65535, T + 256 of 2^22
 * rows or more at d = 128, 2^23 at d = 64). */
size_t parallax_prefill_backward_workspace_size(int B, int H_q, int T, int d);

/* Gradients of the causal prefill output for an upstream gradient
 * dout [B, H_q, T, d] fp32, from the inputs of parallax_prefill_train and its
 * out, mu_v and stats:
 *   dq, drho  [B, H_q, T, d] fp32 (rows t >= seq_lens[b] are 0);
 *   dk, dv    [B, H_kv, S_max, d] fp32, summed over the H_q / H_kv query heads
 *             of each KV head (keys j >= seq_lens[b] are 0).
 * Every output is written in full. Rows of dout at or past seq_lens[b] are
 * ignored. `workspace` (device, 16-byte aligned, caller-owned, at least
 * parallax_prefill_backward_workspace_size bytes) is scratch: the first
 * launch writes its entries for rows below seq_lens[b] and the second reads
 * them. Two launches on `stream`, asynchronous; nothing is allocated. Errors as
 * parallax_prefill, plus PARALLAX_ERR_WORKSPACE for a short workspace; on an
 * error nothing is launched. Deterministic: no atomics, fixed reduction
 * order. */
parallax_status_t parallax_prefill_backward(
    const void* q, const void* rho, const void* k, const void* v, const int32_t* seq_lens,
    const float* out, const float* mu_v, const float* stats, const float* dout, float* dq,
    float* drho, float* dk, float* dv, int B, int H_q, int H_kv, int d, int T, int S_max,
    float scale, parallax_dtype_t dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Fused projection of the layer input into q, k, v and the probe rho (the
 * probe is a learned projection of the input: blog "Parallax: Breaking the
 * Boundary Bias with Parameterized Local Linear Attention", "The Core
 * Insight: Covariance Correction" and "Architecture-Optimizer Codesign", the
 * W_R projection; paper page "Parallax: Parameterized Local Linear Attention
 * for Language Modeling", "Abstract").
 *   x        [B, T, d_model] bf16, row b T + t (device)
 *   w        [(2 H_q + 2 H_kv) d, d_model] bf16: the rows of W_Q (H_q d),
 *            W_K (H_kv d), W_V (H_kv d) and W_R (H_q d), each output
 *            feature's weights contiguous (device)
 *   q, rho   [B, H_q, T, d] bf16 outputs (device)
 *   k_cache, v_cache  [B, H_kv, S_max, d] bf16 (device): row past_lens[b] + t
 *            of sequence b receives token t (rows at or past S_max are not
 *            written); other rows are left as they are
 *   past_lens [B] device int32 or NULL (all 0), clamped to [0, S_max]
 * Each output is the fp32-accumulated dot product rounded to bf16 (nearest
 * even). d_model must be a positive multiple of 64; d in {64, 128};
 * T <= S_max; all tensor pointers 16-byte aligned. Host checks precede the
 * single launch on `stream`; nothing is allocated. Errors: NULL_POINTER,
 * BAD_SHAPE (non-positive sizes, T > S_max, d_model not a multiple of 64),
 * UNSUPPORTED (d not 64/128, sizes past 32-bit offsets), MISALIGNED, HIP. */
parallax_status_t parallax_qkvr_projection(const void* x, const void* w, void* q, void* rho,
                                           void* k_cache, void* v_cache,
                                           const int32_t* past_lens, int B, int T, int d_model,
                                           int H_q, int H_kv, int d, int S_max, void* stream);

/* Measurement support, not part of the method: a plain streaming read that
 * serves as the reference for the decode kernel's KV-stream bandwidth. It
 * reads every 16-byte word of a[0 .. bytes_each) and b[0 .. bytes_each)
 * exactly once (non-temporal loads, about two workgroups per compute unit,
 * each streaming one contiguous share) and XORs every 32-bit word of both
 * into the sink, one workgroup's XOR into word (workgroup mod sink_words):
 *   a, b        device buffers, 16-byte aligned, read only
 *   bytes_each  a positive multiple of 16
 *   sink        device uint32 array of sink_words words; the XOR of all its
 *               words changes by the XOR of the data (clear it first to get
 *               the XOR of the data alone)
 *   sink_words  positive; at least twice the compute-unit count keeps the
 *               workgroups' atomics on distinct words
 * One launch on `stream`, nothing allocated. Errors: NULL_POINTER,
 * BAD_SHAPE (bytes_each not a positive multiple of 16, sink_words <= 0),
 * MISALIGNED, HIP. */
parallax_status_t parallax_read_probe(const void* a, const void* b, size_t bytes_each,
                                      uint32_t* sink, int sink_words, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PARALLAX_H */
