/*
 * Exact scaled-dot-product attention for AMD Instinct MI355X (gfx950): C ABI.
 *
 * Computes O = softmax(scale * Q K^T) V block by block with the online-softmax
 * statistics (running max m, denominator l, un-normalised output u, rescaled by
 * exp(m - m') when a block raises the max, output u / l), so the score matrix is
 * never written to device memory. Definitions: auturnal.com transformer-attention
 * guide (v10), section 2 (the formula) and section 8 (the blockwise statistics);
 * marketmaker.cc "Flash Attention und die Frage nach der Sequenzlaenge", sections
 * on the algorithm, the online-softmax recurrence and causal masking.
 *
 * Conventions shared by every entry point:
 *  - Layout. Q and O are [B, H_q, N_q, d]; K and V are [B, H_kv, N_kv, d]; all
 *    contiguous row-major, all of one element type `dtype` (O has the input
 *    type). LSE, when requested, is float32 [B, H_q, N_q] in natural log
 *    (lse = m + ln l). Tensors are [batch, heads, seq, head_dim] as in the
 *    papanda925.com survey's standard-attention pseudo-code.
 *  - Grouped-query attention: H_q must be a multiple of H_kv; query head h reads
 *    KV head h / (H_q / H_kv) (code-journey.com attention co-design summary,
 *    "Group Size(G)": G query heads share one KV head).
 *  - Causal masking uses bottom-right alignment: query i sees key j iff
 *    j <= i + (n - N_q), n being the number of valid keys. For N_q == n this is
 *    j <= i; a single decode query sees every valid key. Key blocks entirely in
 *    a query block's future are skipped.
 *  - Rows with no visible key produce O = 0 and LSE = -inf.
 *  - Memory. All pointers are device pointers owned by the caller. The library
 *    never allocates, frees or synchronises: it enqueues work on `stream` (a
 *    hipStream_t; NULL is the default stream) and returns. Inputs are read only.
 *    O and LSE must not overlap any input.
 *  - Errors. Arguments are checked before anything is enqueued; on a nonzero
 *    status nothing was enqueued, except ATTN_ERR_LAUNCH (the HIP launch
 *    itself failed). There is no fallback path: inputs the kernels do not
 *    cover are rejected with ATTN_ERR_UNSUPPORTED.
 *  - Supported: dtype ATTN_F32, ATTN_F16, ATTN_BF16 (decode: F16 and BF16);
 *    d in {64, 128}; gfx950 devices only.
 */
#ifndef EXACT_ATTENTION_ATTN_H_
#define EXACT_ATTENTION_ATTN_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ATTN_F32 = 0, ATTN_F16 = 1, ATTN_BF16 = 2 } attn_dtype_t;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,       /* negative or inconsistent sizes, or sizes beyond the grid limits */
  ATTN_ERR_GQA = 3,         /* H_q is not a positive multiple of H_kv */
  ATTN_ERR_UNSUPPORTED = 4, /* dtype, head dim, N_q or device not covered by the kernels */
  ATTN_ERR_WORKSPACE = 5,   /* decode workspace missing or smaller than required */
  ATTN_ERR_LAUNCH = 6,      /* the HIP launch reported an error */
  ATTN_ERR_NO_DEVICE = 7,   /* no HIP device is visible */
  ATTN_ERR_ALIAS = 8,       /* an output overlaps an input */
  ATTN_ERR_VALUE = 9        /* scale not positive and finite, or causal not 0 or 1 */
} attn_status_t;

/*
 * Prefill (and general) forward: every query row of Q attends to the N_kv keys.
 *   q [B,H_q,N_q,d], k/v [B,H_kv,N_kv,d], o [B,H_q,N_q,d] (same dtype);
 *   lse: float32 [B,H_q,N_q] or NULL;
 *   causal: 0 or 1 (bottom-right alignment); scale: positive and finite,
 *   usually 1/sqrt(d).
 * Empty problems (B, N_q or H_q zero) return ATTN_OK and enqueue nothing.
 * Work: 4*d FLOP per visible (query, key) pair per query head, on MFMA.
 */
int attn_prefill_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H_q, int H_kv, int N_q, int N_kv, int d, int causal, float scale,
                     int dtype, void* stream);

/*
 * Bytes of device workspace attn_decode_fwd needs for these sizes (0 if the
 * sizes are invalid or N_q is outside [1, 64]). The size is a pure function of
 * (B, H_q, H_kv, N_q, N_kv, d): it holds the partials of the finest split of
 * the KV sequence the call may use (the kernels may choose a coarser split on
 * the device from kv_lens, which needs no more), so the same sizes always need
 * the same workspace.
 */
size_t attn_decode_workspace_size(int B, int H_q, int H_kv, int N_q, int N_kv, int d, int dtype);

/*
 * Decode forward (split-KV, grouped-query): N_q new query tokens per request
 * (N_q = 1 for plain token-by-token decoding, up to 64 for multi-token decoding
 * such as speculative verification) against a KV cache of capacity N_kv, of
 * which the first kv_lens[b] positions are valid and already hold the new
 * tokens' keys and values. The KV sequence is split into chunks; each chunk
 * produces partial (m, l, u) per query row, which a second kernel merges by
 * log-sum-exp weights exp(m_s - m) (the online-softmax rescaling of the guide's
 * section 8 applied across chunks).
 *   q [B,H_q,N_q,d], k_cache/v_cache [B,H_kv,N_kv,d], o [B,H_q,N_q,d];
 *   kv_lens: device int32 [B] or NULL (all N_kv); values are clamped to [0, N_kv];
 *   lse: float32 [B,H_q,N_q] or NULL; N_q in [0, 64] (0 is a no-op; more is
 *   ATTN_ERR_UNSUPPORTED, use attn_prefill_fwd);
 *   causal: 0 or 1 with bottom-right alignment per request: query i of request
 *   b sees keys j <= i + kv_lens[b] - N_q (for N_q = 1, every valid key);
 *   scale: positive and finite;
 *   workspace: device memory of at least attn_decode_workspace_size(...) bytes,
 *   owned by the caller, overwritten by the call (no initialisation needed).
 * Work: 2 * kv_lens[b] * H_kv * d * sizeof(dtype) bytes of K and V read, once
 * for all N_q * H_q / H_kv query rows that share a KV head.
 */
int attn_decode_fwd(const void* q, const void* k_cache, const void* v_cache, const int* kv_lens,
                    void* o, float* lse, int B, int H_q, int H_kv, int N_q, int N_kv, int d,
                    int causal, float scale, int dtype, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * attn_decode_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The split partials go to a scratch array
 * of ATTN_DECODE_SCRATCH_BYTES that the library holds on every device it runs
 * on, for the life of the process; the call allocates and frees nothing.
 * Arguments, layouts, results and errors are those of attn_decode_fwd, except:
 *  - the split of the KV sequence is coarsened when the finer one's partials
 *    (B * H_q * N_q * splits * (d + 2) * 4 bytes) would not fit the scratch,
 *    so results can differ from attn_decode_fwd's by rounding; when even one
 *    split does not fit (B * H_q * N_q * (d + 2) * 4 > ATTN_DECODE_SCRATCH_BYTES)
 *    the call returns ATTN_ERR_WORKSPACE and enqueues nothing;
 *  - every call on one device shares that device's scratch: calls that overlap
 *    on one device (several streams, or several host threads) race and must be
 *    ordered by the caller. No contents need clearing between calls.
 * ATTN_ERR_LAUNCH is also returned if the scratch's device address cannot be
 * obtained.
 */
#define ATTN_DECODE_SCRATCH_BYTES ((size_t)64 << 20)
int attn_decode_fwd_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            const int* kv_lens, void* o, float* lse, int B, int H_q, int H_kv,
                            int N_q, int N_kv, int d, int causal, float scale, int dtype,
                            void* stream);

/*
 * Bytes of device workspace attn_decode_paged_fwd needs (0 if the sizes are
 * invalid). A pure function of its arguments.
 */
size_t attn_decode_paged_workspace_size(int B, int H_q, int H_kv, int N_q, int max_blocks,
                                        int block_size, int d, int dtype);

/*
 * Decode forward over a paged (block-wise) KV cache: the cache is cut into
 * fixed-size blocks that requests take from one shared pool, which removes the
 * fragmentation of per-request contiguous buffers (papanda925.com survey,
 * block-wise KV cache management in its recent-trends and method sections).
 * Same computation, partial/merge scheme and query layout as attn_decode_fwd.
 *   k_pool/v_pool [num_blocks, H_kv, block_size, d] (dtype), shared by all
 *     requests: block p holds block_size consecutive positions of every KV head;
 *   block_table: device int32 [B, max_blocks]; entry (b, i) is the pool block
 *     holding positions i*block_size .. (i+1)*block_size - 1 of request b. Only
 *     the entries of blocks below kv_lens[b] are read. An entry outside
 *     [0, num_blocks) reads as zero keys and values (the request's result is
 *     then meaningless, but nothing outside the pool is touched);
 *   kv_lens: device int32 [B] or NULL; clamped to [0, max_blocks * block_size];
 *   block_size: a power of two in [16, 4096] (else ATTN_ERR_UNSUPPORTED);
 *   q, o, lse, causal, scale, dtype, N_q, workspace: as for attn_decode_fwd,
 *     with attn_decode_paged_workspace_size(...) bytes of workspace.
 * Work: 2 * kv_lens[b] * H_kv * d * sizeof(dtype) bytes of K and V read.
 */
int attn_decode_paged_fwd(const void* q, const void* k_pool, const void* v_pool,
                          const int* block_table, const int* kv_lens, void* o, float* lse, int B,
                          int H_q, int H_kv, int N_q, int max_blocks, int block_size,
                          int num_blocks, int d, int causal, float scale, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode forward over an FP8 KV cache: keys and values are stored as OCP FP8
 * E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, 0x7F/0xFF NaN) with one dequantisation scale per tensor: the
 * cached value is code_value * k_scale (keys) or * v_scale (values). This halves
 * the bytes decode reads against 16-bit caches; the pages measure decode with
 * an FP8 KV cache (code-journey.com attention co-design summary, arithmetic
 * intensity formulas and decode measurements).
 * Codes are widened exactly to bf16 inside the kernel (every E4M3 value is a
 * bf16 value), so the result is attention over the dequantised cache, computed
 * as for a bf16 cache. Same layout and semantics as attn_decode_fwd with K/V
 * elements of one byte:
 *   k_cache/v_cache [B,H_kv,N_kv,d] uint8 E4M3 codes; q, o bf16 (dtype must be
 *   ATTN_BF16, else ATTN_ERR_UNSUPPORTED);
 *   k_scale, v_scale: positive and finite (else ATTN_ERR_VALUE);
 *   workspace: attn_decode_workspace_size(B, H_q, H_kv, N_q, N_kv, d, ATTN_BF16)
 *   bytes.
 * Work: 2 * kv_lens[b] * H_kv * d bytes of K and V read.
 */
int attn_decode_fp8_fwd(const void* q, const void* k_cache, const void* v_cache, float k_scale,
                        float v_scale, const int* kv_lens, void* o, float* lse, int B, int H_q,
                        int H_kv, int N_q, int N_kv, int d, int causal, float scale, int dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Paged FP8 decode: attn_decode_paged_fwd over pools of E4M3 codes
 * [num_blocks, H_kv, block_size, d] (uint8) with per-tensor scales as in
 * attn_decode_fp8_fwd. Workspace: attn_decode_paged_workspace_size(...,
 * ATTN_BF16) bytes.
 */
int attn_decode_paged_fp8_fwd(const void* q, const void* k_pool, const void* v_pool,
                              float k_scale, float v_scale, const int* block_table,
                              const int* kv_lens, void* o, float* lse, int B, int H_q, int H_kv,
                              int N_q, int max_blocks, int block_size, int num_blocks, int d,
                              int causal, float scale, int dtype, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace attn_backward needs: 2 * B * H_q * N_q floats (0 if
 * the sizes are invalid).
 */
size_t attn_backward_workspace_size(int B, int H_q, int H_kv, int N_q, int N_kv, int d, int dtype);

/*
 * Backward pass by recomputation: the forward pass keeps only O and the per-row
 * log-sum-exp; this call rebuilds the probability tiles from Q, K and that
 * statistic instead of reading a stored score matrix (marketmaker.cc,
 * "Rückwärtsdurchlauf: Neu berechnen statt speichern"). With S = scale Q K^T,
 * P = exp(S - lse) (masked entries 0) and Delta_i = sum_d dO_id O_id:
 *   dV = P^T dO,  dS = P o (dO V^T - Delta),  dQ = scale dS K,  dK = scale dS^T Q,
 * dK and dV summed over the H_q / H_kv query heads of each KV head.
 *   q, o, d_o, dq [B,H_q,N_q,d]; k, v, dk, dv [B,H_kv,N_kv,d]; all of `dtype`
 *   (ATTN_BF16 or ATTN_F16; ATTN_F32 is ATTN_ERR_UNSUPPORTED);
 *   lse: float32 [B,H_q,N_q], the natural-log LSE that attn_prefill_fwd returned
 *   for the same q, k, v, causal and scale (o likewise its output);
 *   causal, scale: as for attn_prefill_fwd (bottom-right alignment);
 *   workspace: attn_backward_workspace_size(...) bytes, overwritten.
 * dq, dk, dv are written in full (no accumulation into them); they must not
 * overlap any input, each other or the workspace. Two kernels run on
 * `stream`: dQ (one workgroup per 256 query rows), which also leaves each
 * row's Delta and log2-unit LSE in the workspace, then dK/dV (one workgroup
 * per 256 keys); no atomics, so results are deterministic.
 * Work: 10*d FLOP per visible (query, key) pair per query head in the five
 * products (the recomputation adds 4*d more).
 */
int attn_backward(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                  const float* lse, void* dq, void* dk, void* dv, int B, int H_q, int H_kv,
                  int N_q, int N_kv, int d, int causal, float scale, int dtype, void* workspace,
                  size_t workspace_bytes, void* stream);

/* Static, human-readable text for a status code (never NULL). */
const char* attn_status_string(int status);

/* Library ABI version (major * 100 + minor). */
int attn_version(void);

/*
 * Tuning knobs. No setting is ever needed for correctness: every value gives
 * the same results up to rounding, and 0 always means "chosen automatically".
 * Settings are process-wide and apply to calls made after the change (thread
 * safe: each knob is one atomic integer). Their initial values come from the
 * environment variable ATTN_TUNING, read once per process at the first call
 * that needs a knob, as comma-separated name=value pairs with the names below
 * (e.g. "prefill_variant=4,decode_chunk=2048"); entries that do not parse or
 * hold an invalid value are ignored.
 *   ATTN_TUNE_PREFILL_VARIANT  "prefill_variant"  1..5: alternative forms of the
 *       16-bit prefill kernel (1: 4 wavefronts per workgroup; 2: two query
 *       blocks per wavefront; 3: one work item per workgroup; 4: direct-to-LDS
 *       ring form; 5: register-staged form).
 *   ATTN_TUNE_PREFILL_SLOTS    "prefill_slots"    n > 0: persistent prefill grid
 *       with at most n workgroups.
 *   ATTN_TUNE_DECODE_CHUNK     "decode_chunk"     n > 0: keys per decode split
 *       (rounded up to 128; at most 2048 for paged caches), used as given. The
 *       decode workspace sizes depend on it.
 *   ATTN_TUNE_DECODE_GROUPS    "decode_groups"    1, 2 or 4 query column groups
 *       per decode wavefront.
 *   ATTN_TUNE_DECODE_ROWS_MODE "decode_rows_mode" 1: multi-token decode of
 *       contiguous 16-bit caches always through the prefill kernel; 2: never.
 * attn_set_tuning returns ATTN_ERR_VALUE (and changes nothing) for an unknown
 * knob or a value outside its range; attn_get_tuning returns the current value,
 * or -1 for an unknown knob.
 */
typedef enum {
  ATTN_TUNE_PREFILL_VARIANT = 0,
  ATTN_TUNE_PREFILL_SLOTS = 1,
  ATTN_TUNE_DECODE_CHUNK = 2,
  ATTN_TUNE_DECODE_GROUPS = 3,
  ATTN_TUNE_DECODE_ROWS_MODE = 4
} attn_tune_t;
int attn_set_tuning(int knob, int value);
int attn_get_tuning(int knob);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_ATTN_H_ */
