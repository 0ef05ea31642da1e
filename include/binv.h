/*
 * binv.h -- libbinv: batch-invariant transformer kernels for AMD Instinct MI355X (gfx950).
 *
 * What "batch-invariant" means here (devpress.csdn.net explainer of "Defeating
 * Nondeterminism in LLM Inference", section 2.3; tom-jerr.github.io
 * "Batch-Invariant Kernel", Motivation): the bits of one row's (or one
 * sequence's) output are a function of that row's own inputs only.  For a
 * fixed weight shape (N, K), feature size d and attention shape (Hq, Hkv, D,
 * page size, scale) they do not depend on M, B or T, on the row's position in
 * the batch, on which other rows share the call, on how a prefill is split
 * into chunks, on where the sequence's pages sit in the cache, or on whether a
 * token is processed by the prefill or the decode entry point.  Every entry
 * point is also run-to-run deterministic: no atomics, no data-dependent
 * scheduling.
 *
 * Conventions shared by every entry point
 *   - All data pointers are DEVICE pointers owned by the caller.  Nothing is
 *     retained after return and the library allocates no device memory.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*, NULL = the
 *     default stream) and runs asynchronously; no entry point synchronises.
 *   - Arguments are validated on the host before anything is launched; a
 *     non-zero status means nothing was enqueued, except BINV_ERR_LAUNCH,
 *     which reports a failed launch (hipGetLastError).
 *   - Data pointers must be 16-byte aligned.  Leading dimensions are in
 *     elements and must keep every row 16-byte aligned (a multiple of 8 for
 *     bf16, of 4 for fp32).
 *   - bf16 is the 16-bit bfloat16 format; every conversion to bf16 rounds to
 *     nearest, ties to even.  Accumulation is fp32.
 *   - Preconditions that live in device memory (kv_lens, cu_q, page-table
 *     entries) cannot be checked without a synchronisation; they are the
 *     caller's contract and are stated per entry point.
 *   - The library keeps no mutable global state (one exception: the entry
 *     point that allocates nothing caches the address of its fixed device
 *     array per GPU, under a lock); calls from several host threads are safe.
 */
#ifndef BINV_H
#define BINV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BINV_OK = 0,
    BINV_ERR_INVALID_ARG = 1,   /* null pointer, negative size, bad leading dimension, misalignment */
    BINV_ERR_UNSUPPORTED = 2,   /* a size or shape outside what the kernels implement */
    BINV_ERR_WORKSPACE = 3,     /* workspace missing or smaller than binv_attn_workspace_bytes() */
    BINV_ERR_LAUNCH = 4,        /* the HIP runtime rejected a launch */
    BINV_ERR_SCRATCH = 5        /* the call needs more than the fixed scratch of the
                                   entry point that allocates nothing */
} binv_status;

typedef enum { BINV_F32 = 0, BINV_BF16 = 1 } binv_dtype;

/* Largest KV length the attention entry points accept: 512 chunks of 256
 * tokens, i.e. the fixed merge-tree depth of 9. */
#define BINV_ATTN_CHUNK 256
#define BINV_ATTN_MAX_CHUNKS 512
#define BINV_ATTN_MAX_KV_LEN (BINV_ATTN_CHUNK * BINV_ATTN_MAX_CHUNKS)
#define BINV_PAGE_SIZE 16

/* Human-readable name of a status code (static storage). */
const char* binv_status_str(int status);

/* Library version string (static storage). */
const char* binv_version(void);

/* ------------------------------------------------------------------------
 * RMSNorm, one workgroup per row.
 * Defines: tom-jerr.github.io "Batch-Invariant Kernel", section RMSNorm
 * (formula and the data-parallel reduction: each row reduced inside one
 * core); devpress.csdn.net explainer, section 3.1 RMSNorm (x * rsqrt(mean(x^2)) * weight).
 *
 *   y[i, j] = x[i, j] * r_i * gamma[j],   r_i = 1 / sqrt((1/d) * sum_j x[i, j]^2 + eps)
 *
 * x      [M, d] row-major, leading dimension ldx, dtype x_dt (BINV_F32 or BINV_BF16)
 * gamma  [d], dtype g_dt
 * y      [M, d] row-major, leading dimension ldy, dtype y_dt
 * The sum of squares of a row is formed inside one workgroup in an order fixed
 * by d alone.  d must be a multiple of 8 (bf16 x) or 4 (fp32 x), 1 <= d <= 16384
 * for bf16 x and <= 8192 for fp32 x (else BINV_ERR_UNSUPPORTED).  M = 0 is a no-op.
 * x and y must not overlap.
 * ------------------------------------------------------------------------ */
int binv_rmsnorm(const void* x, int x_dt, int64_t ldx,
                 const void* gamma, int g_dt,
                 void* y, int y_dt, int64_t ldy,
                 int64_t M, int64_t d, float eps, void* stream);

/* The residual update followed by the RMSNorm of its result, in one launch
 * (a decoder layer's "h += o; x = norm(h)"):
 *   h[i, j] += float(a[i, j]);  then y = binv_rmsnorm of the updated h (fp32)
 * with the bits of binv_residual_add followed by binv_rmsnorm(h, BINV_F32, ...)
 * (the same fp32 adds, and the same per-row reduction).
 * h fp32 [M, d] (ldh), updated in place; a bf16 [M, d] (lda, a multiple of 4,
 * 8-byte aligned); gamma, y and the limits as for binv_rmsnorm with fp32 x.
 * y must not overlap h or a. */
int binv_add_rmsnorm(float* h, int64_t ldh, const void* a, int64_t lda,
                     const void* gamma, int g_dt,
                     void* y, int y_dt, int64_t ldy,
                     int64_t M, int64_t d, float eps, void* stream);

/* ------------------------------------------------------------------------
 * GEMM with one fixed per-element reduction and no split-K.
 * Defines: devpress.csdn.net explainer, section 3.2 Matmul
 * (C[i,j] = sum_k A[i,k] B[k,j]; the reduction of every element fixed for
 * every batch size, split-K disabled); tom-jerr.github.io "Batch-Invariant
 * Kernel", section GEMM (fixed tiling, K strategy decoupled from M).
 *
 *   C[i, j] = sum_k A[i, k] * W[k, j]
 *
 * A  bf16 [M, K] row-major, leading dimension lda
 * W  bf16 [K, N] row-major, leading dimension ldw
 * C  [M, N] row-major, leading dimension ldc, dtype c_dt (BINV_BF16 or BINV_F32)
 * Each C element is accumulated in fp32 by bf16 matrix-core instructions over
 * k in ascending blocks of 32 (K zero-padded to a multiple of 64), one
 * accumulator per element, whatever M is.  Which lanes and workgroups carry
 * which elements (the output tiling) follows the shape; it never enters an
 * element's arithmetic, so a row's bits do not depend on M.  (A deviation
 * from the pages, which keep one tile configuration for every batch size
 * because there the configuration sets the reduction order: here only the
 * per-element reduction is fixed, and the invariance rests on the matrix
 * instruction giving an element the same bits in every lane, tile and
 * kernel, which tests check across every kernel and M.)
 * K and N must be multiples of 8; M, N, K <= 2^31 - 1; lda < 2^22 and
 * ldw < 1.6e7 elements (tiles are addressed with 32-bit offsets).  M = 0 or
 * N = 0 is a no-op; K = 0 writes zeros.  C must not overlap A or W.
 * ------------------------------------------------------------------------ */
int binv_gemm_bf16(const void* A, int64_t lda,
                   const void* W, int64_t ldw,
                   void* C, int c_dt, int64_t ldc,
                   int64_t M, int64_t N, int64_t K, void* stream);

/* Decode batches over pre-packed weights: the same GEMM (same bits as
 * binv_gemm_bf16 for the same A and W, for every M it accepts) with W
 * re-laid out once so that the weights of each 16-column strip of C are one
 * contiguous run (at decode sizes a GEMM is a stream of the weights; a strip
 * of a row-major W is 32 bytes of every row).  Same method citations as
 * binv_gemm_bf16.
 *
 * Packed layout (bf16, binv_gemm_bf16_packed_bytes(N, K) bytes, 16-byte
 * aligned, caller-owned): Wp[s][kb][c][kk] = W[32 kb + kk][16 s + c], zero
 * where 32 kb + kk >= K or 16 s + c >= N; s < ceil(N / 16) strips, kb <
 * 2 ceil(K / 64) k-blocks, c < 16, kk < 32.
 *
 * binv_gemm_bf16_pack: W bf16 [K, N] row-major (ldw) -> Wp, on `stream`.
 *   Same K, N, ldw rules as binv_gemm_bf16.  K = 0 or N = 0 is a no-op.
 * binv_gemm_bf16_packed: C [M, N] (c_dt, ldc) = A [M, K] (lda) x W, with W
 *   given as Wp.  1 <= M <= 64 (else BINV_ERR_UNSUPPORTED; M = 0 is a no-op);
 *   K and N as for binv_gemm_bf16, and Wp must have been packed for this K
 *   and N.  C must not overlap A or Wp.
 * binv_gemm_bf16_packed_bytes returns 0 for negative sizes. */
size_t binv_gemm_bf16_packed_bytes(int64_t N, int64_t K);
int binv_gemm_bf16_pack(const void* W, int64_t ldw, int64_t K, int64_t N, void* Wp,
                        void* stream);
int binv_gemm_bf16_packed(const void* A, int64_t lda, const void* Wp,
                          void* C, int c_dt, int64_t ldc,
                          int64_t M, int64_t N, int64_t K, void* stream);

/* ------------------------------------------------------------------------
 * Paged KV cache layout used by both attention entry points.
 * (The pages describe a KV cache whose reduction length is cached plus new
 * tokens -- devpress.csdn.net explainer, section 3.3 -- but fix no layout.)
 *
 *   k_cache  bf16 [num_pages, Hkv, page_size, D]   (slot, then feature)
 *   v_cache  bf16 [num_pages, Hkv, D, page_size]   (feature, then slot)
 *   page_table int32 [B, pt_stride]
 *   logical token t of sequence b lives in page page_table[b * pt_stride + t / page_size],
 *   slot t % page_size.  page_size must be 16; D must be 64 or 128;
 *   Hq % Hkv == 0 with Hq / Hkv in {1, 2, 4, 8, 16}.
 *
 * Only the first ceil(kv_lens[b] / 16) page-table entries of a sequence are
 * used as page indices (later entries of the row, within its pt_stride, may
 * be read ahead but never dereferenced; they may hold any value), and slots
 * at or past kv_lens[b] are never used (they may hold any bits, NaN
 * included).
 *
 * Attention computed (devpress.csdn.net explainer, section 3.3: two
 * reductions over the KV length; fixed-size split example):
 *   a query row of head h at absolute position p attends to keys 0..p of KV
 *   head h / (Hq / Hkv):  out = sum_j softmax_j(scale * q . k_j) v_j.
 *   The keys are split into fixed 256-token chunks counted from absolute
 *   position 0 (chunk c = [256c, 256c + 256) intersected with [0, p]); each
 *   chunk yields an fp32 partial (max, sum of weights, weighted sum of values)
 *   and the partials are merged by a binary tree padded to a fixed depth of 9
 *   (tom-jerr.github.io "Batch-Invariant Kernel", section Flash Attention,
 *   fixed-size Split-KV with a chunk-count-independent tree merge).
 *   Decode and prefill compute every chunk partial with the same per-element
 *   arithmetic, whichever kernel a call's shape selects (prefill sequences
 *   with long new-token runs share one load of each chunk among 128 rows),
 *   and merge with the same tree, so a token's output bits are the same on
 *   either path and in any call.  An output element that is exactly zero is
 *   written as +0.
 *
 * Workspace: fp32 partials, caller-owned.  Decode needs at least
 *   binv_attn_workspace_bytes(B, Hq, D, max_kv_len) bytes (one partial per
 *   query row and chunk); prefill at least
 *   binv_attn_prefill_workspace_bytes(B, T, max_q_len, max_kv_len, Hq, Hkv, D),
 *   which never exceeds binv_attn_workspace_bytes(T, Hq, D, max_kv_len).
 *   Prefill rows of long new-token runs (D = 128, a sequence with at least
 *   ceil(64 / (Hq / Hkv)) new tokens) keep in memory only the merge tree's
 *   pending subtrees of four or more chunks, max(1, floor(log2(ceil(
 *   max_kv_len / 256))) - 1) per row, so a single-sequence prefill needs
 *   T * Hq * that many * (D + 2) * 4 bytes -- except when a single sequence's
 *   128-row blocks (times Hkv) number fewer than 256 and max_kv_len spans at
 *   most 64 chunks: then each workgroup takes an aligned pair of chunks and
 *   the call keeps one pair node per token, T * Hq * ceil(chunks / 2) *
 *   (D + 2) * 4 bytes; rows
 *   of short runs keep one partial per chunk, indexed per sequence when that
 *   is smaller than per token.  Both functions return 0 for arguments the
 *   entry points reject.
 * ------------------------------------------------------------------------ */
size_t binv_attn_workspace_bytes(int64_t n_query_tokens, int Hq, int D, int64_t max_kv_len);
size_t binv_attn_prefill_workspace_bytes(int64_t B, int64_t T, int64_t max_q_len,
                                         int64_t max_kv_len, int Hq, int Hkv, int D);

/* Decode: one query token per sequence.
 * q    bf16 [B, Hq, D]
 * out  bf16 [B, Hq, D]
 * kv_lens int32 [B]: KV length of each sequence INCLUDING the current token,
 *   whose K/V must already be in the cache; the query sits at position
 *   kv_lens[b] - 1.  Contract: 1 <= kv_lens[b] <= max_kv_len.
 * max_kv_len: host-side upper bound used to size the grid (1..BINV_ATTN_MAX_KV_LEN).
 * B = 0 is a no-op. */
int binv_attn_decode_paged(const void* q,
                           const void* k_cache, const void* v_cache,
                           const int32_t* page_table, int64_t pt_stride,
                           const int32_t* kv_lens,
                           void* out,
                           int64_t B, int64_t max_kv_len, int Hq, int Hkv, int D, int page_size,
                           float scale, void* workspace, size_t ws_bytes, void* stream);

/* Prefill / chunked prefill: a ragged batch of new tokens whose K/V are
 * already written into the cache (one unified reduction over cached + new keys).
 * q    bf16 [T, Hq, D], the new tokens of all sequences, sequence after sequence
 * cu_q int32 [B + 1]: sequence b owns rows cu_q[b] .. cu_q[b+1]-1; cu_q[0] = 0, cu_q[B] = T
 * kv_lens int32 [B]: KV length of sequence b after this step (cached + new)
 * out  bf16 [T, Hq, D]
 * Row i of sequence b sits at position kv_lens[b] - (cu_q[b+1] - cu_q[b]) + i.
 * Contract: 0 <= cu_q[b+1] - cu_q[b] <= min(max_q_len, kv_lens[b]),
 *           kv_lens[b] <= max_kv_len.
 * T = 0 or B = 0 is a no-op. */
int binv_attn_prefill_paged(const void* q, const int32_t* cu_q,
                            const void* k_cache, const void* v_cache,
                            const int32_t* page_table, int64_t pt_stride,
                            const int32_t* kv_lens,
                            void* out,
                            int64_t B, int64_t T, int64_t max_q_len, int64_t max_kv_len,
                            int Hq, int Hkv, int D, int page_size, float scale,
                            void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, contract and results (bit for bit)
 * as binv_attn_decode_paged, whose kernels it runs; the fp32 partials go to a
 * fixed device array inside the library instead of a caller workspace.
 *
 *   - The array holds BINV_NOALLOC_SCRATCH_BYTES (128 MiB) on every GPU the
 *     library's kernels are loaded on, until the process ends.  A call needing
 *     more than that -- binv_attn_workspace_bytes(B, Hq, D, max_kv_len) above
 *     the limit, e.g. B * ceil(max_kv_len / 256) > 8065 at Hq = 32, D = 128 --
 *     returns BINV_ERR_SCRATCH and enqueues nothing.
 *   - The call makes no hipMalloc / hipFree and no allocating library call.
 *     Its first call on a device looks up that device's copy of the array
 *     (hipGetSymbolAddress) and keeps the address; the stream must belong to
 *     the current device.
 *   - Every call on one GPU shares that GPU's array.  Nothing in it needs to
 *     start at zero (every partial a call reads, the same call wrote first),
 *     but two calls that overlap in time on one GPU (different streams, or
 *     host threads without ordering) race on it: order them.
 * ------------------------------------------------------------------------ */
#define BINV_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

int binv_attn_decode_paged_noalloc(const void* q,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* page_table, int64_t pt_stride,
                                   const int32_t* kv_lens,
                                   void* out,
                                   int64_t B, int64_t max_kv_len, int Hq, int Hkv, int D,
                                   int page_size, float scale, void* stream);

/* ------------------------------------------------------------------------
 * Shape-tuned comparators.  NOT batch-invariant, on purpose: they choose their
 * reduction strategy from the batch shape the way the pages say production
 * libraries do (devpress.csdn.net explainer, section 3.2, split-K when M is
 * small; tom-jerr.github.io "Batch-Invariant Kernel", sections RMSNorm, GEMM
 * and Flash Attention, shape-dependent splits).  They exist to measure the
 * price of invariance and as positive controls for the invariance tests.
 * Same arguments as the invariant entry points (plus a workspace for the GEMM).
 * ------------------------------------------------------------------------ */
size_t binv_gemm_bf16_tuned_workspace_bytes(int64_t M, int64_t N, int64_t K);
int binv_gemm_bf16_tuned(const void* A, int64_t lda,
                         const void* W, int64_t ldw,
                         void* C, int c_dt, int64_t ldc,
                         int64_t M, int64_t N, int64_t K,
                         void* workspace, size_t ws_bytes, void* stream);
int binv_rmsnorm_tuned(const void* x, int x_dt, int64_t ldx,
                       const void* gamma, int g_dt,
                       void* y, int y_dt, int64_t ldy,
                       int64_t M, int64_t d, float eps, void* stream);
size_t binv_attn_decode_tuned_workspace_bytes(int64_t B, int Hq, int D, int64_t max_kv_len);
int binv_attn_decode_paged_tuned(const void* q,
                                 const void* k_cache, const void* v_cache,
                                 const int32_t* page_table, int64_t pt_stride,
                                 const int32_t* kv_lens,
                                 void* out,
                                 int64_t B, int64_t max_kv_len, int Hq, int Hkv, int D, int page_size,
                                 float scale, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Decoder glue: the pointwise and selection steps between the kernels above.
 * Each output element is computed from its own inputs by a fixed instruction
 * sequence, so these are batch-invariant as they stand (devpress.csdn.net
 * explainer, section 3: pointwise operations need no change).  Argmax and
 * top-k break ties by the lowest index (paper.xwysyy.cn "19.7", section
 * 19.7.4: near-tied logits are where differences become different tokens).
 * ------------------------------------------------------------------------ */

/* out[t, :] = table[ids[t], :] widened to fp32.  table bf16 [V, H] row-major,
 * out fp32 [T, H] (the residual stream).  An id outside [0, V) gives a zero row.
 * H % 8 == 0; table and out 16-byte aligned. */
int binv_embed(const int32_t* ids, int64_t T, const void* table, int64_t V, int64_t H,
               float* out, void* stream);

/* Rotary position embedding (rotate-half form, angle p * theta^(-2i/D) for the
 * pair (i, i + D/2), evaluated in fp64; rotation in fp32, rounded once to bf16)
 * on the q and k heads of a fused projection row, then the K/V write into the
 * paged cache.
 * qkv     bf16 [T, ld_qkv]: per token Hq query heads, Hkv key heads, Hkv value
 *         heads of D features each, in that order
 * tok_seq, tok_pos  int32 [T]: sequence (row of page_table) and absolute position
 * q_out   bf16 [T, Hq, D]: rotated queries
 * k_cache, v_cache: the paged layout of the attention entry points; token
 *         (seq, pos) goes to page page_table[seq * pt_stride + pos / 16], slot pos % 16.
 * Contract: the page-table entries addressed are valid; no two tokens of the
 * call share (seq, pos). */
int binv_rope_kv_write(const void* qkv, int64_t ld_qkv, const int32_t* tok_seq,
                       const int32_t* tok_pos, int64_t T, int Hq, int Hkv, int D, double theta,
                       void* q_out, void* k_cache, void* v_cache, const int32_t* page_table,
                       int64_t pt_stride, int page_size, void* stream);

/* SwiGLU: out[t, j] = bf16(silu(g) * u), g = gate_up[t, j], u = gate_up[t, F + j],
 * silu(g) = g / (1 + exp(-g)), fp32.  gate_up bf16 [T, ld_gu >= 2F], out bf16
 * [T, ld_out >= F].  F, ld_gu, ld_out multiples of 8, pointers 16-byte aligned;
 * T <= 65535. */
int binv_swiglu(const void* gate_up, int64_t ld_gu, int64_t T, int64_t F, void* out,
                int64_t ld_out, void* stream);

/* Residual update h[t, j] += x[t, j]: h fp32 [T, ldh], x bf16 [T, ldx].
 * H, ldh, ldx multiples of 4; h 16-byte and x 8-byte aligned; T <= 65535. */
int binv_residual_add(float* h, int64_t ldh, const void* x, int64_t ldx, int64_t T, int64_t H,
                      void* stream);

/* dst[r, :] = src[idx[r], :] for rows of `cols` elements of dtype dt, copied bit
 * for bit.  Row sizes and pointers 4-byte aligned.  Contract: idx entries valid. */
int binv_gather_rows(const void* src, int dt, int64_t lds, const int32_t* idx, int64_t R,
                     void* dst, int64_t ldd, int64_t cols, void* stream);

/* Three-way bf16 split of fp32 activations, for the fp32-activation mitigation
 * (devpress.csdn.net explainer of "Defeating Nondeterminism in LLM Inference",
 * sections 2 and 6: weights stay bf16, activations fp32).  For x fp32 [M, ldx]:
 *   out[i, k] = hi = bf16(x[i, k]),  out[i, K + k] = mid = bf16(x[i, k] - hi),
 *   out[i, 2K + k] = lo = bf16(x[i, k] - hi - mid)     (round to nearest even)
 * out bf16 [M, ld_out >= 3K].  hi + mid + lo == x exactly for finite x whose
 * parts stay normal, so binv_gemm_bf16 of out against the weights stacked three
 * times ([W; W; W], 3K x N) with fp32 output contracts the fp32 activations
 * with exact products and one fp32 accumulator per element.  Elementwise, so
 * batch-invariant as it stands.  K, ldx, ld_out multiples of 4; x 16-byte and
 * out 8-byte aligned; M <= 65535.  The caller owns both buffers. */
int binv_split_bf16x3(const float* x, int64_t ldx, int64_t M, int64_t K, void* out,
                      int64_t ld_out, void* stream);

/* Exact top-K (K <= 32) of each fp32 row of x [R, ldx] over its first n entries:
 * ids int32 [R, K] and vals fp32 [R, K], sorted by value descending, equal values
 * by index ascending; NaN is never selected (a row with fewer than K non-NaN
 * entries is padded with id -1, value -inf).  ids[r, 0] is the greedy argmax. */
int binv_topk(const float* x, int64_t ldx, int64_t R, int64_t n, int K, int32_t* ids,
              float* vals, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BINV_H */
