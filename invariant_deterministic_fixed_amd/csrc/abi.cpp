// abi.cpp -- the extern "C" entry points of libbinv: host-side argument
// validation, then the launchers in the .hip files.  Declarations and the
// contract of every entry point are in include/binv.h.
#include "../../include/binv.h"

#include <hip/hip_runtime.h>
#include <math.h>

#include "kernels.hpp"

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int elem_size(int dt) { return dt == BINV_BF16 ? 2 : 4; }
inline bool valid_dt(int dt) { return dt == BINV_BF16 || dt == BINV_F32; }
// a leading dimension keeps every row 16-byte aligned
inline bool ld_ok(int64_t ld, int dt) { return ld > 0 && (ld * elem_size(dt)) % 16 == 0; }
inline int status_of(hipError_t e) { return e == hipSuccess ? BINV_OK : BINV_ERR_LAUNCH; }
constexpr int64_t I32MAX = 2147483647;

int check_rmsnorm(const void* x, int x_dt, int64_t ldx, const void* gamma, int g_dt, void* y,
                  int y_dt, int64_t ldy, int64_t M, int64_t d) {
    if (M < 0 || d < 0) return BINV_ERR_INVALID_ARG;
    if (!valid_dt(x_dt) || !valid_dt(g_dt) || !valid_dt(y_dt)) return BINV_ERR_INVALID_ARG;
    if (M == 0) return BINV_OK;
    if (!x || !gamma || !y) return BINV_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(gamma) || !aligned16(y)) return BINV_ERR_INVALID_ARG;
    if (!ld_ok(ldx, x_dt) || !ld_ok(ldy, y_dt) || ldx < d || ldy < d) return BINV_ERR_INVALID_ARG;
    const int vec = x_dt == BINV_BF16 ? 8 : 4;
    const int64_t dmax = x_dt == BINV_BF16 ? 16384 : 8192;
    if (d == 0 || d % vec != 0 || d > dmax) return BINV_ERR_UNSUPPORTED;
    if (M > I32MAX) return BINV_ERR_UNSUPPORTED;
    return BINV_OK;
}

int check_gemm(const void* A, int64_t lda, const void* W, int64_t ldw, void* C, int c_dt,
               int64_t ldc, int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return BINV_ERR_INVALID_ARG;
    if (!valid_dt(c_dt)) return BINV_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return BINV_OK;
    if (!C || (K > 0 && (!A || !W))) return BINV_ERR_INVALID_ARG;
    if (!aligned16(C) || (K > 0 && (!aligned16(A) || !aligned16(W)))) return BINV_ERR_INVALID_ARG;
    if (!ld_ok(ldc, c_dt) || ldc < N) return BINV_ERR_INVALID_ARG;
    if (K > 0 && (!ld_ok(lda, BINV_BF16) || !ld_ok(ldw, BINV_BF16) || lda < K || ldw < N))
        return BINV_ERR_INVALID_ARG;
    if (K % 8 != 0 || N % 8 != 0) return BINV_ERR_UNSUPPORTED;
    if (M > I32MAX || N > I32MAX || K > I32MAX) return BINV_ERR_UNSUPPORTED;
    // tiles are addressed with 32-bit buffer offsets: 256 rows of A, 64 rows of W
    if (lda >= 4194304 || ldw >= 16000000) return BINV_ERR_UNSUPPORTED;
    if (((M + 127) / 128) * ((N + 127) / 128) > I32MAX) return BINV_ERR_UNSUPPORTED;
    return BINV_OK;
}

int check_attn_common(const void* k_cache, const void* v_cache, const int32_t* page_table,
                      int64_t pt_stride, const int32_t* kv_lens, int64_t B, int64_t max_kv_len,
                      int Hq, int Hkv, int D, int page_size, float scale) {
    if (!k_cache || !v_cache || !page_table || !kv_lens) return BINV_ERR_INVALID_ARG;
    if (!aligned16(k_cache) || !aligned16(v_cache)) return BINV_ERR_INVALID_ARG;
    if (Hq <= 0 || Hkv <= 0 || D <= 0 || page_size <= 0 || pt_stride <= 0)
        return BINV_ERR_INVALID_ARG;
    if (!isfinite(scale)) return BINV_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return BINV_ERR_INVALID_ARG;
    const int G = Hq / Hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return BINV_ERR_UNSUPPORTED;
    if (D != 64 && D != 128) return BINV_ERR_UNSUPPORTED;
    if (page_size != BINV_PAGE_SIZE) return BINV_ERR_UNSUPPORTED;
    if (max_kv_len < 1) return BINV_ERR_INVALID_ARG;
    if (max_kv_len > BINV_ATTN_MAX_KV_LEN) return BINV_ERR_UNSUPPORTED;
    if (B > 65535) return BINV_ERR_UNSUPPORTED;
    return BINV_OK;
}

}  // namespace

extern "C" {

const char* binv_status_str(int status) {
    switch (status) {
        case BINV_OK: return "BINV_OK";
        case BINV_ERR_INVALID_ARG: return "BINV_ERR_INVALID_ARG: invalid argument";
        case BINV_ERR_UNSUPPORTED: return "BINV_ERR_UNSUPPORTED: size or shape not supported";
        case BINV_ERR_WORKSPACE: return "BINV_ERR_WORKSPACE: workspace missing or too small";
        case BINV_ERR_LAUNCH: return "BINV_ERR_LAUNCH: kernel launch failed";
        case BINV_ERR_SCRATCH:
            return "BINV_ERR_SCRATCH: the call needs more partials memory than the fixed "
                   "BINV_NOALLOC_SCRATCH_BYTES of the no-alloc entry point";
        default: return "unknown binv status";
    }
}

const char* binv_version(void) { return "libbinv 0.1 (gfx950)"; }

int binv_rmsnorm(const void* x, int x_dt, int64_t ldx, const void* gamma, int g_dt, void* y,
                 int y_dt, int64_t ldy, int64_t M, int64_t d, float eps, void* stream) {
    const int st = check_rmsnorm(x, x_dt, ldx, gamma, g_dt, y, y_dt, ldy, M, d);
    if (st != BINV_OK || M == 0) return st;
    if (!(eps >= 0.0f) || !isfinite(eps)) return BINV_ERR_INVALID_ARG;
    return status_of(binv::launch_rmsnorm(x, x_dt == BINV_BF16, ldx, gamma, g_dt == BINV_BF16, y,
                                          y_dt == BINV_BF16, ldy, M, (int)d, eps,
                                          (hipStream_t)stream));
}

int binv_add_rmsnorm(float* h, int64_t ldh, const void* a, int64_t lda, const void* gamma,
                     int g_dt, void* y, int y_dt, int64_t ldy, int64_t M, int64_t d, float eps,
                     void* stream) {
    const int st = check_rmsnorm(h, BINV_F32, ldh, gamma, g_dt, y, y_dt, ldy, M, d);
    if (st != BINV_OK || M == 0) return st;
    if (!(eps >= 0.0f) || !isfinite(eps)) return BINV_ERR_INVALID_ARG;
    if (!a || (reinterpret_cast<uintptr_t>(a) & 7u) || lda % 4 || lda < d) return BINV_ERR_INVALID_ARG;
    return status_of(binv::launch_add_rmsnorm(h, ldh, a, lda, gamma, g_dt == BINV_BF16, y,
                                              y_dt == BINV_BF16, ldy, M, (int)d, eps,
                                              (hipStream_t)stream));
}

int binv_rmsnorm_tuned(const void* x, int x_dt, int64_t ldx, const void* gamma, int g_dt,
                       void* y, int y_dt, int64_t ldy, int64_t M, int64_t d, float eps,
                       void* stream) {
    const int st = check_rmsnorm(x, x_dt, ldx, gamma, g_dt, y, y_dt, ldy, M, d);
    if (st != BINV_OK || M == 0) return st;
    if (!(eps >= 0.0f) || !isfinite(eps)) return BINV_ERR_INVALID_ARG;
    return status_of(binv::launch_rmsnorm_tuned(x, x_dt == BINV_BF16, ldx, gamma,
                                                g_dt == BINV_BF16, y, y_dt == BINV_BF16, ldy, M,
                                                (int)d, eps, (hipStream_t)stream));
}

int binv_gemm_bf16(const void* A, int64_t lda, const void* W, int64_t ldw, void* C, int c_dt,
                   int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream) {
    const int st = check_gemm(A, lda, W, ldw, C, c_dt, ldc, M, N, K);
    if (st != BINV_OK || M == 0 || N == 0) return st;
    return status_of(binv::launch_gemm(A, lda, W, ldw, C, c_dt == BINV_F32, ldc, (int)M, (int)N,
                                       (int)K, (hipStream_t)stream));
}

size_t binv_gemm_bf16_packed_bytes(int64_t N, int64_t K) {
    if (N < 0 || K < 0) return 0;
    return binv::gemm_packed_bytes(N, K);
}

int binv_gemm_bf16_pack(const void* W, int64_t ldw, int64_t K, int64_t N, void* Wp,
                        void* stream) {
    if (K < 0 || N < 0) return BINV_ERR_INVALID_ARG;
    if (K == 0 || N == 0) return BINV_OK;
    if (!W || !Wp || !aligned16(W) || !aligned16(Wp)) return BINV_ERR_INVALID_ARG;
    if (!ld_ok(ldw, BINV_BF16) || ldw < N) return BINV_ERR_INVALID_ARG;
    if (K % 8 != 0 || N % 8 != 0) return BINV_ERR_UNSUPPORTED;
    if (N > I32MAX || K > I32MAX || ldw >= 16000000) return BINV_ERR_UNSUPPORTED;
    return status_of(binv::launch_gemm_pack(W, ldw, (int)K, (int)N, Wp, (hipStream_t)stream));
}

int binv_gemm_bf16_packed(const void* A, int64_t lda, const void* Wp, void* C, int c_dt,
                          int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream) {
    // the plain entry point's checks, with the packed array standing in for W
    // (its leading dimension is not used: pass N, once N is known to be valid)
    if (M < 0 || N < 0 || K < 0) return BINV_ERR_INVALID_ARG;
    if (M > 0 && N % 8 != 0) return BINV_ERR_UNSUPPORTED;
    const int st = check_gemm(A, lda, Wp, N, C, c_dt, ldc, M, N, K);
    if (st != BINV_OK || M == 0 || N == 0) return st;
    if (M > 64) return BINV_ERR_UNSUPPORTED;
    return status_of(binv::launch_gemm_packed(A, lda, Wp, C, c_dt == BINV_F32, ldc, (int)M,
                                              (int)N, (int)K, (hipStream_t)stream));
}

size_t binv_gemm_bf16_tuned_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K < 0) return 0;
    return binv::gemm_tuned_workspace_bytes(M, N, K);
}

int binv_gemm_bf16_tuned(const void* A, int64_t lda, const void* W, int64_t ldw, void* C,
                         int c_dt, int64_t ldc, int64_t M, int64_t N, int64_t K, void* workspace,
                         size_t ws_bytes, void* stream) {
    const int st = check_gemm(A, lda, W, ldw, C, c_dt, ldc, M, N, K);
    if (st != BINV_OK || M == 0 || N == 0) return st;
    const size_t need = binv::gemm_tuned_workspace_bytes(M, N, K);
    if (need > 0 && (!workspace || ws_bytes < need || !aligned16(workspace)))
        return BINV_ERR_WORKSPACE;
    return status_of(binv::launch_gemm_tuned(A, lda, W, ldw, C, c_dt == BINV_F32, ldc, (int)M,
                                             (int)N, (int)K, workspace, (hipStream_t)stream));
}

size_t binv_attn_workspace_bytes(int64_t n_query_tokens, int Hq, int D, int64_t max_kv_len) {
    if (n_query_tokens <= 0 || Hq <= 0 || D <= 0 || max_kv_len <= 0) return 0;
    return binv::attn_workspace_bytes(n_query_tokens, Hq, D, max_kv_len);
}

size_t binv_attn_prefill_workspace_bytes(int64_t B, int64_t T, int64_t max_q_len,
                                         int64_t max_kv_len, int Hq, int Hkv, int D) {
    if (B <= 0 || T <= 0 || max_q_len <= 0 || max_kv_len <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 ||
        Hq % Hkv != 0)
        return 0;
    return binv::attn_prefill_workspace_bytes(B, T, max_q_len, max_kv_len, Hq, Hkv, D);
}

int binv_attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* page_table, int64_t pt_stride, const int32_t* kv_lens,
                           void* out, int64_t B, int64_t max_kv_len, int Hq, int Hkv, int D,
                           int page_size, float scale, void* workspace, size_t ws_bytes,
                           void* stream) {
    if (B < 0) return BINV_ERR_INVALID_ARG;
    if (B == 0) return BINV_OK;
    int st = check_attn_common(k_cache, v_cache, page_table, pt_stride, kv_lens, B, max_kv_len,
                               Hq, Hkv, D, page_size, scale);
    if (st != BINV_OK) return st;
    if (!q || !out || !aligned16(q) || !aligned16(out)) return BINV_ERR_INVALID_ARG;
    const size_t need = binv::attn_workspace_bytes(B, Hq, D, max_kv_len);
    if (!workspace || ws_bytes < need || !aligned16(workspace)) return BINV_ERR_WORKSPACE;
    binv::AttnArgs a{q, nullptr, k_cache, v_cache, page_table, pt_stride, kv_lens, out, B, B, 1,
                     max_kv_len, Hq, Hkv, D, (float)((double)scale * 1.4426950408889634),
                     (float*)workspace};
    return status_of(binv::launch_attention(a, (hipStream_t)stream));
}

int binv_attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* page_table, int64_t pt_stride,
                                   const int32_t* kv_lens, void* out, int64_t B,
                                   int64_t max_kv_len, int Hq, int Hkv, int D, int page_size,
                                   float scale, void* stream) {
    if (B < 0) return BINV_ERR_INVALID_ARG;
    if (B == 0) return BINV_OK;
    int st = check_attn_common(k_cache, v_cache, page_table, pt_stride, kv_lens, B, max_kv_len,
                               Hq, Hkv, D, page_size, scale);
    if (st != BINV_OK) return st;
    if (!q || !out || !aligned16(q) || !aligned16(out)) return BINV_ERR_INVALID_ARG;
    if (binv::attn_workspace_bytes(B, Hq, D, max_kv_len) > BINV_NOALLOC_SCRATCH_BYTES)
        return BINV_ERR_SCRATCH;
    void* ws = nullptr;
    if (binv::noalloc_scratch(&ws) != hipSuccess) return BINV_ERR_LAUNCH;
    binv::AttnArgs a{q, nullptr, k_cache, v_cache, page_table, pt_stride, kv_lens, out, B, B, 1,
                     max_kv_len, Hq, Hkv, D, (float)((double)scale * 1.4426950408889634),
                     (float*)ws};
    return status_of(binv::launch_attention(a, (hipStream_t)stream));
}

int binv_attn_prefill_paged(const void* q, const int32_t* cu_q, const void* k_cache,
                            const void* v_cache, const int32_t* page_table, int64_t pt_stride,
                            const int32_t* kv_lens, void* out, int64_t B, int64_t T,
                            int64_t max_q_len, int64_t max_kv_len, int Hq, int Hkv, int D,
                            int page_size, float scale, void* workspace, size_t ws_bytes,
                            void* stream) {
    if (B < 0 || T < 0 || max_q_len < 0) return BINV_ERR_INVALID_ARG;
    if (B == 0 || T == 0) return BINV_OK;
    int st = check_attn_common(k_cache, v_cache, page_table, pt_stride, kv_lens, B, max_kv_len,
                               Hq, Hkv, D, page_size, scale);
    if (st != BINV_OK) return st;
    if (!q || !out || !cu_q || !aligned16(q) || !aligned16(out)) return BINV_ERR_INVALID_ARG;
    if (max_q_len < 1 || max_q_len > max_kv_len) return BINV_ERR_INVALID_ARG;
    if (T > I32MAX) return BINV_ERR_UNSUPPORTED;
    const int G = Hq / Hkv;
    const int64_t nqt = (max_q_len + 16 / G - 1) / (16 / G);
    if (nqt * Hkv > I32MAX) return BINV_ERR_UNSUPPORTED;
    const size_t need = binv::attn_prefill_workspace_bytes(B, T, max_q_len, max_kv_len, Hq, Hkv, D);
    if (!workspace || ws_bytes < need || !aligned16(workspace)) return BINV_ERR_WORKSPACE;
    binv::AttnArgs a{q, cu_q, k_cache, v_cache, page_table, pt_stride, kv_lens, out, B, T,
                     max_q_len, max_kv_len, Hq, Hkv, D,
                     (float)((double)scale * 1.4426950408889634), (float*)workspace};
    return status_of(binv::launch_attention(a, (hipStream_t)stream));
}

size_t binv_attn_decode_tuned_workspace_bytes(int64_t B, int Hq, int D, int64_t max_kv_len) {
    if (B <= 0 || Hq <= 0 || D <= 0 || max_kv_len <= 0) return 0;
    return binv::attn_tuned_workspace_bytes(B, Hq, D, max_kv_len);
}

int binv_attn_decode_paged_tuned(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* page_table, int64_t pt_stride,
                                 const int32_t* kv_lens, void* out, int64_t B, int64_t max_kv_len,
                                 int Hq, int Hkv, int D, int page_size, float scale,
                                 void* workspace, size_t ws_bytes, void* stream) {
    if (B < 0) return BINV_ERR_INVALID_ARG;
    if (B == 0) return BINV_OK;
    int st = check_attn_common(k_cache, v_cache, page_table, pt_stride, kv_lens, B, max_kv_len,
                               Hq, Hkv, D, page_size, scale);
    if (st != BINV_OK) return st;
    if (!q || !out || !aligned16(q) || !aligned16(out)) return BINV_ERR_INVALID_ARG;
    const size_t need = binv::attn_tuned_workspace_bytes(B, Hq, D, max_kv_len);
    if (!workspace || ws_bytes < need || !aligned16(workspace)) return BINV_ERR_WORKSPACE;
    binv::AttnArgs a{q, nullptr, k_cache, v_cache, page_table, pt_stride, kv_lens, out, B, B, 1,
                     max_kv_len, Hq, Hkv, D, (float)((double)scale * 1.4426950408889634),
                     (float*)workspace};
    return status_of(binv::launch_attention_decode_tuned(a, (hipStream_t)stream));
}

// ---------------------------------------------------------------- decoder glue

int binv_embed(const int32_t* ids, int64_t T, const void* table, int64_t V, int64_t H,
               float* out, void* stream) {
    if (T < 0 || V <= 0 || H <= 0) return BINV_ERR_INVALID_ARG;
    if (T == 0) return BINV_OK;
    if (!ids || !table || !out) return BINV_ERR_INVALID_ARG;
    if (!aligned16(table) || !aligned16(out)) return BINV_ERR_INVALID_ARG;
    if (H % 8 != 0) return BINV_ERR_UNSUPPORTED;
    if (T > I32MAX || H > I32MAX) return BINV_ERR_UNSUPPORTED;
    return status_of(binv::launch_embed(ids, table, V, (int)H, T, out, (hipStream_t)stream));
}

int binv_rope_kv_write(const void* qkv, int64_t ld_qkv, const int32_t* tok_seq,
                       const int32_t* tok_pos, int64_t T, int Hq, int Hkv, int D, double theta,
                       void* q_out, void* k_cache, void* v_cache, const int32_t* page_table,
                       int64_t pt_stride, int page_size, void* stream) {
    if (T < 0) return BINV_ERR_INVALID_ARG;
    if (T == 0) return BINV_OK;
    if (!qkv || !tok_seq || !tok_pos || !q_out || !k_cache || !v_cache || !page_table)
        return BINV_ERR_INVALID_ARG;
    if (Hq <= 0 || Hkv <= 0 || pt_stride <= 0 || !(theta > 1.0) || !isfinite(theta))
        return BINV_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return BINV_ERR_UNSUPPORTED;
    if (page_size != BINV_PAGE_SIZE) return BINV_ERR_UNSUPPORTED;
    if (ld_qkv < (int64_t)(Hq + 2 * Hkv) * D) return BINV_ERR_INVALID_ARG;
    if (T > I32MAX) return BINV_ERR_UNSUPPORTED;
    return status_of(binv::launch_rope_kv(qkv, ld_qkv, tok_seq, tok_pos, T, Hq, Hkv, D, theta,
                                          q_out, k_cache, v_cache, page_table, pt_stride,
                                          (hipStream_t)stream));
}

int binv_swiglu(const void* gate_up, int64_t ld_gu, int64_t T, int64_t F, void* out,
                int64_t ld_out, void* stream) {
    if (T < 0 || F < 0) return BINV_ERR_INVALID_ARG;
    if (T == 0 || F == 0) return BINV_OK;
    if (!gate_up || !out || ld_gu < 2 * F || ld_out < F) return BINV_ERR_INVALID_ARG;
    if (!aligned16(gate_up) || !aligned16(out) || ld_gu % 8 || ld_out % 8) return BINV_ERR_INVALID_ARG;
    if (F % 8 != 0) return BINV_ERR_UNSUPPORTED;
    if (T > 65535 || F > I32MAX) return BINV_ERR_UNSUPPORTED;
    return status_of(binv::launch_swiglu(gate_up, ld_gu, T, (int)F, out, ld_out,
                                         (hipStream_t)stream));
}

int binv_residual_add(float* h, int64_t ldh, const void* x, int64_t ldx, int64_t T, int64_t H,
                      void* stream) {
    if (T < 0 || H < 0) return BINV_ERR_INVALID_ARG;
    if (T == 0 || H == 0) return BINV_OK;
    if (!h || !x || ldh < H || ldx < H) return BINV_ERR_INVALID_ARG;
    if (!aligned16(h) || (reinterpret_cast<uintptr_t>(x) & 7u) || ldh % 4 || ldx % 4)
        return BINV_ERR_INVALID_ARG;
    if (H % 4 != 0) return BINV_ERR_UNSUPPORTED;
    if (T > 65535 || H > I32MAX) return BINV_ERR_UNSUPPORTED;
    return status_of(binv::launch_add(h, ldh, x, ldx, T, (int)H, (hipStream_t)stream));
}

int binv_gather_rows(const void* src, int dt, int64_t lds, const int32_t* idx, int64_t R,
                     void* dst, int64_t ldd, int64_t cols, void* stream) {
    if (R < 0 || cols < 0 || !valid_dt(dt)) return BINV_ERR_INVALID_ARG;
    if (R == 0 || cols == 0) return BINV_OK;
    if (!src || !idx || !dst || lds < cols || ldd < cols) return BINV_ERR_INVALID_ARG;
    const int es = elem_size(dt);
    if ((cols * es) % 4 != 0 || (lds * es) % 4 != 0 || (ldd * es) % 4 != 0 ||
        (reinterpret_cast<uintptr_t>(src) & 3u) || (reinterpret_cast<uintptr_t>(dst) & 3u))
        return BINV_ERR_INVALID_ARG;
    if (R > I32MAX || cols * es > I32MAX) return BINV_ERR_UNSUPPORTED;
    return status_of(binv::launch_gather(src, lds * es, idx, R, dst, ldd * es, (int)(cols * es),
                                         (hipStream_t)stream));
}

int binv_split_bf16x3(const float* x, int64_t ldx, int64_t M, int64_t K, void* out,
                      int64_t ld_out, void* stream) {
    if (M < 0 || K < 0) return BINV_ERR_INVALID_ARG;
    if (M == 0 || K == 0) return BINV_OK;
    if (!x || !out || ldx < K || ld_out < 3 * K) return BINV_ERR_INVALID_ARG;
    if (!aligned16(x) || (reinterpret_cast<uintptr_t>(out) & 7u) || ldx % 4 || ld_out % 4)
        return BINV_ERR_INVALID_ARG;
    if (K % 4 != 0) return BINV_ERR_UNSUPPORTED;
    if (M > 65535 || 3 * K > I32MAX) return BINV_ERR_UNSUPPORTED;
    return status_of(binv::launch_split3(x, ldx, M, (int)K, out, ld_out, (hipStream_t)stream));
}

int binv_topk(const float* x, int64_t ldx, int64_t R, int64_t n, int K, int32_t* ids,
              float* vals, void* stream) {
    if (R < 0 || n < 0 || K < 1) return BINV_ERR_INVALID_ARG;
    if (K > 32) return BINV_ERR_UNSUPPORTED;
    if (R == 0) return BINV_OK;
    if (!x || !ids || !vals || ldx < n) return BINV_ERR_INVALID_ARG;
    if (R > I32MAX || n > I32MAX) return BINV_ERR_UNSUPPORTED;
    return status_of(binv::launch_topk(x, ldx, R, n, K, ids, vals, (hipStream_t)stream));
}

}  // extern "C"
