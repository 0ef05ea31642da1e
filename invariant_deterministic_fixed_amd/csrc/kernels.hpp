// kernels.hpp -- host-side launchers implemented in the .hip files.  Arguments
// are already validated by abi.cpp; each launcher returns hipSuccess or the
// launch error.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace binv {

hipError_t launch_rmsnorm(const void* x, int x_bf16, int64_t ldx, const void* g, int g_bf16,
                          void* y, int y_bf16, int64_t ldy, int64_t M, int d, float eps,
                          hipStream_t s);
hipError_t launch_add_rmsnorm(float* h, int64_t ldh, const void* a, int64_t lda, const void* g,
                              int g_bf16, void* y, int y_bf16, int64_t ldy, int64_t M, int d,
                              float eps, hipStream_t s);
hipError_t launch_rmsnorm_tuned(const void* x, int x_bf16, int64_t ldx, const void* g, int g_bf16,
                                void* y, int y_bf16, int64_t ldy, int64_t M, int d, float eps,
                                hipStream_t s);

hipError_t launch_gemm(const void* A, int64_t lda, const void* W, int64_t ldw, void* C,
                       int c_f32, int64_t ldc, int M, int N, int K, hipStream_t s);
size_t gemm_packed_bytes(int64_t N, int64_t K);
hipError_t launch_gemm_pack(const void* W, int64_t ldw, int K, int N, void* Wp, hipStream_t s);
hipError_t launch_gemm_packed(const void* A, int64_t lda, const void* Wp, void* C, int c_f32,
                              int64_t ldc, int M, int N, int K, hipStream_t s);
hipError_t launch_gemm_strips_packed(const void* A, int64_t lda, const void* Wp, void* C,
                                     int c_f32, int64_t ldc, int M, int N, int K, hipStream_t s);
size_t gemm_tuned_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_tuned(const void* A, int64_t lda, const void* W, int64_t ldw, void* C,
                             int c_f32, int64_t ldc, int M, int N, int K, void* ws,
                             hipStream_t s);

struct AttnArgs {
    const void* q;             // bf16 [n_tokens, Hq, D]
    const int32_t* cu_q;       // prefill: [B+1]; decode: nullptr (one token per sequence)
    const void* k_cache;
    const void* v_cache;
    const int32_t* page_table;
    int64_t pt_stride;
    const int32_t* kv_lens;
    void* out;                 // bf16 [n_tokens, Hq, D]
    int64_t B;
    int64_t n_tokens;          // decode: B; prefill: T
    int64_t max_q_len;         // decode: 1
    int64_t max_kv_len;
    int Hq, Hkv, D;
    float scale_log2;          // scale * log2(e), formed once on the host
    float* ws;                 // fp32 partials
};

size_t attn_workspace_bytes(int64_t n_tokens, int Hq, int D, int64_t max_kv_len);
size_t attn_prefill_workspace_bytes(int64_t B, int64_t T, int64_t max_q_len, int64_t max_kv_len,
                                    int Hq, int Hkv, int D);
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);
// device address of this device's fixed no-alloc partials buffer
// (BINV_NOALLOC_SCRATCH_BYTES), looked up on the first call per device
hipError_t noalloc_scratch(void** ptr);
size_t attn_tuned_workspace_bytes(int64_t B, int Hq, int D, int64_t max_kv_len);
hipError_t launch_attention_decode_tuned(const AttnArgs& a, hipStream_t s);

hipError_t launch_embed(const int32_t* ids, const void* table, int64_t V, int H, int64_t T,
                        float* out, hipStream_t s);
hipError_t launch_rope_kv(const void* qkv, int64_t ld, const int32_t* tok_seq,
                          const int32_t* tok_pos, int64_t T, int Hq, int Hkv, int D, double theta,
                          void* q_out, void* k_cache, void* v_cache, const int32_t* page_table,
                          int64_t pt_stride, hipStream_t s);
hipError_t launch_swiglu(const void* gu, int64_t ld, int64_t T, int F, void* out, int64_t ldo,
                         hipStream_t s);
hipError_t launch_add(float* h, int64_t ldh, const void* x, int64_t ldx, int64_t T, int H,
                      hipStream_t s);
hipError_t launch_gather(const void* src, int64_t lds, const int32_t* idx, int64_t R, void* dst,
                         int64_t ldd, int row_bytes, hipStream_t s);
hipError_t launch_topk(const float* x, int64_t ldx, int64_t R, int64_t n, int K, int32_t* ids,
                       float* vals, hipStream_t s);
hipError_t launch_split3(const float* x, int64_t ldx, int64_t M, int K, void* out, int64_t ldo,
                         hipStream_t s);

}  // namespace binv
