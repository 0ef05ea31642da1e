// gemm_packed.hip -- packing of weights for the invariant GEMM of decode
// batches (M <= 64), and its entry (gfx950).
//
// Method: devpress.csdn.net explainer of "Defeating Nondeterminism in LLM
// Inference", section 3.2 Matmul, and tom-jerr.github.io "Batch-Invariant
// Kernel", section GEMM: every output element is reduced in one fixed order
// whatever the batch size.  The products over packed weights run the strip
// kernel of gemm.hip, with its per-element chain: one fp32 accumulator fed by
// v_mfma_f32_16x16x32_bf16 over the 32-wide k-blocks in ascending order, K
// zero-padded to a multiple of 64 (padding blocks included), the A fragment
// as the first operand and the W fragment as the second.  So C has the bits
// of binv_gemm_bf16 for the same A and W; only where W comes from differs.
//
// Why a second layout: at decode sizes a GEMM is a stream of the weights, and
// a strip of 16 output columns of a row-major [K, N] W is 32 bytes out of every
// 2N-byte row -- at N = 4096 each strip touches every 8 KB row of the matrix,
// which the memory system serves at a fraction of its streaming rate.  Packed,
// a strip's weights are one contiguous run:
//   Wp[s][kb][c][kk] = W[32 kb + kk][16 s + c]   (0 past K or N)
// s the strip, kb the k-block (2 ceil(K / 64) of them), c the column in the
// strip, kk the k in the block: 1 KB per (strip, k-block), one DMA of a wave,
// and the 16 bytes lane (g, r) needs as MFMA B operand (column r, k 8g ..
// 8g + 7) sit at r * 64 + g * 16 in it.  The pack is a one-off per weight
// (a product's M never reaches it).
#include "binv.h"
#include "common.hpp"
#include "kernels.hpp"

namespace binv {

namespace {

__device__ __forceinline__ int packed_kblocks(int K) { return 2 * ((K + 63) / 64); }

// one thread per 16-byte piece (s, kb, c, g) of Wp
__global__ __launch_bounds__(256) void gemm_pack_kernel(const bf16_t* __restrict__ W, int64_t ldw,
                                                        int K, int N, bf16_t* __restrict__ Wp,
                                                        int64_t pieces) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= pieces) return;
    const int nkb = packed_kblocks(K);
    const int g = (int)(i & 3), c = (int)((i >> 2) & 15);
    const int64_t sb = i >> 6;
    const int kb = (int)(sb % nkb);
    const int64_t s = sb / nkb;
    const int64_t col = 16 * s + c;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int k0 = 32 * kb + 8 * g + 2 * e;
        const uint32_t lo = (k0 < K && col < N) ? (uint32_t)W[(int64_t)k0 * ldw + col] : 0u;
        const uint32_t hi = (k0 + 1 < K && col < N) ? (uint32_t)W[(int64_t)(k0 + 1) * ldw + col] : 0u;
        w[e] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4*>(Wp + i * 8) = u32x4{w[0], w[1], w[2], w[3]};
}

}  // namespace

size_t gemm_packed_bytes(int64_t N, int64_t K) {
    const int64_t nkb = 2 * ((K + 63) / 64);
    return (size_t)((N + 15) / 16) * nkb * 1024;
}

hipError_t launch_gemm_pack(const void* W, int64_t ldw, int K, int N, void* Wp, hipStream_t s) {
    const int64_t pieces = (int64_t)gemm_packed_bytes(N, K) / 16;
    if (pieces == 0) return hipSuccess;
    hipLaunchKernelGGL(gemm_pack_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s,
                       (const bf16_t*)W, ldw, K, N, (bf16_t*)Wp, pieces);
    return hipGetLastError();
}

hipError_t launch_gemm_packed(const void* A, int64_t lda, const void* Wp, void* C, int c_f32,
                              int64_t ldc, int M, int N, int K, hipStream_t s) {
    return launch_gemm_strips_packed(A, lda, Wp, C, c_f32, ldc, M, N, K, s);
}

}  // namespace binv
