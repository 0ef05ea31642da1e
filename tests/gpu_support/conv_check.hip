// conv_check.hip -- test-only kernel: the two fp32 -> bf16 conversions of the
// library over every one of the 2^32 fp32 bit patterns.
//
// f32_to_bf16 (csrc/common.hpp, one value) is how the GEMM, RMSNorm, the glue
// and the attention outputs round; p_pack (csrc/attn_chunk.hpp, a pair, gfx950's
// v_cvt_pk_bf16_f32) is how every attention kernel rounds its softmax weights.
// Both must be round to nearest even on every input -- the rounding the oracle
// applies -- and the pair's two halves must agree.  Each is compared with the
// rule written out here from the format's definition:
//   NaN (exponent all ones, mantissa != 0) -> top 16 bits with the quiet bit set;
//   otherwise add 0x7fff plus the lowest kept bit, keep the top 16 bits.
// Built into its own library by the package build; never linked into libbinv.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../invariant_deterministic_fixed_amd/csrc/attn_chunk.hpp"

namespace {

__device__ __forceinline__ uint32_t spec_bf16(uint32_t u) {
    const uint32_t e = (u >> 23) & 0xffu, m = u & 0x7fffffu;
    if (e == 0xffu && m != 0u) return ((u >> 16) | 0x40u) & 0xffffu;
    const uint64_t r = (uint64_t)u + 0x7fffu + ((u >> 16) & 1u);
    return (uint32_t)(r >> 16) & 0xffffu;
}

constexpr int THREADS = 256;
constexpr int PER_THREAD = 256;          // 2^32 = 65536 blocks x 256 threads x 256

// counts[3 * block + k]: mismatches of (pair low half vs scalar, scalar vs
// spec, pair high half vs spec) among the block's 65536 inputs; first[block]:
// the lowest input of the block where any of them differ (0xffffffff if none)
__global__ __launch_bounds__(THREADS) void conv_check_kernel(uint32_t* counts, uint32_t* first) {
    __shared__ uint32_t c_hw_br[THREADS], c_hw_sp[THREADS], c_br_sp[THREADS], f_min[THREADS];
    const uint32_t base = (uint32_t)blockIdx.x * (THREADS * PER_THREAD);
    uint32_t a = 0, b = 0, c = 0, fm = 0xffffffffu;
    for (int i = 0; i < PER_THREAD; ++i) {
        const uint32_t u = base + (uint32_t)i * THREADS + threadIdx.x;
        const float f = __uint_as_float(u);
        const uint32_t hw = binv::f32_to_bf16(f) & 0xffffu;
        const uint32_t pk = binv::attn::p_pack(f, f);
        const uint32_t sp = spec_bf16(u);
        const bool d1 = (pk & 0xffffu) != hw, d2 = hw != sp, d3 = (pk >> 16) != sp;
        a += d1; b += d2; c += d3;
        if ((d1 || d2 || d3) && u < fm) fm = u;
    }
    c_hw_br[threadIdx.x] = a; c_hw_sp[threadIdx.x] = b; c_br_sp[threadIdx.x] = c;
    f_min[threadIdx.x] = fm;
    __syncthreads();
    for (int s = THREADS / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) {
            c_hw_br[threadIdx.x] += c_hw_br[threadIdx.x + s];
            c_hw_sp[threadIdx.x] += c_hw_sp[threadIdx.x + s];
            c_br_sp[threadIdx.x] += c_br_sp[threadIdx.x + s];
            f_min[threadIdx.x] = min(f_min[threadIdx.x], f_min[threadIdx.x + s]);
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        counts[3 * blockIdx.x + 0] = c_hw_br[0];
        counts[3 * blockIdx.x + 1] = c_hw_sp[0];
        counts[3 * blockIdx.x + 2] = c_br_sp[0];
        first[blockIdx.x] = f_min[0];
    }
}

}  // namespace

// counts: device uint32 [3 * 65536]; first: device uint32 [65536]
extern "C" int conv_check_all_inputs(uint32_t* counts, uint32_t* first, void* stream) {
    if (!counts || !first) return 1;
    hipLaunchKernelGGL(conv_check_kernel, dim3(65536), dim3(THREADS), 0, (hipStream_t)stream,
                       counts, first);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}
