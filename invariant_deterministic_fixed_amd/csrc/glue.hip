// glue.hip -- the pointwise and selection steps of a decoder layer (gfx950).
//
// The pages note that pointwise operations act on each element alone and are
// batch-invariant as they stand (devpress.csdn.net explainer of "Defeating
// Nondeterminism in LLM Inference", section 3: ReLU, add, multiply and the
// scaling inside norms need no change), and that greedy decoding is exactly
// an argmax whose ties must be broken the same way every time (paper.xwysyy.cn
// "19.7 推理非确定性分析", section 19.7.4 tie-breaking; zhaixingw.cn BlockLock
// post: identical target tokens and top-20 logits are the acceptance test).
// Every kernel here computes each output element from its own inputs with a
// fixed instruction sequence; the selection is exact (comparisons only).
#include "common.hpp"
#include "kernels.hpp"

namespace binv {

namespace {

// ------------------------------------------------------------------ embedding
// out[t, :] = float(table[ids[t], :]); ids outside [0, V) give zeros.
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ ids,
                                                    const bf16_t* __restrict__ table, int64_t V,
                                                    int H, float* __restrict__ out) {
    const int64_t t = blockIdx.x;
    const int32_t id = ids[t];
    const bool ok = id >= 0 && id < V;
    const bf16_t* row = table + (ok ? (int64_t)id : 0) * H;
    float* o = out + t * H;
    for (int j = threadIdx.x; j < H; j += 256) o[j] = ok ? bf16_to_f32(row[j]) : 0.0f;
}

// ------------------------------------------------------------------ RoPE + KV write
// Rotate-half rotary embedding on the q and k heads of one token's fused
// projection row, then the rotated q goes to q_out and k, v go to the paged
// cache at the token's position.
//   angle(p, i) = p * theta^(-2i/D) for i < D/2, evaluated in fp64
//   x'[i]       = x[i] cos - x[i + D/2] sin
//   x'[i + D/2] = x[i + D/2] cos + x[i] sin     (fp32, rounded once to bf16)
// One workgroup per token; lane j handles the pair (i, i + D/2) of one head.
__global__ __launch_bounds__(256) void rope_kv_kernel(
    const bf16_t* __restrict__ qkv, int64_t ld, const int32_t* __restrict__ tok_seq,
    const int32_t* __restrict__ tok_pos, int Hq, int Hkv, int D, double theta,
    bf16_t* __restrict__ q_out, bf16_t* __restrict__ k_cache, bf16_t* __restrict__ v_cache,
    const int32_t* __restrict__ page_table, int64_t pt_stride) {
    const int64_t t = blockIdx.x;
    const int pos = tok_pos[t];
    const int seq = tok_seq[t];
    const int half = D / 2;
    const bf16_t* row = qkv + t * ld;
    const int64_t page = page_table[(int64_t)seq * pt_stride + pos / 16];
    const int slot = pos % 16;
    // q and k heads: Hq + Hkv heads of D features, pairs (i, i + D/2); lane
    // handles frequency i = lane % (D/2) for every (256 / (D/2))-th head
    const int i = threadIdx.x % half;
    const int nh = 256 / half;
    const double inv = pow(theta, -2.0 * (double)i / (double)D);
    const double ang = (double)pos * inv;
    const float cs = (float)cos(ang), sn = (float)sin(ang);
    for (int h = threadIdx.x / half; h < Hq + Hkv; h += nh) {
        const float x1 = bf16_to_f32(row[h * D + i]);
        const float x2 = bf16_to_f32(row[h * D + i + half]);
        const bf16_t y1 = (bf16_t)f32_to_bf16(x1 * cs - x2 * sn);
        const bf16_t y2 = (bf16_t)f32_to_bf16(x2 * cs + x1 * sn);
        if (h < Hq) {
            q_out[(t * Hq + h) * D + i] = y1;
            q_out[(t * Hq + h) * D + i + half] = y2;
        } else {
            const int g = h - Hq;
            bf16_t* kp = k_cache + ((page * Hkv + g) * 16 + slot) * D;     // [page][g][slot][d]
            kp[i] = y1;
            kp[i + half] = y2;
        }
    }
    // v heads: copied as they are, feature-major inside the page
    for (int w = threadIdx.x; w < Hkv * D; w += 256) {
        const int g = w / D, d = w % D;
        v_cache[((page * Hkv + g) * D + d) * 16 + slot] = row[(Hq + Hkv) * D + g * D + d];
    }
}

// ------------------------------------------------------------------ SwiGLU
// out[t, j] = bf16( silu(g) * u ),  g = gu[t, j], u = gu[t, F + j],
// silu(g) = g / (1 + exp(-g)), fp32.
__global__ __launch_bounds__(256) void swiglu_kernel(const bf16_t* __restrict__ gu, int64_t ld,
                                                     int F, bf16_t* __restrict__ out,
                                                     int64_t ldo) {
    const int64_t t = blockIdx.y;
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= F) return;
    const float g = bf16_to_f32(gu[t * ld + j]);
    const float u = bf16_to_f32(gu[t * ld + F + j]);
    const float s = g / (1.0f + expf(-g));
    out[t * ldo + j] = (bf16_t)f32_to_bf16(s * u);
}

// ------------------------------------------------------------------ residual add
// h[t, j] += float(x[t, j])  (fp32 residual stream)
__global__ __launch_bounds__(256) void add_kernel(float* __restrict__ h, int64_t ldh,
                                                  const bf16_t* __restrict__ x, int64_t ldx,
                                                  int H) {
    const int64_t t = blockIdx.y;
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= H) return;
    h[t * ldh + j] += bf16_to_f32(x[t * ldx + j]);
}

// ------------------------------------------------------------------ row gather
// dst[r, :] = src[idx[r], :]  (bf16 or fp32 rows, copied bit for bit)
__global__ __launch_bounds__(256) void gather_kernel(const char* __restrict__ src, int64_t lds,
                                                     const int32_t* __restrict__ idx,
                                                     char* __restrict__ dst, int64_t ldd,
                                                     int row_bytes) {
    const int64_t r = blockIdx.x;
    const char* s = src + (int64_t)idx[r] * lds;
    char* d = dst + r * ldd;
    for (int j = threadIdx.x * 4; j < row_bytes; j += 1024)
        *reinterpret_cast<uint32_t*>(d + j) = *reinterpret_cast<const uint32_t*>(s + j);
}

// ------------------------------------------------------------------ top-k
// Exact top-K of one fp32 row: the K largest values, sorted by value
// descending and, among equal values, by index ascending.  One workgroup per
// row; each lane keeps its own sorted top-K over a strided slice, then the
// workgroup takes K rounds of "best remaining candidate" over the lanes' lists.
constexpr int TOPK_MAX = 32;
constexpr int TOPK_NT = 256;

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(TOPK_NT) void topk_kernel(const float* __restrict__ x, int64_t ldx,
                                                       int64_t n, int K,
                                                       int32_t* __restrict__ ids,
                                                       float* __restrict__ vals) {
    __shared__ float cv[TOPK_NT * TOPK_MAX];
    __shared__ int ci[TOPK_NT * TOPK_MAX];
    __shared__ int head[TOPK_NT];
    __shared__ float wv[TOPK_NT / 64];
    __shared__ int wi[TOPK_NT / 64], wl[TOPK_NT / 64];
    const int64_t r = blockIdx.x;
    const float* row = x + r * ldx;
    const int t = threadIdx.x;
    float lv[TOPK_MAX];
    int li[TOPK_MAX];
    int cnt = 0;
    for (int64_t j = t; j < n; j += TOPK_NT) {
        const float v = row[j];
        const int idx = (int)j;
        if (v != v) continue;                          // NaN never selected
        if (cnt == K && !better(v, idx, lv[K - 1], li[K - 1])) continue;
        // insertion into the lane's sorted list (indices arrive ascending)
        int p = (cnt < K) ? cnt++ : K - 1;
        while (p > 0 && better(v, idx, lv[p - 1], li[p - 1])) {
            lv[p] = lv[p - 1]; li[p] = li[p - 1]; --p;
        }
        lv[p] = v; li[p] = idx;
    }
    for (int k = 0; k < K; ++k) {
        cv[t * TOPK_MAX + k] = k < cnt ? lv[k] : -INFINITY;
        ci[t * TOPK_MAX + k] = k < cnt ? li[k] : 0x7fffffff;
    }
    head[t] = 0;
    __syncthreads();
    for (int k = 0; k < K; ++k) {
        // best head among the lanes' lists
        const int hd = head[t];
        float v = hd < K ? cv[t * TOPK_MAX + hd] : -INFINITY;
        int i = hd < K ? ci[t * TOPK_MAX + hd] : 0x7fffffff;
        int lane_of = t;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(v, off);
            const int oi = __shfl_xor(i, off);
            const int ol = __shfl_xor(lane_of, off);
            if (better(ov, oi, v, i)) { v = ov; i = oi; lane_of = ol; }
        }
        if ((t & 63) == 0) { wv[t >> 6] = v; wi[t >> 6] = i; wl[t >> 6] = lane_of; }
        __syncthreads();
        if (t == 0) {
            float bv = wv[0]; int bi = wi[0], bl = wl[0];
            for (int w = 1; w < TOPK_NT / 64; ++w)
                if (better(wv[w], wi[w], bv, bi)) { bv = wv[w]; bi = wi[w]; bl = wl[w]; }
            ids[r * K + k] = bi == 0x7fffffff ? -1 : bi;
            vals[r * K + k] = bv;
            head[bl] += 1;
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_embed(const int32_t* ids, const void* table, int64_t V, int H, int64_t T,
                        float* out, hipStream_t s) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(embed_kernel, dim3((unsigned)T), dim3(256), 0, s, ids,
                       (const bf16_t*)table, V, H, out);
    return hipGetLastError();
}

hipError_t launch_rope_kv(const void* qkv, int64_t ld, const int32_t* tok_seq,
                          const int32_t* tok_pos, int64_t T, int Hq, int Hkv, int D, double theta,
                          void* q_out, void* k_cache, void* v_cache, const int32_t* page_table,
                          int64_t pt_stride, hipStream_t s) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(rope_kv_kernel, dim3((unsigned)T), dim3(256), 0, s, (const bf16_t*)qkv, ld,
                       tok_seq, tok_pos, Hq, Hkv, D, theta, (bf16_t*)q_out, (bf16_t*)k_cache,
                       (bf16_t*)v_cache, page_table, pt_stride);
    return hipGetLastError();
}

hipError_t launch_swiglu(const void* gu, int64_t ld, int64_t T, int F, void* out, int64_t ldo,
                         hipStream_t s) {
    if (T == 0 || F == 0) return hipSuccess;
    hipLaunchKernelGGL(swiglu_kernel, dim3((unsigned)((F + 255) / 256), (unsigned)T), dim3(256), 0,
                       s, (const bf16_t*)gu, ld, F, (bf16_t*)out, ldo);
    return hipGetLastError();
}

hipError_t launch_add(float* h, int64_t ldh, const void* x, int64_t ldx, int64_t T, int H,
                      hipStream_t s) {
    if (T == 0 || H == 0) return hipSuccess;
    hipLaunchKernelGGL(add_kernel, dim3((unsigned)((H + 255) / 256), (unsigned)T), dim3(256), 0, s,
                       h, ldh, (const bf16_t*)x, ldx, H);
    return hipGetLastError();
}

hipError_t launch_gather(const void* src, int64_t lds, const int32_t* idx, int64_t R, void* dst,
                         int64_t ldd, int row_bytes, hipStream_t s) {
    if (R == 0) return hipSuccess;
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)R), dim3(256), 0, s, (const char*)src, lds,
                       idx, (char*)dst, ldd, row_bytes);
    return hipGetLastError();
}

hipError_t launch_topk(const float* x, int64_t ldx, int64_t R, int64_t n, int K, int32_t* ids,
                       float* vals, hipStream_t s) {
    if (R == 0) return hipSuccess;
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)R), dim3(TOPK_NT), 0, s, x, ldx, n, K, ids,
                       vals);
    return hipGetLastError();
}

}  // namespace binv
