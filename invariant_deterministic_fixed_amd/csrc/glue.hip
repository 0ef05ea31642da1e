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
// H % 8 == 0: each lane moves 8 elements (16 bytes in, 32 bytes out).
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ ids,
                                                    const bf16_t* __restrict__ table, int64_t V,
                                                    int H, float* __restrict__ out) {
    const int64_t t = blockIdx.x;
    const int32_t id = ids[t];
    const bool ok = id >= 0 && id < V;
    const bf16_t* row = table + (ok ? (int64_t)id : 0) * H;
    float* o = out + t * H;
    for (int j = threadIdx.x * 8; j < H; j += 256 * 8) {
        const u32x4 w = ok ? *reinterpret_cast<const u32x4*>(row + j) : u32x4{0u, 0u, 0u, 0u};
        u32x4 a, b;
        a[0] = w[0] << 16; a[1] = w[0] & 0xffff0000u; a[2] = w[1] << 16; a[3] = w[1] & 0xffff0000u;
        b[0] = w[2] << 16; b[1] = w[2] & 0xffff0000u; b[2] = w[3] << 16; b[3] = w[3] & 0xffff0000u;
        *reinterpret_cast<u32x4*>(o + j) = a;
        *reinterpret_cast<u32x4*>(o + j + 4) = b;
    }
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
// silu(g) = g / (1 + exp(-g)), fp32.  F % 8 == 0: 8 outputs per lane.
__global__ __launch_bounds__(256) void swiglu_kernel(const bf16_t* __restrict__ gu, int64_t ld,
                                                     int F, bf16_t* __restrict__ out,
                                                     int64_t ldo) {
    const int64_t t = blockIdx.y;
    const int j = (blockIdx.x * 256 + threadIdx.x) * 8;
    if (j >= F) return;
    const u32x4 gw = *reinterpret_cast<const u32x4*>(gu + t * ld + j);
    const u32x4 uw = *reinterpret_cast<const u32x4*>(gu + t * ld + F + j);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float g0 = lo_bf16(gw[i]), g1 = hi_bf16(gw[i]);
        const float u0 = lo_bf16(uw[i]), u1 = hi_bf16(uw[i]);
        const float s0 = g0 / (1.0f + expf(-g0)), s1 = g1 / (1.0f + expf(-g1));
        o[i] = pack_bf16x2(s0 * u0, s1 * u1);
    }
    *reinterpret_cast<u32x4*>(out + t * ldo + j) = o;
}

// ------------------------------------------------------------------ residual add
// h[t, j] += float(x[t, j])  (fp32 residual stream); H % 4 == 0: 4 per lane.
__global__ __launch_bounds__(256) void add_kernel(float* __restrict__ h, int64_t ldh,
                                                  const bf16_t* __restrict__ x, int64_t ldx,
                                                  int H) {
    const int64_t t = blockIdx.y;
    const int j = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (j >= H) return;
    float4* hp = reinterpret_cast<float4*>(h + t * ldh + j);
    const u32x2 xw = *reinterpret_cast<const u32x2*>(x + t * ldx + j);
    float4 v = *hp;
    v.x += lo_bf16(xw[0]); v.y += hi_bf16(xw[0]); v.z += lo_bf16(xw[1]); v.w += hi_bf16(xw[1]);
    *hp = v;
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
// descending and, among equal values, by index ascending; NaN never selected.
// One workgroup per row:
//   1. each value maps to an order-preserving 32-bit key (NaN -> 0, below every
//      other key); four 8-bit radix passes build histograms of the candidates'
//      next byte and walk them from the top, which pins down the exact key T of
//      the K-th largest entry and how many entries equal to T are needed.  The
//      histograms are integer counts (LDS increments), whose totals do not
//      depend on the order in which lanes add;
//   2. one pass in index order (1024-element tiles, ballots and wave prefix
//      counts) collects every entry with key > T and the lowest-index entries
//      with key == T;
//   3. the <= 32 winners are sorted by (value desc, index asc).
constexpr int TOPK_MAX = 32;
constexpr int TOPK_NT = 1024;
constexpr int TOPK_NW = TOPK_NT / 64;

__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t b = __float_as_uint(v);
    if (v != v) return 0u;
    if ((b & 0x7fffffffu) == 0u) b = 0u;                 // -0 and +0 are one value
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(TOPK_NT) void topk_kernel(const float* __restrict__ x, int64_t ldx,
                                                       int64_t n, int K,
                                                       int32_t* __restrict__ ids,
                                                       float* __restrict__ vals) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t s_prefix, s_need;
    __shared__ uint32_t w_gt[TOPK_NW], w_eq[TOPK_NW];
    __shared__ float sel_v[TOPK_MAX];
    __shared__ int sel_i[TOPK_MAX];
    const int64_t r = blockIdx.x;
    const float* row = x + r * ldx;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;

    // ---- 1. radix select of the K-th largest key
    uint32_t prefix = 0u, mask = 0u, need = (uint32_t)K;
    for (int shift = 24; shift >= 0; shift -= 8) {
        if (t < 256) hist[t] = 0u;
        __syncthreads();
        for (int64_t j = t; j < n; j += TOPK_NT) {
            const uint32_t key = order_key(row[j]);
            if (key != 0u && (key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (t == 0) {
            uint32_t cum = 0u, chosen = 0u, nd = need;
            bool found = false;
            for (int bkt = 255; bkt >= 0; --bkt) {
                const uint32_t h = hist[bkt];
                if (cum + h >= need) { chosen = (uint32_t)bkt; nd = need - cum; found = true; break; }
                cum += h;
            }
            // fewer than `need` candidates left: every valid entry is selected
            s_prefix = found ? (prefix | (chosen << shift)) : 0xffffffffu;
            s_need = found ? nd : 0u;
        }
        __syncthreads();
        if (s_prefix == 0xffffffffu) { prefix = 0u; need = 0u; break; }
        prefix = s_prefix;
        need = s_need;
        mask |= 255u << shift;
    }
    // T = prefix (key of the K-th entry) unless fewer than K valid entries exist
    const bool short_row = (need == 0u);
    const uint32_t T = short_row ? 1u : prefix;          // short row: take every key >= 1
    const uint32_t n_eq_take = short_row ? (uint32_t)K : need;

    // ---- 2. collect winners in index order
    uint32_t run_gt = 0u, run_eq = 0u;
    const uint32_t base_eq_slot = short_row ? 0u : (uint32_t)K - need;
    if (t < TOPK_MAX) { sel_v[t] = -INFINITY; sel_i[t] = -1; }
    __syncthreads();
    for (int64_t j0 = 0; j0 < n; j0 += TOPK_NT) {
        const int64_t j = j0 + t;
        const uint32_t key = j < n ? order_key(row[j]) : 0u;
        const bool gt = !short_row && key > T;
        const bool eq = short_row ? key >= T : key == T;
        const uint64_t bgt = __ballot(gt), beq = __ballot(eq);
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        if (lane == 0) { w_gt[wave] = __popcll(bgt); w_eq[wave] = __popcll(beq); }
        __syncthreads();
        uint32_t off_gt = run_gt, off_eq = run_eq, tot_gt = 0u, tot_eq = 0u;
        for (int w = 0; w < TOPK_NW; ++w) {
            if (w < wave) { off_gt += w_gt[w]; off_eq += w_eq[w]; }
            tot_gt += w_gt[w]; tot_eq += w_eq[w];
        }
        if (gt) {
            const uint32_t slot = off_gt + __popcll(bgt & below);
            if (slot < TOPK_MAX) { sel_v[slot] = row[j]; sel_i[slot] = (int)j; }
        }
        if (eq) {
            const uint32_t k = off_eq + __popcll(beq & below);
            if (k < n_eq_take && base_eq_slot + k < TOPK_MAX) {
                sel_v[base_eq_slot + k] = row[j];
                sel_i[base_eq_slot + k] = (int)j;
            }
        }
        run_gt += tot_gt;
        run_eq += tot_eq;
        __syncthreads();
    }

    // ---- 3. order the winners
    if (t == 0) {
        float v[TOPK_MAX];
        int id[TOPK_MAX];
        for (int k = 0; k < K; ++k) { v[k] = sel_v[k]; id[k] = sel_i[k]; }
        // insertion sort; a missing entry (id -1) sorts after every real one
        for (int a = 1; a < K; ++a) {
            const float va = v[a];
            const int ia = id[a];
            int b = a;
            while (b > 0 && ia >= 0 && (id[b - 1] < 0 || better(va, ia, v[b - 1], id[b - 1]))) {
                v[b] = v[b - 1]; id[b] = id[b - 1]; --b;
            }
            v[b] = va; id[b] = ia;
        }
        for (int k = 0; k < K; ++k) {
            ids[r * K + k] = id[k];
            vals[r * K + k] = id[k] < 0 ? -INFINITY : v[k];
        }
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
    hipLaunchKernelGGL(swiglu_kernel, dim3((unsigned)((F + 2047) / 2048), (unsigned)T), dim3(256), 0,
                       s, (const bf16_t*)gu, ld, F, (bf16_t*)out, ldo);
    return hipGetLastError();
}

hipError_t launch_add(float* h, int64_t ldh, const void* x, int64_t ldx, int64_t T, int H,
                      hipStream_t s) {
    if (T == 0 || H == 0) return hipSuccess;
    hipLaunchKernelGGL(add_kernel, dim3((unsigned)((H + 1023) / 1024), (unsigned)T), dim3(256), 0, s,
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
