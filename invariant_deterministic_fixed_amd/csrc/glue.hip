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
// One workgroup per row.  Each value maps to an order-preserving 32-bit key
// (NaN -> 0, below every other key; -0 and +0 one key).  Let T be the key of
// the K-th largest entry: the result is every entry with key > T plus the
// lowest-index entries with key == T, which is what both paths below select.
//   fast path (two reads of the row):
//     1. histogram of the keys' top byte (LDS increments: integer counts, so
//        the totals do not depend on the order in which lanes add) -> the
//        bucket b holding T and how many entries above it are winners;
//     2. one pass in index order (1024-element tiles, ballots and wave prefix
//        counts) keeps the entries above bucket b and gathers bucket b's
//        entries, still in index order, into LDS;
//     3. radix passes over bytes 2, 1, 0 of the gathered keys pin down T, and
//        an index-ordered pass over them takes the keys > T and the first
//        keys == T;
//   fallback (a row with fewer than K non-NaN entries, or more than
//   TOPK_CAND entries in bucket b): the same radix select over bytes 3..0 and
//   the index-ordered collection, both reading the row.
// The <= 32 winners are then sorted by (value desc, index asc).
constexpr int TOPK_MAX = 32;
constexpr int TOPK_NT = 1024;
constexpr int TOPK_NW = TOPK_NT / 64;
constexpr int TOPK_CAND = 4096;
constexpr int TOPK_E = 8;            // entries per thread per tile in the gathering pass

__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t b = __float_as_uint(v);
    if (v != v) return 0u;
    if ((b & 0x7fffffffu) == 0u) b = 0u;                 // -0 and +0 are one value
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

struct TopkShared {
    uint32_t hist[256];
    uint32_t s_prefix, s_need;
    uint32_t w_a[TOPK_NW], w_b[TOPK_NW];
    uint32_t w_ea[TOPK_E][TOPK_NW], w_eb[TOPK_E][TOPK_NW];
    float sel_v[TOPK_MAX];
    int sel_i[TOPK_MAX];
    float cand_v[TOPK_CAND];
    int cand_i[TOPK_CAND];
};

// Radix select over `m` values read by get(j): keys with (key & mask) == prefix
// are refined byte by byte, shifts `shift`, shift - 8, ..., `last`.  Returns
// false if fewer than `need` such keys exist.  Otherwise prefix holds the
// bytes fixed so far of the need-th largest key (all of T when last = 0) and
// need how many entries with that prefix are still to be taken.  Every thread
// returns the same values.
template <class Get>
__device__ bool radix_select(TopkShared& sh, Get get, int64_t m, int shift, int last,
                             uint32_t& prefix, uint32_t& mask, uint32_t& need) {
    const int t = threadIdx.x;
    for (; shift >= last; shift -= 8) {
        if (t < 256) sh.hist[t] = 0u;
        __syncthreads();
        for (int64_t j0 = 0; j0 < m; j0 += (int64_t)TOPK_E * TOPK_NT) {
            float v[TOPK_E];
#pragma unroll
            for (int e = 0; e < TOPK_E; ++e) {
                const int64_t j = j0 + e * TOPK_NT + t;
                v[e] = j < m ? get(j) : __uint_as_float(0x7fc00000u);
            }
#pragma unroll
            for (int e = 0; e < TOPK_E; ++e) {
                const uint32_t key = order_key(v[e]);
                if (key != 0u && (key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
            }
        }
        __syncthreads();
        if (t == 0) {
            uint32_t cum = 0u, chosen = 0u, nd = need;
            bool found = false;
            for (int bkt = 255; bkt >= 0; --bkt) {
                const uint32_t h = sh.hist[bkt];
                if (cum + h >= need) { chosen = (uint32_t)bkt; nd = need - cum; found = true; break; }
                cum += h;
            }
            sh.s_prefix = found ? (prefix | (chosen << shift)) : 0xffffffffu;
            sh.s_need = found ? nd : 0u;
        }
        __syncthreads();
        if (sh.s_prefix == 0xffffffffu) return false;
        prefix = sh.s_prefix;
        need = sh.s_need;
        mask |= 255u << shift;
    }
    return true;
}

// One index-ordered pass over m values: entries whose key satisfies gt() go
// to sel slots gt_base + (their rank), the first n_eq entries satisfying eq()
// go to slots eq_base + rank.  Returns nothing; sel is complete afterwards.
template <class Get, class Gt, class Eq>
__device__ void collect(TopkShared& sh, Get get, int64_t m, Gt gt_of, Eq eq_of, uint32_t gt_base,
                        uint32_t eq_base, uint32_t n_eq) {
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint32_t run_gt = 0u, run_eq = 0u;
    for (int64_t j0 = 0; j0 < m; j0 += TOPK_NT) {
        const int64_t j = j0 + t;
        const float v = j < m ? get(j) : 0.0f;
        const uint32_t key = j < m ? order_key(v) : 0u;
        const bool gt = gt_of(key), eq = eq_of(key);
        const uint64_t bgt = __ballot(gt), beq = __ballot(eq);
        if (lane == 0) { sh.w_a[wave] = __popcll(bgt); sh.w_b[wave] = __popcll(beq); }
        __syncthreads();
        uint32_t off_gt = run_gt, off_eq = run_eq, tot_gt = 0u, tot_eq = 0u;
        for (int w = 0; w < TOPK_NW; ++w) {
            if (w < wave) { off_gt += sh.w_a[w]; off_eq += sh.w_b[w]; }
            tot_gt += sh.w_a[w]; tot_eq += sh.w_b[w];
        }
        if (gt) {
            const uint32_t slot = gt_base + off_gt + __popcll(bgt & below);
            if (slot < TOPK_MAX) { sh.sel_v[slot] = v; sh.sel_i[slot] = (int)j; }
        }
        if (eq) {
            const uint32_t k = off_eq + __popcll(beq & below);
            if (k < n_eq && eq_base + k < TOPK_MAX) { sh.sel_v[eq_base + k] = v; sh.sel_i[eq_base + k] = (int)j; }
        }
        run_gt += tot_gt;
        run_eq += tot_eq;
        __syncthreads();
    }
}

__global__ __launch_bounds__(TOPK_NT) void topk_kernel(const float* __restrict__ x, int64_t ldx,
                                                       int64_t n, int K,
                                                       int32_t* __restrict__ ids,
                                                       float* __restrict__ vals) {
    __shared__ TopkShared sh;
    const int64_t r = blockIdx.x;
    const float* row = x + r * ldx;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    auto from_row = [&](int64_t j) { return row[j]; };
    if (t < TOPK_MAX) { sh.sel_v[t] = -INFINITY; sh.sel_i[t] = -1; }

    // ---- 1. top byte
    uint32_t prefix = 0u, mask = 0u, need = (uint32_t)K;
    bool fast = radix_select(sh, from_row, n, 24, 24, prefix, mask, need);
    const uint32_t top = prefix >> 24, gt1 = (uint32_t)K - need;

    // ---- 2. winners above the bucket, the bucket's entries gathered in index
    // order; tiles of E x 1024 entries, entry j0 + e * 1024 + t read by thread t
    // (all E loads in flight at once), ranked in (e, t) = index order
    uint32_t n_cand = 0u;
    if (fast) {
        constexpr int E = TOPK_E;
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        uint32_t run_gt = 0u, run_c = 0u;
        for (int64_t j0 = 0; j0 < n; j0 += (int64_t)E * TOPK_NT) {
            float v[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int64_t j = j0 + e * TOPK_NT + t;
                v[e] = j < n ? row[j] : __uint_as_float(0x7fc00000u);   // NaN: never flagged
            }
            uint64_t bgt[E], bcd[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const uint32_t key = order_key(v[e]);
                bgt[e] = __ballot(key != 0u && (key >> 24) > top);
                bcd[e] = __ballot(key != 0u && (key >> 24) == top);
                if (lane == 0) { sh.w_ea[e][wave] = __popcll(bgt[e]); sh.w_eb[e][wave] = __popcll(bcd[e]); }
            }
            __syncthreads();
            uint32_t off_gt = run_gt, off_c = run_c;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                uint32_t pre_gt = 0u, pre_c = 0u, tot_gt = 0u, tot_c = 0u;
                for (int w = 0; w < TOPK_NW; ++w) {
                    if (w < wave) { pre_gt += sh.w_ea[e][w]; pre_c += sh.w_eb[e][w]; }
                    tot_gt += sh.w_ea[e][w]; tot_c += sh.w_eb[e][w];
                }
                const int64_t j = j0 + e * TOPK_NT + t;
                if ((bgt[e] >> lane) & 1ull) {
                    const uint32_t slot = off_gt + pre_gt + __popcll(bgt[e] & below);
                    if (slot < TOPK_MAX) { sh.sel_v[slot] = v[e]; sh.sel_i[slot] = (int)j; }
                }
                if ((bcd[e] >> lane) & 1ull) {
                    const uint32_t c = off_c + pre_c + __popcll(bcd[e] & below);
                    if (c < (uint32_t)TOPK_CAND) { sh.cand_v[c] = v[e]; sh.cand_i[c] = (int)j; }
                }
                off_gt += tot_gt;
                off_c += tot_c;
            }
            run_gt = off_gt;
            run_c = off_c;
            __syncthreads();
        }
        n_cand = run_c;
        fast = n_cand <= (uint32_t)TOPK_CAND;
    }

    if (fast) {
        // ---- 3. bytes 2..0 over the gathered entries, then take them in index order
        auto from_cand = [&](int64_t c) { return sh.cand_v[c]; };
        radix_select(sh, from_cand, (int64_t)n_cand, 16, 0, prefix, mask, need);  // T: >= need entries
        const uint32_t T = prefix;
        // (the gt1 winners above the bucket are in sel slots [0, gt1) already)
        {
            const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
            uint32_t run_gt = 0u, run_eq = 0u;
            for (int64_t c0 = 0; c0 < (int64_t)n_cand; c0 += TOPK_NT) {
                const int64_t c = c0 + t;
                const float v = c < (int64_t)n_cand ? sh.cand_v[c] : 0.0f;
                const uint32_t key = c < (int64_t)n_cand ? order_key(v) : 0u;
                const bool gt = key > T, eq = key == T && key != 0u;
                const uint64_t bgt = __ballot(gt), beq = __ballot(eq);
                __syncthreads();                          // w_a / w_b of the last tile read
                if (lane == 0) { sh.w_a[wave] = __popcll(bgt); sh.w_b[wave] = __popcll(beq); }
                __syncthreads();
                uint32_t off_gt = run_gt, off_eq = run_eq, tot_gt = 0u, tot_eq = 0u;
                for (int w = 0; w < TOPK_NW; ++w) {
                    if (w < wave) { off_gt += sh.w_a[w]; off_eq += sh.w_b[w]; }
                    tot_gt += sh.w_a[w]; tot_eq += sh.w_b[w];
                }
                if (gt) {
                    const uint32_t slot = gt1 + off_gt + __popcll(bgt & below);
                    if (slot < TOPK_MAX) { sh.sel_v[slot] = v; sh.sel_i[slot] = sh.cand_i[c]; }
                }
                if (eq) {
                    const uint32_t k = off_eq + __popcll(beq & below);
                    const uint32_t slot = (uint32_t)K - need + k;
                    if (k < need && slot < TOPK_MAX) { sh.sel_v[slot] = v; sh.sel_i[slot] = sh.cand_i[c]; }
                }
                run_gt += tot_gt;
                run_eq += tot_eq;
            }
        }
    } else {
        // ---- fallback: full radix select and collection over the row
        if (t < TOPK_MAX) { sh.sel_v[t] = -INFINITY; sh.sel_i[t] = -1; }
        prefix = 0u; mask = 0u; need = (uint32_t)K;
        const bool found = radix_select(sh, from_row, n, 24, 0, prefix, mask, need);
        // a row with fewer than K valid entries: every valid entry is selected
        const uint32_t T = found ? prefix : 1u;
        const uint32_t n_eq = found ? need : (uint32_t)K;
        const uint32_t eq_base = found ? (uint32_t)K - need : 0u;
        collect(sh, from_row, n, [&](uint32_t k) { return found && k > T; },
                [&](uint32_t k) { return found ? k == T : k >= T; }, 0u, eq_base, n_eq);
    }
    __syncthreads();

    // ---- 4. order the winners
    if (t == 0) {
        float v[TOPK_MAX];
        int id[TOPK_MAX];
        for (int k = 0; k < K; ++k) { v[k] = sh.sel_v[k]; id[k] = sh.sel_i[k]; }
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
