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

// ------------------------------------------------------------------ fp32 split
// Three bf16 parts of an fp32 activation, for contracting fp32 activations
// against bf16 weights on bf16 matrix cores (the fp32-activation mitigation
// the devpress.csdn.net explainer names in sections 2 and 6: weights stay
// bf16, activations fp32).  hi = bf16(x), mid = bf16(x - hi), lo = bf16(x -
// hi - mid), each rounded to nearest even; both differences are exact in
// fp32 (x - hi keeps at most 16 significant bits, x - hi - mid at most 8), so
// hi + mid + lo = x whenever the parts stay in the normal range.  Row i of
// out holds [hi(x[i, :]) | mid(...) | lo(...)], K elements each.  Four
// elements (16 bytes in, three 8-byte pieces out) per lane.
__global__ __launch_bounds__(256) void split3_kernel(const float* __restrict__ x, int64_t ldx,
                                                     int K, bf16_t* __restrict__ out,
                                                     int64_t ldo) {
    const int64_t row = blockIdx.y;
    const int k = 4 * (blockIdx.x * 256 + threadIdx.x);
    if (k >= K) return;
    const f32x4 v = *reinterpret_cast<const f32x4*>(x + row * ldx + k);
    u32x2 hi, mid, lo;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint32_t ph[2], pm[2], pl[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float xv = v[2 * h + i];
            const uint32_t bh = f32_to_bf16(xv);
            const float r1 = xv - bf16_to_f32(bh);
            const uint32_t bm = f32_to_bf16(r1);
            const float r2 = r1 - bf16_to_f32(bm);
            const uint32_t bl = f32_to_bf16(r2);
            ph[i] = bh; pm[i] = bm; pl[i] = bl;
        }
        hi[h] = ph[0] | (ph[1] << 16);
        mid[h] = pm[0] | (pm[1] << 16);
        lo[h] = pl[0] | (pl[1] << 16);
    }
    bf16_t* o = out + row * ldo + k;
    *reinterpret_cast<u32x2*>(o) = hi;
    *reinterpret_cast<u32x2*>(o + K) = mid;
    *reinterpret_cast<u32x2*>(o + 2 * K) = lo;
}

// ------------------------------------------------------------------ top-k
// Exact top-K of one fp32 row: the K largest values, sorted by value
// descending and, among equal values, by index ascending; NaN never selected.
// One workgroup per row.  Each value maps to an order-preserving 32-bit key
// (NaN -> 0, below every other key; -0 and +0 one key).  Let T be the key of
// the K-th largest entry: the result is every entry with key > T plus the
// lowest-index entries with key == T, which is what every path below selects.
// Counting uses integer LDS increments and slots are reserved with integer LDS
// atomics, so neither counts nor the selected set depend on the order in which
// lanes and waves arrive; where order matters (equal keys) it is the index.
//   1. histogram of the keys' top 11 bits (sign, exponent, two mantissa bits;
//      a bucket is a quarter octave) -> the bucket b holding T and how many
//      entries above it are winners;
//   2. one pass over the row: entries above bucket b go to the winner slots,
//      bucket b's entries to an LDS candidate list (unordered);
//   3. two 8-bit radix passes and a final one over the candidates pin down T;
//      candidates > T are winners; those == T are listed and the `need`
//      lowest indices among them (ranked by index) complete the K;
//   crowded bucket (more than TOPK_CAND entries in b): the radix passes and
//   the pass that lists > T and == T read the row instead;
//   more than TOPK_EQ_MAX entries equal to T, or fewer than K non-NaN entries:
//   one index-ordered pass over the row (ballots and wave prefix counts) takes
//   the keys > T and the first keys == T, stopping once all are placed.
// A row longer than TOPK_SEG entries runs steps 1-3 over its first TOPK_SEG
// entries and then reads the rest once (topk_kernel), so it is read about
// once instead of twice.
// The <= 32 winners are then ranked by (value desc, index asc).
constexpr int TOPK_MAX = 32;
constexpr int TOPK_NT = 1024;
constexpr int TOPK_NW = TOPK_NT / 64;
constexpr int TOPK_CAND = 4096;
constexpr int TOPK_SEG = 16384;       // prefix of a long row selected first

__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t b = __float_as_uint(v);
    if (v != v) return 0u;
    if ((b & 0x7fffffffu) == 0u) b = 0u;                 // -0 and +0 are one value
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

constexpr int TOPK_EQ_MAX = 256;     // entries equal to the K-th key ranked by index in LDS

constexpr int TOPK_HB = 11;           // bits of the first digit (sign, exponent, 2 mantissa bits)

struct TopkShared {
    uint32_t hist[1 << TOPK_HB];
    uint32_t s_prefix, s_need;
    uint32_t w_a[TOPK_NW], w_b[TOPK_NW];
    uint32_t n_gt, n_cand, n_eq;         // slot counters (LDS integer atomics)
    int eq_i[TOPK_EQ_MAX];
    float sel_v[TOPK_MAX];
    int sel_i[TOPK_MAX];
    float cand_v[TOPK_CAND];
    int cand_i[TOPK_CAND];
};

// Radix select over `m` values: keys with (key & mask) == prefix are refined
// digit by digit, BITS bits at shifts `shift`, shift - BITS, ..., down to
// `last` (a digit may overlap bits already fixed: they agree with prefix).
// Returns false if fewer than `need` such keys exist.  Otherwise prefix holds
// the bits fixed so far of the need-th largest key (all of T when last = 0)
// and need how many entries with that prefix are still to be taken.  Every
// thread returns the same values.  get4(i) returns values 4i .. 4i+3 (NaN past
// m); get4_fast(i) the same without bounds checks, used (when fast_ok) for
// tiles wholly inside.  E reads of four per thread per tile, the next tile's
// reads issued before the current tile is counted (integer LDS atomics: the
// order of the increments does not matter).
template <int E, int BITS, class Get4, class Get4Fast>
__device__ bool radix_select(TopkShared& sh, Get4 get4, Get4Fast get4_fast, bool fast_ok,
                             int64_t m, int shift, int last,
                             uint32_t& prefix, uint32_t& mask, uint32_t& need) {
    constexpr int NB = 1 << BITS;
    constexpr int PER = NB >= TOPK_NT ? NB / TOPK_NT : 1;   // bins per thread
    constexpr int NACT = NB / PER;                          // threads that own bins
    static_assert(NACT % 64 == 0 && NACT <= TOPK_NT, "whole waves own the bins");
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t m4 = (m + 3) / 4;
    constexpr int64_t TILE = (int64_t)E * TOPK_NT;
    for (; shift >= last; shift -= BITS) {
        for (int b = t; b < NB; b += TOPK_NT) sh.hist[b] = 0u;
        __syncthreads();
        f32x4 v[E];
        auto load = [&](int64_t i0) {
            if (fast_ok && 4 * (i0 + TILE) <= m) {       // whole tile inside: plain reads
#pragma unroll
                for (int e = 0; e < E; ++e) v[e] = get4_fast(i0 + e * TOPK_NT + t);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int64_t i = i0 + e * TOPK_NT + t;
                    v[e] = i < m4 ? get4(i) : f32x4{NAN, NAN, NAN, NAN};
                }
            }
        };
        load(0);
        for (int64_t i0 = 0; i0 < m4; i0 += TILE) {
            f32x4 cur[E];
#pragma unroll
            for (int e = 0; e < E; ++e) cur[e] = v[e];
            if (i0 + TILE < m4) load(i0 + TILE);
#pragma unroll
            for (int e = 0; e < E; ++e)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t key = order_key(cur[e][q]);
                    if (key != 0u && (key & mask) == prefix)
                        atomicAdd(&sh.hist[(key >> shift) & (NB - 1)], 1u);
                }
        }
        __syncthreads();
        // bucket of the need-th largest key: thread t < NACT owns bins
        // [t PER, t PER + PER); suffix sums over the owners (a shift scan
        // inside each wave, then the wave totals above)
        uint32_t own[PER], sum = 0u, suf = 0u;
        if (t < NACT) {
#pragma unroll
            for (int k = 0; k < PER; ++k) { own[k] = sh.hist[t * PER + k]; sum += own[k]; }
            suf = sum;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const uint32_t y = __shfl_down(suf, d);
                if (lane + d < 64) suf += y;
            }
            if (lane == 0) sh.w_a[wave] = suf;               // wave total
        }
        if (t == 0) { sh.s_prefix = 0xffffffffu; sh.s_need = 0u; }
        __syncthreads();
        if (t < NACT) {
            uint32_t above = suf - sum;                      // owners above t inside the wave
            for (int w = wave + 1; w < NACT / 64; ++w) above += sh.w_a[w];
#pragma unroll
            for (int k = PER - 1; k >= 0; --k) {
                if (above < need && need <= above + own[k]) {
                    sh.s_prefix = prefix | ((uint32_t)(t * PER + k) << shift);
                    sh.s_need = need - above;
                }
                above += own[k];
            }
        }
        __syncthreads();
        if (sh.s_prefix == 0xffffffffu) return false;
        prefix = sh.s_prefix;
        need = sh.s_need;
        mask |= (uint32_t)(NB - 1) << shift;
        __syncthreads();                                     // s_prefix / w_a read by all
    }
    return true;
}

// One index-ordered pass over m values: entries whose key satisfies gt() go
// to sel slots gt_base + (their rank), the first n_eq entries satisfying eq()
// go to slots eq_base + rank; the pass ends once n_gt_all entries above and
// n_eq equal ones have been seen.  sel is complete afterwards.
template <class Get, class Gt, class Eq>
__device__ void collect(TopkShared& sh, Get get, int64_t m, Gt gt_of, Eq eq_of, uint32_t gt_base,
                        uint32_t eq_base, uint32_t n_eq, uint32_t n_gt_all) {
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
        if (run_gt >= n_gt_all && run_eq >= n_eq) break;     // every winner placed
    }
}

// One pass over the m values 4i .. 4i+3 = get4(i) (get4_fast for tiles wholly
// inside when fast_ok): entries whose key satisfies is_gt / is_eq are handed
// to put() with their rank among the flagged lanes of their ballot and the
// base of the slots their wave reserved for that ballot with one LDS atomic
// on *n_gt / *n_eq (slot order is not index order).
template <int E, class Get4, class Get4Fast, class Put, class IsGt, class IsEq>
__device__ void row_pass(Get4 get4, Get4Fast get4_fast, bool fast_ok, int64_t m, Put put,
                         IsGt is_gt, IsEq is_eq, uint32_t* n_gt, uint32_t* n_eq) {
    const int t = threadIdx.x, lane = t & 63;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    constexpr int64_t TILE = (int64_t)E * TOPK_NT;
    const int64_t m4 = (m + 3) / 4;
    f32x4 v[E];
    auto load = [&](int64_t i0) {
        if (fast_ok && 4 * (i0 + TILE) <= m) {            // whole tile inside: plain reads
#pragma unroll
            for (int e = 0; e < E; ++e) v[e] = get4_fast(i0 + e * TOPK_NT + t);
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int64_t i = i0 + e * TOPK_NT + t;
                v[e] = i < m4 ? get4(i) : f32x4{NAN, NAN, NAN, NAN};   // NaN: never flagged
            }
        }
    };
    load(0);
    for (int64_t i0 = 0; i0 < m4; i0 += TILE) {
        f32x4 cur[E];
#pragma unroll
        for (int e = 0; e < E; ++e) cur[e] = v[e];
        if (i0 + TILE < m4) load(i0 + TILE);
#pragma unroll
        for (int e = 0; e < E; ++e)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t key = order_key(cur[e][q]);
                const bool gt = key != 0u && is_gt(key);
                const bool eq = key != 0u && is_eq(key);
                const uint64_t bgt = __ballot(gt), beq = __ballot(eq);
                if (bgt | beq) {
                    uint32_t base_gt = 0u, base_eq = 0u;
                    if (lane == 0) {
                        if (bgt) base_gt = atomicAdd(n_gt, (uint32_t)__popcll(bgt));
                        if (beq) base_eq = atomicAdd(n_eq, (uint32_t)__popcll(beq));
                    }
                    base_gt = (uint32_t)__builtin_amdgcn_readfirstlane((int)base_gt);
                    base_eq = (uint32_t)__builtin_amdgcn_readfirstlane((int)base_eq);
                    put(key, cur[e][q], 4 * (i0 + e * TOPK_NT + t) + q, gt, eq, base_gt, base_eq,
                        (uint32_t)__popcll(bgt & below), (uint32_t)__popcll(beq & below));
                }
            }
    }
}

// Of the n_eq_all entries listed in eq_i (all equal to the K-th key), the
// `need` lowest indices go to sel slots base .. base + need - 1 in index order.
__device__ void rank_equal(TopkShared& sh, const float* row, uint32_t n_eq_all, uint32_t base,
                           uint32_t need) {
    for (uint32_t a = threadIdx.x; a < n_eq_all; a += TOPK_NT) {
        const int ia = sh.eq_i[a];
        uint32_t rank = 0u;
        for (uint32_t b2 = 0; b2 < n_eq_all; ++b2) rank += sh.eq_i[b2] < ia ? 1u : 0u;
        if (rank < need && base + rank < TOPK_MAX) {
            sh.sel_v[base + rank] = row[ia];
            sh.sel_i[base + rank] = ia;
        }
    }
}

// Steps 1-3 above over entries 0 .. n-1 of `row`: the K winners into sel
// (slot order arbitrary; slots of missing entries hold index -1).  Left to
// the compiler as a call: inlined at the kernel's two call sites (or at one,
// inside a loop) it spilled registers in every pass over the row.
__device__ void topk_select(TopkShared& sh, const float* row, int64_t n, int K) {
    const int t = threadIdx.x;
    auto from_row = [&](int64_t j) { return row[j]; };
    // values 4i .. 4i+3 of the row, NaN past n; one 16-byte read when the row
    // is 16-byte aligned and the four are inside it
    const bool row_vec = (reinterpret_cast<uintptr_t>(row) & 15u) == 0u;
    auto row4 = [&](int64_t i) -> f32x4 {
        const int64_t j = 4 * i;
        f32x4 r;
#pragma unroll
        for (int q = 0; q < 4; ++q) r[q] = j + q < n ? row[j + q] : NAN;
        return r;
    };
    auto row4_vec = [&](int64_t i) -> f32x4 { return *reinterpret_cast<const f32x4*>(row + 4 * i); };
    if (t < TOPK_MAX) { sh.sel_v[t] = -INFINITY; sh.sel_i[t] = -1; }

    // ---- 1. the first TOPK_HB bits of the K-th key (one pass over the row)
    uint32_t prefix = 0u, mask = 0u, need = (uint32_t)K;
    const bool ok1 = radix_select<4, TOPK_HB>(sh, row4, row4_vec, row_vec, n, 32 - TOPK_HB,
                                              32 - TOPK_HB, prefix, mask, need);
    const uint32_t top = prefix >> (32 - TOPK_HB);
    [[maybe_unused]] const uint32_t gt1 = (uint32_t)K - need;     // winners above bucket `top`

    // ---- 2. one pass over the row: entries above the bucket go to sel slots
    // [0, gt1), the bucket's entries to the candidate list.  Each wave reserves
    // slots for the flagged lanes of one ballot with one LDS atomic, so slot
    // order is not index order; nothing below depends on it except the choice
    // among entries equal to the K-th key, which is made by index (step 3).
    if (t == 0) { sh.n_gt = 0u; sh.n_cand = 0u; sh.n_eq = 0u; }
    __syncthreads();
    uint32_t n_cand = 0u;
    if (ok1) {
        row_pass<4>(row4, row4_vec, row_vec, n, [&](uint32_t key, float v, int64_t j, bool take_gt,
                                                     bool take_cd, uint32_t base_gt, uint32_t base_cd,
                                                     uint32_t r_gt, uint32_t r_cd) {
            if (take_gt && base_gt + r_gt < TOPK_MAX) { sh.sel_v[base_gt + r_gt] = v; sh.sel_i[base_gt + r_gt] = (int)j; }
            if (take_cd && base_cd + r_cd < (uint32_t)TOPK_CAND) { sh.cand_v[base_cd + r_cd] = v; sh.cand_i[base_cd + r_cd] = (int)j; }
        }, [&](uint32_t key) { return (key >> (32 - TOPK_HB)) > top; },
           [&](uint32_t key) { return (key >> (32 - TOPK_HB)) == top; }, &sh.n_gt, &sh.n_cand);
        __syncthreads();
        n_cand = sh.n_cand;
    }

    // ---- 3. the remaining bits of T, the K-th key; take every entry above T
    // and, of those equal to T, the `need` lowest indices
    bool ordered = true;          // fall back to one index-ordered pass over the row
    bool found = ok1;
    uint32_t T = 0u;
    if (ok1 && n_cand <= (uint32_t)TOPK_CAND) {
        auto cand4 = [&](int64_t i) -> f32x4 {
            f32x4 r;
#pragma unroll
            for (int q = 0; q < 4; ++q) r[q] = 4 * i + q < (int64_t)n_cand ? sh.cand_v[4 * i + q] : NAN;
            return r;
        };
        // bits 20..5 in two 8-bit digits, then bits 7..0 (7..5 already fixed)
        radix_select<1, 8>(sh, cand4, cand4, false, (int64_t)n_cand, 13, 5, prefix, mask, need);
        radix_select<1, 8>(sh, cand4, cand4, false, (int64_t)n_cand, 0, 0, prefix, mask, need);
        T = prefix;
        // (the gt1 winners above the bucket are in sel slots [0, gt1) already)
        for (int64_t c = t; c < (int64_t)n_cand; c += TOPK_NT) {
            const uint32_t key = order_key(sh.cand_v[c]);
            if (key > T) {
                const uint32_t slot = atomicAdd(&sh.n_gt, 1u);      // continues after the gt1 slots
                if (slot < TOPK_MAX) { sh.sel_v[slot] = sh.cand_v[c]; sh.sel_i[slot] = sh.cand_i[c]; }
            } else if (key == T) {
                const uint32_t k = atomicAdd(&sh.n_eq, 1u);
                if (k < (uint32_t)TOPK_EQ_MAX) sh.eq_i[k] = sh.cand_i[c];
            }
        }
        __syncthreads();
        if (sh.n_eq <= (uint32_t)TOPK_EQ_MAX) {
            rank_equal(sh, row, sh.n_eq, (uint32_t)K - need, need);
            ordered = false;
        }
        // else: many exact ties at the K-th key; T and need are final
    } else if (ok1) {
        // a crowded first bucket: the remaining digits over the row, then one
        // pass over the row for the entries above T and those equal to it
        radix_select<4, 8>(sh, row4, row4_vec, row_vec, n, 13, 5, prefix, mask, need);
        radix_select<4, 8>(sh, row4, row4_vec, row_vec, n, 0, 0, prefix, mask, need);
        T = prefix;
        if (t == 0) { sh.n_gt = 0u; sh.n_eq = 0u; }
        __syncthreads();
        row_pass<4>(row4, row4_vec, row_vec, n, [&](uint32_t key, float v, int64_t j, bool take_gt,
                                                     bool take_eq, uint32_t base_gt, uint32_t base_eq,
                                                     uint32_t r_gt, uint32_t r_eq) {
            if (take_gt && base_gt + r_gt < TOPK_MAX) { sh.sel_v[base_gt + r_gt] = v; sh.sel_i[base_gt + r_gt] = (int)j; }
            if (take_eq && base_eq + r_eq < (uint32_t)TOPK_EQ_MAX) sh.eq_i[base_eq + r_eq] = (int)j;
        }, [&](uint32_t key) { return key > T; }, [&](uint32_t key) { return key == T; },
           &sh.n_gt, &sh.n_eq);
        __syncthreads();
        if (sh.n_eq <= (uint32_t)TOPK_EQ_MAX) {
            rank_equal(sh, row, sh.n_eq, (uint32_t)K - need, need);
            ordered = false;
        }
    }
    if (ordered) {
        // one index-ordered pass over the row: entries above T, then the
        // first `need` equal to T (a row with fewer than K valid entries:
        // every valid entry)
        __syncthreads();
        if (t < TOPK_MAX) { sh.sel_v[t] = -INFINITY; sh.sel_i[t] = -1; }
        const uint32_t Tc = found ? T : 1u;
        const uint32_t n_eq = found ? need : (uint32_t)K;
        const uint32_t eq_base = found ? (uint32_t)K - need : 0u;
        collect(sh, from_row, n, [&](uint32_t k) { return found && k > Tc; },
                [&](uint32_t k) { return found ? k == Tc : k >= Tc; }, 0u, eq_base, n_eq,
                (uint32_t)K - n_eq);
    }
    __syncthreads();
}

__global__ __launch_bounds__(TOPK_NT) void topk_kernel(const float* __restrict__ x, int64_t ldx,
                                                       int64_t n, int K,
                                                       int32_t* __restrict__ ids,
                                                       float* __restrict__ vals) {
    __shared__ TopkShared sh;
    const int64_t r = blockIdx.x;
    const float* row = x + r * ldx;
    const int t = threadIdx.x;
    // A long row is read once, not twice: the winners of its first TOPK_SEG
    // entries (two passes over 64 KB, the second from the cache) fix the key
    // T0 of the prefix's K-th entry.  An entry past the prefix can only be a
    // winner if its key is above T0 (an entry with key T0 there has a higher
    // index than the prefix's K winners, and loses to all of them), so one pass
    // over the rest lists those entries as candidates beside the prefix's
    // winners, and the K winners of the row are the K winners among the
    // candidates, found as in step 3 (the K-th key by three radix digits, the
    // entries above it, the lowest indices among those equal to it).  A prefix
    // with fewer than K non-NaN entries, more candidates than the list holds,
    // or more entries equal to the K-th key than are ranked in LDS: the whole
    // row through steps 1-3.
    const int64_t n1 = n > TOPK_SEG ? (int64_t)TOPK_SEG : n;
    topk_select(sh, row, n1, K);
    if (n > n1) {
        __syncthreads();
        if (t == 0) { sh.s_prefix = 0xffffffffu; sh.s_need = 1u; sh.n_cand = (uint32_t)K; }
        __syncthreads();
        if (t < K) {
            if (sh.sel_i[t] < 0) atomicAnd(&sh.s_need, 0u);
            else atomicMin(&sh.s_prefix, order_key(sh.sel_v[t]));
            sh.cand_v[t] = sh.sel_v[t];
            sh.cand_i[t] = sh.sel_i[t];
        }
        __syncthreads();
        const bool full = sh.s_need != 0u;
        const uint32_t T0 = sh.s_prefix;
        bool done = false;
        if (full) {
            const float* rest = row + n1;
            const int64_t m = n - n1;
            const bool rest_vec = (reinterpret_cast<uintptr_t>(rest) & 15u) == 0u;
            auto rest4 = [&](int64_t i) -> f32x4 {
                const int64_t j = 4 * i;
                f32x4 v;
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = j + q < m ? rest[j + q] : NAN;
                return v;
            };
            auto rest4_vec = [&](int64_t i) -> f32x4 { return *reinterpret_cast<const f32x4*>(rest + 4 * i); };
            if (t == 0) sh.n_eq = 0u;
            __syncthreads();
            row_pass<2>(rest4, rest4_vec, rest_vec, m, [&](uint32_t key, float v, int64_t j,
                                                          bool take, bool, uint32_t base, uint32_t,
                                                          uint32_t rk, uint32_t) {
                if (take && base + rk < (uint32_t)TOPK_CAND) {
                    sh.cand_v[base + rk] = v;
                    sh.cand_i[base + rk] = (int)(j + n1);
                }
            }, [&](uint32_t key) { return key > T0; }, [&](uint32_t) { return false; },
               &sh.n_cand, &sh.n_eq);
            __syncthreads();
            const uint32_t nc = sh.n_cand;
            if (nc <= (uint32_t)TOPK_CAND) {
                auto cand4 = [&](int64_t i) -> f32x4 {
                    f32x4 v;
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[q] = 4 * i + q < (int64_t)nc ? sh.cand_v[4 * i + q] : NAN;
                    return v;
                };
                uint32_t prefix = 0u, mask = 0u, need = (uint32_t)K;
                // at least K candidates (the prefix's winners): the K-th key exists
                radix_select<1, 8>(sh, cand4, cand4, false, (int64_t)nc, 24, 0, prefix, mask, need);
                const uint32_t T = prefix;
                if (t < TOPK_MAX) { sh.sel_v[t] = -INFINITY; sh.sel_i[t] = -1; }
                if (t == 0) { sh.n_gt = 0u; sh.n_eq = 0u; }
                __syncthreads();
                for (int64_t c = t; c < (int64_t)nc; c += TOPK_NT) {
                    const uint32_t key = order_key(sh.cand_v[c]);
                    if (key > T) {
                        const uint32_t slot = atomicAdd(&sh.n_gt, 1u);
                        if (slot < TOPK_MAX) { sh.sel_v[slot] = sh.cand_v[c]; sh.sel_i[slot] = sh.cand_i[c]; }
                    } else if (key == T) {
                        const uint32_t k = atomicAdd(&sh.n_eq, 1u);
                        if (k < (uint32_t)TOPK_EQ_MAX) sh.eq_i[k] = sh.cand_i[c];
                    }
                }
                __syncthreads();
                if (sh.n_eq <= (uint32_t)TOPK_EQ_MAX) {
                    rank_equal(sh, row, sh.n_eq, (uint32_t)K - need, need);
                    done = true;
                }
            }
        }
        if (!done) {
            __syncthreads();
            topk_select(sh, row, n, K);
        }
    }
    __syncthreads();

    // ---- 4. order the winners: thread k < K ranks entry k against all K (real
    // entries by value descending, index ascending -- ids are distinct, so the
    // ranks are a permutation; missing entries (id -1) after them in slot order)
    if (t < K) {
        const float v = sh.sel_v[t];
        const int id = sh.sel_i[t];
        int rank = 0;
        for (int k = 0; k < K; ++k) {
            const float vk = sh.sel_v[k];
            const int ik = sh.sel_i[k];
            const bool before = (id < 0) ? (ik >= 0 || k < t) : (ik >= 0 && better(vk, ik, v, id));
            rank += before ? 1 : 0;
        }
        ids[r * K + rank] = id;
        vals[r * K + rank] = id < 0 ? -INFINITY : v;
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

hipError_t launch_split3(const float* x, int64_t ldx, int64_t M, int K, void* out, int64_t ldo,
                         hipStream_t s) {
    if (M == 0 || K == 0) return hipSuccess;
    hipLaunchKernelGGL(split3_kernel, dim3((unsigned)((K / 4 + 255) / 256), (unsigned)M), dim3(256),
                       0, s, x, ldx, K, (bf16_t*)out, ldo);
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
