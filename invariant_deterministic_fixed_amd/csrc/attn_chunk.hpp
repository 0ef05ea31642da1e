// attn_chunk.hpp -- per-chunk attention arithmetic shared by the invariant
// chunk kernel (attention.hip: decode, and prefill runs too short for the
// 128-row block kernel) and the shape-tuned comparator (attention_tuned.hip).
// Sharing it is what makes a row's partial for a chunk the same bits on every
// path; the block kernel repeats the same per-element operations in the same
// order.
//
// A workgroup handles R tiles of 16 query rows (R = 1 in every current launch)
// against one 256-key chunk.  Nothing a row computes depends on R or
// on the row's slot: the q.k and p.v products are per-element MFMA chains over
// fixed k-blocks, the max is exact, and l is summed in one fixed order; R only
// decides how many rows share one load of the chunk's K and V.
#pragma once
#include <type_traits>

#include "common.hpp"

namespace binv {
namespace attn {

constexpr int CHUNK = 256;
constexpr int PAGE = 16;
constexpr int NT = 256;
constexpr int ROWS = 16;           // rows of one MFMA row tile
constexpr int STACK = 10;          // binary counter slots: enough for 1023 leaves

// The softmax weights of a chunk, as every kernel that forms them (decode, the
// prefill block and chunk paths, the tuned comparator) computes them, so they
// agree bit for bit.  s is a raw score q.k, c = scale * log2(e); the row's
// max in the log2 domain is m = c * max_j s_j (rounded once: since rounding
// is monotonic this is the max of the rounded c s_j), and
//   p = bf16(2^(fma(s, c, -m)))
// with the hardware v_exp_f32 as it stands (exp2f adds a range reduction
// that keeps results below 2^-126, weights more than 126 binary orders under
// the row's largest, as fp32 denormals: five more instructions per score).
// The fused form rounds s c - m once; for the row's largest score it can be a
// few units of the last place above 0, which the bf16 rounding of p absorbs.
__device__ __forceinline__ float p_of(float s, float c, float m) {
    return __builtin_amdgcn_exp2f(__builtin_fmaf(s, c, -m));
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// two weights -> bf16 pair, round to nearest even (v_cvt_pk_bf16_f32), lo first
__device__ __forceinline__ uint32_t p_pack(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
// l += p_lo + p_hi of a packed pair, by v_dot2c_f32_bf16 against (1, 1): the
// sum of a row's weights in every kernel is this chain over its pairs in the
// key order of the p.v products
__device__ __forceinline__ float l_add(uint32_t pk, float acc) {
    const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk), one, acc, false);
}


__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Workgroup barrier for LDS data only: this wave's LDS accesses done, then
// s_barrier.  Unlike __syncthreads() it does not wait for global loads, so a
// V copy requested before it stays in flight.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}


struct RowInfo {
    int64_t token;   // global query-token index (row of q / out / partials), -1 if padding
    int head;        // query head
    int pos;         // absolute position of the query
};

// Row slot r (0 .. 16R-1) of tile `qt` of sequence b: token r / G of the tile,
// head g*G + r % G; a tile holds 16R/G consecutive new tokens.
template <int G, int R>
__device__ __forceinline__ RowInfo row_info(int r, int b, int g, int qt, int q_len,
                                            int64_t q_start, int kv_len) {
    constexpr int TQ = ROWS * R / G;
    RowInfo ri;
    const int tq = r / G;
    const int i = qt * TQ + tq;                    // index among the sequence's new tokens
    ri.head = g * G + (r % G);
    if (tq < TQ && i < q_len) {
        ri.token = q_start + i;
        ri.pos = kv_len - q_len + i;
        if (ri.pos < 0) ri.token = -1;
    } else {
        ri.token = -1;
        ri.pos = -1;
    }
    return ri;
}

// NW = D/16 waves: for q.k each wave owns 16/NW pages (16 keys each) of the
// chunk; for p.v each wave owns one 16-wide feature tile over all 256 keys.
template <int D>
struct ChunkShape {
    static constexpr int NW = D / 16;            // 8 waves at D = 128, 4 at D = 64
    static constexpr int NTH = 64 * NW;
    static constexpr int JT = 16 / NW;           // pages of the chunk per wave (q.k)
    static constexpr int KS = D / 32;            // k-steps of the q.k product
};

// Everything a workgroup knows about its (sequence, KV head, query tile).
struct TileCtx {
    int b, g, qt;
    int kv_len, q_len;
    int64_t q_start;
    int pos_max;         // highest query position in the tile (-1: empty tile)
    int64_t pt_row;
    int n_pages;
};

// kv_len_b = kv_lens[b] as read by the caller
template <int G, int R>
__device__ __forceinline__ TileCtx tile_ctx_len(int b, int g, int qt, const int32_t* cu_q,
                                                int kv_len_b, int64_t pt_stride, int max_kv_len) {
    constexpr int TQ = ROWS * R / G;
    TileCtx x;
    x.b = b; x.g = g; x.qt = qt;
    x.kv_len = min(kv_len_b, max_kv_len);
    if (cu_q) {
        x.q_start = cu_q[b];
        x.q_len = cu_q[b + 1] - cu_q[b];
    } else {
        x.q_start = b;
        x.q_len = 1;
    }
    if (x.q_len > x.kv_len) x.q_len = x.kv_len;
    const int last_i = min(x.q_len, (qt + 1) * TQ) - 1;
    x.pos_max = (last_i < qt * TQ) ? -1 : x.kv_len - x.q_len + last_i;
    x.pt_row = (int64_t)b * pt_stride;
    x.n_pages = (x.kv_len + PAGE - 1) / PAGE;
    return x;
}

template <int G, int R>
__device__ __forceinline__ TileCtx tile_ctx(int b, int g, int qt, const int32_t* cu_q,
                                            const int32_t* kv_lens, int64_t pt_stride,
                                            int max_kv_len) {
    return tile_ctx_len<G, R>(b, g, qt, cu_q, kv_lens[b], pt_stride, max_kv_len);
}

// The order of the keys in the k-slots of a p.v product.  The scores are
// formed transposed (S^T = K Q^T): in 16-key tile kt, lane (ag, ar) = (lane
// >> 4, lane & 15) holds row ar's scores of keys 16 kt + 4 ag + e, e = 0..3.
// The p.v products (O^T = V^T P^T) take the keys in 32-key blocks kb whose
// k-slots 8 ag .. 8 ag + 7 hold keys 32 kb + 4 ag + (0..3) and then
// 32 kb + 16 + 4 ag + (0..3): exactly the p values lane (ag, ar) computed in
// tiles 2 kb and 2 kb + 1, so p reaches the matrix cores without changing
// lanes.  Every kernel (chunk, block, comparator) uses this order; the sum l
// of a row's p is taken in the same order too: per lane group sequentially
// over kb ascending and then the 8 slots ascending, and the four group sums
// as (g0 + g1) + (g2 + g3).

template <int D, int R>
struct ChunkLds {
    // the chunk's 16 V page blocks of this KV head, [page][D][16 slots] bf16
    // with the 16-byte half h of feature d at h ^ ((d >> 3) & 1) (v_src),
    // copied HBM -> LDS by global_load_lds (one 1 KB piece per instruction)
    __attribute__((aligned(1024))) char v[16 * D * PAGE * 2];
    // p as p.v operand: [row tile][32-key block][lane] 16 bytes each
    __attribute__((aligned(16))) char p[R * 8 * 64 * 16];
    float red_max[ChunkShape<D>::NW][ROWS * R];
    // q fragments of the tile for a workgroup that loops over chunks (its rows
    // do not change): [row tile][k-step][lane] 16 bytes each
    __attribute__((aligned(16))) char qf[R * ChunkShape<D>::KS * 64 * 16];
};

// Result of one chunk for the workgroup's 16R rows; lane (ag, ar) of every
// wave holds row 16 rt + ar:
//   m[rt]  the row's max, -inf if the row sees no key
//   l[rt]  the row's sum of p
//   o[rt]  the row's p.v for features 16 wave + 4 ag + i, i = 0..3
template <int R>
struct ChunkOut {
    float m[R], l[R];
    f32x4 o[R];
};

// Page-table entries of the JT pages this wave reads in chunk c (independent
// of kv_len, so they can be fetched up front; only x.pt_row is used).
// t = threadIdx.x, passed in so that a caller looping over chunks can keep
// the lane-derived arithmetic inside its loop.
template <int D>
__device__ __forceinline__ void load_phys(const TileCtx& x, int c,
                                          const int32_t* __restrict__ page_table,
                                          int64_t pt_stride, int (&phys)[ChunkShape<D>::JT], int t) {
    constexpr int JT = ChunkShape<D>::JT;
    const int wave = t >> 6;
#pragma unroll
    for (int u = 0; u < JT; ++u) {
        // an index past the row reads the row's last entry (no branch around
        // the load, so nothing waits for it before its use); every user
        // replaces entries at or past the sequence's page count by page 0
        const int pidx = min(16 * c + JT * wave + u, (int)pt_stride - 1);
        phys[u] = page_table[x.pt_row + pidx];
    }
}

// K fragments (A operand of q.k) of chunk c: page 16c + JT*wave + u, key slot
// lane&15, features 32ks + 8(lane>>4) .. +8.  Pages past the sequence's last
// one read page 0 of the cache instead (no branch around the loads): all
// their keys are past every row's position and masked.
template <int D>
__device__ __forceinline__ void load_k(const TileCtx& x, int c, const int (&phys_in)[ChunkShape<D>::JT],
                                       const bf16_t* __restrict__ kc, int64_t pt_stride, int Hkv,
                                       u32x4 (&kf)[ChunkShape<D>::JT][ChunkShape<D>::KS], int t) {
    constexpr int JT = ChunkShape<D>::JT, KS = ChunkShape<D>::KS;
    const int lane = t & 63, wave = t >> 6, ag = lane >> 4;
#pragma unroll
    for (int u = 0; u < JT; ++u) {
        const int pidx = 16 * c + JT * wave + u;
        const int64_t ph = (pidx < x.n_pages && pidx < pt_stride) ? (int64_t)phys_in[u] : 0;
        const bf16_t* kp = kc + ((ph * Hkv + x.g) * PAGE + (lane & 15)) * D + 8 * ag;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[u][ks] = ld16(kp + 32 * ks);
    }
}

// q fragments of the workgroup's tile -> sh.qf (wave 0 loads and writes them;
// the caller's barrier makes them visible).  A padding row reads the tile's
// first token: every key is masked for it.
template <int D, int G, int R>
__device__ __forceinline__ void stage_q(const TileCtx& x, const bf16_t* __restrict__ q, int Hq,
                                        ChunkLds<D, R>& sh, int t) {
    constexpr int KS = ChunkShape<D>::KS;
    const int lane = t & 63, ar = lane & 15, ag = lane >> 4;
    if (t >= 64) return;
#pragma unroll
    for (int rt = 0; rt < R; ++rt) {
        const RowInfo a_row = row_info<G, R>(16 * rt + ar, x.b, x.g, x.qt, x.q_len, x.q_start, x.kv_len);
        const int64_t tok = a_row.token >= 0 ? a_row.token : x.q_start;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            *reinterpret_cast<u32x4*>(sh.qf + ((rt * KS + ks) * 64 + lane) * 16) =
                ld16(q + (tok * Hq + a_row.head) * D + 32 * ks + 8 * ag);
    }
}

// V page blocks in LDS: [D][16 slots] bf16 per page, the 16-byte half h of
// feature d stored at position h ^ ((d >> 3) & 1).  With that swizzle the 8-byte
// reads of v_frag from 16 consecutive features by four lane groups hit every
// bank once per half wave (unswizzled, features 8 apart share banks).  v_src:
// the source offset (bytes, within a page block) of the 16 bytes that
// global_load_lds lane `lane` of copy `part` (1 KB) puts at part * 1024 + 16 lane.
__device__ __forceinline__ int v_src(int part, int lane) {
    const int d = 32 * part + (lane >> 1), h = lane & 1;
    return d * (PAGE * 2) + ((h ^ ((d >> 3) & 1)) << 4);
}

// V^T fragment (A operand of p.v) from a [page][D][16 slots] block of LDS:
// feature d, the 8 keys of 32-key block kb that lane group ag holds (pages
// 2 kb and 2 kb + 1 of the chunk, slots 4 ag .. 4 ag + 3 of each); with
// MASK, slots at or past the sequence end (chunk-relative key >= nvalid)
// read as zero -- they may hold any bits, NaN included.  MASK is a template
// argument: callers pick the masked loop once per chunk (only a sequence's
// last chunk has such slots), so no fragment read waits behind a branch.
// vlane = V block + d * 32 + 8 ag is formed once per lane (and kept opaque):
// the fragments then differ from it by constants, which the reads carry in
// their offset fields instead of one address register per fragment.
typedef const __attribute__((address_space(3))) char* lds_cptr;
__device__ __forceinline__ lds_cptr v_lane(const char* vbuf, int d, int ag) {
    // slots 4 ag .. 4 ag + 3: half ag >> 1, swizzled, then 8 (ag & 1) bytes in
    lds_cptr p = (lds_cptr)(vbuf + d * (PAGE * 2) + 8 * (ag ^ ((d >> 2) & 2)));
    asm volatile("" : "+v"(p));
    return p;
}
// VP: the byte stride of the page blocks in LDS (D * 32, or more when the
// blocks are spaced apart so that the same slot of different pages falls in
// different banks).
template <int D, bool MASK, int VP = D * PAGE * 2>
__device__ __forceinline__ u32x4 v_frag(lds_cptr vlane, int kb, int ag, int nvalid) {
    lds_cptr p0 = vlane + (2 * kb) * VP;
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 a = *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(p0);
    const u32x2 b = *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(p0 + VP);
    u32x4 v = u32x4{a.x, a.y, b.x, b.y};
    if constexpr (MASK) {
        // dword 2 h + i holds keys 32 kb + 16 h + 4 ag + 2 i, + 1
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int n = nvalid - (32 * kb + 16 * h + 4 * ag);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                if (2 * i + 1 >= n) v[2 * h + i] &= (2 * i < n) ? 0x0000ffffu : 0u;
            }
        }
    }
    return v;
}

// The per-chunk arithmetic shared by decode, short prefill runs and the
// comparator: keys [256c, 256c+256) of the tile's sequence, each row limited
// to keys <= its position.  LDS may be reused only after a __syncthreads().
// t = threadIdx.x.  V reaches the matrix cores through LDS, copied while q.k
// runs.  KPRE: kf already holds chunk c's K (requested by the previous
// chunk); once this chunk's V is requested, chunk c_nx's K (c_nx >= 0) is
// requested into kf, to arrive while this chunk's softmax and p.v run.
// Without KPRE chunk c's K is requested here.
template <int D, int G, int R, bool KPRE = false>
__device__ __forceinline__ ChunkOut<R> chunk_compute(
    const TileCtx& x, int c, const int (&phys_in)[ChunkShape<D>::JT],
    const int32_t* __restrict__ page_table, const bf16_t* __restrict__ q,
    const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc, int64_t pt_stride,
    int Hq, int Hkv, float scale_log2, ChunkLds<D, R>& sh, int t,
    u32x4 (&kf)[ChunkShape<D>::JT][ChunkShape<D>::KS], int c_nx = -1,
    const int (&phys_nx)[ChunkShape<D>::JT] = {}) {
    using S = ChunkShape<D>;
    constexpr int NW = S::NW, JT = S::JT, KS = S::KS;
    static_assert(JT % 2 == 0, "a wave's pages form whole 32-key blocks");
    const int lane = t & 63, wave = t >> 6;
    const int ar = lane & 15, ag = lane >> 4;
    const int j0 = c * CHUNK;
    const int g = x.g;
    const int kv_len = x.kv_len;

    // ---- this wave's JT pages; entries past the sequence's last page are not used
    int64_t phys[JT];
#pragma unroll
    for (int u = 0; u < JT; ++u) {
        const int pidx = 16 * c + JT * wave + u;
        phys[u] = (pidx < x.n_pages && pidx < pt_stride) ? (int64_t)phys_in[u] : 0;
    }

    // ---- Q fragments (B operand) of each row tile: row 16 rt + (lane&15),
    // features 32ks + 8(lane>>4) .. +8.  A padding row (no token) reads the
    // tile's first token instead of branching around its load: every key is
    // masked for it (position -1), so its scores, p and partial are never
    // used, and no row's result depends on another row's q.
    u32x4 qf[R][KS];
    if constexpr (KPRE) {
        // a looping workgroup's q, staged in LDS once (stage_q)
#pragma unroll
        for (int rt = 0; rt < R; ++rt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[rt][ks] = *reinterpret_cast<const u32x4*>(sh.qf + ((rt * KS + ks) * 64 + lane) * 16);
    } else {
#pragma unroll
        for (int rt = 0; rt < R; ++rt) {
            const RowInfo a_row = row_info<G, R>(16 * rt + ar, x.b, g, x.qt, x.q_len, x.q_start, kv_len);
            const int64_t tok = a_row.token >= 0 ? a_row.token : x.q_start;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[rt][ks] = ld16(q + (tok * Hq + a_row.head) * D + 32 * ks + 8 * ag);
        }
    }
    // ---- K fragments (A operand of q.k)
    if constexpr (!KPRE) load_k<D>(x, c, phys_in, kc, pt_stride, Hkv, kf, t);

    // ---- S^T = K Q^T on the matrix cores: tile (rt, u) holds, in lane
    // (ag, ar), row 16 rt + ar against keys 16 (JT wave + u) + 4 ag + e
    f32x4 s[R][JT];
#pragma unroll
    for (int rt = 0; rt < R; ++rt)
#pragma unroll
        for (int u = 0; u < JT; ++u) {
            s[rt][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) s[rt][u] = mfma16x16x32(kf[u][ks], qf[rt][ks], s[rt][u]);
        }
#pragma unroll
    for (int rt = 0; rt < R; ++rt)
#pragma unroll
        for (int u = 0; u < JT; ++u) asm volatile("" : "+v"(s[rt][u]) : : "memory");
    // ---- V page blocks of the same JT pages -> LDS (4 KB at D = 128, 2 KB at
    // D = 64, 1 KB per instruction), requested once the q.k products are
    // issued (the fence ties the scores to this point), so that q.k waits for
    // q and K only and V arrives while the scores are masked, reduced and
    // turned into p.  Pages past the sequence end copy page 0 of the cache;
    // all their slots are >= kv_len and are zeroed when read.
#pragma unroll
    for (int u = 0; u < JT; ++u) {
        const int pl = JT * wave + u;                      // page within the chunk
        const char* src = reinterpret_cast<const char*>(vc + (phys[u] * Hkv + g) * (D * PAGE));
#pragma unroll
        for (int part = 0; part < D * PAGE * 2 / 1024; ++part)
            __builtin_amdgcn_global_load_lds(
                (const void*)(src + v_src(part, lane)),
                (__attribute__((address_space(3))) void*)(sh.v + pl * (D * PAGE * 2) + part * 1024),
                16, 0, 0);
    }
    // ---- the next chunk's K, requested after this chunk's V (loads retire in
    // issue order: the wait for V below leaves these JT*KS loads in flight)
    constexpr int KPRE_LOADS = KPRE ? JT * KS : 0;
    const bool kpre = KPRE && c_nx >= 0;
    if constexpr (KPRE) {
        asm volatile("" ::: "memory");
        if (kpre) load_k<D>(x, c_nx, phys_nx, kc, pt_stride, Hkv, kf, t);
    }

    // ---- mask (key <= the row's position), row max of the raw scores: over
    // the lane's keys, its row's four lane groups, then the waves (through LDS)
    const int key_lane = j0 + 16 * JT * wave + 4 * ag;     // + 16 u + e
    ChunkOut<R> r;
#pragma unroll
    for (int rt = 0; rt < R; ++rt) {
        const int rpos = row_info<G, R>(16 * rt + ar, x.b, g, x.qt, x.q_len, x.q_start, kv_len).pos;
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < JT; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool valid = key_lane + 16 * u + e <= rpos;
                const float v = valid ? s[rt][u][e] : -INFINITY;
                s[rt][u][e] = v;
                mx = fmaxf(mx, v);
            }
        // max is exact, so the exchange order does not reach the bits
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (ag == 0) sh.red_max[wave][16 * rt + ar] = mx;
    }
    lds_barrier();     // every wave's row maxima visible (V may still be in flight)
#pragma unroll
    for (int rt = 0; rt < R; ++rt) {
        float mm = sh.red_max[0][16 * rt + ar];
#pragma unroll
        for (int w = 1; w < NW; ++w) mm = fmaxf(mm, sh.red_max[w][16 * rt + ar]);
        r.m[rt] = mm * scale_log2;
    }

    // ---- P = bf16(2^(s c - m)) into LDS as p.v operand: this wave's tiles
    // 2 kb, 2 kb + 1 form block kb of the key order above
#pragma unroll
    for (int rt = 0; rt < R; ++rt)
#pragma unroll
        for (int u2 = 0; u2 < JT / 2; ++u2) {
            const int kb = (JT / 2) * wave + u2;
            u32x4 pk;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    float pp[2];
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const float v = s[rt][2 * u2 + h][2 * i + k];
                        pp[k] = (v == -INFINITY) ? 0.0f : p_of(v, scale_log2, r.m[rt]);
                    }
                    pk[2 * h + i] = p_pack(pp[0], pp[1]);
                }
            *reinterpret_cast<u32x4*>(sh.p + ((rt * 8 + kb) * 64 + lane) * 16) = pk;
        }
    if (kpre)                                          // this wave's V copies landed
        asm volatile("s_waitcnt vmcnt(%0)" :: "n"(KPRE_LOADS) : "memory");
    else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();     // p and every wave's V pages visible

    // ---- l of each row (key order above) and O^T = V^T P^T on the matrix
    // cores, 32-key blocks ascending; the wave owns features 16 wave .. + 15
    const lds_cptr vl = v_lane(sh.v, 16 * wave + ar, ag);
    auto pv = [&](auto masked) {
#pragma unroll
        for (int rt = 0; rt < R; ++rt) {
            r.o[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
            float acc = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                const u32x4 pb = *reinterpret_cast<const u32x4*>(sh.p + ((rt * 8 + kb) * 64 + lane) * 16);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc = l_add(pb[i], acc);
                const u32x4 v = v_frag<D, decltype(masked)::value>(vl, kb, ag, kv_len - j0);
                r.o[rt] = mfma16x16x32(v, pb, r.o[rt]);
            }
            acc += __shfl_xor(acc, 16);
            acc += __shfl_xor(acc, 32);
            r.l[rt] = acc;
        }
    };
    if (j0 + CHUNK > kv_len) pv(std::true_type{});
    else pv(std::false_type{});
    return r;
}

struct Partial {
    float m, l;
    float o[2];
};

// left-to-right combine of two partials (m in the log2 domain):
//   m = max(ma, mb); fa = 2^(ma - m); fb = 2^(mb - m);
//   l = fa la + fb lb; o = fa oa + fb ob   (one fmaf each, product fb x first)
// Every combine of the merge tree, wherever it runs, is this function.  The
// powers of two use the hardware v_exp_f32 (exact at 0, giving 1, and 0 at
// -inf, so merging with the identity (-inf, 0, 0) returns the other operand;
// weights below 2^-126 flush to 0, far below what an fp32 sum can register).
__device__ __forceinline__ void combine_scale(float ma, float mb, float& m, float& fa, float& fb) {
    m = fmaxf(ma, mb);
    fa = __builtin_amdgcn_exp2f(ma - m);
    fb = __builtin_amdgcn_exp2f(mb - m);
}
__device__ __forceinline__ float combine_val(float fa, float a, float fb, float b) {
    return fmaf(fa, a, fb * b);
}

template <int NO>
__device__ __forceinline__ Partial combine(const Partial& a, const Partial& b) {
    Partial r;
    float fa, fb;
    combine_scale(a.m, b.m, r.m, fa, fb);
    r.l = combine_val(fa, a.l, fb, b.l);
#pragma unroll
    for (int i = 0; i < NO; ++i) r.o[i] = combine_val(fa, a.o[i], fb, b.o[i]);
    return r;
}

// the same combine on chunk results as a workgroup holds them (per lane one
// row: its max, sum and four features)
template <int R>
__device__ __forceinline__ ChunkOut<R> combine_out(const ChunkOut<R>& a, const ChunkOut<R>& b) {
    ChunkOut<R> r;
#pragma unroll
    for (int rt = 0; rt < R; ++rt) {
        float fa, fb;
        combine_scale(a.m[rt], b.m[rt], r.m[rt], fa, fb);
        r.l[rt] = combine_val(fa, a.l[rt], fb, b.l[rt]);
#pragma unroll
        for (int e = 0; e < 4; ++e) r.o[rt][e] = combine_val(fa, a.o[rt][e], fb, b.o[rt][e]);
    }
    return r;
}

}  // namespace attn
}  // namespace binv
