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
#include "common.hpp"

namespace binv {
namespace attn {

constexpr int CHUNK = 256;
constexpr int PAGE = 16;
constexpr int NT = 256;
constexpr int ROWS = 16;           // rows of one MFMA row tile
constexpr int STACK = 10;          // binary counter slots: enough for 1023 leaves

// p = 2^(s - m) of a score, s <= m: the hardware v_exp_f32 as it stands.
// exp2f adds a range reduction that keeps results below 2^-126 (weights more
// than 126 binary orders under the row's largest) as fp32 denormals, five
// more vector instructions per score; every kernel that forms p (decode, the
// prefill block and chunk paths, the tuned comparator) calls this one
// function, so they agree bit for bit.
__device__ __forceinline__ float exp2_score(float x) { return __builtin_amdgcn_exp2f(x); }


__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Workgroup barrier for LDS data only: this wave's LDS accesses done, then
// s_barrier.  Unlike __syncthreads() it does not wait for global loads, so a
// V copy requested before it stays in flight.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// P tile in LDS: [16 R rows][256 keys] bf16, rows of 512 bytes = 32 chunks of
// 16 bytes; chunk ch of row r is stored at position ch ^ (r & 31).
__device__ __forceinline__ int p_off(int r, int ch) { return (r << 9) + ((ch ^ (r & 31)) << 4); }

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

template <int D, int R, bool VL>
struct ChunkLds {
    // with VL: the chunk's 16 V page blocks of this KV head, [page][D][16 slots]
    // bf16, copied HBM -> LDS by global_load_lds (one 1 KB piece per instruction)
    __attribute__((aligned(1024))) char v[VL ? 16 * D * PAGE * 2 : 16];
    __attribute__((aligned(16))) char p[ROWS * R * CHUNK * 2];
    float red_max[ChunkShape<D>::NW][ROWS * R];
    // q fragments of the tile for a workgroup that loops over chunks (its rows
    // do not change): [row tile][k-step][lane] 16 bytes each
    __attribute__((aligned(16))) char qf[R * ChunkShape<D>::KS * 64 * 16];
};

// Result of one chunk for the workgroup's 16R rows:
//   m[rt][e]  max of row 16 rt + 4*(lane>>4) + e (every lane), -inf if the row
//             sees no key
//   o[rt]     p.v of those rows for features 16*wave + (lane&15)
//   l, ml_m   (threads t < 256R with t % 16 == 0) sum of p and max of row t >> 4
template <int R>
struct ChunkOut {
    float m[R][4];
    f32x4 o[R];
    float l, ml_m;
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

// K fragments (B operand of q.k) of chunk c: page 16c + JT*wave + u, key slot
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
template <int D, int G, int R, bool VL>
__device__ __forceinline__ void stage_q(const TileCtx& x, const bf16_t* __restrict__ q, int Hq,
                                        ChunkLds<D, R, VL>& sh, int t) {
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

// The per-chunk arithmetic shared by decode, prefill and the comparator: keys
// [256c, 256c+256) of the tile's sequence, each row limited to keys <= its
// position.  LDS may be reused only after a __syncthreads().  t = threadIdx.x.
// VL: V reaches the matrix cores through LDS (copied while q.k runs; decode)
// or straight from memory into registers after q.k (prefill, where 16R rows
// share each V fragment and LDS is better spent on more workgroups per CU).
// Either way every lane feeds the same V values into the same p.v chain.
// KPRE: kf already holds chunk c's K (requested by the previous chunk); once
// this chunk's V is requested, chunk c_nx's K (c_nx >= 0) is requested into
// kf, to arrive while this chunk's softmax and p.v run.  Without KPRE chunk
// c's K is requested here.
template <int D, int G, int R, bool VL, bool KPRE = false>
__device__ __forceinline__ ChunkOut<R> chunk_compute(
    const TileCtx& x, int c, const int (&phys_in)[ChunkShape<D>::JT],
    const int32_t* __restrict__ page_table, const bf16_t* __restrict__ q,
    const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc, int64_t pt_stride,
    int Hq, int Hkv, float scale_log2, ChunkLds<D, R, VL>& sh, int t,
    u32x4 (&kf)[ChunkShape<D>::JT][ChunkShape<D>::KS], int c_nx = -1,
    const int (&phys_nx)[ChunkShape<D>::JT] = {}) {
    using S = ChunkShape<D>;
    constexpr int NW = S::NW, JT = S::JT, KS = S::KS;
    static_assert(S::NTH >= 256 * R, "one thread per (row, 16-key segment) for l");
    const int lane = t & 63, wave = t >> 6;
    const int ar = lane & 15, ag = lane >> 4;
    const int j0 = c * CHUNK;
    const int g = x.g;
    const int kv_len = x.kv_len;

    // ---- this wave's JT pages; entries past the sequence's last page are not used
    int64_t phys[JT];
    bool page_ok[JT];
#pragma unroll
    for (int u = 0; u < JT; ++u) {
        const int pidx = 16 * c + JT * wave + u;
        page_ok[u] = pidx < x.n_pages && pidx < pt_stride;
        phys[u] = page_ok[u] ? (int64_t)phys_in[u] : 0;
    }

    // ---- Q fragments (A operand) of each row tile: row 16 rt + (lane&15),
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
    // ---- K fragments (B operand of q.k)
    if constexpr (!KPRE) load_k<D>(x, c, phys_in, kc, pt_stride, Hkv, kf, t);


    // ---- S = Q K^T on the matrix cores
    f32x4 s[R][JT];
#pragma unroll
    for (int rt = 0; rt < R; ++rt)
#pragma unroll
        for (int u = 0; u < JT; ++u) {
            s[rt][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) s[rt][u] = mfma16x16x32(qf[rt][ks], kf[u][ks], s[rt][u]);
        }
    if constexpr (VL) {
#pragma unroll
        for (int rt = 0; rt < R; ++rt)
#pragma unroll
            for (int u = 0; u < JT; ++u) asm volatile("" : "+v"(s[rt][u]) : : "memory");
    }
    // ---- V page blocks of the same JT pages -> LDS (4 KB at D = 128, 2 KB at
    // D = 64, 1 KB per instruction), requested once the q.k products are
    // issued (the fence ties the scores to this point), so that q.k waits for
    // q and K only and V arrives while the scores are masked, reduced and
    // turned into p.  Pages past the sequence end copy page 0 of the cache;
    // all their slots are >= kv_len and are zeroed when read.
    if constexpr (VL) {
#pragma unroll
        for (int u = 0; u < JT; ++u) {
            const int pl = JT * wave + u;                      // page within the chunk
            const char* src = reinterpret_cast<const char*>(vc + (phys[u] * Hkv + g) * (D * PAGE));
#pragma unroll
            for (int part = 0; part < D * PAGE * 2 / 1024; ++part)
                __builtin_amdgcn_global_load_lds(
                    (const void*)(src + part * 1024 + 16 * lane),
                    (__attribute__((address_space(3))) void*)(sh.v + pl * (D * PAGE * 2) + part * 1024),
                    16, 0, 0);
        }
    }
    // ---- the next chunk's K, requested after this chunk's V (loads retire in
    // issue order: the wait for V below leaves these JT*KS loads in flight)
    constexpr int KPRE_LOADS = KPRE ? JT * KS : 0;
    const bool kpre = KPRE && c_nx >= 0;
    if constexpr (KPRE) {
        asm volatile("" ::: "memory");
        if (kpre) load_k<D>(x, c_nx, phys_nx, kc, pt_stride, Hkv, kf, t);
    }

    // ---- without VL: V fragments straight into registers, issued once the
    // q.k products are queued: feature d = 16 wave + (lane&15), keys
    // 32ks + 8(lane>>4) .. +8 = page 16c + 2ks + (ag>>1), slots 8(ag&1) .. +8
    u32x4 vreg[VL ? 1 : 8];
    if constexpr (!VL) {
        const int d = 16 * wave + (lane & 15);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int pidx = 16 * c + 2 * ks + (ag >> 1);
            const bool ok = pidx < x.n_pages && pidx < pt_stride;
            const int64_t ph = ok ? (int64_t)page_table[x.pt_row + pidx] : 0;
            vreg[ks] = ok ? ld16(vc + ((ph * Hkv + g) * D + d) * PAGE + 8 * (ag & 1))
                          : u32x4{0u, 0u, 0u, 0u};
        }
    }

    // lane holds rows 16 rt + 4*(lane>>4) + e, key j0 + 16*(JT*wave + u) + (lane&15)
    const int key_lane = j0 + 16 * JT * wave + (lane & 15);
    ChunkOut<R> r;
#pragma unroll
    for (int rt = 0; rt < R; ++rt) {
        float mx[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int rpos = row_info<G, R>(16 * rt + 4 * ag + e, x.b, g, x.qt, x.q_len,
                                            x.q_start, kv_len).pos;
            mx[e] = -INFINITY;
#pragma unroll
            for (int u = 0; u < JT; ++u) {
                const bool valid = key_lane + 16 * u <= rpos;
                const float v = valid ? s[rt][u][e] * scale_log2 : -INFINITY;
                s[rt][u][e] = v;
                mx[e] = fmaxf(mx[e], v);
            }
            {
                // max over the 16 lanes of the row group by DPP row rotations
                // (max is exact, so the exchange order does not reach the bits)
                mx[e] = fmaxf(mx[e], __int_as_float(__builtin_amdgcn_update_dpp(
                                         0, __float_as_int(mx[e]), 0x121, 0xf, 0xf, false)));
                mx[e] = fmaxf(mx[e], __int_as_float(__builtin_amdgcn_update_dpp(
                                         0, __float_as_int(mx[e]), 0x122, 0xf, 0xf, false)));
                mx[e] = fmaxf(mx[e], __int_as_float(__builtin_amdgcn_update_dpp(
                                         0, __float_as_int(mx[e]), 0x124, 0xf, 0xf, false)));
                mx[e] = fmaxf(mx[e], __int_as_float(__builtin_amdgcn_update_dpp(
                                         0, __float_as_int(mx[e]), 0x128, 0xf, 0xf, false)));
            }
        }
        if ((lane & 15) == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) sh.red_max[wave][16 * rt + 4 * ag + e] = mx[e];
        }
    }
    lds_barrier();     // every wave's row maxima visible (V may still be in flight)
#pragma unroll
    for (int rt = 0; rt < R; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * rt + 4 * ag + e;
            float mm = sh.red_max[0][row];
#pragma unroll
            for (int w = 1; w < NW; ++w) mm = fmaxf(mm, sh.red_max[w][row]);
            r.m[rt][e] = mm;
        }

    // ---- P = bf16(exp2(s - m)) into LDS
#pragma unroll
    for (int rt = 0; rt < R; ++rt)
#pragma unroll
        for (int u = 0; u < JT; ++u) {
            const int key = 16 * (JT * wave + u) + (lane & 15);       // key within the chunk
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float v = s[rt][u][e];
                const float p = (v == -INFINITY) ? 0.0f : exp2_score(v - r.m[rt][e]);
                const int row = 16 * rt + 4 * ag + e;
                *reinterpret_cast<bf16_t*>(sh.p + p_off(row, key >> 3) + 2 * (key & 7)) =
                    (bf16_t)f32_to_bf16_branch(p);
            }
        }
    if constexpr (VL) {                                // this wave's V copies landed
        if (kpre)
            asm volatile("s_waitcnt vmcnt(%0)" :: "n"(KPRE_LOADS) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    lds_barrier();     // p, and with VL every wave's V pages, visible

    // ---- l (threads 0 .. 256R-1): thread t sums keys 16(t&15) .. +15 of row t>>4
    // in key order, then a 4-level xor butterfly over the 16 segment sums of the row
    r.l = 0.0f;
    r.ml_m = -INFINITY;
    if (t < 256 * R) {
        const int row = t >> 4, seg = t & 15;
        const u32x4 p0 = *reinterpret_cast<const u32x4*>(sh.p + p_off(row, 2 * seg));
        const u32x4 p1 = *reinterpret_cast<const u32x4*>(sh.p + p_off(row, 2 * seg + 1));
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) { acc += lo_bf16(p0[i]); acc += hi_bf16(p0[i]); }
#pragma unroll
        for (int i = 0; i < 4; ++i) { acc += lo_bf16(p1[i]); acc += hi_bf16(p1[i]); }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) acc += __shfl_xor(acc, off);
        r.l = acc;
        float mm = sh.red_max[0][row];
#pragma unroll
        for (int w = 1; w < NW; ++w) mm = fmaxf(mm, sh.red_max[w][row]);
        r.ml_m = mm;
    }

    // ---- O = P V on the matrix cores, keys ascending; wave owns features 16 wave ..
    // V fragment: feature d = 16 wave + (lane&15), keys 32ks + 8(lane>>4) .. +8,
    // i.e. page 2ks + (ag>>1) of the chunk, slots 8(ag&1) .. +8; slots at or
    // past kv_len read as 0.  Each V fragment serves all R row tiles.
#pragma unroll
    for (int rt = 0; rt < R; ++rt) r.o[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
        const int d = 16 * wave + (lane & 15);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int pl = 2 * ks + (ag >> 1);
            u32x4 v;
            if constexpr (VL)
                v = *reinterpret_cast<const u32x4*>(sh.v + pl * (D * PAGE * 2) + d * (PAGE * 2) + 16 * (ag & 1));
            else
                v = vreg[ks];
            const int nvalid = kv_len - ((16 * c + pl) * PAGE + 8 * (ag & 1));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (2 * i + 1 >= nvalid) v[i] &= (2 * i < nvalid) ? 0x0000ffffu : 0u;
            }
#pragma unroll
            for (int rt = 0; rt < R; ++rt) {
                const u32x4 pa = *reinterpret_cast<const u32x4*>(sh.p + p_off(16 * rt + ar, 4 * ks + ag));
                r.o[rt] = mfma16x16x32(pa, v, r.o[rt]);
            }
        }
    }
    return r;
}

struct Partial {
    float m, l;
    float o[2];
};

// left-to-right combine of two partials (m in the log2 domain):
//   m = max(ma, mb); fa = 2^(ma - m); fb = 2^(mb - m);
//   l = fa la + fb lb; o = fa oa + fb ob   (one fmaf each, product fb x first)
// Every combine of the merge tree, wherever it runs, is this function.
__device__ __forceinline__ void combine_scale(float ma, float mb, float& m, float& fa, float& fb) {
    m = fmaxf(ma, mb);
    fa = exp2f(ma - m);
    fb = exp2f(mb - m);
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

// the same combine on chunk results as a workgroup holds them: per lane the
// o and m of its rows, per l-thread the row's l and max
template <int R>
__device__ __forceinline__ ChunkOut<R> combine_out(const ChunkOut<R>& a, const ChunkOut<R>& b) {
    ChunkOut<R> r;
#pragma unroll
    for (int rt = 0; rt < R; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float fa, fb;
            combine_scale(a.m[rt][e], b.m[rt][e], r.m[rt][e], fa, fb);
            r.o[rt][e] = combine_val(fa, a.o[rt][e], fb, b.o[rt][e]);
        }
    float fa, fb;
    combine_scale(a.ml_m, b.ml_m, r.ml_m, fa, fb);
    r.l = combine_val(fa, a.l, fb, b.l);
    return r;
}

}  // namespace attn
}  // namespace binv
