// attention.hip -- paged decode / prefill attention with a fixed 256-token
// split-KV and a fixed-depth merge tree (gfx950).
//
// Method: devpress.csdn.net explainer of "Defeating Nondeterminism in LLM
// Inference", section 3.3 Attention (split the KV sequence into chunks of a
// FIXED number of tokens, 256 in its example, never into a fixed number of
// chunks; keep cached and new tokens in one reduction so a token's reduction
// does not depend on how its sequence was split across steps);
// tom-jerr.github.io "Batch-Invariant Kernel", section Flash Attention
// (fixed-size Split-KV, partials merged by a binary tree padded to a fixed
// depth, prefill and decode producing bit-identical intermediates).
//
// Kernel 1 (chunk): one workgroup = one sequence b, one KV head g, one tile of
// 16R query rows (16R/G tokens x the G = Hq/Hkv query heads of g); for each
// chunk c = keys [256c, 256c+256) it takes, every row's partial (m, l, o[D])
// of the keys of chunk c that the row may see (key j <= the row's position):
//     s_j = (q . k_j) * scale * log2(e)      (scores kept in the log2 domain)
//     m   = max_j s_j
//     p_j = bf16(exp2(s_j - m))              (0 for keys the row may not see)
//     l   = sum_j p_j                        (fixed order, below)
//     o   = sum_j p_j v_j                    (matrix cores, keys ascending)
// Decode tiles hold one token and hand over nodes of the merge tree (subtrees
// of one or two consecutive chunks, merged in the workgroup); prefill tiles
// hold up to 16R/G consecutive new tokens of one sequence and hand over leaves.
// Kernel 2 (merge): one wave per (token, head) row merges the row's nodes with
// a binary counter, which reproduces exactly the left-aligned binary tree over
// 512 leaves whose padding leaves are the identity (a padding leaf only ever
// meets a real subtree, and merging with the identity returns the real subtree
// bit for bit) -- at whatever level the nodes were handed over.
// out = bf16(o / l).
//
// Why the bits of a row do not depend on the batch: every per-row quantity is
// computed by the same instruction sequence whatever else is in the tile --
//   * q.k and p.v come from v_mfma_f32_16x16x32_bf16 chains over 32-element
//     k-blocks in ascending order; a row's slot in the 16-row tile only
//     decides which lane carries it;
//   * the max is exact;
//   * l is the sum of 16 sequential 16-key sums combined by a 4-level xor
//     butterfly, the same code on every path;
//   * chunk boundaries are absolute positions, so chunked prefill, one-shot
//     prefill and decode see the same chunks;
//   * keys past the sequence end are never loaded as values (V reads of slots
//     >= kv_len are replaced by zeros; no page past the last one is touched).
// A key that one row of a prefill tile may not see but another may (causal
// mask) enters the first row's p.v chain as the product 0 * v, where decode
// has 0 * 0: the two agree except for the sign of an exactly-zero result, so
// outputs are written with -0 turned into +0.
#include "attn_chunk.hpp"
#include "binv.h"
#include "kernels.hpp"

#include <mutex>

namespace binv {

namespace {
using namespace attn;

// workgroups per (query tile, KV head) of a decode sequence; they loop over
// the sequence's nodes
constexpr int CHUNK_LANES = 32;

// Level of the merge tree at which a decode row's partials are handed from
// the chunk kernel to the merge kernel, from the row's chunk count n: the
// level that keeps the longest chain of chunks one workgroup computes in
// sequence, ceil(n / (CHUNK_LANES 2^L)) 2^L, shortest, and among those the
// highest (fewest partials).  Both kernels evaluate it for the row; the root
// is the same for every level.
template <int GMAX>
__device__ __forceinline__ int node_level(int n) {
    int best = 0, best_chain = (n + CHUNK_LANES - 1) / CHUNK_LANES;
#pragma unroll
    for (int L = 1; L <= GMAX; ++L) {
        const int per = CHUNK_LANES << L;
        const int chain = ((n + per - 1) / per) << L;
        if (chain <= best_chain) { best = L; best_chain = chain; }
    }
    return best;
}

// Grid: x = (query tile, KV head), y = lane, z = sequence.
//
// Decode (R = 1, no cu_q) workgroups write nodes of the merge tree at level
// L = node_level(n): node j covers the aligned chunks [2^L j, 2^L (j + 1)).
// Workgroup (x, y, z) takes the nodes j = y, y + gridDim.y, ... that reach
// the sequence's position; for each it computes the node's chunks in order
// and merges them with the merge kernel's binary counter and combine, so the
// node is the subtree value that kernel would have formed from the leaves (a
// node's chunks past the sequence end are identity leaves, which leave a
// subtree unchanged).  Which workgroup takes a node, and the level at which
// the tree is handed over, do not enter any row's arithmetic; a higher level
// writes and re-reads fewer partials.  gridDim.y is capped at CHUNK_LANES, so
// a grid sized for the longest allowed sequence does not spend a workgroup
// per empty node slot of every short sequence.
// Prefill (cu_q given; R = 1, looping): leaves (L = 0), for the sequences of
// a call with fewer than q_skip new tokens (all of them at D = 64, and at
// D = 128 when no run can fill half a 128-row block); longer runs at D = 128
// go to attn_prefill_kernel.  Without looping gridDim.y = the chunk count and
// a workgroup takes chunk y alone.
//
// Partials: slot (row * n_chunks + node) * Hq + head of ws_o [.., D] and
// ws_ml [..] (the G heads of one tile are adjacent), where row is the token,
// or with leaf_seq > 0 the compact b * leaf_seq + i of new token i of
// sequence b (only the short sequences of a call that sends its long runs to
// the block kernel have leaves, fewer than leaf_seq new tokens each).
template <int D, int G, int R, bool LOOP, int GMAX>
__global__ __launch_bounds__(ChunkShape<D>::NTH, D == 128 ? 4 : 3) void attn_chunk_kernel(
    const bf16_t* __restrict__ q, const int32_t* __restrict__ cu_q,
    const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc,
    const int32_t* __restrict__ page_table, int64_t pt_stride,
    const int32_t* __restrict__ kv_lens, float* __restrict__ ws_o,
    float2* __restrict__ ws_ml, int Hq, int Hkv, int n_chunks, int max_kv_len,
    float scale_log2, int q_skip, int leaf_seq) {
    constexpr bool VL = (R == 1);           // V through LDS for single-tile (decode) workgroups
    // prefill: sequences with q_skip or more new tokens belong to the block kernel
    if (cu_q && cu_q[blockIdx.z + 1] - cu_q[blockIdx.z] >= q_skip) return;
    static_assert(LOOP || GMAX == 0, "workgroups that take one chunk write leaves");
    __shared__ ChunkLds<D, R, VL> sh;
    constexpr int JT = ChunkShape<D>::JT;
    const int kv_len_b = kv_lens[blockIdx.z];          // read once, kept in a register
    const int pos_max = tile_ctx_len<G, R>(blockIdx.z, blockIdx.x % Hkv, blockIdx.x / Hkv, cu_q,
                                           kv_len_b, pt_stride, max_kv_len).pos_max;
    const int glog = (GMAX > 0 && !cu_q && pos_max >= 0) ? node_level<GMAX>(pos_max / CHUNK + 1) : 0;
    const int gs = 1 << glog;
    int phys_next[JT];
    // K of the workgroup's current chunk: the first chunk's requested here,
    // every later one by the chunk before it
    u32x4 kf[JT][ChunkShape<D>::KS];
    {
        TileCtx x0;
        x0.pt_row = (int64_t)blockIdx.z * pt_stride;
        load_phys<D>(x0, blockIdx.y * gs, page_table, pt_stride, phys_next, threadIdx.x);
        if (blockIdx.y * gs * CHUNK <= pos_max) {
            const TileCtx x1 = tile_ctx_len<G, R>(blockIdx.z, blockIdx.x % Hkv, blockIdx.x / Hkv,
                                                  cu_q, kv_len_b, pt_stride, max_kv_len);
            load_k<D>(x1, blockIdx.y * gs, phys_next, kc, pt_stride, Hkv, kf, threadIdx.x);
            // the tile's q, the same for every chunk, staged in LDS once
            if constexpr (LOOP) {
                stage_q<D, G, R, VL>(x1, q, Hq, sh, threadIdx.x);
                lds_barrier();
            }
        }
    }
#pragma clang loop unroll(disable)
    for (int node = blockIdx.y; node * gs * CHUNK <= pos_max; node += gridDim.y) {
        ChunkOut<R> slot[GMAX + 1];
        unsigned count = 0;
#pragma clang loop unroll(disable)
        for (int i = 0; i < gs; ++i) {
            const int c = node * gs + i;
            if (c * CHUNK > pos_max) break;
            // the tile context, q fragments, row maps and lane-derived
            // addresses are re-derived per chunk (a few ALU operations and
            // cache hits) rather than held live across chunks, which would spill
            asm volatile("" ::: "memory");
            int t = threadIdx.x;
            if constexpr (LOOP) asm volatile("" : "+v"(t));
            const TileCtx x = tile_ctx_len<G, R>(blockIdx.z, blockIdx.x % Hkv, blockIdx.x / Hkv,
                                                 cu_q, kv_len_b, pt_stride, max_kv_len);
            int phys[JT];
#pragma unroll
            for (int u = 0; u < JT; ++u) phys[u] = phys_next[u];
            // the next chunk this workgroup takes: its page-table entries now,
            // its K once this chunk's V is requested
            int c_nx = -1;
            if constexpr (LOOP) {
                const int c_next = (i + 1 < gs) ? c + 1 : (node + (int)gridDim.y) * gs;
                if (c_next * CHUNK <= pos_max) {
                    load_phys<D>(x, c_next, page_table, pt_stride, phys_next, t);
                    c_nx = c_next;
                }
            }
            ChunkOut<R> carry = chunk_compute<D, G, R, VL, LOOP>(
                x, c, phys, page_table, q, kc, vc, pt_stride, Hq, Hkv, scale_log2, sh, t, kf, c_nx,
                phys_next);
            // binary increment: equal-size subtrees merge, the older one on the left
            bool live = true;
#pragma unroll
            for (int s = 0; s <= GMAX; ++s) {
                if (live) {
                    if (count & (1u << s)) {
                        carry = combine_out<R>(slot[s], carry);
                    } else {
                        slot[s] = carry;
                        live = false;
                    }
                }
            }
            ++count;
            if constexpr (LOOP) __syncthreads();           // LDS free for the next chunk
        }
        // the node: remaining subtrees, smallest (rightmost) first
        ChunkOut<R> r = slot[0];
        bool have = false;
#pragma unroll
        for (int s = 0; s <= GMAX; ++s) {
            if (count & (1u << s)) {
                if (!have) { r = slot[s]; have = true; }
                else r = combine_out<R>(slot[s], r);
            }
        }
        int t = threadIdx.x;
        if constexpr (LOOP) asm volatile("" : "+v"(t));
        const int lane = t & 63, wave = t >> 6, ag = lane >> 4;
        const TileCtx x = tile_ctx_len<G, R>(blockIdx.z, blockIdx.x % Hkv, blockIdx.x / Hkv, cu_q,
                                             kv_len_b, pt_stride, max_kv_len);
        const int j0 = node * gs * CHUNK;
        // partials of the rows that see at least one key of this node
#pragma unroll
        for (int rt = 0; rt < R; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const RowInfo ri = row_info<G, R>(16 * rt + 4 * ag + e, x.b, x.g, x.qt, x.q_len,
                                                  x.q_start, x.kv_len);
                if (ri.token < 0 || ri.pos < j0) continue;
                const int64_t lr = leaf_seq ? (int64_t)x.b * leaf_seq + (ri.token - x.q_start) : ri.token;
                const int64_t slot_i = (lr * n_chunks + node) * Hq + ri.head;
                ws_o[slot_i * D + 16 * wave + (lane & 15)] = r.o[rt][e];
            }
        if (t < 256 * R && (t & 15) == 0) {
            const RowInfo ri = row_info<G, R>(t >> 4, x.b, x.g, x.qt, x.q_len, x.q_start, x.kv_len);
            if (ri.token >= 0 && ri.pos >= j0) {
                const int64_t lr = leaf_seq ? (int64_t)x.b * leaf_seq + (ri.token - x.q_start) : ri.token;
                const int64_t slot_i = (lr * n_chunks + node) * Hq + ri.head;
                ws_ml[slot_i] = make_float2(r.ml_m, r.l);
            }
        }
        if constexpr (!LOOP) break;
    }
}

// Prefill at D = 128: one workgroup = one sequence, one KV head, a block of
// 128 query rows (128/G new tokens x the G query heads), walking every chunk
// the block's rows see, in order, and writing the finished output rows.  Each
// of the eight waves owns one 16-row tile outright -- per chunk its q.k over
// all 256 keys, row max, p, l and p.v for all 128 features -- so rows need no
// cross-wave reduction; each chunk's K and V pages are copied HBM -> LDS once
// (global_load_lds) and read by all eight tiles, so 128 rows share one load
// of the chunk where a chunk-kernel workgroup shares it among 16.  Every
// per-element operation is the chunk kernel's, in the same order: q.k as
// v_mfma_f32_16x16x32_bf16 over features 32ks + 8(lane>>4) .. +8, ks
// ascending; scale, mask, exact max; p = bf16(exp2(s - m)); l = sixteen
// sequential 16-key sums combined as the pairwise tree ((s0+s1)+(s2+s3)) +
// ... (what the chunk kernel's xor butterfly forms); p.v over keys 32ks +
// 8(lane>>4) .. +8, ks ascending, V slots at or past kv_len read as zero --
// so a row's chunk partial has the same bits as from the chunk kernel.
// The partials are merged in the workgroup as they come, by the merge
// kernel's binary counter and combine (the left-aligned tree padded to a fixed
// depth): the counter's lowest slot (a single chunk) stays in registers, the
// higher slots (subtrees of 2, 4, ... chunks) go to a per-row stack in the
// workspace, [token][level][head], so the workspace grows with the logarithm
// of the KV length and only every second chunk's subtree leaves the
// workgroup.  The rows of a block see the same chunks except that a block
// crossing a chunk boundary has rows that do not reach its last chunk: their
// partial of that chunk has every key masked (max -inf, sum 0, values 0), the
// identity of the merge, so every row pushes every chunk (one counter for the
// block) and the root is the same as from the row's own leaves (merging with
// the identity is exact; the sign of an exactly-zero value is normalised at
// the output).  The root o / l, bf16, is the merge kernel's last step; so a
// prefill row equals the decode of the same position bit for bit.
// LDS: K [16 pages][16 keys][128] with 16-byte chunk c of key k at c ^ (k & 15);
// V [16 pages][128 features][16 slots] with the 16-byte half h of feature d
// at h ^ ((d >> 3) & 1); once every tile has its scores, the K area holds each
// tile's p [16 rows][256 keys] (8 KB per wave, the chunk kernel's swizzle).
// The q area holds the block's 128 query rows for all chunks.
constexpr int PF_WAVES = 8;
constexpr int PF_ROWS = 16 * PF_WAVES;

// a chunk partial (or a subtree of them) of a wave's 16 rows as the block
// kernel holds it: the max of rows 4(lane>>4) + e (me) and of row lane & 15
// (mr), the sum of weights of row lane & 15 (lr), and the weighted values of
// rows 4(lane>>4) + e, features 16 f + (lane & 15) (o)
struct PfNode {
    float me[4];
    float mr, lr;
    f32x4 o[8];
};

// the merge kernel's combine (combine_scale, combine_val), a on the left
__device__ __forceinline__ PfNode pf_combine(const PfNode& a, const PfNode& b) {
    PfNode r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float fa, fb;
        combine_scale(a.me[e], b.me[e], r.me[e], fa, fb);
#pragma unroll
        for (int f = 0; f < 8; ++f) r.o[f][e] = combine_val(fa, a.o[f][e], fb, b.o[f][e]);
    }
    float fa, fb;
    combine_scale(a.mr, b.mr, r.mr, fa, fb);
    r.lr = combine_val(fa, a.lr, fb, b.lr);
    return r;
}

template <int G>
__global__ __launch_bounds__(64 * PF_WAVES) void attn_prefill_kernel(
    const bf16_t* __restrict__ q, const int32_t* __restrict__ cu_q,
    const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc,
    const int32_t* __restrict__ page_table, int64_t pt_stride,
    const int32_t* __restrict__ kv_lens, bf16_t* __restrict__ out,
    float* __restrict__ st_o, float2* __restrict__ st_ml, int Hq, int Hkv, int st_stride,
    int max_kv_len, float scale_log2, int q_min, int nqb) {
    constexpr int D = 128, KS = D / 32, NKT = CHUNK / 16;
    // sequences with fewer than q_min new tokens belong to the chunk kernel
    if (cu_q[blockIdx.z + 1] - cu_q[blockIdx.z] < q_min) return;
    // one object, so that the compiler can tell the V copy's destination from
    // the q and K areas read while it is in flight
    struct PfLds {
        __attribute__((aligned(1024))) char k[16 * PAGE * D * 2];   // K, then p
        __attribute__((aligned(1024))) char v[16 * D * PAGE * 2];
        // q of the block's 128 rows [row][D], 16-byte chunk c of row r at c ^ (r & 15)
        __attribute__((aligned(1024))) char q[PF_ROWS * D * 2];
    };
    __shared__ PfLds sh;
    char* const kbuf = sh.k;
    char* const vbuf = sh.v;
    char* const qbuf = sh.q;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    // blocks in reverse order: the blocks that see the most chunks start first
    const int g = blockIdx.x % Hkv, qb = nqb - 1 - (int)(blockIdx.x / Hkv), b = blockIdx.z;
    const TileCtx x = tile_ctx<G, PF_WAVES>(b, g, qb, cu_q, kv_lens, pt_stride, max_kv_len);
    if (x.pos_max < 0) return;                        // no row in this block
    const int kv_len = x.kv_len;
    const int nc = x.pos_max / CHUNK + 1;             // chunks the block's rows see
    // The lane index and everything derived from it (LDS and HBM addresses,
    // row maps) are re-derived in every chunk from an opaque copy of the
    // thread index: hoisted out of the chunk loop, the many per-lane addresses
    // would stay live across it and spill.
    auto lane_id = []() {
        int t = threadIdx.x;
        asm volatile("" : "+v"(t));
        return t & 63;
    };
    auto row = [&](int r) {
        return row_info<G, PF_WAVES>(16 * wave + r, b, g, qb, x.q_len, x.q_start, kv_len);
    };

    // ---- the block's q rows HBM -> LDS (a row without a token copies the
    // block's first token: every key is masked for it)
    {
        const int lane = lane_id();
        const char* qsrc[4];
#pragma unroll
        for (int part = 0; part < 4; ++part) {
            // LDS position part*1024 + 16 lane: row 4 part + lane / 16 of the wave's
            // tile, chunk lane & 15 holding feature chunk (lane & 15) ^ row
            const int rr = 4 * part + (lane >> 4);
            const RowInfo ri = row(rr);
            const int64_t tok = ri.token >= 0 ? ri.token : x.q_start;
            qsrc[part] = reinterpret_cast<const char*>(q + (tok * Hq + ri.head) * D) +
                         (((lane & 15) ^ rr) << 4);
        }
#pragma unroll
        for (int part = 0; part < 4; ++part)
            __builtin_amdgcn_global_load_lds(
                (const void*)qsrc[part],
                (__attribute__((address_space(3))) void*)(qbuf + wave * (16 * D * 2) + part * 1024),
                16, 0, 0);
    }
    // K and then V pages 2 wave, 2 wave + 1 of chunk c (pages past the
    // sequence copy page 0 of the cache: their keys are masked, their V slots
    // read as zero).  Copies retire in issue order, so q.k waits for K while V
    // is in flight.
    auto copy_kv = [&](int c, int lane) {
        const char* ksrc[2];
        const char* vsrc[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int pidx = 16 * c + 2 * wave + u;
            const bool ok = pidx < x.n_pages && pidx < pt_stride;
            const int64_t ph = ok ? (int64_t)page_table[x.pt_row + pidx] : 0;
            ksrc[u] = reinterpret_cast<const char*>(kc + (ph * Hkv + g) * (PAGE * D));
            vsrc[u] = reinterpret_cast<const char*>(vc + (ph * Hkv + g) * (D * PAGE));
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int pl = 2 * wave + u;
#pragma unroll
            for (int part = 0; part < 4; ++part) {
                // LDS position part*1024 + 16 lane: key 4 part + lane / 16, chunk lane & 15
                const int key = 4 * part + (lane >> 4), pos = lane & 15;
                __builtin_amdgcn_global_load_lds(
                    (const void*)(ksrc[u] + key * (D * 2) + ((pos ^ key) << 4)),
                    (__attribute__((address_space(3))) void*)(kbuf + pl * (PAGE * D * 2) + part * 1024),
                    16, 0, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int pl = 2 * wave + u;
#pragma unroll
            for (int part = 0; part < 4; ++part) {
                // LDS position part*1024 + 16 lane: feature 32 part + lane / 2, half lane & 1
                const int d = 32 * part + (lane >> 1), h = lane & 1;
                __builtin_amdgcn_global_load_lds(
                    (const void*)(vsrc[u] + d * (PAGE * 2) + ((h ^ ((d >> 3) & 1)) << 4)),
                    (__attribute__((address_space(3))) void*)(vbuf + pl * (D * PAGE * 2) + part * 1024),
                    16, 0, 0);
            }
        }
    };
    copy_kv(0, lane_id());
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");  // this wave's q and K copies landed
    lds_barrier();                                    // every wave's: q and K of the block in LDS

    // ---- the per-row stack of the counter's slots >= 1: level s of a row at
    // ((token * st_stride + s - 1) * Hq + head); each lane stores and loads only
    // the values it holds (o of rows 4(lane>>4) + e; (max, sum) of row lane & 15
    // by the lanes of group 0, passed to the other lanes by shuffles)
    auto slot_of = [&](int r, int s) -> int64_t {
        const RowInfo ri = row(r);
        return ri.token < 0 ? (int64_t)-1 : ((ri.token * st_stride + (s - 1)) * Hq + ri.head);
    };
    auto stack_store = [&](int s, const PfNode& nd, int lane) {
        const int ar = lane & 15, ag = lane >> 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t sl = slot_of(4 * ag + e, s);
            if (sl < 0) continue;
#pragma unroll
            for (int f = 0; f < 8; ++f) st_o[sl * D + 16 * f + ar] = nd.o[f][e];
        }
        if (ag == 0) {
            const int64_t sl = slot_of(ar, s);
            if (sl >= 0) st_ml[sl] = make_float2(nd.mr, nd.lr);
        }
    };
    auto stack_load = [&](int s, int lane) -> PfNode {
        const int ar = lane & 15, ag = lane >> 4;
        PfNode nd;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t sl = slot_of(4 * ag + e, s);
#pragma unroll
            for (int f = 0; f < 8; ++f) nd.o[f][e] = sl < 0 ? 0.0f : st_o[sl * D + 16 * f + ar];
        }
        float2 ml = make_float2(-INFINITY, 0.0f);
        if (ag == 0) {
            const int64_t sl = slot_of(ar, s);
            if (sl >= 0) ml = st_ml[sl];
        }
        nd.mr = __shfl(ml.x, ar);
        nd.lr = __shfl(ml.y, ar);
#pragma unroll
        for (int e = 0; e < 4; ++e) nd.me[e] = __shfl(ml.x, 4 * ag + e);
        return nd;
    };

    PfNode slot0;
    unsigned count = 0;
#pragma clang loop unroll(disable)
    for (int c = 0; c < nc; ++c) {
        const int j0 = c * CHUNK;
        const int lane = lane_id(), ar = lane & 15, ag = lane >> 4;
        if (c > 0) {
            copy_kv(c, lane);
            asm volatile("s_waitcnt vmcnt(8)" ::: "memory");  // this wave's K copies landed
            lds_barrier();                                    // every wave's
        }
        int rpos[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) rpos[e] = row(4 * ag + e).pos;
        char* const pt = kbuf + wave * (16 * CHUNK * 2);     // this tile's p

        // ---- S = Q K^T: key tile kt holds keys 16 kt .. 16 kt + 15 of the
        // chunk; q fragments: row 16 wave + (lane & 15), features 32 ks +
        // 8 (lane >> 4) .. +8
        f32x4 sc[NKT];
        {
            u32x4 qf[KS];
            const char* qrow = qbuf + (16 * wave + ar) * (D * 2);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[ks] = *reinterpret_cast<const u32x4*>(qrow + (((4 * ks + ag) ^ ar) << 4));
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                sc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
                const char* krow = kbuf + (16 * kt + ar) * (D * 2);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const u32x4 kf = *reinterpret_cast<const u32x4*>(krow + (((4 * ks + ag) ^ ar) << 4));
                    sc[kt] = mfma16x16x32(qf[ks], kf, sc[kt]);
                }
            }
        }
        // scale, mask (key <= the row's position), row max over the 256 keys,
        // then p = bf16(2^(s - m)) into this tile's 8 KB of the K area.  Below
        // the diagonal every key of the chunk is valid for every row of the
        // wave and the mask is left out; the two versions are separate
        // wave-uniform paths (same values), each with the one barrier that
        // frees the K area.  p = 0 for a masked key comes from 2^(-inf - m): a
        // row whose keys are all masked (m = -inf) takes m = 0 there, which
        // gives p = 0 as well -- the per-score test v == -inf of the chunk
        // kernel, per row instead.
        float mx[4];
        auto softmax = [&](auto masked) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                mx[e] = -INFINITY;
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) {
                    float v = sc[kt][e] * scale_log2;
                    if constexpr (decltype(masked)::value) {
                        if (j0 + 16 * kt + ar > rpos[e]) v = -INFINITY;
                    }
                    sc[kt][e] = v;
                    mx[e] = fmaxf(mx[e], v);
                }
                // max over the 16 lanes of the row group: rotations by 1, 2, 4, 8
                // within each 16-lane DPP row (max is exact, so the order of the
                // exchange does not matter)
                mx[e] = fmaxf(mx[e], __int_as_float(__builtin_amdgcn_update_dpp(
                                         0, __float_as_int(mx[e]), 0x121, 0xf, 0xf, false)));
                mx[e] = fmaxf(mx[e], __int_as_float(__builtin_amdgcn_update_dpp(
                                         0, __float_as_int(mx[e]), 0x122, 0xf, 0xf, false)));
                mx[e] = fmaxf(mx[e], __int_as_float(__builtin_amdgcn_update_dpp(
                                         0, __float_as_int(mx[e]), 0x124, 0xf, 0xf, false)));
                mx[e] = fmaxf(mx[e], __int_as_float(__builtin_amdgcn_update_dpp(
                                         0, __float_as_int(mx[e]), 0x128, 0xf, 0xf, false)));
            }
            lds_barrier();                            // every tile done with K: its area takes p
            float mu[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) mu[e] = (mx[e] == -INFINITY) ? 0.0f : mx[e];
            // p_off(row, key >> 3) + 2 (key & 7) with row = 4 ag + e, key = 16 kt + ar:
            // (key >> 3) ^ row = 2 kt ^ ((ar >> 3) ^ row), so the byte offset is a
            // per-row base plus (32 kt) ^ z -- one xor-add per store
            int base[4], z[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * ag + e;
                base[e] = (r << 9) + 2 * (ar & 7);
                z[e] = ((ar >> 3) ^ (r & 31)) << 4;
            }
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p = exp2_score(sc[kt][e] - mu[e]);
                    *reinterpret_cast<bf16_t*>(pt + (((32 * kt) ^ z[e]) + base[e])) =
                        (bf16_t)f32_to_bf16(p);
                }
            }
        };
        if (__all(j0 + CHUNK - 1 <= min(min(rpos[0], rpos[1]), min(rpos[2], rpos[3]))))
            softmax(std::false_type{});
        else
            softmax(std::true_type{});
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the tile's p, read below by its own wave

        // ---- l of row ar: segments 4(lane>>4) .. +3 summed key by key, then the
        // pairwise tree over the 16 segment sums
        float lrow;
        {
            float seg[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int sg = 4 * ag + k;
                const u32x4 p0 = *reinterpret_cast<const u32x4*>(pt + p_off(ar, 2 * sg));
                const u32x4 p1 = *reinterpret_cast<const u32x4*>(pt + p_off(ar, 2 * sg + 1));
                float acc = 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) { acc += lo_bf16(p0[i]); acc += hi_bf16(p0[i]); }
#pragma unroll
                for (int i = 0; i < 4; ++i) { acc += lo_bf16(p1[i]); acc += hi_bf16(p1[i]); }
                seg[k] = acc;
            }
            float c4 = (seg[0] + seg[1]) + (seg[2] + seg[3]);
            c4 += __shfl_xor(c4, 16);
            c4 += __shfl_xor(c4, 32);
            lrow = c4;
        }

        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's V copies landed
        lds_barrier();                                    // every wave's: V of the chunk in LDS

        // ---- O = P V: feature tile f holds features 16 f .. 16 f + 15; keys
        // ascending in k-blocks of 32 per (tile, f)
        PfNode leaf;
        {
            u32x4 pa[8];
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
                pa[ks] = *reinterpret_cast<const u32x4*>(pt + p_off(ar, 4 * ks + ag));
            // V slots at or past kv_len exist only in the sequence's last chunk;
            // in every other chunk the zeroing is skipped (block-uniform branch)
            auto pv = [&](auto masked) {
#pragma unroll
                for (int f = 0; f < D / 16; ++f) {
                    leaf.o[f] = f32x4{0.f, 0.f, 0.f, 0.f};
                    const int d = 16 * f + ar;
#pragma unroll
                    for (int ks = 0; ks < 8; ++ks) {
                        const int pl = 2 * ks + (ag >> 1), h = ag & 1;
                        u32x4 v = *reinterpret_cast<const u32x4*>(
                            vbuf + pl * (D * PAGE * 2) + d * (PAGE * 2) + ((h ^ ((d >> 3) & 1)) << 4));
                        if constexpr (decltype(masked)::value) {
                            const int nvalid = kv_len - ((16 * c + pl) * PAGE + 8 * h);
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                if (2 * i + 1 >= nvalid) v[i] &= (2 * i < nvalid) ? 0x0000ffffu : 0u;
                            }
                        }
                        leaf.o[f] = mfma16x16x32(pa[ks], v, leaf.o[f]);
                    }
                }
            };
            if (j0 + CHUNK > kv_len) pv(std::true_type{});
            else pv(std::false_type{});
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) leaf.me[e] = mx[e];
        {
            // the max of row lane & 15, from a lane of its row group
            const int src = 16 * (ar >> 2);
            const float m0 = __shfl(mx[0], src), m1 = __shfl(mx[1], src);
            const float m2 = __shfl(mx[2], src), m3 = __shfl(mx[3], src);
            const int e = ar & 3;
            leaf.mr = e == 0 ? m0 : e == 1 ? m1 : e == 2 ? m2 : m3;
        }
        leaf.lr = lrow;

        // ---- push the chunk into the binary counter: equal-size subtrees
        // merge, the older one on the left (uniform over the block)
        if (!(count & 1u)) {
            slot0 = leaf;
        } else {
            PfNode carry = pf_combine(slot0, leaf);
            int sl = 1;
#pragma clang loop unroll(disable)
            while (count & (1u << sl)) {
                carry = pf_combine(stack_load(sl, lane), carry);
                ++sl;
            }
            stack_store(sl, carry, lane);
        }
        ++count;
        lds_barrier();                                    // K, p and V free for the next chunk
    }

    // ---- the root: remaining subtrees, smallest (rightmost) first
    const int lane = lane_id(), ar = lane & 15, ag = lane >> 4;
    PfNode res = slot0;
    bool have = (count & 1u) != 0;
#pragma clang loop unroll(disable)
    for (int sl = 1; (count >> sl) != 0; ++sl) {
        if (count & (1u << sl)) {
            if (!have) { res = stack_load(sl, lane); have = true; }
            else res = pf_combine(stack_load(sl, lane), res);
        }
    }
    // out = o / l as bf16, an exact zero written as +0 (the merge kernel's last step)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float l = __shfl(res.lr, 4 * ag + e);
        const RowInfo ri = row(4 * ag + e);
        if (ri.token < 0) continue;
        bf16_t* orow = out + (ri.token * Hq + ri.head) * D;
#pragma unroll
        for (int f = 0; f < 8; ++f)
            orow[16 * f + ar] = (bf16_t)f32_to_bf16(res.o[f][e] / l + 0.0f);
    }
}

// A node as the merge holds it: per lane VPL consecutive features of one row.
template <int VPL>
struct MergeNode {
    float m, l;
    float o[VPL];
};
template <int VPL>
__device__ __forceinline__ MergeNode<VPL> combine_node(const MergeNode<VPL>& a,
                                                       const MergeNode<VPL>& b) {
    MergeNode<VPL> r;
    float fa, fb;
    combine_scale(a.m, b.m, r.m, fa, fb);
    r.l = combine_val(fa, a.l, fb, b.l);
#pragma unroll
    for (int i = 0; i < VPL; ++i) r.o[i] = combine_val(fa, a.o[i], fb, b.o[i]);
    return r;
}

constexpr int MERGE_VPL = 4;

// D / VPL lanes per (token, head) row, each owning VPL = 4 consecutive
// features: one 16-byte load per node and lane (single-feature lanes took
// 4 % longer on a 4096-token prefill), 64 VPL / D rows per wave.  SK
// binary-counter slots hold any row of at most 2^SK - 1 nodes.  Prefill rows
// of sequences with q_min or more new tokens were finished by the block
// kernel and are skipped; leaf rows are indexed as the chunk kernel wrote them
// (leaf_seq).
template <int D, int GMAX, int SK>
__global__ __launch_bounds__(NT) void attn_merge_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ kv_lens, int64_t B,
    int64_t n_tokens, int Hq, int n_chunks, int max_kv_len,
    const float* __restrict__ ws_o, const float2* __restrict__ ws_ml, bf16_t* __restrict__ out,
    int q_min, int leaf_seq) {
    constexpr int VPL = MERGE_VPL, LPR = D / VPL, RPW = 64 / LPR;
    static_assert(D % VPL == 0 && 64 % LPR == 0, "");
    typedef float Vec __attribute__((ext_vector_type(VPL)));
    typedef uint32_t Packed __attribute__((ext_vector_type(VPL / 2)));
    using Node = MergeNode<VPL>;
    const int lane = threadIdx.x & 63, sub = lane % LPR;
    const int64_t row = ((int64_t)blockIdx.x * (NT / 64) + (threadIdx.x >> 6)) * RPW + lane / LPR;
    if (row >= n_tokens * Hq) return;
    const int64_t token = row / Hq;

    // the query's absolute position and the row of its leaves
    int pos;
    int64_t leaf_row = token;
    if (cu_q) {
        int64_t lo = 0, hi = B - 1;            // last b with cu_q[b] <= token
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) >> 1;
            if (cu_q[mid] <= token) lo = mid; else hi = mid - 1;
        }
        int kv_len = kv_lens[lo];
        if (kv_len > max_kv_len) kv_len = max_kv_len;
        int q_len = cu_q[lo + 1] - cu_q[lo];
        if (q_len >= q_min) return;
        if (q_len > kv_len) q_len = kv_len;
        const int i = (int)(token - cu_q[lo]);
        pos = (i < q_len) ? kv_len - q_len + i : -1;
        if (leaf_seq) leaf_row = lo * leaf_seq + i;
    } else {
        int kv_len = kv_lens[token];
        if (kv_len > max_kv_len) kv_len = max_kv_len;
        pos = kv_len - 1;
    }
    bf16_t* orow = out + row * D + VPL * sub;
    if (pos < 0) {
        *reinterpret_cast<Packed*>(orow) = Packed(0u);
        return;
    }
    // the row's pos / CHUNK + 1 chunks arrive as nodes of the level the chunk
    // kernel chose for it (leaves for prefill rows)
    int n_leaf = pos / CHUNK + 1;
    if (n_leaf > n_chunks) n_leaf = n_chunks;
    const int glog = (GMAX > 0 && !cu_q) ? node_level<GMAX>(n_leaf) : 0;
    const int n = ((n_leaf - 1) >> glog) + 1;

    // node c of the row: slot (leaf_row * n_chunks + c) * Hq + head
    const int64_t slot0 = leaf_row * n_chunks * Hq + (row - token * Hq);
    const float* po = ws_o + slot0 * D + VPL * sub;
    const float2* pml = ws_ml + slot0;

    Node slot[SK];
    unsigned count = 0;
    // nodes are loaded GRP at a time into two buffers used in turn: while one
    // group is pushed into the binary counter, in node order, the next group's
    // loads are in flight (no register copy between the buffers, so no wait
    // for data that is not yet needed).  Loads past the row's last node read
    // that last node again and are not pushed.
    constexpr int GRP = 4;
    Node ba[GRP], bb[GRP];
    auto load_group = [&](Node (&dst)[GRP], int c0) {
#pragma unroll
        for (int k = 0; k < GRP; ++k) {
            const int c = min(c0 + k, n - 1);
            const float2 ml = pml[(int64_t)c * Hq];
            dst[k].m = ml.x; dst[k].l = ml.y;
            const Vec v = *reinterpret_cast<const Vec*>(po + (int64_t)c * Hq * D);
#pragma unroll
            for (int i = 0; i < VPL; ++i) dst[k].o[i] = v[i];
        }
    };
    auto push_group = [&](const Node (&src)[GRP], int c0) {
#pragma unroll
        for (int k = 0; k < GRP; ++k) {
            if (c0 + k >= n) break;
            Node carry = src[k];
            // binary increment: equal-size subtrees merge, the older one on the left
            bool live = true;
#pragma unroll
            for (int s = 0; s < SK; ++s) {
                if (live) {
                    if (count & (1u << s)) {
                        carry = combine_node<VPL>(slot[s], carry);
                    } else {
                        slot[s] = carry;
                        live = false;
                    }
                }
            }
            ++count;
        }
    };
    load_group(ba, 0);
    for (int c0 = 0; c0 < n; c0 += 2 * GRP) {
        if (c0 + GRP < n) load_group(bb, c0 + GRP);
        push_group(ba, c0);
        if (c0 + GRP >= n) break;
        if (c0 + 2 * GRP < n) load_group(ba, c0 + 2 * GRP);
        push_group(bb, c0 + GRP);
    }
    // remaining subtrees, smallest (rightmost) first: root = s_hi (+) (... (+) s_lo)
    Node res;
    bool have = false;
#pragma unroll
    for (int k = 0; k < SK; ++k) {
        if (count & (1u << k)) {
            if (!have) { res = slot[k]; have = true; }
            else res = combine_node<VPL>(slot[k], res);
        }
    }
    Packed w;
#pragma unroll
    for (int i = 0; i < VPL / 2; ++i)        // + 0.0f turns -0 into +0
        w[i] = pack_bf16x2(res.o[2 * i] / res.l + 0.0f, res.o[2 * i + 1] / res.l + 0.0f);
    *reinterpret_cast<Packed*>(orow) = w;
}

#ifndef BINV_DECODE_GMAX
#define BINV_DECODE_GMAX 2
#endif

// Where a call's partials go in the workspace.  Node slots hold one row's
// partial of one chunk or subtree: D floats of o in the o region, (max, sum)
// in the float2 region after it.
//   * Leaves (chunk kernel -> merge kernel): [leaf row][chunk][head].
//   * Block-kernel stacks: [token][level - 1][head], st_stride slots a token.
// When every leaf row is a token (leaf_seq = 0), the stacks live in the leaf
// region with st_stride = the chunk count (a token has leaves or a stack,
// never both); otherwise the stacks come first, then the compact leaves.
struct Layout {
    bool block = false;      // long new-token runs go to the block kernel
    int q_split = 0x7fffffff;   // fewest new tokens of a sequence the block kernel takes
    bool leaves = true;      // the chunk and merge kernels run
    int leaf_seq = 0;        // 0: leaf row = token; > 0: row b * leaf_seq + i
    int64_t st_stride = 0;
    int64_t st_nodes = 0;    // node slots (per head) of the stacks, when separate
    int64_t leaf_nodes = 0;  // node slots (per head) of the leaves
};

int64_t n_chunks_of(int64_t max_kv_len) { return (max_kv_len + CHUNK - 1) / CHUNK; }

// block kernel at D = 128 when the longest run fills half a 128-row block
Layout layout_of(int64_t B, int64_t n_tokens, int64_t max_q_len, int64_t max_kv_len, int Hq,
                 int Hkv, int D, bool prefill) {
    Layout L;
    const int64_t C = n_chunks_of(max_kv_len);
    const int G = Hq / Hkv;
    L.leaf_nodes = n_tokens * C;
    L.st_stride = C;
    if (!prefill || D != 128 || max_q_len * G < PF_ROWS / 2) return L;
    L.block = true;
    L.q_split = (PF_ROWS / 2 + G - 1) / G;
    // the counter's slots >= 1 that a row of C chunks can fill: levels 1 .. floor(log2 C)
    int64_t levels = 1;
    while ((int64_t)2 << levels <= C) ++levels;
    // one sequence of q_split or more tokens: no leaves at all
    if (B == 1 && n_tokens >= L.q_split) {
        L.leaves = false;
        L.leaf_nodes = 0;
        L.st_stride = levels;
        L.st_nodes = n_tokens * levels;
        return L;
    }
    const int64_t compact_rows = B * (L.q_split - 1);
    if (compact_rows < n_tokens && n_tokens * levels + compact_rows * C < n_tokens * C) {
        L.leaf_seq = L.q_split - 1;
        L.leaf_nodes = compact_rows * C;
        L.st_stride = levels;
        L.st_nodes = n_tokens * levels;
    }
    return L;
}

struct Regions {
    float* leaf_o;
    float2* leaf_ml;
    float* st_o;
    float2* st_ml;
};

Regions regions_of(const Layout& L, float* ws, int Hq, int D) {
    const int64_t total = (L.st_nodes + L.leaf_nodes) * Hq;
    Regions r;
    r.st_o = ws;
    r.leaf_o = ws + L.st_nodes * Hq * D;
    float2* ml = reinterpret_cast<float2*>(ws + total * D);
    r.st_ml = ml;
    r.leaf_ml = ml + L.st_nodes * Hq;
    if (L.st_nodes == 0) {          // stacks inside the leaf region
        r.st_o = r.leaf_o;
        r.st_ml = r.leaf_ml;
    }
    return r;
}

// chunk kernel over query tiles [0, nqt) of every sequence; prefill sequences
// with q_skip or more new tokens are left to the block kernel
template <int D, int G, int R, bool LOOP, int GMAX>
hipError_t launch_chunk(const AttnArgs& a, hipStream_t s, int64_t nqt, int q_skip,
                        const Regions& rg, int leaf_seq) {
    const int n_chunks = (int)n_chunks_of(a.max_kv_len);
    dim3 grid1((unsigned)(nqt * a.Hkv),
               (unsigned)(LOOP && n_chunks > CHUNK_LANES ? CHUNK_LANES : n_chunks), (unsigned)a.B);
    hipLaunchKernelGGL((attn_chunk_kernel<D, G, R, LOOP, GMAX>), grid1, dim3(ChunkShape<D>::NTH),
                       0, s, (const bf16_t*)a.q, a.cu_q, (const bf16_t*)a.k_cache,
                       (const bf16_t*)a.v_cache, a.page_table, a.pt_stride, a.kv_lens, rg.leaf_o,
                       rg.leaf_ml, a.Hq, a.Hkv, n_chunks, (int)a.max_kv_len, a.scale_log2, q_skip,
                       leaf_seq);
    return hipGetLastError();
}

template <int D, int GMAX>
hipError_t launch_merge(const AttnArgs& a, hipStream_t s, const Regions& rg, int q_min,
                        int leaf_seq) {
    const int n_chunks = (int)n_chunks_of(a.max_kv_len);
    const int64_t Rows = a.n_tokens * a.Hq;
    constexpr int RPB = (NT / 64) * (64 * MERGE_VPL / D);      // rows per workgroup
    dim3 grid2((unsigned)((Rows + RPB - 1) / RPB));
    // binary-counter depth for the most nodes a row can have (a row's nodes
    // never outnumber its leaves; unused slots would never be touched)
    if (n_chunks <= 31)
        hipLaunchKernelGGL((attn_merge_kernel<D, GMAX, 5>), grid2, dim3(NT), 0, s, a.cu_q,
                           a.kv_lens, a.B, a.n_tokens, a.Hq, n_chunks, (int)a.max_kv_len,
                           rg.leaf_o, rg.leaf_ml, (bf16_t*)a.out, q_min, leaf_seq);
    else if (n_chunks <= 255)
        hipLaunchKernelGGL((attn_merge_kernel<D, GMAX, 8>), grid2, dim3(NT), 0, s, a.cu_q,
                           a.kv_lens, a.B, a.n_tokens, a.Hq, n_chunks, (int)a.max_kv_len,
                           rg.leaf_o, rg.leaf_ml, (bf16_t*)a.out, q_min, leaf_seq);
    else
        hipLaunchKernelGGL((attn_merge_kernel<D, GMAX, STACK>), grid2, dim3(NT), 0, s, a.cu_q,
                           a.kv_lens, a.B, a.n_tokens, a.Hq, n_chunks, (int)a.max_kv_len,
                           rg.leaf_o, rg.leaf_ml, (bf16_t*)a.out, q_min, leaf_seq);
    return hipGetLastError();
}

template <int D, int G, int R, bool LOOP, int GMAX>
hipError_t launch_dgr(const AttnArgs& a, hipStream_t s, const Regions& rg) {
    constexpr int TQ = ROWS * R / G;
    const int64_t nqt = a.cu_q ? (a.max_q_len + TQ - 1) / TQ : 1;
    hipError_t e = launch_chunk<D, G, R, LOOP, GMAX>(a, s, nqt, 0x7fffffff, rg, 0);
    if (e != hipSuccess) return e;
    return launch_merge<D, GMAX>(a, s, rg, 0x7fffffff, 0);
}

// Prefill at D = 128 with long new-token runs: sequences with at least
// q_split = 64 / G new tokens (half a 128-row block) go to the block kernel,
// which writes their output rows; the others (e.g. the decode rows of a mixed
// engine step) to the looping one-tile chunk kernel, whose grid then needs
// only the query tiles of fewer than q_split tokens, and the merge kernel.
template <int G>
hipError_t launch_prefill128(const AttnArgs& a, hipStream_t s, const Layout& L, const Regions& rg) {
    constexpr int TQ = PF_ROWS / G, TQ1 = ROWS / G;
    const int64_t nqb = (a.max_q_len + TQ - 1) / TQ;
    dim3 grid1((unsigned)(nqb * a.Hkv), 1, (unsigned)a.B);
    hipLaunchKernelGGL((attn_prefill_kernel<G>), grid1, dim3(64 * PF_WAVES), 0, s,
                       (const bf16_t*)a.q, a.cu_q, (const bf16_t*)a.k_cache,
                       (const bf16_t*)a.v_cache, a.page_table, a.pt_stride, a.kv_lens,
                       (bf16_t*)a.out, rg.st_o, rg.st_ml, a.Hq, a.Hkv, (int)L.st_stride,
                       (int)a.max_kv_len, a.scale_log2, L.q_split, (int)nqb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !L.leaves) return e;
    // max_q_len only bounds the runs: any sequence may be short
    const int64_t nqt = (L.q_split - 1 + TQ1 - 1) / TQ1;
    e = launch_chunk<128, G, 1, true, 0>(a, s, nqt, L.q_split, rg, L.leaf_seq);
    if (e != hipSuccess) return e;
    return launch_merge<128, 0>(a, s, rg, L.q_split, L.leaf_seq);
}

// Prefill calls at D = 128 whose longest new-token run fills at least half a
// 128-row block take the block kernel for their long runs; calls of a few new
// tokens per sequence (the decode steps of a mixed-batch engine) take the
// looping chunk kernel alone, which spends one 16-row tile, not eight, per
// (sequence, KV head, chunk).  Every row's chunk partials and their merge have
// the same bits from either kernel (the per-element arithmetic and the tree
// are the same), so the choice never reaches the output.
template <int D, int G>
hipError_t launch_dg(const AttnArgs& a, hipStream_t s, const Layout& L, const Regions& rg) {
    if (a.cu_q) {
        if constexpr (D == 128)
            if (L.block) return launch_prefill128<G>(a, s, L, rg);
        return launch_dgr<D, G, 1, true, 0>(a, s, rg);
    }
    return launch_dgr<D, G, 1, true, BINV_DECODE_GMAX>(a, s, rg);
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t s, const Layout& L, const Regions& rg) {
    switch (a.Hq / a.Hkv) {
        case 1: return launch_dg<D, 1>(a, s, L, rg);
        case 2: return launch_dg<D, 2>(a, s, L, rg);
        case 4: return launch_dg<D, 4>(a, s, L, rg);
        case 8: return launch_dg<D, 8>(a, s, L, rg);
        case 16: return launch_dg<D, 16>(a, s, L, rg);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Fixed partials buffer of the decode entry point that allocates nothing.
// Each GPU that loads this code object holds its own copy for the life of the
// process.  Host code must never pass `scratch` itself to a kernel (on the host
// the name stands for a host-side shadow, not a device address): the device
// address comes from hipGetSymbolAddress, once per device, below.
static __device__ __align__(256) char scratch[BINV_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[NOALLOC_MAX_DEVICES] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

size_t attn_workspace_bytes(int64_t n_tokens, int Hq, int D, int64_t max_kv_len) {
    return (size_t)n_tokens * Hq * n_chunks_of(max_kv_len) * (D + 2) * sizeof(float);
}

size_t attn_prefill_workspace_bytes(int64_t B, int64_t T, int64_t max_q_len, int64_t max_kv_len,
                                    int Hq, int Hkv, int D) {
    const Layout L = layout_of(B, T, max_q_len, max_kv_len, Hq, Hkv, D, true);
    return (size_t)(L.st_nodes + L.leaf_nodes) * Hq * (D + 2) * sizeof(float);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
    if (a.n_tokens == 0 || a.B == 0) return hipSuccess;
    const Layout L = layout_of(a.B, a.n_tokens, a.max_q_len, a.max_kv_len, a.Hq, a.Hkv, a.D,
                               a.cu_q != nullptr);
    const Regions rg = regions_of(L, a.ws, a.Hq, a.D);
    if (a.D == 64) return launch_d<64>(a, s, L, rg);
    if (a.D == 128) return launch_d<128>(a, s, L, rg);
    return hipErrorInvalidValue;
}

}  // namespace binv
