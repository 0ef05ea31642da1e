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

// workgroups per (query tile, KV head) of a sequence; they loop over the
// sequence's nodes (decode) or chunks (prefill)
constexpr int CHUNK_LANES = 32;

// Decode scheduling, from the batch size only (neither reaches a row's bits):
// from 4 sequences on a workgroup computes at least a pair of chunks (its
// start -- page-table entries, then K and V -- costs about two chunks' worth
// of compute, and with many rows in flight fewer, longer chains stream the
// cache faster); from 128 on, at most 16 workgroups per sequence.  Measured
// at B = 256 (log-uniform lengths 128..32768): 5.09 -> 5.35 TB/s.
struct DecodeSched {
    int lanes, lmin;
};
DecodeSched decode_sched(int64_t B) {
    return DecodeSched{B >= 128 ? 16 : CHUNK_LANES, B >= 4 ? 1 : 0};
}

// Level of the merge tree at which a decode row's partials are handed from
// the chunk kernel to the merge kernel, from the row's chunk count n and the
// call's workgroups per sequence (lanes) and lowest level (lmin, 0 or 1): the
// level from lmin up that keeps the longest chain of chunks one workgroup
// computes in sequence, ceil(n / (lanes 2^L)) 2^L, shortest, and among those
// the highest (fewest partials).  Both kernels evaluate it for the row; the
// root is the same for every level, so lanes and lmin are scheduling only.
template <int GMAX>
__device__ __forceinline__ int node_level(int n, int lanes, int lmin) {
    int best = lmin, best_chain = ((n + (lanes << lmin) - 1) / (lanes << lmin)) << lmin;
#pragma unroll
    for (int L = 1; L <= GMAX; ++L) {
        if (L <= lmin) continue;
        const int per = lanes << L;
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
// writes and re-reads fewer partials.  gridDim.y is capped at the call's lanes, so
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
    float scale_log2, int q_skip, int leaf_seq, int lanes, int lmin) {
    // prefill: sequences with q_skip or more new tokens belong to the block kernel
    if (cu_q && cu_q[blockIdx.z + 1] - cu_q[blockIdx.z] >= q_skip) return;
    static_assert(LOOP || GMAX == 0, "workgroups that take one chunk write leaves");
    __shared__ ChunkLds<D, R> sh;
    constexpr int JT = ChunkShape<D>::JT;
    // the page-table entries of the first node at the call's lowest level,
    // requested before the sequence's length (which fixes the level) arrives:
    // entries within the row may be read ahead, and they are used only if the
    // row's level turns out to be that one (every prefill row; decode rows of
    // up to 2 lanes chunks at lmin = 1)
    const int c_spec = (GMAX > 0 && !cu_q) ? ((int)blockIdx.y << lmin) : (int)blockIdx.y;
    int phys_spec[JT];
    {
        TileCtx xs;
        xs.pt_row = (int64_t)blockIdx.z * pt_stride;
        load_phys<D>(xs, c_spec, page_table, pt_stride, phys_spec, threadIdx.x);
    }
    const int kv_len_b = kv_lens[blockIdx.z];          // read once, kept in a register
    const int pos_max = tile_ctx_len<G, R>(blockIdx.z, blockIdx.x % Hkv, blockIdx.x / Hkv, cu_q,
                                           kv_len_b, pt_stride, max_kv_len).pos_max;
    const int glog =
        (GMAX > 0 && !cu_q && pos_max >= 0) ? node_level<GMAX>(pos_max / CHUNK + 1, lanes, lmin) : 0;
    const int gs = 1 << glog;
    int phys_next[JT];
    // K of the workgroup's current chunk: the first chunk's requested here,
    // every later one by the chunk before it
    u32x4 kf[JT][ChunkShape<D>::KS];
    {
        TileCtx x0;
        x0.pt_row = (int64_t)blockIdx.z * pt_stride;
        if ((int)blockIdx.y * gs == c_spec) {
#pragma unroll
            for (int u = 0; u < JT; ++u) phys_next[u] = phys_spec[u];
        } else {
            load_phys<D>(x0, blockIdx.y * gs, page_table, pt_stride, phys_next, threadIdx.x);
        }
        if (blockIdx.y * gs * CHUNK <= pos_max) {
            const TileCtx x1 = tile_ctx_len<G, R>(blockIdx.z, blockIdx.x % Hkv, blockIdx.x / Hkv,
                                                  cu_q, kv_len_b, pt_stride, max_kv_len);
            load_k<D>(x1, blockIdx.y * gs, phys_next, kc, pt_stride, Hkv, kf, threadIdx.x);
            // the tile's q, the same for every chunk, staged in LDS once
            if constexpr (LOOP) {
                stage_q<D, G, R>(x1, q, Hq, sh, threadIdx.x);
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
            ChunkOut<R> carry = chunk_compute<D, G, R, LOOP>(
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
        const int lane = t & 63, wave = t >> 6, ar = lane & 15, ag = lane >> 4;
        const TileCtx x = tile_ctx_len<G, R>(blockIdx.z, blockIdx.x % Hkv, blockIdx.x / Hkv, cu_q,
                                             kv_len_b, pt_stride, max_kv_len);
        const int j0 = node * gs * CHUNK;
        // partials of the rows that see at least one key of this node: lane
        // (ag, ar) writes features 16 wave + 4 ag .. + 3 of row 16 rt + ar,
        // lanes ag = 0 of wave 0 the row's (max, sum)
#pragma unroll
        for (int rt = 0; rt < R; ++rt) {
            const RowInfo ri = row_info<G, R>(16 * rt + ar, x.b, x.g, x.qt, x.q_len, x.q_start,
                                              x.kv_len);
            if (ri.token < 0 || ri.pos < j0) continue;
            const int64_t lr = leaf_seq ? (int64_t)x.b * leaf_seq + (ri.token - x.q_start) : ri.token;
            const int64_t slot_i = (lr * n_chunks + node) * Hq + ri.head;
            *reinterpret_cast<f32x4*>(ws_o + slot_i * D + 16 * wave + 4 * ag) = r.o[rt];
            if (wave == 0 && ag == 0) ws_ml[slot_i] = make_float2(r.m[rt], r.l[rt]);
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
// per-element operation is the chunk kernel's, in the same order: S^T = K Q^T
// as v_mfma_f32_16x16x32_bf16 over features 32 ks + 8 (lane >> 4) .. + 8, ks
// ascending; scale, mask, exact max; p = bf16(exp2(s - m)); l and
// O^T = V^T P^T in the key order of the p.v products (attn_chunk.hpp), V
// slots at or past kv_len read as zero -- so a row's chunk partial has the
// same bits as from the chunk kernel.  Lane (ag, ar) of a wave holds one row,
// ar, throughout: its scores of keys 16 kt + 4 ag + e, then its p as the p.v
// operand (p never leaves the registers), then features 16 f + 4 ag + e.
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
// V [16 pages][128 features][16 slots] swizzled as in v_src, the page blocks
// PF_VPAGE = 4096 + 16 bytes apart: a V fragment's two halves (pages 2 kb and
// 2 kb + 1) and the same slots of any two pages of a chunk then lie in
// different banks (4096 bytes apart they share every bank, and the paired
// read of a fragment's halves ran at half rate).  q stays in registers (its
// four fragments per lane), which leaves LDS room for that spacing.  The K
// area is free once every tile has its scores, and the next chunk's K is
// copied into it while the scores become p and p.v runs; the next chunk's V
// is copied once p.v is done, while the partial is merged and the next
// chunk's q.k runs.
constexpr int PF_WAVES = 8;
constexpr int PF_ROWS = 16 * PF_WAVES;
constexpr int PF_VPAGE = 128 * PAGE * 2 + 16;     // LDS bytes between V page blocks
// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8; the other counters left at their no-wait maxima), given to the
// compiler's own builtin so that its wait insertion knows they were done
constexpr int WAIT_VM8 = 0x0F78;   // vmcnt(8)
constexpr int WAIT_VM0 = 0x0F70;   // vmcnt(0)

// a chunk partial (or a subtree of them) of one row as a lane of the block
// kernel holds it: the row's max and sum of weights, and its weighted values
// of features 16 f + 4 (lane >> 4) + e
struct PfNode {
    float m, l;
    f32x4 o[8];
};

// the merge kernel's combine (combine_scale, combine_val), a on the left
__device__ __forceinline__ PfNode pf_combine(const PfNode& a, const PfNode& b) {
    PfNode r;
    float fa, fb;
    combine_scale(a.m, b.m, r.m, fa, fb);
    r.l = combine_val(fa, a.l, fb, b.l);
#pragma unroll
    for (int f = 0; f < 8; ++f)
#pragma unroll
        for (int e = 0; e < 4; ++e) r.o[f][e] = combine_val(fa, a.o[f][e], fb, b.o[f][e]);
    return r;
}

template <int G>
__global__ __launch_bounds__(64 * PF_WAVES) void attn_prefill_kernel(
    const bf16_t* __restrict__ q, const int32_t* __restrict__ cu_q,
    const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc,
    const int32_t* __restrict__ page_table, int64_t pt_stride,
    const int32_t* __restrict__ kv_lens, bf16_t* __restrict__ out,
    float* __restrict__ st_o, float2* __restrict__ st_ml, int Hq, int Hkv, int st_stride,
    int max_kv_len, float scale_log2, int q_min, int nqb, int node_pair) {
    constexpr int D = 128, KS = D / 32, NKT = CHUNK / 16;
    // sequences with fewer than q_min new tokens belong to the chunk kernel
    if (cu_q[blockIdx.z + 1] - cu_q[blockIdx.z] < q_min) return;
    // one object, so that the compiler can tell the copies' destinations from
    // the areas read while they are in flight
    struct PfLds {
        __attribute__((aligned(1024))) char k[16 * PAGE * D * 2];
        __attribute__((aligned(1024))) char v[16 * PF_VPAGE];
    };
    __shared__ PfLds sh;
    char* const kbuf = sh.k;
    char* const vbuf = sh.v;
    // (the mask bounds the value for the compiler, which then can tell the K
    // and V areas' copies and reads apart and waits only for what a read needs)
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) & (PF_WAVES - 1);
    // blocks in reverse order: the blocks that see the most chunks start first
    const int g = blockIdx.x % Hkv, qb = nqb - 1 - (int)(blockIdx.x / Hkv), b = blockIdx.z;
    const TileCtx x = tile_ctx<G, PF_WAVES>(b, g, qb, cu_q, kv_lens, pt_stride, max_kv_len);
    if (x.pos_max < 0) return;                        // no row in this block
    const int kv_len = x.kv_len;
    const int nc_all = x.pos_max / CHUNK + 1;         // chunks the block's rows see
    // node_pair: this workgroup takes the aligned pair of chunks 2 y, 2 y + 1
    // (y = blockIdx.y) and writes the pair's subtree as a node (level 1 of
    // the merge tree) for the merge kernel; else every chunk, and the rows
    const int c_first = node_pair ? 2 * (int)blockIdx.y : 0;
    if (c_first >= nc_all) return;
    const int nc = node_pair ? min(nc_all, c_first + 2) : nc_all;
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

    // ---- q fragments of this wave's tile, for every chunk: row 16 wave + ar,
    // features 32 ks + 8 ag .. + 8 (a row without a token reads the block's
    // first token: every key is masked for it)
    u32x4 qf[KS];
    {
        const int lane = lane_id(), ar = lane & 15, ag = lane >> 4;
        const RowInfo ri = row(ar);
        const int64_t tok = ri.token >= 0 ? ri.token : x.q_start;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = ld16(q + (tok * Hq + ri.head) * D + 32 * ks + 8 * ag);
    }
    // K or V pages 2 wave, 2 wave + 1 of chunk c, 8 copies of 1 KB per wave
    // (pages past the sequence copy page 0 of the cache: their keys are
    // masked, their V slots read as zero)
    auto page_of = [&](int c, int u) -> int64_t {
        const int pidx = 16 * c + 2 * wave + u;
        const bool ok = pidx < x.n_pages && pidx < pt_stride;
        return ok ? (int64_t)page_table[x.pt_row + pidx] : 0;
    };
    auto copy_k = [&](int c, int lane) {
        const char* src[2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
            src[u] = reinterpret_cast<const char*>(kc + (page_of(c, u) * Hkv + g) * (PAGE * D));
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int pl = 2 * wave + u;
#pragma unroll
            for (int part = 0; part < 4; ++part) {
                // LDS position part*1024 + 16 lane: key 4 part + lane / 16, chunk lane & 15
                const int key = 4 * part + (lane >> 4), pos = lane & 15;
                __builtin_amdgcn_global_load_lds(
                    (const void*)(src[u] + key * (D * 2) + ((pos ^ key) << 4)),
                    (__attribute__((address_space(3))) void*)(kbuf + pl * (PAGE * D * 2) + part * 1024),
                    16, 0, 0);
            }
        }
    };
    auto copy_v = [&](int c, int lane) {
        const char* src[2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
            src[u] = reinterpret_cast<const char*>(vc + (page_of(c, u) * Hkv + g) * (D * PAGE));
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int pl = 2 * wave + u;
#pragma unroll
            for (int part = 0; part < 4; ++part)
                __builtin_amdgcn_global_load_lds(
                    (const void*)(src[u] + v_src(part, lane)),
                    (__attribute__((address_space(3))) void*)(vbuf + pl * PF_VPAGE + part * 1024),
                    16, 0, 0);
        }
    };
    {
        const int lane = lane_id();
        copy_k(c_first, lane);
        copy_v(c_first, lane);
    }

    // ---- the per-row stack of the counter's slots >= 2 (slots 0 and 1 stay in
    // registers): level s of a row at ((token * st_stride + s - 2) * Hq + head);
    // each lane stores and loads only
    // the values it holds (features 16 f + 4 ag .. + 3 of row ar; the row's
    // (max, sum) by the lanes of group 0, passed to the others by shuffles)
    auto slot_of = [&](int ar, int s) -> int64_t {
        const RowInfo ri = row(ar);
        return ri.token < 0 ? (int64_t)-1 : ((ri.token * st_stride + (s - 2)) * Hq + ri.head);
    };
    auto stack_store = [&](int s, const PfNode& nd, int lane) {
        const int ar = lane & 15, ag = lane >> 4;
        const int64_t sl = slot_of(ar, s);
        if (sl < 0) return;
#pragma unroll
        for (int f = 0; f < 8; ++f) *reinterpret_cast<f32x4*>(st_o + sl * D + 16 * f + 4 * ag) = nd.o[f];
        if (ag == 0) st_ml[sl] = make_float2(nd.m, nd.l);
    };
    auto stack_load = [&](int s, int lane) -> PfNode {
        const int ar = lane & 15, ag = lane >> 4;
        const int64_t sl = slot_of(ar, s);
        PfNode nd;
        float2 ml = make_float2(-INFINITY, 0.0f);
#pragma unroll
        for (int f = 0; f < 8; ++f)
            nd.o[f] = sl < 0 ? f32x4{0.f, 0.f, 0.f, 0.f}
                             : *reinterpret_cast<const f32x4*>(st_o + sl * D + 16 * f + 4 * ag);
        if (ag == 0 && sl >= 0) ml = st_ml[sl];
        nd.m = __shfl(ml.x, ar);
        nd.l = __shfl(ml.y, ar);
        return nd;
    };

    __builtin_amdgcn_s_waitcnt(WAIT_VM8);             // this wave's q and K copies landed
    lds_barrier();                                    // every wave's K(0) in LDS

    PfNode slot0, slot1;
    unsigned count = 0;
#pragma clang loop unroll(disable)
    for (int c = c_first; c < nc; ++c) {
        const int j0 = c * CHUNK;
        const bool more = c + 1 < nc;
        const int lane = lane_id(), ar = lane & 15, ag = lane >> 4;
        if (c > c_first) {
            // K(c) and the stack stores landed (only V(c) may be in flight)
            __builtin_amdgcn_s_waitcnt(WAIT_VM8);
            lds_barrier();                                    // every wave's K(c) in LDS
        }
        const int rpos = row(ar).pos;

        // ---- S^T = K Q^T: tile kt holds, in lane (ag, ar), row ar against
        // keys 16 kt + 4 ag + e; K fragment: key 16 kt + ar, features
        // 32 ks + 8 ag .. + 8 (the q fragments' features)
        f32x4 sc[NKT];
        {
            // k-steps outer, the 16 independent tiles inner (each tile's
            // chain still runs over ks ascending)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) sc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int kofs = ar * (D * 2) + (((4 * ks + ag) ^ ar) << 4);
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) {
                    const u32x4 kf = *reinterpret_cast<const u32x4*>(kbuf + kt * (16 * D * 2) + kofs);
                    sc[kt] = mfma16x16x32(kf, qf[ks], sc[kt]);
                }
            }
        }
        lds_barrier();                                    // every tile done with K(c)
        if (more) copy_k(c + 1, lane);

        // ---- mask (key <= the row's position), the row's max over its four
        // lane groups, p = bf16(2^(s c - m)) packed as the p.v operand, and l
        // in the key order of the p.v products.  Below the diagonal every key
        // of the chunk is valid for every row of the wave and the mask is left
        // out.  p = 0 for a masked key (s = -inf) comes from 2^(-inf): a row
        // whose keys are all masked (m = -inf) takes m = 0 there, which gives
        // p = 0 as well -- the per-score test s == -inf of the chunk kernel.
        float mx = -INFINITY;
        const int key_lane = j0 + 4 * ag;                 // + 16 kt + e
        if (__all(j0 + CHUNK - 1 <= rpos)) {
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sc[kt][e]);
        } else {
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v = key_lane + 16 * kt + e <= rpos ? sc[kt][e] : -INFINITY;
                    sc[kt][e] = v;
                    mx = fmaxf(mx, v);
                }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        mx *= scale_log2;                                 // the row's max, log2 domain
        const float mu = (mx == -INFINITY) ? 0.0f : mx;
        u32x4 pb[8];
        float acc = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    pb[kb][2 * h + i] = p_pack(p_of(sc[2 * kb + h][2 * i], scale_log2, mu),
                                               p_of(sc[2 * kb + h][2 * i + 1], scale_log2, mu));
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = l_add(pb[kb][i], acc);
        }
        acc += __shfl_xor(acc, 16);
        acc += __shfl_xor(acc, 32);

        // V(c) landed (K(c + 1) may still be in flight), in every wave
        if (more) __builtin_amdgcn_s_waitcnt(WAIT_VM8);
        else __builtin_amdgcn_s_waitcnt(WAIT_VM0);
        lds_barrier();

        // ---- O^T = V^T P^T: feature tile f holds, in lane (ag, ar), row ar,
        // features 16 f + 4 ag + e; 32-key blocks ascending.  V slots at or
        // past kv_len exist only in the sequence's last chunk.
        PfNode leaf;
        {
            // key blocks outer, the 8 independent feature tiles inner (each
            // tile's chain still runs over kb ascending); the masked loop only
            // for the sequence's last chunk (block-uniform branch)
            // one opaque lane base per feature tile (from a shared base the
            // compiler would pair reads of neighbouring feature tiles into one
            // instruction and move the halves into place after)
            lds_cptr vl[D / 16];
#pragma unroll
            for (int f = 0; f < D / 16; ++f) vl[f] = v_lane(vbuf, 16 * f + ar, ag);
            auto pv = [&](auto masked) {
#pragma unroll
                for (int f = 0; f < D / 16; ++f) leaf.o[f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 8; ++kb)
#pragma unroll
                    for (int f = 0; f < D / 16; ++f)
                        leaf.o[f] = mfma16x16x32(
                            v_frag<D, decltype(masked)::value, PF_VPAGE>(vl[f], kb, ag, kv_len - j0),
                            pb[kb], leaf.o[f]);
            };
            if (j0 + CHUNK > kv_len) pv(std::true_type{});
            else pv(std::false_type{});
        }
        leaf.m = mx;
        leaf.l = acc;
        lds_barrier();                                    // every tile done with V(c)
        if (more) copy_v(c + 1, lane);

        // ---- push the chunk into the binary counter: equal-size subtrees
        // merge, the older one on the left (uniform over the block)
        if (!(count & 1u)) {
            slot0 = leaf;
        } else {
            PfNode carry = pf_combine(slot0, leaf);
            if (!(count & 2u)) {
                slot1 = carry;
            } else {
                carry = pf_combine(slot1, carry);
                int sl = 2;
#pragma clang loop unroll(disable)
                while (count & (1u << sl)) {
                    carry = pf_combine(stack_load(sl, lane), carry);
                    ++sl;
                }
                stack_store(sl, carry, lane);
            }
        }
        ++count;
    }

    // ---- the root: remaining subtrees, smallest (rightmost) first
    const int lane = lane_id(), ar = lane & 15, ag = lane >> 4;
    PfNode res = slot0;
    bool have = (count & 1u) != 0;
    if (count & 2u) {
        res = have ? pf_combine(slot1, res) : slot1;
        have = true;
    }
#pragma clang loop unroll(disable)
    for (int sl = 2; (count >> sl) != 0; ++sl) {
        if (count & (1u << sl)) {
            if (!have) { res = stack_load(sl, lane); have = true; }
            else res = pf_combine(stack_load(sl, lane), res);
        }
    }
    const RowInfo ri = row(ar);
    if (node_pair) {
        // the pair's node for the rows that reach it: slot (token * st_stride
        // + y) * Hq + head of the node region (st_o, st_ml), as the chunk
        // kernel writes its nodes
        if (ri.token < 0 || ri.pos < c_first * CHUNK) return;
        const int64_t sl = (ri.token * st_stride + (int)blockIdx.y) * Hq + ri.head;
#pragma unroll
        for (int f = 0; f < 8; ++f) *reinterpret_cast<f32x4*>(st_o + sl * D + 16 * f + 4 * ag) = res.o[f];
        if (ag == 0) st_ml[sl] = make_float2(res.m, res.l);
        return;
    }
    // out = o / l as bf16, an exact zero written as +0 (the merge kernel's last step)
    if (ri.token >= 0) {
        bf16_t* orow = out + (ri.token * Hq + ri.head) * D + 4 * ag;
#pragma unroll
        for (int f = 0; f < 8; ++f) {
            uint2 w;
            w.x = pack_bf16x2(res.o[f][0] / res.l + 0.0f, res.o[f][1] / res.l + 0.0f);
            w.y = pack_bf16x2(res.o[f][2] / res.l + 0.0f, res.o[f][3] / res.l + 0.0f);
            *reinterpret_cast<uint2*>(orow + 16 * f) = w;
        }
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
    int q_min, int leaf_seq, int node_stride, int pf_level, int lanes, int lmin) {
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
    // kernel chose for it (decode), or of the call's prefill level pf_level
    // (leaves, or the block kernel's chunk pairs)
    int n_leaf = pos / CHUNK + 1;
    if (n_leaf > n_chunks) n_leaf = n_chunks;
    const int glog = cu_q ? pf_level : (GMAX > 0 ? node_level<GMAX>(n_leaf, lanes, lmin) : 0);
    const int n = ((n_leaf - 1) >> glog) + 1;

    // node c of the row: slot (leaf_row * node_stride + c) * Hq + head
    const int64_t slot0 = leaf_row * node_stride * Hq + (row - token * Hq);
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
//   * Block-kernel stacks: [token][level - 2][head], st_stride slots a token
//     (the counter's levels 0 and 1 stay in registers).
// When every leaf row is a token (leaf_seq = 0), the stacks live in the leaf
// region with st_stride = the chunk count (a token has leaves or a stack,
// never both); otherwise the stacks come first, then the compact leaves.
struct Layout {
    bool block = false;      // long new-token runs go to the block kernel
    bool pairs = false;      // block kernel in chunk pairs, nodes to the merge kernel
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
    // the counter's slots >= 2 that a row of C chunks can fill: levels
    // 2 .. floor(log2 C) (at least one slot, so that the layout is never empty)
    int64_t levels = 1;
    while ((int64_t)4 << levels <= C) ++levels;
    // one sequence whose 128-row blocks number fewer than the CUs (a short
    // prompt, or a prompt chunk, over a context of at most 64 chunks): a
    // workgroup per (block, KV head, aligned pair of chunks), the pairs' nodes
    // ceil(C / 2) per token, merged by the merge kernel -- the same tree, more
    // workgroups
    const int64_t blocks = (n_tokens * G + PF_ROWS - 1) / PF_ROWS;
    if (B == 1 && n_tokens >= L.q_split && blocks * Hkv < 256 && C >= 2 && C <= 64) {
        L.pairs = true;
        L.leaf_nodes = n_tokens * ((C + 1) / 2);
        L.st_stride = (C + 1) / 2;
        return L;
    }
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
                        const Regions& rg, int leaf_seq,
                        DecodeSched ds = DecodeSched{CHUNK_LANES, 0}) {
    const int n_chunks = (int)n_chunks_of(a.max_kv_len);
    dim3 grid1((unsigned)(nqt * a.Hkv),
               (unsigned)(LOOP && n_chunks > ds.lanes ? ds.lanes : n_chunks), (unsigned)a.B);
    hipLaunchKernelGGL((attn_chunk_kernel<D, G, R, LOOP, GMAX>), grid1, dim3(ChunkShape<D>::NTH),
                       0, s, (const bf16_t*)a.q, a.cu_q, (const bf16_t*)a.k_cache,
                       (const bf16_t*)a.v_cache, a.page_table, a.pt_stride, a.kv_lens, rg.leaf_o,
                       rg.leaf_ml, a.Hq, a.Hkv, n_chunks, (int)a.max_kv_len, a.scale_log2, q_skip,
                       leaf_seq, ds.lanes, ds.lmin);
    return hipGetLastError();
}

template <int D, int GMAX>
hipError_t launch_merge(const AttnArgs& a, hipStream_t s, const Regions& rg, int q_min,
                        int leaf_seq, int pf_level = 0, int node_stride = 0,
                        DecodeSched ds = DecodeSched{CHUNK_LANES, 0}) {
    const int lanes = ds.lanes, lmin = ds.lmin;
    const int n_chunks = (int)n_chunks_of(a.max_kv_len);
    if (node_stride == 0) node_stride = n_chunks;
    const int64_t Rows = a.n_tokens * a.Hq;
    constexpr int RPB = (NT / 64) * (64 * MERGE_VPL / D);      // rows per workgroup
    dim3 grid2((unsigned)((Rows + RPB - 1) / RPB));
    // binary-counter depth for the most nodes a row can have (a row's nodes
    // never outnumber its leaves; unused slots would never be touched)
    if (n_chunks <= 31)
        hipLaunchKernelGGL((attn_merge_kernel<D, GMAX, 5>), grid2, dim3(NT), 0, s, a.cu_q,
                           a.kv_lens, a.B, a.n_tokens, a.Hq, n_chunks, (int)a.max_kv_len,
                           rg.leaf_o, rg.leaf_ml, (bf16_t*)a.out, q_min, leaf_seq, node_stride,
                           pf_level, lanes, lmin);
    else if (n_chunks <= 255)
        hipLaunchKernelGGL((attn_merge_kernel<D, GMAX, 8>), grid2, dim3(NT), 0, s, a.cu_q,
                           a.kv_lens, a.B, a.n_tokens, a.Hq, n_chunks, (int)a.max_kv_len,
                           rg.leaf_o, rg.leaf_ml, (bf16_t*)a.out, q_min, leaf_seq, node_stride,
                           pf_level, lanes, lmin);
    else
        hipLaunchKernelGGL((attn_merge_kernel<D, GMAX, STACK>), grid2, dim3(NT), 0, s, a.cu_q,
                           a.kv_lens, a.B, a.n_tokens, a.Hq, n_chunks, (int)a.max_kv_len,
                           rg.leaf_o, rg.leaf_ml, (bf16_t*)a.out, q_min, leaf_seq, node_stride,
                           pf_level, lanes, lmin);
    return hipGetLastError();
}

template <int D, int G, int R, bool LOOP, int GMAX>
hipError_t launch_dgr(const AttnArgs& a, hipStream_t s, const Regions& rg) {
    constexpr int TQ = ROWS * R / G;
    const int64_t nqt = a.cu_q ? (a.max_q_len + TQ - 1) / TQ : 1;
    // decode calls take the batch-size schedule; prefill calls (leaves) the default
    const DecodeSched ds = a.cu_q ? DecodeSched{CHUNK_LANES, 0} : decode_sched(a.B);
    hipError_t e = launch_chunk<D, G, R, LOOP, GMAX>(a, s, nqt, 0x7fffffff, rg, 0, ds);
    if (e != hipSuccess) return e;
    return launch_merge<D, GMAX>(a, s, rg, 0x7fffffff, 0, 0, 0, ds);
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
    if (L.pairs) {
        // chunk pairs: nodes into the leaf region, [token][pair][head]
        dim3 grid1((unsigned)(nqb * a.Hkv), (unsigned)L.st_stride, (unsigned)a.B);
        hipLaunchKernelGGL((attn_prefill_kernel<G>), grid1, dim3(64 * PF_WAVES), 0, s,
                           (const bf16_t*)a.q, a.cu_q, (const bf16_t*)a.k_cache,
                           (const bf16_t*)a.v_cache, a.page_table, a.pt_stride, a.kv_lens,
                           (bf16_t*)a.out, rg.leaf_o, rg.leaf_ml, a.Hq, a.Hkv, (int)L.st_stride,
                           (int)a.max_kv_len, a.scale_log2, L.q_split, (int)nqb, 1);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_merge<128, 0>(a, s, rg, 0x7fffffff, 0, 1, (int)L.st_stride);
    }
    dim3 grid1((unsigned)(nqb * a.Hkv), 1, (unsigned)a.B);
    hipLaunchKernelGGL((attn_prefill_kernel<G>), grid1, dim3(64 * PF_WAVES), 0, s,
                       (const bf16_t*)a.q, a.cu_q, (const bf16_t*)a.k_cache,
                       (const bf16_t*)a.v_cache, a.page_table, a.pt_stride, a.kv_lens,
                       (bf16_t*)a.out, rg.st_o, rg.st_ml, a.Hq, a.Hkv, (int)L.st_stride,
                       (int)a.max_kv_len, a.scale_log2, L.q_split, (int)nqb, 0);
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
