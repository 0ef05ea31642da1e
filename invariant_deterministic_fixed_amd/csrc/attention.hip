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
// 16 query rows (16/G tokens x the G = Hq/Hkv query heads of g), one chunk c
// = keys [256c, 256c+256).  Decode tiles hold one token; prefill tiles hold up
// to 16/G consecutive new tokens of one sequence.  For every row it writes the
// fp32 partial (m, l, o[D]) of the keys of chunk c that the row may see
// (key j <= the row's position):
//     s_j = (q . k_j) * scale * log2(e)      (scores kept in the log2 domain)
//     m   = max_j s_j
//     p_j = bf16(exp2(s_j - m))              (0 for keys the row may not see)
//     l   = sum_j p_j                        (fixed order, below)
//     o   = sum_j p_j v_j                    (matrix cores, keys ascending)
// Kernel 2 (merge): one wave per (token, head) row merges the row's
// n = pos/256 + 1 partials with a binary counter, which reproduces exactly the
// left-aligned binary tree over 512 leaves whose padding leaves are the
// identity (a padding leaf only ever meets a real subtree, and merging with the
// identity returns the real subtree bit for bit).  out = bf16(o / l).
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
#include "kernels.hpp"

namespace binv {

namespace {
using namespace attn;

// Grid: x = (query tile, KV head), y = chunk lane, z = sequence.  With LOOP,
// workgroup (x, y, z) takes the chunks c = y, y + gridDim.y, ... that reach
// the tile's last position, so a grid sized for the longest allowed sequence
// does not spend one workgroup launch per chunk slot of every short
// sequence; without it, gridDim.y is the chunk count and the workgroup takes
// chunk y alone.  Which workgroup takes a chunk does not enter the chunk's
// arithmetic.  R = row tiles of 16 rows per workgroup (1 for decode, 2 for
// prefill at D = 128).
template <int D, int G, int R, bool LOOP>
__global__ __launch_bounds__(ChunkShape<D>::NTH, D == 128 ? 4 : 3) void attn_chunk_kernel(
    const bf16_t* __restrict__ q, const int32_t* __restrict__ cu_q,
    const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc,
    const int32_t* __restrict__ page_table, int64_t pt_stride,
    const int32_t* __restrict__ kv_lens, float* __restrict__ ws_o,
    float2* __restrict__ ws_ml, int Hq, int Hkv, int n_chunks, int max_kv_len,
    float scale_log2) {
    constexpr bool VL = (R == 1);           // V through LDS for single-tile (decode) workgroups
    __shared__ ChunkLds<D, R, VL> sh;
    constexpr int JT = ChunkShape<D>::JT;
    // page-table entries of the first chunk: in bounds whatever kv_len is
    // (row b, entries < pt_stride), so they are read alongside kv_lens rather
    // than after it; later chunks' entries are read one chunk ahead
    int phys_next[JT];
    {
        TileCtx x0;
        x0.pt_row = (int64_t)blockIdx.z * pt_stride;
        load_phys<D>(x0, blockIdx.y, page_table, pt_stride, phys_next, threadIdx.x);
    }
    const int pos_max = tile_ctx<G, R>(blockIdx.z, blockIdx.x % Hkv, blockIdx.x / Hkv, cu_q,
                                       kv_lens, pt_stride, max_kv_len).pos_max;
#pragma clang loop unroll(disable)
    for (int c = blockIdx.y; c * CHUNK <= pos_max; c += gridDim.y) {
        // the tile context, q fragments, row maps and lane-derived addresses
        // are re-derived per chunk (cache hits and a few ALU operations)
        // rather than held live across chunks, which would spill
        asm volatile("" ::: "memory");
        int t = threadIdx.x;
        if constexpr (LOOP) asm volatile("" : "+v"(t));
        const int lane = t & 63, wave = t >> 6, ag = lane >> 4;
        const TileCtx x = tile_ctx<G, R>(blockIdx.z, blockIdx.x % Hkv, blockIdx.x / Hkv, cu_q,
                                         kv_lens, pt_stride, max_kv_len);
        int phys[JT];
#pragma unroll
        for (int u = 0; u < JT; ++u) phys[u] = phys_next[u];
        if (LOOP && (c + (int)gridDim.y) * CHUNK <= pos_max)
            load_phys<D>(x, c + gridDim.y, page_table, pt_stride, phys_next, t);
        const ChunkOut<R> r = chunk_compute<D, G, R, VL>(x, c, phys, page_table, q, kc, vc,
                                                         pt_stride, Hq, Hkv, scale_log2, sh, t);
        const int j0 = c * CHUNK;
        // partials of the rows that see at least one key of this chunk
#pragma unroll
        for (int rt = 0; rt < R; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const RowInfo ri = row_info<G, R>(16 * rt + 4 * ag + e, x.b, x.g, x.qt, x.q_len,
                                                  x.q_start, x.kv_len);
                if (ri.token < 0 || ri.pos < j0) continue;
                const int64_t slot = (ri.token * Hq + ri.head) * (int64_t)n_chunks + c;
                ws_o[slot * D + 16 * wave + (lane & 15)] = r.o[rt][e];
            }
        if (t < 256 * R && (t & 15) == 0) {
            const RowInfo ri = row_info<G, R>(t >> 4, x.b, x.g, x.qt, x.q_len, x.q_start, x.kv_len);
            if (ri.token >= 0 && ri.pos >= j0) {
                const int64_t slot = (ri.token * Hq + ri.head) * (int64_t)n_chunks + c;
                ws_ml[slot] = make_float2(r.ml_m, r.l);
            }
        }
        if constexpr (!LOOP) break;
        __syncthreads();                    // LDS free for the next chunk
    }
}

// One wave per (token, head) row; lane owns features lane (+ 64).
template <int D>
__global__ __launch_bounds__(NT) void attn_merge_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ kv_lens, int64_t B,
    int64_t n_tokens, int Hq, int n_chunks, int max_kv_len,
    const float* __restrict__ ws_o, const float2* __restrict__ ws_ml, bf16_t* __restrict__ out) {
    constexpr int NO = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (NT / 64) + (threadIdx.x >> 6);
    if (row >= n_tokens * Hq) return;
    const int64_t token = row / Hq;

    // the query's absolute position
    int pos;
    if (cu_q) {
        int64_t lo = 0, hi = B - 1;            // last b with cu_q[b] <= token
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) >> 1;
            if (cu_q[mid] <= token) lo = mid; else hi = mid - 1;
        }
        int kv_len = kv_lens[lo];
        if (kv_len > max_kv_len) kv_len = max_kv_len;
        int q_len = cu_q[lo + 1] - cu_q[lo];
        if (q_len > kv_len) q_len = kv_len;
        const int i = (int)(token - cu_q[lo]);
        pos = (i < q_len) ? kv_len - q_len + i : -1;
    } else {
        int kv_len = kv_lens[token];
        if (kv_len > max_kv_len) kv_len = max_kv_len;
        pos = kv_len - 1;
    }
    bf16_t* orow = out + row * D;
    if (pos < 0) {
#pragma unroll
        for (int i = 0; i < NO; ++i) orow[lane + 64 * i] = 0;
        return;
    }
    int n = pos / CHUNK + 1;
    if (n > n_chunks) n = n_chunks;

    const float* po = ws_o + row * (int64_t)n_chunks * D;
    const float2* pml = ws_ml + row * (int64_t)n_chunks;

    Partial slot[STACK];
    unsigned count = 0;
    // leaves are loaded four at a time, the next four in flight while the
    // current four are pushed into the binary counter in leaf order
    constexpr int GRP = 4;
    Partial cur[GRP], nxt[GRP];
    auto load_group = [&](Partial (&dst)[GRP], int c0) {
#pragma unroll
        for (int k = 0; k < GRP; ++k) {
            const int c = c0 + k;
            if (c < n) {
                const float2 ml = pml[c];
                dst[k].m = ml.x; dst[k].l = ml.y;
#pragma unroll
                for (int i = 0; i < NO; ++i) dst[k].o[i] = po[(int64_t)c * D + lane + 64 * i];
            }
        }
    };
    load_group(cur, 0);
    for (int c0 = 0; c0 < n; c0 += GRP) {
        if (c0 + GRP < n) load_group(nxt, c0 + GRP);
#pragma unroll
        for (int k = 0; k < GRP; ++k) {
            if (c0 + k >= n) break;
            Partial carry = cur[k];
            // binary increment: equal-size subtrees merge, the older one on the left
            bool live = true;
#pragma unroll
            for (int s = 0; s < STACK; ++s) {
                if (live) {
                    if (count & (1u << s)) {
                        carry = combine<NO>(slot[s], carry);
                    } else {
                        slot[s] = carry;
                        live = false;
                    }
                }
            }
            ++count;
        }
#pragma unroll
        for (int k = 0; k < GRP; ++k) cur[k] = nxt[k];
    }
    // remaining subtrees, smallest (rightmost) first: root = s_hi (+) (... (+) s_lo)
    Partial res;
    bool have = false;
#pragma unroll
    for (int k = 0; k < STACK; ++k) {
        if (count & (1u << k)) {
            if (!have) { res = slot[k]; have = true; }
            else res = combine<NO>(slot[k], res);
        }
    }
#pragma unroll
    for (int i = 0; i < NO; ++i) {
        const float v = res.o[i] / res.l + 0.0f;       // + 0.0f turns -0 into +0
        orow[lane + 64 * i] = (bf16_t)f32_to_bf16(v);
    }
}

// workgroups per (query tile, KV head) when they loop over chunks: a sequence
// of n chunks is covered in ceil(n / CHUNK_LANES) rounds
constexpr int CHUNK_LANES = 16;

template <int D, int G, int R>
hipError_t launch_dgr(const AttnArgs& a, hipStream_t s) {
    constexpr int TQ = ROWS * R / G;
    const int n_chunks = (int)((a.max_kv_len + CHUNK - 1) / CHUNK);
    const int64_t nqt = a.cu_q ? (a.max_q_len + TQ - 1) / TQ : 1;
    const int64_t Rows = a.n_tokens * a.Hq;
    float* ws_o = a.ws;
    float2* ws_ml = reinterpret_cast<float2*>(a.ws + Rows * n_chunks * a.D);
    // decode workgroups (R = 1) loop over their sequence's chunks; prefill
    // tiles already fill the machine with one chunk per workgroup
    constexpr bool LOOP = (R == 1);
    dim3 grid1((unsigned)(nqt * a.Hkv),
               (unsigned)(LOOP && n_chunks > CHUNK_LANES ? CHUNK_LANES : n_chunks), (unsigned)a.B);
    hipLaunchKernelGGL((attn_chunk_kernel<D, G, R, LOOP>), grid1, dim3(ChunkShape<D>::NTH), 0, s,
                       (const bf16_t*)a.q, a.cu_q, (const bf16_t*)a.k_cache,
                       (const bf16_t*)a.v_cache, a.page_table, a.pt_stride, a.kv_lens, ws_o,
                       ws_ml, a.Hq, a.Hkv, n_chunks, (int)a.max_kv_len, a.scale_log2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid2((unsigned)((Rows + 3) / 4));
    hipLaunchKernelGGL((attn_merge_kernel<D>), grid2, dim3(NT), 0, s, a.cu_q, a.kv_lens, a.B,
                       a.n_tokens, a.Hq, n_chunks, (int)a.max_kv_len, (const float*)ws_o,
                       (const float2*)ws_ml, (bf16_t*)a.out);
    return hipGetLastError();
}

// decode: one token per sequence, one row tile; prefill: two row tiles at D = 128
template <int D, int G>
hipError_t launch_dg(const AttnArgs& a, hipStream_t s) {
    if constexpr (D == 128) {
        if (a.cu_q) return launch_dgr<D, G, 2>(a, s);
    }
    return launch_dgr<D, G, 1>(a, s);
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t s) {
    switch (a.Hq / a.Hkv) {
        case 1: return launch_dg<D, 1>(a, s);
        case 2: return launch_dg<D, 2>(a, s);
        case 4: return launch_dg<D, 4>(a, s);
        case 8: return launch_dg<D, 8>(a, s);
        case 16: return launch_dg<D, 16>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t attn_workspace_bytes(int64_t n_tokens, int Hq, int D, int64_t max_kv_len) {
    const int64_t C = (max_kv_len + CHUNK - 1) / CHUNK;
    return (size_t)n_tokens * Hq * C * (D + 2) * sizeof(float);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
    if (a.n_tokens == 0 || a.B == 0) return hipSuccess;
    if (a.D == 64) return launch_d<64>(a, s);
    if (a.D == 128) return launch_d<128>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace binv
