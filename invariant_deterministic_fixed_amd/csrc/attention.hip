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
#include "common.hpp"
#include "kernels.hpp"

namespace binv {

namespace {

constexpr int CHUNK = 256;
constexpr int PAGE = 16;
constexpr int NT = 256;
constexpr int ROWS = 16;
constexpr int STACK = 10;          // binary counter slots: enough for 1023 leaves

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// P tile in LDS: [16 rows][256 keys] bf16, rows of 512 bytes = 32 chunks of 16
// bytes; chunk ch of row r is stored at position ch ^ r.
__device__ __forceinline__ int p_off(int r, int ch) { return (r << 9) + ((ch ^ r) << 4); }

struct RowInfo {
    int64_t token;   // global query-token index (row of q / out / partials), -1 if padding
    int head;        // query head
    int pos;         // absolute position of the query
};

// Row slot r of tile `qt` of sequence b:  token (r / G) of the tile, head g*G + r % G.
template <int G>
__device__ __forceinline__ RowInfo row_info(int r, int b, int g, int qt, int q_len,
                                            int64_t q_start, int kv_len) {
    constexpr int TQ = ROWS / G;
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

template <int D, int G>
__global__ __launch_bounds__(NT) void attn_chunk_kernel(
    const bf16_t* __restrict__ q, const int32_t* __restrict__ cu_q,
    const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc,
    const int32_t* __restrict__ page_table, int64_t pt_stride,
    const int32_t* __restrict__ kv_lens, float* __restrict__ ws_o,
    float2* __restrict__ ws_ml, int Hq, int Hkv, int n_chunks, int max_kv_len,
    float scale_log2) {
    constexpr int KS = D / 32;                    // k-steps of the q.k product
    constexpr int DT_PER_WAVE = D / 64;           // 16-wide d tiles per wave (2 or 1)
    constexpr int TQ = ROWS / G;
    static_assert(D == 64 || D == 128, "");

    __shared__ __attribute__((aligned(16))) char p_lds[ROWS * CHUNK * 2];
    __shared__ float red_max[4][ROWS];
    __shared__ int row_pos[ROWS];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int b = blockIdx.z;
    const int c = blockIdx.y;
    const int g = blockIdx.x % Hkv;
    const int qt = blockIdx.x / Hkv;

    int kv_len = kv_lens[b];
    if (kv_len > max_kv_len) kv_len = max_kv_len;
    int q_len;
    int64_t q_start;
    if (cu_q) {
        q_start = cu_q[b];
        q_len = cu_q[b + 1] - cu_q[b];
    } else {
        q_start = b;
        q_len = 1;
    }
    if (q_len > kv_len) q_len = kv_len;
    // highest position in this tile; the chunk is skipped if no row reaches it
    const int last_i = min(q_len, (qt + 1) * TQ) - 1;
    if (last_i < qt * TQ) return;
    const int pos_max = kv_len - q_len + last_i;
    const int j0 = c * CHUNK;
    if (j0 > pos_max) return;

    const int64_t pt_row = (int64_t)b * pt_stride;
    const int n_pages = (kv_len + PAGE - 1) / PAGE;

    // ---- Q fragments (A operand): row lane&15, features 32ks + 8(lane>>4) .. +8
    const int ar = lane & 15, ag = lane >> 4;
    const RowInfo a_row = row_info<G>(ar, b, g, qt, q_len, q_start, kv_len);
    u32x4 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        qf[ks] = u32x4{0u, 0u, 0u, 0u};
        if (a_row.token >= 0)
            qf[ks] = ld16(q + (a_row.token * Hq + a_row.head) * D + 32 * ks + 8 * ag);
    }
    if (t < ROWS) row_pos[t] = row_info<G>(t, b, g, qt, q_len, q_start, kv_len).pos;

    // ---- K fragments (B operand): wave w owns keys 64w .. 64w+63 = pages 16c+4w+jt
    u32x4 kf[4][KS];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        const int pidx = 16 * c + 4 * wave + jt;
        const bool ok = pidx < n_pages && pidx < pt_stride;
        const int64_t phys = ok ? (int64_t)page_table[pt_row + pidx] : 0;
        const bf16_t* kp = kc + ((phys * Hkv + g) * PAGE + (lane & 15)) * D + 8 * ag;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[jt][ks] = ok ? ld16(kp + 32 * ks) : u32x4{0u, 0u, 0u, 0u};
    }

    // ---- V fragments (B operand of P.V), issued early: d = 16 dt + (lane&15),
    // keys 32ks + 8(lane>>4) .. +8 = page 16c + 2ks + (ag>>1), slots 8(ag&1) .. +8
    u32x4 vf[DT_PER_WAVE][8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        const int pidx = 16 * c + 2 * ks + (ag >> 1);
        const bool ok = pidx < n_pages && pidx < pt_stride;
        const int64_t phys = ok ? (int64_t)page_table[pt_row + pidx] : 0;
        const int key0 = pidx * PAGE + 8 * (ag & 1);
        const int nvalid = kv_len - key0;          // slots key0 + e valid for e < nvalid
#pragma unroll
        for (int u = 0; u < DT_PER_WAVE; ++u) {
            const int d = 16 * (wave * DT_PER_WAVE + u) + (lane & 15);
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (ok) v = ld16(vc + ((phys * Hkv + g) * D + d) * PAGE + 8 * (ag & 1));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (2 * i + 1 >= nvalid) v[i] &= (2 * i < nvalid) ? 0x0000ffffu : 0u;
            }
            vf[u][ks] = v;
        }
    }

    // ---- S = Q K^T on the matrix cores
    f32x4 s[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        s[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s[jt] = mfma16x16x32(qf[ks], kf[jt][ks], s[jt]);
    }
    __syncthreads();   // row_pos visible

    // lane holds rows 4*(lane>>4)+e, key j0 + 64*wave + 16*jt + (lane&15)
    const int key_lane = j0 + 64 * wave + (lane & 15);
    int rpos[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) rpos[e] = row_pos[4 * ag + e];
    float mx[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        mx[e] = -INFINITY;
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            const bool valid = key_lane + 16 * jt <= rpos[e];
            const float v = valid ? s[jt][e] * scale_log2 : -INFINITY;
            s[jt][e] = v;
            mx[e] = fmaxf(mx[e], v);
        }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) mx[e] = fmaxf(mx[e], __shfl_xor(mx[e], off));
    }
    if ((lane & 15) == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) red_max[wave][4 * ag + e] = mx[e];
    }
    __syncthreads();
    float m[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = 4 * ag + e;
        m[e] = fmaxf(fmaxf(red_max[0][r], red_max[1][r]), fmaxf(red_max[2][r], red_max[3][r]));
    }

    // ---- P = bf16(exp2(s - m)) into LDS
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        const int key = 64 * wave + 16 * jt + (lane & 15);       // key within the chunk
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float v = s[jt][e];
            const float p = (v == -INFINITY) ? 0.0f : exp2f(v - m[e]);
            const int r = 4 * ag + e;
            *reinterpret_cast<bf16_t*>(p_lds + p_off(r, key >> 3) + 2 * (key & 7)) =
                (bf16_t)f32_to_bf16(p);
        }
    }
    __syncthreads();

    // ---- l: thread t sums keys 16(t&15) .. +15 of row t>>4 in key order, then a
    // 4-level xor butterfly over the 16 segment sums of the row
    float lsum;
    {
        const int r = t >> 4, seg = t & 15;
        const u32x4 p0 = *reinterpret_cast<const u32x4*>(p_lds + p_off(r, 2 * seg));
        const u32x4 p1 = *reinterpret_cast<const u32x4*>(p_lds + p_off(r, 2 * seg + 1));
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) { acc += lo_bf16(p0[i]); acc += hi_bf16(p0[i]); }
#pragma unroll
        for (int i = 0; i < 4; ++i) { acc += lo_bf16(p1[i]); acc += hi_bf16(p1[i]); }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) acc += __shfl_xor(acc, off);
        lsum = acc;
    }

    // ---- O = P V on the matrix cores, keys ascending
    f32x4 o[DT_PER_WAVE];
#pragma unroll
    for (int u = 0; u < DT_PER_WAVE; ++u) o[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        const u32x4 pa = *reinterpret_cast<const u32x4*>(p_lds + p_off(ar, 4 * ks + ag));
#pragma unroll
        for (int u = 0; u < DT_PER_WAVE; ++u) o[u] = mfma16x16x32(pa, vf[u][ks], o[u]);
    }

    // ---- write partials of the rows that see at least one key of this chunk
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = 4 * ag + e;
        const RowInfo ri = row_info<G>(r, b, g, qt, q_len, q_start, kv_len);
        if (ri.token < 0 || ri.pos < j0) continue;
        const int64_t slot = (ri.token * Hq + ri.head) * (int64_t)n_chunks + c;
        float* po = ws_o + slot * D;
#pragma unroll
        for (int u = 0; u < DT_PER_WAVE; ++u)
            po[16 * (wave * DT_PER_WAVE + u) + (lane & 15)] = o[u][e];
    }
    // (m, l): thread 16 r holds the butterfly total l of row r
    if ((t & 15) == 0) {
        const int r = t >> 4;
        const RowInfo ri = row_info<G>(r, b, g, qt, q_len, q_start, kv_len);
        if (ri.token >= 0 && ri.pos >= j0) {
            const float mr = fmaxf(fmaxf(red_max[0][r], red_max[1][r]),
                                   fmaxf(red_max[2][r], red_max[3][r]));
            const int64_t slot = (ri.token * Hq + ri.head) * (int64_t)n_chunks + c;
            ws_ml[slot] = make_float2(mr, lsum);
        }
    }
}

struct Partial {
    float m, l;
    float o[2];
};

// left-to-right combine of two partials (m in the log2 domain)
template <int NO>
__device__ __forceinline__ Partial combine(const Partial& a, const Partial& b) {
    Partial r;
    r.m = fmaxf(a.m, b.m);
    const float fa = exp2f(a.m - r.m);
    const float fb = exp2f(b.m - r.m);
    r.l = fmaf(fa, a.l, fb * b.l);
#pragma unroll
    for (int i = 0; i < NO; ++i) r.o[i] = fmaf(fa, a.o[i], fb * b.o[i]);
    return r;
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
    Partial next;
    {
        const float2 ml = pml[0];
        next.m = ml.x; next.l = ml.y;
#pragma unroll
        for (int i = 0; i < NO; ++i) next.o[i] = po[lane + 64 * i];
    }
    for (int c = 0; c < n; ++c) {
        Partial carry = next;
        if (c + 1 < n) {                                  // prefetch the next leaf
            const float2 ml = pml[c + 1];
            next.m = ml.x; next.l = ml.y;
#pragma unroll
            for (int i = 0; i < NO; ++i) next.o[i] = po[(int64_t)(c + 1) * D + lane + 64 * i];
        }
        // binary increment: equal-size subtrees merge, the older one on the left
        bool live = true;
#pragma unroll
        for (int k = 0; k < STACK; ++k) {
            if (live) {
                if (count & (1u << k)) {
                    carry = combine<NO>(slot[k], carry);
                } else {
                    slot[k] = carry;
                    live = false;
                }
            }
        }
        ++count;
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

template <int D, int G>
hipError_t launch_dg(const AttnArgs& a, hipStream_t s) {
    constexpr int TQ = ROWS / G;
    const int n_chunks = (int)((a.max_kv_len + CHUNK - 1) / CHUNK);
    const int64_t nqt = a.cu_q ? (a.max_q_len + TQ - 1) / TQ : 1;
    const int64_t R = a.n_tokens * a.Hq;
    float* ws_o = a.ws;
    float2* ws_ml = reinterpret_cast<float2*>(a.ws + R * n_chunks * a.D);
    dim3 grid1((unsigned)(nqt * a.Hkv), (unsigned)n_chunks, (unsigned)a.B);
    hipLaunchKernelGGL((attn_chunk_kernel<D, G>), grid1, dim3(NT), 0, s, (const bf16_t*)a.q,
                       a.cu_q, (const bf16_t*)a.k_cache, (const bf16_t*)a.v_cache, a.page_table,
                       a.pt_stride, a.kv_lens, ws_o, ws_ml, a.Hq, a.Hkv, n_chunks,
                       (int)a.max_kv_len, a.scale_log2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid2((unsigned)((R + 3) / 4));
    hipLaunchKernelGGL((attn_merge_kernel<D>), grid2, dim3(NT), 0, s, a.cu_q, a.kv_lens, a.B,
                       a.n_tokens, a.Hq, n_chunks, (int)a.max_kv_len, (const float*)ws_o,
                       (const float2*)ws_ml, (bf16_t*)a.out);
    return hipGetLastError();
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
