// attention_tuned.hip -- shape-tuned paged decode attention: the comparator
// for the price of invariance, NOT batch-invariant on purpose.
//
// It follows the strategy the pages name as the cause of nondeterminism
// (tom-jerr.github.io "Batch-Invariant Kernel", section Flash Attention:
// FlashDecoding picks the number of KV splits from how many cores are free;
// devpress.csdn.net explainer, section 3.3): the number of splits per
// sequence is chosen from B * Hkv so that the grid fills the GPU, each split
// walks its consecutive 256-key chunks with an online-softmax merge, and the
// splits are merged left to right.  The per-chunk arithmetic is the invariant
// path's own (attn_chunk.hpp); what changes with the batch is which chunks are
// merged in which order, so a sequence's output bits depend on B.
#include "attn_chunk.hpp"
#include "kernels.hpp"

namespace binv {

namespace {
using namespace attn;

constexpr int MAX_SPLITS = 64;
constexpr int CHUNKS_PER_SPLIT_CAP = 16;     // at most 4096 keys per split

int split_target(int64_t B, int Hkv) {
    const int64_t items = B * Hkv;
    int64_t s = (1024 + items - 1) / items;   // aim at ~1024 workgroups
    if (s > MAX_SPLITS) s = MAX_SPLITS;
    return (int)(s < 1 ? 1 : s);
}

// chunks [c0, c1) of split s for a sequence with n chunks
__device__ __forceinline__ void split_range(int n, int s_target, int s, int& c0, int& c1) {
    int S = (n + CHUNKS_PER_SPLIT_CAP - 1) / CHUNKS_PER_SPLIT_CAP;
    if (S < s_target) S = s_target;
    const int per = (n + S - 1) / S;
    c0 = s * per;
    c1 = min(n, c0 + per);
}

template <int D, int G>
__global__ __launch_bounds__(ChunkShape<D>::NTH, D == 128 ? 4 : 3) void attn_split_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc,
    const int32_t* __restrict__ page_table, int64_t pt_stride, const int32_t* __restrict__ kv_lens,
    float* __restrict__ ws_o, float2* __restrict__ ws_ml, int Hq, int Hkv, int s_target,
    int s_max, int max_kv_len, float scale_log2) {
    __shared__ ChunkLds<D, 1> sh;
    const int s = blockIdx.y;
    const TileCtx x = tile_ctx<G, 1>(blockIdx.z, blockIdx.x, 0, nullptr, kv_lens, pt_stride, max_kv_len);
    if (x.pos_max < 0) return;
    const int n = x.pos_max / CHUNK + 1;
    int c0, c1;
    split_range(n, s_target, s, c0, c1);
    if (c0 >= c1) return;

    // lane (ag, ar) of every wave: row ar, features 16 wave + 4 ag .. + 3
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, ar = lane & 15, ag = lane >> 4;
    float M = -INFINITY, L = 0.0f;
    f32x4 O = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c = c0; c < c1; ++c) {
        __syncthreads();                           // LDS of the previous chunk is free
        int phys[ChunkShape<D>::JT];
        load_phys<D>(x, c, page_table, pt_stride, phys, t);
        u32x4 kf[ChunkShape<D>::JT][ChunkShape<D>::KS];
        const ChunkOut<1> r = chunk_compute<D, G, 1>(x, c, phys, page_table, q, kc, vc,
                                                     pt_stride, Hq, Hkv, scale_log2, sh, t, kf);
        if (r.m[0] != -INFINITY) {
            const float mn = fmaxf(M, r.m[0]);
            const float fa = (M == -INFINITY) ? 0.0f : exp2f(M - mn);
            const float fb = exp2f(r.m[0] - mn);
#pragma unroll
            for (int e = 0; e < 4; ++e) O[e] = fa * O[e] + fb * r.o[0][e];
            L = fa * L + fb * r.l[0];
            M = mn;
        }
    }
    const RowInfo ri = row_info<G, 1>(ar, x.b, x.g, 0, x.q_len, x.q_start, x.kv_len);
    if (ri.token >= 0) {
        const int64_t slot = (ri.token * Hq + ri.head) * (int64_t)s_max + s;
        *reinterpret_cast<f32x4*>(ws_o + slot * D + 16 * wave + 4 * ag) = O;
        if (wave == 0 && ag == 0) ws_ml[slot] = make_float2(M, L);
    }
}

// one wave per (sequence, head): splits merged left to right
template <int D>
__global__ __launch_bounds__(256) void attn_split_merge_kernel(
    const int32_t* __restrict__ kv_lens, int64_t B, int Hq, int s_target, int s_max,
    int max_kv_len, const float* __restrict__ ws_o, const float2* __restrict__ ws_ml,
    bf16_t* __restrict__ out) {
    constexpr int NO = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= B * Hq) return;
    const int kv_len = min(kv_lens[row / Hq], max_kv_len);
    bf16_t* orow = out + row * D;
    if (kv_len < 1) {
#pragma unroll
        for (int i = 0; i < NO; ++i) orow[lane + 64 * i] = 0;
        return;
    }
    const int n = (kv_len - 1) / CHUNK + 1;
    Partial res;
    bool have = false;
    for (int s = 0; s < s_max; ++s) {
        int c0, c1;
        split_range(n, s_target, s, c0, c1);
        if (c0 >= c1) break;
        const int64_t slot = row * s_max + s;
        Partial p;
        const float2 ml = ws_ml[slot];
        p.m = ml.x; p.l = ml.y;
#pragma unroll
        for (int i = 0; i < NO; ++i) p.o[i] = ws_o[slot * D + lane + 64 * i];
        res = have ? combine<NO>(res, p) : p;
        have = true;
    }
#pragma unroll
    for (int i = 0; i < NO; ++i) orow[lane + 64 * i] = (bf16_t)f32_to_bf16(res.o[i] / res.l + 0.0f);
}

template <int D, int G>
hipError_t launch_split(const AttnArgs& a, hipStream_t s) {
    const int s_target = split_target(a.B, a.Hkv);
    const int n_chunks = (int)((a.max_kv_len + CHUNK - 1) / CHUNK);
    int s_max = (n_chunks + CHUNKS_PER_SPLIT_CAP - 1) / CHUNKS_PER_SPLIT_CAP;
    if (s_max < s_target) s_max = s_target;
    const int64_t R = a.B * a.Hq;
    float* ws_o = a.ws;
    float2* ws_ml = reinterpret_cast<float2*>(a.ws + R * s_max * a.D);
    hipLaunchKernelGGL((attn_split_kernel<D, G>), dim3(a.Hkv, s_max, (unsigned)a.B),
                       dim3(ChunkShape<D>::NTH), 0, s, (const bf16_t*)a.q, (const bf16_t*)a.k_cache,
                       (const bf16_t*)a.v_cache, a.page_table, a.pt_stride, a.kv_lens, ws_o, ws_ml,
                       a.Hq, a.Hkv, s_target, s_max, (int)a.max_kv_len, a.scale_log2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_split_merge_kernel<D>), dim3((unsigned)((R + 3) / 4)), dim3(256), 0, s,
                       a.kv_lens, a.B, a.Hq, s_target, s_max, (int)a.max_kv_len,
                       (const float*)ws_o, (const float2*)ws_ml, (bf16_t*)a.out);
    return hipGetLastError();
}

template <int D>
hipError_t launch_split_d(const AttnArgs& a, hipStream_t s) {
    switch (a.Hq / a.Hkv) {
        case 1: return launch_split<D, 1>(a, s);
        case 2: return launch_split<D, 2>(a, s);
        case 4: return launch_split<D, 4>(a, s);
        case 8: return launch_split<D, 8>(a, s);
        case 16: return launch_split<D, 16>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t attn_tuned_workspace_bytes(int64_t B, int Hq, int D, int64_t max_kv_len) {
    (void)max_kv_len;   // the split count never exceeds MAX_SPLITS
    return (size_t)B * Hq * MAX_SPLITS * (D + 2) * sizeof(float);
}

hipError_t launch_attention_decode_tuned(const AttnArgs& a, hipStream_t s) {
    if (a.B == 0) return hipSuccess;
    if (a.D == 64) return launch_split_d<64>(a, s);
    if (a.D == 128) return launch_split_d<128>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace binv
