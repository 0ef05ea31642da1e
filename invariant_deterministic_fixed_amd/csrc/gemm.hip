// gemm.hip -- bf16 GEMM with one fixed reduction per element and no split-K (gfx950).
//
// Method: devpress.csdn.net explainer of "Defeating Nondeterminism in LLM
// Inference", section 3.2 Matmul (C = A B as elementwise products plus a
// reduction over k; 2-D output tiles, each reducing the whole K inside one
// core; split-K disabled, because splitting the reduction by batch size is
// what makes the bits depend on the batch); tom-jerr.github.io
// "Batch-Invariant Kernel", section GEMM (fixed tiling, the K strategy
// decoupled from M).
//
// Per output element the arithmetic is one fp32 accumulator updated by
// v_mfma_f32_16x16x32_bf16 over k-blocks [0,32), [32,64), ... in ascending
// order, with K padded by zeros to a multiple of 64.  On the pages a single
// tile configuration is what pins that order; here no tile parameter enters
// the chain at all (a row's slot in a tile only decides which lane carries
// it), so the output tile can follow the shape without the bits following:
//   * 256 x 256 tiles when that gives >= 192 tiles (large M; gemm_pp_kernel,
//     its two wave groups taking turns at LDS reads and MFMAs),
//   * for M <= 64 (decode batches), strips of 16 or 32 columns held by a
//     four-wave workgroup up to 8192-wide outputs (gemm_strip_kernel), strips
//     of 64 columns one wave each beyond (gemm_skinny_kernel),
//   * 128 x 128 tiles (four LDS stages) when that gives >= 192 tiles,
//   * 64 x 64 tiles (4 waves of 32 x 32, four LDS stages) otherwise.
// Tests check a row's bits across M = 1 .. 8192 and every kernel against the
// others.  The comparator below (128 x 128 with split-K chosen from the tile
// count) is the one that does change with M.
//
// Tile kernel (256 x 256 shown; 128 x 128 and 64 x 64 are the same code with
// 4 waves, 64 x 64 with four LDS stages and 64-column W rows swizzled by
// swz_w64):
// 512 lanes = 8 waves in a 2 x 4 grid, each wave owning 128 x 64 outputs
// (8 x 4 MFMA tiles, 128 fp32 accumulators per lane).  A and W travel
// HBM -> LDS by buffer_load ... lds (16 bytes per lane, no registers,
// out-of-range lanes read zero, which handles ragged M, N and K) into two LDS
// stages of 64 KB; the next K-tile streams in while the current one feeds the
// matrix cores.
//   * A tile [256][64]: rows of 128 bytes, 16-byte chunk c of row r stored at
//     c ^ (r & 7); A fragments are ds_read_b128, free of bank conflicts on
//     gfx950's 64-bank LDS (a (r ^ r>>3) & 7 pattern measured two-way
//     conflicts and half the read rate).
//   * W tile [64][256] stays k-major as in HBM; chunk c of row k stored at
//     c ^ 2((k & 3) + 4((k >> 3) & 1)).  A B fragment (8 consecutive k of one
//     column) is two ds_read_b64_tr_b16: in each 16-lane group, lane i of the
//     result takes element i%4 of the 8-byte reads of lanes i/4 + 4t, t=0..3,
//     so when lane 4t+q of the group reads row k+t, columns 4q..4q+3, lane
//     p ends up holding rows k..k+3 of column p.  The swizzle spreads the 16
//     rows a wave reads over all 64 banks, two lanes per bank.
//   * Workgroup ids are dispatched round-robin over the 8 XCDs; each XCD is
//     given a contiguous range of tiles in groups of 8 tile-rows, so tiles
//     running together on one XCD share A and W panels in its L2.
#include "common.hpp"
#include "kernels.hpp"

namespace binv {

namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int BK = 64;
constexpr unsigned RSRC_WORD3 = 0x00020000u;   // raw buffer: 32-bit data format, no swizzle
constexpr int OOB = 0x7ffffff0;                // offset past any num_records: reads zero

__device__ __forceinline__ int swz_a(int r) { return r & 7; }
__device__ __forceinline__ int swz_w(int k) { return 2 * ((k & 3) + 4 * ((k >> 3) & 1)); }
// 64-column W tiles (rows of 128 bytes, 8 chunks): rows of one parity share a
// bank group, so the chunk index is XORed with a function of bits 1 and 3 of k
__device__ __forceinline__ int swz_w64(int k) { return 2 * (((k >> 1) & 1) + 2 * ((k >> 3) & 1)); }

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// linear workgroup id -> output tile; contiguous tile ranges per XCD, then
// groups of GROUP_M tile-rows walked column by column
template <int GROUP_M>
__device__ __forceinline__ void tile_of(int i, int Mt, int Nt, int& tm, int& tn) {
    const int T = Mt * Nt;
    const int q = T / 8, r = T % 8;
    const int x = i % 8, local = i / 8;
    const int t = (x < r) ? x * (q + 1) + local : r * (q + 1) + (x - r) * q + local;
    const int per_group = GROUP_M * Nt;
    const int first_m = (t / per_group) * GROUP_M;
    const int gsz = min(Mt - first_m, GROUP_M);
    tm = first_m + (t % per_group) % gsz;
    tn = (t % per_group) / gsz;
}

template <int BM, int BN, int WGM, int WGN, int GROUP_M, int NS = 2>
struct Tile {
    static constexpr int BM_ = BM, BN_ = BN;
    static constexpr int NW = WGM * WGN, NT = 64 * NW;
    static constexpr int TM = BM / WGM, TN = BN / WGN, FM = TM / 16, FN = TN / 16;
    static constexpr int A_BYTES = BM * BK * 2, W_BYTES = BK * BN * 2, STAGE = A_BYTES + W_BYTES;
    static constexpr int A_PW = A_BYTES / 1024 / NW, W_PW = W_BYTES / 1024 / NW;
    static constexpr int WROWS = 1024 / (BN * 2);        // W rows per 1 KB DMA instruction
    static_assert(A_PW * NW * 1024 == A_BYTES && W_PW * NW * 1024 == W_BYTES, "");
    static_assert(BN >= 64 && BN <= 512, "");
    static constexpr int NS_ = NS;                       // LDS stages (K-tiles in flight + 1)
    static constexpr int PW = A_PW + W_PW;               // DMA instructions per wave per stage
    static_assert((NS - 2) * PW <= 63, "vmcnt holds 6 bits");
    __device__ static int swzw(int k) { return BN == 64 ? swz_w64(k) : swz_w(k); }

    // DMA of K-tile kt into LDS stage `st`
    __device__ static void issue(char* smem, int st, int kt, const bf16_t* A, int64_t lda,
                                 const bf16_t* W, int64_t ldw, int m0, int n0, int M, int N, int K,
                                 int wave, int lane) {
        char* As = smem + st * STAGE;
        char* Ws = As + A_BYTES;
        const int k0 = kt * BK;
        {
            const int rows = min(BM, M - m0);
            __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(A + (int64_t)m0 * lda), (short)0, (int)((int64_t)rows * lda * 2), RSRC_WORD3);
#pragma unroll
            for (int u = 0; u < A_PW; ++u) {
                const int j = wave * A_PW + u;                  // 1 KB block = 8 rows
                const int row = 8 * j + (lane >> 3);
                const int c = (lane & 7) ^ swz_a(row);
                const int kk = k0 + 8 * c;
                const int off = (row < rows && kk < K) ? (row * (int)lda + kk) * 2 : OOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(As + j * 1024), 16, off, 0, 0, 0);
            }
        }
        {
            const int krows = min(BK, K - k0);
            __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(W + (int64_t)k0 * ldw + n0), (short)0, (int)((int64_t)krows * ldw * 2),
                RSRC_WORD3);
#pragma unroll
            for (int u = 0; u < W_PW; ++u) {
                const int j = wave * W_PW + u;
                const int row = WROWS * j + lane / (BN / 8);
                const int c = (lane % (BN / 8)) ^ swzw(row);
                const int off = (row < krows && n0 + 8 * c < N) ? (row * (int)ldw + 8 * c) * 2 : OOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(Ws + j * 1024), 16, off, 0, 0, 0);
            }
        }
    }

    __device__ static void compute(const char* As, const char* Ws, f32x4 (&acc)[FM][FN], int wm,
                                   int wn, int lane) {
        const int r = lane & 15, g = lane >> 4;
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            u32x4 b[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int c = (wn * TN + 16 * j + 4 * (r & 3)) >> 3;
                const int k_lo = 32 * ks + 8 * g + (r >> 2), k_hi = k_lo + 4;
                const v4i16 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_v4i16*)(Ws + k_lo * BN * 2 + ((c ^ swzw(k_lo)) << 4) + 8 * (r & 1)));
                const v4i16 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_v4i16*)(Ws + k_hi * BN * 2 + ((c ^ swzw(k_hi)) << 4) + 8 * (r & 1)));
                const u32x2 p0 = __builtin_bit_cast(u32x2, h0), p1 = __builtin_bit_cast(u32x2, h1);
                b[j] = u32x4{p0[0], p0[1], p1[0], p1[1]};
            }
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * TM + 16 * i + r;
                const u32x4 a = *reinterpret_cast<const u32x4*>(
                    As + (row << 7) + (((4 * ks + g) ^ swz_a(row)) << 4));
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32(a, b[j], acc[i][j]);
            }
            if constexpr (FM == 8 && FN == 4) {
                // 16 LDS reads and 32 MFMAs per k-step: issue them as 16 x (1 read,
                // 2 MFMAs) so a wave's own reads overlap its matrix work (measured
                // +2-5 % on the 256 x 256 tile; scheduling only)
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
                }
            }
        }
    }

    // the wave's FM x FN accumulator tiles -> C rows r0 .., columns c0 ..
    // (lane l holds rows 4(l/16) + e, column l % 16 of each 16 x 16 tile)
    __device__ static void store_c(const f32x4 (&acc)[FM][FN], void* __restrict__ C, int64_t ldc,
                                   int r0, int c0, int lane, int M, int N, int c_f32) {
        const int col_base = c0 + (lane & 15);
        const int row_base = r0 + 4 * (lane >> 4);
        if (c_f32) {
            float* Cf = reinterpret_cast<float*>(C);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int col = col_base + 16 * j;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int row = row_base + 16 * i + e;
                        if (row < M && col < N) Cf[(int64_t)row * ldc + col] = acc[i][j][e];
                    }
                }
        } else {
            bf16_t* Cb = reinterpret_cast<bf16_t*>(C);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int col = col_base + 16 * j;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int row = row_base + 16 * i + e;
                        if (row < M && col < N)
                            Cb[(int64_t)row * ldc + col] = (bf16_t)f32_to_bf16(acc[i][j][e]);
                    }
                }
        }
    }

    // K-tiles [kt_begin, kt_end) of tile blockIdx.x; fp32 partials of split z
    // go to C + z * split_stride (comparator only).
    template <bool SPLIT>
    __device__ static void run(const bf16_t* __restrict__ A, int64_t lda,
                               const bf16_t* __restrict__ W, int64_t ldw, void* __restrict__ C,
                               int64_t ldc, int64_t split_stride, int M, int N, int K,
                               int kt_per_split, int c_f32, char* smem) {
        const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
        const int wm = wave / WGN, wn = wave % WGN;
        int tm, tn;
        tile_of<GROUP_M>(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
        const int m0 = tm * BM, n0 = tn * BN;
        const int nk = (K + BK - 1) / BK;
        // without SPLIT the whole K range, known at compile time to start at 0
        const int kt_begin = SPLIT ? (int)blockIdx.z * kt_per_split : 0;
        const int kt_end = SPLIT ? min(nk, kt_begin + kt_per_split) : nk;

        f32x4 acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
        for (int s = 0; s < NS - 1; ++s)
            if (kt_begin + s < kt_end)
                issue(smem, s, kt_begin + s, A, lda, W, ldw, m0, n0, M, N, K, wave, lane);
        for (int kt = kt_begin; kt < kt_end; ++kt) {
            const int st = (kt - kt_begin) % NS;
            // this wave's part of stage kt has landed (the NS - 2 later stages
            // may still be in flight) ...
            if constexpr (NS > 2) {
                if (kt + NS - 2 < kt_end)
                    asm volatile("s_waitcnt vmcnt(%0)" :: "n"((NS - 2) * PW) : "memory");
                else
                    wait_vm0();
            } else {
                wait_vm0();
            }
            __builtin_amdgcn_s_barrier();        // ... and every wave's; stage kt-1 is free
            if (kt + NS - 1 < kt_end)
                issue(smem, (kt - kt_begin + NS - 1) % NS, kt + NS - 1, A, lda, W, ldw, m0, n0, M,
                      N, K, wave, lane);
            const char* As = smem + st * STAGE;
            compute(As, As + A_BYTES, acc, wm, wn, lane);
        }

        store_c(acc, SPLIT ? (void*)((char*)C + (c_f32 ? 4 : 2) * (int64_t)blockIdx.z *
                                                  split_stride)
                           : C,
                ldc, m0 + wm * TM, n0 + wn * TN, lane, M, N, c_f32);
    }
};


// ------------------------------------------------------------------ few rows
// M <= 64 (decode batches).  The 256 x 256 tile would give N / 256 workgroups
// (16 for N = 4096) and stream the weights through as many CUs.  Here a
// workgroup is one wave owning a strip of 16 FN columns of W and all M
// (<= 16 FM) rows; FN is the widest of 1, 2, 4 that still gives >= 192
// strips (wider strips read longer pieces of each W row and spend fewer
// instructions per byte; narrower ones spread N = 4096 over all CUs).  Each
// element's arithmetic is the tile kernel's exactly: one fp32 accumulator, the
// same v_mfma_f32_16x16x32_bf16 over the same 32-wide k-blocks in ascending
// order, the same zero padding of a ragged K-tile of 64 -- so a row's bits do
// not change when M crosses from this path to a tile one.
//   * LDS ring of NS stages (A [16 FM][64] as in the big tile; W [64][16 FN]);
//     each iteration first refills the slot the previous K-tile used, then
//     waits for its own K-tile and reads both of its k-steps' fragments in one
//     LDS round trip.
//   * Bank spreading of the 16 W rows one ds_read_b64_tr_b16 touches: FN = 1
//     (32-byte rows) stores row k at row k ^ 4 ((k >> 3) & 1); FN >= 2 XORs the
//     16-byte chunk index with a function of k instead.
//   * Strips that share 128-byte lines of a W row go to the same XCD.
//   * The transposing LDS reads are issued as inline asm: for the builtin the
//     compiler waits for every outstanding global -> LDS copy first
//     (vmcnt(0)), which would drain the ring on each K-tile.  The lgkmcnt
//     wait that follows them takes their results as operands, so nothing
//     reads the registers before the data has arrived.
__device__ __forceinline__ int skinny_row(int k) { return k ^ (((k >> 3) & 1) << 2); }

__device__ __forceinline__ u32x2 ds_read_tr_b64(const char* p) {
    u32x2 v;
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(a) : "memory");
    return v;
}
__device__ __forceinline__ u32x4 ds_read_b128_asm(const char* p) {
    u32x4 v;
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(a) : "memory");
    return v;
}

template <int FM, int FN, int NS>
__global__ __launch_bounds__(64) void gemm_skinny_kernel(const bf16_t* __restrict__ A, int64_t lda,
                                                         const bf16_t* __restrict__ W, int64_t ldw,
                                                         void* __restrict__ C, int64_t ldc, int M,
                                                         int N, int K, int c_f32) {
    constexpr int BN = 16 * FN, RB = 2 * BN;                 // row bytes of the W strip
    constexpr int A_BYTES = 16 * FM * BK * 2, W_BYTES = BK * RB, STAGE = A_BYTES + W_BYTES;
    constexpr int PA = A_BYTES / 1024, PW = W_BYTES / 1024, P = PA + PW;
    constexpr int RPI = 1024 / RB, LPR = RB / 16;             // rows per DMA, lanes per row
    static_assert((NS - 1) * P <= 63, "vmcnt holds 6 bits");
    __shared__ __attribute__((aligned(1024))) char smem[NS * STAGE];
    const int lane = threadIdx.x, r = lane & 15, g = lane >> 4;
    const int b = blockIdx.x, x = b & 7, local = b >> 3;
    constexpr int GS = (FN >= 8) ? 1 : 8 / FN;                // strips per 128-byte line group
    const int n0 = ((local / GS) * 8 * GS + x * GS + (local % GS)) * BN;
    if (n0 >= N) return;
    const int nk = (K + BK - 1) / BK;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)A, (short)0, (int)((int64_t)M * lda * 2), RSRC_WORD3);
    // physical chunk of (row k, chunk c): FN = 1 permutes rows, FN >= 2 XORs chunks
    auto wpos = [&](int k, int c) -> int {
        if constexpr (FN == 1) return skinny_row(k) * RB + c * 16;
        else if constexpr (FN == 2) return k * RB + ((c ^ (2 * ((k >> 3) & 1))) << 4);
        else return k * RB + ((c ^ (2 * (((k >> 1) & 1) + 2 * ((k >> 3) & 1)))) << 4);
    };
    auto issue = [&](int st, int kt) {
        char* As = smem + st * STAGE;
        char* Ws = As + A_BYTES;
        const int k0 = kt * BK;
#pragma unroll
        for (int u = 0; u < PA; ++u) {
            const int row = 8 * u + (lane >> 3);
            const int c = (lane & 7) ^ swz_a(row);
            const int kk = k0 + 8 * c;
            const int off = (row < M && kk < K) ? (row * (int)lda + kk) * 2 : OOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(As + u * 1024), 16, off, 0, 0, 0);
        }
        const int krows = min(BK, K - k0);
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(W + (int64_t)k0 * ldw + n0), (short)0, (int)((int64_t)krows * ldw * 2), RSRC_WORD3);
#pragma unroll
        for (int u = 0; u < PW; ++u) {
            // physical slot: row pr, chunk pcpos; find which logical (k, c) lives there
            const int pr = RPI * u + lane / LPR, pcpos = lane % LPR;
            int kr, pc;
            if constexpr (FN == 1) { kr = skinny_row(pr); pc = pcpos; }
            else if constexpr (FN == 2) { kr = pr; pc = pcpos ^ (2 * ((pr >> 3) & 1)); }
            else { kr = pr; pc = pcpos ^ (2 * (((pr >> 1) & 1) + 2 * ((pr >> 3) & 1))); }
            const int off = (kr < krows && n0 + 8 * pc < N) ? (kr * (int)ldw + 8 * pc) * 2 : OOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(Ws + u * 1024), 16, off, 0, 0, 0);
        }
    };
    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < NS - 1; ++st)
        if (st < nk) issue(st, st);
    for (int kt = 0; kt < nk; ++kt) {
        // refill the slot K-tile kt - 1 used (its fragments were consumed by
        // the MFMAs of the previous iteration) before waiting on K-tile kt
        if (kt + NS - 1 < nk) issue((kt + NS - 1) % NS, kt + NS - 1);
        if (kt + NS - 1 < nk)
            asm volatile("s_waitcnt vmcnt(%0)" :: "n"((NS - 1) * P) : "memory");
        else
            wait_vm0();
        const char* As = smem + (kt % NS) * STAGE;
        const char* Ws = As + A_BYTES;
        u32x2 p0[2][FN], p1[2][FN];
        u32x4 a[2][FM];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int k_lo = 32 * ks + 8 * g + (r >> 2), k_hi = k_lo + 4;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int c = 2 * j + ((r & 3) >> 1);
                p0[ks][j] = ds_read_tr_b64(Ws + wpos(k_lo, c) + 8 * (r & 1));
                p1[ks][j] = ds_read_tr_b64(Ws + wpos(k_hi, c) + 8 * (r & 1));
            }
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = 16 * i + r;
                a[ks][i] = *reinterpret_cast<const u32x4*>(As + (row << 7) + (((4 * ks + g) ^ swz_a(row)) << 4));
            }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(p0[ks][j]), "+v"(p1[ks][j]) : : "memory");
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const u32x4 bf = u32x4{p0[ks][j][0], p0[ks][j][1], p1[ks][j][0], p1[ks][j][1]};
#pragma unroll
                for (int i = 0; i < FM; ++i) acc[i][j] = mfma16x16x32(a[ks][i], bf, acc[i][j]);
            }
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int col = n0 + 16 * j + r;
        if (col >= N) continue;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * i + 4 * g + e;
                if (row >= M) continue;
                if (c_f32)
                    reinterpret_cast<float*>(C)[(int64_t)row * ldc + col] = acc[i][j][e];
                else
                    reinterpret_cast<bf16_t*>(C)[(int64_t)row * ldc + col] = (bf16_t)f32_to_bf16(acc[i][j][e]);
            }
    }
}

template <int FM, int FN, int NS>
hipError_t launch_skinny(const void* A, int64_t lda, const void* W, int64_t ldw, void* C,
                         int64_t ldc, int M, int N, int K, int c_f32, hipStream_t s) {
    const int strips = (N + 16 * FN - 1) / (16 * FN);
    constexpr int GS = (FN >= 8) ? 1 : 8 / FN;
    const int grid = (strips + 8 * GS - 1) / (8 * GS) * (8 * GS);
    hipLaunchKernelGGL((gemm_skinny_kernel<FM, FN, NS>), dim3((unsigned)grid), dim3(64), 0, s,
                       (const bf16_t*)A, lda, (const bf16_t*)W, ldw, C, ldc, M, N, K, c_f32);
    return hipGetLastError();
}

// ------------------------------------------------------- few rows, four waves
// M <= 64 (decode batches).  A single wave can issue only about one 1 KB
// HBM -> LDS copy (buffer_load ... lds) per ~70 cycles, however deep its ring
// (measured: ~13 bytes per clock per CU from one wave, ~47 from eight), so a
// strip streamed by one wave is bound by that issue rate, not by memory.  Here
// a workgroup of four waves owns one strip of 16 FN columns of W and all M
// rows (RT row tiles of 16).  K-tile kt (64 rows of W, the matching 64 columns
// of A) is copied into stage kt % (4 R) of an LDS ring by wave kt % 4; one
// round = four consecutive K-tiles, one per wave; copies run up to D rounds
// ahead.  One workgroup barrier per round publishes the next round's stages
// and frees the current round's stages for the copies of round r + D (D <= R),
// so a computing wave reads round r + 1's fragments while round r's MFMAs run.
// Wave w computes row tile w (rows 16w .. 16w + 15) if it holds rows < M.
// Each element's arithmetic is the tile kernels' exactly: one fp32
// accumulator, v_mfma_f32_16x16x32_bf16 over the same 32-wide k-blocks in
// ascending order, the same zero padding of a ragged K-tile and of columns
// past N (copies of rows k >= K and of columns n >= N read zero).
// LDS layout per stage: A [16 RT][64] as in the big tile (chunk c of row r at
// c ^ (r & 7)), W [64][16 FN] as in gemm_skinny_kernel (wpos).
template <int FN, int RT, int R, int D, bool PK>
__global__ __launch_bounds__(256) void gemm_strip_kernel(const bf16_t* __restrict__ A, int64_t lda,
                                                         const bf16_t* __restrict__ W, int64_t ldw,
                                                         void* __restrict__ C, int64_t ldc, int M,
                                                         int N, int K, int c_f32) {
    constexpr int NWV = 4;
    // copying waves: with one row tile the computing wave 0 copies nothing
    // (each copy instruction costs its wave tens of cycles to issue), and a
    // round is two K-tiles per copying wave; with four row tiles every wave
    // copies one K-tile per round
    constexpr int NCW = RT == 1 ? 3 : 4, CW0 = NWV - NCW, PER = RT == 1 ? 2 : 1;
    constexpr int KR = NCW * PER;                              // K-tiles per round
    constexpr int BN = 16 * FN, RB = 2 * BN;                 // row bytes of the W strip
    constexpr int A_BYTES = 16 * RT * BK * 2, W_BYTES = BK * RB, STAGE = A_BYTES + W_BYTES;
    constexpr int PA = A_BYTES / 1024, PW = W_BYTES / 1024, P = PER * (PA + PW);
    constexpr int NSTG = KR * R;
    constexpr int RPI = 1024 / RB, LPR = RB / 16;             // W rows per copy, lanes per row
    static_assert(D >= 2 && D <= R, "copies run at most R rounds ahead");
    static_assert((D - 1) * P <= 63, "vmcnt holds 6 bits");
    __shared__ __attribute__((aligned(1024))) char smem[NSTG * STAGE];
    // the wave index as a scalar, so that every copy's LDS address is known
    // to be wave-uniform (no per-lane loop around the copies)
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int b = blockIdx.x, x = b & 7, local = b >> 3;
    constexpr int GS = (FN >= 8) ? 1 : 8 / FN;                // strips per 128-byte line group
    const int n0 = ((local / GS) * 8 * GS + x * GS + (local % GS)) * BN;
    if (n0 >= N) return;                                      // whole workgroup
    const int nk = (K + BK - 1) / BK;
    const int nr = (nk + KR - 1) / KR;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)A, (short)0, (int)((int64_t)M * lda * 2), RSRC_WORD3);
    // packed weights (PK): the runs of this workgroup's strips, nkb k-blocks
    // of 1 KB each, bounded at the last strip that holds columns < N
    const int nkb = 2 * nk;
    const int s0 = n0 / 16, sv = min(FN, (N + 15) / 16 - s0);
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(W) + (int64_t)s0 * nkb * 1024), (short)0,
        PK ? sv * nkb * 1024 : 0, RSRC_WORD3);
    // this wave's first K-tile of round rd (copying waves only)
    const int cw = wave - CW0;
    auto first_kt = [&](int rd) { return KR * rd + PER * cw; };
    auto wpos = [&](int k, int c) -> int {
        if constexpr (FN == 1) return skinny_row(k) * RB + c * 16;
        else if constexpr (FN == 2) return k * RB + ((c ^ (2 * ((k >> 3) & 1))) << 4);
        else return k * RB + ((c ^ (2 * (((k >> 1) & 1) + 2 * ((k >> 3) & 1)))) << 4);
    };
    auto issue = [&](int kt) {
        char* As = smem + (kt % NSTG) * STAGE;
        char* Ws = As + A_BYTES;
        const int k0 = kt * BK;
#pragma unroll
        for (int u = 0; u < PA; ++u) {
            const int row = 8 * u + (lane >> 3);
            const int c = (lane & 7) ^ swz_a(row);
            const int kk = k0 + 8 * c;
            const int off = (row < M && kk < K) ? (row * (int)lda + kk) * 2 : OOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(As + u * 1024), 16, off, 0, 0, 0);
        }
        if constexpr (PK) {
            // packed weights: the K-tile of strip s0 + jj is the 2 KB at
            // k-blocks 2 kt, 2 kt + 1 of that strip's run; strips past N lie
            // past the buffer's bound and read zero
#pragma unroll
            for (int u = 0; u < PW; ++u) {
                const int off = ((u >> 1) * nkb + 2 * kt + (u & 1)) * 1024 + lane * 16;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rp, (lds_void*)(Ws + u * 1024), 16, off, 0, 0, 0);
            }
            return;
        }
        const int krows = min(BK, K - k0);
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(W + (int64_t)k0 * ldw + n0), (short)0, (int)((int64_t)krows * ldw * 2), RSRC_WORD3);
#pragma unroll
        for (int u = 0; u < PW; ++u) {
            const int pr = RPI * u + lane / LPR, pcpos = lane % LPR;
            int kr, pc;
            if constexpr (FN == 1) { kr = skinny_row(pr); pc = pcpos; }
            else if constexpr (FN == 2) { kr = pr; pc = pcpos ^ (2 * ((pr >> 3) & 1)); }
            else { kr = pr; pc = pcpos ^ (2 * (((pr >> 1) & 1) + 2 * ((pr >> 3) & 1))); }
            const int off = (kr < krows && n0 + 8 * pc < N) ? (kr * (int)ldw + 8 * pc) * 2 : OOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(Ws + u * 1024), 16, off, 0, 0, 0);
        }
    };
    // the copies of round rd by this wave (its PER K-tiles that exist)
    auto copy_round = [&](int rd) {
        if (cw < 0) return;
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int kt = first_kt(rd) + p;
            if (kt < nk) issue(kt);
        }
    };
#pragma unroll
    for (int rr = 0; rr < D; ++rr) copy_round(rr);
    f32x4 acc[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool computes = (wave < RT) && (16 * wave < M);
    // fragments of one round, as the computing wave reads them from LDS
    struct Frags {
        u32x2 p0[KR][2][FN], p1[KR][2][FN];
        u32x4 b[KR][2][FN];                           // packed weights: whole fragments
        u32x4 a[KR][2];
    };
    // read round rd's fragments (stages of K-tiles >= nk hold stale data that
    // is read but never fed to an MFMA).  With one row tile the computing wave
    // issues no copies and reads through the compiler's transposing-read
    // builtin, so the compiler tracks the reads (its wait for outstanding LDS
    // copies before them is empty for this wave) and they may stay in flight
    // across the next barrier.  With four row tiles every wave also copies, so
    // the reads are inline asm (no wait for the wave's own copies in flight)
    // and are waited for before anything else uses their registers.
    constexpr bool PIPE = (RT == 1);
    auto read_round = [&](Frags& f, int rd) {
#pragma unroll
        for (int j = 0; j < KR; ++j) {
            const char* As = smem + ((KR * rd + j) % NSTG) * STAGE;
            const char* Ws = As + A_BYTES;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int k_lo = 32 * ks + 8 * g + (r >> 2), k_hi = k_lo + 4;
#pragma unroll
                for (int jj = 0; jj < FN; ++jj) {
                    if constexpr (PK) {
                        // packed: column r, k 8 g .. 8 g + 7 of the k-block
                        // are the 16 bytes at r * 64 + g * 16
                        const char* pb = Ws + jj * 2048 + ks * 1024 + r * 64 + g * 16;
                        if constexpr (PIPE) f.b[j][ks][jj] = *reinterpret_cast<const u32x4*>(pb);
                        else f.b[j][ks][jj] = ds_read_b128_asm(pb);
                        continue;
                    }
                    const int c = 2 * jj + ((r & 3) >> 1);
                    const char* plo = Ws + wpos(k_lo, c) + 8 * (r & 1);
                    const char* phi = Ws + wpos(k_hi, c) + 8 * (r & 1);
                    if constexpr (PIPE) {
                        f.p0[j][ks][jj] = __builtin_bit_cast(
                            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)plo));
                        f.p1[j][ks][jj] = __builtin_bit_cast(
                            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)phi));
                    } else {
                        f.p0[j][ks][jj] = ds_read_tr_b64(plo);
                        f.p1[j][ks][jj] = ds_read_tr_b64(phi);
                    }
                }
                const int row = 16 * wave + r;
                f.a[j][ks] = *reinterpret_cast<const u32x4*>(
                    As + (row << 7) + (((4 * ks + g) ^ swz_a(row)) << 4));
            }
        }
        if constexpr (!PIPE) {
#pragma unroll
            for (int j = 0; j < KR; ++j)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int jj = 0; jj < FN; ++jj) {
                        if constexpr (PK)
                            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(f.b[j][ks][jj]) : : "memory");
                        else
                            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(f.p0[j][ks][jj]), "+v"(f.p1[j][ks][jj]) : : "memory");
                    }
        }
    };
    // MFMAs of round rd, K-tiles in order, each k-step in order
    auto mfma_tile = [&](Frags& f, int j) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int jj = 0; jj < FN; ++jj) {
                const u32x4 bf = PK ? f.b[j][ks][jj]
                                    : u32x4{f.p0[j][ks][jj][0], f.p0[j][ks][jj][1],
                                            f.p1[j][ks][jj][0], f.p1[j][ks][jj][1]};
                acc[jj] = mfma16x16x32(f.a[j][ks], bf, acc[jj]);
            }
    };
    auto mfma_round = [&](Frags& f, int rd) {
        if (KR * (rd + 1) <= nk) {                    // a full round: no per-tile test
#pragma unroll
            for (int j = 0; j < KR; ++j) mfma_tile(f, j);
        } else {
#pragma unroll
            for (int j = 0; j < KR; ++j)
                if (KR * rd + j < nk) mfma_tile(f, j);
        }
    };
    // barrier certifying round rd: this wave's copies of round rd have landed
    // (`later` rounds after it may still be in flight: an exact count only
    // while every one of them was issued, else wait for everything) and so
    // have every other wave's; the computing waves have finished reading the
    // rounds before rd
    auto certify = [&](int rd, auto later) {
        constexpr int L = decltype(later)::value;
        if (cw < 0) {
        } else if (first_kt(rd + L) + PER - 1 < nk) {
            asm volatile("s_waitcnt vmcnt(%0)" :: "n"(L * P) : "memory");
        } else {
            wait_vm0();
        }
        // every LDS read retired, as a builtin so that the compiler knows it
        // (no further wait for them before the MFMAs that use them): gfx9
        // s_waitcnt encoding, lgkmcnt 0, vmcnt 63 and expcnt 7 (no wait)
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    Frags fa, fb;
    certify(0, std::integral_constant<int, D - 1>{});
    if (computes) read_round(fa, 0);
    // round rd: certify round rd + 1, copy round rd + D into the stage of
    // round rd + D - R (read before this barrier, as D <= R), read round
    // rd + 1 while round rd's MFMAs run
    auto step = [&](Frags& cur, Frags& nxt, int rd) {
        if (rd + 1 < nr) certify(rd + 1, std::integral_constant<int, D - 2>{});
        if (rd + 1 < nr) copy_round(rd + D);
        if (computes) {
            if (rd + 1 < nr) read_round(nxt, rd + 1);
            mfma_round(cur, rd);
        }
    };
    for (int rd = 0; rd < nr; rd += 2) {
        step(fa, fb, rd);
        if (rd + 1 < nr) step(fb, fa, rd + 1);
    }
    if (!computes) return;
#pragma unroll
    for (int jj = 0; jj < FN; ++jj) {
        const int col = n0 + 16 * jj + r;
        if (col >= N) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * wave + 4 * g + e;
            if (row >= M) continue;
            if (c_f32)
                reinterpret_cast<float*>(C)[(int64_t)row * ldc + col] = acc[jj][e];
            else
                reinterpret_cast<bf16_t*>(C)[(int64_t)row * ldc + col] = (bf16_t)f32_to_bf16(acc[jj][e]);
        }
    }
}

template <int FN, int RT, int R, int D, bool PK = false>
hipError_t launch_strip(const void* A, int64_t lda, const void* W, int64_t ldw, void* C,
                        int64_t ldc, int M, int N, int K, int c_f32, hipStream_t s) {
    const int strips = (N + 16 * FN - 1) / (16 * FN);
    constexpr int GS = (FN >= 8) ? 1 : 8 / FN;
    const int grid = (strips + 8 * GS - 1) / (8 * GS) * (8 * GS);
    hipLaunchKernelGGL((gemm_strip_kernel<FN, RT, R, D, PK>), dim3((unsigned)grid), dim3(256), 0, s,
                       (const bf16_t*)A, lda, (const bf16_t*)W, ldw, C, ldc, M, N, K, c_f32);
    return hipGetLastError();
}

using BigTile = Tile<256, 256, 2, 4, 8>;
using MidTile = Tile<128, 128, 2, 2, 8>;         // the comparator's tile
// 8 waves of 32 x 64 (two per SIMD) and four LDS stages: 12-16 % faster at
// M = 768-1024 than 4 waves of 64 x 64
using MidTile4 = Tile<128, 128, 4, 2, 8, 4>;
using SmallTile = Tile<64, 64, 2, 2, 8, 4>;      // 4 waves of 32 x 32, four stages
// 16 waves of 64 x 32 (four per SIMD), three stages: 5-9 % faster at M = 2048,
// N = 4096 than 8 waves of 64 x 64, the same at N = 14336
using WideTile = Tile<256, 128, 4, 4, 8, 3>;

// ------------------------------------------------------------------ large M
// The 256 x 256 tile of BigTile (same LDS stages, same DMA, same fragments,
// same per-element MFMA chain, so the same bits), scheduled so that the matrix
// cores of a SIMD are not kept waiting on LDS reads.  The eight waves form two
// groups of four: group 0 (waves 0-3) owns tile rows 0-127, group 1 rows
// 128-255, and each SIMD runs one wave of each group.  Per K-tile a wave has
// two phases: M, reading all its A and W fragments of the K-tile (both
// 32-wide k-steps) from LDS into registers, and C, its 64 MFMAs on those
// registers alone.  Group 1 starts one workgroup barrier behind group 0, and
// every wave passes one barrier per phase, so the two waves on a SIMD are
// always in opposite phases: one feeds its MFMAs back to back while the other
// reads LDS.  With barrier events e1, e2, ...:
//   group 0: e(2kt+1) M(kt) e(2kt+2) C(kt)       (one extra barrier at the end)
//   group 1: e(2kt+2) M(kt) e(2kt+3) C(kt)       (one extra barrier at the start)
// Stage kt & 1 is read by group 0 in [e(2kt+1), e(2kt+2)] and by group 1 in
// [e(2kt+2), e(2kt+3)], so it is free after e(2kt+3).  K-tile kt + 2 goes into
// it then: group 0 requests its share during M(kt + 1), group 1 at the start
// of C(kt); each wave waits for its own share before the barrier at which
// group 0 starts reading that K-tile (e(2kt+5)), two phases later.  Every
// barrier is preceded by lgkmcnt(0), so no LDS read is in flight when a stage
// is handed to the DMA.
__device__ __forceinline__ void pp_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

template <class T>
__device__ __forceinline__ void pp_load(const char* As, const char* Ws, u32x4 (&a)[2][T::FM],
                                        u32x4 (&b)[2][T::FN], int wm, int wn, int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
            const int c = (wn * T::TN + 16 * j + 4 * (r & 3)) >> 3;
            const int k_lo = 32 * ks + 8 * g + (r >> 2), k_hi = k_lo + 4;
            const v4i16 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4i16*)(Ws + k_lo * T::BN_ * 2 + ((c ^ T::swzw(k_lo)) << 4) + 8 * (r & 1)));
            const v4i16 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4i16*)(Ws + k_hi * T::BN_ * 2 + ((c ^ T::swzw(k_hi)) << 4) + 8 * (r & 1)));
            const u32x2 p0 = __builtin_bit_cast(u32x2, h0), p1 = __builtin_bit_cast(u32x2, h1);
            b[ks][j] = u32x4{p0[0], p0[1], p1[0], p1[1]};
        }
#pragma unroll
        for (int i = 0; i < T::FM; ++i) {
            const int row = wm * T::TM + 16 * i + r;
            a[ks][i] = *reinterpret_cast<const u32x4*>(As + (row << 7) +
                                                       (((4 * ks + g) ^ swz_a(row)) << 4));
        }
    }
}

template <class T>
__device__ __forceinline__ void pp_mfma(const u32x4 (&a)[2][T::FM], const u32x4 (&b)[2][T::FN],
                                        f32x4 (&acc)[T::FM][T::FN]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
#pragma unroll
            for (int j = 0; j < T::FN; ++j) acc[i][j] = mfma16x16x32(a[ks][i], b[ks][j], acc[i][j]);
}

// DMA of K-tile kt into stage kt & 1 for a tile that lies wholly inside A, W
// and C with K a multiple of 64 (the tiles that take the two-group schedule): the same copies as Tile::issue (same LDS
// positions, same swizzles), with no bounds tests, each lane's offset a
// per-lane base plus a wave-uniform part.
struct PPFull {
    int va, vw0, vw1;          // per-lane byte offsets: A; W rows of even / odd u
    __device__ PPFull(int64_t lda, int64_t ldw, int wave, int lane) {
        const int ra = lane >> 3;
        va = ra * (int)lda * 2 + (((lane & 7) ^ swz_a(ra)) << 4);
        const int rw = lane >> 5;
        vw0 = rw * (int)ldw * 2 + (((lane & 31) ^ swz_w(8 * wave + 0 + rw)) << 4);
        vw1 = rw * (int)ldw * 2 + (((lane & 31) ^ swz_w(8 * wave + 2 + rw)) << 4);
    }
    __device__ void issue(char* smem, int kt, const bf16_t* A, int64_t lda, const bf16_t* W,
                          int64_t ldw, int m0, int n0, int wave) const {
        using T = BigTile;
        char* As = smem + (kt & 1) * T::STAGE;
        char* Ws = As + T::A_BYTES;
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(A + (int64_t)m0 * lda), (short)0, (int)(T::BM_ * lda * 2), RSRC_WORD3);
#pragma unroll
        for (int u = 0; u < T::A_PW; ++u) {
            const int j = wave * T::A_PW + u;                  // rows 8j .. 8j + 7
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(As + j * 1024), 16, va,
                                                     8 * j * (int)lda * 2 + kt * BK * 2, 0, 0);
        }
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(W + (int64_t)kt * BK * ldw + n0), (short)0, (int)(BK * ldw * 2), RSRC_WORD3);
#pragma unroll
        for (int u = 0; u < T::W_PW; ++u) {
            const int j = wave * T::W_PW + u;                  // rows 2j, 2j + 1
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(Ws + j * 1024), 16,
                                                     (u & 1) ? vw1 : vw0, 2 * j * (int)ldw * 2, 0,
                                                     0);
        }
    }
};
static_assert(BigTile::W_PW == 4 && BigTile::WROWS == 2 && BigTile::BN_ / 8 == 32,
              "PPFull assumes the 256 x 256 tile's W copy geometry");

__device__ __forceinline__ void pp_body(const bf16_t* __restrict__ A, int64_t lda,
                                        const bf16_t* __restrict__ W, int64_t ldw,
                                        void* __restrict__ C, int64_t ldc, int M, int N, int K,
                                        int c_f32, int m0, int n0, char* smem) {
    using T = BigTile;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int grp = wave >> 2, wm = grp, wn = wave & 3;
    const int nk = (K + BK - 1) / BK;
    f32x4 acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 a[2][T::FM], b[2][T::FN];
    const PPFull pf(lda, ldw, wave, lane);
    auto issue = [&](int kt) { pf.issue(smem, kt, A, lda, W, ldw, m0, n0, wave); };
    if (grp == 0) {
        if (nk > 0) issue(0);
        wait_vm0();
        for (int kt = 0; kt < nk; ++kt) {
            pp_barrier();                                         // e(2kt+1)
            const char* As = smem + (kt & 1) * T::STAGE;
            pp_load<T>(As, As + T::A_BYTES, a, b, wm, wn, lane);
            if (kt + 1 < nk) issue(kt + 1);                       // stage (kt+1)&1 freed at e(2kt+1)
            pp_barrier();                                         // e(2kt+2)
            pp_mfma<T>(a, b, acc);
            // the wait stays after the MFMAs (the scheduler would otherwise
            // hoist it above them and stall on the copy just issued)
            __builtin_amdgcn_sched_barrier(0);
            wait_vm0();                                           // this wave's share of kt+1
        }
        pp_barrier();                                             // e(2nk+1)
    } else {
        if (nk > 0) issue(0);
        if (nk > 1) {
            issue(1);
            asm volatile("s_waitcnt vmcnt(%0)" :: "n"(T::PW) : "memory");
        } else {
            wait_vm0();
        }
        pp_barrier();                                             // e1
        for (int kt = 0; kt < nk; ++kt) {
            pp_barrier();                                         // e(2kt+2)
            const char* As = smem + (kt & 1) * T::STAGE;
            pp_load<T>(As, As + T::A_BYTES, a, b, wm, wn, lane);
            __builtin_amdgcn_sched_barrier(0);
            wait_vm0();                                           // this wave's share of kt+1
            pp_barrier();                                         // e(2kt+3): stage kt&1 free
            if (kt + 2 < nk) issue(kt + 2);
            pp_mfma<T>(a, b, acc);
        }
    }
    T::store_c(acc, C, ldc, m0 + wm * T::TM, n0 + wn * T::TN, lane, M, N, c_f32);
}

__global__ __launch_bounds__(512) void gemm_pp_kernel(const bf16_t* __restrict__ A, int64_t lda,
                                                      const bf16_t* __restrict__ W, int64_t ldw,
                                                      void* __restrict__ C, int64_t ldc, int M,
                                                      int N, int K, int c_f32) {
    using T = BigTile;
    __shared__ __attribute__((aligned(1024))) char smem[2 * T::STAGE];
    int tm, tn;
    tile_of<8>(blockIdx.x, (M + T::BM_ - 1) / T::BM_, (N + T::BN_ - 1) / T::BN_, tm, tn);
    const int m0 = tm * T::BM_, n0 = tn * T::BN_;
    // A tile wholly inside A, W and C with no ragged K-tile takes the two-group
    // schedule, whose copies need no bounds tests; a tile on the edge of C or
    // of a ragged K takes BigTile's one-group schedule with its bounds-tested
    // copies (uniform branch).  Both run the same per-element MFMA chain.
    if (m0 + T::BM_ <= M && n0 + T::BN_ <= N && K % BK == 0)
        pp_body(A, lda, W, ldw, C, ldc, M, N, K, c_f32, m0, n0, smem);
    else
        T::template run<false>(A, lda, W, ldw, C, ldc, 0, M, N, K, 0, c_f32, smem);
}

template <class T, bool SPLIT>
__global__ __launch_bounds__(T::NT) void gemm_tile_kernel(const bf16_t* __restrict__ A, int64_t lda,
                                                          const bf16_t* __restrict__ W, int64_t ldw,
                                                          void* __restrict__ C, int64_t ldc,
                                                          int64_t split_stride, int M, int N, int K,
                                                          int kt_per_split, int c_f32) {
    __shared__ __attribute__((aligned(1024))) char smem[T::NS_ * T::STAGE];
    T::template run<SPLIT>(A, lda, W, ldw, C, ldc, split_stride, M, N, K, kt_per_split, c_f32,
                           smem);
}

// comparator only: out[i, j] = sum over splits s = 0..S-1 (ascending) of part[s][i, j]
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int S, int64_t MN, int N,
                                                            void* __restrict__ C, int64_t ldc,
                                                            int c_f32) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= MN) return;
    float s = part[idx];
    for (int z = 1; z < S; ++z) s += part[(int64_t)z * MN + idx];
    const int64_t row = idx / N, col = idx % N;
    if (c_f32)
        reinterpret_cast<float*>(C)[row * ldc + col] = s;
    else
        reinterpret_cast<bf16_t*>(C)[row * ldc + col] = (bf16_t)f32_to_bf16(s);
}

template <class T>
hipError_t launch_tile(const void* A, int64_t lda, const void* W, int64_t ldw, void* C,
                       int64_t ldc, int64_t split_stride, int M, int N, int K, int S, int per,
                       int c_f32, hipStream_t s) {
    const int tiles = ((M + T::BM_ - 1) / T::BM_) * ((N + T::BN_ - 1) / T::BN_);
    dim3 grid((unsigned)tiles, 1, (unsigned)S), block(T::NT);
    if (S > 1)
        hipLaunchKernelGGL((gemm_tile_kernel<T, true>), grid, block, 0, s, (const bf16_t*)A, lda,
                           (const bf16_t*)W, ldw, C, ldc, split_stride, M, N, K, per, c_f32);
    else
        hipLaunchKernelGGL((gemm_tile_kernel<T, false>), grid, block, 0, s, (const bf16_t*)A, lda,
                           (const bf16_t*)W, ldw, C, ldc, split_stride, M, N, K, per, c_f32);
    return hipGetLastError();
}

}  // namespace

// Which kernel computes the outputs is chosen from the shape: the 256 x 256
// tile once it gives at least 192 tiles (fills most of the 256 CUs); else
// strips for M <= 64; else 256 x 128, then 128 x 128 tiles if they give at
// least 192; else 64 x 64 tiles.  (Each tile kernel moves about the same
// bytes per CU per second from L2 into LDS, so the largest tile that still
// fills the GPU -- the most flops per operand byte -- is the fastest.)  All of them run
// the same per-element arithmetic -- one accumulator, one MFMA chain over the
// same ascending 32-wide k-blocks and the same zero-padded K-tiles of 64 --
// so the choice, and with it M, never reaches the bits.
hipError_t launch_gemm(const void* A, int64_t lda, const void* W, int64_t ldw, void* C,
                       int c_f32, int64_t ldc, int M, int N, int K, hipStream_t s) {
    if (M == 0 || N == 0) return hipSuccess;
    const int nk = (K + BK - 1) / BK;
    const int64_t big_tiles = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
    if (big_tiles >= 192) {
        hipLaunchKernelGGL(gemm_pp_kernel, dim3((unsigned)big_tiles), dim3(512), 0, s,
                           (const bf16_t*)A, lda, (const bf16_t*)W, ldw, C, ldc, M, N, K, c_f32);
        return hipGetLastError();
    }
    if (M > 64) {
        const int64_t wide_tiles = (int64_t)((M + 255) / 256) * ((N + 127) / 128);
        if (wide_tiles >= 192)
            return launch_tile<WideTile>(A, lda, W, ldw, C, ldc, 0, M, N, K, 1, nk > 0 ? nk : 1,
                                         c_f32, s);
        const int64_t mid_tiles = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
        if (mid_tiles >= 192)
            return launch_tile<MidTile4>(A, lda, W, ldw, C, ldc, 0, M, N, K, 1, nk > 0 ? nk : 1,
                                         c_f32, s);
        return launch_tile<SmallTile>(A, lda, W, ldw, C, ldc, 0, M, N, K, 1, nk > 0 ? nk : 1,
                                      c_f32, s);
    }
    {
        // strips of 16 FN columns, FN the widest that still gives >= 192 strips.
        // Up to 8192-wide outputs (FN = 1, 2: at most 512 strips) a strip is one
        // four-wave workgroup (gemm_strip_kernel, one row tile for decode
        // batches of up to 16, four up to 64; ring of R rounds, copies D rounds
        // ahead, sized to the LDS and the 6-bit copy counter; FN = 2 with one
        // row tile fits two workgroups per CU).  Wider outputs (FN = 4) give
        // each CU several one-wave strips (gemm_skinny_kernel), whose copies
        // then come from several waves as well.
        const int fn = (N / 64 >= 192) ? 4 : (N / 32 >= 192) ? 2 : 1;
        if (fn == 4) {
            if (M <= 16) return launch_skinny<1, 4, 6>(A, lda, W, ldw, C, ldc, M, N, K, c_f32, s);
            if (M <= 32) return launch_skinny<2, 4, 4>(A, lda, W, ldw, C, ldc, M, N, K, c_f32, s);
            return launch_skinny<4, 4, 4>(A, lda, W, ldw, C, ldc, M, N, K, c_f32, s);
        }
        if (M <= 16) {
            if (fn == 2) return launch_strip<2, 1, 3, 3>(A, lda, W, ldw, C, ldc, M, N, K, c_f32, s);
            return launch_strip<1, 1, 6, 6>(A, lda, W, ldw, C, ldc, M, N, K, c_f32, s);
        }
        if (fn == 2) return launch_strip<2, 4, 3, 3>(A, lda, W, ldw, C, ldc, M, N, K, c_f32, s);
        return launch_strip<1, 4, 3, 3>(A, lda, W, ldw, C, ldc, M, N, K, c_f32, s);
    }
    return hipErrorInvalidValue;        // not reached
}

// Decode batches over packed weights (binv_gemm_bf16_packed): the strip
// kernel with each DMA one whole 1 KB k-block of one strip (no row pieces),
// the B fragment one 16-byte LDS read.  The MFMA chain is the one above.
hipError_t launch_gemm_strips_packed(const void* A, int64_t lda, const void* Wp, void* C,
                                     int c_f32, int64_t ldc, int M, int N, int K, hipStream_t s) {
    if (M == 0 || N == 0) return hipSuccess;
    // Up to 16 rows one row tile: one-strip workgroups, with a ring of 6
    // rounds (one workgroup per CU) up to 6144 columns, of 3 rounds (two per
    // CU) beyond.  Up to 64 rows four row tiles, two strips per workgroup
    // from 6144 columns on.
    const int fn = (N / 32 >= 192) ? 2 : 1;
    if (M <= 16) {
        if (fn == 2) return launch_strip<1, 1, 3, 3, true>(A, lda, Wp, 0, C, ldc, M, N, K, c_f32, s);
        return launch_strip<1, 1, 6, 6, true>(A, lda, Wp, 0, C, ldc, M, N, K, c_f32, s);
    }
    if (fn == 2) return launch_strip<2, 4, 3, 3, true>(A, lda, Wp, 0, C, ldc, M, N, K, c_f32, s);
    return launch_strip<1, 4, 3, 3, true>(A, lda, Wp, 0, C, ldc, M, N, K, c_f32, s);
}

// Comparator: split-K whose split count is chosen from the number of output
// tiles, i.e. from M -- the strategy the invariant kernel refuses.
static int tuned_splits(int64_t M, int64_t N, int64_t K) {
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    const int64_t nk = (K + BK - 1) / BK;
    int64_t S = (512 + tiles - 1) / tiles;
    if (S > 16) S = 16;
    if (S > nk / 4) S = nk / 4;
    if (S < 1) S = 1;
    return (int)S;
}

size_t gemm_tuned_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const int S = tuned_splits(M, N, K);
    return S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_gemm_tuned(const void* A, int64_t lda, const void* W, int64_t ldw, void* C,
                             int c_f32, int64_t ldc, int M, int N, int K, void* ws,
                             hipStream_t s) {
    if (M == 0 || N == 0) return hipSuccess;
    const int S = tuned_splits(M, N, K);
    const int nk = (K + BK - 1) / BK;
    if (S == 1)
        return launch_tile<MidTile>(A, lda, W, ldw, C, ldc, 0, M, N, K, 1, nk > 0 ? nk : 1,
                                      c_f32, s);
    const int per = (nk + S - 1) / S;
    const int Sused = (nk + per - 1) / per;
    hipError_t e = launch_tile<MidTile>(A, lda, W, ldw, ws, N, (int64_t)M * N, M, N, K, Sused,
                                          per, 1, s);
    if (e != hipSuccess) return e;
    const int64_t MN = (int64_t)M * N;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, s,
                       (const float*)ws, Sused, MN, N, C, ldc, c_f32);
    return hipGetLastError();
}

}  // namespace binv
