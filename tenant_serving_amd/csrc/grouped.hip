// Grouped multi-variant linear: one shared bf16 base, up to 64 packed deltas,
// each token with its own variant.
//
// "BitDelta : servir 14 modèles Zen depuis un seul cluster GPU" (hanzo-blog,
// 2026-02-28), "Serving architecture": the base weights are HBM resident and
// read by every variant ("shared read"), the delta cache holds one
// (α, sign(Δ)) entry per variant, and the router sends each request to its
// variant's entry.  Here one launch serves a batch that mixes variants:
// y[m] = x[m]·W_eff(ids[m])ᵀ.
//
// Three kernels:
//  1. bucket: counts tokens per variant, orders them by variant (stable),
//     cuts each variant's tokens into m-tiles of <= 16 and groups the
//     m-tiles into passes of <= kMaxTiles tiles / kMaxSegs variants.
//  2. main: a workgroup owns 128 rows of the base (8 waves x 16 rows) and a
//     K range.  Per 64-wide k stage every lane loads 16 base weights of its
//     row once, and for each variant present rebuilds them with that
//     variant's sign bits and α (recon8) and feeds them, as the B operand of
//     v_mfma_f32_16x16x32_bf16, to every m-tile of that variant; the
//     m-tiles' x rows are gathered once per stage into LDS and shared by the
//     8 waves.  The base is therefore read from HBM once per K range,
//     however many variants there are; the rebuild is paid once per
//     (variant, weight).
//  3. reduce: sums the K-range partials in a fixed order into y, and writes
//     NaN rows for tokens whose id is out of range.
//
// K ranges are assigned by workgroup id modulo the split, and workgroups are
// dealt to the 8 XCDs round robin, so each XCD works on one K range and the
// gathered x slice of that range stays in its L2.
#include <type_traits>

#include "bd_device.h"
#include "bd_internal.h"

namespace bd {
namespace {

constexpr int kMaxTiles = 32;  // m-tiles per pass (accumulators per wave)
constexpr int kMaxSegs = 16;   // variants per pass
constexpr int kWaves = 8;
constexpr int kRowsPerBlock = kWaves * 16;
constexpr int kStage = 64;     // k per LDS stage
constexpr int kBucketThreads = 1024;

struct Layout {
    int64_t max_segs, max_tiles, max_passes;
    size_t hdr, tile_var, tile_off, tile_cnt, tile_seg, pass_first, pass_nseg, seg_var, seg_off,
        seg_cnt, perm, part, total;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int choose_ksplit(int64_t N) {
    int64_t rowblocks = (N + kRowsPerBlock - 1) / kRowsPerBlock;
    int ks = 1;
    while (ks < 8 && rowblocks * ks < 256) ks *= 2;
    return ks;
}

// Segments: (variant, up to 32 consecutive tokens of it in variant order),
// each covering two m-tiles of 16 (the second possibly short or empty); a
// pass holds up to kMaxSegs segments.  Every variant with n tokens gives
// ceil(n/32) segments, so there are at most G + M/32 of them.
Layout make_layout(int64_t M, int32_t G, int64_t N) {
    Layout L;
    L.max_segs = (int64_t)G + (M + 31) / 32;
    L.max_tiles = 2 * L.max_segs;
    L.max_passes = L.max_segs;
    size_t o = 0;
    L.hdr = o; o = align256(o + 4 * sizeof(int32_t));
    L.tile_var = o; o = align256(o + L.max_tiles * sizeof(int32_t));
    L.tile_off = o; o = align256(o + L.max_tiles * sizeof(int32_t));
    L.tile_cnt = o; o = align256(o + L.max_tiles * sizeof(int32_t));
    L.tile_seg = o; o = align256(o + L.max_tiles * sizeof(int32_t));
    L.pass_first = o; o = align256(o + (L.max_passes + 1) * sizeof(int32_t));
    L.pass_nseg = o; o = align256(o + L.max_passes * sizeof(int32_t));
    L.seg_var = o; o = align256(o + L.max_passes * kMaxSegs * sizeof(int32_t));
    L.seg_off = o; o = align256(o + L.max_passes * kMaxSegs * sizeof(int32_t));
    L.seg_cnt = o; o = align256(o + L.max_passes * kMaxSegs * sizeof(int32_t));
    L.perm = o; o = align256(o + (size_t)M * sizeof(int32_t));
    L.part = o; o = align256(o + (size_t)choose_ksplit(N) * M * N * sizeof(float));
    L.total = o;
    return L;
}

struct WsPtrs {
    int32_t *hdr, *tile_var, *tile_off, *tile_cnt, *tile_seg, *pass_first, *pass_nseg, *seg_var,
        *seg_off, *seg_cnt, *perm;
    float* part;
};

__global__ __launch_bounds__(kBucketThreads) void bucket_kernel(const int32_t* __restrict__ ids,
                                                               int64_t M, int G, WsPtrs ws) {
    __shared__ int count[kMaxVariants], offset[kMaxVariants], cursor[kMaxVariants];
    __shared__ int wcount[kBucketThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid < kMaxVariants) count[tid] = 0;
    __syncthreads();
    for (int64_t m = tid; m < M; m += kBucketThreads) {
        int g = ids[m];
        if (g >= 0 && g < G) atomicAdd(&count[g], 1);
    }
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int g = 0; g < G; ++g) {
            offset[g] = run;
            cursor[g] = run;
            run += count[g];
        }
    }
    __syncthreads();
    // Stable placement: token order is kept within each variant.
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int64_t base = 0; base < M; base += kBucketThreads) {
        int64_t m = base + tid;
        int g = m < M ? ids[m] : -1;
        for (int gg = 0; gg < G; ++gg) {
            bool f = (g == gg);
            uint64_t b = __ballot(f);
            if (lane == 0) wcount[wave] = __popcll(b);
            __syncthreads();
            int prefix = 0, total = 0;
            for (int w = 0; w < kBucketThreads / 64; ++w) {
                int c = wcount[w];
                prefix += w < wave ? c : 0;
                total += c;
            }
            if (f) ws.perm[cursor[gg] + prefix + __popcll(b & below)] = (int32_t)m;
            __syncthreads();
            if (tid == 0) cursor[gg] += total;
            __syncthreads();
        }
    }
    if (tid == 0) {
        // segments of <= 32 tokens, kMaxSegs per pass; the per-tile arrays
        // (two tiles per segment) serve the register-staged kernel
        int p = 0, nseg = 0, t = 0;
        ws.pass_first[0] = 0;
        for (int g = 0; g < G; ++g) {
            for (int r = 0; r < count[g]; r += 32) {
                if (nseg == kMaxSegs) {
                    ws.pass_nseg[p] = nseg;
                    ++p;
                    ws.pass_first[p] = t;
                    nseg = 0;
                }
                const int j = nseg++;
                const int off = offset[g] + r, cnt = min(32, count[g] - r);
                ws.seg_var[p * kMaxSegs + j] = g;
                ws.seg_off[p * kMaxSegs + j] = off;
                ws.seg_cnt[p * kMaxSegs + j] = cnt;
                for (int u = 0; u < 2; ++u, ++t) {
                    ws.tile_var[t] = g;
                    ws.tile_off[t] = off + 16 * u;
                    ws.tile_cnt[t] = max(0, min(16, cnt - 16 * u));
                    ws.tile_seg[t] = j;
                }
            }
        }
        if (nseg > 0) {
            ws.pass_nseg[p] = nseg;
            ++p;
            ws.pass_first[p] = t;
        }
        ws.hdr[0] = t;
        ws.hdr[1] = p;
    }
}

__device__ __forceinline__ int xswz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

__global__ __launch_bounds__(kWaves * 64) void grouped_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, VariantTable tab,
    int per_row, int64_t M, int64_t N, int64_t K, int ksplit, int64_t kchunk, WsPtrs ws) {
    __shared__ uint4 xs[kMaxTiles * 16 * 8];          // [tile row][8 chunks of 16 bytes]
    __shared__ float als[kMaxSegs][kRowsPerBlock];      // α of each pass variant, per row

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int kpart = blockIdx.x % ksplit;
    const int64_t rowblock = blockIdx.x / ksplit;
    const int64_t n = rowblock * kRowsPerBlock + wave * 16 + col;
    const int64_t nc = n < N ? n : N - 1;
    const int64_t kbeg = (int64_t)kpart * kchunk;
    const int64_t kend = kbeg + kchunk < K ? kbeg + kchunk : K;
    const int64_t kbytes = K / 8;
    const int64_t srow_off = nc * kbytes;  // same for every variant
    const uint4* wrow = reinterpret_cast<const uint4*>(w + nc * K);
    float* part = ws.part + (int64_t)kpart * M * N;

    const int npass = ws.hdr[1];
    for (int p = 0; p < npass; ++p) {
        const int t0 = ws.pass_first[p];
        const int nt = ws.pass_first[p + 1] - t0;
        const int nseg = ws.pass_nseg[p];

        // α of each variant of the pass for the workgroup's rows.
        for (int q = tid; q < kMaxSegs * kRowsPerBlock; q += kWaves * 64) {
            int j = q / kRowsPerBlock, r = q % kRowsPerBlock;
            int64_t rn = rowblock * kRowsPerBlock + r;
            rn = rn < N ? rn : N - 1;
            float v = 0.0f;
            if (j < nseg) v = tab.alpha[ws.seg_var[p * kMaxSegs + j]][per_row ? rn : 0];
            als[j][r] = v;
        }
        // Gather slots: fixed (tile row, chunk) per thread for the whole pass.
        constexpr int kSlots = kMaxTiles * 16 * 8 / (kWaves * 64);
        int32_t xtok[kSlots];
#pragma unroll
        for (int i = 0; i < kSlots; ++i) {
            int q = tid + i * kWaves * 64, row = q >> 3;
            int t = row >> 4, r = row & 15;
            xtok[i] = -1;
            if (t < nt && r < ws.tile_cnt[t0 + t]) xtok[i] = ws.perm[ws.tile_off[t0 + t] + r];
        }

        f32x4_t acc[kMaxTiles];
#pragma unroll
        for (int t = 0; t < kMaxTiles; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        for (int64_t k0 = kbeg; k0 < kend; k0 += kStage) {
            // This lane's 16 weights: k0 + 16·grp .. +16, as two 8-wide groups.
            const int64_t ka = k0 + 16 * grp, kb = ka + 8;
            const bool va = ka < kend, vb = kb < kend;
            uint4 w0 = va ? load_stream16(wrow + (ka >> 3)) : make_uint4(0, 0, 0, 0);
            uint4 w1 = vb ? load_stream16(wrow + (kb >> 3)) : make_uint4(0, 0, 0, 0);
            // Sign bytes of every pass variant: 16 bits each, two variants per register.
            uint32_t sb[kMaxSegs / 2];
#pragma unroll
            for (int j = 0; j < kMaxSegs; ++j) {
                uint32_t v = 0;
                if (j < nseg) {
                    const uint8_t* srow = tab.signs[ws.seg_var[p * kMaxSegs + j]] + srow_off;
                    // ordinary (cached) loads: a lane takes 2 bytes of a row
                    // per stage and the following stages find the rest of
                    // the line in cache
                    uint32_t lo = va ? (uint32_t)srow[ka >> 3] : 0u;
                    uint32_t hi = vb ? (uint32_t)srow[kb >> 3] : 0u;
                    v = lo | (hi << 8);
                }
                if (j & 1) sb[j >> 1] |= v << 16;
                else sb[j >> 1] = v;
            }
#pragma unroll
            for (int i = 0; i < kSlots; ++i) {
                int q = tid + i * kWaves * 64, row = q >> 3, c = q & 7;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (xtok[i] >= 0 && k0 + 8 * c < kend)
                    v = *reinterpret_cast<const uint4*>(x + (int64_t)xtok[i] * K + k0 + 8 * c);
                if ((row >> 4) < nt) xs[xswz(row, c)] = v;
            }
            __syncthreads();

            int cur = -1;
            bf16x8_t b0 = {}, b1 = {};
#pragma unroll
            for (int t = 0; t < kMaxTiles; ++t) {
                if (t < nt) {
                    const int seg = ws.tile_seg[t0 + t];
                    if (seg != cur) {
                        uint32_t s = sb[0];
#pragma unroll
                        for (int j = 1; j < kMaxSegs / 2; ++j) s = ((seg >> 1) == j) ? sb[j] : s;
                        s = (seg & 1) ? (s >> 16) : (s & 0xffffu);
                        const float a = als[seg][wave * 16 + col];
                        b0 = as_bf16x8(recon8(w0, s & 0xffu, a));
                        b1 = as_bf16x8(recon8(w1, s >> 8, a));
                        cur = seg;
                    }
                    bf16x8_t a0 = as_bf16x8(xs[xswz(t * 16 + col, 2 * grp)]);
                    bf16x8_t a1 = as_bf16x8(xs[xswz(t * 16 + col, 2 * grp + 1)]);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, acc[t], 0, 0, 0);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, acc[t], 0, 0, 0);
                }
            }
            __syncthreads();
        }

        // D layout of the 16x16 MFMA: lane holds rows 4·(lane/16) + i, column lane%16.
        if (n < N) {
#pragma unroll
            for (int t = 0; t < kMaxTiles; ++t) {
                if (t < nt) {
                    const int cnt = ws.tile_cnt[t0 + t], off = ws.tile_off[t0 + t];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        int r = 4 * grp + i;
                        if (r < cnt) part[(int64_t)ws.perm[off + r] * N + n] = acc[t][i];
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Direct-load kernel for d_in % 32 == 0 (and 4-byte aligned sign planes).
//
// A workgroup owns 32 base rows (two MFMA n-tiles) over all of K, so no
// partial sums are needed.  Its 8 waves split the work of a pass as
// (n-tile, group of 4 segments): each wave rebuilds its 16 rows once per
// variant of its 4 segments and runs their 8 m-tiles on
// v_mfma_f32_16x16x32_bf16.  A stage is 32 k; three LDS buffers hold stages
// s (being multiplied), s+1 (arrived) and s+2 (in flight), filled by direct
// global->LDS loads: the x rows of every m-tile of the pass (32 KiB), the 32
// raw base rows (2 KiB) and one 32-bit sign word per row for every pass
// variant (2 KiB).  Each wave issues exactly kDmaPerWave direct loads per
// stage, so "stage s+1 has arrived" is the wait vmcnt <= kDmaPerWave.
//
// The sign planes are the per-variant [d_out, d_in/8] arrays; a stage reads
// 4 bytes of each of the workgroup's rows.  With 32 rows per workgroup the
// 128-byte lines those words come from (32 stages' worth) stay in L2 until
// they are used up, so the planes are read from HBM about once.
constexpr int kGStage = 32;
constexpr int kGBufs = 3;
constexpr int kGChunks = kGStage / 8;      // 16-byte chunks per row per stage
constexpr int kGRows = 32;                 // base rows per workgroup
constexpr int kXRows = kMaxSegs * 32;      // x rows of a full pass (two m-tiles per segment)
constexpr int kXLoads = kXRows * kGChunks / 64 / kWaves;          // 16-byte loads per wave: 4
constexpr int kDmaPerWave = kXLoads + 1 + 1;                      // + base words + sign words
static_assert(kGRows * kGChunks * 4 == 64 * kWaves, "one 4-byte base load per wave per stage");
static_assert(kMaxSegs * kGRows == 64 * kWaves, "one 4-byte sign load per wave per stage");
static_assert(kDmaPerWave <= 15, "the wait below encodes vmcnt in 4 bits");

// Direct global->LDS loads (16 or 4 bytes per lane): lane l's bytes land at
// LDS byte address lds + l·size (the layout was checked on the device).
// Written as inline asm so that the compiler does not track them: it would
// otherwise wait for every one of them before the next LDS read.  The kernel
// keeps the count itself (see kWaitOlder) and drains them before any code
// that issues ordinary loads.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}

// 16-byte slot of (row, chunk) in a stage buffer: the chunk is XORed with
// bits 2..3 of the row so that the 16 rows of an operand load (64 bytes
// apart) spread over the banks.
__device__ __forceinline__ int gslot(int row, int c) { return row * kGChunks + (c ^ ((row >> 2) & 3)); }

__global__ __launch_bounds__(kWaves * 64) void grouped_dma_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids, const uint16_t* __restrict__ w,
    VariantTable tab, int per_row, int G, int64_t M, int64_t N, int64_t K, WsPtrs ws,
    float* __restrict__ y) {
    __shared__ uint4 xs[kGBufs][kXRows * kGChunks];
    __shared__ uint32_t wt[kGBufs][kGRows * kGChunks * 4];
    __shared__ uint32_t sgw[kGBufs][kMaxSegs * kGRows];
    __shared__ float als[kMaxSegs][kGRows];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const int ntile = wave & 1, sgrp = wave >> 1;  // this wave: n-tile, segments 4·sgrp .. +4
    const int64_t row0 = (int64_t)blockIdx.x * kGRows;
    const int lrow = 16 * ntile + col;           // row within the workgroup for operand reads
    const int64_t n = row0 + lrow;                // this lane's output row
    const int64_t nst = K / kGStage;
    const int64_t kbytes = K / 8;

    const int npass = ws.hdr[1];
    for (int p = 0; p < npass; ++p) {
        const int nseg = ws.pass_nseg[p];
        __syncthreads();  // the previous pass is done with every buffer
        for (int q = tid; q < kMaxSegs * kGRows; q += kWaves * 64) {
            const int j = q / kGRows, r = q % kGRows;
            int64_t rn = row0 + r;
            rn = rn < N ? rn : N - 1;
            float v = 0.0f;
            if (j < nseg) v = tab.alpha[ws.seg_var[p * kMaxSegs + j]][per_row ? rn : 0];
            als[j][r] = v;
        }

        // Direct-load sources of this lane, fixed for the pass (k added per stage).
        // x: load i of this wave fills tile rows (wave*kXLoads + i)*16 .. +16;
        // tile row 32j + r is token r of segment j; rows without a token read
        // token 0 (their outputs are dropped).
        const uint16_t* xsrc[kXLoads];
#pragma unroll
        for (int i = 0; i < kXLoads; ++i) {
            const int row = (wave * kXLoads + i) * 16 + lane / kGChunks;
            const int c = (lane % kGChunks) ^ ((row >> 2) & 3);
            const int j = row >> 5, r = row & 31;
            int tok = 0;
            if (j < nseg && r < ws.seg_cnt[p * kMaxSegs + j]) tok = ws.perm[ws.seg_off[p * kMaxSegs + j] + r];
            xsrc[i] = x + (int64_t)tok * K + 8 * c;
        }
        // base rows: word slot wave*64 + lane of the stage's 32 rows x 16
        // words, laid out as 16-byte slots gslot(row, chunk)
        const char* wsrc;
        {
            const int slot = wave * 64 + lane;
            const int row = slot / (kGChunks * 4), q = slot % (kGChunks * 4);
            const int c = (q / 4) ^ ((row >> 2) & 3), e = q % 4;
            int64_t rn = row0 + row;
            rn = rn < N ? rn : N - 1;
            wsrc = reinterpret_cast<const char*>(w + rn * K + 8 * c) + 4 * e;
        }
        // sign words: slot wave*64 + lane = (segment j, row r); segments past
        // nseg repeat segment 0 (never stored)
        const uint8_t* ssrc;
        {
            const int slot = wave * 64 + lane, j = slot / kGRows, r = slot % kGRows;
            int64_t rn = row0 + r;
            rn = rn < N ? rn : N - 1;
            const int var = ws.seg_var[p * kMaxSegs + (j < nseg ? j : 0)];
            ssrc = tab.signs[var] + rn * kbytes;
        }
        auto issue = [&](int64_t st, int b) {
            int64_t k0 = st * kGStage;
            k0 = k0 + kGStage <= K ? k0 : K - kGStage;  // stages past the end: in bounds, unused
#pragma unroll
            for (int i = 0; i < kXLoads; ++i) dma16(xsrc[i] + k0, lds_addr(&xs[b][(wave * kXLoads + i) * 64]));
            dma4(wsrc + 2 * k0, lds_addr(&wt[b][wave * 64]));
            dma4(ssrc + k0 / 8, lds_addr(&sgw[b][wave * 64]));
        };
        // vmcnt <= kDmaPerWave: everything but the latest stage's loads is done
        constexpr int kWaitOlder = (kDmaPerWave & 15) | (0x7 << 4) | (0xF << 8);
        // Wait until this wave's loads of the next stage have landed in LDS,
        // then meet the other waves.  The wavefront-scope fences only keep
        // the compiler from moving LDS accesses across the barrier.
        auto stage_barrier = [&]() {
            __builtin_amdgcn_s_waitcnt(kWaitOlder);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        };

        f32x4_t acc[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        issue(0, 0);
        issue(1, 1);
        stage_barrier();  // also publishes als
        float al[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) al[jj] = als[4 * sgrp + jj][lrow];
        for (int64_t st = 0; st < nst; ++st) {
            const int b = (int)(st % kGBufs);
            const uint4* wtb = reinterpret_cast<const uint4*>(wt[b]);
            const uint4 wf = wtb[gslot(lrow, grp)];
            uint32_t sw[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) sw[jj] = sgw[b][(4 * sgrp + jj) * kGRows + lrow];
            // all 4 segments run (one basic block); those past nseg work on
            // valid data and are never stored
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int j = 4 * sgrp + jj;
                const bf16x8_t bf = as_bf16x8(recon8(wf, (sw[jj] >> (8 * grp)) & 0xffu, al[jj]));
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const bf16x8_t xa = as_bf16x8(xs[b][gslot(32 * j + 16 * u + col, grp)]);
                    acc[2 * jj + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bf, acc[2 * jj + u], 0, 0, 0);
                }
            }
            issue(st + 2, (int)((st + 2) % kGBufs));
            stage_barrier();
        }
        __builtin_amdgcn_s_waitcnt(0);  // the last (unused) stages' loads

        // D layout of the 16x16 MFMA: lane holds rows 4·(lane/16) + i, column lane%16.
        if (n < N) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int j = 4 * sgrp + jj;
                if (j < nseg) {
                    const int cnt = ws.seg_cnt[p * kMaxSegs + j], off = ws.seg_off[p * kMaxSegs + j];
#pragma unroll
                    for (int u = 0; u < 2; ++u)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int r = 16 * u + 4 * grp + i;
                            if (r < cnt) y[(int64_t)ws.perm[off + r] * N + n] = acc[2 * jj + u][i];
                        }
                }
            }
        }
    }
    // Tokens whose variant id is out of range belong to no segment: NaN rows.
    for (int64_t m = tid; m < M; m += kWaves * 64) {
        const int g = ids[m];
        if (g < 0 || g >= G) {
            for (int r = 0; r < kGRows; ++r)
                if (row0 + r < N) y[m * N + row0 + r] = __builtin_nanf("");
        }
    }
}

__global__ __launch_bounds__(256) void reduce_kernel(const float* __restrict__ part,
                                                     const int32_t* __restrict__ ids, int G,
                                                     int64_t M, int64_t N, int ksplit,
                                                     float* __restrict__ y) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= M * N) return;
    const int64_t m = i / N;
    const int g = ids[m];
    float s;
    if (g < 0 || g >= G) {
        s = __builtin_nanf("");
    } else {
        s = part[i];
        for (int p = 1; p < ksplit; ++p) s += part[(int64_t)p * M * N + i];
    }
    y[i] = s;
}

}  // namespace

size_t grouped_workspace_bytes(int64_t M, int32_t G, int64_t N) { return make_layout(M, G, N).total; }

hipError_t launch_grouped(const uint16_t* x, const int32_t* ids, const uint16_t* w,
                          const VariantTable& table, bool per_row, int32_t G, float* y,
                          int64_t M, int64_t N, int64_t K, void* workspace, hipStream_t stream) {
    Layout L = make_layout(M, G, N);
    char* base = static_cast<char*>(workspace);
    WsPtrs ws;
    ws.hdr = reinterpret_cast<int32_t*>(base + L.hdr);
    ws.tile_var = reinterpret_cast<int32_t*>(base + L.tile_var);
    ws.tile_off = reinterpret_cast<int32_t*>(base + L.tile_off);
    ws.tile_cnt = reinterpret_cast<int32_t*>(base + L.tile_cnt);
    ws.tile_seg = reinterpret_cast<int32_t*>(base + L.tile_seg);
    ws.pass_first = reinterpret_cast<int32_t*>(base + L.pass_first);
    ws.pass_nseg = reinterpret_cast<int32_t*>(base + L.pass_nseg);
    ws.seg_var = reinterpret_cast<int32_t*>(base + L.seg_var);
    ws.seg_off = reinterpret_cast<int32_t*>(base + L.seg_off);
    ws.seg_cnt = reinterpret_cast<int32_t*>(base + L.seg_cnt);
    ws.perm = reinterpret_cast<int32_t*>(base + L.perm);
    ws.part = reinterpret_cast<float*>(base + L.part);

    hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(kBucketThreads), 0, stream, ids, M, (int)G, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    // The direct-load kernel reads sign words (4 bytes): every sign plane must
    // be 4-byte aligned and rows whole words (d_in % 32 == 0).
    bool words = K % kGStage == 0;
    for (int g = 0; g < G && words; ++g) words = (reinterpret_cast<uintptr_t>(table.signs[g]) & 3) == 0;
    if (words) {
        const int64_t blocks = (N + kGRows - 1) / kGRows;
        hipLaunchKernelGGL(grouped_dma_kernel, dim3((unsigned)blocks), dim3(kWaves * 64), 0, stream, x,
                           ids, w, table, per_row ? 1 : 0, (int)G, M, N, K, ws, y);
        return hipGetLastError();
    }
    const int ksplit = choose_ksplit(N);
    const int64_t rowblocks = (N + kRowsPerBlock - 1) / kRowsPerBlock;
    int64_t kchunk = (K + ksplit - 1) / ksplit;
    kchunk = (kchunk + kStage - 1) / kStage * kStage;
    hipLaunchKernelGGL(grouped_kernel, dim3((unsigned)(rowblocks * ksplit)), dim3(kWaves * 64), 0,
                       stream, x, w, table, per_row ? 1 : 0, M, N, K, ksplit, kchunk, ws);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    const int64_t total = M * N;
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       ws.part, ids, (int)G, M, N, ksplit, y);
    return hipGetLastError();
}

}  // namespace bd
