// Grouped multi-variant linear: one shared bf16 base, up to 64 packed deltas,
// each token with its own variant.
//
// "BitDelta : servir 14 modèles Zen depuis un seul cluster GPU" (hanzo-blog,
// 2026-02-28), "Serving architecture": the base weights are HBM resident and
// read by every variant, the delta cache holds one
// (α, sign(Δ)) entry per variant, and the router sends each request to its
// variant's entry.  Here one launch serves a batch that mixes variants:
// y[m] = x[m]·W_eff(ids[m])ᵀ.
//
// Kernels:
//  1. bucket: counts tokens per variant, orders them by variant (stable) and
//     cuts each variant's tokens into segments of <= 32, grouped into passes
//     of <= kMaxSegs segments (and m-tiles of <= 16 for the fallback).
//  2. grouped_stage_kernel (d_in % 64 == 0): a workgroup owns 32 base rows
//     over all of K; per 64-wide k stage it reads the base rows once, rebuilds
//     them for each segment's variant (one widening of the base, then ±α per
//     sign set) and multiplies each segment's 32 tokens on
//     v_mfma_f32_32x32x16_bf16.  The base is read from HBM once per pass,
//     however many variants there are; the rebuild is paid once per
//     (variant, weight).  Writes y directly.
//  3. fallback for other d_in: grouped_kernel (128 rows and a K range per
//     workgroup, m-tiles of 16 on v_mfma_f32_16x16x32_bf16) writes fp32
//     partials, and reduce_kernel adds them in a fixed order.
// Tokens whose id is out of range get NaN rows.
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

// K ranges of the staged kernel: blocks of 32 rows times ks ranges of K of
// `per` stages each (per even, every range at least one stage).  ks is the
// one of 1, 2, 4, 8 (ranges of at least 8 stages) with the least modelled
// time, rounds of 256 workgroups x (stages per workgroup + 2 for the
// prologue); ties go to fewer ranges.  Few rows (k/v: 32 blocks) take 8
// ranges; 896 blocks (gate/up) take 2, which turns 3.5 rounds into 7 full
// ones.
void stage_split(int64_t N, int64_t K, int* per_out, int* ks_out) {
    const int64_t blocks = (N + 31) / 32;
    const int nst = (int)(K / 64);
    if (nst < 1) {
        *per_out = 2;
        *ks_out = 1;
        return;
    }
    int best_ks = 1, best_per = nst + (nst & 1);
    int64_t best_t = -1;
    for (int ks = 1; ks <= 8; ks *= 2) {
        if (ks > 1 && nst / ks < 8) break;
        int per = (nst + ks - 1) / ks;
        per += per & 1;
        const int kse = (nst + per - 1) / per;
        const int64_t t = (blocks * kse + 255) / 256 * (per + 2);
        if (best_t < 0 || t < best_t) {
            best_t = t;
            best_ks = kse;
            best_per = per;
        }
    }
    *per_out = best_per;
    *ks_out = best_ks;
}

// Segments: (variant, up to 32 consecutive tokens of it in variant order),
// each covering two m-tiles of 16 (the second possibly short or empty); a
// pass holds up to kMaxSegs segments.  Every variant with n tokens gives
// ceil(n/32) segments, so there are at most G + M/32 of them.
Layout make_layout(int64_t M, int32_t G, int64_t N, int64_t K) {
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
    // fp32 partials of the K ranges: the fallback's split or the staged
    // kernel's, whichever is larger
    int per, kss;
    stage_split(N, K, &per, &kss);
    int nparts = choose_ksplit(N) > kss ? choose_ksplit(N) : kss;
    // the decode path's K ranges (up to kGdecMaxM tokens)
    const GdecPlan gp = gdec_plan(M, N, K);
    if (gp.grid > 0 && gp.nkr > nparts) nparts = gp.nkr;
    L.part = o; o = align256(o + (size_t)nparts * M * N * sizeof(float));
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
    __shared__ int wc[kBucketThreads / 64][kMaxVariants];  // per wave: count, then first slot
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
    // Stable placement: token order is kept within each variant.  Per block
    // of 1024 tokens, each wave ranks its tokens among the same-variant
    // tokens before them in the wave (one ballot per distinct variant in the
    // wave) and counts them per variant; the waves' counts, added up in wave
    // order onto the variant's cursor, place each wave's tokens after the
    // earlier waves'.
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int64_t base = 0; base < M; base += kBucketThreads) {
        for (int q = tid; q < kBucketThreads / 64 * kMaxVariants; q += kBucketThreads) (&wc[0][0])[q] = 0;
        __syncthreads();
        const int64_t m = base + tid;
        const int g = m < M ? ids[m] : -1;
        const bool valid = g >= 0 && g < G;
        int rank = 0;
        uint64_t todo = __ballot(valid);
        while (todo) {
            const int lead = __ffsll((unsigned long long)todo) - 1;
            const int gl = __shfl(g, lead, 64);
            const uint64_t mine = __ballot(g == gl);
            if (g == gl) rank = __popcll(mine & below);
            if (lane == 0) wc[wave][gl] = __popcll(mine);
            todo &= ~mine;
        }
        __syncthreads();
        if (tid < G) {
            int run = cursor[tid];
            for (int w = 0; w < kBucketThreads / 64; ++w) {
                const int c = wc[w][tid];
                wc[w][tid] = run;
                run += c;
            }
            cursor[tid] = run;
        }
        __syncthreads();
        if (valid) ws.perm[wc[wave][g] + rank] = (int32_t)m;
        __syncthreads();
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
        // what the plan was made for: consumers given other sizes run no
        // passes (wrong rows, but no access outside the arguments)
        ws.hdr[2] = (int32_t)M;
        ws.hdr[3] = G;
    }
}

// Passes of the plan in the workspace, or 0 if it was made for another M or G.
__device__ __forceinline__ int plan_passes(const WsPtrs& ws, int64_t M, int G) {
    return ws.hdr[2] == (int32_t)M && ws.hdr[3] == G ? ws.hdr[1] : 0;
}

__device__ __forceinline__ int xswz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

__global__ __launch_bounds__(kWaves * 64) void grouped_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, VariantTable tab,
    int per_row, int G, int64_t M, int64_t N, int64_t K, int ksplit, int64_t kchunk, WsPtrs ws) {
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

    const int npass = plan_passes(ws, M, G);
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
// Main kernel, for d_in % 64 == 0 (x and the base under 4 GiB each).
//
// A workgroup owns 32 base rows over all of K (or, on projections with too
// few rows to fill the GPU, over one of ks ranges of K, writing fp32
// partials that reduce_kernel adds in range order).  Wave w of its 8 takes
// segments w and w+8 of a pass, so a pass with fewer than 16 segments (a
// decode batch: one or two tokens per variant) spreads them over all four
// SIMDs, and a wave skips the rebuild and MFMAs of a segment the pass does
// not have.  A stage is 64 k.  The base rows are widened to fp32 on their
// way into LDS (4 weights per lane, once for all segments of all waves);
// a wave rebuilds its row's weights with the sign bits and α of each of its
// segments (recon8_word) and runs each segment's 32 tokens on
// v_mfma_f32_32x32x16_bf16, so every x fragment read from LDS serves 32
// rows.
//
// Staging: the stage's x rows of the pass's tokens (in variant order, so
// segment j's 32 operand rows start at its first token; rows past a
// segment's count belong to the next segment or are stale, and only reach
// outputs that are dropped) and the 32 base rows (4 KiB) are loaded into
// registers two stages ahead and written to one of two LDS buffers one stage
// ahead.  kXL x loads per lane cover kXL·64 token rows, chosen by the host
// from M.  The sign bytes skip LDS: each lane loads its own row's bytes of
// its wave's two segments, 16 bytes (two stages) per load, two stage pairs
// ahead.  Every load and store is unconditional (x rows past the pass's
// tokens and sign bytes past a plane's end read past the buffer's end, which
// returns zeros), so the loop is one basic block and the compiler's load
// counters stay exact.
//
// What bounds it: every CU reads its own copy of the x rows (from L2) and
// 8 bytes of each (segment, row) sign line per stage, and a CU keeps only so
// many L2 requests in flight; requests, more than bytes, set the pace.  So x
// and the base go through registers in whole 128-byte rows per stage (the
// direct global->LDS path moves about 16 bytes per clock per CU on gfx950),
// and each sign line is requested once per two stages.  One barrier per
// stage.
constexpr int kGStage = 64;
constexpr int kGChunks = kGStage / 8;                        // 16-byte chunks per row per stage
constexpr int kGRows = 32;                                   // base rows per workgroup
constexpr int kXRows = kMaxSegs * 32;                        // token rows of a full pass
constexpr int kXTileRows = kXRows + 32;                      // + the last segment's overhang
constexpr int kXRowsPerLoad = 64 * kWaves / kGChunks;        // token rows per x load slot: 64
static_assert(kGRows * kGStage * 2 == 64 * kWaves * 8, "one 8-byte base load per lane per stage");
static_assert(kMaxSegs * kGRows == 64 * kWaves, "one 8-byte sign load per lane per stage");
static_assert(kMaxSegs == 2 * kWaves, "two segments per wave");

// 16-byte slot of (row, chunk) in a stage buffer: the chunk is XORed with
// bits 1..3 of the row, so the 16 consecutive rows of one operand read phase
// (128 bytes apart, same chunk) fall on 16 different 16-byte bank groups.
__device__ __forceinline__ int gslot(int row, int c) { return row * kGChunks + (c ^ ((row >> 1) & 7)); }

template <int kXL>
struct StageRegs {
    uint4 x[kXL];
    uint2 w;
};

template <int kXL>
__global__ __launch_bounds__(kWaves * 64) void grouped_stage_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids, const uint16_t* __restrict__ w,
    VariantTable tab, int per_row, int G, int64_t M, int64_t N, int64_t K, WsPtrs ws,
    float* __restrict__ y, int ks, int per) {
    static_assert(kXL * kXRowsPerLoad <= kXRows, "at most a full pass of token rows");
    __shared__ uint4 xs[2][kXTileRows * kGChunks];  // 2 x 68 KiB
    // The base rows of a stage, already widened to fp32 by the waves that
    // stage them: 16-byte unit q (4 weights) of row r at r·16 + (q ^ (r % 16)).
    __shared__ float4 wtf[2][kGRows * 16];     // 2 x 8 KiB
    __shared__ float als[kMaxSegs][kGRows];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // 32x32x16 operands: lane holds row lane%32 (token row of A, base row of
    // B) and k 8·(lane/32) .. +8 of each 16-k quarter of the stage
    const int lrow = lane & 31, half = lane >> 5;
    // workgroup b: row block b % blocks, K range b / blocks (stages
    // [kp·per, kp·per + nst), per even, nst >= 1)
    const int64_t blocks = (N + kGRows - 1) / kGRows;
    const int kp = (int)(blockIdx.x / blocks);
    const int64_t row0 = (int64_t)(blockIdx.x % blocks) * kGRows;
    const int64_t n = row0 + lrow;  // this lane's output row
    const int nst_all = (int)(K / kGStage);
    const int sbeg = kp * per;
    const int nst = nst_all - sbeg < per ? nst_all - sbeg : per;
    float* __restrict__ dst = ks > 1 ? ws.part + (int64_t)kp * M * N : y;
    const int64_t kbytes = K / 8;
    const rsrc_t xrs = make_rsrc(x, (uint32_t)(M * K * 2));
    const rsrc_t wrs = make_rsrc(w, (uint32_t)(N * K * 2));

    // Base rows: 8-byte piece q (of 16 per row per stage) of row wrow.
    const int wslot = wave * 64 + lane, wrow = wslot / 16, wq = wslot % 16;
    int64_t wrn = row0 + wrow;
    wrn = wrn < N ? wrn : N - 1;  // rows past the end: computed, never stored
    const uint32_t woff = (uint32_t)(wrn * K * 2) + 8 * wq;
    const int wpos = wrow * 16 + (wq ^ (wrow & 15));      // its widened unit
    // Sign bytes: each lane reads its own row's bytes of its wave's two
    // segments, 16 bytes (two stages) per load.
    const uint32_t soff = (uint32_t)((n < N ? n : N - 1) * kbytes);
    const SignShifts sh[2] = {sign_shifts(half), sign_shifts(half + 2)};

    const int npass = plan_passes(ws, M, G);
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

        // x: load i of this lane fills tile row (i*kWaves + wave)*8 + lane/8,
        // chunk lane%8: the pass's token q = that row, in variant order.
        const int tok0 = ws.seg_off[p * kMaxSegs];
        const int ntok = ws.seg_off[p * kMaxSegs + nseg - 1] + ws.seg_cnt[p * kMaxSegs + nseg - 1] - tok0;
        uint32_t xoff[kXL];
        int xpos[kXL];
#pragma unroll
        for (int i = 0; i < kXL; ++i) {
            const int row = (i * kWaves + wave) * 8 + lane / 8, c = lane % 8;
            xoff[i] = row < ntok ? (uint32_t)((int64_t)ws.perm[tok0 + row] * K * 2) + 16 * c
                                 : (uint32_t)(M * K * 2);  // past the end: reads zeros
            xpos[i] = gslot(row, c);
        }
        // the wave's segments: wave and wave + kWaves; how many the pass has
        const int nmine = (wave < nseg) + (wave + kWaves < nseg);
        int segrow[2];  // first tile row of each of the wave's segments
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int j = wave + kWaves * jj;
            segrow[jj] = j < nseg ? ws.seg_off[p * kMaxSegs + j] - tok0 : 0;
        }
        // segments past nseg read segment 0's plane (never used)
        rsrc_t srs[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int j = wave + kWaves * jj;
            srs[jj] = make_rsrc(tab.signs[ws.seg_var[p * kMaxSegs + (j < nseg ? j : 0)]], (uint32_t)(N * kbytes));
        }

        auto load = [&](StageRegs<kXL>& R, int st) {
            st = sbeg + (st < nst ? st : nst - 1);  // stages past the end: in bounds, unused
            const uint32_t kb = (uint32_t)st * (kGStage * 2);
#pragma unroll
            for (int i = 0; i < kXL; ++i) R.x[i] = buf_load16(xrs, xoff[i], kb);
            R.w = buf_load8(wrs, woff, kb);
        };
        // sign bytes of stages st0 and st0+1 (st0 even); past the plane's end
        // the buffer returns zeros (those stages are never multiplied)
        // (NS: the wave's segments; only theirs are loaded)
        auto load_signs = [&](auto ns_tag, uint4 (&S)[2], int st0) {
#pragma unroll
            for (int jj = 0; jj < decltype(ns_tag)::value; ++jj)
                S[jj] = buf_load16(srs[jj], soff, (uint32_t)(sbeg + st0) * 8);
        };
        auto store = [&](const StageRegs<kXL>& R, int b) {
#pragma unroll
            for (int i = 0; i < kXL; ++i) xs[b][xpos[i]] = R.x[i];
            wtf[b][wpos] = make_float4(__uint_as_float(R.w.x << 16), __uint_as_float(R.w.x & 0xffff0000u),
                                       __uint_as_float(R.w.y << 16), __uint_as_float(R.w.y & 0xffff0000u));
        };

        f32x16_t acc[2];
        uint32_t nal[2];  // -α of this lane's row for each of the wave's segments

        // S: the sign bytes of the stage pair; odd: which stage of the pair;
        // NS: the wave's segments in this pass (1 or 2)
        auto compute = [&](auto ns_tag, int b, const uint4 (&S)[2], bool odd) {
            constexpr int NS = decltype(ns_tag)::value;
            uint64_t sp[2][2];  // [segment][low or high sign word of the stage]
#pragma unroll
            for (int jj = 0; jj < NS; ++jj) {
                sp[jj][0] = sign_spread(odd ? S[jj].z : S[jj].x);
                sp[jj][1] = sign_spread(odd ? S[jj].w : S[jj].y);
            }
            // With registers to spare (kXL <= 4), all of the stage's LDS
            // operands are read up front (the base rows of the 4 quarters,
            // the x fragments of both segments; the scheduling barrier keeps
            // the compiler from sinking the reads to their uses), so the LDS
            // latency is paid once per stage rather than before every rebuild
            // and MFMA.
            // The 8 widened base weights of chunk c of this lane's row (units
            // 2c and 2c + 1 of the row).
            auto base8 = [&](int c) {
                const float4 f0 = wtf[b][lrow * 16 + ((2 * c) ^ (lrow & 15))];
                const float4 f1 = wtf[b][lrow * 16 + ((2 * c + 1) ^ (lrow & 15))];
                Widened8 wb;
                wb.lo[0] = f0.x; wb.hi[0] = f0.y; wb.lo[1] = f0.z; wb.hi[1] = f0.w;
                wb.lo[2] = f1.x; wb.hi[2] = f1.y; wb.lo[3] = f1.z; wb.hi[3] = f1.w;
                return wb;
            };
            constexpr bool kEarly = kXL <= 4;
            Widened8 wq[4];
            uint4 xq[4][2];
            if constexpr (kEarly) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int c = half + 2 * u;  // this lane's chunk in quarter u
                    wq[u] = base8(c);
#pragma unroll
                    for (int jj = 0; jj < NS; ++jj) xq[u][jj] = xs[b][gslot(segrow[jj] + lrow, c)];
                }
                __builtin_amdgcn_sched_barrier(0);
                // Rebuild one quarter ahead of the multiply: the MFMAs of
                // quarter u go in after the rebuild of quarter u+1, so an
                // MFMA's operand has long been written when it issues and the
                // VALU work that follows it is independent of it.
                bf16x8_t bq[4][2];
                auto rebuild = [&](int u) {
#pragma unroll
                    for (int jj = 0; jj < NS; ++jj)
                        bq[u][jj] = as_bf16x8(recon8_word(wq[u], sp[jj][u >> 1], sh[u & 1], nal[jj]));
                };
                auto multiply = [&](int u) {
#pragma unroll
                    for (int jj = 0; jj < NS; ++jj)
                        acc[jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(xq[u][jj]), bq[u][jj], acc[jj],
                                                                          0, 0, 0);
                };
                rebuild(0);
                rebuild(1);
                multiply(0);
                rebuild(2);
                multiply(1);
                rebuild(3);
                multiply(2);
                multiply(3);
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int c = half + 2 * u;
                    const Widened8 wb = base8(c);
#pragma unroll
                    for (int jj = 0; jj < NS; ++jj) {
                        const bf16x8_t bf = as_bf16x8(recon8_word(wb, sp[jj][u >> 1], sh[u & 1], nal[jj]));
                        const uint4 xa = xs[b][gslot(segrow[jj] + lrow, c)];
                        acc[jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(xa), bf, acc[jj], 0, 0, 0);
                    }
                }
            }
        };

        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        // The pass's pipeline for a wave with NS segments, compiled once per
        // NS, so that each version has its own registers and a wave without
        // segments only loads, stores and meets the barriers (every version
        // has the same barriers).
        // Registers: R[1 - b] holds stage s+1 when stage s (buffer b) starts,
        // R[b] stage s+2.  SG[q] holds the sign bytes of stages 4i + 2q and
        // 4i + 2q + 1 during loop iteration i, and is reloaded (two pairs
        // ahead) right after its second stage is multiplied.
        // The scheduling barriers keep the prologue's loads in the order the
        // loop has them at its head, so the compiler's wait counts stay exact.
        auto run = [&](auto ns_tag) {
            constexpr int NS = decltype(ns_tag)::value;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;
            StageRegs<kXL> R[2];
            uint4 SG[2][2];
            load(R[0], 0);
            load_signs(ns_tag, SG[0], 0);
            __builtin_amdgcn_sched_barrier(0);
            load(R[1], 1);
            __builtin_amdgcn_sched_barrier(0);
            store(R[0], 0);
            load(R[0], 2);
            load_signs(ns_tag, SG[1], 2);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();  // buffer 0 and als
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) nal[jj] = __float_as_uint(-als[wave + kWaves * jj][lrow]);

            // stage s in buffer b = s % 2, signs from SG[q], q = (s / 2) % 2
            auto step = [&](auto B, auto Q, int s) {
                constexpr int b = decltype(B)::value, q = decltype(Q)::value;
                store(R[1 - b], 1 - b);   // stage s+1 -> the other buffer (read at s-1, before the last barrier)
                load(R[1 - b], s + 3);
                if constexpr (NS > 0) compute(ns_tag, b, SG[q], b == 1);
                if (b == 1) load_signs(ns_tag, SG[q], s + 3);  // stages s+3, s+4
                __syncthreads();
            };
            int s = 0;
            for (; s + 3 < nst; s += 4) {
                step(I0{}, I0{}, s);
                step(I1{}, I0{}, s + 1);
                step(I0{}, I1{}, s + 2);
                step(I1{}, I1{}, s + 3);
            }
            if (s < nst) step(I0{}, I0{}, s);
            if (s + 1 < nst) step(I1{}, I0{}, s + 1);
            if (s + 2 < nst) step(I0{}, I1{}, s + 2);
        };
        if (nmine == 2) run(I2{});
        else if (nmine == 1) run(I1{});
        else run(I0{});

        // D layout of the 32x32 MFMA: lane holds column lane%32 (the base row)
        // and token rows 8·(e/4) + 4·(lane/32) + e%4, e = 0..15.
        if (n < N) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int j = wave + kWaves * jj;
                if (j < nseg) {
                    const int cnt = ws.seg_cnt[p * kMaxSegs + j], off = ws.seg_off[p * kMaxSegs + j];
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int r = 8 * (e / 4) + 4 * half + e % 4;
                        if (r < cnt) dst[(int64_t)ws.perm[off + r] * N + n] = acc[jj][e];
                    }
                }
            }
        }
    }
    // Tokens whose variant id is out of range belong to no segment: NaN rows
    // (with K ranges, reduce_kernel writes them).
    if (ks > 1) return;
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
        // ranges added in order, 8 loaded at a time (all in flight together)
        // so their latency is paid once per 8; a range index past the last
        // repeats the last range, and that copy is added as -0 (x + -0 = x
        // for every x, signed zeros included)
        const int64_t MN = M * N;
        s = 0.0f;
        for (int p0 = 0; p0 < ksplit; p0 += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(p0 + u < ksplit ? p0 + u : ksplit - 1) * MN + i];
            __builtin_amdgcn_sched_barrier(0);  // the batch's loads are all issued before the adds
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float t = p0 + u < ksplit ? v[u] : __uint_as_float(0x80000000u);
                s = (u == 0 && p0 == 0) ? t : s + t;
            }
        }
    }
    y[i] = s;
}

}  // namespace

size_t grouped_workspace_bytes(int64_t M, int32_t G, int64_t N, int64_t K) { return make_layout(M, G, N, K).total; }

namespace {
WsPtrs ws_ptrs(const Layout& L, void* workspace) {
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
    return ws;
}
}  // namespace

// The bucketing's part of the workspace is its prefix and depends on M and G
// only, so one plan serves grouped calls of any shape over the same ids.
size_t grouped_plan_bytes(int64_t M, int32_t G) { return make_layout(M, G, 1, 64).part; }

hipError_t launch_grouped_plan(const int32_t* ids, int64_t M, int32_t G, void* workspace, hipStream_t stream) {
    const WsPtrs ws = ws_ptrs(make_layout(M, G, 1, 64), workspace);
    hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(kBucketThreads), 0, stream, ids, M, (int)G, ws);
    return hipGetLastError();
}

hipError_t launch_grouped(const uint16_t* x, const int32_t* ids, const uint16_t* w,
                          const VariantTable& table, bool per_row, int32_t G, float* y,
                          int64_t M, int64_t N, int64_t K, void* workspace, bool planned,
                          hipStream_t stream) {
    const Layout L = make_layout(M, G, N, K);
    const WsPtrs ws = ws_ptrs(L, workspace);
    hipError_t e = hipSuccess;
    // Up to kGdecMaxM tokens: the decode path (rows streamed once, no
    // bucketing; a plan, if given, is not read).
    const GdecPlan gp = gdec_plan(M, N, K);
    if (gp.grid > 0) {
        e = launch_gdec(x, ids, w, table, per_row, G, y, M, N, K, ws.part, stream);
        if (e != hipSuccess || gp.nkr == 1) return e;
        const int64_t total = M * N;
        hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                           ws.part, ids, (int)G, M, N, gp.nkr, y);
        return hipGetLastError();
    }
    if (!planned) {
        hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(kBucketThreads), 0, stream, ids, M, (int)G, ws);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }

    // The staged kernel reads 8 sign bytes per row per stage and addresses x
    // and the base with 32-bit buffer offsets: every sign plane 8-byte
    // aligned, d_in % 64 == 0, and x and the base under 4 GiB.
    constexpr int64_t kMaxBufBytes = 0xffffffffLL;
    bool staged = K % kGStage == 0 && (M + 1) * K * 2 <= kMaxBufBytes && N * K * 2 <= kMaxBufBytes;
    for (int g = 0; g < G && staged; ++g) staged = (reinterpret_cast<uintptr_t>(table.signs[g]) & 7) == 0;
    if (staged) {
        const int64_t blocks = (N + kGRows - 1) / kGRows;
        // x load slots: enough for the most tokens a pass can hold
        const int64_t rows = M < kXRows ? M : kXRows;
        const int64_t need = (rows + kXRowsPerLoad - 1) / kXRowsPerLoad;
        int per, ks;
        stage_split(N, K, &per, &ks);
        auto launch = [&](auto kernel) {
            hipLaunchKernelGGL(kernel, dim3((unsigned)(blocks * ks)), dim3(kWaves * 64), 0, stream, x, ids, w,
                               table, per_row ? 1 : 0, (int)G, M, N, K, ws, y, ks, per);
        };
        if (need <= 1) launch(grouped_stage_kernel<1>);
        else if (need <= 2) launch(grouped_stage_kernel<2>);
        else if (need <= 4) launch(grouped_stage_kernel<4>);
        else launch(grouped_stage_kernel<8>);
        e = hipGetLastError();
        if (e != hipSuccess || ks == 1) return e;
        const int64_t total = M * N;
        hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                           ws.part, ids, (int)G, M, N, ks, y);
        return hipGetLastError();
    }
    const int ksplit = choose_ksplit(N);
    const int64_t rowblocks = (N + kRowsPerBlock - 1) / kRowsPerBlock;
    int64_t kchunk = (K + ksplit - 1) / ksplit;
    kchunk = (kchunk + kStage - 1) / kStage * kStage;
    hipLaunchKernelGGL(grouped_kernel, dim3((unsigned)(rowblocks * ksplit)), dim3(kWaves * 64), 0,
                       stream, x, w, table, per_row ? 1 : 0, (int)G, M, N, K, ksplit, kchunk, ws);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    const int64_t total = M * N;
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       ws.part, ids, (int)G, M, N, ksplit, y);
    return hipGetLastError();
}

}  // namespace bd
