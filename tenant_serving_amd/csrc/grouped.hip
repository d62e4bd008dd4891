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
    int64_t max_tiles, max_passes;
    size_t hdr, tile_var, tile_off, tile_cnt, tile_seg, pass_first, pass_nseg, seg_var, perm,
        part, total;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int choose_ksplit(int64_t N) {
    int64_t rowblocks = (N + kRowsPerBlock - 1) / kRowsPerBlock;
    int ks = 1;
    while (ks < 8 && rowblocks * ks < 256) ks *= 2;
    return ks;
}

Layout make_layout(int64_t M, int32_t G, int64_t N) {
    Layout L;
    L.max_tiles = (int64_t)G + (M + 15) / 16;
    L.max_passes = L.max_tiles;
    size_t o = 0;
    L.hdr = o; o = align256(o + 4 * sizeof(int32_t));
    L.tile_var = o; o = align256(o + L.max_tiles * sizeof(int32_t));
    L.tile_off = o; o = align256(o + L.max_tiles * sizeof(int32_t));
    L.tile_cnt = o; o = align256(o + L.max_tiles * sizeof(int32_t));
    L.tile_seg = o; o = align256(o + L.max_tiles * sizeof(int32_t));
    L.pass_first = o; o = align256(o + (L.max_passes + 1) * sizeof(int32_t));
    L.pass_nseg = o; o = align256(o + L.max_passes * sizeof(int32_t));
    L.seg_var = o; o = align256(o + L.max_passes * kMaxSegs * sizeof(int32_t));
    L.perm = o; o = align256(o + (size_t)M * sizeof(int32_t));
    L.part = o; o = align256(o + (size_t)choose_ksplit(N) * M * N * sizeof(float));
    L.total = o;
    return L;
}

struct WsPtrs {
    int32_t *hdr, *tile_var, *tile_off, *tile_cnt, *tile_seg, *pass_first, *pass_nseg, *seg_var,
        *perm;
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
        int t = 0, p = 0, nseg = 0, in_pass = 0, last_g = -1;
        ws.pass_first[0] = 0;
        for (int g = 0; g < G; ++g) {
            for (int r = 0; r < count[g]; r += 16) {
                bool new_seg = (g != last_g);
                if (in_pass == kMaxTiles || (new_seg && nseg == kMaxSegs)) {
                    ws.pass_nseg[p] = nseg;
                    ++p;
                    ws.pass_first[p] = t;
                    in_pass = 0;
                    nseg = 0;
                    new_seg = true;
                }
                if (new_seg) {
                    ws.seg_var[p * kMaxSegs + nseg] = g;
                    ++nseg;
                    last_g = g;
                }
                ws.tile_var[t] = g;
                ws.tile_off[t] = offset[g] + r;
                ws.tile_cnt[t] = min(16, count[g] - r);
                ws.tile_seg[t] = nseg - 1;
                ++t;
                ++in_pass;
            }
        }
        if (in_pass > 0) {
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
                    uint32_t lo = va ? load_stream_u8(srow + (ka >> 3)) : 0u;
                    uint32_t hi = vb ? load_stream_u8(srow + (kb >> 3)) : 0u;
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
    ws.perm = reinterpret_cast<int32_t*>(base + L.perm);
    ws.part = reinterpret_cast<float*>(base + L.part);

    hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(kBucketThreads), 0, stream, ids, M, (int)G, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    const int ksplit = choose_ksplit(N);
    int64_t kchunk = (K + ksplit - 1) / ksplit;
    kchunk = (kchunk + kStage - 1) / kStage * kStage;
    const int64_t rowblocks = (N + kRowsPerBlock - 1) / kRowsPerBlock;
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
