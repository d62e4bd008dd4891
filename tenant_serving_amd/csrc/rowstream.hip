// Decode path on MFMA for large projections: row-streaming workgroups.
//
// Definition as in the other linear paths ("BitDelta : servir 14 modèles Zen
// depuis un seul cluster GPU", hanzo-blog 2026-02-28, "Serving
// architecture": base weights and delta bits read together, W_eff rebuilt on
// chip and never stored to HBM, then multiplied).
//
// HBM streams fastest when each wave reads one or two rows front to back in
// 1 KiB pieces; the MFMA B operand, however, wants 16 rows at once.  So a
// workgroup of 16 waves owns 32 rows: wave w streams rows w and w+16 of the
// block (lane l holds elements 8l..8l+7 of a 512-wide chunk), rebuilds them
// with recon8 and writes them into a shared LDS tile [32 rows][512].  After
// one barrier per chunk, wave w takes MFMA k-step w of the chunk (k 32w ..
// 32w+31) for both 16-row n-tiles with the same x fragment, so x is fetched
// once per 32 rows.  The tile is double buffered (one barrier per chunk
// suffices).  At the end the waves' partial sums meet in LDS and are added
// in a fixed order.
//
// Each wave keeps a ring of kDepth chunks in flight (weights, sign bytes and
// x fragments), every load issued unconditionally from an address inside the
// buffers, so that each wait covers exactly the chunk about to be used.  One
// chunk ahead is fastest with 16 waves per workgroup; more loads in flight
// per CU were slower on every shape measured.  On projections whose 16-row
// blocks fit one per CU (4096 rows on 256 CUs) a 32-row workgroup would leave
// half the CUs idle, so there the workgroup is 8 waves over 16 rows (one
// n-tile, each wave two k-steps) with two chunks in flight.
#include "bd_device.h"
#include "bd_internal.h"

namespace bd {
namespace {

constexpr int kRsChunk = 512;         // k per chunk: 64 lanes x 8
constexpr int kRsGroups = kRsChunk / 8;

// LDS tile [32 rows][64 groups of 16 bytes]; the group index is XORed with
// the row so that the 16 rows read at one k position fall in different banks.
__device__ __forceinline__ int rs_slot(int row, int group) { return row * kRsGroups + (group ^ (row & 15)); }

// 16 bytes ANDed with a lane mask (all ones or zero); a select on a uint4
// would be lowered through private memory.
__device__ __forceinline__ uint4 mask16(uint4 v, uint32_t m) {
    return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

// kWaves = 16: 32 rows (two n-tiles) per workgroup, each wave one MFMA k-step
//              of the chunk for both n-tiles (one x fragment per chunk);
// kWaves = 8:  16 rows (one n-tile) per workgroup, each wave k-steps w and
//              w+8 of the chunk (more, smaller workgroups).
template <int MTILES, int kWaves, int kRsDepth>
__global__ __launch_bounds__(kWaves * 64) void rowstream_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const uint8_t* __restrict__ signs, const float* __restrict__ alpha, int per_row,
    YOut y, int64_t M, int64_t N, int64_t K) {
    constexpr int kRsRows = 2 * kWaves;   // rows per workgroup: 2 per wave
    constexpr int kNT = kRsRows / 16;     // n-tiles per workgroup
    constexpr int kSteps = 16 * kNT / kWaves;  // (k-step, n-tile) pairs per wave per chunk: 2
    __shared__ uint4 tile[2][kRsRows * kRsGroups];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * kRsRows;
    const int64_t kbytes = K / 8;
    const int64_t nchunks = (K + kRsChunk - 1) / kRsChunk;

    // The two rows this wave streams (rows past the end: computed, not stored).
    int64_t r0 = n0 + wave, r1 = n0 + wave + kWaves;
    r0 = r0 < N ? r0 : N - 1;
    r1 = r1 < N ? r1 : N - 1;
    const uint4* wrow0 = reinterpret_cast<const uint4*>(w + r0 * K);
    const uint4* wrow1 = reinterpret_cast<const uint4*>(w + r1 * K);
    const uint8_t* srow0 = signs + r0 * kbytes;
    const uint8_t* srow1 = signs + r1 * kbytes;
    const float a0 = alpha[per_row ? r0 : 0], a1 = alpha[per_row ? r1 : 0];
    const int64_t kgroups = K / 8;  // 16-byte groups per row

    // This wave's (k-step, n-tile) pairs of every chunk.
    int step_k[kSteps], step_nt[kSteps];
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
        step_k[j] = kNT == 2 ? wave : wave + kWaves * j;
        step_nt[j] = kNT == 2 ? j : 0;
    }
    constexpr int kXS = kNT == 2 ? 1 : kSteps;  // distinct x fragments per chunk
    // x fragment of a k-step s: token m = 16t + col, k = 32·s + 8·grp.
    const uint4* xrow[MTILES];
    bool mvalid[MTILES];
#pragma unroll
    for (int t = 0; t < MTILES; ++t) {
        int64_t m = (int64_t)t * 16 + col;
        mvalid[t] = m < M;
        xrow[t] = reinterpret_cast<const uint4*>(x + (mvalid[t] ? m : 0) * K);
    }

    f32x4_t acc[kNT][MTILES];
#pragma unroll
    for (int h = 0; h < kNT; ++h)
#pragma unroll
        for (int t = 0; t < MTILES; ++t) acc[h][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Ring of in-flight chunks (registers); chunk c lives in slot c % depth,
    // with its x fragments.  Every load is issued unconditionally from an
    // address inside the buffers (a weight or sign load past K, or of a chunk
    // past the last one, reads the first 16 bytes of x, which are in cache;
    // an x load past K reads x again), and what lies past K or M is zeroed
    // where it is used, so no load sits behind a branch and each wait covers
    // only the chunk about to be used.
    uint4 wv0[kRsDepth], wv1[kRsDepth];
    // bytes, so that their widening stays at the use (kept as 32-bit values,
    // the widening would be merged into the loop head and wait there)
    uint8_t sb0[kRsDepth], sb1[kRsDepth];
    uint4 xq[kRsDepth][kXS][MTILES];
    const uint4* const xfirst = reinterpret_cast<const uint4*>(x);
    auto issue = [&](int slot, int64_t c) {
        const int64_t g = c * kRsGroups + lane;  // >= kgroups past K and for every chunk past the last
        const bool ok = g < kgroups;
        wv0[slot] = load_stream16(ok ? wrow0 + g : xfirst);
        wv1[slot] = load_stream16(ok ? wrow1 + g : xfirst);
        sb0[slot] = __builtin_nontemporal_load(ok ? srow0 + g : reinterpret_cast<const uint8_t*>(xfirst));
        sb1[slot] = __builtin_nontemporal_load(ok ? srow1 + g : reinterpret_cast<const uint8_t*>(xfirst));
#pragma unroll
        for (int j = 0; j < kXS; ++j) {
            const int64_t gx = c * kRsGroups + 4 * step_k[j] + grp;
#pragma unroll
            for (int t = 0; t < MTILES; ++t) xq[slot][j][t] = xrow[t][gx < kgroups ? gx : 0];
        }
    };
    // Issued in chunk order (the scheduler would otherwise interleave the
    // groups, and the first use of chunk 0 would then wait for everything).
#pragma unroll
    for (int d = 0; d < kRsDepth; ++d) {
        issue(d, d);
        __builtin_amdgcn_sched_barrier(0);
    }

    // Whole rounds of kRsDepth chunks: a chunk past the last one is all zeros
    // after the masks below and adds nothing, and the loop body has no exit.
    const int64_t nround = (nchunks + kRsDepth - 1) / kRsDepth * kRsDepth;
    int64_t c0 = 0;
    do {  // at least one round (K >= 8); no guard, so the loads above stay put
#pragma unroll
        for (int d = 0; d < kRsDepth; ++d) {
            const int64_t c = c0 + d;
            const int buf = (int)(c & 1);
            // keeps each chunk's arithmetic in its own slot: an operation of a
            // later chunk moved up here would wait for that chunk's loads
            __builtin_amdgcn_sched_barrier(0);
            // rebuild this wave's two rows into the shared tile (zero past K)
            const uint32_t kin = c * kRsChunk + 8 * lane < K ? ~0u : 0u;
            tile[buf][rs_slot(wave, lane)] = mask16(recon8(wv0[d], sb0[d], a0), kin);
            tile[buf][rs_slot(wave + kWaves, lane)] = mask16(recon8(wv1[d], sb1[d], a1), kin);
            // x fragments of this chunk (zero past K or past M)
            uint4 xv[kXS][MTILES];
#pragma unroll
            for (int j = 0; j < kXS; ++j) {
                const bool kx = c * kRsChunk + 32 * step_k[j] + 8 * grp < K;
#pragma unroll
                for (int t = 0; t < MTILES; ++t) xv[j][t] = mask16(xq[d][j][t], mvalid[t] && kx ? ~0u : 0u);
            }
            issue(d, c + kRsDepth);
            __syncthreads();
            // this wave's MFMA k-steps of the chunk
#pragma unroll
            for (int j = 0; j < kSteps; ++j) {
                bf16x8_t b = as_bf16x8(tile[buf][rs_slot(16 * step_nt[j] + col, 4 * step_k[j] + grp)]);
                const int xj = kXS == 1 ? 0 : j;
#pragma unroll
                for (int t = 0; t < MTILES; ++t)
                    acc[step_nt[j]][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        as_bf16x8(xv[xj][t]), b, acc[step_nt[j]][t], 0, 0, 0);
            }
        }
        c0 += kRsDepth;
    } while (c0 < nround);

    // Sum the 16 waves' partials in a fixed order.  D layout of the 16x16
    // MFMA: lane holds rows m = 4·(lane/16) + i, column n = lane%16.
    __syncthreads();
    static_assert(MTILES <= 2, "partials must fit the two tile buffers");
    float* red = reinterpret_cast<float*>(&tile[0][0]);  // [waves][kNT][MTILES*4][64]
    constexpr int kPer = kNT * MTILES * 4;
#pragma unroll
    for (int h = 0; h < kNT; ++h)
#pragma unroll
        for (int t = 0; t < MTILES; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[(wave * kPer + (h * MTILES + t) * 4 + i) * 64 + lane] = acc[h][t][i];
    __syncthreads();
    // kPer x 64 outputs per workgroup, spread over its 1024 threads.
    for (int q = threadIdx.x; q < kPer * 64; q += kWaves * 64) {
        const int e = q / 64, l = q % 64;
        float s = red[e * 64 + l];
        for (int v = 1; v < kWaves; ++v) s += red[(v * kPer + e) * 64 + l];
        const int h = e / (MTILES * 4), t = (e / 4) % MTILES, i = e % 4;
        const int64_t n = n0 + 16 * h + (l & 15);
        const int64_t m = (int64_t)t * 16 + 4 * (l >> 4) + i;
        if (n < N && m < M) store_y(y, m * N + n, s);
    }
}

template <int MTILES, int kWaves, int kDepth>
hipError_t launch_rs(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                     const float* alpha, bool per_row, YOut y, int64_t M, int64_t N, int64_t K,
                     hipStream_t stream) {
    const int64_t rows = 2 * kWaves;
    dim3 grid((unsigned)((N + rows - 1) / rows)), block(kWaves * 64);
    hipLaunchKernelGGL((rowstream_kernel<MTILES, kWaves, kDepth>), grid, block, 0, stream, x, w, signs,
                       alpha, per_row ? 1 : 0, y, M, N, K);
    return hipGetLastError();
}

// 16-row workgroups where they fit one per CU, else 32-row ones.  Same-process
// timings at 8..32 tokens: 4096x14336 37.8-47.8 -> 24.6-40.0 us, 4096x4096
// 15.3-17.1 -> 11.2-14.4; at 4100, 5120 and 6152 rows the 32-row workgroups
// stay ahead.
bool rowstream_small(int64_t N, int num_cu) { return N <= 16 * (int64_t)num_cu; }

}  // namespace

const char* rowstream_name(int64_t M, int64_t N, int num_cu) {
    const bool small = rowstream_small(N, num_cu);
    if (M <= 16) return small ? "rowstream_kernel<1,8,2>" : "rowstream_kernel<1,16,1>";
    return small ? "rowstream_kernel<2,8,2>" : "rowstream_kernel<2,16,1>";
}

hipError_t launch_rowstream(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                            const float* alpha, bool per_row, YOut y, int64_t M, int64_t N,
                            int64_t K, int num_cu, hipStream_t stream) {
    const bool small = rowstream_small(N, num_cu);
    if (M <= 16)
        return small ? launch_rs<1, 8, 2>(x, w, signs, alpha, per_row, y, M, N, K, stream)
                     : launch_rs<1, 16, 1>(x, w, signs, alpha, per_row, y, M, N, K, stream);
    if (M <= 32)
        return small ? launch_rs<2, 8, 2>(x, w, signs, alpha, per_row, y, M, N, K, stream)
                     : launch_rs<2, 16, 1>(x, w, signs, alpha, per_row, y, M, N, K, stream);
    return hipErrorInvalidValue;  // the partial-sum exchange is sized for <= 2 m-tiles
}

}  // namespace bd
