// Decode path on MFMA, 1 <= M <= 64 tokens.
//
// Same definition as the VALU path ("BitDelta : servir 14 modèles Zen depuis
// un seul cluster GPU", hanzo-blog 2026-02-28, "Serving architecture": base
// weights and delta bits read together, W_eff rebuilt on chip, never stored
// to HBM), with the dot products on v_mfma_f32_16x16x32_bf16: a 16-row
// n-tile of W_eff is the B operand, up to 4 m-tiles of 16 tokens are the A
// operands.
//
// Memory side.  The MFMA B layout wants 16 rows per load instruction (64
// bytes of each), which streams HBM markedly slower than reading rows
// contiguously.  So each wave streams its 16 rows row-contiguously -- one
// load instruction covers two rows x 512 bytes -- rebuilds W_eff in
// registers (the lane's sign byte is one coalesced byte load), and writes it
// to a wave-private LDS tile, from which it reads the B fragments in MFMA
// layout.  The tile is private to the wave, so no barrier is needed; the
// loads of chunk c+1 are issued before chunk c is processed.
//
// Work split.  Each wave owns one 16-row n-tile and a share of the K chunks;
// when n-tiles are few (k/v projections) the waves of a workgroup split the
// chunks of the same n-tile and combine partial sums through LDS in a fixed
// order.
#include "bd_device.h"
#include "bd_internal.h"

namespace bd {
namespace {

constexpr int kTileRows = 16;  // rows per wave (one MFMA n-tile)

// Geometry of one K chunk of width CK: a load instruction covers
// kRowsPerLoad rows x (CK x 2) bytes, lane = (row in load, 16-byte group).
template <int CK>
struct Chunk {
    static constexpr int kGroups = CK / 8;                 // 16-byte groups per row
    static constexpr int kRowsPerLoad = 64 / kGroups;
    static constexpr int kLoads = kTileRows / kRowsPerLoad;
    static constexpr int kSteps = CK / 32;                 // MFMA k-steps
};

// LDS tile: [16 rows][CK/8 chunks of 16 bytes], chunk index XOR row so that
// the 16 rows read at one chunk position fall in different banks.
template <int CK>
__device__ __forceinline__ int tslot(int row, int chunk) {
    return row * Chunk<CK>::kGroups + (chunk ^ row);
}

// Phase 1: rebuild the chunk's weights into the wave's LDS tile.
template <int CK>
__device__ __forceinline__ void stage_chunk(const uint4 (&wv)[Chunk<CK>::kLoads],
                                            const uint32_t (&sb)[Chunk<CK>::kLoads],
                                            const float (&a)[Chunk<CK>::kLoads],
                                            uint4* __restrict__ tile, int lane) {
    using C = Chunk<CK>;
    const int rsub = lane / C::kGroups, kg = lane % C::kGroups;
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i)
        tile[tslot<CK>(C::kRowsPerLoad * i + rsub, kg)] = recon8(wv[i], sb[i], a[i]);
}

// Phase 2: MFMA over the chunk, B fragments from the tile, A fragments (x)
// through the caches (issued first, so their latency overlaps the rebuild
// of the caller's next chunk and the tile reads).
template <int MTILES, int CK, bool kFull>
__device__ __forceinline__ void mfma_chunk(const uint4* __restrict__ tile,
                                           const uint4* const (&xrow)[MTILES],
                                           const bool (&mvalid)[MTILES], int64_t k0, int64_t K,
                                           int lane, f32x4_t (&acc)[MTILES]) {
    using C = Chunk<CK>;
    const int col = lane & 15, grp = lane >> 4;
    uint4 xv[C::kSteps][MTILES];
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) {
        const int64_t k = k0 + s * 32 + 8 * grp;
#pragma unroll
        for (int t = 0; t < MTILES; ++t) {
            bool ok = mvalid[t] && (kFull || k < K);
            xv[s][t] = ok ? xrow[t][k >> 3] : make_uint4(0, 0, 0, 0);
        }
    }
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) {
        bf16x8_t b = as_bf16x8(tile[tslot<CK>(col, 4 * s + grp)]);
#pragma unroll
        for (int t = 0; t < MTILES; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xv[s][t]), b, acc[t], 0, 0, 0);
    }
}

template <int MTILES, int kWaves, int CK, int U, int kMinWaves>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(kMinWaves))) void skinny_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const uint8_t* __restrict__ signs, const float* __restrict__ alpha, int per_row,
    YOut y, int64_t M, int64_t N, int64_t K, int ksplit) {
    using C = Chunk<CK>;
    __shared__ uint4 lds[kWaves * kTileRows * C::kGroups];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t ntile = (int64_t)blockIdx.x * (kWaves / ksplit) + wave / ksplit;
    const int kpart = wave % ksplit;
    const int col = lane & 15, grp = lane >> 4;
    const int rsub = lane / C::kGroups, kg = lane % C::kGroups;
    const int64_t kbytes = K / 8;
    const int64_t nchunks = (K + CK - 1) / CK;
    const int64_t nfull = K / CK;
    uint4* tile = lds + wave * kTileRows * C::kGroups;

    // This lane's load slots: rows kRowsPerLoad·i + rsub of the tile, 16-byte
    // group kg of a chunk.  Rows past the end are computed, never stored.
    int32_t rowi[C::kLoads];
    float a[C::kLoads];
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
        int64_t n = ntile * kTileRows + C::kRowsPerLoad * i + rsub;
        n = n < N ? n : N - 1;
        rowi[i] = (int32_t)n;
        a[i] = alpha[per_row ? n : 0];
    }
    auto wptr = [&](int i, int64_t c) {
        return reinterpret_cast<const uint4*>(w + (int64_t)rowi[i] * K + c * CK + 8 * kg);
    };
    auto sptr = [&](int i, int64_t c) { return signs + (int64_t)rowi[i] * kbytes + c * (CK / 8) + kg; };
    const uint4* xrow[MTILES];
    bool mvalid[MTILES];
#pragma unroll
    for (int t = 0; t < MTILES; ++t) {
        int64_t m = (int64_t)t * 16 + col;
        mvalid[t] = m < M;
        xrow[t] = reinterpret_cast<const uint4*>(x + (mvalid[t] ? m : 0) * K);
    }

    f32x4_t acc[MTILES];
#pragma unroll
    for (int t = 0; t < MTILES; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Full chunks in groups of U: the group's loads are issued together, then
    // each chunk is rebuilt into the LDS tile and multiplied.  Memory
    // parallelism comes from the many resident waves (small register
    // footprint), as in the VALU path.
    for (int64_t c0 = kpart; c0 < nfull; c0 += (int64_t)ksplit * U) {
        uint4 wv[U][C::kLoads];
        uint32_t sb[U][C::kLoads];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + (int64_t)u * ksplit;
            if (u == 0 || c < nfull) {
#pragma unroll
                for (int i = 0; i < C::kLoads; ++i) {
                    wv[u][i] = load_stream16(wptr(i, c));
                    sb[u][i] = load_stream_u8(sptr(i, c));
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + (int64_t)u * ksplit;
            if (u == 0 || c < nfull) {
                stage_chunk<CK>(wv[u], sb[u], a, tile, lane);
                mfma_chunk<MTILES, CK, true>(tile, xrow, mvalid, c * CK, K, lane, acc);
            }
        }
    }
    // The ragged last chunk (K % CK != 0), if this wave owns it.
    if (nfull < nchunks && (nchunks - 1) % ksplit == kpart) {
        const int64_t c = nchunks - 1;
        uint4 wv[C::kLoads];
        uint32_t sb[C::kLoads];
        const bool ok = c * CK + 8 * kg < K;
#pragma unroll
        for (int i = 0; i < C::kLoads; ++i) {
            wv[i] = ok ? load_stream16(wptr(i, c)) : make_uint4(0, 0, 0, 0);
            sb[i] = ok ? load_stream_u8(sptr(i, c)) : 0u;
        }
        stage_chunk<CK>(wv, sb, a, tile, lane);
        mfma_chunk<MTILES, CK, false>(tile, xrow, mvalid, c * CK, K, lane, acc);
    }

    // D layout of the 16x16 MFMA: lane holds rows m = 4·(lane/16) + i,
    // column n = lane%16.  K-split partials meet in LDS (reusing the tiles).
    const int64_t n = ntile * kTileRows + col;
    if (ksplit == 1) {
        if (n < N) {
#pragma unroll
            for (int t = 0; t < MTILES; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    int64_t m = (int64_t)t * 16 + 4 * grp + i;
                    if (m < M) store_y(y, m * N + n, acc[t][i]);
                }
        }
        return;
    }
    __syncthreads();
    float* red = reinterpret_cast<float*>(lds);  // [wave][MTILES*4][64]
#pragma unroll
    for (int t = 0; t < MTILES; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[(wave * MTILES * 4 + t * 4 + i) * 64 + lane] = acc[t][i];
    __syncthreads();
    if (kpart == 0 && n < N) {
#pragma unroll
        for (int t = 0; t < MTILES; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float s = red[(wave * MTILES * 4 + t * 4 + i) * 64 + lane];
                for (int p = 1; p < ksplit; ++p)
                    s += red[((wave + p) * MTILES * 4 + t * 4 + i) * 64 + lane];
                int64_t m = (int64_t)t * 16 + 4 * grp + i;
                if (m < M) store_y(y, m * N + n, s);
            }
    }
}

template <int MTILES, int kWaves, int CK, int U, int kMinWaves>
hipError_t launch_cfg(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                      const float* alpha, bool per_row, YOut y, int64_t M, int64_t N, int64_t K,
                      int ksplit, hipStream_t stream) {
    const int64_t tiles = (N + kTileRows - 1) / kTileRows;
    const int per_block = kWaves / ksplit;
    dim3 grid((unsigned)((tiles + per_block - 1) / per_block)), block(kWaves * 64);
    hipLaunchKernelGGL((skinny_kernel<MTILES, kWaves, CK, U, kMinWaves>), grid, block, 0, stream, x, w, signs,
                       alpha, per_row ? 1 : 0, y, M, N, K, ksplit);
    return hipGetLastError();
}

// K split over the waves of a workgroup so that enough waves stream
// (tiles x split >= 4096, at most 8 ways).
int skinny_split(int64_t N) {
    const int64_t tiles = (N + kTileRows - 1) / kTileRows;
    int ksplit = 1;
    while (ksplit < 8 && tiles * ksplit < 4096) ksplit *= 2;
    return ksplit;
}

template <int MTILES>
hipError_t launch_tiles(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                        const float* alpha, bool per_row, YOut y, int64_t M, int64_t N,
                        int64_t K, hipStream_t stream) {
    const int ksplit = skinny_split(N);
    if (MTILES == 1) {
        // 256-wide chunks, one chunk per load group, >= 4 waves per SIMD.
        if (ksplit <= 4)
            return launch_cfg<MTILES, 4, 256, 1, 4>(x, w, signs, alpha, per_row, y, M, N, K, ksplit, stream);
        return launch_cfg<MTILES, 8, 256, 1, 4>(x, w, signs, alpha, per_row, y, M, N, K, ksplit, stream);
    }
    // More m-tiles need more registers: no occupancy bound, 128-wide chunks
    // when split more than 4 ways.
    if (ksplit <= 4)
        return launch_cfg<MTILES, 4, 256, 1, 1>(x, w, signs, alpha, per_row, y, M, N, K, ksplit, stream);
    return launch_cfg<MTILES, 8, 128, 2, 1>(x, w, signs, alpha, per_row, y, M, N, K, ksplit, stream);
}

}  // namespace

const char* skinny_name(int64_t M, int64_t N) {
    const int ks = skinny_split(N);
    if (M <= 16) return ks <= 4 ? "skinny_kernel<1,4,256,1,4>" : "skinny_kernel<1,8,256,1,4>";
    const int t = (int)((M + 15) / 16);
    static const char* const names[2][3] = {
        {"skinny_kernel<2,4,256,1,1>", "skinny_kernel<3,4,256,1,1>", "skinny_kernel<4,4,256,1,1>"},
        {"skinny_kernel<2,8,128,2,1>", "skinny_kernel<3,8,128,2,1>", "skinny_kernel<4,8,128,2,1>"}};
    return names[ks <= 4 ? 0 : 1][t - 2];
}

hipError_t launch_skinny(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                         const float* alpha, bool per_row, YOut y, int64_t M, int64_t N,
                         int64_t K, hipStream_t stream) {
    if (M <= 16) return launch_tiles<1>(x, w, signs, alpha, per_row, y, M, N, K, stream);
    if (M <= 32) return launch_tiles<2>(x, w, signs, alpha, per_row, y, M, N, K, stream);
    if (M <= 48) return launch_tiles<3>(x, w, signs, alpha, per_row, y, M, N, K, stream);
    if (M <= 64) return launch_tiles<4>(x, w, signs, alpha, per_row, y, M, N, K, stream);
    return hipErrorInvalidValue;
}

}  // namespace bd
