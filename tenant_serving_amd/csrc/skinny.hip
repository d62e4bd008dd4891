// Decode path on MFMA, 4 < M <= 64 tokens.
//
// Same definition as the VALU path ("BitDelta : servir 14 modèles Zen depuis
// un seul cluster GPU", hanzo-blog 2026-02-28, "Serving architecture"), but
// with more tokens the dot products would exceed the VALU budget at HBM
// speed, so they go to v_mfma_f32_16x16x32_bf16: the 16-row n-tile of W_eff
// is the B operand, up to 4 m-tiles of 16 tokens are the A operands.
//
// Per 32-wide k-step a lane holds 8 consecutive weights of one row
// (row = n0 + lane%16, k = 8·(lane/16)), which is exactly the B layout of
// the 16x16x32 MFMA, plus the matching sign byte; it rebuilds them with
// recon8 and feeds them straight to the MFMA, so W_eff exists only in VGPRs.
// The workgroup's 4 waves either take 4 different n-tiles or split the K
// range of fewer n-tiles; split partial sums are combined through LDS in a
// fixed order.
#include "bd_device.h"
#include "bd_internal.h"

namespace bd {
namespace {

constexpr int kSkinnyThreads = 256;
constexpr int kKStep = 32;

template <int MTILES, int kUnroll>
__global__ __launch_bounds__(kSkinnyThreads) void skinny_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const uint8_t* __restrict__ signs, const float* __restrict__ alpha, int per_row,
    float* __restrict__ y, int64_t M, int64_t N, int64_t K, int ksplit) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t tile = (int64_t)blockIdx.x * (4 / ksplit) + wave / ksplit;
    const int kpart = wave % ksplit;
    const int col = lane & 15;  // n within the tile (B), m within an m-tile (A)
    const int grp = lane >> 4;  // which 8 of the 32 k of a step
    const int64_t kbytes = K / 8;
    const int64_t nsteps = (K + kKStep - 1) / kKStep;

    int64_t n = tile * 16 + col;
    const int64_t nc = n < N ? n : N - 1;
    const uint4* wrow = reinterpret_cast<const uint4*>(w + nc * K);
    const uint8_t* srow = signs + nc * kbytes;
    const float a = alpha[per_row ? nc : 0];

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

    for (int64_t s0 = kpart; s0 < nsteps; s0 += (int64_t)ksplit * kUnroll) {
        uint4 wv[kUnroll];
        uint32_t sb[kUnroll];
        uint4 xv[kUnroll][MTILES];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            int64_t s = s0 + (int64_t)u * ksplit;
            int64_t k = s * kKStep + 8 * grp;
            bool valid = s < nsteps && k < K;
            wv[u] = valid ? load_stream16(wrow + (k >> 3)) : make_uint4(0, 0, 0, 0);
            sb[u] = valid ? load_stream_u8(srow + (k >> 3)) : 0u;
#pragma unroll
            for (int t = 0; t < MTILES; ++t)
                xv[u][t] = (valid && mvalid[t]) ? xrow[t][k >> 3] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            bf16x8_t b = as_bf16x8(recon8(wv[u], sb[u], a));
#pragma unroll
            for (int t = 0; t < MTILES; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xv[u][t]), b, acc[t],
                                                                 0, 0, 0);
        }
    }

    // D layout of the 16x16 MFMA: lane holds rows m = 4·(lane/16) + i, column
    // n = lane%16, i = 0..3.
    __shared__ float red[4][MTILES * 4][64];
#pragma unroll
    for (int t = 0; t < MTILES; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][t * 4 + i][lane] = acc[t][i];
    __syncthreads();
    if (kpart == 0 && n < N) {
#pragma unroll
        for (int t = 0; t < MTILES; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float s = red[wave][t * 4 + i][lane];
                for (int p = 1; p < ksplit; ++p) s += red[wave + p][t * 4 + i][lane];
                int64_t m = (int64_t)t * 16 + 4 * grp + i;
                if (m < M) y[m * N + n] = s;
            }
    }
}

template <int MTILES>
hipError_t launch_tiles(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                        const float* alpha, bool per_row, float* y, int64_t M, int64_t N,
                        int64_t K, hipStream_t stream) {
    constexpr int kUnroll = MTILES <= 2 ? 8 : 4;
    int64_t tiles = (N + 15) / 16;
    // Aim for >= 2048 waves in flight: split K when n-tiles are few.
    int ksplit = tiles >= 2048 ? 1 : (tiles >= 1024 ? 2 : 4);
    int per_block = 4 / ksplit;
    dim3 grid((unsigned)((tiles + per_block - 1) / per_block)), block(kSkinnyThreads);
    hipLaunchKernelGGL((skinny_kernel<MTILES, kUnroll>), grid, block, 0, stream, x, w, signs,
                       alpha, per_row ? 1 : 0, y, M, N, K, ksplit);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_skinny(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                         const float* alpha, bool per_row, float* y, int64_t M, int64_t N,
                         int64_t K, hipStream_t stream) {
    if (M <= 16) return launch_tiles<1>(x, w, signs, alpha, per_row, y, M, N, K, stream);
    if (M <= 32) return launch_tiles<2>(x, w, signs, alpha, per_row, y, M, N, K, stream);
    if (M <= 48) return launch_tiles<3>(x, w, signs, alpha, per_row, y, M, N, K, stream);
    if (M <= 64) return launch_tiles<4>(x, w, signs, alpha, per_row, y, M, N, K, stream);
    return hipErrorInvalidValue;
}

}  // namespace bd
