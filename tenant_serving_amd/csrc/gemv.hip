// Decode path, VALU dot products, 1 <= M <= 4 tokens.
//
// y[m][n] = Σ_k x[m][k]·W_eff[n][k] with W_eff rebuilt in registers
// ("BitDelta : servir 14 modèles Zen depuis un seul cluster GPU", hanzo-blog
// 2026-02-28, "Serving architecture": the fused kernel reads base weights and
// delta bits together and never writes W_eff to HBM).
//
// HBM bound: per weight 2 bytes of base + 1/8 byte of sign.  Each wave owns
// kRows output rows and streams them with 16-byte loads, lane l taking
// elements [512c + 8l, 512c + 8l + 8) of chunk c, so one load instruction
// covers 1 KiB contiguous per row and the matching 64 sign bytes are one
// coalesced byte load.  x comes through the caches (it is tiny and shared by
// every wave).  The dot products use v_dot2c_f32_bf16 on the packed bf16
// pairs, 8 products per chain, added into fp32 accumulators.  When there are too few rows to fill the GPU
// (k/v projections), the 4 waves of a workgroup split the chunks of the same
// rows and combine their partial sums through LDS in a fixed order.
#include "bd_device.h"
#include "bd_internal.h"

namespace bd {
namespace {

constexpr int kGemvThreads = 256;
constexpr int kChunk = 512;  // elements per wave-wide 16-byte load

template <int MT, int kRows, int kUnroll, int kWaves>
__device__ __forceinline__ void gemv_body(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const uint8_t* __restrict__ signs, const float* __restrict__ alpha, int per_row,
    YOut y, int64_t N, int64_t K, int ksplit) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t group = (int64_t)blockIdx.x * (kWaves / ksplit) + wave / ksplit;
    const int kpart = wave % ksplit;
    const int64_t n0 = group * kRows;
    const int64_t kbytes = K / 8;
    const int64_t nchunks = (K + kChunk - 1) / kChunk;

    const uint4* wrow[kRows];
    const uint8_t* srow[kRows];
    float a[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        int64_t n = n0 + r < N ? n0 + r : N - 1;  // rows past the end recompute row N-1, never stored
        wrow[r] = reinterpret_cast<const uint4*>(w + n * K);
        srow[r] = signs + n * kbytes;
        a[r] = alpha[per_row ? n : 0];
    }

    float acc[kRows][MT];
#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

    // Every load is unconditional and in bounds: a lane past K, or a chunk
    // past the last, reads its row's first 8 weights and x's first 8 values,
    // and both are zeroed with a bit mask where they are used (conditional
    // loads become branches, after which the compiler may wait for every
    // outstanding load).
    for (int64_t c0 = kpart; c0 < nchunks; c0 += (int64_t)ksplit * kUnroll) {
        uint4 wv[kUnroll][kRows];
        uint32_t sb[kUnroll][kRows];
        uint4 xv[kUnroll][MT];
        uint32_t vm[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t c = c0 + (int64_t)u * ksplit;
            const int64_t k = c * kChunk + 8 * lane;
            const bool valid = c < nchunks && k < K;
            const int64_t kc = valid ? k : 0;
            vm[u] = valid ? 0xffffffffu : 0u;
#pragma unroll
            for (int r = 0; r < kRows; ++r) {
                wv[u][r] = load_stream16(wrow[r] + (kc >> 3));
                sb[u][r] = load_stream_u8(srow[r] + (kc >> 3));
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) xv[u][m] = *reinterpret_cast<const uint4*>(x + m * K + kc);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t q = vm[u];
#pragma unroll
            for (int r = 0; r < kRows; ++r) {
                uint4 e = recon8(wv[u][r], sb[u][r], a[r]);
                e = make_uint4(e.x & q, e.y & q, e.z & q, e.w & q);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    const uint4 xm = make_uint4(xv[u][m].x & q, xv[u][m].y & q, xv[u][m].z & q, xv[u][m].w & q);
                    acc[r][m] += dot8_bf16(e, xm);
                }
            }
        }
    }

    __shared__ float red[kWaves][kRows * MT];
#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            float s = wave_sum(acc[r][m]);
            if (lane == 0) red[wave][r * MT + m] = s;
        }
    __syncthreads();
    if (kpart == 0 && lane < kRows * MT) {
        int r = lane / MT, m = lane % MT;
        float s = red[wave][lane];
        for (int p = 1; p < ksplit; ++p) s += red[wave + p][lane];
        int64_t n = n0 + r;
        if (n < N) store_y(y, (int64_t)m * N + n, s);
    }
}

template <int MT, int kRows, int kUnroll>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const uint8_t* __restrict__ signs, const float* __restrict__ alpha, int per_row,
    YOut y, int64_t N, int64_t K, int ksplit) {
    gemv_body<MT, kRows, kUnroll, 4>(x, w, signs, alpha, per_row, y, N, K, ksplit);
}

// The same with 8 waves to a workgroup, which split the K chunks of its rows
// 8 ways.
template <int MT, int kRows, int kUnroll>
__global__ __launch_bounds__(8 * 64) void gemv8_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const uint8_t* __restrict__ signs, const float* __restrict__ alpha, int per_row,
    YOut y, int64_t N, int64_t K, int ksplit) {
    gemv_body<MT, kRows, kUnroll, 8>(x, w, signs, alpha, per_row, y, N, K, ksplit);
}

// Two to four tokens on projections with many rows, x small enough for LDS:
// the same VALU dot products with x resident in LDS.  Each workgroup copies
// the whole x [MT, K] into LDS once (at most 64 KiB, so two workgroups of 8
// waves share a CU), then each wave streams one row at a time over all of K
// exactly as the GEMV does (1 KiB per load, kU chunks per batch) and reads
// its x fragments from LDS instead of through the caches, which would
// otherwise queue with the weight stream.  Wave g of the grid takes rows
// g, g + T, ... (T waves), so every wave gets the same number of rows when T
// divides N (4096 waves: 7 rows of gate/up, 2 of q/o).  An x of more than
// 64 KiB (up to 128 KiB) takes one workgroup of 16 waves per CU instead.
template <int MT, int kU, int kWaves, int kXBytes>
__global__ __launch_bounds__(kWaves * 64) void xres_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const uint8_t* __restrict__ signs, const float* __restrict__ alpha, int per_row,
    YOut y, int64_t N, int64_t K) {
    __shared__ uint4 xs[kXBytes / 16];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t kg = K / 8;  // 16-byte groups per x row
    {
        const uint4* x4 = reinterpret_cast<const uint4*>(x);
        for (int64_t e = threadIdx.x; e < MT * kg; e += kWaves * 64) xs[e] = x4[e];
    }
    __syncthreads();
    const int64_t T = (int64_t)gridDim.x * kWaves;
    const int64_t nchunks = (K + kChunk - 1) / kChunk;
    const int64_t kbytes = K / 8;
    for (int64_t n = (int64_t)blockIdx.x * kWaves + wave; n < N; n += T) {
        const uint4* wrow = reinterpret_cast<const uint4*>(w + n * K);
        const uint8_t* srow = signs + n * kbytes;
        const float a = alpha[per_row ? n : 0];
        float acc[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
        for (int64_t c0 = 0; c0 < nchunks; c0 += kU) {
            uint4 wv[kU];
            uint32_t sb[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int64_t k = (c0 + u) * kChunk + 8 * lane;
                const bool valid = c0 + u < nchunks && k < K;
                wv[u] = valid ? load_stream16(wrow + (k >> 3)) : make_uint4(0, 0, 0, 0);
                sb[u] = valid ? load_stream_u8(srow + (k >> 3)) : 0u;
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int64_t k = (c0 + u) * kChunk + 8 * lane;
                const bool valid = c0 + u < nchunks && k < K;
                const uint4 e = recon8(wv[u], sb[u], a);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    const uint4 xv = valid ? xs[m * kg + (k >> 3)] : make_uint4(0, 0, 0, 0);
                    acc[m] += dot8_bf16(e, xv);
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const float s = wave_sum(acc[m]);
            if (lane == 0) store_y(y, (int64_t)m * N + n, s);
        }
    }
}

template <int MT>
hipError_t launch_xres_mt(const uint16_t* x, const uint16_t* w, const uint8_t* signs, const float* alpha,
                          bool per_row, YOut y, int64_t N, int64_t K, int num_cu, hipStream_t stream) {
    const int64_t max_waves = (int64_t)16 * num_cu;  // 16 waves per CU either way
    const int64_t waves = N < max_waves ? N : max_waves;
    if (MT * K * 2 <= 65536) {
        const int64_t grid = (waves + 7) / 8;
        hipLaunchKernelGGL((xres_kernel<MT, 4, 8, 65536>), dim3((unsigned)grid), dim3(8 * 64), 0, stream, x, w,
                           signs, alpha, per_row ? 1 : 0, y, N, K);
    } else {
        const int64_t grid = (waves + 15) / 16;
        hipLaunchKernelGGL((xres_kernel<MT, 4, 16, 131072>), dim3((unsigned)grid), dim3(16 * 64), 0, stream, x,
                           w, signs, alpha, per_row ? 1 : 0, y, N, K);
    }
    return hipGetLastError();
}

template <int MT, int kRows, int kUnroll = (MT <= 2 ? 4 : 2)>
hipError_t launch_mt(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                     const float* alpha, bool per_row, YOut y, int64_t N, int64_t K, int ksplit,
                     hipStream_t stream) {
    int64_t groups = (N + kRows - 1) / kRows;
    int per_block = 4 / ksplit;
    dim3 grid((unsigned)((groups + per_block - 1) / per_block)), block(kGemvThreads);
    hipLaunchKernelGGL((gemv_kernel<MT, kRows, kUnroll>), grid, block, 0, stream, x, w, signs,
                       alpha, per_row ? 1 : 0, y, N, K, ksplit);
    return hipGetLastError();
}

// One token on 4096..8191 rows of 8192..16384 weights: two rows per
// 8-wave workgroup, the K chunks split 8 ways, 2 per batch.
hipError_t launch_gemv8(const uint16_t* x, const uint16_t* w, const uint8_t* signs, const float* alpha,
                        bool per_row, YOut y, int64_t N, int64_t K, hipStream_t stream) {
    const int64_t groups = (N + 1) / 2;
    hipLaunchKernelGGL((gemv8_kernel<1, 2, 2>), dim3((unsigned)groups), dim3(8 * 64), 0, stream, x, w, signs,
                       alpha, per_row ? 1 : 0, y, N, K, 8);
    return hipGetLastError();
}

// One token: the workgroup shape by row count (same-process timings against
// two rows per 4-wave workgroup, split 2 ways on 4096..8191 rows and 4 ways
// below): fewer than 2048 rows of up to 16K weights take one row per
// workgroup (1024x8192 6.3 -> 5.9 us, 512x8192 4.7 -> 4.4, 1024x5000 5.7 ->
// 5.1; level at 2048 and 3072 rows), 4096..8191 rows of 8192..16384 weights
// the 8-wave workgroups (4096x8192 15.3 -> 14.3, 6144x8192 21.1 -> 19.7,
// 6152x14336 35.7 -> 32.4; at 4104x4096 they lose, 9.3 -> 11.3).
bool gemv_one_row(int64_t N, int64_t K) { return N < 2048 && K <= 16384; }
bool gemv_eight(int64_t N, int64_t K) { return N >= 4096 && N < 8192 && K >= 8192 && K <= 16384; }

template <int MT>
hipError_t launch_rows(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                       const float* alpha, bool per_row, YOut y, int64_t N, int64_t K,
                       hipStream_t stream) {
    // Two rows per wave, and the 4 waves of a workgroup split the K chunks of
    // the same two rows, so a workgroup reads whole rows at once and exits.
    // Waves that each walk their own rows in batches of 4 chunks were slower
    // wherever it was measured, most on rows of 16 KiB (a power-of-two pitch:
    // every wave then reads the same offsets of rows 16 KiB apart), at one
    // token: 28672x8192 79.0 -> 72.0 us, 57344x8192 154.0 -> 147.3, 8192x28672
    // 79.5 -> 77.4, 16384x28672 160.4 -> 157.6, q/o 8192x8192 26.3 -> 25.7.
    // Eight or sixteen waves per row pair, or 8 chunks per batch, were slower
    // again on 28672-wide rows (78.5..110.7 us).  4096..8191 rows split 2 ways.
    if (MT == 1 && gemv_eight(N, K)) return launch_gemv8(x, w, signs, alpha, per_row, y, N, K, stream);
    if (MT == 1 && gemv_one_row(N, K)) return launch_mt<1, 1, 4>(x, w, signs, alpha, per_row, y, N, K, 4, stream);
    const int ksplit = N >= 4096 && N < 8192 ? 2 : 4;
    return launch_mt<MT, 2>(x, w, signs, alpha, per_row, y, N, K, ksplit, stream);
}

}  // namespace

const char* xres_name(int64_t M, int64_t K) {
    static const char* const names[2][3] = {
        {"xres_kernel<2,4,8,65536>", "xres_kernel<3,4,8,65536>", "xres_kernel<4,4,8,65536>"},
        {"xres_kernel<2,4,16,131072>", "xres_kernel<3,4,16,131072>", "xres_kernel<4,4,16,131072>"}};
    if (M < 2 || M > kXresMaxM) return "";
    return names[M * K * 2 <= 65536 ? 0 : 1][M - 2];
}

hipError_t launch_xres(const uint16_t* x, const uint16_t* w, const uint8_t* signs, const float* alpha,
                       bool per_row, YOut y, int64_t M, int64_t N, int64_t K, int num_cu,
                       hipStream_t stream) {
    if (M * K * 2 > kXresXBytes || num_cu < 1) return hipErrorInvalidValue;
    switch (M) {
        case 2: return launch_xres_mt<2>(x, w, signs, alpha, per_row, y, N, K, num_cu, stream);
        case 3: return launch_xres_mt<3>(x, w, signs, alpha, per_row, y, N, K, num_cu, stream);
        case 4: return launch_xres_mt<4>(x, w, signs, alpha, per_row, y, N, K, num_cu, stream);
        default: return hipErrorInvalidValue;
    }
}

const char* gemv_name(int64_t M, int64_t N, int64_t K) {
    static const char* const names[4] = {"gemv_kernel<1,2,4>", "gemv_kernel<2,2,4>",
                                         "gemv_kernel<3,2,2>", "gemv_kernel<4,2,2>"};
    if (M == 1 && gemv_eight(N, K)) return "gemv8_kernel<1,2,2>";
    if (M == 1 && gemv_one_row(N, K)) return "gemv_kernel<1,1,4>";
    return (M >= 1 && M <= 4) ? names[M - 1] : "";
}

hipError_t launch_gemv(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                       const float* alpha, bool per_row, YOut y, int64_t M, int64_t N,
                       int64_t K, hipStream_t stream) {
    switch (M) {
        case 1: return launch_rows<1>(x, w, signs, alpha, per_row, y, N, K, stream);
        case 2: return launch_rows<2>(x, w, signs, alpha, per_row, y, N, K, stream);
        case 3: return launch_rows<3>(x, w, signs, alpha, per_row, y, N, K, stream);
        case 4: return launch_rows<4>(x, w, signs, alpha, per_row, y, N, K, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace bd
