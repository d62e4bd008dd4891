// Compression pass: Δ (fp32) -> packed sign bits + α.
//
// "BitDelta : servir 14 modèles Zen depuis un seul cluster GPU" (hanzo-blog,
// 2026-02-28), "Mathematical foundation": sign(Δ) keeps one bit per element,
// α = (1/n)·||Δ||_1 = mean |Δ_ij| (per matrix); "Infrastructure details":
// signs packed 8 per byte, one fp32 α per output dimension.  Bit b of byte j
// of row n is !(Δ[n][8j+b] < 0) (bit 1 = +1, zero counts as +1), least
// significant bit first along d_in.
//
// One pass over Δ at 4 + 1/8 bytes per element: HBM bound.  One workgroup per
// row (512 lanes with 4 steps in flight on rows of 8192 or more elements, 256
// lanes with 8 on shorter ones); each lane takes one float4 per step (a wave
// reads 1 KiB contiguous) and builds a 4-bit nibble.  When the sign
// rows are 4-byte aligned, 8 lanes OR their nibbles into one dword (32
// consecutive elements) that one of them stores; otherwise the even lane of
// each pair merges its partner's nibble into one byte.  |Δ| is summed in fp32
// over each float4 and in fp64 from there on, in a fixed order.
#include "bd_device.h"
#include "bd_internal.h"

namespace bd {
namespace {


__device__ __forceinline__ uint32_t nibble(float4 v) {
    return (uint32_t)!(v.x < 0.0f) | ((uint32_t)!(v.y < 0.0f) << 1) |
           ((uint32_t)!(v.z < 0.0f) << 2) | ((uint32_t)!(v.w < 0.0f) << 3);
}

// kThreads lanes per row, kUnroll float4 loads in flight per lane: 512 x 4
// on rows of 8192 or more elements, 256 x 8 on shorter ones (same-process
// A/B against 256 x 8 everywhere: 28672x8192 157.1 -> 153.4 us, 8192x8192
// 45.5 -> 42.5, 8192x28672 167.8 -> 163.7, 1024x8192 7.9 -> 7.3; on
// 8192x4096, half of 512 x 4 idle, 22.5 -> 25.7, so shorter rows keep 256 x 8).
template <bool kPerRow, bool kWords, int kThreads, int kUnroll>
__global__ __launch_bounds__(kThreads) void compress_rows(
    const float* __restrict__ delta, int64_t d_in, uint8_t* __restrict__ signs,
    float* __restrict__ alpha, double* __restrict__ row_sums) {
    const int64_t n = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t nf4 = d_in / 4;  // even, since d_in % 8 == 0
    const float4* row = reinterpret_cast<const float4*>(delta + n * d_in);
    uint8_t* srow = signs + n * (d_in / 8);

    double acc = 0.0;
    for (int64_t base = 0; base < nf4; base += (int64_t)kThreads * kUnroll) {
        float4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            int64_t i = base + (int64_t)u * kThreads + tid;
            v[u] = i < nf4 ? load_stream16(row + i) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            int64_t i = base + (int64_t)u * kThreads + tid;
            bool valid = i < nf4;
            float part = (fabsf(v[u].x) + fabsf(v[u].y)) + (fabsf(v[u].z) + fabsf(v[u].w));
            acc += (double)part;
            const uint32_t nib = nibble(v[u]);
            if (kWords) {
                // lanes i .. i+7 (i % 8 == 0) -> one dword of 32 signs; rows
                // of a multiple of 32 elements, so a group is whole or absent
                uint32_t word = nib << (4 * (tid & 7));
                word |= (uint32_t)__shfl_xor((int)word, 1, 64);
                word |= (uint32_t)__shfl_xor((int)word, 2, 64);
                word |= (uint32_t)__shfl_xor((int)word, 4, 64);
                if (valid && (tid & 7) == 0) *reinterpret_cast<uint32_t*>(srow + (i >> 1)) = word;
            } else {
                uint32_t other = (uint32_t)__shfl_xor((int)nib, 1, 64);
                // pairs (i, i^1) are both valid or both not: nf4 is even
                if (valid && (i & 1) == 0) srow[i >> 1] = (uint8_t)(nib | (other << 4));
            }
        }
    }

    __shared__ double partial[kThreads / 64];
    acc = wave_sum(acc);
    if ((tid & 63) == 0) partial[tid >> 6] = acc;
    __syncthreads();
    if (tid == 0) {
        double total = partial[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) total += partial[w];
        if (kPerRow)
            alpha[n] = (float)(total / (double)d_in);
        else
            row_sums[n] = total;
    }
}

// Compression from a (fine-tuned, base) bf16 pair ("Mathematical foundation":
// Δ = W_ft − W_base): Δ is formed in registers as the fp32 difference of the
// two widened bf16 weights and never stored.  One workgroup of lanes per
// row; each lane takes 8 consecutive weights of both matrices per step (a
// wave reads 1 KiB contiguous of each) and writes their sign byte directly.
// |Δ| is summed in fp32 over each group of 8 and in fp64 from there on, in a
// fixed order.  2 + 2 + 1/8 bytes per element.
// kThreads lanes per row, kUnroll groups of 8 in flight per lane: 512 x 2 on
// rows of 8192 or more weights, 256 x 4 on shorter ones (same-process A/B
// against 256 x 4 everywhere: 28672x8192 156.3 -> 152.7 us, 8192x8192 44.7
// -> 43.7, 8192x28672 168.0 -> 164.9; 8192x4096 21.9 -> 22.7).
template <bool kPerRow, int kThreads, int kUnroll>
__global__ __launch_bounds__(kThreads) void compress_pair_rows(
    const uint16_t* __restrict__ w_ft, const uint16_t* __restrict__ w_base, int64_t d_in,
    uint8_t* __restrict__ signs, float* __restrict__ alpha, double* __restrict__ row_sums) {
    const int64_t n = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t ng = d_in / 8;  // groups of 8 weights (16 bytes) in the row
    const uint4* fr = reinterpret_cast<const uint4*>(w_ft + n * d_in);
    const uint4* br = reinterpret_cast<const uint4*>(w_base + n * d_in);
    uint8_t* srow = signs + n * ng;

    double acc = 0.0;
    for (int64_t base = 0; base < ng; base += (int64_t)kThreads * kUnroll) {
        uint4 f[kUnroll], b[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + (int64_t)u * kThreads + tid;
            f[u] = i < ng ? load_stream16(fr + i) : make_uint4(0, 0, 0, 0);
            b[u] = i < ng ? load_stream16(br + i) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + (int64_t)u * kThreads + tid;
            const uint32_t fw[4] = {f[u].x, f[u].y, f[u].z, f[u].w};
            const uint32_t bw[4] = {b[u].x, b[u].y, b[u].z, b[u].w};
            uint32_t byte = 0;
            float part = 0.0f;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float dlo = __uint_as_float(fw[p] << 16) - __uint_as_float(bw[p] << 16);
                const float dhi = __uint_as_float(fw[p] & 0xffff0000u) - __uint_as_float(bw[p] & 0xffff0000u);
                byte |= ((uint32_t)!(dlo < 0.0f) << (2 * p)) | ((uint32_t)!(dhi < 0.0f) << (2 * p + 1));
                part += fabsf(dlo) + fabsf(dhi);
            }
            acc += (double)part;
            if (i < ng) srow[i] = (uint8_t)byte;
        }
    }

    __shared__ double partial[kThreads / 64];
    acc = wave_sum(acc);
    if ((tid & 63) == 0) partial[tid >> 6] = acc;
    __syncthreads();
    if (tid == 0) {
        double total = partial[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) total += partial[w];
        if (kPerRow)
            alpha[n] = (float)(total / (double)d_in);
        else
            row_sums[n] = total;
    }
}

// Per-matrix α: fixed-order reduction of the per-row sums.
__global__ __launch_bounds__(256) void reduce_row_sums(const double* __restrict__ row_sums,
                                                      int64_t d_out, int64_t d_in,
                                                      float* __restrict__ alpha) {
    const int tid = threadIdx.x;
    // thread tid adds rows tid, tid + 256, ... in that order; 16 of them are
    // loaded at a time so the loads' latency is paid once per 16 rows
    constexpr int kBatch = 16;
    double acc = 0.0;
    int64_t r = tid;
    for (; r + (int64_t)(kBatch - 1) * 256 < d_out; r += (int64_t)kBatch * 256) {
        double v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) v[u] = row_sums[r + (int64_t)u * 256];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) acc += v[u];
    }
    for (; r < d_out; r += 256) acc += row_sums[r];
    __shared__ double partial[4];
    acc = wave_sum(acc);
    if ((tid & 63) == 0) partial[tid >> 6] = acc;
    __syncthreads();
    if (tid == 0) {
        double total = ((partial[0] + partial[1]) + partial[2]) + partial[3];
        alpha[0] = (float)(total / ((double)d_out * (double)d_in));
    }
}

}  // namespace

template <bool kPerRow>
void launch_pair_rows(const uint16_t* w_ft, const uint16_t* w_base, int64_t d_out, int64_t d_in, uint8_t* signs,
                      float* alpha, double* row_sums, hipStream_t stream) {
    const dim3 grid((unsigned)d_out);
    if (d_in >= 8192)
        hipLaunchKernelGGL((compress_pair_rows<kPerRow, 512, 2>), grid, dim3(512), 0, stream, w_ft, w_base, d_in,
                           signs, alpha, row_sums);
    else
        hipLaunchKernelGGL((compress_pair_rows<kPerRow, 256, 4>), grid, dim3(256), 0, stream, w_ft, w_base, d_in,
                           signs, alpha, row_sums);
}

hipError_t launch_compress_pair(const uint16_t* w_ft, const uint16_t* w_base, int64_t d_out,
                                int64_t d_in, bool per_row, uint8_t* signs, float* alpha,
                                double* row_sums, hipStream_t stream) {
    if (per_row) {
        launch_pair_rows<true>(w_ft, w_base, d_out, d_in, signs, alpha, row_sums, stream);
        return hipGetLastError();
    }
    launch_pair_rows<false>(w_ft, w_base, d_out, d_in, signs, alpha, row_sums, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(reduce_row_sums, dim3(1), dim3(256), 0, stream, row_sums, d_out, d_in,
                       alpha);
    return hipGetLastError();
}

template <bool kPerRow, bool kWords>
void launch_rows(const float* delta, int64_t d_out, int64_t d_in, uint8_t* signs, float* alpha, double* row_sums,
                 hipStream_t stream) {
    const dim3 grid((unsigned)d_out);
    if (d_in >= 8192)
        hipLaunchKernelGGL((compress_rows<kPerRow, kWords, 512, 4>), grid, dim3(512), 0, stream, delta, d_in, signs,
                           alpha, row_sums);
    else
        hipLaunchKernelGGL((compress_rows<kPerRow, kWords, 256, 8>), grid, dim3(256), 0, stream, delta, d_in, signs,
                           alpha, row_sums);
}

hipError_t launch_compress(const float* delta, int64_t d_out, int64_t d_in, bool per_row,
                           uint8_t* signs, float* alpha, double* row_sums, hipStream_t stream) {
    // dword sign stores need every sign row 4-byte aligned
    const bool words = d_in % 32 == 0 && (reinterpret_cast<uintptr_t>(signs) & 3) == 0;
    if (per_row) {
        if (words)
            launch_rows<true, true>(delta, d_out, d_in, signs, alpha, row_sums, stream);
        else
            launch_rows<true, false>(delta, d_out, d_in, signs, alpha, row_sums, stream);
        return hipGetLastError();
    }
    if (words)
        launch_rows<false, true>(delta, d_out, d_in, signs, alpha, row_sums, stream);
    else
        launch_rows<false, false>(delta, d_out, d_in, signs, alpha, row_sums, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(reduce_row_sums, dim3(1), dim3(256), 0, stream, row_sums, d_out, d_in,
                       alpha);
    return hipGetLastError();
}

}  // namespace bd
