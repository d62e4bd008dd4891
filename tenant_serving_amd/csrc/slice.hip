// Decode path for projections with few rows (up to 16 tokens): K slices.
//
// Definition as in the other linear paths ("BitDelta : servir 14 modèles Zen
// depuis un seul cluster GPU", hanzo-blog 2026-02-28, "Serving
// architecture": base weights and delta bits read together, W_eff rebuilt on
// chip and never stored to HBM, then multiplied).
//
// A projection like k or v of a 70B layer (1024 rows x 8192) is 18 MB, a few
// microseconds at HBM speed.  To fill the chip, a workgroup that covers all
// of d_in can only own a handful of rows, and then every workgroup pulls all
// of x (256 KiB at 16 tokens) through its compute unit for 68 KiB of weights.
// Here a workgroup owns 16 rows over one 2048-wide slice of d_in instead, so
// a compute unit pulls 64 KiB of x for as many bytes of weights, and 1024
// rows x 4 slices is again 256 workgroups.
//
// Workgroup: 16 waves; wave w takes k = 128 w .. 128 w + 127 of the slice for
// all 16 rows.  Its four 16-byte loads per lane cover 4 rows x 256 bytes each
// (lane l: row 4 i + l / 16, weights 8 (l % 16) .. + 7), with the matching
// sign bytes; so the workgroup reads its 16 rows' 4 KiB pieces whole, all at
// once.  The wave rebuilds them into a private LDS tile (XOR-swizzled by row)
// and reads them back as the B operand of v_mfma_f32_16x16x32_bf16, all 16
// columns real rows; the A operand is x (16 token rows; rows >= M are
// zero and their outputs are dropped), four k-steps.  The 16 waves'
// tiles of sums meet in LDS once and are added in wave order.
//
// With one slice the workgroup writes y; otherwise it writes its fp32 sums to
// plane `slice` of the workspace ([slices][M][N]) and slice_sum_kernel adds
// the planes in slice order.  Every load is unconditional and in bounds
// (rows past N repeat row N-1, weights past d_in read k = 0 and are masked
// at the use, x past its end reads zeros), so the compiler's load counters
// stay exact.  All sums are in fixed orders:
// the result is run-to-run reproducible.
#include "bd_device.h"
#include "bd_internal.h"

namespace bd {
namespace {

constexpr int kSlWaves = 16;
constexpr int kSlRows = 16;                     // rows per workgroup: the B operand's columns
constexpr int kSlSub = 128;                     // k per wave
constexpr int kSlGroups = kSlSub / 8;           // 16-byte groups per row of a wave's tile
constexpr int64_t kSlWidth = kSlWaves * kSlSub; // k per workgroup: one slice

__device__ __forceinline__ void slice_wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint4 mask16(uint4 v, uint32_t q) {
    return make_uint4(v.x & q, v.y & q, v.z & q, v.w & q);
}

__global__ __launch_bounds__(kSlWaves * 64) void slice_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, const uint8_t* __restrict__ signs,
    const float* __restrict__ alpha, int per_row, float* __restrict__ part, YOut y, int64_t M, int64_t N,
    int64_t K, int nslices) {
    __shared__ uint4 tiles[kSlWaves][kSlRows * kSlGroups];  // 64 KiB; afterwards the sums

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t slice = (int64_t)blockIdx.x % nslices;
    const int64_t row0 = (int64_t)blockIdx.x / nslices * kSlRows;
    const int64_t kbytes = K / 8;
    const int64_t kbase = slice * kSlWidth + (int64_t)wave * kSlSub;

    // x: the A operand, lane (token col, k-group grp), k-step t: k = kbase + 32 t + 8 grp.
    // Through a buffer resource that ends with x: lanes of token rows >= M
    // and k past d_in read past its end, which returns zeros and touches no
    // memory.
    const int col = lane & 15, grp = lane >> 4;
    const rsrc_t xr = make_rsrc(x, (uint32_t)(M * K * 2));
    uint4 xv[kSlSub / 32];
#pragma unroll
    for (int t = 0; t < kSlSub / 32; ++t) {
        const int64_t kx = kbase + 32 * t + 8 * grp;
        xv[t] = buf_load16(xr, (col < M && kx < K) ? (uint32_t)((col * K + kx) * 2) : 0x80000000u, 0);
    }

    // weights: load i covers rows 4i .. 4i+3 of the block, lane l row 4i + l/16
    const int lr = lane >> 4, lg = lane & 15;
    const int64_t kl = kbase + 8 * lg;
    const uint32_t kmask = kl < K ? 0xffffffffu : 0u;
    const int64_t kw = kl < K ? kl : 0;
    uint4 wv[4];
    uint32_t sb[4];
    float a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t row = row0 + 4 * i + lr;
        const int64_t rown = row < N ? row : N - 1;  // rows past the end: computed, never stored
        wv[i] = load_stream16(reinterpret_cast<const uint4*>(w + rown * K + kw));
        sb[i] = load_stream_u8(signs + rown * kbytes + (kw >> 3));
        a[i] = alpha[per_row ? rown : 0];
    }
    __builtin_amdgcn_sched_barrier(0);  // every load is issued before the rebuild starts

    uint4* tile = tiles[wave];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * i + lr;
        tile[r * kSlGroups + (lg ^ r)] = mask16(recon8(wv[i], sb[i], a[i]), kmask);
    }
    slice_wave_sync();
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < kSlSub / 32; ++t) {
        const int g = 4 * t + grp;
        const bf16x8_t b = as_bf16x8(tile[col * kSlGroups + (g ^ col)]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xv[t]), b, acc, 0, 0, 0);
    }
    slice_wave_sync();

    // D layout: lane l holds column l % 16 (row of the block) and token rows
    // 4 (l / 16) + e.  Each wave parks its sums in its own LDS tile, whose
    // reads above came first in this wave's order.
    float* mine = reinterpret_cast<float*>(tile);  // [e][lane]
#pragma unroll
    for (int e = 0; e < 4; ++e) mine[e * 64 + lane] = acc[e];
    __syncthreads();
    if (threadIdx.x < 16 * kSlRows) {
        const int m = threadIdx.x / kSlRows, nl = threadIdx.x % kSlRows;
        const int src = nl + 16 * (m / 4), e = m % 4;
        float s = 0.0f;
#pragma unroll
        for (int v = 0; v < kSlWaves; ++v) s += reinterpret_cast<const float*>(tiles[v])[e * 64 + src];
        const int64_t n = row0 + nl;
        if (m < M && n < N) {
            if (nslices == 1)
                store_y(y, (int64_t)m * N + n, s);
            else
                part[(slice * M + m) * N + n] = s;
        }
    }
}

// y[e] = sum of the planes' element e, in plane order.  Four adjacent
// elements per lane with 16-byte loads when M·N is a multiple of 4.  The
// planes are loaded kSumBatch at a time, all in flight together, so a call
// pays about one memory latency per batch instead of one per plane: a plane
// index past the last repeats the last plane, and that copy is added as -0
// (x + -0 = x for every x, signed zeros included).
constexpr int kSumBatch = 8;

__device__ __forceinline__ float keep_or_negzero(float v, uint32_t q) {
    return __uint_as_float((__float_as_uint(v) & q) | (0x80000000u & ~q));
}

template <bool kVec>
__global__ __launch_bounds__(256) void slice_sum_kernel(const float* __restrict__ part, int nslices, int64_t MN,
                                                        YOut y) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    const int64_t items = kVec ? MN / 4 : MN;
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < items; q += stride) {
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int p0 = 0; p0 < nslices; p0 += kSumBatch) {
            float4 v[kSumBatch];
#pragma unroll
            for (int i = 0; i < kSumBatch; ++i) {
                const int64_t p = p0 + i < nslices ? p0 + i : nslices - 1;
                if (kVec)
                    v[i] = reinterpret_cast<const float4*>(part + p * MN)[q];
                else
                    v[i] = make_float4(part[p * MN + q], 0.f, 0.f, 0.f);
            }
            __builtin_amdgcn_sched_barrier(0);  // the batch's loads are all issued before the adds
#pragma unroll
            for (int i = 0; i < kSumBatch; ++i) {
                const uint32_t k = p0 + i < nslices ? 0xffffffffu : 0u;
                const float4 t = make_float4(keep_or_negzero(v[i].x, k), keep_or_negzero(v[i].y, k),
                                             keep_or_negzero(v[i].z, k), keep_or_negzero(v[i].w, k));
                if (i == 0) {
                    s = p0 == 0 ? t : make_float4(s.x + t.x, s.y + t.y, s.z + t.z, s.w + t.w);
                } else {
                    s = make_float4(s.x + t.x, s.y + t.y, s.z + t.z, s.w + t.w);
                }
            }
        }
        if (kVec) {
            store_y(y, 4 * q, s.x);
            store_y(y, 4 * q + 1, s.y);
            store_y(y, 4 * q + 2, s.z);
            store_y(y, 4 * q + 3, s.w);
        } else {
            store_y(y, q, s.x);
        }
    }
}

}  // namespace

int64_t slice_count(int64_t K) { return (K + kSlWidth - 1) / kSlWidth; }

size_t slice_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const int64_t s = slice_count(K);
    return s > 1 ? (size_t)s * (size_t)M * (size_t)N * sizeof(float) : 0;
}

const char* slice_name() { return "slice_kernel"; }

hipError_t launch_slice(const uint16_t* x, const uint16_t* w, const uint8_t* signs, const float* alpha,
                        bool per_row, YOut y, int64_t M, int64_t N, int64_t K, void* workspace,
                        hipStream_t stream) {
    if (M < 1 || M > kSliceMaxM || K >= kSliceMaxK) return hipErrorInvalidValue;
    const int64_t ns = slice_count(K);
    if (ns > 1 && !workspace) return hipErrorInvalidValue;
    const int64_t blocks = (N + kSlRows - 1) / kSlRows * ns;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    float* part = static_cast<float*>(workspace);
    hipLaunchKernelGGL(slice_kernel, dim3((unsigned)blocks), dim3(kSlWaves * 64), 0, stream, x, w, signs, alpha,
                       per_row ? 1 : 0, part, y, M, N, K, (int)ns);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ns == 1) return e;
    const int64_t MN = M * N;
    const bool vec = (MN & 3) == 0;
    const int64_t items = vec ? MN / 4 : MN;
    int64_t grid = (items + 255) / 256;
    if (grid > 4096) grid = 4096;
    if (vec)
        hipLaunchKernelGGL(slice_sum_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream, part, (int)ns, MN, y);
    else
        hipLaunchKernelGGL(slice_sum_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream, part, (int)ns, MN, y);
    return hipGetLastError();
}

}  // namespace bd
