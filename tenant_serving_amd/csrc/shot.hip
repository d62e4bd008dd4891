// Decode path for projections with few rows (up to 16 tokens): one-shot
// workgroups.
//
// Definition as in the other linear paths ("BitDelta : servir 14 modèles Zen
// depuis un seul cluster GPU", hanzo-blog 2026-02-28, "Serving
// architecture": base weights and delta bits read together, W_eff rebuilt on
// chip and never stored to HBM, then multiplied).
//
// A projection like k or v of a 70B layer (1024 rows x 8192) is 18 MB: at
// HBM speed a few microseconds, so what counts is issuing all of it at once.
// A workgroup of 16 waves owns 4 rows; wave w takes the 512-wide K chunks w,
// w + 16, ... (for d_in = 8192 exactly one), loads its 4 row pieces (1 KiB
// each), their sign bytes and the x fragments of its chunk together, rebuilds
// the rows into a wave-private LDS tile and multiplies on
// v_mfma_f32_16x16x32_bf16 (B columns 4..15 repeat rows 0..3, A rows past the
// M tokens are zero; those outputs are dropped).  The 16 waves' partial sums
// meet in LDS once, added in a fixed order.  With 1024 rows that is 256
// workgroups, one per CU, and the whole matrix in flight at the start.
#include "bd_device.h"
#include "bd_internal.h"

namespace bd {
namespace {

constexpr int kShotChunk = 512;
constexpr int kShotGroups = 64;
constexpr int kShotRows = 4;       // rows per workgroup
constexpr int kShotWaves = 16;

__device__ __forceinline__ void shot_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(kShotWaves * 64) void shot_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const uint8_t* __restrict__ signs, const float* __restrict__ alpha, int per_row,
    YOut y, int64_t M, int64_t N, int64_t K) {
    __shared__ uint4 tiles[kShotWaves][kShotRows * kShotGroups];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const int64_t row0 = (int64_t)blockIdx.x * kShotRows;
    const int64_t nchunks = (K + kShotChunk - 1) / kShotChunk;
    const int64_t kbytes = K / 8;
    uint4* tile = tiles[wave];

    float a[kShotRows];
    int64_t rown[kShotRows];
#pragma unroll
    for (int i = 0; i < kShotRows; ++i) {
        rown[i] = row0 + i < N ? row0 + i : N - 1;  // rows past the end: computed, never stored
        a[i] = alpha[per_row ? rown[i] : 0];
    }
    const int c3 = col & 3;

    const rsrc_t xr = make_rsrc(x, (uint32_t)(M * K * 2));
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int64_t c = wave; c < nchunks; c += kShotWaves) {
        const int64_t kl = c * kShotChunk + 8 * lane;  // this lane's 8 weights of each row
        const bool kok = kl < K;
        const int64_t k = kok ? kl : K - 8;
        uint4 wv[kShotRows];
        uint32_t sb[kShotRows];
#pragma unroll
        for (int i = 0; i < kShotRows; ++i) {
            wv[i] = load_stream16(reinterpret_cast<const uint4*>(w + rown[i] * K + k));
            sb[i] = load_stream_u8(signs + rown[i] * kbytes + (k >> 3));
        }
        // x fragments of the chunk: k-step s covers k 32s .. 32s+31, this lane
        // token `col`, k 32s + 8·grp .. +8, through a buffer resource that ends
        // with x: lanes of token rows >= M and k past K read past its end,
        // which returns zeros and touches no memory
        uint4 xv[kShotChunk / 32];
#pragma unroll
        for (int s = 0; s < kShotChunk / 32; ++s) {
            const int64_t kx = c * kShotChunk + 32 * s + 8 * grp;
            const uint32_t off = (col < M && kx < K) ? (uint32_t)((col * K + kx) * 2) : 0x80000000u;
            xv[s] = buf_load16(xr, off, 0);
        }
        __builtin_amdgcn_sched_barrier(0);  // every load is issued before the rebuild starts
#pragma unroll
        for (int i = 0; i < kShotRows; ++i) {
            uint4 e = recon8(wv[i], sb[i], a[i]);
            tile[i * kShotGroups + (lane ^ i)] = kok ? e : make_uint4(0, 0, 0, 0);
        }
        shot_lds_sync();
#pragma unroll
        for (int s = 0; s < kShotChunk / 32; ++s) {
            const int g = 4 * s + grp;
            const bf16x8_t b = as_bf16x8(tile[c3 * kShotGroups + (g ^ c3)]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xv[s]), b, acc, 0, 0, 0);
        }
        shot_lds_sync();
    }

    // Partial sums of the 16 waves, added in wave order.  D layout: lane l
    // holds column l%16 (rows 0..3 of the group are columns 0..3) and token
    // rows 4·(l/16) + e.
    __syncthreads();
    float* red = reinterpret_cast<float*>(&tiles[0][0]);  // [wave][4][64]
#pragma unroll
    for (int e = 0; e < 4; ++e) red[(wave * 4 + e) * 64 + lane] = acc[e];
    __syncthreads();
    if (threadIdx.x < 16 * kShotRows) {
        const int m = threadIdx.x / kShotRows, nl = threadIdx.x % kShotRows;
        const int src = nl + 16 * (m / 4), e = m % 4;
        float s = 0.0f;
        for (int v = 0; v < kShotWaves; ++v) s += red[(v * 4 + e) * 64 + src];
        const int64_t n = row0 + nl;
        if (m < M && n < N) store_y(y, (int64_t)m * N + n, s);
    }
}

}  // namespace

const char* shot_name() { return "shot_kernel"; }

hipError_t launch_shot(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                       const float* alpha, bool per_row, YOut y, int64_t M, int64_t N, int64_t K,
                       hipStream_t stream) {
    if (M > 16 || K >= kShotMaxK) return hipErrorInvalidValue;
    const int64_t blocks = (N + kShotRows - 1) / kShotRows;
    hipLaunchKernelGGL(shot_kernel, dim3((unsigned)blocks), dim3(kShotWaves * 64), 0, stream, x, w, signs,
                       alpha, per_row ? 1 : 0, y, M, N, K);
    return hipGetLastError();
}

}  // namespace bd
