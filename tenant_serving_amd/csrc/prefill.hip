// Prefill path: LDS-tiled bf16 MFMA with on-the-fly sign unpacking.
//
// "BitDelta : servir 14 modèles Zen depuis un seul cluster GPU" (hanzo-blog,
// 2026-02-28), "Serving architecture": reconstruction and matrix product in
// one kernel pass, W_eff rebuilt in registers or on-chip memory and never
// stored to HBM.  Here each BN x 64 tile of W_base and its sign bytes are
// loaded once per workgroup, rebuilt into bf16 W_eff by recon8, written to
// LDS, and consumed together with the BM x 64 tile of x by
// v_mfma_f32_32x32x16_bf16.  Rebuilding is paid once per (M-tile, weight),
// so tall M-tiles keep it a small fraction of the MFMA time.  Global loads
// of step s+1 are issued before the MFMAs of step s.
//
// LDS rows are 128 bytes (64 bf16); the 16-byte chunk index is XOR-swizzled
// with the row so that the 32 rows read by one MFMA operand load spread over
// the banks.
#include "bd_device.h"
#include "bd_internal.h"

namespace bd {
namespace {

constexpr int kBK = 64;

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void prefill_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const uint8_t* __restrict__ signs, const float* __restrict__ alpha, int per_row,
    float* __restrict__ y, int64_t M, int64_t N, int64_t K, int tiles_n) {
    constexpr int NT = 64 * WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
    constexpr int TM = WTM / 32, TN = WTN / 32;  // 32x32 MFMA tiles per wave
    constexpr int ACH = BM * 8 / NT;             // 16-byte chunks of x per thread per step
    constexpr int BCH = BN * 8 / NT;             // 16-byte chunks of W per thread per step
    static_assert(ACH * NT == BM * 8 && BCH * NT == BN * 8, "tile/thread mismatch");

    __shared__ uint4 As[BM * 8];
    __shared__ uint4 Bs[BN * 8];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // Tiles of one M-row band are consecutive block ids, so concurrently
    // running workgroups share x rows in L2.
    const int64_t tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
    const int64_t m0 = tm * BM, n0 = tn * BN;
    const int64_t kbytes = K / 8;
    const int64_t nsteps = (K + kBK - 1) / kBK;

    // Fixed per-thread load slots.
    const uint16_t* aptr[ACH];
    bool arow_ok[ACH];
    int aslot[ACH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        int q = tid + i * NT, row = q >> 3, c = q & 7;
        int64_t gm = m0 + row;
        arow_ok[i] = gm < M;
        aptr[i] = x + (arow_ok[i] ? gm : 0) * K + c * 8;
        aslot[i] = swz(row, c);
    }
    const uint16_t* bptr[BCH];
    const uint8_t* sptr[BCH];
    float balpha[BCH];
    int bslot[BCH];
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
        int q = tid + i * NT, row = q >> 3, c = q & 7;
        int64_t gn = n0 + row < N ? n0 + row : N - 1;  // rows past N: computed, never stored
        bptr[i] = w + gn * K + c * 8;
        sptr[i] = signs + gn * kbytes + c;
        balpha[i] = alpha[per_row ? gn : 0];
        bslot[i] = swz(row, c);
    }

    uint4 ra[ACH], rb[BCH];
    uint32_t rs[BCH];
    auto load_step = [&](int64_t s) {
        const int64_t k0 = s * kBK;
#pragma unroll
        for (int i = 0; i < ACH; ++i) {
            int c = (tid + i * NT) & 7;
            bool ok = arow_ok[i] && k0 + c * 8 < K;
            ra[i] = ok ? *reinterpret_cast<const uint4*>(aptr[i] + k0) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < BCH; ++i) {
            int c = (tid + i * NT) & 7;
            bool ok = k0 + c * 8 < K;
            rb[i] = ok ? load_stream16(reinterpret_cast<const uint4*>(bptr[i] + k0))
                       : make_uint4(0, 0, 0, 0);
            rs[i] = ok ? load_stream_u8(sptr[i] + k0 / 8) : 0u;
        }
    };

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    load_step(0);
    for (int64_t s = 0; s < nsteps; ++s) {
#pragma unroll
        for (int i = 0; i < ACH; ++i) As[aslot[i]] = ra[i];
#pragma unroll
        for (int i = 0; i < BCH; ++i) Bs[bslot[i]] = recon8(rb[i], rs[i], balpha[i]);
        __syncthreads();
        if (s + 1 < nsteps) load_step(s + 1);

        const int r32 = lane & 31, half = lane >> 5;
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            const int chunk = 2 * kk + half;
            bf16x8_t af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) af[i] = as_bf16x8(As[swz(wm * WTM + i * 32 + r32, chunk)]);
#pragma unroll
            for (int j = 0; j < TN; ++j) bfr[j] = as_bf16x8(Bs[swz(wn * WTN + j * 32 + r32, chunk)]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }

    // D layout of the 32x32 MFMA: register r of lane l is row
    // 8·(r/4) + 4·(l/32) + r%4, column l%32.
    const int col = lane & 31, half = lane >> 5;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            int64_t n = n0 + wn * WTN + j * 32 + col;
            if (n >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int64_t m = m0 + wm * WTM + i * 32 + 8 * (r / 4) + 4 * half + (r % 4);
                if (m < M) y[m * N + n] = acc[i][j][r];
            }
        }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                      const float* alpha, bool per_row, float* y, int64_t M, int64_t N, int64_t K,
                      hipStream_t stream) {
    int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    dim3 grid((unsigned)(tiles_m * tiles_n)), block(64 * WM * WN);
    hipLaunchKernelGGL((prefill_kernel<BM, BN, WM, WN>), grid, block, 0, stream, x, w, signs,
                       alpha, per_row ? 1 : 0, y, M, N, K, (int)tiles_n);
    return hipGetLastError();
}

}  // namespace

const char* prefill_name() { return "prefill_kernel<256,128,4,2>"; }

hipError_t launch_prefill(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                          const float* alpha, bool per_row, float* y, int64_t M, int64_t N,
                          int64_t K, hipStream_t stream) {
    return launch_cfg<256, 128, 4, 2>(x, w, signs, alpha, per_row, y, M, N, K, stream);
}

}  // namespace bd
