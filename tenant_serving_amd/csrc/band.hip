// Decode path for 4..16 tokens on projections whose rows hold 4097..8192
// weights (2048 or more rows; the dispatch picks the shapes where it wins):
// the band kernel.
//
// Definition as in the other linear paths ("BitDelta : servir 14 modèles Zen
// depuis un seul cluster GPU", hanzo-blog 2026-02-28, "Serving
// architecture": base weights and delta bits read together, W_eff rebuilt on
// chip and never stored to HBM, then multiplied).
//
// Reads.  A workgroup of 16 waves, one per compute unit, walks bands of 4
// consecutive rows (bands b, b + G, ... for G workgroups), and wave w takes
// the 512-wide chunk w of every band: per band the workgroup reads its 4 rows
// whole (4 x 16 KiB contiguous at d_in = 8192), each wave one 1 KiB piece per
// row and the 64 matching sign bytes.  Plain-read probes put this pattern at
// 6.3-6.5 TB/s, against 5.4-5.9 for waves that each walk their own rows.
//
// x.  A wave always works on the same chunk, so its x fragment (16 token rows
// x 512, the A operand of v_mfma_f32_16x16x32_bf16 over 16 k-steps) is loaded
// once per call and stays in registers.
//
// Products.  The wave rebuilds its 4 row pieces into a wave-private LDS tile
// and reads them back in the B layout (columns 4..15 repeat rows 0..3; their
// outputs are dropped).  The next band's loads go out as soon as the current
// band is rebuilt, one band in flight per wave.
//
// Sums.  Each wave writes its partial sums of each band (the first mp token
// rows x 4 rows, mp = M rounded up to 4) into LDS slots of its own, with no
// workgroup barrier until the end; then the 16 slots of each band are added
// in wave order and y is written.  64 KiB of slots hold 16384 / (64 mp)
// bands per workgroup: 64 at four tokens, 16 at sixteen.  The sums are in a
// fixed order, so the result is run-to-run reproducible.
#include "bd_device.h"
#include "bd_internal.h"

namespace bd {
namespace {

constexpr int kBWaves = 16;
constexpr int kBChunk = 512;
constexpr int kBGroups = kBChunk / 8;   // 16-byte groups per chunk row
constexpr int kBSlotFloats = 16384;     // 64 KiB of partial-sum slots

__device__ __forceinline__ void band_wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(kBWaves * 64) void band_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, const uint8_t* __restrict__ signs,
    const float* __restrict__ alpha, int per_row, YOut y, int64_t M, int64_t N, int64_t K) {
    __shared__ uint4 tiles[kBWaves][4 * kBGroups];  // 64 KiB: the wave's 4 row pieces
    __shared__ float part[kBSlotFloats];            // [band][wave][token][row], token rows < mp

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, grp = lane >> 4, c3 = col & 3;
    const int64_t nbands = (N + 3) / 4;
    const int64_t G = gridDim.x;
    const int nb = (int)((nbands - (int64_t)blockIdx.x + G - 1) / G);  // >= 1: the grid is at most nbands
    const int64_t nchunks = (K + kBChunk - 1) / kBChunk;                // at most kBWaves
    const int64_t kbytes = K / 8;
    const int tok = col < M ? col : 0;     // token rows >= M repeat token 0 (outputs dropped)
    const int mp = (int)((M + 3) & ~3);    // token rows kept per band
    const int bstride = kBWaves * 4 * mp;  // floats per band in `part`
    uint4* tile = tiles[wave];
    const bool act = wave < nchunks;       // uniform per wave
    const int64_t kl = (int64_t)wave * kBChunk + 8 * lane;
    const bool kok = act && kl < K;
    const int64_t kw = kok ? kl : 0;  // lanes past K, or of an idle wave, read column 0, zeroed at the use

    // loads of band `band` (rows past N repeat row N-1, never stored); an idle
    // wave, or a band past the last, reads the first 16 bytes of x instead
    uint4 wv[4];
    uint32_t sb[4];
    auto load = [&](int64_t band, bool real) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = 4 * band + r < N ? 4 * band + r : N - 1;
            const bool rl = real && act;
            const uint4* wp = rl ? reinterpret_cast<const uint4*>(w + row * K + kw) : reinterpret_cast<const uint4*>(x);
            const uint8_t* sp = rl ? signs + row * kbytes + (kw >> 3) : reinterpret_cast<const uint8_t*>(x);
            wv[r] = load_stream16(wp);
            sb[r] = load_stream_u8(sp);
        }
    };

    load(blockIdx.x, true);
    // x fragment of this wave's chunk: k-step s, token tok, k = 512 wave + 32 s + 8 grp (zero past K)
    uint4 xv[kBChunk / 32];
#pragma unroll
    for (int s = 0; s < kBChunk / 32; ++s) {
        const int64_t kx = (int64_t)wave * kBChunk + 32 * s + 8 * grp;
        xv[s] = (act && kx < K) ? *reinterpret_cast<const uint4*>(x + tok * K + kx) : make_uint4(0, 0, 0, 0);
    }

    for (int i = 0; i < nb; ++i) {
        const int64_t band = (int64_t)blockIdx.x + (int64_t)i * G;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        if (act) {  // uniform
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = 4 * band + r < N ? 4 * band + r : N - 1;
                const uint4 e = recon8(wv[r], sb[r], alpha[per_row ? row : 0]);
                tile[r * kBGroups + (lane ^ r)] = kok ? e : make_uint4(0, 0, 0, 0);
            }
        }
        // the next band's loads go out as soon as this one is in the tile
        load(band + G, i + 1 < nb);
        if (act) {
            band_wave_sync();
#pragma unroll
            for (int s = 0; s < kBChunk / 32; ++s) {
                const int g = 4 * s + grp;
                const bf16x8_t b = as_bf16x8(tile[c3 * kBGroups + (g ^ c3)]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xv[s]), b, acc, 0, 0, 0);
            }
            band_wave_sync();
        }
        // D layout: lane l holds column l % 16 (row (l % 16) % 4 of the band)
        // and token rows 4 (l / 16) + e; columns 0..3 are the band's rows
        float* slot = part + i * bstride + wave * 4 * mp;
        if (col < 4 && 4 * grp < mp) {
#pragma unroll
            for (int e = 0; e < 4; ++e) slot[(4 * grp + e) * 4 + col] = acc[e];
        }
    }

    // the 16 waves' partial sums of every band, added in wave order
    __syncthreads();
    const int per_band = 4 * mp;
    for (int e = threadIdx.x; e < nb * per_band; e += kBWaves * 64) {
        const int i = e / per_band, o = e % per_band;
        float sum = 0.0f;
#pragma unroll
        for (int v = 0; v < kBWaves; ++v) sum += part[i * bstride + v * per_band + o];
        const int t = o >> 2;
        const int64_t n = 4 * ((int64_t)blockIdx.x + (int64_t)i * G) + (o & 3);
        if (t < M && n < N) store_y(y, (int64_t)t * N + n, sum);
    }
}

}  // namespace

int64_t band_grid(int64_t M, int64_t N, int64_t K, int num_cu) {
    if (M < 1 || M > kBandMaxM || N < 1 || K < 8 || K > kBandMaxK || num_cu < 1) return 0;
    const int64_t nbands = (N + 3) / 4;
    const int64_t grid = nbands < num_cu ? nbands : num_cu;
    const int64_t mp = (M + 3) & ~int64_t(3);
    const int64_t per = (nbands + grid - 1) / grid;
    return per * kBWaves * 4 * mp <= kBSlotFloats ? grid : 0;
}

const char* band_name() { return "band_kernel"; }

hipError_t launch_band(const uint16_t* x, const uint16_t* w, const uint8_t* signs, const float* alpha,
                       bool per_row, YOut y, int64_t M, int64_t N, int64_t K, int num_cu, hipStream_t stream) {
    const int64_t grid = band_grid(M, N, K, num_cu);
    if (grid == 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(band_kernel, dim3((unsigned)grid), dim3(kBWaves * 64), 0, stream, x, w, signs, alpha,
                       per_row ? 1 : 0, y, M, N, K);
    return hipGetLastError();
}

}  // namespace bd
