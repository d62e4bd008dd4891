// Decode path on MFMA (2 <= M <= 16 tokens) for projections with many rows:
// the x-stationary streaming kernel.
//
// Definition as in the other linear paths ("BitDelta : servir 14 modèles Zen
// depuis un seul cluster GPU", hanzo-blog 2026-02-28, "Serving
// architecture": base weights and delta bits read together, W_eff rebuilt on
// chip and never stored to HBM, then multiplied).
//
// At decode the whole cost is streaming W_base (2 bytes per weight) and the
// sign planes (1/8 byte).  What limits a streaming kernel on gfx950 once
// M > 1 is not HBM but the vector memory path: if every wave reloads x for
// every chunk it multiplies, those cache hits queue with the weight stream
// (measured: 16 such loads per 8 KiB of weights halve the stream rate).  So
// here x is read from LDS, where it sits one K range at a time, and the
// weights are the only traffic on the vector memory path.
//
// Layout of the work.  A workgroup is 8 waves in two teams of 4 and owns
// 2·R row groups of 8 rows (team t takes the groups with odd or even slot
// numbers).  The K axis is cut into ranges whose x slice [M, range] fits the
// LDS buffer; for each range the workgroup copies the slice into LDS, then
// each team walks its R row groups, and within a group the 4 waves of the
// team split the range's 512-wide chunks (chunk c goes to wave c mod 4).  A
// wave therefore keeps one accumulator tile per row group it owns (R tiles,
// registers), across all ranges; after the last range the 4 waves of a
// team add their tiles in LDS in a fixed order and write y.  One CU thus
// streams 16 rows at a time, 1 KiB per row per load instruction, with no
// barrier inside a range, which is the pattern that streams fastest here;
// the next item's loads are always in flight while the current one is
// rebuilt and multiplied, including across the range switch.
//
// The multiply: the item's 8 rows are rebuilt (recon8) into a wave-private
// LDS tile and read back in the B layout of v_mfma_f32_16x16x32_bf16 (B
// columns 8..15 are zero; the MFMA has ample headroom at decode); the A
// operand is x from the LDS slice, zero for token rows >= M.
#include "bd_device.h"
#include "bd_internal.h"

namespace bd {
namespace {

constexpr int kChunk = 512;    // k per row load instruction: 64 lanes x 8
constexpr int kGroups = 64;    // 16-byte groups per chunk row
constexpr int kItemRows = 8;   // rows per row group
constexpr int kWaves = 8;      // two teams of 4
constexpr int kTeam = 4;
constexpr int kXsUints = kXstatXsBytes / 16;

// LDS position of 16-byte group g of x row t (row stride `stride` groups):
// the low 3 bits of the group are XORed with the row, so the 8 token rows an
// operand load reads at one k land in 8 different 16-byte bank groups.
__device__ __forceinline__ int xs_pos(int t, int g, int stride) { return t * stride + (g ^ (t & 7)); }
__device__ __forceinline__ int wt_pos(int r, int g) { return r * kGroups + (g ^ r); }

// Orders a wave's own LDS stores before its loads of other lanes' data (and
// those loads before the next stores): only a wait, no barrier.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One work item: 8 rows x one 512-wide chunk, with the rows' α (uniform
// across the wave, so scalar loads into scalar registers).
struct Item {
    uint4 w[kItemRows];
    uint32_t s[kItemRows];
    float a[kItemRows];
};

template <int R>
__global__ __launch_bounds__(kWaves * 64) void xstat_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const uint8_t* __restrict__ signs, const float* __restrict__ alpha, int per_row,
    YOut y, int64_t M, int64_t N, int64_t K, int krc, int nkr) {
    __shared__ uint4 xs[kXsUints];
    __shared__ uint4 wt[kWaves][kItemRows * kGroups];

    const int lane = threadIdx.x & 63;
    // wave-uniform indices (readfirstlane lets the compiler keep row
    // addresses and α in scalar registers)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int team = wave / kTeam, u = wave % kTeam;
    const int col = lane & 15, grp = lane >> 4;
    const int64_t nchunks = (K + kChunk - 1) / kChunk;
    const int64_t groups_total = (N + kItemRows - 1) / kItemRows;
    const int64_t kbytes = K / 8;
    const int stride = krc * kGroups;  // x row stride in LDS, 16-byte groups

    // Row group of slot j of this wave's team (slots 2j + team of the
    // workgroup, strided by the grid).  Groups past the end are computed on
    // row N-1 and never stored.
    auto group_of = [&](int j) { return (int64_t)blockIdx.x + (int64_t)gridDim.x * (2 * j + team); };
    // Chunks of range r handled by this wave: c_begin + u, + 4, ...
    auto range_chunks = [&](int64_t r) {
        const int64_t b = r * krc, e = (b + krc < nchunks ? b + krc : nchunks);
        return e - b > u ? (e - b - u + kTeam - 1) / kTeam : (int64_t)0;
    };

    // Item (r, cc, j): range r, this wave's cc-th chunk of it, slot j.  One
    // uniform base per row group and 32-bit per-lane offsets, so a row costs
    // no scalar registers of its own.  Every load is in bounds and
    // unconditional (rows past N repeat row N-1 and are never stored; lanes
    // past K read the row's last 8 weights, zeroed later), so that one slot of
    // the pipeline is one basic block.
    auto load = [&](Item& it, int64_t r, int64_t cc, int j) {
        const int64_t c = r * krc + u + (int64_t)kTeam * cc;
        int64_t k = c * kChunk + 8 * lane;
        k = k < K ? k : K - 8;
        const int64_t g = group_of(j);
        const int64_t row0 = g * kItemRows < N ? g * kItemRows : N - 1;
        const int64_t last = N - 1 - row0;  // rows of the group that exist, minus one
        const char* wb = reinterpret_cast<const char*>(w + row0 * K);
        const uint8_t* sb = signs + row0 * kbytes;
#pragma unroll
        for (int i = 0; i < kItemRows; ++i) {
            const uint32_t ri = (uint32_t)(i < last ? i : last);
            const uint32_t wo = ri * (uint32_t)(K * 2) + (uint32_t)(k * 2);
            const uint32_t so = ri * (uint32_t)kbytes + (uint32_t)(k >> 3);
            it.w[i] = load_stream16(reinterpret_cast<const uint4*>(wb + wo));
            it.s[i] = load_stream_u8(sb + so);
            it.a[i] = alpha[per_row ? row0 + ri : 0];
        }
    };

    f32x4_t acc[R];
#pragma unroll
    for (int j = 0; j < R; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Operand addresses.  B (the rebuilt rows): lane reads tile row c7 =
    // col & 7 (columns 8..15 repeat rows 0..7; their outputs are dropped) at
    // 16-byte group gb = 4s + grp, stored at gb ^ c7.  A (x): token row
    // col, or row 0 for col >= M (those outputs are dropped too).  Because
    // (4s + grp) ^ c = 4(s ^ (c >> 2)) + (grp ^ (c & 3)), the position is a
    // per-lane base plus 4s, with one base for even and one for odd s.
    uint4* tile = wt[wave];
    const int c7 = col & 7;
    const int wq = grp ^ (c7 & 3), wsel = c7 >> 2;
    const int w_even = c7 * kGroups + 4 * wsel + wq, w_odd = c7 * kGroups - 4 * wsel + wq;
    const int tx = col < M ? col : 0, t7 = tx & 7;
    const int xq = grp ^ (t7 & 3), xsel = t7 >> 2;
    const int x_even = tx * stride + 4 * xsel + xq, x_odd = tx * stride - 4 * xsel + xq;

    auto compute = [&](const Item& it, int j, int cl, bool ragged) {
        uint4 e[kItemRows];
#pragma unroll
        for (int i = 0; i < kItemRows; ++i) e[i] = recon8(it.w[i], it.s[i], it.a[i]);
        if (ragged) {  // uniform: the range's last chunk runs past K
            const bool kok = (int64_t)(nchunks - 1) * kChunk + 8 * lane < K;
#pragma unroll
            for (int i = 0; i < kItemRows; ++i) e[i] = kok ? e[i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < kItemRows; ++i) tile[wt_pos(i, lane)] = e[i];
        wave_lds_sync();
        const int xo = cl * kGroups;
#pragma unroll
        for (int s = 0; s < kChunk / 32; ++s) {
            const bf16x8_t b = as_bf16x8(tile[(s & 1 ? w_odd : w_even) + 4 * s]);
            const bf16x8_t xa = as_bf16x8(xs[(s & 1 ? x_odd : x_even) + xo + 4 * s]);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, b, acc[j], 0, 0, 0);
        }
        wave_lds_sync();
    };

    // x[:, range r] -> LDS (zero past K); rows >= M are never read.
    auto load_x = [&](int64_t r) {
        const int mrows = (int)M;
        for (int e = threadIdx.x; e < mrows * stride; e += kWaves * 64) {
            const int t = e / stride, g = e % stride;
            const int64_t k = (r * krc * kGroups + g) * 8;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (k < K) v = *reinterpret_cast<const uint4*>(x + t * K + k);
            xs[xs_pos(t, g, stride)] = v;
        }
    };

    const bool k_ragged = K % kChunk != 0;
    Item cur;
    load(cur, 0, 0, 0);
    for (int64_t r = 0; r < nkr; ++r) {
        if (r > 0) __syncthreads();  // every wave is done with the previous slice
        load_x(r);
        __syncthreads();
        const int64_t ncc = range_chunks(r);
        for (int64_t cc = 0; cc < ncc; ++cc) {
            const int cl = u + kTeam * (int)cc;  // chunk index within the range
            const bool ragged = k_ragged && r * krc + cl == nchunks - 1;
#pragma unroll
            for (int j = 0; j < R; ++j) {
                // the following item: next slot, else next chunk, else the
                // first chunk of the next range (after the very last item this
                // reloads the first one, which is never used)
                int64_t rn = r, ccn = cc;
                int jn = j + 1;
                if (j + 1 == R) {
                    jn = 0;
                    const bool next_range = cc + 1 >= ncc;
                    ccn = next_range ? 0 : cc + 1;
                    rn = next_range ? (r + 1 < nkr ? r + 1 : 0) : r;
                }
                Item nxt;
                load(nxt, rn, ccn, jn);
                compute(cur, j, cl, ragged);
                cur = nxt;
            }
        }
    }

    // Add the 4 waves of each team in a fixed order and write y.  D layout of
    // the 16x16 MFMA: lane holds column n = lane%16 (rows 0..7 of the group),
    // token rows 4·(lane/16) + e.
    __syncthreads();
    float* red = reinterpret_cast<float*>(xs);  // [team][u][R][4][64]
    static_assert(kWaves * R * 4 * 64 * 4 <= kXstatXsBytes, "reduction buffer exceeds the x slice");
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[(((team * kTeam + u) * R + j) * 4 + e) * 64 + lane] = acc[j][e];
    __syncthreads();
    for (int j = u; j < R; j += kTeam) {
        const int64_t n = group_of(j) * kItemRows + col;
        if (col >= kItemRows || n >= N || group_of(j) >= groups_total) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t m = 4 * grp + e;
            if (m >= M) continue;
            float s = 0.0f;
#pragma unroll
            for (int v = 0; v < kTeam; ++v) s += red[(((team * kTeam + v) * R + j) * 4 + e) * 64 + lane];
            store_y(y, m * N + n, s);
        }
    }
}

template <int R>
hipError_t launch_r(const uint16_t* x, const uint16_t* w, const uint8_t* signs, const float* alpha,
                    bool per_row, YOut y, int64_t M, int64_t N, int64_t K, const XstatPlan& p,
                    hipStream_t stream) {
    hipLaunchKernelGGL((xstat_kernel<R>), dim3((unsigned)p.grid), dim3(kWaves * 64), 0, stream, x, w,
                       signs, alpha, per_row ? 1 : 0, y, M, N, K, p.krc, p.nkr);
    return hipGetLastError();
}

}  // namespace

const char* xstat_name(int64_t M, int64_t N, int64_t K, int num_cu) {
    static const char* const names[kXstatMaxR] = {
        "xstat_kernel<1>", "xstat_kernel<2>", "xstat_kernel<3>", "xstat_kernel<4>",
        "xstat_kernel<5>", "xstat_kernel<6>", "xstat_kernel<7>", "xstat_kernel<8>"};
    const XstatPlan p = xstat_plan(M, N, K, num_cu);
    return p.r >= 1 && p.r <= kXstatMaxR ? names[p.r - 1] : "";
}

hipError_t launch_xstat(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                        const float* alpha, bool per_row, YOut y, int64_t M, int64_t N,
                        int64_t K, int num_cu, hipStream_t stream) {
    const XstatPlan p = xstat_plan(M, N, K, num_cu);
    switch (p.r) {
        case 1: return launch_r<1>(x, w, signs, alpha, per_row, y, M, N, K, p, stream);
        case 2: return launch_r<2>(x, w, signs, alpha, per_row, y, M, N, K, p, stream);
        case 3: return launch_r<3>(x, w, signs, alpha, per_row, y, M, N, K, p, stream);
        case 4: return launch_r<4>(x, w, signs, alpha, per_row, y, M, N, K, p, stream);
        case 5: return launch_r<5>(x, w, signs, alpha, per_row, y, M, N, K, p, stream);
        case 6: return launch_r<6>(x, w, signs, alpha, per_row, y, M, N, K, p, stream);
        case 7: return launch_r<7>(x, w, signs, alpha, per_row, y, M, N, K, p, stream);
        case 8: return launch_r<8>(x, w, signs, alpha, per_row, y, M, N, K, p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace bd
