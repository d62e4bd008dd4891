// Decode path for two to four tokens on projections with many rows: the
// row-quad kernel.
//
// Definition as in the other linear paths ("BitDelta : servir 14 modèles Zen
// depuis un seul cluster GPU", hanzo-blog 2026-02-28, "Serving
// architecture": base weights and delta bits read together, W_eff rebuilt on
// chip and never stored to HBM, then multiplied).
//
// The weights stream exactly as in the one-token GEMV, which reads at the
// chip's practical rate: a load instruction covers 1 KiB of one row (lane l
// takes weights 8l .. 8l+7 of a 512-wide chunk), with the 64 matching sign
// bytes as one byte load.  With VALU dot products every extra token costs
// 4 v_dot2 per 8 weights, which at four tokens leaves the stream starved.
// Here the products run on v_mfma_f32_4x4x4_16b_bf16 instead: its 16 blocks
// each multiply 4 tokens (A, from the x slice in LDS) by 4 rows (B) over
// 4 k, so a wave works on a quad of 4 rows.  The rebuilt rows go through a
// wave-private LDS tile into the B layout: lane 4b+j of a block holds row j,
// so one 16-byte read per lane and chunk quarter gives 8 weights of its row,
// two MFMAs' worth, at the same k as the x fragment the lane reads for
// token j.  At the end the 16 blocks' partial sums of each (token, row) are
// added with lane shuffles in a fixed order.
//
// Work layout.  One workgroup of 16 waves per compute unit owns a contiguous
// range of row quads.  K is cut into phases whose x slice (4 tokens, at most
// 8192 wide, 64 KiB) sits in LDS; within a phase each quad's chunks are cut
// into S sub-ranges, and the workgroup's (quad, sub-range) units are dealt
// to the waves round robin.  A wave streams its units one after another,
// the next item's loads in flight while the current one is rebuilt and
// multiplied, and adds each unit's 16 partial sums into the unit's slot in
// LDS (one wave per unit, phases in order).  After the last phase the slots
// of each quad are added in sub-range order and y is written.  All sums are
// in fixed orders, so the result is run-to-run reproducible.
#include "bd_device.h"
#include "bd_internal.h"

namespace bd {
namespace {

constexpr int kQWaves = 16;
constexpr int kQChunk = 512;
constexpr int kQPhaseChunks = kQuadPhaseMax / kQChunk;  // 16
constexpr int kQXGroups = kQuadPhaseMax / 8;            // 16-byte groups per token row of the slice
typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma4x4x4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4_t, make_uint2(a0, a1)),
                                                  __builtin_bit_cast(s16x4_t, make_uint2(b0, b1)), c, 0, 0, 0);
}

__device__ __forceinline__ void quad_wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One item: kU chunks of the quad's 4 rows.
template <int kU>
struct QItem {
    uint4 w[kU][4];
    uint32_t s[kU][4];
};

template <int kU>
__global__ __launch_bounds__(kQWaves * 64) void quad_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const uint8_t* __restrict__ signs, const float* __restrict__ alpha, int per_row,
    YOut y, int64_t M, int64_t N, int64_t K, int qpw, int log2s) {
    __shared__ uint4 xs[4 * kQXGroups];            // 64 KiB: the phase's x slice, 4 token rows
    __shared__ uint4 tiles[kQWaves][4 * 64];       // 64 KiB: one 4-row chunk per wave
    __shared__ float red[kQuadMaxUnits * 16];      // partial sums per unit: [token][row]

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 3, b = lane >> 2;
    const int S = 1 << log2s;
    const int64_t nquads = (N + 3) / 4;
    const int64_t qb = (int64_t)blockIdx.x * qpw;
    const int qn = (int)(qb + qpw < nquads ? qpw : nquads - qb);  // quads of this workgroup (grid <= quads)
    const int units = qn << log2s;
    const int64_t kbytes = K / 8;
    const int nchunks = (int)((K + kQChunk - 1) / kQChunk);
    const int nphases = (nchunks + kQPhaseChunks - 1) / kQPhaseChunks;
    uint4* tile = tiles[wave];

    for (int e = threadIdx.x; e < units * 16; e += kQWaves * 64) red[e] = 0.0f;

    // A wave's work is one stream of items: phases in order, within a phase
    // its units u = wave, wave + 16, ..., within a unit its chunks kU at a
    // time.  The next item's loads are always in flight while the current one
    // is rebuilt and multiplied, also across unit and phase switches, so the
    // weight stream starts before the first x slice has landed in LDS.
    struct Unit {
        const char* wrow[4];
        const uint8_t* srow[4];
        float a[4];
        int c0, c1;  // chunks [c0, c1) of the unit
    };
    auto unit_at = [&](int p, int u) {
        Unit un;
        const int64_t q = qb + (u >> log2s);
        const int sr = u & (S - 1);
        const int pb = p * kQPhaseChunks;
        const int pc = nchunks - pb < kQPhaseChunks ? nchunks - pb : kQPhaseChunks;  // chunks of the phase
        un.c0 = pb + pc * sr / S;
        un.c1 = pb + pc * (sr + 1) / S;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = 4 * q + r < N ? 4 * q + r : N - 1;  // rows past N: computed, never stored
            un.wrow[r] = reinterpret_cast<const char*>(w + row * K);
            un.srow[r] = signs + row * kbytes;
            un.a[r] = alpha[per_row ? row : 0];
        }
        return un;
    };
    // item at chunk c of unit un: kU chunks of the 4 rows (chunks at or past
    // c1 are loaded in bounds and never used)
    auto load = [&](QItem<kU>& it, const Unit& un, int c) {
#pragma unroll
        for (int v = 0; v < kU; ++v) {
            int64_t k = (int64_t)(c + v) * kQChunk + 8 * lane;
            k = k < K ? k : K - 8;  // in bounds always; zeroed below when past K
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                it.w[v][r] = load_stream16(reinterpret_cast<const uint4*>(un.wrow[r] + 2 * k));
                it.s[v][r] = load_stream_u8(un.srow[r] + (k >> 3));
            }
        }
    };
    // the wave's units in stream order: (phase, unit) pairs with at least one
    // chunk; next_unit advances (p, u) to the following one, or p = nphases
    auto next_unit = [&](int& p, int& u) {
        for (;;) {
            u += kQWaves;
            if (u >= units) {
                u = wave;
                if (++p >= nphases) return;
            }
            const int pb = p * kQPhaseChunks;
            const int pc = nchunks - pb < kQPhaseChunks ? nchunks - pb : kQPhaseChunks;
            const int sr = u & (S - 1);
            if (pc * (sr + 1) / S > pc * sr / S) return;
        }
    };

    // position of the item in flight: (lp, lu) and chunk lc of unit lun
    int lp = 0, lu = wave - kQWaves;
    if (wave < units) next_unit(lp, lu);
    else lp = nphases;  // a wave without units only meets the barriers
    Unit lun;
    int lc = 0;
    QItem<kU> cur;
    if (lp < nphases) {
        lun = unit_at(lp, lu);
        lc = lun.c0;
        load(cur, lun, lc);
    }

    for (int p = 0; p < nphases; ++p) {
        // x[:, phase p] -> LDS (zero past K and for tokens >= M)
        __syncthreads();  // every wave is done with the previous slice (and red is initialised)
        const int64_t pk = (int64_t)p * kQuadPhaseMax;
        for (int e = threadIdx.x; e < 4 * kQXGroups; e += kQWaves * 64) {
            const int t = e / kQXGroups, g = e % kQXGroups;
            const int64_t k = pk + 8 * (int64_t)g;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (t < M && k < K) v = *reinterpret_cast<const uint4*>(x + t * K + k);
            xs[t * kQXGroups + (g ^ (4 * t))] = v;
        }
        __syncthreads();
        const int pb = p * kQPhaseChunks;

        while (lp == p) {  // the units of this phase, in order
            const int u = lu;
            const Unit un = lun;
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            for (int c = un.c0; c < un.c1; c += kU) {
                // the following item: the next chunks of this unit, else the
                // first chunks of the wave's next unit (this or a later phase)
                QItem<kU> nxt;
                bool more = true;
                if (c + kU < un.c1) {
                    lc = c + kU;
                } else {
                    next_unit(lp, lu);
                    if (lp < nphases) {
                        lun = unit_at(lp, lu);
                        lc = lun.c0;
                    } else {
                        more = false;
                    }
                }
                if (more) load(nxt, lun, lc);
#pragma unroll
                for (int v = 0; v < kU; ++v) {
                    if (c + v >= un.c1) break;  // uniform
                    const bool kok = (int64_t)(c + v) * kQChunk + 8 * lane < K;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const uint4 e = recon8(cur.w[v][r], cur.s[v][r], un.a[r]);
                        tile[r * 64 + (lane ^ (4 * r))] = kok ? e : make_uint4(0, 0, 0, 0);
                    }
                    quad_wave_sync();
                    const int xg = (c + v - pb) * 64;
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const uint4 wt = tile[j * 64 + ((b + 16 * h) ^ (4 * j))];
                        const uint4 xv = xs[j * kQXGroups + ((xg + b + 16 * h) ^ (4 * j))];
                        acc = mfma4x4x4(xv.x, xv.y, wt.x, wt.y, acc);
                        acc = mfma4x4x4(xv.z, xv.w, wt.z, wt.w, acc);
                    }
                    quad_wave_sync();
                }
                if (more) cur = nxt;
            }
            // lane 4b+j, register i: partial (token i, row j) of block b; add
            // the 16 blocks (fixed order) into the unit's slot
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = acc[i];
                v += __shfl_xor(v, 4, 64);
                v += __shfl_xor(v, 8, 64);
                v += __shfl_xor(v, 16, 64);
                v += __shfl_xor(v, 32, 64);
                if (lane < 4) red[u * 16 + i * 4 + lane] += v;
            }
        }
    }
    __syncthreads();
    // y[token i][row 4q + j] = sum over the quad's sub-ranges, in order
    for (int e = threadIdx.x; e < qn * 16; e += kQWaves * 64) {
        const int ql = e / 16, i = (e % 16) / 4, jj = e % 4;
        const int64_t n = 4 * (qb + ql) + jj;
        if (i >= M || n >= N) continue;
        float s = 0.0f;
        for (int t = 0; t < S; ++t) s += red[((ql << log2s) + t) * 16 + i * 4 + jj];
        store_y(y, i * N + n, s);
    }
}

}  // namespace

QuadPlan quad_plan(int64_t N, int64_t K, int num_cu) {
    QuadPlan p{0, 0, 0};
    if (N < 1 || K < 8 || num_cu < 1 || K >= (int64_t(1) << 30)) return p;
    const int64_t nquads = (N + 3) / 4;
    const int64_t grid = nquads < num_cu ? nquads : num_cu;
    const int64_t qpw = (nquads + grid - 1) / grid;
    const int64_t nchunks = (K + kQChunk - 1) / kQChunk;
    const int64_t pc = nchunks < kQPhaseChunks ? nchunks : kQPhaseChunks;  // chunks of a full phase
    // sub-ranges per quad (a power of two): whole quads per wave when the
    // workgroup has at least one per wave, else enough units for all waves,
    // never more sub-ranges than a phase has chunks
    int log2s = 0;
    while ((qpw << log2s) < kQWaves && (int64_t(2) << log2s) <= pc) ++log2s;
    if ((qpw << log2s) > kQuadMaxUnits) return p;
    p.grid = grid;
    p.qpw = qpw;
    p.s = log2s;
    return p;
}

const char* quad_name(int64_t N) { return N >= 1 ? "quad_kernel<2>" : ""; }

hipError_t launch_quad(const uint16_t* x, const uint16_t* w, const uint8_t* signs, const float* alpha,
                       bool per_row, YOut y, int64_t M, int64_t N, int64_t K, int num_cu, hipStream_t stream) {
    const QuadPlan p = quad_plan(N, K, num_cu);
    if (p.grid == 0 || M < 1 || M > 4) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quad_kernel<2>, dim3((unsigned)p.grid), dim3(kQWaves * 64), 0, stream, x, w, signs, alpha,
                       per_row ? 1 : 0, y, M, N, K, (int)p.qpw, p.s);
    return hipGetLastError();
}

}  // namespace bd
