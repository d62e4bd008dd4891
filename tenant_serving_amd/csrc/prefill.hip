// Prefill path: LDS-tiled bf16 MFMA with on-the-fly sign unpacking.
//
// "BitDelta : servir 14 modèles Zen depuis un seul cluster GPU" (hanzo-blog,
// 2026-02-28), "Serving architecture": reconstruction and matrix product in
// one kernel pass, W_eff rebuilt in registers or on-chip memory and never
// stored to HBM; the post notes the reconstruction is compute-bound at
// prefill, which is where this path lives.
//
// Workgroup tile 256 (tokens) x 256 (output rows) x 64 (k), 8 waves in a 2x4
// grid (two waves per SIMD, so one wave's LDS and barrier stalls are covered
// by the other's MFMAs), each wave owning a 128x64 block of y as 8
// v_mfma_f32_32x32x16_bf16 accumulators (128 AGPRs).  Each k step, the
// workgroup loads the 256x64 slice of x and of W_base (+ sign bytes),
// rebuilds the weight slice to bf16 W_eff with recon8 and stores both to
// LDS; rebuilding costs ~4 VALU ops per weight, about half the MFMA time of
// the step at this tile height.  To overlap the two, LDS is double buffered:
// while the MFMAs of step s read buffer s%2, the same waves rebuild and store
// step s+1 into the other buffer; global loads run two steps ahead.  One
// barrier per step.
//
// Workgroups are dealt to the 8 XCDs round robin; the tile order is chosen so
// that each XCD sweeps all M-tiles of one N-strip back to back, which keeps
// the strip's weights in that XCD's L2 while they are reused.
#include <type_traits>

#include "bd_device.h"
#include "bd_internal.h"

namespace bd {
namespace {

constexpr int kBM = kPrefillTile, kBN = kPrefillTile, kBK = 64;
constexpr int kWavesM = 2, kWavesN = 4;
constexpr int kThreads = 64 * kWavesM * kWavesN;
constexpr int kWTM = kBM / kWavesM, kWTN = kBN / kWavesN;  // 128 x 64 per wave
constexpr int kTM = kWTM / 32, kTN = kWTN / 32;            // 4 x 2 MFMA tiles
constexpr int kChunks = 8;                                 // 16-byte chunks per 64-k row
constexpr int kPrefillSets = 1;                            // register sets of loads in flight
constexpr int kSlotsA = kBM * kChunks / kThreads;          // 4 per thread
constexpr int kSlotsB = kBN * kChunks / kThreads;          // 4 per thread
static_assert(kSlotsA == kBK / 16 && kSlotsB == kBK / 16, "one load slot per MFMA sub-step");

// LDS row = 128 bytes = 8 chunks; the chunk index is XORed with (row / 2) so
// that the 16 rows read together by an MFMA operand load (a quarter wave)
// land in distinct 16-byte bank groups.
__device__ __forceinline__ int pswz(int row, int chunk) { return row * kChunks + (chunk ^ ((row >> 1) & 7)); }

struct StepRegs {
    uint4 a[kSlotsA];
    uint4 w[kSlotsB];
    uint32_t s[kSlotsB];
};

template <int kSets>
__global__ __launch_bounds__(kThreads) void prefill_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const uint8_t* __restrict__ signs, const float* __restrict__ alpha, int per_row,
    YOut y, int64_t M, int64_t N, int64_t K, int tiles_m, int tiles_n,
    int full, int ks, float* __restrict__ part) {
    // Two LDS buffers as four separate arrays, so the compiler can see that
    // stores into one buffer never alias the MFMA operand reads of the other.
    __shared__ uint4 As0[kBM * kChunks], As1[kBM * kChunks];
    __shared__ uint4 Bs0[kBN * kChunks], Bs1[kBN * kChunks];
    // Mark the kernel as using accumulation registers, so the MFMAs keep their
    // 128 accumulators in AGPRs and the VGPRs stay free for the pipeline.
    asm volatile("" ::: "a0");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / kWavesN, wn = wave % kWavesN;

    // Work of this workgroup: workgroups b < full each compute one whole
    // tile; the remaining tiles are split over K into ks parts, one per
    // workgroup, whose fp32 partial tiles a second kernel adds up.
    const int b = blockIdx.x;
    const int tiles = tiles_m * tiles_n;
    const int t = b < full ? b : full + (b - full) / ks;
    const int kp = b < full ? 0 : (b - full) % ks;
    // XCD-aware tile order: workgroup b runs on XCD b % 8; XCD x walks the
    // N-strips x, x+8, ... and, within a strip, all M-tiles.
    int tm, tn;
    {
        const int grouped = (tiles_n / 8) * 8 * tiles_m;  // tiles in complete 8-strip groups
        if (tiles % 8 == 0 && t < grouped) {
            const int xcd = t % 8, j = t / 8;
            tm = j % tiles_m;
            tn = (j / tiles_m) * 8 + xcd;
        } else {  // the remaining strips are walked in plain order
            const int r = t - (tiles % 8 == 0 ? grouped : 0);
            const int base_tn = tiles % 8 == 0 ? (tiles_n / 8) * 8 : 0;
            tm = r % tiles_m;
            tn = base_tn + r / tiles_m;
        }
    }
    const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
    const int64_t kbytes = K / 8;
    // k steps of this workgroup: [s_begin, s_begin + nsteps)
    const int64_t all_steps = (K + kBK - 1) / kBK;
    const int64_t per_part = (all_steps + ks - 1) / ks;
    const int64_t s_begin = b < full ? 0 : kp * per_part;
    const int64_t s_end = b < full ? all_steps : (s_begin + per_part < all_steps ? s_begin + per_part : all_steps);
    const int64_t nsteps = s_end > s_begin ? s_end - s_begin : 0;

    // Per-thread load slots: rows row0 + 64·i of the tile (i = 0..3), chunk
    // cthr of each 64-k step.  Buffer resources cover exactly the tile's
    // valid rows, so slots on rows past M or N read zeros; the per-lane offset
    // holds the row, the uniform offset the step.
    const int cthr = tid & 7, row0 = tid >> 3;
    constexpr int kRowStep = kThreads / kChunks;  // 64
    const int64_t arows = M - m0 < kBM ? M - m0 : kBM;
    const int64_t brows = N - n0 < kBN ? N - n0 : kBN;
    const rsrc_t ra = make_rsrc(x + m0 * K, (uint32_t)(arows * K * 2));
    const rsrc_t rw = make_rsrc(w + n0 * K, (uint32_t)(brows * K * 2));
    const rsrc_t rs = make_rsrc(signs + n0 * kbytes, (uint32_t)(brows * kbytes));
    const uint32_t row_bytes = (uint32_t)(K * 2), row_sbytes = (uint32_t)kbytes;
    const uint32_t voff_a = (uint32_t)row0 * row_bytes + cthr * 16;
    const uint32_t voff_s = (uint32_t)row0 * row_sbytes + cthr;
    float balpha[kSlotsB];
#pragma unroll
    for (int i = 0; i < kSlotsB; ++i) {
        const int64_t gn = n0 + row0 + kRowStep * i;
        balpha[i] = alpha[per_row ? (gn < N ? gn : N - 1) : 0];
    }

    // Load slot i of step s into R (zeros past K, and past the last step).
    // kFull: the step is known to be complete, so the load is unconditional
    // and a whole pipeline stage stays one basic block.
    auto load_slot = [&](StepRegs& R, int i, int64_t s, auto full_tag) {
        constexpr bool kFull = decltype(full_tag)::value;
        const int64_t k0 = (s_begin + s) * kBK;
        const uint32_t soff = (uint32_t)(k0 * 2), soff_s = (uint32_t)(k0 / 8);
        const bool kok = kFull || (s < nsteps && k0 + cthr * 8 < K);
        R.a[i] = kok ? buf_load16(ra, voff_a + i * kRowStep * row_bytes, soff) : make_uint4(0, 0, 0, 0);
        R.w[i] = kok ? buf_load16(rw, voff_a + i * kRowStep * row_bytes, soff) : make_uint4(0, 0, 0, 0);
        R.s[i] = kok ? buf_load_u8(rs, voff_s + i * kRowStep * row_sbytes, soff_s) : 0u;
    };
    auto store_slot = [&](const StepRegs& R, int i, uint4* Ad, uint4* Bd) {
        Ad[pswz(row0 + kRowStep * i, cthr)] = R.a[i];
        Bd[pswz(row0 + kRowStep * i, cthr)] = recon8(R.w[i], R.s[i], balpha[i]);
    };

    f32x16_t acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int r32 = lane & 31, half = lane >> 5;

    // One pipeline stage: the MFMAs of the step held in LDS buffer `mb`,
    // interleaved with rebuilding the step in R into buffer `sb` and refilling
    // R with step `ls`.  Each of the 4 MFMA sub-steps (8 MFMAs) carries one
    // load slot's worth of rebuild (about 35 VALU ops), its 2 stores and 3
    // loads; the scheduling groups lay them out as one MFMA followed by a few
    // VALU ops, so the vector ALU works in the MFMA's shadow.
    auto stage = [&](StepRegs& R, auto sb_tag, int64_t ls, auto full_tag, auto mb_tag) {
        uint4* Ad = decltype(sb_tag)::value ? As1 : As0;
        uint4* Bd = decltype(sb_tag)::value ? Bs1 : Bs0;
        const uint4* Am = decltype(mb_tag)::value ? As1 : As0;
        const uint4* Bm = decltype(mb_tag)::value ? Bs1 : Bs0;
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            const int chunk = 2 * kk + half;
            bf16x8_t af[kTM], bfr[kTN];
#pragma unroll
            for (int i = 0; i < kTM; ++i) af[i] = as_bf16x8(Am[pswz(wm * kWTM + i * 32 + r32, chunk)]);
#pragma unroll
            for (int j = 0; j < kTN; ++j) bfr[j] = as_bf16x8(Bm[pswz(wn * kWTN + j * 32 + r32, chunk)]);
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int j = 0; j < kTN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
            store_slot(R, kk, Ad, Bd);
            load_slot(R, kk, ls, full_tag);
            // groups: 6 LDS reads, then 8 x (MFMA, 5 VALU) with the 2 LDS
            // writes and 3 buffer loads spread between them
            __builtin_amdgcn_sched_group_barrier(0x100, kTM + kTN, 0);
#pragma unroll
            for (int t = 0; t < kTM * kTN; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
                if (t % 4 == 3) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                if (t >= 2 && t % 2 == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
        }
    };

    // The loop takes two steps per trip (one per LDS buffer) and never exits
    // early: an odd trailing step is all zeros (its loads are masked and its
    // MFMAs add nothing), so the accumulators stay one set.  With two register
    // sets (kSets = 2) loads run two steps ahead; with the two waves per SIMD
    // of this tiling that set no longer fits the 128 VGPRs a wave has, so the
    // default is one set, one step ahead.
    using Full = std::true_type;
    using Any = std::false_type;
    using B0 = std::false_type;
    using B1 = std::true_type;
    // local steps that lie wholly inside K
    const int64_t nfull = K / kBK - s_begin < nsteps ? K / kBK - s_begin : nsteps;
    int64_t s = 0;
    if constexpr (kSets == 2) {
        StepRegs P, Q;
#pragma unroll
        for (int i = 0; i < kSlotsA; ++i) load_slot(P, i, 0, Any{});
#pragma unroll
        for (int i = 0; i < kSlotsA; ++i) load_slot(Q, i, 1, Any{});
#pragma unroll
        for (int i = 0; i < kSlotsA; ++i) {
            store_slot(P, i, As0, Bs0);
            load_slot(P, i, 2, Any{});
        }
        __syncthreads();
        auto trip = [&](int64_t s, auto full_tag) {
            stage(Q, B1{}, s + 3, full_tag, B0{});  // MFMAs of step s; step s+1 -> buffer 1
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            stage(P, B0{}, s + 4, full_tag, B1{});  // MFMAs of step s+1; step s+2 -> buffer 0
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
        };
        for (; s + 4 < nfull; s += 2) trip(s, Full{});  // prefetched steps s+3, s+4 complete
        for (; s < nsteps; s += 2) trip(s, Any{});
    } else {
        // One register set, loads one step ahead; the second wave on each
        // SIMD covers the shorter lead.
        StepRegs P;
#pragma unroll
        for (int i = 0; i < kSlotsA; ++i) load_slot(P, i, 0, Any{});
#pragma unroll
        for (int i = 0; i < kSlotsA; ++i) {
            store_slot(P, i, As0, Bs0);
            load_slot(P, i, 1, Any{});
        }
        __syncthreads();
        auto trip = [&](int64_t s, auto full_tag) {
            stage(P, B1{}, s + 2, full_tag, B0{});  // MFMAs of step s; step s+1 -> buffer 1
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            stage(P, B0{}, s + 3, full_tag, B1{});  // MFMAs of step s+1; step s+2 -> buffer 0
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
        };
        for (; s + 3 < nfull; s += 2) trip(s, Full{});  // prefetched steps s+2, s+3 complete
        for (; s < nsteps; s += 2) trip(s, Any{});
    }

    // D layout of the 32x32 MFMA: register r of lane l is row
    // 8·(r/4) + 4·(l/32) + r%4, column l%32.
    if (b < full) {
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int j = 0; j < kTN; ++j) {
                const int64_t n = n0 + wn * kWTN + j * 32 + r32;
                if (n >= N) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t m = m0 + wm * kWTM + i * 32 + 8 * (r / 4) + 4 * half + (r % 4);
                    if (m < M) store_y(y, m * N + n, acc[i][j][r]);
                }
            }
    } else {
        // partial tile [256 rows][256 columns] of part (b - full)
        float* pt = part + (int64_t)(b - full) * kBM * kBN;
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int j = 0; j < kTN; ++j) {
                const int nl = wn * kWTN + j * 32 + r32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int ml = wm * kWTM + i * 32 + 8 * (r / 4) + 4 * half + (r % 4);
                    pt[ml * kBN + nl] = acc[i][j][r];
                }
            }
    }
}

static_assert(kBN % 4 == 0, "the sum kernel takes 4 outputs of one tile row per lane");

__device__ __forceinline__ float keep_or_negzero(float v, uint32_t q) {
    return __uint_as_float((__float_as_uint(v) & q) | (0x80000000u & ~q));
}

// y of every split tile = the sum of its ks partial tiles, in part order.
// A lane takes 4 outputs that are adjacent along n (16-byte loads of the
// partials, which the workspace's 16-byte alignment allows); each output is
// still the parts added one by one in part order.
__global__ __launch_bounds__(256) void prefill_sum_kernel(const float* __restrict__ part, int full, int ks,
                                                          int tiles_m, int tiles_n, int64_t M, int64_t N,
                                                          YOut y) {
    const int tiles = tiles_m * tiles_n;
    const int64_t per_tile = (int64_t)kBM * kBN;
    const int64_t total4 = (int64_t)(tiles - full) * per_tile / 4;
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total4; q += (int64_t)gridDim.x * 256) {
        const int64_t e = 4 * q;
        const int ts = (int)(e / per_tile);
        const int el = (int)(e % per_tile);
        // same tile order as prefill_kernel
        const int t = full + ts;
        int tm, tn;
        const int grouped = (tiles_n / 8) * 8 * tiles_m;
        if (tiles % 8 == 0 && t < grouped) {
            const int xcd = t % 8, j = t / 8;
            tm = j % tiles_m;
            tn = (j / tiles_m) * 8 + xcd;
        } else {
            const int r = t - (tiles % 8 == 0 ? grouped : 0);
            const int base_tn = tiles % 8 == 0 ? (tiles_n / 8) * 8 : 0;
            tm = r % tiles_m;
            tn = base_tn + r / tiles_m;
        }
        const int64_t m = (int64_t)tm * kBM + el / kBN, n = (int64_t)tn * kBN + el % kBN;  // n .. n+3: one tile row
        if (m >= M || n >= N) continue;
        const float4* src = reinterpret_cast<const float4*>(part + (int64_t)ts * ks * per_tile + el);
        // parts added in order, 8 loaded at a time (all in flight together) so
        // their latency is paid once per 8; a part index past the last
        // repeats the last part, and that copy is added as -0 (x + -0 = x for
        // every x, signed zeros included)
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int p0 = 0; p0 < ks; p0 += 8) {
            float4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = src[(int64_t)(p0 + u < ks ? p0 + u : ks - 1) * (per_tile / 4)];
            __builtin_amdgcn_sched_barrier(0);  // the batch's loads are all issued before the adds
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t q = p0 + u < ks ? 0xffffffffu : 0u;
                const float4 t = make_float4(keep_or_negzero(v[u].x, q), keep_or_negzero(v[u].y, q),
                                             keep_or_negzero(v[u].z, q), keep_or_negzero(v[u].w, q));
                if (u == 0)
                    s = p0 == 0 ? t : make_float4(s.x + t.x, s.y + t.y, s.z + t.z, s.w + t.w);
                else
                    s = make_float4(s.x + t.x, s.y + t.y, s.z + t.z, s.w + t.w);
            }
        }
        const float sv[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (n + i < N) store_y(y, m * N + n + i, sv[i]);
    }
}

}  // namespace

const char* prefill_name() { return "prefill_kernel"; }

hipError_t launch_prefill(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                          const float* alpha, bool per_row, YOut y, int64_t M, int64_t N,
                          int64_t K, void* workspace, hipStream_t stream) {
    const PrefillPlan p = prefill_plan(M, N, K);
    float* part = static_cast<float*>(workspace);
    hipLaunchKernelGGL(prefill_kernel<kPrefillSets>, dim3((unsigned)p.grid), dim3(kThreads), 0, stream,
                       x, w, signs, alpha, per_row ? 1 : 0, y, M, N, K, (int)p.tiles_m, (int)p.tiles_n,
                       (int)p.full, p.ks, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.full == p.tiles_m * p.tiles_n) return e;
    const int64_t total4 = (p.tiles_m * p.tiles_n - p.full) * (int64_t)kBM * kBN / 4;
    int64_t blocks = (total4 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(prefill_sum_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, part, (int)p.full,
                       p.ks, (int)p.tiles_m, (int)p.tiles_n, M, N, y);
    return hipGetLastError();
}

}  // namespace bd
