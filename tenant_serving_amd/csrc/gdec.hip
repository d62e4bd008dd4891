// Grouped multi-variant linear at decode (up to 4 tokens): rows streamed
// once, each present variant rebuilt from the shared base row, VALU dot
// products per token.
//
// "BitDelta : servir 14 modèles Zen depuis un seul cluster GPU" (hanzo-blog,
// 2026-02-28), "Serving architecture": one HBM-resident base shared by every
// variant, one (α, sign(Δ)) entry per variant, each request routed to its
// variant's entry; y[m] = x[m]·W_eff(ids[m])ᵀ with W_eff rebuilt on chip.
//
// A decode batch of a few tokens carries one or two tokens per variant, so
// the bytes are the base once plus each present variant's sign plane, and the
// work per weight is one rebuild per present variant.  The
// base streams the way the one-token GEMV streams it: a wave owns two rows
// and reads them in 1 KiB pieces (lane l: elements 8l..8l+7 of a 512-wide
// chunk), with the next piece's loads in flight while the current one is
// used.  With each piece come the sign bytes of the same 8 elements for every
// token's variant.  The tokens are taken in a stable order by variant id, so
// a row piece is widened once and rebuilt (recon8_word) once per variant and its dot products
// (v_dot2) go to that variant's tokens.  x sits in LDS one K range at a time;
// a workgroup of 8 waves owns a block of rows for one range.  With one range
// it writes y; otherwise each range writes fp32 partials that reduce_kernel
// adds in range order.  Tokens whose id is out of range get NaN rows.
#include "bd_device.h"
#include "bd_internal.h"

namespace bd {
namespace {

constexpr int kGdWaves = 8;
constexpr int kGdChunk = 512;               // k per row piece: 64 lanes x 8
constexpr int kGdXsUints = kGdXsBytes / 16;  // x slice, 16-byte groups

// One work item: two rows x one chunk, with the sign bytes of every token
// position (bytes, so that their widening stays where they are used).
template <int MP>
struct GdItem {
    uint4 w0, w1;
    uint8_t s0[MP], s1[MP];
};

template <int MP>
__global__ __launch_bounds__(kGdWaves * 64) void gdec_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids, const uint16_t* __restrict__ w,
    VariantTable tab, int per_row, int G, int64_t M, int64_t N, int64_t K, int krc, int nkr,
    int pairs, float* __restrict__ part, float* __restrict__ y) {
    __shared__ uint4 xs[kGdXsUints];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int range = (int)(blockIdx.x % nkr);
    const int64_t rb = blockIdx.x / nkr;
    const int64_t nchunks = (K + kGdChunk - 1) / kGdChunk;
    const int64_t kbytes = K / 8;
    const int64_t c0 = (int64_t)range * krc;                            // first chunk of the range
    const int nc = (int)((c0 + krc <= nchunks ? c0 + krc : nchunks) - c0);  // chunks in the range
    const int stride = krc * (kGdChunk / 8);                            // x row stride in LDS, groups

    // Token positions: the valid tokens in a stable order by variant id
    // (uniform; at most MP tokens).  tok[p] is the token at position p.
    int idv[MP];
#pragma unroll
    for (int m = 0; m < MP; ++m) {
        const int g = m < M ? ids[m] : -1;
        idv[m] = g >= 0 && g < G ? g : -1;
    }
    int tok[MP], var[MP];
    int npos = 0;
#pragma unroll
    for (int p = 0; p < MP; ++p) {
        tok[p] = 0;
        var[p] = 0;
    }
#pragma unroll
    for (int m = 0; m < MP; ++m) {
        if (idv[m] < 0) continue;
        int rank = 0;
#pragma unroll
        for (int j = 0; j < MP; ++j)
            rank += (idv[j] >= 0 && (idv[j] < idv[m] || (idv[j] == idv[m] && j < m))) ? 1 : 0;
#pragma unroll
        for (int p = 0; p < MP; ++p)
            if (p == rank) {
                tok[p] = m;
                var[p] = idv[m];
            }
        ++npos;
    }
    const uint8_t* sp[MP];
    const float* ap[MP];
#pragma unroll
    for (int p = 0; p < MP; ++p) {
        const int pp = p < npos ? p : 0;  // positions past the valid tokens repeat position 0
        sp[p] = tab.signs[var[pp]];
        ap[p] = tab.alpha[var[pp]];
    }

    // Rows of item (pair q, chunk c): the wave's pairs are consecutive.
    const int64_t row_base = rb * (int64_t)(kGdWaves * pairs * 2) + (int64_t)wave * pairs * 2;
    auto rows_of = [&](int q, int64_t& r0, int64_t& r1) {
        r0 = row_base + 2 * (int64_t)q;
        r1 = r0 + 1;
        r0 = r0 < N ? r0 : N - 1;  // rows past the end: computed, never stored
        r1 = r1 < N ? r1 : N - 1;
    };
    // Every load is unconditional and in bounds: lanes past K read the row's
    // last 8 weights (zeroed where used), positions past the valid tokens
    // read position 0's signs.
    auto load = [&](GdItem<MP>& it, int q, int c) {
        int64_t r0, r1;
        rows_of(q, r0, r1);
        int64_t k = (c0 + c) * kGdChunk + 8 * lane;
        k = k < K ? k : K - 8;
        const uint32_t g = (uint32_t)(k >> 3);  // this lane's 16-byte group = its sign byte
        // uniform row bases, 32-bit lane offsets
        it.w0 = load_stream16(reinterpret_cast<const uint4*>(w + r0 * K) + g);
        it.w1 = load_stream16(reinterpret_cast<const uint4*>(w + r1 * K) + g);
#pragma unroll
        for (int p = 0; p < MP; ++p) {
            it.s0[p] = __builtin_nontemporal_load(sp[p] + r0 * kbytes + g);
            it.s1[p] = __builtin_nontemporal_load(sp[p] + r1 * kbytes + g);
        }
    };

    GdItem<MP> cur;
    load(cur, 0, 0);

    // x[:, range] -> LDS (zero past K); token rows >= M are never read.
    for (int e = threadIdx.x; e < (int)M * stride; e += kGdWaves * 64) {
        const int t = e / stride, gi = e % stride;
        const int64_t kx = (c0 * (kGdChunk / 8) + gi) * 8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (kx < K) v = *reinterpret_cast<const uint4*>(x + t * K + kx);
        xs[t * stride + gi] = v;
    }
    __syncthreads();

    float acc0[MP], acc1[MP];
#pragma unroll
    for (int p = 0; p < MP; ++p) acc0[p] = acc1[p] = 0.0f;
    uint32_t na0[MP], na1[MP];  // bit patterns of -α of the two rows, per position
    const SignShifts sh0 = sign_shifts(0);

    for (int q = 0; q < pairs; ++q) {
        int64_t r0, r1;
        rows_of(q, r0, r1);
#pragma unroll
        for (int p = 0; p < MP; ++p) {
            na0[p] = __float_as_uint(-ap[p][per_row ? r0 : 0]);
            na1[p] = __float_as_uint(-ap[p][per_row ? r1 : 0]);
        }
        for (int c = 0; c < nc; ++c) {
            // the following item: next chunk, else the next pair's first
            // (after the wave's last item this reloads its first one, unused)
            int qn = q, cn = c + 1;
            if (cn == nc) {
                cn = 0;
                qn = q + 1 < pairs ? q + 1 : 0;
            }
            GdItem<MP> nxt;
            load(nxt, qn, cn);

            // the two row pieces widened once for all variants; in a chunk
            // that runs past K the lanes there get zero weights (W_eff = ±α,
            // against x = 0)
            Widened8 b0 = widen8(cur.w0), b1 = widen8(cur.w1);
            if ((c0 + c + 1) * kGdChunk > K) {  // uniform
                const bool kin = (c0 + c) * kGdChunk + 8 * lane < K;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    b0.lo[i] = kin ? b0.lo[i] : 0.0f;
                    b0.hi[i] = kin ? b0.hi[i] : 0.0f;
                    b1.lo[i] = kin ? b1.lo[i] : 0.0f;
                    b1.hi[i] = kin ? b1.hi[i] : 0.0f;
                }
            }
            const int xo = c * (kGdChunk / 8) + lane;
            uint4 e0 = make_uint4(0, 0, 0, 0), e1 = make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int p = 0; p < MP; ++p) {
                if (p < npos) {
                    if (p == 0 || var[p] != var[p > 0 ? p - 1 : 0]) {  // a new variant: rebuild the two rows
                        e0 = recon8_word(b0, sign_spread(cur.s0[p]), sh0, na0[p]);
                        e1 = recon8_word(b1, sign_spread(cur.s1[p]), sh0, na1[p]);
                    }
                    const uint4 xv = xs[tok[p] * stride + xo];
                    acc0[p] += dot8_bf16(e0, xv);
                    acc1[p] += dot8_bf16(e1, xv);
                }
            }
            cur = nxt;
        }
        // the pair's sums over the range: one wave reduction per (token, row)
        const int64_t n0 = row_base + 2 * (int64_t)q;
#pragma unroll
        for (int p = 0; p < MP; ++p) {
            if (p < npos) {
                const float s0 = wave_sum(acc0[p]);
                const float s1 = wave_sum(acc1[p]);
                if (lane == 0) {
                    float* dst = nkr == 1 ? y : part + (int64_t)range * M * N;
                    const int64_t base = (int64_t)tok[p] * N;
                    if (n0 < N) dst[base + n0] = s0;
                    if (n0 + 1 < N) dst[base + n0 + 1] = s1;
                }
            }
            acc0[p] = acc1[p] = 0.0f;
        }
        // tokens with an id out of range: NaN rows (with one range; otherwise
        // reduce_kernel writes them)
        if (nkr == 1 && lane < M) {
            const int m = lane;
            const int g = ids[m];
            if (g < 0 || g >= G) {
                if (n0 < N) y[(int64_t)m * N + n0] = __builtin_nanf("");
                if (n0 + 1 < N) y[(int64_t)m * N + n0 + 1] = __builtin_nanf("");
            }
        }
    }
}

}  // namespace

GdecPlan gdec_plan(int64_t M, int64_t N, int64_t K) {
    GdecPlan p{0, 0, 0, 0, 0};
    if (M < 1 || M > kGdecMaxM || K < 8 || N < kGdecMinN) return p;
    const int64_t nchunks = (K + kGdChunk - 1) / kGdChunk;
    int64_t krc = kGdXsBytes / (M * kGdChunk * 2);
    if (krc < 1) krc = 1;
    if (krc > nchunks) krc = nchunks;
    const int64_t nkr = (nchunks + krc - 1) / krc;
    // about two workgroups per CU of kPlanCUs: row blocks of 16 rows x pairs
    const int64_t target_rb = (2 * (int64_t)kPlanCUs + nkr - 1) / nkr;
    int64_t pairs = (N + 16 * target_rb - 1) / (16 * target_rb);
    if (pairs < 1) pairs = 1;
    const int64_t rows_per_block = (int64_t)kGdWaves * 2 * pairs;
    p.mp = kGdecMaxM;
    p.krc = (int)krc;
    p.nkr = (int)nkr;
    p.pairs = (int)pairs;
    p.grid = ((N + rows_per_block - 1) / rows_per_block) * nkr;
    return p;
}

const char* gdec_name() { return "gdec_kernel<4>"; }

hipError_t launch_gdec(const uint16_t* x, const int32_t* ids, const uint16_t* w, const VariantTable& table,
                       bool per_row, int32_t G, float* y, int64_t M, int64_t N, int64_t K, float* part,
                       hipStream_t stream) {
    const GdecPlan p = gdec_plan(M, N, K);
    if (p.grid == 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gdec_kernel<kGdecMaxM>, dim3((unsigned)p.grid), dim3(kGdWaves * 64), 0, stream, x, ids, w,
                       table, per_row ? 1 : 0, (int)G, M, N, K, p.krc, p.nkr, p.pairs, part, y);
    return hipGetLastError();
}

}  // namespace bd
