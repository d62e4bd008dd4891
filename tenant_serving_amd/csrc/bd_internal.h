// Host-side launch entry points of the BitDelta kernels.  The C ABI layer
// validates every argument before calling these; they only size grids and
// enqueue work on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bd {

// api.cpp: records a HIP error for bd_last_hip_error() (calling thread).
void note_hip_error(hipError_t e);

constexpr int kMaxVariants = 64;

// The output y of the single-variant linear: fp32, or bf16 (each fp32 result
// rounded to nearest even, the bf16 result of the listing's F.linear on bf16
// operands).  `bf16` is uniform over a launch.
struct YOut {
    void* p;
    int bf16;
};
// y advanced by `elems` elements.
inline YOut y_at(YOut y, int64_t elems) {
    return YOut{static_cast<char*>(y.p) + elems * (y.bf16 ? 2 : 4), y.bf16};
}

// Per-variant delta-cache entries, passed to kernels by value.
struct VariantTable {
    const uint8_t* signs[kMaxVariants];
    const float* alpha[kMaxVariants];
};

// compress.hip
hipError_t launch_compress_pair(const uint16_t* w_ft, const uint16_t* w_base, int64_t d_out,
                                int64_t d_in, bool per_row, uint8_t* signs, float* alpha,
                                double* row_sums, hipStream_t stream);
hipError_t launch_compress(const float* delta, int64_t d_out, int64_t d_in, bool per_row,
                           uint8_t* signs, float* alpha, double* row_sums, hipStream_t stream);

// gemv.hip: VALU dot-product path, 1 <= M <= kGemvMaxM
constexpr int kGemvMaxM = 4;
// gemv.hip: VALU dot products with x resident in LDS, 2 <= M <= kXresMaxM on
// projections with at least kXresMinN rows and x of at most kXresXBytes
constexpr int kXresMaxM = 4;
constexpr int64_t kXresMinN = 2048;
constexpr int64_t kXresXBytes = 131072;
hipError_t launch_xres(const uint16_t* x, const uint16_t* w, const uint8_t* signs, const float* alpha,
                       bool per_row, YOut y, int64_t M, int64_t N, int64_t K, int num_cu,
                       hipStream_t stream);
const char* xres_name(int64_t M, int64_t K);
hipError_t launch_gemv(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                       const float* alpha, bool per_row, YOut y, int64_t M, int64_t N,
                       int64_t K, hipStream_t stream);
const char* gemv_name(int64_t M, int64_t N, int64_t K);

// skinny.hip: MFMA path for M <= kSkinnyMaxM
constexpr int kSkinnyMaxM = 64;
const char* skinny_name(int64_t M, int64_t N);
hipError_t launch_skinny(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                         const float* alpha, bool per_row, YOut y, int64_t M, int64_t N,
                         int64_t K, hipStream_t stream);

// band.hip: MFMA path for 4..16 tokens on rows of up to kBandMaxK weights.
// band_grid is its launch grid (one workgroup per compute unit, at most one
// per band of 4 rows), or 0 where its partial-sum slots cannot hold a
// workgroup's bands (16384 / (64 mp) bands, mp = M rounded up to 4).
constexpr int kBandMaxM = 16;
constexpr int64_t kBandMaxK = 8192;
int64_t band_grid(int64_t M, int64_t N, int64_t K, int num_cu);
hipError_t launch_band(const uint16_t* x, const uint16_t* w, const uint8_t* signs, const float* alpha,
                       bool per_row, YOut y, int64_t M, int64_t N, int64_t K, int num_cu, hipStream_t stream);
const char* band_name();

// rowstream.hip: MFMA path for M <= kRowstreamMaxM on projections with 4096
// or more rows (workgroups of 32 rows, or 16 where those fit one per CU,
// each wave streaming whole rows)
constexpr int kRowstreamMaxM = 32;
hipError_t launch_rowstream(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                            const float* alpha, bool per_row, YOut y, int64_t M, int64_t N,
                            int64_t K, int num_cu, hipStream_t stream);
const char* rowstream_name(int64_t M, int64_t N, int num_cu);

// decode.hip: x-stationary MFMA streaming path, 2 <= M <= kXstatMaxM tokens
// on projections with many rows.  Workgroups of two teams own 2·r row groups
// of 8 rows each; K is cut into nkr ranges of krc 512-wide chunks whose x
// slice fits kXstatXsBytes of LDS.
constexpr int kXstatMaxM = 16;
constexpr int kXstatXsBytes = 65536;
constexpr int kXstatMaxR = 8;
struct XstatPlan {
    int r;         // row groups per team (0: shape not served by this path)
    int krc;       // chunks per K range (a multiple of 4: one per wave of a team)
    int nkr;       // K ranges
    int64_t grid;  // workgroups
};
inline XstatPlan xstat_plan(int64_t M, int64_t N, int64_t K, int num_cu) {
    XstatPlan p{0, 0, 0, 0};
    // (row offsets within a group of 8 rows are 32-bit: K < 2^27)
    if (M < 2 || M > kXstatMaxM || K < 8 || K >= (int64_t(1) << 27) || N < 1 || num_cu < 1) return p;
    const int64_t groups = (N + 7) / 8;
    if (groups < 2 * (int64_t)num_cu) return p;  // too few rows to fill the GPU
    const int64_t r = (groups + 2 * (int64_t)num_cu - 1) / (2 * (int64_t)num_cu);
    if (r > kXstatMaxR) return p;
    const int64_t nchunks = (K + 511) / 512;
    const int64_t krc_max = (kXstatXsBytes / (M * 1024)) / 4 * 4;  // x row chunk = 1 KiB
    int64_t nkr = (nchunks + krc_max - 1) / krc_max;
    int64_t krc = ((nchunks + nkr - 1) / nkr + 3) / 4 * 4;
    nkr = (nchunks + krc - 1) / krc;
    p.r = (int)r;
    p.krc = (int)krc;
    p.nkr = (int)nkr;
    p.grid = (groups + 2 * r - 1) / (2 * r);
    return p;
}
hipError_t launch_xstat(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                        const float* alpha, bool per_row, YOut y, int64_t M, int64_t N,
                        int64_t K, int num_cu, hipStream_t stream);
const char* xstat_name(int64_t M, int64_t N, int64_t K, int num_cu);

// shot.hip: MFMA path for up to 16 tokens on projections with few rows
// (workgroups of 16 waves own 4 rows, one K chunk per wave)
constexpr int kShotMaxM = 16;
constexpr int64_t kShotMaxK = int64_t(1) << 26;  // x (M <= 16 rows) within a 2 GiB buffer resource
hipError_t launch_shot(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                       const float* alpha, bool per_row, YOut y, int64_t M, int64_t N, int64_t K,
                       hipStream_t stream);
const char* shot_name();

// slice.hip: MFMA path for up to 16 tokens on projections with few rows:
// workgroups of 16 waves own 16 rows over one 2048-wide slice of K.  With
// several slices their fp32 sums go to the workspace ([slices][M][N]) and a
// second kernel adds the planes in slice order.
constexpr int kSliceMaxM = 16;
constexpr int64_t kSliceMaxK = int64_t(1) << 26;  // x (M <= 16 rows) within a 2 GiB buffer resource
int64_t slice_count(int64_t K);
size_t slice_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_slice(const uint16_t* x, const uint16_t* w, const uint8_t* signs, const float* alpha,
                        bool per_row, YOut y, int64_t M, int64_t N, int64_t K, void* workspace,
                        hipStream_t stream);
const char* slice_name();
// Shapes that may take the slice path (a function of the shape alone, so that
// the workspace query needs no device): 3..16 tokens on fewer than 4096 rows
// of 2048 or more weights, where the one-shot kernel's workgroups would each
// pull at least 256 KiB of x (M·K >= 131072), or on 2048..4095 rows.  The
// band kernel, checked first, keeps 4..16 tokens on 2048..4095 rows of
// 4097..8192 weights.  Same-process timings against the one-shot kernel
// (us): 1024x8192 at 12/16 tokens 10.2/11.6 -> 10.1/10.3, 512x8192 at 16
// 11.3 -> 8.9, 1024x16384 at 8/16 15.0/20.5 -> 14.0/14.9, 3072x4096 at 3/16
// 13.8/20.1 -> 11.4/12.5, 4000x2048 14.1 -> 6.9 at 4, 2048x2048 8.0 -> 5.4 at
// 4; the one-shot kernel stays ahead below that much x (1024x8192 at 4
// tokens 8.0 against 9.9, 1024x4096 at 16 7.8 against 8.2, 1000x5000 at 16
// 7.9 against 9.9).
inline bool use_slice(int64_t M, int64_t N, int64_t K) {
    return M >= 3 && M <= kSliceMaxM && N < 4096 && K >= 2048 && K < kSliceMaxK &&
           (N >= 2048 || M * K >= 131072);
}

// quad.hip: two to four tokens, MFMA 4x4x4 over row quads, x slices of up
// to kQuadPhaseMax columns in LDS.  A plan deals row quads to workgroups
// (qpw each) and cuts each quad's chunks of a phase into s sub-ranges; the
// workgroup's units (quads x sub-ranges) are at most kQuadMaxUnits.
constexpr int64_t kQuadPhaseMax = 8192;
constexpr int kQuadMaxUnits = 128;
struct QuadPlan {
    int64_t grid;  // workgroups (0: shape not served)
    int64_t qpw;   // row quads per workgroup
    int s;         // log2 of the sub-ranges per quad and phase
};
QuadPlan quad_plan(int64_t N, int64_t K, int num_cu);
hipError_t launch_quad(const uint16_t* x, const uint16_t* w, const uint8_t* signs, const float* alpha,
                       bool per_row, YOut y, int64_t M, int64_t N, int64_t K, int num_cu, hipStream_t stream);
const char* quad_name(int64_t N);

// Which decode/prefill path serves bd_linear for a shape.
// The tiled prefill path addresses a 256-row tile of x or of the base with
// 32-bit buffer offsets, so it takes d_in <= kPrefillMaxK; longer rows (far
// beyond any model's) go through the skinny path 64 tokens at a time.
constexpr int64_t kPrefillMaxK = (int64_t(1) << 23) - 8;
enum class LinearPath { kGemv, kXres, kSlice, kBand, kQuad, kXstat, kShot, kRowstream, kSkinny, kSkinnyBlocks, kPrefill };
inline LinearPath choose_linear_path(int64_t M, int64_t N, int64_t K, int num_cu) {
    // In order: 4..16 tokens on rows of 4097..8192 weights where the band
    // kernel wins (below).  3..16 tokens on fewer than 4096 rows with much x
    // per row (use_slice): K slices.  Four tokens on 8192 or more rows: the
    // row-quad kernel.  3..16 tokens on fewer than 4096 rows otherwise:
    // one-shot workgroups (the whole matrix in flight at once; at 4 tokens on
    // 1024x8192, 7.5 against 8.3 us on the VALU path).  Two to four tokens with x within 128 KiB: x
    // resident in LDS.  One token, or two, or a few on a projection with
    // fewer than 8192 rows: VALU dot products.  4 to 32 tokens on up to 1.5
    // row-streaming workgroups per CU: row streaming.  Up to 16 tokens on
    // projections with many rows: the x-stationary MFMA streaming path,
    // unless the x slice would change every few items.  Otherwise up to 32
    // tokens on 4096 or more rows: row streaming.
    // Otherwise up to 64 tokens the skinny MFMA path; beyond, LDS tiles.
    // Two tokens on rows of up to 16K weights: still the VALU path (measured
    // 4-5% ahead of the x-stationary one on q and gate; behind on down).
    // Two to four tokens on 2048 or more rows with x within 128 KiB (four
    // only below 8192 rows): the VALU path with x resident in LDS (gate 85.6
    // -> 81.8 us at two tokens, 86.8 -> 83.5 at three; down at two 86.2 ->
    // 82.7; 8192x16384 at three 67.4 -> 56.8; 4096x14336 at 2/3/4 tokens
    // 26.0/27.6/30.5 -> 23.0/23.9/26.3 against the GEMV; on 8192 or more rows
    // at four it only matches the x-stationary path).
    // Four tokens on 8192 or more rows of up to 16K weights: the row-quad
    // kernel (same-process A/B against the x-stationary kernel: 28672x8192
    // 87.6 -> 83.9 us, 8192x8192 30.9 -> 29.9, 8195x8200 40.6 -> 36.7; on
    // 8192x28672 its four x phases lose, 89.4 -> 94.7, and at two or three
    // tokens the x-resident VALU kernel is as fast or faster).
    // (only where its plan fits: at most kQuadMaxUnits units per workgroup,
    // so up to 4 · kQuadMaxUnits · num_cu rows)
    // 4..16 tokens on 8192 or more rows of 4097..8192 weights where the band
    // kernel's slots hold a workgroup's bands in one round (and on fewer rows,
    // below); at four tokens
    // only up to 16 bands per workgroup (16384 rows on 256 CUs): beyond, the
    // row-quad kernel stays ahead (28672x8192 83.2 against 84.7 us), and two
    // rounds lost to the x-stationary kernel (28672x8192 at 12/16 tokens
    // 90.8/92.3 -> 95.4/99.5).  Same-process timings against the kernels it
    // replaces: 8192x8192 at 4/8/12/16 tokens 30.3/32.0/32.1/32.8 ->
    // 28.1/29.4/30.9/32.1 us, 16384x8192 53.9/53.9/56.8/58.6 ->
    // 51.1/52.1/54.2/56.4, 28672x8192 at 8 tokens 90.7 -> 86.2, 12296x5000
    // at 4/8/12/16 tokens 34.3/36.7/38.3/40.2 -> 30.6/31.3/32.2/33.6.
    // On 2048..4095 rows it replaces the one-shot kernel (2048x8192 at 4/16
    // tokens 14.4/21.8 -> 11.6/15.2 us, 3072x8192 21.2/31.0 -> 14.9/17.3; on
    // 1024 rows it loses, 7.8 -> 8.8 at 4 tokens), and on 4096..8191 rows it
    // takes 4..8 tokens where at least 15 of its 16 waves have a chunk
    // (4104x8192 at 4/8 tokens 20.0/20.9 -> 17.7/18.6, 8188x8192 30.0/32.0 ->
    // 27.8/29.3; at 16 tokens, or with fewer chunks, level or behind:
    // 6144x8192 at 16 25.2 -> 26.8, 6152x5000 at 8 16.6 -> 19.1).
    if (M >= 4 && M <= kBandMaxM && N >= 2048 && K > 4096 && K <= kBandMaxK) {
        const int64_t g = band_grid(M, N, K, num_cu);
        const bool wins = N >= 8192 ? (M > 4 || (N + 3) / 4 <= 16 * g) : N >= 4096 ? (M <= 8 && K > 7168) : true;
        if (g > 0 && wins) return LinearPath::kBand;
    }
    if (use_slice(M, N, K)) return LinearPath::kSlice;
    if (M == 4 && N >= 8192 && K <= 2 * kQuadPhaseMax && quad_plan(N, K, num_cu).grid > 0) return LinearPath::kQuad;
    if (M >= 3 && M <= kShotMaxM && N < 4096 && K < kShotMaxK) return LinearPath::kShot;
    if (M >= 2 && M <= kXresMaxM && N >= kXresMinN && (M <= 3 || N < 8192) && M * K * 2 <= kXresXBytes)
        return LinearPath::kXres;
    if (M == 1 || (M <= kGemvMaxM && N < 8192) || (M == 2 && K <= 16384)) return LinearPath::kGemv;
    // 4..32 tokens where row streaming's 32-row workgroups number at most 1.5
    // per CU: row streaming ahead of the x-stationary path (same-process
    // timings: 8192x28672 at 4/5/8 tokens 85.9/86.9/90.9 -> 83.8/83.2/83.1 us,
    // 8192x8192 at 5/8 32.0/32.9 -> 31.7/31.8, 6152x8200 at 5/8 31.3/33.7 ->
    // 24.3/25.1, 12000x3000 level or ahead; at 16384 rows, two workgroups per
    // CU, the x-stationary path stays ahead: 30-33 against 34-36 us).
    if (M >= 4 && M <= kRowstreamMaxM && N >= 4096 && N <= 16384 && 2 * ((N + 31) / 32) <= 3 * (int64_t)num_cu)
        return LinearPath::kRowstream;
    const XstatPlan xp = xstat_plan(M, N, K, num_cu);
    // Each switch of x slice costs two workgroup barriers; the streaming path
    // pays off when a wave has at least 4 items per slice (or one slice).
    if (xp.r > 0 && (xp.nkr == 1 || xp.r * (xp.krc / 4) >= 4)) return LinearPath::kXstat;
    if (M <= kShotMaxM && N < 4096 && K < kShotMaxK) return LinearPath::kShot;
    // Otherwise up to 32 tokens on 4096 or more rows: row streaming (on more
    // than 16384 rows, same-process timings against the skinny path: 28672x8192
    // at 17/32 tokens 130.5/153.9 -> 109.7/121.2 us, 40000x4096 at 16 tokens
    // 92.9 -> 76.0, 131080x1024 at 4..16 tokens 56.6..68.1 -> 52.3..61.0;
    // 57344x8192 at 8 tokens 187 -> 197, level at 4 and 5).
    if (M <= kRowstreamMaxM && N >= 4096) return LinearPath::kRowstream;
    if (M <= kSkinnyMaxM) return LinearPath::kSkinny;
    if (K > kPrefillMaxK) return LinearPath::kSkinnyBlocks;
    return LinearPath::kPrefill;
}

// prefill.hip: LDS-tiled MFMA path for large M.  Tiles of kPrefillTile^2
// outputs.  The work is planned for kPlanCUs compute units: whole rounds of
// tiles run over all of K; the tiles of a last, partial round (or all tiles,
// when there are fewer than kPlanCUs) are split over K into ks parts so that
// the round is full, and their fp32 partial tiles (the workspace) are added
// up in part order by a second kernel.
constexpr int kPrefillTile = 256;
constexpr int kPlanCUs = 256;
struct PrefillPlan {
    int64_t tiles_m, tiles_n;
    int64_t full;  // tiles computed whole, by workgroups 0 .. full-1
    int ks;        // parts of each remaining tile
    int64_t grid;
};
inline PrefillPlan prefill_plan(int64_t M, int64_t N, int64_t K) {
    PrefillPlan p;
    p.tiles_m = (M + kPrefillTile - 1) / kPrefillTile;
    p.tiles_n = (N + kPrefillTile - 1) / kPrefillTile;
    const int64_t tiles = p.tiles_m * p.tiles_n;
    const int64_t steps = (K + 63) / 64;
    p.full = tiles >= kPlanCUs ? tiles / kPlanCUs * kPlanCUs : 0;
    const int64_t rem = tiles - p.full;
    int64_t ks = rem > 0 ? kPlanCUs / rem : 1;
    if (ks > steps / 4) ks = steps / 4;  // at least 4 k steps per part
    if (ks < 2) {
        p.full = tiles;
        ks = 1;
    }
    p.ks = (int)ks;
    p.grid = p.full + (tiles - p.full) * ks;
    return p;
}
inline size_t prefill_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const PrefillPlan p = prefill_plan(M, N, K);
    return (size_t)(p.tiles_m * p.tiles_n - p.full) * p.ks * kPrefillTile * kPrefillTile * sizeof(float);
}
hipError_t launch_prefill(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                          const float* alpha, bool per_row, YOut y, int64_t M, int64_t N,
                          int64_t K, void* workspace, hipStream_t stream);
const char* prefill_name();

// grouped.hip
size_t grouped_workspace_bytes(int64_t M, int32_t G, int64_t N, int64_t K);
// gdec.hip: grouped path at decode (M <= kGdecMaxM tokens): rows streamed
// once, VALU dot products per token, x one K range at a time in LDS
// (kGdXsBytes).  A workgroup owns kGdWaves x 2 x pairs rows for one K range
// of krc 512-wide chunks; with nkr > 1 ranges the fp32 partials of each range
// ([nkr][M][N] in the workspace) are added by reduce_kernel.  Same-process
// timings against the staged grouped kernel, 1..4 tokens on as many
// variants: 28672x8192 191..213 -> 95..139 us, 8192x8192 52..66 -> 30..47,
// 8192x28672 166..189 -> 90..144; at 8 tokens mixed, at 16 behind (the
// per-token sign loads and sums grow with the tokens), and on 1024 rows
// level at 1..2 tokens and behind at 3..4 (19..21 -> 23..28 us), so at
// least kGdecMinN rows.
constexpr int kGdecMaxM = 4;
constexpr int64_t kGdecMinN = 4096;
constexpr int kGdXsBytes = 65536;
struct GdecPlan {
    int mp;        // token positions compiled for
    int krc;       // chunks per K range
    int nkr;       // K ranges
    int pairs;     // row pairs per wave
    int64_t grid;  // workgroups (0: shape not served)
};
GdecPlan gdec_plan(int64_t M, int64_t N, int64_t K);
const char* gdec_name();
hipError_t launch_gdec(const uint16_t* x, const int32_t* ids, const uint16_t* w, const VariantTable& table,
                       bool per_row, int32_t G, float* y, int64_t M, int64_t N, int64_t K, float* part,
                       hipStream_t stream);
size_t grouped_plan_bytes(int64_t M, int32_t G);
hipError_t launch_grouped_plan(const int32_t* ids, int64_t M, int32_t G, void* workspace, hipStream_t stream);
// planned: the workspace already holds launch_grouped_plan's result for ids
hipError_t launch_grouped(const uint16_t* x, const int32_t* ids, const uint16_t* w,
                          const VariantTable& table, bool per_row, int32_t G, float* y,
                          int64_t M, int64_t N, int64_t K, void* workspace, bool planned,
                          hipStream_t stream);

}  // namespace bd
