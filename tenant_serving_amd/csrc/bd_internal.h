// Host-side launch entry points of the BitDelta kernels.  The C ABI layer
// validates every argument before calling these; they only size grids and
// enqueue work on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bd {

constexpr int kMaxVariants = 64;

// Per-variant delta-cache entries, passed to kernels by value.
struct VariantTable {
    const uint8_t* signs[kMaxVariants];
    const float* alpha[kMaxVariants];
};

// compress.hip
hipError_t launch_compress(const float* delta, int64_t d_out, int64_t d_in, bool per_row,
                           uint8_t* signs, float* alpha, double* row_sums, hipStream_t stream);

// gemv.hip: VALU dot-product path, 1 <= M <= kGemvMaxM
constexpr int kGemvMaxM = 4;
hipError_t launch_gemv(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                       const float* alpha, bool per_row, float* y, int64_t M, int64_t N,
                       int64_t K, hipStream_t stream);
const char* gemv_name(int64_t M);

// skinny.hip: MFMA path for M <= kSkinnyMaxM
constexpr int kSkinnyMaxM = 64;
const char* skinny_name(int64_t M, int64_t N);
hipError_t launch_skinny(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                         const float* alpha, bool per_row, float* y, int64_t M, int64_t N,
                         int64_t K, hipStream_t stream);

// rowstream.hip: MFMA path for M <= kRowstreamMaxM on projections with many
// rows (workgroups of 32 rows, each wave streaming whole rows)
constexpr int kRowstreamMaxM = 32;
hipError_t launch_rowstream(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                            const float* alpha, bool per_row, float* y, int64_t M, int64_t N,
                            int64_t K, hipStream_t stream);
const char* rowstream_name(int64_t M);

// Which decode/prefill path serves bd_linear for a shape.
enum class LinearPath { kGemv, kRowstream, kSkinny, kPrefill };
inline LinearPath choose_linear_path(int64_t M, int64_t N) {
    // One token, or a few tokens on a projection with few rows: VALU dot
    // products.  2..32 tokens on projections of 4096..16384 rows: the
    // row-streaming MFMA path (one or two waves of 32-row workgroups).
    // Otherwise up to 64 tokens: the skinny MFMA path; beyond: LDS tiles.
    if (M == 1 || (M <= kGemvMaxM && N < 8192)) return LinearPath::kGemv;
    if (M <= kRowstreamMaxM && N >= 4096 && N <= 16384) return LinearPath::kRowstream;
    if (M <= kSkinnyMaxM) return LinearPath::kSkinny;
    return LinearPath::kPrefill;
}

// prefill.hip: LDS-tiled MFMA path for large M
hipError_t launch_prefill(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                          const float* alpha, bool per_row, float* y, int64_t M, int64_t N,
                          int64_t K, hipStream_t stream);
const char* prefill_name();

// grouped.hip
size_t grouped_workspace_bytes(int64_t M, int32_t G, int64_t N);
hipError_t launch_grouped(const uint16_t* x, const int32_t* ids, const uint16_t* w,
                          const VariantTable& table, bool per_row, int32_t G, float* y,
                          int64_t M, int64_t N, int64_t K, void* workspace, hipStream_t stream);

}  // namespace bd
