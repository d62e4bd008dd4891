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

// skinny.hip: MFMA path for M <= kSkinnyMaxM (used for 2..4 tokens only when
// d_out >= kSkinnyMinRowsSmallM)
constexpr int kSkinnyMaxM = 64;
constexpr int64_t kSkinnyMinRowsSmallM = 8192;
hipError_t launch_skinny(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                         const float* alpha, bool per_row, float* y, int64_t M, int64_t N,
                         int64_t K, hipStream_t stream);

// prefill.hip: LDS-tiled MFMA path for large M
hipError_t launch_prefill(const uint16_t* x, const uint16_t* w, const uint8_t* signs,
                          const float* alpha, bool per_row, float* y, int64_t M, int64_t N,
                          int64_t K, hipStream_t stream);

// grouped.hip
size_t grouped_workspace_bytes(int64_t M, int32_t G, int64_t N);
hipError_t launch_grouped(const uint16_t* x, const int32_t* ids, const uint16_t* w,
                          const VariantTable& table, bool per_row, int32_t G, float* y,
                          int64_t M, int64_t N, int64_t K, void* workspace, hipStream_t stream);

}  // namespace bd
