// C ABI of libbitdelta: argument validation, workspace sizing and dispatch.
// Every check runs on the host before anything is enqueued; kernels only run
// on arguments that passed.  See include/bitdelta.h for the contract.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>

#include "../../include/bitdelta.h"
#include "bd_internal.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

constexpr int kMaxDevices = 64;
// 0 = not yet checked, 1 = gfx950, 2 = other.  Filled once per device,
// together with the device's compute unit count (grid sizing).
std::atomic<int> g_device_ok[kMaxDevices];
std::atomic<int> g_num_cu[kMaxDevices];

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;

bd_status hip_fail(hipError_t e) {
    g_last_hip_error = static_cast<int32_t>(e);
    return BD_ERR_HIP;
}

bd_status check_device(int* num_cu = nullptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices) return BD_ERR_DEVICE;
    int state = g_device_ok[dev].load(std::memory_order_acquire);
    if (state == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail(e);
        state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_num_cu[dev].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1,
                            std::memory_order_relaxed);
        g_device_ok[dev].store(state, std::memory_order_release);
    }
    if (num_cu) *num_cu = g_num_cu[dev].load(std::memory_order_relaxed);
    return state == 1 ? BD_OK : BD_ERR_DEVICE;
}

// Compute units of the current device for host-only queries: the cached
// count once a call has checked the device, else what HIP reports, else the
// MI355X's 256.
int host_num_cu() {
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
        if (g_device_ok[dev].load(std::memory_order_acquire) != 0)
            return g_num_cu[dev].load(std::memory_order_relaxed);
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            return n;
    }
    (void)hipGetLastError();
    return 256;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_mode(int32_t mode) { return mode == BD_ALPHA_PER_MATRIX || mode == BD_ALPHA_PER_ROW; }

bd_status check_matrix(int64_t d_out, int64_t d_in) {
    if (d_out < 1 || d_in < 8 || d_in % 8 != 0 || d_out > kMaxDim || d_in > kMaxDim)
        return BD_ERR_SHAPE;
    return BD_OK;
}

bd_status finish(hipError_t e) { return e == hipSuccess ? BD_OK : hip_fail(e); }

}  // namespace

namespace bd {
void note_hip_error(hipError_t e) { g_last_hip_error = static_cast<int32_t>(e); }
}  // namespace bd

extern "C" {

int32_t bd_abi_version(void) { return BD_ABI_VERSION; }

const char* bd_status_string(bd_status s) {
    switch (s) {
        case BD_OK: return "ok";
        case BD_ERR_NULL: return "a required pointer is NULL";
        case BD_ERR_SHAPE: return "invalid shape (need d_out >= 1, d_in >= 8, d_in % 8 == 0, M >= 0)";
        case BD_ERR_ALIGN: return "misaligned pointer (x, w_base, delta, y need 16-byte alignment)";
        case BD_ERR_WORKSPACE: return "workspace too small or misaligned";
        case BD_ERR_MODE: return "unknown alpha mode";
        case BD_ERR_HIP: return "HIP call failed";
        case BD_ERR_DEVICE: return "current device is not a gfx950 GPU";
    }
    return "unknown status";
}

int32_t bd_last_hip_error(void) { return g_last_hip_error; }

size_t bd_compress_workspace_bytes(int64_t d_out, int64_t d_in, int32_t mode) {
    (void)d_in;
    if (mode == BD_ALPHA_PER_MATRIX && d_out > 0) return static_cast<size_t>(d_out) * sizeof(double);
    return 0;
}

bd_status bd_compress(const float* delta, int64_t d_out, int64_t d_in, int32_t mode,
                      uint8_t* signs, float* alpha, void* workspace, size_t workspace_bytes,
                      void* stream) {
    if (!delta || !signs || !alpha) return BD_ERR_NULL;
    if (!valid_mode(mode)) return BD_ERR_MODE;
    bd_status st = check_matrix(d_out, d_in);
    if (st != BD_OK) return st;
    if (!aligned(delta, 16) || !aligned(alpha, 4)) return BD_ERR_ALIGN;
    size_t need = bd_compress_workspace_bytes(d_out, d_in, mode);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 8)))
        return BD_ERR_WORKSPACE;
    st = check_device();
    if (st != BD_OK) return st;
    return finish(bd::launch_compress(delta, d_out, d_in, mode == BD_ALPHA_PER_ROW, signs, alpha,
                                      static_cast<double*>(workspace),
                                      static_cast<hipStream_t>(stream)));
}

bd_status bd_compress_pair(const uint16_t* w_ft, const uint16_t* w_base, int64_t d_out,
                           int64_t d_in, int32_t mode, uint8_t* signs, float* alpha, void* workspace,
                           size_t workspace_bytes, void* stream) {
    if (!w_ft || !w_base || !signs || !alpha) return BD_ERR_NULL;
    if (!valid_mode(mode)) return BD_ERR_MODE;
    bd_status st = check_matrix(d_out, d_in);
    if (st != BD_OK) return st;
    if (!aligned(w_ft, 16) || !aligned(w_base, 16) || !aligned(alpha, 4)) return BD_ERR_ALIGN;
    size_t need = bd_compress_workspace_bytes(d_out, d_in, mode);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 8)))
        return BD_ERR_WORKSPACE;
    st = check_device();
    if (st != BD_OK) return st;
    return finish(bd::launch_compress_pair(w_ft, w_base, d_out, d_in, mode == BD_ALPHA_PER_ROW, signs,
                                           alpha, static_cast<double*>(workspace),
                                           static_cast<hipStream_t>(stream)));
}

size_t bd_linear_workspace_bytes(int64_t M, int64_t d_out, int64_t d_in) {
    // the slice path's K-split planes, or the tiled prefill path's split tiles
    if (d_out <= 0 || d_in < 8) return 0;
    if (bd::use_slice(M, d_out, d_in)) return bd::slice_workspace_bytes(M, d_out, d_in);
    if (M <= bd::kSkinnyMaxM || d_in > bd::kPrefillMaxK) return 0;
    return bd::prefill_workspace_bytes(M, d_out, d_in);
}

}  // extern "C"

namespace {
// bd_linear and bd_linear_bf16: the same checks and dispatch; y is fp32 or bf16.
bd_status linear_common(const uint16_t* x, const uint16_t* w_base, const uint8_t* signs,
                        const float* alpha, int32_t mode, void* y, bool y_bf16, int64_t M, int64_t d_out,
                        int64_t d_in, void* workspace, size_t workspace_bytes, void* stream) {
    if (!w_base || !signs || !alpha) return BD_ERR_NULL;
    if (M > 0 && (!x || !y)) return BD_ERR_NULL;
    if (!valid_mode(mode)) return BD_ERR_MODE;
    bd_status st = check_matrix(d_out, d_in);
    if (st != BD_OK) return st;
    if (M < 0 || M > kMaxDim) return BD_ERR_SHAPE;
    if (!aligned(w_base, 16) || !aligned(alpha, 4) || (M > 0 && (!aligned(x, 16) || !aligned(y, 16))))
        return BD_ERR_ALIGN;
    if (M == 0) return BD_OK;
    const size_t need = bd_linear_workspace_bytes(M, d_out, d_in);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
        return BD_ERR_WORKSPACE;
    int num_cu = 0;
    st = check_device(&num_cu);
    if (st != BD_OK) return st;
    const bd::LinearPath path = bd::choose_linear_path(M, d_out, d_in, num_cu);
    const bool per_row = mode == BD_ALPHA_PER_ROW;
    const bd::YOut yo{y, y_bf16 ? 1 : 0};
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (path) {
        case bd::LinearPath::kGemv:
            return finish(bd::launch_gemv(x, w_base, signs, alpha, per_row, yo, M, d_out, d_in, s));
        case bd::LinearPath::kXres:
            return finish(bd::launch_xres(x, w_base, signs, alpha, per_row, yo, M, d_out, d_in, num_cu, s));
        case bd::LinearPath::kSlice:
            return finish(bd::launch_slice(x, w_base, signs, alpha, per_row, yo, M, d_out, d_in, workspace, s));
        case bd::LinearPath::kBand:
            return finish(bd::launch_band(x, w_base, signs, alpha, per_row, yo, M, d_out, d_in, num_cu, s));
        case bd::LinearPath::kQuad:
            return finish(bd::launch_quad(x, w_base, signs, alpha, per_row, yo, M, d_out, d_in, num_cu, s));
        case bd::LinearPath::kXstat:
            return finish(bd::launch_xstat(x, w_base, signs, alpha, per_row, yo, M, d_out, d_in,
                                           num_cu, s));
        case bd::LinearPath::kShot:
            return finish(bd::launch_shot(x, w_base, signs, alpha, per_row, yo, M, d_out, d_in, s));
        case bd::LinearPath::kRowstream:
            return finish(bd::launch_rowstream(x, w_base, signs, alpha, per_row, yo, M, d_out, d_in, num_cu, s));
        case bd::LinearPath::kSkinny:
            return finish(bd::launch_skinny(x, w_base, signs, alpha, per_row, yo, M, d_out, d_in, s));
        case bd::LinearPath::kSkinnyBlocks:
            for (int64_t m0 = 0; m0 < M; m0 += bd::kSkinnyMaxM) {
                const int64_t mb = M - m0 < bd::kSkinnyMaxM ? M - m0 : bd::kSkinnyMaxM;
                const hipError_t e = bd::launch_skinny(x + m0 * d_in, w_base, signs, alpha, per_row,
                                                       bd::y_at(yo, m0 * d_out), mb, d_out, d_in, s);
                if (e != hipSuccess) return finish(e);
            }
            return BD_OK;
        case bd::LinearPath::kPrefill:
            break;
    }
    return finish(bd::launch_prefill(x, w_base, signs, alpha, per_row, yo, M, d_out, d_in, workspace, s));
}
}  // namespace

extern "C" {

bd_status bd_linear(const uint16_t* x, const uint16_t* w_base, const uint8_t* signs,
                    const float* alpha, int32_t mode, float* y, int64_t M, int64_t d_out,
                    int64_t d_in, void* workspace, size_t workspace_bytes, void* stream) {
    return linear_common(x, w_base, signs, alpha, mode, y, false, M, d_out, d_in, workspace, workspace_bytes,
                         stream);
}

bd_status bd_linear_bf16(const uint16_t* x, const uint16_t* w_base, const uint8_t* signs,
                         const float* alpha, int32_t mode, uint16_t* y, int64_t M, int64_t d_out,
                         int64_t d_in, void* workspace, size_t workspace_bytes, void* stream) {
    return linear_common(x, w_base, signs, alpha, mode, y, true, M, d_out, d_in, workspace, workspace_bytes,
                         stream);
}

const char* bd_linear_path(int64_t M, int64_t d_out, int64_t d_in) {
    if (M <= 0 || d_out <= 0 || d_in < 8) return "";
    const int num_cu = host_num_cu();
    switch (bd::choose_linear_path(M, d_out, d_in, num_cu)) {
        case bd::LinearPath::kGemv: return bd::gemv_name(M, d_out, d_in);
        case bd::LinearPath::kXres: return bd::xres_name(M, d_in);
        case bd::LinearPath::kSlice: return bd::slice_name();
        case bd::LinearPath::kBand: return bd::band_name();
        case bd::LinearPath::kQuad: return bd::quad_name(d_out);
        case bd::LinearPath::kXstat: return bd::xstat_name(M, d_out, d_in, num_cu);
        case bd::LinearPath::kShot: return bd::shot_name();
        case bd::LinearPath::kRowstream: return bd::rowstream_name(M, d_out, num_cu);
        case bd::LinearPath::kSkinny: return bd::skinny_name(M, d_out);
        case bd::LinearPath::kSkinnyBlocks: return bd::skinny_name(bd::kSkinnyMaxM, d_out);
        case bd::LinearPath::kPrefill: break;
    }
    return bd::prefill_name();
}

size_t bd_linear_grouped_workspace_bytes(int64_t M, int64_t d_out, int64_t d_in,
                                         int32_t num_variants) {
    if (M <= 0 || d_out <= 0 || d_in <= 0 || num_variants < 1 || num_variants > BD_MAX_VARIANTS) return 0;
    return bd::grouped_workspace_bytes(M, num_variants, d_out, d_in);
}

}  // extern "C"

// The grouped linear without any allocation: its workspace is a fixed device
// array of the library (one per GPU), for callers that cannot allocate.
namespace {

static __device__ __align__(256) unsigned char scratch[BD_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on each device, looked up once per device
// (the array's host-side name is not a device address).
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

bd_status scratch_of_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices) return BD_ERR_DEVICE;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol);
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return BD_OK;
}

}  // namespace

namespace {
// use_scratch: the workspace is the current device's `scratch` array (the
// workspace arguments are ignored), for bd_linear_grouped_noalloc.
bd_status grouped_common(const uint16_t* x, const int32_t* variant_ids, const uint16_t* w_base,
                         const uint8_t* const* signs, const float* const* alpha, int32_t mode,
                         int32_t num_variants, float* y, int64_t M, int64_t d_out, int64_t d_in,
                         void* workspace, size_t workspace_bytes, bool planned, void* stream,
                         bool use_scratch = false) {
    if (!w_base || !signs || !alpha) return BD_ERR_NULL;
    if (M > 0 && (!x || !y || !variant_ids)) return BD_ERR_NULL;
    if (!valid_mode(mode)) return BD_ERR_MODE;
    bd_status st = check_matrix(d_out, d_in);
    if (st != BD_OK) return st;
    if (M < 0 || M > kMaxDim || num_variants < 1 || num_variants > BD_MAX_VARIANTS)
        return BD_ERR_SHAPE;
    bd::VariantTable table;
    std::memset(&table, 0, sizeof(table));
    for (int32_t g = 0; g < num_variants; ++g) {
        if (!signs[g] || !alpha[g]) return BD_ERR_NULL;
        if (!aligned(alpha[g], 4)) return BD_ERR_ALIGN;
        table.signs[g] = signs[g];
        table.alpha[g] = alpha[g];
    }
    if (!aligned(w_base, 16) ||
        (M > 0 && (!aligned(x, 16) || !aligned(y, 16) || !aligned(variant_ids, 4))))
        return BD_ERR_ALIGN;
    if (M == 0) return BD_OK;
    size_t need = bd_linear_grouped_workspace_bytes(M, d_out, d_in, num_variants);
    if (use_scratch) {
        if (need > BD_NOALLOC_SCRATCH_BYTES) return BD_ERR_WORKSPACE;
    } else if (!workspace || workspace_bytes < need || !aligned(workspace, 8)) {
        return BD_ERR_WORKSPACE;
    }
    st = check_device();
    if (st != BD_OK) return st;
    if (use_scratch) {
        st = scratch_of_current_device(&workspace);
        if (st != BD_OK) return st;
    }
    return finish(bd::launch_grouped(x, variant_ids, w_base, table, mode == BD_ALPHA_PER_ROW,
                                     num_variants, y, M, d_out, d_in, workspace, planned,
                                     static_cast<hipStream_t>(stream)));
}
}  // namespace

extern "C" {

bd_status bd_linear_grouped(const uint16_t* x, const int32_t* variant_ids,
                            const uint16_t* w_base, const uint8_t* const* signs,
                            const float* const* alpha, int32_t mode, int32_t num_variants,
                            float* y, int64_t M, int64_t d_out, int64_t d_in, void* workspace,
                            size_t workspace_bytes, void* stream) {
    return grouped_common(x, variant_ids, w_base, signs, alpha, mode, num_variants, y, M, d_out, d_in,
                          workspace, workspace_bytes, false, stream);
}

size_t bd_linear_grouped_plan_bytes(int64_t M, int32_t num_variants) {
    if (M <= 0 || num_variants < 1 || num_variants > BD_MAX_VARIANTS) return 0;
    return bd::grouped_plan_bytes(M, num_variants);
}

bd_status bd_linear_grouped_plan(const int32_t* variant_ids, int64_t M, int32_t num_variants,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    if (M < 0 || M > kMaxDim || num_variants < 1 || num_variants > BD_MAX_VARIANTS) return BD_ERR_SHAPE;
    if (M == 0) return BD_OK;
    if (!variant_ids) return BD_ERR_NULL;
    if (!aligned(variant_ids, 4)) return BD_ERR_ALIGN;
    if (!workspace || workspace_bytes < bd_linear_grouped_plan_bytes(M, num_variants) || !aligned(workspace, 8))
        return BD_ERR_WORKSPACE;
    const bd_status st = check_device();
    if (st != BD_OK) return st;
    return finish(bd::launch_grouped_plan(variant_ids, M, num_variants, workspace,
                                          static_cast<hipStream_t>(stream)));
}

bd_status bd_linear_grouped_planned(const uint16_t* x, const int32_t* variant_ids,
                                    const uint16_t* w_base, const uint8_t* const* signs,
                                    const float* const* alpha, int32_t mode, int32_t num_variants,
                                    float* y, int64_t M, int64_t d_out, int64_t d_in, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    return grouped_common(x, variant_ids, w_base, signs, alpha, mode, num_variants, y, M, d_out, d_in,
                          workspace, workspace_bytes, true, stream);
}

}  // extern "C"


extern "C" {

bd_status bd_linear_grouped_noalloc(const uint16_t* x, const int32_t* variant_ids,
                                    const uint16_t* w_base, const uint8_t* const* signs,
                                    const float* const* alpha, int32_t mode, int32_t num_variants,
                                    float* y, int64_t M, int64_t d_out, int64_t d_in, void* stream) {
    return grouped_common(x, variant_ids, w_base, signs, alpha, mode, num_variants, y, M, d_out, d_in,
                          nullptr, 0, false, stream, true);
}

}  // extern "C"
