// Measurement aid, not part of the BitDelta path: a plain streaming read of a
// device buffer, the achievable read rate that the decode kernels' HBM
// fractions are read against (the graded denominator stays the 8 TB/s
// published peak).  Built into its own library, libbdprobe.so, which only the
// benchmark loads.
//
// Each lane reads 16-byte words with non-temporal loads, four per trip, in a
// grid-stride loop over [0, bytes/16); the XOR of what it read goes to
// out[global thread], so nothing is optimised away.  Every load index is
// below bytes/16 and every store index below the grid's thread count, which
// the caller sizes `out` for.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ p, int64_t n16,
                                                          uint32_t* __restrict__ out) {
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * 256;
    u32x4_t acc = {0, 0, 0, 0};
    int64_t i = tid;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
    out[tid] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

extern "C" {

// Threads of the largest launch (the size, in uint32 words, that `out` must
// have): 16 workgroups of 256 threads per compute unit.
int64_t bd_probe_stream_read_threads(int32_t num_cu) { return (int64_t)num_cu * 16 * 256; }

// Read `bytes` (a multiple of 16, 16-byte aligned) at device pointer `buf`
// once on `stream`, with `wg_per_cu` (1..16) workgroups per compute unit and
// `loads` (4 or 8) 16-byte loads in flight per lane; `out` is a device buffer
// of bd_probe_stream_read_threads uint32 words.  Returns a hipError_t as int.
int32_t bd_probe_stream_read(const void* buf, int64_t bytes, uint32_t* out, int32_t num_cu, int32_t wg_per_cu,
                             int32_t loads, void* stream) {
    if (!buf || !out || bytes < 16 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15) || num_cu < 1 ||
        wg_per_cu < 1 || wg_per_cu > 16 || (loads != 4 && loads != 8))
        return (int32_t)hipErrorInvalidValue;
    const dim3 grid((unsigned)(num_cu * wg_per_cu));
    const u32x4_t* p = static_cast<const u32x4_t*>(buf);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (loads == 4) hipLaunchKernelGGL(stream_read_kernel<4>, grid, dim3(256), 0, s, p, bytes / 16, out);
    else hipLaunchKernelGGL(stream_read_kernel<8>, grid, dim3(256), 0, s, p, bytes / 16, out);
    return (int32_t)hipGetLastError();
}

}  // extern "C"
