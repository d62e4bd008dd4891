// Measurement aid, not part of the BitDelta path: plain streaming reads of a
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

// The decode GEMV's access pattern without its arithmetic: the buffer as
// `rows` rows of `row_bytes` (a multiple of U KiB; rows even).  Wave g of the
// grid reads row pairs g, g + waves, ...; per batch U 1 KiB pieces of each of
// its two rows (lane l: bytes 16 l .. 16 l + 15 of a piece), the next batch's
// loads issued before the current one is folded in.  Every load lies inside
// the buffer: pieces c < row_bytes / 1024 of rows below `rows`.
template <int U>
__global__ __launch_bounds__(256) void stream_rows_kernel(const uint8_t* __restrict__ p, int64_t rows,
                                                          int64_t row_bytes, uint32_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t wave = tid >> 6, nwaves = (int64_t)gridDim.x * 4;
    const int64_t pieces = row_bytes / 1024;
    u32x4_t acc = {0, 0, 0, 0};
    for (int64_t pr = wave; 2 * pr + 1 < rows; pr += nwaves) {
        const uint8_t* r0 = p + 2 * pr * row_bytes + 16 * lane;
        const uint8_t* r1 = r0 + row_bytes;
        u32x4_t cur[2][U], nxt[2][U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            cur[0][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(r0 + u * 1024));
            cur[1][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(r1 + u * 1024));
        }
        for (int64_t c = 0; c < pieces; c += U) {
            const int64_t cn = c + U < pieces ? c + U : c;  // the last batch reloads itself (in bounds)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                nxt[0][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(r0 + (cn + u) * 1024));
                nxt[1][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(r1 + (cn + u) * 1024));
            }
#pragma unroll
            for (int u = 0; u < U; ++u) acc ^= cur[0][u] ^ cur[1][u];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                cur[0][u] = nxt[0][u];
                cur[1][u] = nxt[1][u];
            }
        }
    }
    out[tid] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// The one-token GEMV's present pattern: workgroup b (4 waves) reads row pair
// b, its waves splitting the pair's 1 KiB pieces (wave w: pieces w, w + 4,
// ...), all of a wave's loads of a batch of 4 pieces issued together, then
// exits.  rows/2 workgroups; row_bytes a multiple of 4 KiB, so every piece
// index is below row_bytes / 1024 and every row below `rows`.  The XOR of
// what a lane read is stored only if it equals a value the data never gives
// (`out` slot taken modulo out_threads), so the loads stay and no slot is
// written out of bounds.
__global__ __launch_bounds__(256) void stream_pairs_kernel(const uint8_t* __restrict__ p, int64_t row_bytes,
                                                           uint32_t* __restrict__ out, int64_t out_threads) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint8_t* r0 = p + 2 * (int64_t)blockIdx.x * row_bytes + 16 * lane;
    const uint8_t* r1 = r0 + row_bytes;
    const int64_t per_wave = row_bytes / 4096;  // pieces of each row per wave
    u32x4_t acc = {0, 0, 0, 0};
    for (int64_t u0 = 0; u0 < per_wave; u0 += 4) {
        u32x4_t v[2][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t piece = wave + 4 * (u0 + u < per_wave ? u0 + u : u0);
            v[0][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(r0 + piece * 1024));
            v[1][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(r1 + piece * 1024));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= v[0][u] ^ v[1][u];
    }
    const uint32_t h = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (h == 0x9e3779b9u) out[((int64_t)blockIdx.x * 256 + threadIdx.x) % out_threads] = h;
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

// Read `rows` rows of `row_bytes` at `buf` once in the GEMV's pattern (two
// rows per wave, `batch` (2 or 4) 1 KiB pieces of each in flight), with
// `wg_per_cu` (1..16) workgroups of 4 waves per compute unit.  rows must be
// even and row_bytes a multiple of batch KiB; `out` as for
// bd_probe_stream_read.  Returns a hipError_t as int.
int32_t bd_probe_stream_rows(const void* buf, int64_t rows, int64_t row_bytes, uint32_t* out, int32_t num_cu,
                             int32_t wg_per_cu, int32_t batch, void* stream) {
    if (!buf || !out || rows < 2 || rows % 2 != 0 || (batch != 2 && batch != 4) || row_bytes < 1024 * batch ||
        row_bytes % (1024 * batch) != 0 || (reinterpret_cast<uintptr_t>(buf) & 15) || num_cu < 1 || wg_per_cu < 1 ||
        wg_per_cu > 16)
        return (int32_t)hipErrorInvalidValue;
    const dim3 grid((unsigned)(num_cu * wg_per_cu));
    const uint8_t* p = static_cast<const uint8_t*>(buf);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (batch == 2) hipLaunchKernelGGL(stream_rows_kernel<2>, grid, dim3(256), 0, s, p, rows, row_bytes, out);
    else hipLaunchKernelGGL(stream_rows_kernel<4>, grid, dim3(256), 0, s, p, rows, row_bytes, out);
    return (int32_t)hipGetLastError();
}

// Read `rows` rows of `row_bytes` at `buf` once in the one-token GEMV's
// present pattern (one workgroup of 4 waves per row pair, the waves splitting
// the pair's 1 KiB pieces, rows/2 workgroups).  rows must be even and
// row_bytes a multiple of 4 KiB; `out` as for bd_probe_stream_read.  Returns
// a hipError_t as int.
int32_t bd_probe_stream_pairs(const void* buf, int64_t rows, int64_t row_bytes, uint32_t* out, int32_t num_cu,
                              void* stream) {
    if (!buf || !out || rows < 2 || rows % 2 != 0 || rows / 2 > 0x7fffffff || row_bytes < 4096 ||
        row_bytes % 4096 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15) || num_cu < 1)
        return (int32_t)hipErrorInvalidValue;
    const uint8_t* p = static_cast<const uint8_t*>(buf);
    hipLaunchKernelGGL(stream_pairs_kernel, dim3((unsigned)(rows / 2)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), p, row_bytes, out, bd_probe_stream_read_threads(num_cu));
    return (int32_t)hipGetLastError();
}

}  // extern "C"
