/*
 * A plain C program that uses libbitdelta through its C ABI only: the
 * library is opened with dlopen and every entry point is looked up by the
 * name include/bitdelta.h declares; device memory and the stream come from
 * the HIP runtime.  No Python and no torch.  Test infrastructure: a GPU test
 * feeds it seeded inputs through files and checks its outputs against the
 * oracle.
 *
 * Usage: bd_client LIB DIR N K M G
 *   reads  DIR/delta.f32 (G x [N, K] fp32), DIR/w.bf16 ([N, K]),
 *          DIR/x.bf16 ([M, K]), DIR/ids.i32 ([M])
 *   writes DIR/signs.u8 (G x [N, K/8]), DIR/alpha.f32 (G x [N]),
 *          DIR/y.f32 ([M, N], variant 0 for every token: bd_linear),
 *          DIR/yg.f32 ([M, N], token m on variant ids[m]: bd_linear_grouped)
 * Compress and linear use one scale per output row.  Exit status 0 on
 * success; otherwise the failing call and its status are printed.
 */
#include <dlfcn.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "bitdelta.h"

#define LOOKUP(h, name) __typeof__(&name) p_##name = (__typeof__(&name))dlsym(h, #name)

static int fail(const char* what, const char* why) {
    fprintf(stderr, "bd_client: %s: %s\n", what, why);
    return 1;
}

static void* read_file(const char* dir, const char* name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) return NULL;
    void* p = malloc(bytes ? bytes : 1);
    if (p && fread(p, 1, bytes, f) != bytes) {
        free(p);
        p = NULL;
    }
    fclose(f);
    return p;
}

static int write_file(const char* dir, const char* name, const void* p, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "wb");
    if (!f) return 1;
    const int bad = fwrite(p, 1, bytes, f) != bytes;
    fclose(f);
    return bad;
}

static void* dev_alloc(size_t bytes) {
    void* p = NULL;
    return hipMalloc(&p, bytes ? bytes : 16) == hipSuccess ? p : NULL;
}

int main(int argc, char** argv) {
    if (argc != 7) return fail("usage", "bd_client LIB DIR N K M G");
    const char* dir = argv[2];
    const int64_t N = atoll(argv[3]), K = atoll(argv[4]), M = atoll(argv[5]);
    const int32_t G = atoi(argv[6]);
    if (N < 1 || K < 8 || K % 8 || M < 1 || G < 1 || G > BD_MAX_VARIANTS) return fail("arguments", "bad sizes");

    void* h = dlopen(argv[1], RTLD_NOW | RTLD_LOCAL);
    if (!h) return fail("dlopen", dlerror());
    LOOKUP(h, bd_abi_version);
    LOOKUP(h, bd_status_string);
    LOOKUP(h, bd_compress_workspace_bytes);
    LOOKUP(h, bd_compress);
    LOOKUP(h, bd_linear_workspace_bytes);
    LOOKUP(h, bd_linear);
    LOOKUP(h, bd_linear_grouped_workspace_bytes);
    LOOKUP(h, bd_linear_grouped);
    if (!p_bd_abi_version || !p_bd_status_string || !p_bd_compress_workspace_bytes || !p_bd_compress ||
        !p_bd_linear_workspace_bytes || !p_bd_linear || !p_bd_linear_grouped_workspace_bytes ||
        !p_bd_linear_grouped)
        return fail("dlsym", "an entry point is missing");
    if (p_bd_abi_version() != BD_ABI_VERSION) return fail("bd_abi_version", "mismatch with the header");

    const size_t nk = (size_t)N * (size_t)K, sb = nk / 8;
    float* delta = read_file(dir, "delta.f32", (size_t)G * nk * 4);
    uint16_t* w = read_file(dir, "w.bf16", nk * 2);
    uint16_t* x = read_file(dir, "x.bf16", (size_t)M * K * 2);
    int32_t* ids = read_file(dir, "ids.i32", (size_t)M * 4);
    if (!delta || !w || !x || !ids) return fail("inputs", "cannot read the input files");

    hipStream_t stream;
    if (hipStreamCreate(&stream) != hipSuccess) return fail("hipStreamCreate", "failed");
    float* d_delta = dev_alloc(nk * 4);
    uint16_t* d_w = dev_alloc(nk * 2);
    uint16_t* d_x = dev_alloc((size_t)M * K * 2);
    int32_t* d_ids = dev_alloc((size_t)M * 4);
    float* d_y = dev_alloc((size_t)M * N * 4);
    uint8_t* d_signs[BD_MAX_VARIANTS];
    float* d_alpha[BD_MAX_VARIANTS];
    for (int g = 0; g < G; ++g) {
        d_signs[g] = dev_alloc(sb);
        d_alpha[g] = dev_alloc((size_t)N * 4);
        if (!d_signs[g] || !d_alpha[g]) return fail("hipMalloc", "out of memory");
    }
    if (!d_delta || !d_w || !d_x || !d_ids || !d_y) return fail("hipMalloc", "out of memory");
    if (hipMemcpy(d_w, w, nk * 2, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(d_x, x, (size_t)M * K * 2, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(d_ids, ids, (size_t)M * 4, hipMemcpyHostToDevice) != hipSuccess)
        return fail("hipMemcpy", "failed");

    /* compress every variant (per-row alpha needs no workspace) */
    const size_t cws = p_bd_compress_workspace_bytes(N, K, BD_ALPHA_PER_ROW);
    void* d_cws = cws ? dev_alloc(cws) : NULL;
    for (int g = 0; g < G; ++g) {
        if (hipMemcpy(d_delta, delta + (size_t)g * nk, nk * 4, hipMemcpyHostToDevice) != hipSuccess)
            return fail("hipMemcpy", "failed");
        const bd_status st = p_bd_compress(d_delta, N, K, BD_ALPHA_PER_ROW, d_signs[g], d_alpha[g], d_cws, cws,
                                           stream);
        if (st != BD_OK) return fail("bd_compress", p_bd_status_string(st));
        /* the next copy into d_delta must not overtake this compression */
        if (hipStreamSynchronize(stream) != hipSuccess) return fail("hipStreamSynchronize", "failed");
    }

    /* the fused linear on variant 0 */
    const size_t lws = p_bd_linear_workspace_bytes(M, N, K);
    void* d_lws = lws ? dev_alloc(lws) : NULL;
    bd_status st = p_bd_linear(d_x, d_w, d_signs[0], d_alpha[0], BD_ALPHA_PER_ROW, d_y, M, N, K, d_lws, lws,
                               stream);
    if (st != BD_OK) return fail("bd_linear", p_bd_status_string(st));
    float* y = malloc((size_t)M * N * 4);
    if (!y) return fail("malloc", "out of memory");
    if (hipStreamSynchronize(stream) != hipSuccess ||
        hipMemcpy(y, d_y, (size_t)M * N * 4, hipMemcpyDeviceToHost) != hipSuccess)
        return fail("hipMemcpy", "failed");
    if (write_file(dir, "y.f32", y, (size_t)M * N * 4)) return fail("outputs", "cannot write y");

    /* the grouped linear: token m on variant ids[m] */
    const size_t gws = p_bd_linear_grouped_workspace_bytes(M, N, K, G);
    void* d_gws = gws ? dev_alloc(gws) : NULL;
    if (gws && !d_gws) return fail("hipMalloc", "out of memory");
    st = p_bd_linear_grouped(d_x, d_ids, d_w, (const uint8_t* const*)d_signs, (const float* const*)d_alpha,
                             BD_ALPHA_PER_ROW, G, d_y, M, N, K, d_gws, gws, stream);
    if (st != BD_OK) return fail("bd_linear_grouped", p_bd_status_string(st));
    if (hipStreamSynchronize(stream) != hipSuccess ||
        hipMemcpy(y, d_y, (size_t)M * N * 4, hipMemcpyDeviceToHost) != hipSuccess)
        return fail("hipMemcpy", "failed");
    if (write_file(dir, "yg.f32", y, (size_t)M * N * 4)) return fail("outputs", "cannot write yg");

    /* compressed outputs of every variant */
    uint8_t* signs = malloc((size_t)G * sb);
    float* alpha = malloc((size_t)G * N * 4);
    if (!signs || !alpha) return fail("malloc", "out of memory");
    for (int g = 0; g < G; ++g)
        if (hipMemcpy(signs + (size_t)g * sb, d_signs[g], sb, hipMemcpyDeviceToHost) != hipSuccess ||
            hipMemcpy(alpha + (size_t)g * N, d_alpha[g], (size_t)N * 4, hipMemcpyDeviceToHost) != hipSuccess)
            return fail("hipMemcpy", "failed");
    if (write_file(dir, "signs.u8", signs, (size_t)G * sb) ||
        write_file(dir, "alpha.f32", alpha, (size_t)G * N * 4))
        return fail("outputs", "cannot write signs or alpha");

    for (int g = 0; g < G; ++g) {
        (void)hipFree(d_signs[g]);
        (void)hipFree(d_alpha[g]);
    }
    (void)hipFree(d_delta);
    (void)hipFree(d_w);
    (void)hipFree(d_x);
    (void)hipFree(d_ids);
    (void)hipFree(d_y);
    if (d_cws) (void)hipFree(d_cws);
    if (d_lws) (void)hipFree(d_lws);
    if (d_gws) (void)hipFree(d_gws);
    (void)hipStreamDestroy(stream);
    free(delta);
    free(w);
    free(x);
    free(ids);
    free(y);
    free(signs);
    free(alpha);
    printf("bd_client: ok\n");
    return 0;
}
