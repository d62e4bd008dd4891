"""The C-ABI library loads on any host and exports what include/bitdelta.h
declares; argument validation happens on the host before any HIP call, so
it can be exercised without a GPU.  No compute call is made here."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(bd_[a-z_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    from tenant_serving_amd import bitdelta
    if not os.path.exists(bitdelta.LIBRARY):
        from tenant_serving_amd import build
        build.build()
    return bitdelta.library()


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("bd_compress", "bd_compress_pair", "bd_linear", "bd_linear_grouped",
                     "bd_compress_workspace_bytes",
                     "bd_linear_workspace_bytes", "bd_linear_grouped_workspace_bytes",
                     "bd_abi_version", "bd_status_string", "bd_last_hip_error",
                     "bd_cache_create", "bd_cache_acquire", "bd_cache_acquire_batch",
                     "bd_cache_release", "bd_cache_request"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_and_status_strings(lib):
    assert lib.bd_abi_version() == 4
    for s in range(8):
        assert lib.bd_status_string(s).decode()
    assert lib.bd_status_string(0).decode() == "ok"
    assert lib.bd_last_hip_error() == 0


def test_workspace_queries(lib):
    assert lib.bd_compress_workspace_bytes(28672, 8192, 0) == 28672 * 8
    assert lib.bd_compress_workspace_bytes(28672, 8192, 1) == 0
    for M in (0, 1, 4, 16, 64, 2048):
        assert lib.bd_linear_workspace_bytes(M, 8192, 8192) == 0
    # tiled path: the tiles of a partial last round of 256 are split over K
    tile = 256 * 256 * 4
    assert lib.bd_linear_workspace_bytes(2048, 28672, 8192) == 128 * 2 * tile   # 896 tiles
    assert lib.bd_linear_workspace_bytes(2048, 1024, 8192) == 32 * 8 * tile     # 32 tiles
    assert lib.bd_linear_workspace_bytes(300, 300, 520) == 4 * 2 * tile         # >= 4 k steps a part
    assert lib.bd_linear_workspace_bytes(65, 256, 128) == 0                     # too short to split
    # slice path: one fp32 plane of M x d_out per 2048-wide slice of d_in,
    # none with one slice; sized wherever the path may run, whatever the device
    assert lib.bd_linear_workspace_bytes(16, 1024, 8192) == 4 * 16 * 1024 * 4
    assert lib.bd_linear_workspace_bytes(3, 2050, 5000) == 3 * 3 * 2050 * 4
    assert lib.bd_linear_workspace_bytes(16, 4095, 2048) == 0
    assert lib.bd_linear_workspace_bytes(12, 1024, 8192) == 0
    assert lib.bd_linear_workspace_bytes(2, 2048, 8192) == 0
    # rows longer than the tiled path's 32-bit tile offsets allow: 64-token
    # blocks on the skinny path, no workspace
    kmax = (1 << 23) - 8
    assert lib.bd_linear_workspace_bytes(2048, 256, kmax) > 0
    assert lib.bd_linear_workspace_bytes(2048, 256, kmax + 8) == 0
    g = lib.bd_linear_grouped_workspace_bytes(256, 8192, 28672, 14)
    assert g >= 256 * 8192 * 4  # at least one partial output buffer
    assert lib.bd_linear_grouped_workspace_bytes(256, 8192, 28672, 65) == 0
    assert lib.bd_linear_grouped_workspace_bytes(0, 8192, 28672, 14) == 0
    assert lib.bd_linear_grouped_workspace_bytes(16, 8192, 0, 14) == 0
    # K ranges: the partial buffer holds as many outputs as the larger of the
    # staged kernel's split (8 on k/v's 32 blocks of 32 rows, 2 on gate/up's
    # 896, none on q/o's 256) and the fallback's (128-row blocks up to 256
    # workgroups: 8, 2 and 4)
    kv = lib.bd_linear_grouped_workspace_bytes(16, 1024, 8192, 14)
    gu = lib.bd_linear_grouped_workspace_bytes(16, 28672, 8192, 14)
    qo = lib.bd_linear_grouped_workspace_bytes(16, 8192, 8192, 14)
    assert 8 * 16 * 1024 * 4 <= kv < 8 * 16 * 1024 * 4 + 65536
    assert 2 * 16 * 28672 * 4 <= gu < 2 * 16 * 28672 * 4 + 65536
    assert 4 * 16 * 8192 * 4 <= qo < 4 * 16 * 8192 * 4 + 65536


FAKE = ctypes.c_void_p(1 << 20)      # 16-byte aligned, never dereferenced
MISALIGNED = ctypes.c_void_p((1 << 20) + 2)
NULL = ctypes.c_void_p(0)


def test_compress_validation(lib):
    c = lib.bd_compress
    assert c(NULL, 4, 16, 0, FAKE, FAKE, FAKE, 64, NULL) == 1          # NULL delta
    assert c(FAKE, 4, 16, 7, FAKE, FAKE, FAKE, 64, NULL) == 5          # bad mode
    assert c(FAKE, 4, 12, 0, FAKE, FAKE, FAKE, 64, NULL) == 2          # d_in % 8
    assert c(FAKE, 0, 16, 0, FAKE, FAKE, FAKE, 64, NULL) == 2          # d_out < 1
    assert c(FAKE, 4, 0, 0, FAKE, FAKE, FAKE, 64, NULL) == 2           # d_in < 8
    assert c(MISALIGNED, 4, 16, 0, FAKE, FAKE, FAKE, 64, NULL) == 3    # delta alignment
    assert c(FAKE, 4, 16, 0, FAKE, FAKE, FAKE, 16, NULL) == 4          # workspace too small
    assert c(FAKE, 4, 16, 0, FAKE, FAKE, NULL, 0, NULL) == 4           # missing workspace


def test_compress_pair_validation(lib):
    c = lib.bd_compress_pair
    assert c(NULL, FAKE, 4, 16, 0, FAKE, FAKE, FAKE, 64, NULL) == 1          # NULL w_ft
    assert c(FAKE, NULL, 4, 16, 0, FAKE, FAKE, FAKE, 64, NULL) == 1          # NULL w_base
    assert c(FAKE, FAKE, 4, 16, 0, NULL, FAKE, FAKE, 64, NULL) == 1          # NULL signs
    assert c(FAKE, FAKE, 4, 16, 3, FAKE, FAKE, FAKE, 64, NULL) == 5          # bad mode
    assert c(FAKE, FAKE, 4, 12, 0, FAKE, FAKE, FAKE, 64, NULL) == 2          # d_in % 8
    assert c(FAKE, FAKE, 0, 16, 0, FAKE, FAKE, FAKE, 64, NULL) == 2          # d_out < 1
    assert c(MISALIGNED, FAKE, 4, 16, 0, FAKE, FAKE, FAKE, 64, NULL) == 3    # w_ft alignment
    assert c(FAKE, MISALIGNED, 4, 16, 0, FAKE, FAKE, FAKE, 64, NULL) == 3    # w_base alignment
    assert c(FAKE, FAKE, 4, 16, 0, FAKE, FAKE, FAKE, 16, NULL) == 4          # workspace too small
    assert c(FAKE, FAKE, 4, 16, 0, FAKE, FAKE, NULL, 0, NULL) == 4           # missing workspace


def test_linear_validation(lib):
    f = lib.bd_linear
    assert f(FAKE, NULL, FAKE, FAKE, 0, FAKE, 1, 4, 16, NULL, 0, NULL) == 1
    assert f(NULL, FAKE, FAKE, FAKE, 0, FAKE, 1, 4, 16, NULL, 0, NULL) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, 2, FAKE, 1, 4, 16, NULL, 0, NULL) == 5
    assert f(FAKE, FAKE, FAKE, FAKE, 0, FAKE, 1, 4, 20, NULL, 0, NULL) == 2
    assert f(FAKE, FAKE, FAKE, FAKE, 0, FAKE, -1, 4, 16, NULL, 0, NULL) == 2
    assert f(MISALIGNED, FAKE, FAKE, FAKE, 0, FAKE, 1, 4, 16, NULL, 0, NULL) == 3
    assert f(FAKE, FAKE, FAKE, FAKE, 0, MISALIGNED, 1, 4, 16, NULL, 0, NULL) == 3
    # M == 0 is a no-op that never touches the device, x and y may be NULL
    assert f(NULL, FAKE, FAKE, FAKE, 1, NULL, 0, 4, 16, NULL, 0, NULL) == 0
    # a tiled shape that splits its tiles needs the workspace
    need = lib.bd_linear_workspace_bytes(300, 300, 520)
    assert f(FAKE, FAKE, FAKE, FAKE, 0, FAKE, 300, 300, 520, NULL, 0, NULL) == 4
    assert f(FAKE, FAKE, FAKE, FAKE, 0, FAKE, 300, 300, 520, FAKE, need - 16, NULL) == 4
    assert f(FAKE, FAKE, FAKE, FAKE, 0, FAKE, 300, 300, 520, MISALIGNED, need, NULL) == 4
    # and so does a decode shape on the slice path (K split over workgroups)
    need = lib.bd_linear_workspace_bytes(16, 1024, 8192)
    assert need > 0
    assert f(FAKE, FAKE, FAKE, FAKE, 0, FAKE, 16, 1024, 8192, NULL, 0, NULL) == 4
    assert f(FAKE, FAKE, FAKE, FAKE, 0, FAKE, 16, 1024, 8192, FAKE, need - 16, NULL) == 4



def test_grouped_validation(lib):
    f = lib.bd_linear_grouped
    two = (ctypes.c_void_p * 2)(FAKE.value, FAKE.value)
    one_null = (ctypes.c_void_p * 2)(FAKE.value, 0)
    ws = lib.bd_linear_grouped_workspace_bytes(8, 4, 16, 2)
    args = lambda s, a, G, ws_ptr, ws_n, M=8: (FAKE, FAKE, FAKE, s, a, 1, G, FAKE, M, 4, 16,
                                               ws_ptr, ws_n, NULL)
    assert f(*args(two, two, 0, FAKE, ws)) == 2                  # G < 1
    assert f(*args(two, two, 65, FAKE, ws)) == 2                 # G > 64
    assert f(*args(one_null, two, 2, FAKE, ws)) == 1             # a NULL signs entry
    assert f(*args(two, one_null, 2, FAKE, ws)) == 1             # a NULL alpha entry
    assert f(*args(two, two, 2, FAKE, ws - 8)) == 4              # workspace too small
    assert f(*args(two, two, 2, NULL, 0)) == 4
    assert f(*args(two, two, 2, NULL, 0, M=0)) == 0              # M == 0 no-op
    # the planned form checks the same way
    fp = lib.bd_linear_grouped_planned
    assert fp(*args(two, two, 0, FAKE, ws)) == 2
    assert fp(*args(one_null, two, 2, FAKE, ws)) == 1
    assert fp(*args(two, two, 2, FAKE, ws - 8)) == 4
    assert fp(*args(two, two, 2, NULL, 0, M=0)) == 0


def test_grouped_plan_validation(lib):
    pb = lib.bd_linear_grouped_plan_bytes(16, 10)
    # the plan is the workspace's prefix: no larger than any grouped workspace
    # of the same batch, and independent of the projection's shape
    assert 0 < pb <= lib.bd_linear_grouped_workspace_bytes(16, 1024, 8192, 10)
    assert pb <= lib.bd_linear_grouped_workspace_bytes(16, 28672, 8192, 10)
    assert lib.bd_linear_grouped_plan_bytes(0, 10) == 0
    assert lib.bd_linear_grouped_plan_bytes(16, 65) == 0
    p = lib.bd_linear_grouped_plan
    assert p(FAKE, 16, 0, FAKE, pb, NULL) == 2                     # G < 1
    assert p(FAKE, -1, 10, FAKE, pb, NULL) == 2                    # M < 0
    assert p(NULL, 16, 10, FAKE, pb, NULL) == 1                    # no ids
    assert p(ctypes.c_void_p((1 << 20) + 2), 16, 10, FAKE, pb, NULL) == 3
    assert p(FAKE, 16, 10, FAKE, pb - 8, NULL) == 4                # too small
    assert p(FAKE, 16, 10, NULL, pb, NULL) == 4
    assert p(NULL, 0, 10, NULL, 0, NULL) == 0                      # M == 0 no-op


def test_binding_refuses_cpu_tensors():
    import torch
    import tenant_serving_amd as bd
    with pytest.raises(ValueError, match="GPU"):
        bd.bd_compress(torch.zeros(4, 16))
    with pytest.raises(ValueError, match="GPU"):
        bd.bd_compress_pair(torch.zeros(4, 16, dtype=torch.bfloat16), torch.zeros(4, 16, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="GPU"):
        bd.bd_linear(torch.zeros(1, 16, dtype=torch.bfloat16), torch.zeros(4, 16, dtype=torch.bfloat16),
                     torch.zeros(4, 2, dtype=torch.uint8), torch.zeros(4))


def test_linear_path_names_a_kernel(lib):
    # pure host query: which kernel instance bd_linear picks for a shape
    names = {lib.bd_linear_path(M, N, K).decode() for M, N, K in
             [(1, 28672, 8192), (4, 1024, 8192), (16, 8192, 8192), (16, 28672, 8192),
              (48, 8192, 8192), (2048, 8192, 8192)]}
    assert all(names) and len(names) >= 4
    assert lib.bd_linear_path(0, 16, 16).decode() == ""
    # two to four tokens: x resident in LDS while it fits 128 KiB (four only
    # below 8192 rows), the one-shot kernel on few rows, the GEMV otherwise
    path = lambda M, N, K: lib.bd_linear_path(M, N, K).decode()
    assert path(2, 8192, 16384) == "xres_kernel<2,4,8,65536>"
    assert path(2, 8192, 16392) == "xres_kernel<2,4,16,131072>"
    assert path(2, 8192, 32768) == "xres_kernel<2,4,16,131072>"
    assert path(2, 8192, 32776).startswith("xstat_kernel")
    assert path(3, 28672, 8192) == "xres_kernel<3,4,8,65536>"
    # 4..16 tokens on 8192+ rows of 4097..8192 weights: the band kernel where
    # its partial-sum slots hold a workgroup's bands in one round (64 / 32 /
    # 21 / 16 bands of 4 rows at 4 / 8 / 12 / 16 tokens, 256 compute units
    # when no GPU is present), at four tokens only up to 16 bands
    assert path(4, 8192, 8192) == "band_kernel"
    assert path(16, 8192, 8192) == "band_kernel"
    assert path(4, 16384, 8192) == "band_kernel"
    assert path(4, 16388, 8192) == "quad_kernel<2>"
    assert path(8, 28672, 8192) == "band_kernel"
    assert path(8, 32768, 8192) == "band_kernel"
    assert not path(8, 32772, 8192).startswith("band_kernel")
    assert path(12, 28672, 8192).startswith("xstat_kernel")
    assert path(16, 16384, 8192) == "band_kernel"
    assert path(16, 28672, 8192).startswith("xstat_kernel")
    assert path(13, 12296, 5000) == "band_kernel"
    assert path(8, 8192, 4104) == "band_kernel"
    assert path(8, 8192, 4096) == "rowstream_kernel<1,16,1>"
    assert path(8, 8192, 8200) == "rowstream_kernel<1,16,1>"
    assert path(16, 8188, 8192) == "rowstream_kernel<1,16,1>"
    assert path(3, 8192, 8192) == "xres_kernel<3,4,8,65536>"
    # and on fewer rows: 2048..4095 rows at 4..16 tokens, 4096..8191 rows at
    # 4..8 tokens with at least 15 chunks per row
    assert path(16, 2048, 8192) == "band_kernel"
    assert path(4, 3072, 4104) == "band_kernel"
    # 3..16 tokens on fewer rows: K slices where a one-shot workgroup would
    # pull 256 KiB of x or more (M * d_in >= 131072), or on 2048..4095 rows
    # that the band kernel does not take; else the one-shot kernel
    assert path(16, 2044, 8192) == "slice_kernel"
    assert path(16, 1024, 8192) == "slice_kernel"
    assert path(12, 1024, 8192) == "shot_kernel"
    assert path(8, 1024, 16384) == "slice_kernel"
    assert path(16, 1024, 4096) == "shot_kernel"
    assert path(16, 1000, 5000) == "shot_kernel"
    assert path(3, 2048, 8192) == "slice_kernel"
    assert path(3, 3072, 4096) == "slice_kernel"
    assert path(16, 4095, 2048) == "slice_kernel"
    assert path(4, 2048, 2040) == "shot_kernel"
    assert path(2, 2048, 2048).startswith("xres_kernel")
    assert path(8, 6144, 8192) == "band_kernel"
    assert path(8, 6144, 7680) == "band_kernel"
    assert path(8, 6144, 7168).startswith("rowstream_kernel")
    assert path(16, 6144, 8192).startswith("rowstream_kernel")
    assert path(8, 6152, 5000).startswith("rowstream_kernel")
    # four tokens on more rows of up to 16K weights: the row-quad kernel;
    # longer rows keep the x-stationary kernel
    assert path(4, 28672, 8192) == "quad_kernel<2>"
    assert path(4, 8192, 16384) == "quad_kernel<2>"
    # the row-quad plan holds at most 128 units per workgroup: up to 4 x 128
    # rows per compute unit (256 of them when no GPU is present); more rows go
    # to the row-streaming path instead of failing at launch
    assert path(4, 4 * 128 * 256, 8192) == "quad_kernel<2>"
    assert path(4, 4 * 128 * 256 + 4, 8192) == "rowstream_kernel<1,16,1>"
    # up to 32 tokens on more than 16384 rows: row streaming; beyond, skinny
    assert path(17, 28672, 8192) == "rowstream_kernel<2,16,1>"
    assert path(32, 28672, 8192) == "rowstream_kernel<2,16,1>"
    assert path(16, 40000, 4096) == "rowstream_kernel<1,16,1>"
    assert path(33, 28672, 8192).startswith("skinny_kernel")
    # longer rows at four tokens, and 4..32 tokens: row streaming where its
    # 32-row workgroups number at most 1.5 per compute unit, else the
    # x-stationary kernel; three tokens with x beyond 128 KiB stay x-stationary
    assert path(4, 8192, 16392) == "rowstream_kernel<1,16,1>"
    assert path(4, 8192, 28672) == "rowstream_kernel<1,16,1>"
    assert path(8, 12288, 8200) == "rowstream_kernel<1,16,1>"
    assert path(8, 12296, 8200).startswith("xstat_kernel")
    assert path(4, 16400, 28672).startswith("xstat_kernel")
    assert path(3, 8192, 28672).startswith("xstat_kernel")
    assert path(16, 4096, 14336) == "rowstream_kernel<1,8,2>"
    assert path(32, 4096, 14336) == "rowstream_kernel<2,8,2>"
    assert path(17, 4104, 14336) == "rowstream_kernel<2,16,1>"
    assert path(4, 8191, 8192) == "band_kernel"
    assert path(4, 8191, 7168) == "xres_kernel<4,4,8,65536>"
    assert path(4, 4096, 4096) == "xres_kernel<4,4,8,65536>"
    assert path(4, 4104, 16904) == "gemv_kernel<4,2,2>"
    assert path(2, 2040, 8192) == "gemv_kernel<2,2,4>"
    # one token: one row per workgroup below 2048 rows (d_in <= 16384), 8-wave
    # workgroups on 4096..8191 rows of 8192..16384 weights
    assert path(1, 1024, 8192) == "gemv_kernel<1,1,4>"
    assert path(1, 1024, 16392) == "gemv_kernel<1,2,4>"
    assert path(1, 2048, 8192) == "gemv_kernel<1,2,4>"
    assert path(1, 4096, 8192) == "gemv8_kernel<1,2,2>"
    assert path(1, 8191, 16384) == "gemv8_kernel<1,2,2>"
    assert path(1, 4096, 8184) == "gemv_kernel<1,2,4>"
    assert path(1, 8192, 8192) == "gemv_kernel<1,2,4>"
    assert path(3, 1024, 8192) == "shot_kernel"
    kmax = (1 << 23) - 8
    assert lib.bd_linear_path(65, 8, kmax).decode() == "prefill_kernel"
    assert lib.bd_linear_path(65, 8, kmax + 8).decode().startswith("skinny_kernel<4,")


# ----------------------------------------------------------------------------
# the Python binding rejects malformed arguments before any library call; the
# checks run on host tensors (shapes, dtypes, the α size a mode reads), and
# tensors that pass them but are not on a GPU are refused too

def _grouped_args(N=64, K=128, M=5, G=3, per_row=True):
    import torch
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    ids = torch.zeros((M,), dtype=torch.int32)
    w = torch.zeros((N, K), dtype=torch.bfloat16)
    sl = [torch.zeros((N, K // 8), dtype=torch.uint8) for _ in range(G)]
    al = [torch.zeros((N if per_row else 1,), dtype=torch.float32) for _ in range(G)]
    return x, ids, w, sl, al


def test_binding_grouped_rejects_a_wrong_out(lib):
    import torch
    import tenant_serving_amd as bd
    x, ids, w, sl, al = _grouped_args()
    for bad in (torch.zeros((4, 64)), torch.zeros((5, 63)), torch.zeros(320),
                torch.zeros((5, 64), dtype=torch.float64), torch.zeros((64, 5)).t()):
        with pytest.raises((ValueError, TypeError), match="out"):
            bd.bd_linear_grouped(x, ids, w, sl, al, out=bad)
    # a well-formed call on host tensors: refused for the device, not run
    with pytest.raises(ValueError, match="GPU"):
        bd.bd_linear_grouped(x, ids, w, sl, al, out=torch.zeros((5, 64)))


def test_binding_grouped_checks_every_alpha(lib):
    import torch
    import tenant_serving_amd as bd
    x, ids, w, sl, al = _grouped_args()
    short = list(al)
    short[2] = torch.zeros((63,), dtype=torch.float32)      # per-row set, variant 2 one short
    with pytest.raises(ValueError, match="alpha"):
        bd.bd_linear_grouped(x, ids, w, sl, short)
    with pytest.raises(ValueError, match="alpha"):
        bd.bd_linear_grouped(x, ids, w, sl, short, mode=bd.BD_ALPHA_PER_ROW)
    mixed = list(al)
    mixed[1] = torch.zeros((1,), dtype=torch.float32)       # a per-matrix α among per-row ones
    with pytest.raises(ValueError, match="alpha"):
        bd.bd_linear_grouped(x, ids, w, sl, mixed)
    with pytest.raises(TypeError, match="alpha"):
        bd.bd_linear_grouped(x, ids, w, sl, al[:2] + [al[2].double()])
    bad_signs = list(sl)
    bad_signs[1] = torch.zeros((64, 15), dtype=torch.uint8)
    with pytest.raises(ValueError, match="signs"):
        bd.bd_linear_grouped(x, ids, w, bad_signs, al)


def test_binding_explicit_mode_checks_alpha_size(lib):
    import torch
    import tenant_serving_amd as bd
    x, _, w, sl, al = _grouped_args(M=2)
    one = torch.zeros((1,), dtype=torch.float32)
    with pytest.raises(ValueError, match="per-row alpha"):
        bd.bd_linear(x, w, sl[0], one, mode=bd.BD_ALPHA_PER_ROW)
    with pytest.raises(ValueError, match="per-matrix alpha"):
        bd.bd_linear(x, w, sl[0], al[0], mode=bd.BD_ALPHA_PER_MATRIX)
    with pytest.raises(ValueError, match="1 or d_out"):
        bd.bd_linear(x, w, sl[0], torch.zeros((7,), dtype=torch.float32))
    with pytest.raises(ValueError, match="out"):
        bd.bd_linear(x, w, sl[0], al[0], out=torch.zeros((2, 63)))
    with pytest.raises(ValueError, match="GPU"):
        bd.bd_linear(x, w, sl[0], al[0], mode=bd.BD_ALPHA_PER_ROW)
    x1, _, w1, sl1, al1 = _grouped_args(M=2, G=1, per_row=False)
    with pytest.raises(ValueError, match="GPU"):
        bd.bd_linear(x1, w1, sl1[0], al1[0], mode=bd.BD_ALPHA_PER_MATRIX)


def test_noalloc_refuses_shapes_beyond_its_scratch(lib):
    # the size check runs on the host before any device call, so it answers
    # without a GPU: 293 tokens on 28672x8192 need more than the 64 MiB array
    from tenant_serving_amd import bitdelta
    assert bitdelta.BD_NOALLOC_SCRATCH_BYTES == 64 << 20
    fake = ctypes.c_void_p(1 << 20)                   # aligned, never dereferenced
    sp = (ctypes.c_void_p * 2)(fake, fake)
    for M, N, K in ((293, 28672, 8192), (512, 8192, 8192)):
        assert lib.bd_linear_grouped_workspace_bytes(M, N, K, 2) > bitdelta.BD_NOALLOC_SCRATCH_BYTES
        st = lib.bd_linear_grouped_noalloc(fake, fake, fake, sp, sp, 1, 2, fake, M, N, K, None)
        assert st == 4, st
    assert lib.bd_linear_grouped_workspace_bytes(292, 28672, 8192, 14) <= bitdelta.BD_NOALLOC_SCRATCH_BYTES
    # argument errors come before the size check and the device
    assert lib.bd_linear_grouped_noalloc(None, fake, fake, sp, sp, 1, 2, fake, 4, 64, 64, None) == 1
    assert lib.bd_linear_grouped_noalloc(fake, fake, fake, sp, sp, 1, 2, fake, 4, 64, 60, None) == 2
    assert lib.bd_linear_grouped_noalloc(fake, fake, fake, sp, sp, 1, 0, fake, 4, 64, 64, None) == 2
    assert lib.bd_linear_grouped_noalloc(fake, fake, fake, sp, sp, 1, 2, fake, 0, 64, 64, None) == 0
