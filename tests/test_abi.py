"""The C-ABI boundary on the CPU: the library loads, exports every entry
point the header declares, and rejects invalid arguments with the
documented status before touching a device (no GPU needed: every check
runs on the host before any HIP call)."""

import ctypes
import os
import re

import pytest

from fp8_fine_grained_x1_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8fg.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from fp8_fine_grained_x1_amd import build
        build.build(verbose=False)
    return B.lib()


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"FP8FG_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_header_declares_the_entry_points():
    assert sorted(declared_functions()) == sorted(B.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_only_declared_symbols_are_exported(lib):
    # the shared object exports exactly the C ABI (everything else is hidden)
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True).stdout
    text_syms = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert text_syms == set(declared_functions())


def test_status_strings(lib):
    for st in range(6):
        assert B.status_string(st)
    assert B.status_string(99) == "unknown status"


# Fake but well-aligned device addresses: validation must reject the calls
# below before any of these is dereferenced or any HIP call is made.
P16 = 1 << 20


def rowtile(**kw):
    args = dict(x=P16, x_type=B.FP8FG_BF16, rows=128, cols=256, ldx=256, x_scale=None, xs_rs=0,
                xs_ts=0, tile=B.FP8FG_TILE_1x128, scale_rule=B.FP8FG_SCALE_AMAX, q=P16, ldq=256,
                s=P16, s_rs=2, s_ts=1, stream=0, check=False)
    args.update(kw)
    return B.fp8_quantize_rowtile(**args)


def block(**kw):
    args = dict(w=P16, w_type=B.FP8FG_BF16, rows=256, cols=128, ldw=128,
                scale_rule=B.FP8FG_SCALE_AMAX, transpose_out=1, q=P16, ldq=256, s=P16, s_rs=1,
                s_cs=1, stream=0, check=False)
    args.update(kw)
    return B.fp8_quantize_block(**args)


def gemm(**kw):
    args = dict(M=64, N=128, K=256, a=P16, lda=256, sa=P16, sa_ms=2, sa_ks=1, b=P16, ldb=256,
                sb=P16, sb_ns=1, sb_ks=1, b_scale_mode=B.FP8FG_BSCALE_BLOCK128, c=P16,
                c_type=B.FP8FG_BF16, ldc=128, flags=0, stream=0, check=False)
    args.update(kw)
    return B.fp8_gemm_blockscaled(**args)


def grouped(**kw):
    args = dict(G=2, offsets=P16, M_total=64, N=128, K=256, a=P16, lda=256, sa=P16, sa_ms=2,
                sa_ks=1, b=P16, ldb=256, b_gs=128 * 256, sb=P16, sb_ns=1, sb_ks=1, sb_gs=2,
                c=P16, c_type=B.FP8FG_BF16, ldc=128, flags=0, stream=0, check=False)
    args.update(kw)
    return B.fp8_grouped_gemm_blockscaled(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(x_type=7), B.FP8FG_EINVAL),
    (dict(tile=5), B.FP8FG_EINVAL),
    (dict(scale_rule=2), B.FP8FG_EINVAL),
    (dict(rows=-1), B.FP8FG_EINVAL),
    (dict(s_rs=-1), B.FP8FG_EINVAL),
    (dict(cols=200, ldx=256), B.FP8FG_ESHAPE),
    (dict(tile=B.FP8FG_TILE_128x1, rows=100), B.FP8FG_ESHAPE),
    (dict(x=None), B.FP8FG_EINVAL),
    (dict(q=None), B.FP8FG_EINVAL),
    (dict(s=None), B.FP8FG_EINVAL),
    (dict(ldx=128), B.FP8FG_ESHAPE),
    (dict(ldq=128), B.FP8FG_ESHAPE),
    (dict(x=P16 + 8), B.FP8FG_EALIGN),
    (dict(q=P16 + 4), B.FP8FG_EALIGN),
    (dict(s=P16 + 2), B.FP8FG_EALIGN),
    (dict(ldx=260), B.FP8FG_EALIGN),
    (dict(ldq=264), B.FP8FG_EALIGN),
    (dict(x_type=B.FP8FG_E4M3, x_scale=P16), B.FP8FG_EUNSUPPORTED),     # requant is 128x1 only
    (dict(x_type=B.FP8FG_E4M3, tile=B.FP8FG_TILE_128x1, ldq=128), B.FP8FG_EINVAL),  # no scales
    (dict(tile=B.FP8FG_TILE_128x1, ldq=64), B.FP8FG_ESHAPE),          # ldq < rows (transposed)
    (dict(rows=0), B.FP8FG_OK),                                       # empty: no-op
    (dict(rows=0, x=None, q=None, s=None), B.FP8FG_OK),
])
def test_rowtile_validation(lib, kw, status):
    assert rowtile(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(w_type=B.FP8FG_E4M3), B.FP8FG_EINVAL),
    (dict(transpose_out=2), B.FP8FG_EINVAL),
    (dict(rows=200), B.FP8FG_ESHAPE),
    (dict(cols=100, ldw=128), B.FP8FG_ESHAPE),
    (dict(ldq=128), B.FP8FG_ESHAPE),                   # transposed output needs ldq >= rows
    (dict(transpose_out=0, ldq=64), B.FP8FG_ESHAPE),
    (dict(w=P16 + 2), B.FP8FG_EALIGN),
    (dict(w_type=B.FP8FG_F32, ldw=130), B.FP8FG_EALIGN),
    (dict(s=None), B.FP8FG_EINVAL),
    (dict(cols=0), B.FP8FG_OK),
])
def test_block_validation(lib, kw, status):
    assert block(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(b_scale_mode=3), B.FP8FG_EINVAL),
    (dict(c_type=B.FP8FG_E4M3), B.FP8FG_EINVAL),
    (dict(flags=32), B.FP8FG_EINVAL),
    (dict(flags=B.FP8FG_GEMM_TILES_WIDE | B.FP8FG_GEMM_TILES_NARROW), B.FP8FG_EINVAL),
    (dict(flags=B.FP8FG_GEMM_TILES_WIDE | B.FP8FG_GEMM_FP8_MFMA), B.FP8FG_EINVAL),
    (dict(flags=B.FP8FG_GEMM_TILES_NARROW | B.FP8FG_GEMM_E8M0_SCALES), B.FP8FG_EINVAL),
    (dict(flags=B.FP8FG_GEMM_TILES_NARROW, b_scale_mode=B.FP8FG_BSCALE_COL), B.FP8FG_EINVAL),
    (dict(flags=B.FP8FG_GEMM_TILES_WIDE, c=None), B.FP8FG_EINVAL),   # flag accepted, then null c
    (dict(flags=B.FP8FG_GEMM_TILES_NARROW, c=None), B.FP8FG_EINVAL),
    (dict(flags=B.FP8FG_GEMM_FP8_MFMA, c=None), B.FP8FG_EINVAL),   # flag accepted, then null c
    (dict(flags=B.FP8FG_GEMM_E8M0_SCALES, c=None), B.FP8FG_EINVAL),
    (dict(flags=B.FP8FG_GEMM_E8M0_SCALES | B.FP8FG_GEMM_FP8_MFMA, c=None), B.FP8FG_EINVAL),
    (dict(flags=B.FP8FG_GEMM_E8M0_SCALES | B.FP8FG_GEMM_NO_PROMOTION, sa_ks=0, sb_ks=0), B.FP8FG_EINVAL),
    (dict(M=-1), B.FP8FG_EINVAL),
    (dict(sa_ms=-2), B.FP8FG_EINVAL),
    (dict(flags=B.FP8FG_GEMM_NO_PROMOTION), B.FP8FG_EINVAL),   # per-K scales with no promotion
    (dict(K=200, lda=256, ldb=256), B.FP8FG_ESHAPE),
    (dict(N=100, ldc=128), B.FP8FG_ESHAPE),
    (dict(lda=128), B.FP8FG_ESHAPE),
    (dict(ldc=64), B.FP8FG_ESHAPE),
    (dict(a=None), B.FP8FG_EINVAL),
    (dict(sb=None), B.FP8FG_EINVAL),
    (dict(c=None), B.FP8FG_EINVAL),
    (dict(a=P16 + 8), B.FP8FG_EALIGN),
    (dict(ldb=264), B.FP8FG_EALIGN),
    (dict(c=P16 + 1), B.FP8FG_EALIGN),
    (dict(c_type=B.FP8FG_F32, c=P16 + 2), B.FP8FG_EALIGN),
    (dict(M=0), B.FP8FG_OK),
])
def test_gemm_validation(lib, kw, status):
    assert gemm(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(G=-1), B.FP8FG_EINVAL),
    (dict(G=0), B.FP8FG_EINVAL),                         # rows but no experts
    (dict(G=0, M_total=0), B.FP8FG_OK),
    (dict(offsets=None), B.FP8FG_EINVAL),
    (dict(offsets=P16 + 2), B.FP8FG_EALIGN),
    (dict(b_gs=100), B.FP8FG_EALIGN),
    (dict(b_gs=-16), B.FP8FG_EINVAL),
    (dict(K=100), B.FP8FG_ESHAPE),
    (dict(M_total=0), B.FP8FG_OK),
])
def test_grouped_validation(lib, kw, status):
    assert grouped(**kw) == status


# Size limits: valid calls beyond what the kernels' 32-bit tile offsets,
# grids or int32 expert offsets can address are refused with EUNSUPPORTED
# (on the host, before any HIP call; every other argument is valid).
@pytest.mark.parametrize("kw,status", [
    (dict(rows=(1 << 30) + 1, cols=256, ldx=256, s_rs=2), B.FP8FG_EUNSUPPORTED),  # > 2^31 tiles
    (dict(rows=1 << 30, cols=256, ldx=256, s_rs=2, x=None), B.FP8FG_EINVAL),      # checked first
    (dict(tile=B.FP8FG_TILE_128x1, rows=128 * 65536, cols=128, ldx=128, ldq=128 * 65536),
     B.FP8FG_EUNSUPPORTED),                                               # grid rows > 65535
])
def test_rowtile_size_limits(lib, kw, status):
    assert rowtile(**kw) == status


def test_block_size_limit(lib):
    assert block(rows=128 * 65536, ldq=128 * 65536) == B.FP8FG_EUNSUPPORTED
    # grid columns: at most (2^32 - 1) / 256 workgroups of 256 threads
    assert block(rows=128, cols=1 << 31, ldw=1 << 31, ldq=128) == B.FP8FG_EUNSUPPORTED
    assert rowtile(tile=B.FP8FG_TILE_128x1, rows=128, cols=1 << 31, ldx=1 << 31, ldq=128,
                   s_rs=1) == B.FP8FG_EUNSUPPORTED


@pytest.mark.parametrize("kw", [
    dict(lda=1 << 23),                                   # A row pitch: 256 rows * lda >= 2^31
    dict(ldb=1 << 24),                                   # B row pitch: 256 rows * ldb >= 2^32
    dict(K=1 << 31, lda=1 << 31, ldb=1 << 31),           # lda >= K: the pitch limit holds K
    dict(sa_ms=1 << 21),                                 # A scale row stride
    dict(sa_ks=(1 << 29) // 2),                          # sa_ks * K/128 >= 2^29 (K = 256)
    dict(sb_ks=(1 << 29) // 2),
    dict(b_scale_mode=B.FP8FG_BSCALE_COL, sb_ns=1 << 21),
])
def test_gemm_size_limits(lib, kw):
    assert gemm(**kw) == B.FP8FG_EUNSUPPORTED


def test_gemm_size_limits_are_exclusive(lib):
    # one below each limit passes validation; with M = 0 nothing is launched
    for kw in (dict(lda=(1 << 23) - 16), dict(ldb=(1 << 24) - 16), dict(sa_ms=(1 << 21) - 1),
               dict(sa_ks=(1 << 29) // 2 - 1)):
        assert gemm(M=0, **kw) == B.FP8FG_OK, kw
        # and with rows, the limit check is not what rejects a bad pointer
        assert gemm(a=None, **kw) == B.FP8FG_EINVAL, kw


def test_gemm_grid_limit_counts_the_tiles_that_launch(lib):
    # 2^30 rows on the 64x128 tiles: 2^24 workgroups of 256 threads, one past
    # HIP's 2^32 - 1 work-items (on the 256-row tiles the same call needs a
    # quarter of that); 2^31 rows on the 256x256 tiles: 2^23 workgroups of 512
    big = dict(K=128, lda=128, ldb=128, sa_ms=1, sa_ks=1)
    assert gemm(M=1 << 30, flags=B.FP8FG_GEMM_TILES_NARROW, **big) == B.FP8FG_EUNSUPPORTED
    assert gemm(M=1 << 31, N=256, ldc=256, flags=B.FP8FG_GEMM_TILES_WIDE, **big) == B.FP8FG_EUNSUPPORTED
    assert grouped(G=1, M_total=(1 << 30), flags=B.FP8FG_GEMM_TILES_NARROW, **big) == B.FP8FG_EUNSUPPORTED


def test_grouped_size_limits(lib):
    # int32 expert offsets cannot address more than 2^31 - 1 rows
    assert grouped(M_total=1 << 31) == B.FP8FG_EUNSUPPORTED
    assert grouped(M_total=1 << 31, offsets=None) == B.FP8FG_EUNSUPPORTED
    assert grouped(G=1 << 31) == B.FP8FG_EUNSUPPORTED
    assert grouped(lda=1 << 23) == B.FP8FG_EUNSUPPORTED


def test_binding_raises_on_error(lib):
    with pytest.raises(B.Fp8fgError) as ei:
        B.fp8_quantize_rowtile(P16, 9, 1, 128, 128, None, 0, 0, 0, 0, P16, 128, P16, 1, 1, 0)
    assert ei.value.status == B.FP8FG_EINVAL
