"""Tensor-level helpers over the C ABI: allocate outputs with torch on the
inputs' device and call the binding.  No arithmetic happens here.

Layouts (row-major, last index contiguous):
  quantize_1x128(x [M][K])            -> q u8 [M][K],  s f32 [M][K/128]
  quantize_128x1(x [T][F])            -> qT u8 [F][T], sT f32 [F][T/128]
  requantize_128x1(q [T][F], s [T][F/128]) -> same as quantize_128x1
  Per-row tile scales are indexed s[row][group] in every case; by default
  they are stored group-major (the returned tensor is a transposed view of
  a [groups][rows] buffer, strides (1, rows)), so that the GEMM's per-group
  load of consecutive rows' scales is one contiguous read.
  scale_layout="row_major" stores them [rows][groups] instead.
  quantize_block(w [K][N], transpose) -> q u8 [N][K] (transpose) or [K][N],
                                         s f32 [K/128][N/128]
  gemm(qa [M][K], sa [M][K/128], qb [N][K], sb)  -> c [M][N]
       sb [K/128][N/128] (block scales) or [N][K/128] (per-column scales)
  grouped_gemm(qa, sa, offsets i32 [G+1], qb [G][N][K], sb [G][K/128][N/128])
"""

import torch

from . import binding as B

_XTYPE = {torch.bfloat16: B.FP8FG_BF16, torch.float32: B.FP8FG_F32}
_CTYPE = {torch.bfloat16: B.FP8FG_BF16, torch.float32: B.FP8FG_F32}


def _rule(pow2):
    return B.FP8FG_SCALE_POW2 if pow2 else B.FP8FG_SCALE_AMAX


def _scales(rows, groups, layout, device):
    """Scale tensor indexed [row][group]."""
    if layout == "group_major":
        return torch.empty((groups, rows), dtype=torch.float32, device=device).t()
    if layout == "row_major":
        return torch.empty((rows, groups), dtype=torch.float32, device=device)
    raise ValueError("scale_layout must be 'group_major' or 'row_major'")


def quantize_1x128(x, pow2=False, scale_layout="group_major", stream=None):
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    s = _scales(M, K // 128, scale_layout, x.device)
    B.fp8_quantize_rowtile(x, _XTYPE[x.dtype], M, K, x.stride(0), None, 0, 0,
                           B.FP8FG_TILE_1x128, _rule(pow2), q, q.stride(0), s, s.stride(0),
                           s.stride(1), stream)
    return q, s


def quantize_128x1(x, pow2=False, scale_layout="group_major", stream=None):
    T, F = x.shape
    qt = torch.empty((F, T), dtype=torch.uint8, device=x.device)
    st = _scales(F, T // 128, scale_layout, x.device)
    B.fp8_quantize_rowtile(x, _XTYPE[x.dtype], T, F, x.stride(0), None, 0, 0,
                           B.FP8FG_TILE_128x1, _rule(pow2), qt, qt.stride(0), st, st.stride(0),
                           st.stride(1), stream)
    return qt, st


def requantize_128x1(q, s, pow2=False, scale_layout="group_major", stream=None):
    T, F = q.shape
    qt = torch.empty((F, T), dtype=torch.uint8, device=q.device)
    st = _scales(F, T // 128, scale_layout, q.device)
    B.fp8_quantize_rowtile(q, B.FP8FG_E4M3, T, F, q.stride(0), s, s.stride(0), s.stride(1),
                           B.FP8FG_TILE_128x1, _rule(pow2), qt, qt.stride(0), st, st.stride(0),
                           st.stride(1), stream)
    return qt, st


def quantize_block(w, pow2=False, transpose=True, stream=None):
    K, N = w.shape
    shape = (N, K) if transpose else (K, N)
    q = torch.empty(shape, dtype=torch.uint8, device=w.device)
    s = torch.empty((K // 128, N // 128), dtype=torch.float32, device=w.device)
    B.fp8_quantize_block(w, _XTYPE[w.dtype], K, N, w.stride(0), _rule(pow2), int(transpose), q,
                         q.stride(0), s, s.stride(0), s.stride(1), stream)
    return q, s


def tile_flags(tiles):
    """None (chosen from the shape), 'wide' (256-row tiles) or 'narrow'
    (64x128 tiles) -> the GEMM flag bits that fix the default path's tiles."""
    return {None: 0, "wide": B.FP8FG_GEMM_TILES_WIDE, "narrow": B.FP8FG_GEMM_TILES_NARROW}[tiles]


def gemm(qa, sa, qb, sb, out_dtype=torch.bfloat16, col_scales=False, no_promotion=False,
         fp8_mfma=False, e8m0_scales=False, out=None, stream=None, tiles=None):
    """col_scales=False: sb [K/128][N/128] block scales; True: sb [N][K/128].
    no_promotion: per-tensor scales (sa, sb hold one value each), whole-K
    FP8 matrix-core accumulation.  fp8_mfma: K-group partial sums from the
    FP8 MFMA instead of the exact default path.  e8m0_scales: the FP8 MFMA
    applies the scales' powers of two as its E8M0 operand scales.  tiles:
    see tile_flags (default path only)."""
    M, K = qa.shape
    N = qb.shape[0]
    c = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=qa.device)
    mode = B.FP8FG_BSCALE_COL if col_scales else B.FP8FG_BSCALE_BLOCK128
    if no_promotion:
        # per-tensor scales broadcast with zero strides
        sa_ms, sa_ks, sb_ns, sb_ks = 0, 0, 0, 0
    else:
        sa_ms, sa_ks = sa.stride(0), sa.stride(1)
        if col_scales:
            sb_ns, sb_ks = sb.stride(0), sb.stride(1)
        else:
            sb_ns, sb_ks = sb.stride(1), sb.stride(0)
    flags = ((B.FP8FG_GEMM_NO_PROMOTION if no_promotion else 0) | (B.FP8FG_GEMM_FP8_MFMA if fp8_mfma else 0) |
             (B.FP8FG_GEMM_E8M0_SCALES if e8m0_scales else 0) | tile_flags(tiles))
    B.fp8_gemm_blockscaled(M, N, K, qa, qa.stride(0), sa, sa_ms, sa_ks, qb, qb.stride(0), sb,
                           sb_ns, sb_ks, mode, c, _CTYPE[c.dtype], c.stride(0), flags, stream)
    return c


def grouped_gemm(qa, sa, offsets, qb, sb, out_dtype=torch.bfloat16, out=None, stream=None,
                 flags=B.FP8FG_GEMM_DEFAULT, tiles=None):
    M, K = qa.shape
    G, N, _ = qb.shape
    c = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=qa.device)
    B.fp8_grouped_gemm_blockscaled(G, offsets, M, N, K, qa, qa.stride(0), sa, sa.stride(0),
                                   sa.stride(1), qb, qb.stride(1), qb.stride(0), sb, sb.stride(2),
                                   sb.stride(1), sb.stride(0), c, _CTYPE[c.dtype], c.stride(0),
                                   flags | tile_flags(tiles), stream)
    return c
