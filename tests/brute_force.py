"""Dense per-pixel formulation of the MSDA core, used as an independent pin.

Bilinear (trilinear) interpolation with zero padding equals a sum over EVERY
pixel of the level weighted by the separable tent kernel
max(0, 1 - |x_hat - j|) * max(0, 1 - |y_hat - i|) [* max(0, 1 - |z_hat - k|)].
This form has no floor, no corner enumeration and no border test, so it
shares none of the oracle's steps.  The pixel-space coordinate is the same
reading as everywhere else (pixel centre of pixel j at (j + 0.5) / W, rounded
once to float32): x*W - 0.5 is exact in float64 for a float32 x and an
integer W < 2^24, so casting it to float32 rounds once, exactly as fmaf does.

Runs in float64 with numpy; meant for small grids and small query subsets.
"""
import numpy as np


def _pixel(x, extent):
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        return (x * float(extent) - 0.5).astype(np.float32).astype(np.float64)


def _tent(coord, n):
    """[..., n] tent weights of every integer position 0..n-1 around coord."""
    idx = np.arange(n, dtype=np.float64)
    with np.errstate(invalid="ignore"):
        # fmax drops NaN (NaN or +-inf coordinates give weight 0 everywhere)
        return np.fmax(0.0, 1.0 - np.abs(coord[..., None] - idx))


def dense_forward(value, shapes, starts, loc, attw):
    """value [N,S,M,D], shapes [L,dims], starts [L], loc [N,Lq,M,L,P,dims],
    attw [N,Lq,M,L,P]; returns float64 [N, Lq, M*D]."""
    value = np.asarray(value, dtype=np.float64)
    shapes = np.asarray(shapes, dtype=np.int64)
    starts = np.asarray(starts, dtype=np.int64)
    loc = np.asarray(loc, dtype=np.float32)
    attw = np.asarray(attw, dtype=np.float64)
    N, S, M, D = value.shape
    _, Lq, _, L, P, dims = loc.shape
    out = np.zeros((N, Lq, M, D), dtype=np.float64)
    for l in range(L):
        shp = [int(e) for e in shapes[l]]
        size = int(np.prod(shp))
        lv = value[:, starts[l]:starts[l] + size]            # [N, size, M, D]
        if dims == 2:
            H, W = shp
            tx = _tent(_pixel(loc[:, :, :, l, :, 0], W), W)    # [N,Lq,M,P,W]
            ty = _tent(_pixel(loc[:, :, :, l, :, 1], H), H)    # [N,Lq,M,P,H]
            wgt = ty[..., :, None] * tx[..., None, :]          # [N,Lq,M,P,H,W]
        else:
            Z, H, W = shp
            tx = _tent(_pixel(loc[:, :, :, l, :, 0], W), W)
            ty = _tent(_pixel(loc[:, :, :, l, :, 1], H), H)
            tz = _tent(_pixel(loc[:, :, :, l, :, 2], Z), Z)
            wgt = (tz[..., :, None, None] * ty[..., None, :, None]
                   * tx[..., None, None, :])                   # [N,Lq,M,P,Z,H,W]
        wgt = wgt.reshape(N, Lq, M, P, size)
        wgt = (wgt * attw[:, :, :, l, :, None]).sum(axis=3)     # [N,Lq,M,size]
        out += np.einsum("nqms,nsmd->nqmd", wgt, lv)
    return out.reshape(N, Lq, M * D)
