"""Pins of the CPU oracle: checks that fix what the oracle computes without
comparing it with itself.

Each pin takes an oracle library handle (``None`` = the in-tree build) and
raises AssertionError when the oracle disagrees with what the pages and the
mathematics fix. The same functions run against deliberately broken builds of
the oracle in ``test_oracle_mutants.py``, which shows that a plausible mistake
(a dropped term, a wrong sign, a swapped axis, a wrong pixel convention) is
caught by at least one of them.

Conventions being pinned (pages on deformable attention):
  * the core sum over heads' levels and points, weighted by A
    (discosf.com tutorial, section 2.2; cf-1.com article, section 3.1);
  * cell-centre coordinates x = u*W - 0.5 (grid_sample, align_corners=False:
    cf-1.com 5.3, CSDN explainer section 3 note 2);
  * bilinear interpolation, zero outside the level, gradients through the
    weights (discosf.com 2.1, 2.2, 3.2; cf-1.com 5.3 zeros padding);
  * flattened levels with (H, W) rows and start indices (cf-1.com 3.3);
  * locations as (x, y) = (width, height) (offset normalizer stacked (W, H),
    cf-1.com 3.2).
"""
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- helpers
def level_tables(shapes):
    shapes = np.asarray(shapes, np.int64).reshape(-1, 2)
    lsi = np.concatenate([[0], np.cumsum(shapes[:, 0] * shapes[:, 1])[:-1]]).astype(np.int64)
    return shapes, lsi


def coord32(u, n):
    """The single-precision fused multiply-add u*n - 0.5, correctly rounded.
    u is float32 and n a small integer, so u*n - 0.5 is exact in double and one
    rounding to float32 gives the correctly rounded fma."""
    return (np.asarray(u, np.float32).astype(np.float64) * n - 0.5).astype(np.float32)


def random_case(rng, B=2, M=3, D=5, shapes=((5, 7), (3, 4), (2, 2)), Nq=6, K=3,
                lo=-0.15, hi=1.15):
    """Random inputs in a box around [0,1]^2 (so some corners fall outside)."""
    shapes, lsi = level_tables(shapes)
    L = shapes.shape[0]
    Nv = int((shapes[:, 0] * shapes[:, 1]).sum())
    value = rng.standard_normal((B, Nv, M, D))
    loc = rng.uniform(lo, hi, size=(B, Nq, M, L, K, 2)).astype(np.float32)
    attn = rng.standard_normal((B, Nq, M, L, K))
    g = rng.standard_normal((B, Nq, M, D))
    return value, shapes, lsi, loc, attn, g


def fwd(lib, value, shapes, lsi, loc, attn):
    return oracle.forward(value, shapes, lsi, loc, attn, lib=lib)


def bwd(lib, value, shapes, lsi, loc, attn, g):
    return oracle.backward(value, shapes, lsi, loc, attn, g, lib=lib)


def _close(a, b, tol, what):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    scale = max(1.0, np.max(np.abs(b)) if b.size else 0.0)
    assert err <= tol * scale, f"{what}: max |diff| {err:.3e} > {tol:.1e} * {scale:.3g}"


# ----------------------------------------------------------------------------- pins
def pin_golden_hand_worked(lib=None):
    """Hand-worked 2x2 samples (tests/golden/bilinear_2x2_hand.txt)."""
    rows = np.loadtxt(os.path.join(GOLDEN, "bilinear_2x2_hand.txt"), comments="#")
    shapes, lsi = level_tables([(2, 2)])
    value = np.array([1.0, 2.0, 3.0, 4.0]).reshape(1, 4, 1, 1)
    for u, v, a, g, out, gu, gv, ga in rows:
        loc = np.array([u, v], np.float32).reshape(1, 1, 1, 1, 1, 2)
        attn = np.array([a]).reshape(1, 1, 1, 1, 1)
        go = np.array([g]).reshape(1, 1, 1, 1)
        o = fwd(lib, value, shapes, lsi, loc, attn)
        _, gl, gat = bwd(lib, value, shapes, lsi, loc, attn, go)
        got = (o.item(), gl[..., 0].item(), gl[..., 1].item(), gat.item())
        np.testing.assert_allclose(got, (out, gu, gv, ga), rtol=0, atol=1e-12,
                                   err_msg=f"golden sample u={u} v={v}")


def pin_pixel_centres(lib=None):
    """Sampling exactly at a pixel centre with a one-hot weight returns that
    pixel's value: fixes the level offsets, the (x, y) order, the row/column
    strides and the half-pixel convention. Power-of-two levels make it exact;
    other widths leave the fp32 coordinate at most an ulp off an integer."""
    rng = np.random.default_rng(11)
    for shp, exact in ((((8, 8), (4, 4), (2, 16)), True), (((5, 7), (3, 11), (1, 1)), False)):
        shapes, lsi = level_tables(shp)
        L = len(shp)
        Nv = int((shapes[:, 0] * shapes[:, 1]).sum())
        B, M, D, K, Nq = 2, 3, 4, 2, 12
        value = rng.standard_normal((B, Nv, M, D))
        loc = np.zeros((B, Nq, M, L, K, 2), np.float32)
        attn = np.zeros((B, Nq, M, L, K))
        expect = np.zeros((B, Nq, M, D))
        for b in range(B):
            for q in range(Nq):
                for m in range(M):
                    l = rng.integers(L)
                    k = rng.integers(K)
                    H, W = shapes[l]
                    i, j = rng.integers(H), rng.integers(W)          # row i, column j
                    loc[b, q, m, l, k] = ((j + 0.5) / W, (i + 0.5) / H)
                    attn[b, q, m, l, k] = 1.0
                    expect[b, q, m] = value[b, lsi[l] + i * W + j, m]
        out = fwd(lib, value, shapes, lsi, loc, attn)
        if exact:
            assert np.array_equal(out, expect), "pixel-centre sample is not the pixel value"
        else:
            _close(out, expect, 1e-6, "pixel-centre sample (non power-of-two level)")


def pin_constant_field(lib=None):
    """A constant field is returned unchanged when every corner is inside and the
    weights sum to one; the location gradient vanishes; the weight gradient is
    g . c for every sample."""
    rng = np.random.default_rng(12)
    shapes, lsi = level_tables(((6, 9), (3, 5)))
    L = 2
    B, M, D, K, Nq = 2, 2, 3, 3, 7
    Nv = int((shapes[:, 0] * shapes[:, 1]).sum())
    c = rng.standard_normal((M, D))
    value = np.broadcast_to(c, (B, Nv, M, D)).copy()
    # in-bounds: x in [0, W-1), y in [0, H-1)
    loc = np.empty((B, Nq, M, L, K, 2), np.float32)
    for l in range(L):
        H, W = shapes[l]
        loc[:, :, :, l, :, 0] = (rng.uniform(0.0, W - 1 - 1e-3, (B, Nq, M, K)) + 0.5) / W
        loc[:, :, :, l, :, 1] = (rng.uniform(0.0, H - 1 - 1e-3, (B, Nq, M, K)) + 0.5) / H
    logits = rng.standard_normal((B, Nq, M, L * K))
    attn = (np.exp(logits) / np.exp(logits).sum(-1, keepdims=True)).reshape(B, Nq, M, L, K)
    g = rng.standard_normal((B, Nq, M, D))
    out = fwd(lib, value, shapes, lsi, loc, attn)
    _close(out, np.broadcast_to(c, out.shape), 1e-13, "constant field")
    _, gl, ga = bwd(lib, value, shapes, lsi, loc, attn, g)
    _close(gl, np.zeros_like(gl), 1e-12, "location gradient on a constant field")
    expect_ga = np.einsum("bqmd,md->bqm", g, c)[..., None, None] * np.ones((L, K))
    _close(ga, expect_ga, 1e-12, "weight gradient on a constant field")


def pin_bilinear_field(lib=None):
    """Bilinear interpolation reproduces any field alpha + beta x + gamma y +
    delta x y exactly (inside the level), and its location gradient is the
    field's own derivative times W (or H) and A."""
    rng = np.random.default_rng(13)
    shapes, lsi = level_tables(((6, 9), (4, 3), (7, 5)))
    L = shapes.shape[0]
    B, M, D, K, Nq = 2, 2, 3, 2, 9
    Nv = int((shapes[:, 0] * shapes[:, 1]).sum())
    coef = rng.standard_normal((B, L, M, D, 4))                 # alpha, beta, gamma, delta
    value = np.empty((B, Nv, M, D))
    for l in range(L):
        H, W = shapes[l]
        yy, xx = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
        xx, yy = xx.reshape(-1), yy.reshape(-1)
        for b in range(B):
            a0, bx, cy, dxy = np.moveaxis(coef[b, l], -1, 0)    # each [M, D]
            value[b, lsi[l]:lsi[l] + H * W] = (a0 + bx * xx[:, None, None] + cy * yy[:, None, None]
                                               + dxy * (xx * yy)[:, None, None])
    loc = np.empty((B, Nq, M, L, K, 2), np.float32)
    for l in range(L):
        H, W = shapes[l]
        loc[:, :, :, l, :, 0] = (rng.uniform(1e-3, W - 1 - 1e-3, (B, Nq, M, K)) + 0.5) / W
        loc[:, :, :, l, :, 1] = (rng.uniform(1e-3, H - 1 - 1e-3, (B, Nq, M, K)) + 0.5) / H
    attn = rng.standard_normal((B, Nq, M, L, K))
    g = rng.standard_normal((B, Nq, M, D))
    out = fwd(lib, value, shapes, lsi, loc, attn)
    _, gl, ga = bwd(lib, value, shapes, lsi, loc, attn, g)
    exp_out = np.zeros((B, Nq, M, D))
    exp_ga = np.zeros((B, Nq, M, L, K))
    exp_gl = np.zeros((B, Nq, M, L, K, 2))
    for l in range(L):
        H, W = shapes[l]
        x = coord32(loc[..., l, :, 0], W).astype(np.float64)    # [B,Nq,M,K]
        y = coord32(loc[..., l, :, 1], H).astype(np.float64)
        a0, bx, cy, dxy = [coef[:, l, :, :, i][:, None, :, None, :] for i in range(4)]
        s = a0 + bx * x[..., None] + cy * y[..., None] + dxy * (x * y)[..., None]   # [B,Nq,M,K,D]
        a = attn[..., l, :]
        exp_out += np.einsum("bqmk,bqmkd->bqmd", a, s)
        gq = g[:, :, :, None, :]
        exp_ga[..., l, :] = (gq * s).sum(-1)
        exp_gl[..., l, :, 0] = W * a * (gq * (bx + dxy * y[..., None])).sum(-1)
        exp_gl[..., l, :, 1] = H * a * (gq * (cy + dxy * x[..., None])).sum(-1)
    _close(out, exp_out, 1e-12, "bilinear field, forward")
    _close(ga, exp_ga, 1e-12, "bilinear field, weight gradient")
    _close(gl, exp_gl, 1e-11, "bilinear field, location gradient")


def pin_out_of_bounds(lib=None):
    """Zero padding per corner: a sample whose four corners are all outside the
    level contributes nothing and receives zero gradients; a sample straddling
    the left edge keeps only the inside column's weight (no renormalization);
    non-finite locations count as outside."""
    shapes, lsi = level_tables(((4, 6),))
    H, W = 4, 6
    B, M, D, K = 1, 1, 2, 1
    value = np.arange(1, 1 + 24 * D, dtype=np.float64).reshape(B, 24, M, D)
    # all-outside samples: x <= -1 - eps, x >= W, y <= -1 - eps, y >= H, NaN, Inf
    far = [(-1.02 / W, 0.5), ((W + 0.01 + 0.5) / W, 0.5), (0.5, -0.3),
           (0.5, (H + 0.2 + 0.5) / H), (np.nan, 0.5), (0.5, np.inf), (-np.inf, np.nan),
           (1e30, 0.5), (-1e30, -1e30)]
    for u, v in far:
        loc = np.array([u, v], np.float32).reshape(1, 1, 1, 1, 1, 2)
        attn = np.ones((1, 1, 1, 1, 1))
        g = np.ones((1, 1, 1, D))
        out = fwd(lib, value, shapes, lsi, loc, attn)
        gv, gl, ga = bwd(lib, value, shapes, lsi, loc, attn, g)
        assert np.all(out == 0.0), f"outside sample ({u},{v}) contributed {out}"
        assert np.all(gv == 0.0) and np.all(gl == 0.0) and np.all(ga == 0.0), \
            f"outside sample ({u},{v}) has a nonzero gradient"
    # straddling the left edge: x = -0.25 -> only column 0 with weight 0.75
    row = 2
    u, v = np.float32(0.25 / W), np.float32((row + 0.5) / H)   # x = -0.25, y = row
    loc = np.array([u, v], np.float32).reshape(1, 1, 1, 1, 1, 2)
    out = fwd(lib, value, shapes, lsi, loc, np.full((1, 1, 1, 1, 1), 2.0))
    expect = 2.0 * 0.75 * value[0, row * W + 0, 0]
    np.testing.assert_allclose(out.reshape(-1), expect, rtol=1e-15, atol=0,
                               err_msg="edge sample must keep the in-level weight only")


def pin_linearity(lib=None):
    """The output is linear in the value field and in the weights: scaling
    either by 2 scales it exactly; adding fields adds outputs."""
    rng = np.random.default_rng(14)
    value, shapes, lsi, loc, attn, _ = random_case(rng)
    o = fwd(lib, value, shapes, lsi, loc, attn)
    assert np.array_equal(fwd(lib, 2 * value, shapes, lsi, loc, attn), 2 * o)
    assert np.array_equal(fwd(lib, value, shapes, lsi, loc, 2 * attn), 2 * o)
    v2 = rng.standard_normal(value.shape)
    _close(fwd(lib, value + v2, shapes, lsi, loc, attn), o + fwd(lib, v2, shapes, lsi, loc, attn),
           1e-13, "additivity in the value field")


def _grid_sample_reference(value, shapes, lsi, loc, attn, g):
    """Per-level torch grid_sample (bilinear, zeros padding, align_corners
    False), weighted by A and summed, in float64 with autograd -- the library
    routine the cf-1.com fallback (section 5.3) names. The grid is rebuilt from
    the single-precision pixel coordinates so that both sides sample the same
    point."""
    import torch
    import torch.nn.functional as F
    B, Nv, M, D = value.shape
    _, Nq, _, L, K, _ = loc.shape
    V = torch.tensor(value, dtype=torch.float64, requires_grad=True)
    A = torch.tensor(attn, dtype=torch.float64, requires_grad=True)
    # normalized location reproducing the fp32 pixel coordinate: u' = (x32 + 0.5) / W
    u_in = np.empty(loc.shape, np.float64)
    for l in range(L):
        H, W = shapes[l]
        u_in[..., l, :, 0] = (coord32(loc[..., l, :, 0], W).astype(np.float64) + 0.5) / W
        u_in[..., l, :, 1] = (coord32(loc[..., l, :, 1], H).astype(np.float64) + 0.5) / H
    U = torch.tensor(u_in, requires_grad=True)
    out = torch.zeros(B, Nq, M, D, dtype=torch.float64)
    for l in range(L):
        H, W = int(shapes[l][0]), int(shapes[l][1])
        v_l = V[:, lsi[l]:lsi[l] + H * W]                               # [B, HW, M, D]
        v_l = v_l.permute(0, 2, 3, 1).reshape(B * M, D, H, W)
        grid = 2.0 * U[:, :, :, l] - 1.0                                # [B, Nq, M, K, 2]
        grid = grid.permute(0, 2, 1, 3, 4).reshape(B * M, Nq, K, 2)
        s = F.grid_sample(v_l, grid, mode="bilinear", padding_mode="zeros",
                          align_corners=False)                          # [B*M, D, Nq, K]
        s = s.reshape(B, M, D, Nq, K).permute(0, 3, 1, 4, 2)            # [B, Nq, M, K, D]
        out = out + (A[:, :, :, l, :, None] * s).sum(3)
    G = torch.tensor(g, dtype=torch.float64)
    (out * G).sum().backward()
    return (out.detach().numpy(), V.grad.numpy(), U.grad.numpy(), A.grad.numpy())


def pin_grid_sample(lib=None):
    """Forward and backward equal the per-level grid_sample formulation
    (library routine, independent code) on random inputs with out-of-level
    samples."""
    for seed in (15, 16):
        rng = np.random.default_rng(seed)
        value, shapes, lsi, loc, attn, g = random_case(rng)
        ro, rgv, rgl, rga = _grid_sample_reference(value, shapes, lsi, loc, attn, g)
        o = fwd(lib, value, shapes, lsi, loc, attn)
        gv, gl, ga = bwd(lib, value, shapes, lsi, loc, attn, g)
        _close(o, ro, 1e-12, "forward vs grid_sample")
        _close(gv, rgv, 1e-12, "value gradient vs grid_sample")
        _close(ga, rga, 1e-12, "weight gradient vs grid_sample")
        _close(gl, rgl, 1e-10, "location gradient vs grid_sample")


def _tent_dense(value, shapes, lsi, loc, attn, g):
    """Brute force without floor(): every pixel n of level l is weighted by the
    tent kernel max(0, 1-|x-x_n|) * max(0, 1-|y-y_n|); the output is the
    dense weighted sum over all Nv pixels. Gradients by differentiating the
    tent kernel (valid away from kinks)."""
    B, Nv, M, D = value.shape
    _, Nq, _, L, K, _ = loc.shape
    out = np.zeros((B, Nq, M, D))
    gv = np.zeros_like(value)
    gl = np.zeros(loc.shape)
    ga = np.zeros(attn.shape)
    for l in range(L):
        H, W = shapes[l]
        yy, xx = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
        xn, yn = xx.reshape(-1).astype(np.float64), yy.reshape(-1).astype(np.float64)
        vl = value[:, lsi[l]:lsi[l] + H * W]                          # [B, HW, M, D]
        x = coord32(loc[..., l, :, 0], W).astype(np.float64)[..., None]   # [B,Nq,M,K,1]
        y = coord32(loc[..., l, :, 1], H).astype(np.float64)[..., None]
        tx = np.maximum(0.0, 1.0 - np.abs(x - xn))
        ty = np.maximum(0.0, 1.0 - np.abs(y - yn))
        dtx = np.where(np.abs(x - xn) < 1.0, -np.sign(x - xn), 0.0)
        dty = np.where(np.abs(y - yn) < 1.0, -np.sign(y - yn), 0.0)
        wt = tx * ty                                                  # [B,Nq,M,K,HW]
        a = attn[..., l, :]                                           # [B,Nq,M,K]
        s = np.einsum("bqmkn,bnmd->bqmkd", wt, vl)
        out += np.einsum("bqmk,bqmkd->bqmd", a, s)
        gs = np.einsum("bqmd,bqmkd->bqmk", g, s)
        ga[..., l, :] = gs
        gdot = np.einsum("bqmd,bnmd->bqmn", g, vl)[:, :, :, None, :]  # [B,Nq,M,1,HW]
        gl[..., l, :, 0] = W * a * (dtx * ty * gdot).sum(-1)
        gl[..., l, :, 1] = H * a * (tx * dty * gdot).sum(-1)
        gv[:, lsi[l]:lsi[l] + H * W] += np.einsum("bqmk,bqmkn,bqmd->bnmd", a, wt, g)
    return out, gv, gl, ga


def pin_brute_force(lib=None):
    """Dense tent-kernel brute force over every pixel (no floor, no corner
    enumeration) on tiny inputs."""
    for seed in (17, 18, 19):
        rng = np.random.default_rng(seed)
        value, shapes, lsi, loc, attn, g = random_case(rng, lo=-0.3, hi=1.3)
        ro, rgv, rgl, rga = _tent_dense(value, shapes, lsi, loc, attn, g)
        o = fwd(lib, value, shapes, lsi, loc, attn)
        gv, gl, ga = bwd(lib, value, shapes, lsi, loc, attn, g)
        _close(o, ro, 1e-12, "forward vs tent brute force")
        _close(gv, rgv, 1e-12, "value gradient vs tent brute force")
        _close(ga, rga, 1e-12, "weight gradient vs tent brute force")
        _close(gl, rgl, 1e-11, "location gradient vs tent brute force")


def pin_finite_differences(lib=None):
    """Analytic gradients equal finite differences of L = sum(g * out).
    L is linear in the value and the weights (central differences are exact);
    inside one cell it is linear in x at fixed y, so the difference quotient
    over the actual fp32 coordinates is exact too."""
    rng = np.random.default_rng(20)
    value, shapes, lsi, loc, attn, g = random_case(rng, B=1, M=2, D=3, Nq=3, K=2,
                                                   shapes=((4, 5), (3, 3)))
    loss = lambda v, lc, a: float((fwd(lib, v, shapes, lsi, lc, a) * g).sum())  # noqa: E731
    gv, gl, ga = bwd(lib, value, shapes, lsi, loc, attn, g)
    # value and weights
    for idx in np.ndindex(*value.shape):
        vp, vm = value.copy(), value.copy()
        vp[idx] += 0.5
        vm[idx] -= 0.5
        fd = loss(vp, loc, attn) - loss(vm, loc, attn)
        assert abs(fd - gv[idx]) <= 1e-12 * max(1.0, abs(fd)), f"d/dvalue{idx}"
    for idx in np.ndindex(*attn.shape):
        ap, am = attn.copy(), attn.copy()
        ap[idx] += 0.5
        am[idx] -= 0.5
        fd = loss(value, loc, ap) - loss(value, loc, am)
        assert abs(fd - ga[idx]) <= 1e-12 * max(1.0, abs(fd)), f"d/dweight{idx}"
    # locations: step 2^-12 in normalized units, skipped when the step crosses a cell
    h = np.float32(2.0 ** -12)
    checked = 0
    for idx in np.ndindex(*loc.shape):
        l, axis = idx[3], idx[5]
        n = shapes[l][1] if axis == 0 else shapes[l][0]
        lp, lm = loc.copy(), loc.copy()
        lp[idx] = np.float32(loc[idx] + h)
        lm[idx] = np.float32(loc[idx] - h)
        xp, xm = coord32(lp[idx], n), coord32(lm[idx], n)
        if np.floor(xp) != np.floor(xm) or np.floor(xm) != np.floor(coord32(loc[idx], n)):
            continue
        fd = (loss(value, lp, attn) - loss(value, lm, attn)) / (float(xp) - float(xm)) * n
        assert abs(fd - gl[idx]) <= 1e-9 * max(1.0, abs(fd)), f"d/dloc{idx}: {fd} vs {gl[idx]}"
        checked += 1
    assert checked > loc.size // 2, "too few location coordinates checked"


def pin_single_scale_resampling(lib=None):
    """With one level, one point and one head, the core is plain bilinear
    resampling of one image with zero padding: scipy.ndimage.map_coordinates
    (order 1, mode 'grid-constant', cval 0)."""
    from scipy import ndimage
    rng = np.random.default_rng(21)
    H, W, D, Nq = 7, 10, 3, 50
    shapes, lsi = level_tables(((H, W),))
    value = rng.standard_normal((1, H * W, 1, D))
    loc = rng.uniform(-0.2, 1.2, size=(1, Nq, 1, 1, 1, 2)).astype(np.float32)
    attn = np.ones((1, Nq, 1, 1, 1))
    out = fwd(lib, value, shapes, lsi, loc, attn)[0, :, 0]           # [Nq, D]
    x = coord32(loc[0, :, 0, 0, 0, 0], W).astype(np.float64)
    y = coord32(loc[0, :, 0, 0, 0, 1], H).astype(np.float64)
    for d in range(D):
        img = value[0, :, 0, d].reshape(H, W)
        ref = ndimage.map_coordinates(img, [y, x], order=1, mode="grid-constant", cval=0.0,
                                      prefilter=False)
        _close(out[:, d], ref, 1e-12, "single-scale resampling vs map_coordinates")


def pin_scatter_conservation(lib=None):
    """Summing the value gradient over all pixels gives, per (b, m, d),
    sum over samples of A * (sum of the inside corners' weights) * g; with
    every corner inside and softmax weights that is sum_q g."""
    rng = np.random.default_rng(22)
    shapes, lsi = level_tables(((6, 8), (3, 4)))
    B, M, D, K, Nq, L = 2, 2, 4, 3, 10, 2
    Nv = int((shapes[:, 0] * shapes[:, 1]).sum())
    value = rng.standard_normal((B, Nv, M, D))
    loc = np.empty((B, Nq, M, L, K, 2), np.float32)
    for l in range(L):
        H, W = shapes[l]
        loc[..., l, :, 0] = (rng.uniform(0, W - 1 - 1e-3, (B, Nq, M, K)) + 0.5) / W
        loc[..., l, :, 1] = (rng.uniform(0, H - 1 - 1e-3, (B, Nq, M, K)) + 0.5) / H
    logits = rng.standard_normal((B, Nq, M, L * K))
    attn = (np.exp(logits) / np.exp(logits).sum(-1, keepdims=True)).reshape(B, Nq, M, L, K)
    g = rng.standard_normal((B, Nq, M, D))
    gv, _, _ = bwd(lib, value, shapes, lsi, loc, attn, g)
    _close(gv.sum(1), g.sum(1), 1e-12, "value-gradient conservation")


def pin_permutation(lib=None):
    """Permuting queries, heads or batch entries (with their locations and
    weights) permutes the outputs the same way."""
    rng = np.random.default_rng(23)
    value, shapes, lsi, loc, attn, g = random_case(rng)
    o = fwd(lib, value, shapes, lsi, loc, attn)
    pq = rng.permutation(loc.shape[1])
    assert np.array_equal(fwd(lib, value, shapes, lsi, loc[:, pq], attn[:, pq]), o[:, pq])
    pm = rng.permutation(value.shape[2])
    assert np.array_equal(fwd(lib, value[:, :, pm], shapes, lsi, loc[:, :, pm], attn[:, :, pm]),
                          o[:, :, pm])
    pb = rng.permutation(value.shape[0])
    assert np.array_equal(fwd(lib, value[pb], shapes, lsi, loc[pb], attn[pb]), o[pb])


# ----------------------------------------------------------------------------- term sums S
# Every GPU parity gate is |gpu - r| <= rho |r| + 1e-5 S, where S is the sum of
# the absolute values of the terms the oracle adds up for that element. These
# pins fix S without reading the oracle's own S code: where every term of an
# element is non-negative (the bilinear weights are), S is that element's
# result on inputs replaced by their absolute values; the location terms
# carry signed weight derivatives, so their S is summed from the dense tent
# form; and |r| <= S everywhere.

def _le_abs_sum(r, s, what):
    r, s = np.asarray(r, np.float64), np.asarray(s, np.float64)
    assert np.all(np.isfinite(s)), f"{what}: non-finite term sum"
    assert np.all(np.abs(r) <= s * (1.0 + 1e-12) + 1e-300), f"{what}: |result| exceeds its term sum"


def _tent_abs_location(value, shapes, lsi, loc, attn, g):
    """S of the location gradients from the dense tent form: level pixel n of
    the sample enters with the derivative of its tent weight, so
    S_x = W |A| sum_d |g_d| sum_n |d tent_n / dx| |v_n,d| (and the same in y
    with H). Valid away from integer coordinates."""
    B, Nv, M, D = value.shape
    out = np.zeros(loc.shape)
    for l in range(loc.shape[3]):
        H, W = shapes[l]
        yy, xx = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
        xn, yn = xx.reshape(-1).astype(np.float64), yy.reshape(-1).astype(np.float64)
        vl = np.abs(value[:, lsi[l]:lsi[l] + H * W])
        x = coord32(loc[..., l, :, 0], W).astype(np.float64)[..., None]
        y = coord32(loc[..., l, :, 1], H).astype(np.float64)[..., None]
        tx = np.maximum(0.0, 1.0 - np.abs(x - xn))
        ty = np.maximum(0.0, 1.0 - np.abs(y - yn))
        near_x = (np.abs(x - xn) < 1.0).astype(np.float64)
        near_y = (np.abs(y - yn) < 1.0).astype(np.float64)
        gv = np.einsum("bqmd,bnmd->bqmn", np.abs(g), vl)[:, :, :, None, :]
        a = np.abs(attn[..., l, :])
        out[..., l, :, 0] = W * a * (near_x * ty * gv).sum(-1)
        out[..., l, :, 1] = H * a * (tx * near_y * gv).sum(-1)
    return out


def pin_abs_sums_core(lib=None):
    """Term sums of the core forward and backward: forward S = forward of
    |value| with |A|; grad_value S = grad_value with |A| and |g|; weight
    gradient S = weight gradient of |value| and |g|; location gradient S from
    the tent form; |result| <= S."""
    for seed in (24, 25):
        rng = np.random.default_rng(seed)
        value, shapes, lsi, loc, attn, g = random_case(rng, lo=-0.3, hi=1.3)
        o, oa = oracle.forward(value, shapes, lsi, loc, attn, with_abs=True, lib=lib)
        gv, gl, ga, gva, gla, gaa = oracle.backward(value, shapes, lsi, loc, attn, g,
                                                    with_abs=True, lib=lib)
        av, aa, ag = np.abs(value), np.abs(attn), np.abs(g)
        _close(oa, fwd(lib, av, shapes, lsi, loc, aa), 1e-13, "forward S = forward(|value|, |A|)")
        gv_pos, _, ga_pos = bwd(lib, av, shapes, lsi, loc, aa, ag)
        gv_a, _, _ = bwd(lib, value, shapes, lsi, loc, aa, ag)
        _close(gva, gv_a, 1e-13, "grad_value S = grad_value(|A|, |g|)")
        _close(gaa, ga_pos, 1e-13, "weight-gradient S = weight gradient(|value|, |g|)")
        _close(gla, _tent_abs_location(value, shapes, lsi, loc, attn, g), 1e-12,
               "location-gradient S vs tent form")
        for r, s, what in ((o, oa, "output"), (gv, gva, "grad_value"), (gl, gla, "grad_loc"),
                           (ga, gaa, "grad_attn")):
            _le_abs_sum(r, s, what)
        # non-negative inputs: every term of the output is non-negative
        _close(fwd(lib, av, shapes, lsi, loc, aa), oa, 1e-13, "S equals r for non-negative terms")


def _fused_locations(shapes, ref, off):
    """Single-precision locations of the fused front-end (quotient, then sum,
    each rounded to float) and the matching (W, H) per level."""
    L = ref.shape[2]
    loc = np.empty(off.shape, np.float32)
    for l in range(L):
        H, W = shapes[l]
        q = (off[:, :, :, l] / np.array([W, H], np.float32)).astype(np.float32)
        loc[:, :, :, l] = (ref[:, :, None, l, None, :] + q).astype(np.float32)
    return loc


def pin_abs_sums_fused(lib=None):
    """Term sums of the fused front-end, from the core's (pinned above): the
    value-gradient S is the core's at the fused locations and softmax weights;
    the offset S is the core location S over (W, H); the reference-point S is
    its sum over heads and points; the logit S is A_j (S_gA_j + sum_i A_i
    S_gA_i), the two terms of the softmax Jacobian; |result| <= S."""
    rng = np.random.default_rng(35)
    value, shapes, lsi, ref, off, logits, g = random_fused_case(rng)
    B, Nq, M, L, K, _ = off.shape
    o, oa = oracle.forward_fused(value, shapes, lsi, ref, off, logits, with_abs=True, lib=lib)
    outs = oracle.backward_fused(value, shapes, lsi, ref, off, logits, g, with_abs=True, lib=lib)
    gv, gr, go, gz, gva, gra, goa, gza = outs
    z = logits.astype(np.float64)
    e = np.exp(z - z.max(-1, keepdims=True))
    A = (e / e.sum(-1, keepdims=True)).reshape(B, Nq, M, L, K)
    loc = _fused_locations(shapes, ref, off)
    _, coa = oracle.forward(value, shapes, lsi, loc, A, with_abs=True, lib=lib)
    _, _, _, cgva, cgla, cgaa = oracle.backward(value, shapes, lsi, loc, A, g, with_abs=True,
                                                lib=lib)
    _close(oa, coa, 1e-12, "fused forward S")
    _close(gva, cgva, 1e-12, "fused grad_value S")
    wh = np.array([[shapes[l][1], shapes[l][0]] for l in range(L)], np.float64)
    _close(goa, cgla / wh[None, None, None, :, None, :], 1e-12, "offset-gradient S")
    _close(gra, cgla.sum(axis=(2, 4)), 1e-12, "reference-point-gradient S")
    ga_s = cgaa.reshape(B, Nq, M, L * K)
    a = A.reshape(B, Nq, M, L * K)
    _close(gza, a * (ga_s + (a * ga_s).sum(-1, keepdims=True)), 1e-12, "logit-gradient S")
    for r, s, what in ((o, oa, "fused output"), (gv, gva, "fused grad_value"),
                       (gr, gra, "grad_ref"), (go, goa, "grad_off"), (gz, gza, "grad_logits")):
        _le_abs_sum(r, s, what)


# ----------------------------------------------------------------------------- fused front-end
# Pinned conventions (cf-1.com section 3.2): location = reference point +
# offset / (W_l, H_l) with offsets in level pixels and the normalizer stacked
# (W, H); weights = softmax of the logits over the L*K samples of one (query,
# head) (also CSDN explainer section 3 note 3).

def random_fused_case(rng, B=2, M=3, D=4, shapes=((4, 6), (3, 5), (2, 2)), Nq=5, K=2):
    shapes, lsi = level_tables(shapes)
    L = shapes.shape[0]
    Nv = int((shapes[:, 0] * shapes[:, 1]).sum())
    value = rng.standard_normal((B, Nv, M, D))
    ref = rng.uniform(0.0, 1.0, size=(B, Nq, L, 2)).astype(np.float32)
    off = (rng.standard_normal((B, Nq, M, L, K, 2)) * 1.5).astype(np.float32)
    logits = (rng.standard_normal((B, Nq, M, L * K)) * 2.0).astype(np.float32)
    g = rng.standard_normal((B, Nq, M, D))
    return value, shapes, lsi, ref, off, logits, g


def fused_torch(V, R, O, Z, shapes, lsi, ref32, off32):
    """The fused front-end and the core on torch float64 tensors V [B,Nv,M,D],
    R [B,Nq,L,2], O [B,Nq,M,L,K,2], Z [B,Nq,M,L*K] (any of them may be
    non-leaf): torch's softmax for the weights, per-level grid_sample
    (bilinear, zeros padding, align_corners=False) for the samples. The
    normalized location carries the single-precision value the core samples
    at, formed from the float32 arrays ref32 and off32 (the quotient and the
    sum rounded to float), while its gradient flows through the exact float64
    expression of R and O. Returns out [B,Nq,M,D]."""
    import torch
    import torch.nn.functional as F
    B, Nv, M, D = V.shape
    _, Nq, _, L, K, _ = O.shape
    A = torch.softmax(Z, dim=-1).reshape(B, Nq, M, L, K)
    out = torch.zeros(B, Nq, M, D, dtype=torch.float64)
    for l in range(L):
        H, W = int(shapes[l][0]), int(shapes[l][1])
        norm = torch.tensor([W, H], dtype=torch.float64)
        u = R[:, :, None, l, None, :] + O[:, :, :, l] / norm          # [B, Nq, M, K, 2]
        q32 = (off32[:, :, :, l] / np.array([W, H], np.float32)).astype(np.float32)
        u32 = (ref32[:, :, None, l, None, :] + q32).astype(np.float32)
        x32 = np.stack([coord32(u32[..., 0], W), coord32(u32[..., 1], H)], -1)
        u_at = torch.tensor((x32.astype(np.float64) + 0.5) / np.array([W, H], np.float64))
        u_used = u + (u_at - u).detach()
        v_l = V[:, lsi[l]:lsi[l] + H * W].permute(0, 2, 3, 1).reshape(B * M, D, H, W)
        grid = (2.0 * u_used - 1.0).permute(0, 2, 1, 3, 4).reshape(B * M, Nq, K, 2)
        s = F.grid_sample(v_l, grid, mode="bilinear", padding_mode="zeros",
                          align_corners=False)                            # [B*M, D, Nq, K]
        s = s.reshape(B, M, D, Nq, K).permute(0, 3, 1, 4, 2)              # [B, Nq, M, K, D]
        out = out + (A[:, :, :, l, :, None] * s).sum(3)
    return out


def _fused_torch_reference(value, shapes, lsi, ref, off, logits, g):
    """fused_torch on leaf tensors made from numpy inputs, with the
    gradients of sum(g * out)."""
    import torch
    V = torch.tensor(value, dtype=torch.float64, requires_grad=True)
    R = torch.tensor(ref.astype(np.float64), requires_grad=True)
    O = torch.tensor(off.astype(np.float64), requires_grad=True)
    Z = torch.tensor(logits.astype(np.float64), requires_grad=True)
    out = fused_torch(V, R, O, Z, shapes, lsi, ref, off)
    (out * torch.tensor(g, dtype=torch.float64)).sum().backward()
    return (out.detach().numpy(), V.grad.numpy(), R.grad.numpy(), O.grad.numpy(),
            Z.grad.numpy())


def pin_fused_torch(lib=None):
    """Fused forward and all four gradients equal torch's softmax + per-level
    grid_sample with autograd (library routines, independent code)."""
    for seed in (31, 32):
        rng = np.random.default_rng(seed)
        value, shapes, lsi, ref, off, logits, g = random_fused_case(rng)
        ro, rgv, rgr, rgo, rgz = _fused_torch_reference(value, shapes, lsi, ref, off, logits, g)
        o = oracle.forward_fused(value, shapes, lsi, ref, off, logits, lib=lib)
        gv, gr, go, gz = oracle.backward_fused(value, shapes, lsi, ref, off, logits, g, lib=lib)
        _close(o, ro, 1e-12, "fused forward vs torch")
        _close(gv, rgv, 1e-12, "fused value gradient vs torch")
        _close(gz, rgz, 1e-12, "logit gradient vs torch")
        _close(go, rgo, 1e-10, "offset gradient vs torch")
        _close(gr, rgr, 1e-10, "reference-point gradient vs torch")


def pin_fused_pixel_shift(lib=None):
    """Closed form: reference points at pixel centres of power-of-two levels and
    whole-pixel offsets (all exact in float) land on pixel centres; with one
    logit far above the others the output is the value at the shifted pixel."""
    shapes, lsi = level_tables([(4, 8), (2, 4)])
    L, K, M, D, Nq = 2, 2, 2, 3, 4
    rng = np.random.default_rng(33)
    Nv = int((shapes[:, 0] * shapes[:, 1]).sum())
    value = rng.standard_normal((1, Nv, M, D))
    ref = np.zeros((1, Nq, L, 2), np.float32)
    off = np.zeros((1, Nq, M, L, K, 2), np.float32)
    logits = np.full((1, Nq, M, L * K), -200.0, np.float32)
    want = np.zeros((1, Nq, M, D))
    for q in range(Nq):
        for l in range(L):
            H, W = shapes[l]
            i, j = rng.integers(0, W), rng.integers(0, H)
            ref[0, q, l] = ((i + 0.5) / W, (j + 0.5) / H)
        for m in range(M):
            l, k = rng.integers(0, L), rng.integers(0, K)
            H, W = shapes[l]
            i = int(round(ref[0, q, l, 0] * W - 0.5))
            j = int(round(ref[0, q, l, 1] * H - 0.5))
            di, dj = rng.integers(-i, W - i), rng.integers(-j, H - j)
            off[0, q, m, l, k] = (di, dj)
            logits[0, q, m, l * K + k] = 0.0
            want[0, q, m] = value[0, lsi[l] + (j + dj) * W + (i + di), m]
    o = oracle.forward_fused(value, shapes, lsi, ref, off, logits, lib=lib)
    _close(o, want, 1e-12, "fused pixel shift")


def pin_fused_finite_differences(lib=None):
    """Gradients of L = sum(g * out) with respect to logits, offsets and
    reference points equal difference quotients of the fused oracle (smooth in
    the logits; linear in the pixel coordinate inside a cell)."""
    rng = np.random.default_rng(34)
    value, shapes, lsi, ref, off, logits, g = random_fused_case(rng, B=1, M=2, D=3, Nq=2, K=2,
                                                                shapes=((3, 4), (2, 3)))
    loss = lambda r, o, z: float((oracle.forward_fused(value, shapes, lsi, r, o, z, lib=lib)  # noqa: E731
                                  * g).sum())
    _, gr, go, gz = oracle.backward_fused(value, shapes, lsi, ref, off, logits, g, lib=lib)
    for idx in np.ndindex(*logits.shape):
        zp, zm = logits.copy(), logits.copy()
        h = 2.0 ** -8
        zp[idx] += h
        zm[idx] -= h
        fd = (loss(ref, off, zp) - loss(ref, off, zm)) / (2 * h)
        assert abs(fd - gz[idx]) <= 1e-4 * max(1.0, abs(fd)), f"d/dlogit{idx}: {fd} vs {gz[idx]}"
    h = np.float32(2.0 ** -10)
    checked = 0
    for idx in np.ndindex(*off.shape):
        l, axis = idx[3], idx[5]
        n = shapes[l][1] if axis == 0 else shapes[l][0]
        op, om = off.copy(), off.copy()
        op[idx] = np.float32(off[idx] + h)
        om[idx] = np.float32(off[idx] - h)
        base = ref[idx[0], idx[1], l, axis]
        xs = [coord32(np.float32(base + np.float32(o_ / np.float32(n))), n)
              for o_ in (op[idx], om[idx], off[idx])]
        if len({float(np.floor(x)) for x in xs}) != 1:
            continue
        fd = (loss(ref, op, logits) - loss(ref, om, logits)) / (float(xs[0]) - float(xs[1]))
        assert abs(fd - go[idx]) <= 1e-6 * max(1.0, abs(fd)), f"d/doffset{idx}: {fd} vs {go[idx]}"
        checked += 1
    assert checked > off.size // 2, "too few offsets checked"
    # a reference point moves every head's and point's location on its level
    h = np.float32(2.0 ** -12)
    checked = 0
    for idx in np.ndindex(*ref.shape):
        l, axis = idx[2], idx[3]
        n = shapes[l][1] if axis == 0 else shapes[l][0]
        rp, rm = ref.copy(), ref.copy()
        rp[idx] = np.float32(ref[idx] + h)
        rm[idx] = np.float32(ref[idx] - h)
        q = (off[idx[0], idx[1], :, l, :, axis] / np.float32(n)).astype(np.float32)
        cells = [np.floor(coord32((r_[idx] + q).astype(np.float32), n)) for r_ in (rp, rm, ref)]
        if not (np.array_equal(cells[0], cells[2]) and np.array_equal(cells[1], cells[2])):
            continue
        fd = (loss(rp, off, logits) - loss(rm, off, logits)) / (float(rp[idx]) - float(rm[idx]))
        assert abs(fd - gr[idx]) <= 1e-4 * max(1.0, abs(fd)), f"d/dref{idx}: {fd} vs {gr[idx]}"
        checked += 1
    assert checked > 0, "no reference point checked"


ALL_PINS = [pin_golden_hand_worked, pin_pixel_centres, pin_constant_field, pin_bilinear_field,
            pin_out_of_bounds, pin_linearity, pin_grid_sample, pin_brute_force,
            pin_finite_differences, pin_single_scale_resampling, pin_scatter_conservation,
            pin_permutation, pin_fused_torch, pin_fused_pixel_shift, pin_fused_finite_differences,
            pin_abs_sums_core, pin_abs_sums_fused]


# ----------------------------------------------------------------------------- DCNv3 aggregation
def _dcn_out_size(H, W, kernel, stride, pad, dilation):
    return ((H + 2 * pad[0] - dilation[0] * (kernel[0] - 1) - 1) // stride[0] + 1,
            (W + 2 * pad[1] - dilation[1] * (kernel[1] - 1) - 1) // stride[1] + 1)


def _depthwise_correlation(x, kern, stride, pad, dilation):
    """scipy.signal.correlate2d of each channel plane of x [H, W, G, D] with
    its group's kernel kern [G, kh, kw], dilated by inserting zeros, over the
    zero-padded input, then strided: a depthwise convolution layer."""
    from scipy.signal import correlate2d
    H, W, G, D = x.shape
    kh, kw = kern.shape[1:]
    Ho, Wo = _dcn_out_size(H, W, (kh, kw), stride, pad, dilation)
    out = np.zeros((Ho, Wo, G, D))
    for g in range(G):
        kd = np.zeros(((kh - 1) * dilation[0] + 1, (kw - 1) * dilation[1] + 1))
        kd[::dilation[0], ::dilation[1]] = kern[g]
        for d in range(D):
            xp = np.pad(x[:, :, g, d], ((pad[0], pad[0]), (pad[1], pad[1])))
            full = correlate2d(xp, kd, mode="valid")
            out[:, :, g, d] = full[::stride[0], ::stride[1]][:Ho, :Wo]
    return out


DCN_CONFIGS = [((3, 3), (1, 1), (1, 1), (1, 1)), ((3, 3), (2, 2), (1, 1), (1, 1)),
               ((5, 3), (1, 2), (4, 1), (2, 1)), ((3, 2), (2, 1), (2, 3), (1, 3)),
               ((1, 1), (1, 1), (0, 0), (1, 1))]


def pin_dcn_depthwise_conv(lib=None):
    """Zero offsets and a mask that depends only on (g, k): the aggregation is
    a depthwise convolution (scipy correlate2d over the zero-padded input,
    dilated kernel, strided), for several kernel/stride/pad/dilation sets."""
    rng = np.random.default_rng(51)
    for kernel, stride, pad, dil in DCN_CONFIGS:
        H, W, G, D = 7, 9, 2, 3
        x = rng.standard_normal((1, H, W, G, D))
        Ho, Wo = _dcn_out_size(H, W, kernel, stride, pad, dil)
        K = kernel[0] * kernel[1]
        kern = rng.standard_normal((G, kernel[0], kernel[1]))
        mask = np.broadcast_to(kern.reshape(1, 1, 1, G, K), (1, Ho, Wo, G, K)).copy()
        off = np.zeros((1, Ho, Wo, G, K, 2), np.float32)
        got = oracle.dcn_forward(x, off, mask, kernel, stride, pad, dil, lib=lib)
        want = _depthwise_correlation(x[0], kern, stride, pad, dil)
        _close(got[0], want, 1e-12, f"dcn as depthwise conv {kernel} {stride} {pad} {dil}")


def pin_dcn_integer_shift(lib=None):
    """Whole-pixel offsets (dx, dy), the same for every sample: the result is
    the zero-offset aggregation of the input translated by (-dx, -dy)."""
    rng = np.random.default_rng(52)
    H, W, G, D = 8, 10, 2, 2
    x = rng.standard_normal((1, H, W, G, D))
    kernel, stride, pad, dil = (3, 3), (1, 1), (1, 1), (1, 1)
    Ho, Wo = _dcn_out_size(H, W, kernel, stride, pad, dil)
    mask = rng.standard_normal((1, Ho, Wo, G, 9))
    for dx, dy in ((1, 0), (0, -2), (3, 1)):
        off = np.zeros((1, Ho, Wo, G, 9, 2), np.float32)
        off[..., 0], off[..., 1] = dx, dy
        xs = np.zeros_like(x)
        ys, ye = max(0, -dy), min(H, H - dy)
        xs_, xe = max(0, -dx), min(W, W - dx)
        xs[0, ys:ye, xs_:xe] = x[0, ys + dy:ye + dy, xs_ + dx:xe + dx]
        got = oracle.dcn_forward(x, off, mask, kernel, stride, pad, dil, lib=lib)
        want = oracle.dcn_forward(xs, np.zeros_like(off), mask, kernel, stride, pad, dil, lib=lib)
        # compare the output pixels whose grid points, shifted or not, all lie
        # inside the input (elsewhere the translated copy has lost pixels)
        ho, wo = np.arange(Ho)[:, None], np.arange(Wo)[None, :]
        inside = (ho - 1 >= 0) & (ho + 1 < H) & (wo - 1 >= 0) & (wo + 1 < W) & \
            (ho - 1 + dy >= 0) & (ho + 1 + dy < H) & (wo - 1 + dx >= 0) & (wo + 1 + dx < W)
        assert inside.sum() >= 6
        _close(got[0][inside], want[0][inside], 1e-12, f"dcn integer shift ({dx}, {dy})")


def _dcn_as_core(rng, B=2):
    """A DCNv3 problem on a power-of-two input with dyadic offsets, and the same
    problem as a core problem: the pixel point P maps to the normalized
    location (P + 0.5) / (W, H) exactly (heads = groups, one level, weights =
    mask)."""
    H, W, G, D = 8, 16, 2, 3
    kernel, stride, pad, dil = (3, 3), (1, 2), (1, 1), (2, 1)
    Ho, Wo = _dcn_out_size(H, W, kernel, stride, pad, dil)
    K = 9
    x = rng.standard_normal((B, H, W, G, D))
    off = (rng.integers(-48, 49, size=(B, Ho, Wo, G, K, 2)) / 16.0).astype(np.float32)
    mask = rng.standard_normal((B, Ho, Wo, G, K))
    g = rng.standard_normal((B, Ho, Wo, G, D))
    ky, kx = np.divmod(np.arange(K), kernel[1])
    ho = np.arange(Ho)[None, :, None, None, None]
    wo = np.arange(Wo)[None, None, :, None, None]
    kx, ky = kx[None, None, None, None, :], ky[None, None, None, None, :]
    Px = (wo * stride[1] - pad[1] + kx * dil[1]) + off[..., 0].astype(np.float64)
    Py = (ho * stride[0] - pad[0] + ky * dil[0]) + off[..., 1].astype(np.float64)
    loc = np.stack([(Px + 0.5) / W, (Py + 0.5) / H], -1)                # [B,Ho,Wo,G,K,2]
    loc = loc.reshape(B, Ho * Wo, G, 1, K, 2).astype(np.float32)
    shapes, lsi = level_tables([(H, W)])
    core = dict(value=x.reshape(B, H * W, G, D), shapes=shapes, lsi=lsi, loc=loc,
                attn=mask.reshape(B, Ho * Wo, G, 1, K), g=g.reshape(B, Ho * Wo, G, D))
    dcn = dict(x=x, off=off, mask=mask, g=g, kernel=kernel, stride=stride, pad=pad, dil=dil)
    return dcn, core, (W, H)


def pin_dcn_matches_core(lib=None):
    """On power-of-two sizes with dyadic offsets the pixel point P maps to the
    normalized location (P + 0.5) / (W, H) exactly, so the aggregation equals
    the core on one level (heads = groups, weights = mask), and its gradients
    equal the core's: grad_offset = grad_loc / (W, H), grad_mask = grad_attn."""
    dc, c, (W, H) = _dcn_as_core(np.random.default_rng(53))
    geo = (dc["kernel"], dc["stride"], dc["pad"], dc["dil"])
    want = oracle.forward(c["value"], c["shapes"], c["lsi"], c["loc"], c["attn"], lib=lib)
    got = oracle.dcn_forward(dc["x"], dc["off"], dc["mask"], *geo, lib=lib)
    _close(got.reshape(want.shape), want, 1e-12, "dcn forward vs core")
    rgv, rgl, rga = oracle.backward(c["value"], c["shapes"], c["lsi"], c["loc"], c["attn"],
                                    c["g"], lib=lib)
    gi, go, gm = oracle.dcn_backward(dc["x"], dc["off"], dc["mask"], dc["g"], *geo, lib=lib)
    _close(gi.reshape(rgv.shape), rgv, 1e-12, "dcn grad_input vs core grad_value")
    _close(gm.reshape(rga.shape), rga, 1e-12, "dcn grad_mask vs core grad_attn")
    _close(go.reshape(rgl.shape), rgl / np.array([W, H], np.float64), 1e-12,
           "dcn grad_offset vs core grad_loc / (W, H)")


def pin_abs_sums_dcn(lib=None):
    """Term sums of the DCNv3 aggregation: forward S = aggregation of |input|
    with |mask|; grad_input S = grad_input with |mask| and |g|; grad_mask S =
    grad_mask of |input| and |g|; offset S = the core's location S (pinned by
    the tent form) over (W, H) on the exact mapping above; |result| <= S."""
    dc, c, (W, H) = _dcn_as_core(np.random.default_rng(55))
    geo = (dc["kernel"], dc["stride"], dc["pad"], dc["dil"])
    x, off, mask, g = dc["x"], dc["off"], dc["mask"], dc["g"]
    o, oa = oracle.dcn_forward(x, off, mask, *geo, with_abs=True, lib=lib)
    gi, go, gm, gia, goa, gma = oracle.dcn_backward(x, off, mask, g, *geo, with_abs=True, lib=lib)
    _close(oa, oracle.dcn_forward(np.abs(x), off, np.abs(mask), *geo, lib=lib), 1e-13,
           "dcn forward S = forward(|input|, |mask|)")
    gi_a, _, _ = oracle.dcn_backward(x, off, np.abs(mask), np.abs(g), *geo, lib=lib)
    _close(gia, gi_a, 1e-13, "dcn grad_input S = grad_input(|mask|, |g|)")
    _, _, gm_a = oracle.dcn_backward(np.abs(x), off, mask, np.abs(g), *geo, lib=lib)
    _close(gma, gm_a, 1e-13, "dcn grad_mask S = grad_mask(|input|, |g|)")
    _, _, _, _, cgla, _ = oracle.backward(c["value"], c["shapes"], c["lsi"], c["loc"], c["attn"],
                                          c["g"], with_abs=True, lib=lib)
    _close(goa.reshape(cgla.shape), cgla / np.array([W, H], np.float64), 1e-12,
           "dcn offset S = core location S / (W, H)")
    for r, s, what in ((o, oa, "dcn output"), (gi, gia, "grad_input"), (go, goa, "grad_offset"),
                       (gm, gma, "grad_mask")):
        _le_abs_sum(r, s, what)


def pin_dcn_finite_differences(lib=None):
    """Gradients of L = sum(g * out) equal difference quotients: exact for the
    mask and the input (L is linear in them), and for offsets moved by less
    than the distance to the next pixel line (L is bilinear inside a cell)."""
    rng = np.random.default_rng(54)
    H, W, G, D = 5, 6, 2, 2
    kernel, stride, pad, dil = (3, 3), (1, 1), (1, 1), (1, 1)
    Ho, Wo = _dcn_out_size(H, W, kernel, stride, pad, dil)
    x = rng.standard_normal((1, H, W, G, D))
    off = (rng.uniform(-1.5, 1.5, size=(1, Ho, Wo, G, 9, 2))).astype(np.float32)
    # keep offsets away from pixel lines so a small step stays in its cell
    off = (np.floor(off) + 0.25 + 0.5 * (off - np.floor(off))).astype(np.float32)
    mask = rng.standard_normal((1, Ho, Wo, G, 9))
    g = rng.standard_normal((1, Ho, Wo, G, D))
    loss = lambda x_, o_, m_: float((oracle.dcn_forward(x_, o_, m_, kernel, stride, pad, dil,  # noqa: E731
                                                        lib=lib) * g).sum())
    gi, go, gm = oracle.dcn_backward(x, off, mask, g, kernel, stride, pad, dil, lib=lib)
    for idx in [(0, 1, 2, 1, 4), (0, 0, 0, 0, 0), (0, 3, 5, 1, 8)]:
        mp, mm = mask.copy(), mask.copy()
        mp[idx] += 0.5
        mm[idx] -= 0.5
        fd = (loss(x, off, mp) - loss(x, off, mm)) / 1.0
        assert abs(fd - gm[idx]) <= 1e-9 * max(1.0, abs(fd)), f"d/dmask{idx}: {fd} vs {gm[idx]}"
        for c in range(2):
            op, om = off.copy(), off.copy()
            h = 2.0 ** -10
            op[idx + (c,)] += h
            om[idx + (c,)] -= h
            fd = (loss(x, op, mask) - loss(x, om, mask)) / (2 * h)
            assert abs(fd - go[idx + (c,)]) <= 1e-6 * max(1.0, abs(fd)), \
                f"d/doffset{idx + (c,)}: {fd} vs {go[idx + (c,)]}"
    for idx in [(0, 2, 3, 1, 0), (0, 4, 5, 0, 1)]:
        xp, xm = x.copy(), x.copy()
        xp[idx] += 0.5
        xm[idx] -= 0.5
        fd = loss(xp, off, mask) - loss(xm, off, mask)
        assert abs(fd - gi[idx]) <= 1e-9 * max(1.0, abs(fd)), f"d/dinput{idx}: {fd} vs {gi[idx]}"


ALL_PINS += [pin_dcn_depthwise_conv, pin_dcn_integer_shift, pin_dcn_matches_core,
             pin_dcn_finite_differences, pin_abs_sums_dcn]
