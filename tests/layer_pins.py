"""Pins of the layer oracle (oracle/layer.py) against things other than
itself: plain loops for the linear layer's definition, finite differences for
its gradients, and torch float64 autograd (F.linear, softmax, grid_sample) for
the composed MSDeformAttn layer. Every pin takes the oracle layer module so
that the mutation tests can hand in planted-mistake copies."""
import numpy as np

import pins


def _close(got, want, tol, what):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    scale = max(1.0, float(np.max(np.abs(want))) if want.size else 1.0)
    err = float(np.max(np.abs(got - want))) if want.size else 0.0
    assert err <= tol * scale, f"{what}: max error {err:.3e} (scale {scale:.3e})"


def pin_linear_loops(L):
    """y = x W^T + b equals the plain triple loop on a tiny non-square case;
    identity weights return x + b."""
    rng = np.random.default_rng(41)
    x = rng.standard_normal((3, 5))
    w = rng.standard_normal((4, 5))
    b = rng.standard_normal(4)
    want = np.zeros((3, 4))
    for r in range(3):
        for o in range(4):
            acc = b[o]
            for i in range(5):
                acc += x[r, i] * w[o, i]
            want[r, o] = acc
    _close(L.linear_forward(x, w, b), want, 1e-14, "linear forward vs loops")
    _close(L.linear_forward(x, np.eye(5), np.arange(5.0)), x + np.arange(5.0), 0.0,
           "linear with identity weights")


def pin_linear_finite_differences(L):
    """Gradients of sum(g * (x W^T + b)) equal central differences (exact up to
    rounding: the function is linear in each argument)."""
    rng = np.random.default_rng(42)
    x = rng.standard_normal((3, 5))
    w = rng.standard_normal((4, 5))
    b = rng.standard_normal(4)
    g = rng.standard_normal((3, 4))
    gx, gw, gb = L.linear_backward(x, w, g)
    f = lambda x_, w_, b_: float((L.linear_forward(x_, w_, b_) * g).sum())  # noqa: E731
    h = 0.5
    for arr, grad, name in ((x, gx, "x"), (w, gw, "w"), (b, gb, "b")):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(*arr.shape):
            p, m = arr.copy(), arr.copy()
            p[idx] += h
            m[idx] -= h
            args_p = [x, w, b]
            args_m = [x, w, b]
            k = {"x": 0, "w": 1, "b": 2}[name]
            args_p[k], args_m[k] = p, m
            fd[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
        _close(grad, fd, 1e-12, f"linear grad_{name} vs finite differences")


def random_layer_case(rng, B=2, Nq=5, M=2, D=3, K=2, shapes=((4, 6), (3, 5)), Nv_extra=0):
    shapes, lsi = pins.level_tables(shapes)
    L = shapes.shape[0]
    Nv = int((shapes[:, 0] * shapes[:, 1]).sum())
    C, A = M * D, M * L * K
    p = {
        "w_value": rng.standard_normal((C, C)) * 0.5, "b_value": rng.standard_normal(C) * 0.1,
        "w_offset": rng.standard_normal((2 * A, C)), "b_offset": rng.standard_normal(2 * A),
        "w_attn": rng.standard_normal((A, C)), "b_attn": rng.standard_normal(A) * 0.5,
        "w_out": rng.standard_normal((C, C)) * 0.5, "b_out": rng.standard_normal(C) * 0.1,
    }
    query = rng.standard_normal((B, Nq, C))
    inp = rng.standard_normal((B, Nv, C))
    ref = rng.uniform(0.0, 1.0, size=(B, Nq, L, 2)).astype(np.float32)
    g = rng.standard_normal((B, Nq, C))
    return p, query, inp, ref, shapes, lsi, M, L, K, g


def _torch_layer(p, query, inp, ref, shapes, lsi, M, L, K, g):
    """The layer as torch float64 autograd: F.linear for the four projections,
    views as the pages' module takes them, pins.fused_torch for the core. The
    core samples at the location formed from the offsets rounded to float (the
    layer's tensors are single precision between steps)."""
    import torch
    import torch.nn.functional as F
    B, Nq, C = query.shape
    Nv = inp.shape[1]
    D = C // M
    T = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in p.items()}
    Q = torch.tensor(query, dtype=torch.float64, requires_grad=True)
    X = torch.tensor(inp, dtype=torch.float64, requires_grad=True)
    R = torch.tensor(ref.astype(np.float64), requires_grad=True)
    value = F.linear(X, T["w_value"], T["b_value"]).reshape(B, Nv, M, D)
    O = F.linear(Q, T["w_offset"], T["b_offset"]).reshape(B, Nq, M, L, K, 2)
    Z = F.linear(Q, T["w_attn"], T["b_attn"]).reshape(B, Nq, M, L * K)
    # the core reads the offsets and logits as single-precision tensors
    off32 = O.detach().numpy().astype(np.float32)
    Zs = Z + (torch.tensor(Z.detach().numpy().astype(np.float32).astype(np.float64)) -
              Z).detach()
    core = pins.fused_torch(value, R, O, Zs, shapes, lsi, ref, off32).reshape(B, Nq, C)
    out = F.linear(core, T["w_out"], T["b_out"])
    (out * torch.tensor(g, dtype=torch.float64)).sum().backward()
    grads = {k: t.grad.numpy() for k, t in T.items()}
    grads.update(query=Q.grad.numpy(), input_flatten=X.grad.numpy(),
                 reference_points=R.grad.numpy())
    return out.detach().numpy(), grads


def pin_layer_torch(L):
    """Layer forward and every gradient equal torch float64 autograd."""
    import torch  # noqa: F401
    for seed in (43, 44):
        rng = np.random.default_rng(seed)
        p, query, inp, ref, shapes, lsi, M, Lv, K, g = random_layer_case(rng)
        want, wgrads = _torch_layer(p, query, inp, ref, shapes, lsi, M, Lv, K, g)
        got = L.layer_forward(p, query, inp, ref, shapes, lsi, M, Lv, K)
        _close(got, want, 1e-10, "layer forward vs torch")
        grads = L.layer_backward(p, query, inp, ref, shapes, lsi, M, Lv, K, g)
        for k, v in wgrads.items():
            _close(grads[k], v, 1e-9, f"layer grad {k} vs torch")


def pin_layer_abs_bounds(L):
    """The propagated term sums S bound the results: |r| <= S everywhere, and
    S equals |r| where every term is non-negative (all inputs and weights
    non-negative: then no cancellation anywhere in the forward)."""
    rng = np.random.default_rng(45)
    p, query, inp, ref, shapes, lsi, M, Lv, K, g = random_layer_case(rng)
    out, s = L.layer_forward(p, query, inp, ref, shapes, lsi, M, Lv, K, with_abs=True)
    assert np.all(np.abs(out) <= s * (1 + 1e-12) + 1e-300), "forward bound"
    grads, sg = L.layer_backward(p, query, inp, ref, shapes, lsi, M, Lv, K, g, with_abs=True)
    for k in grads:
        assert np.all(np.abs(grads[k]) <= sg[k] * (1 + 1e-12) + 1e-300), f"bound of {k}"
    pa = {k: (np.abs(v) if k not in ("w_offset", "b_offset", "w_attn", "b_attn") else v)
          for k, v in p.items()}
    out, s = L.layer_forward(pa, np.abs(query), np.abs(inp), ref, shapes, lsi, M, Lv, K,
                             with_abs=True)
    _close(s, out, 1e-12, "S of a forward without cancellation")


ALL_LAYER_PINS = [pin_linear_loops, pin_linear_finite_differences, pin_layer_torch,
                  pin_layer_abs_bounds]
