"""Pins for the oracle's backward pass.

Independent checks: central finite differences in fp64, torch fp64 autograd of a dense
formulation (a library), the adjoint identity of the linear router map, numpy scatter-add, and
invariants (router gradients sum to zero per token; experts without rows get zero gradient)."""
import numpy as np
import pytest
import torch

import oracle
from inputs import bf16_bits_to_f32, make_layer_inputs, normal


def as64(a):
    return (bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


def exact_grid_logits(T, E, seed):
    # multiples of 2^-12 in [-4, 4): perturbing by 2^-10 stays exact in fp32
    g = np.random.default_rng(seed)
    return (g.integers(-2 ** 14, 2 ** 14, (T, E)) * 2.0 ** -12).astype(np.float32)


@pytest.mark.parametrize("renorm", [True, False])
def test_router_topk_bwd_finite_differences(renorm):
    T, E, k = 6, 10, 3
    l = exact_grid_logits(T, E, 1)
    idx, w = oracle.router_topk(l, k, renorm)
    dw = np.random.default_rng(2).standard_normal((T, k))
    dl = oracle.router_topk_bwd(l, idx, dw, renorm)
    h = 2.0 ** -10
    for t in range(T):
        for e in range(E):
            lp, lm = l.copy(), l.copy()
            lp[t, e] += h
            lm[t, e] -= h
            ip, wp = oracle.router_topk(lp, k, renorm)
            im, wm = oracle.router_topk(lm, k, renorm)
            assert np.array_equal(ip[t], idx[t]) and np.array_equal(im[t], idx[t])  # selection unchanged
            fd = ((wp[t] - wm[t]) * dw[t]).sum() / (2 * h)
            assert abs(fd - dl[t, e]) <= 1e-5 * max(1.0, abs(fd))
        assert abs(dl[t].sum()) < 1e-13                 # softmax gradients sum to zero
        if renorm:
            off = np.setdiff1d(np.arange(E), idx[t])
            assert np.all(dl[t, off] == 0.0)


def test_router_logits_bwd_adjoint_and_autograd():
    T, H, E = 9, 14, 5
    x = normal((T, H), 1.0, (920, 1), "bf16")
    wg = normal((H, E), 0.3, (920, 2), "bf16")
    dl = np.random.default_rng(3).standard_normal((T, E))
    dwg, dx = oracle.router_logits_bwd(x, wg, dl)
    x64, w64 = as64(x), as64(wg)
    lin = x64 @ w64
    # adjoint identity of l = x W: <dl, x W> = <x^T dl, W> = <dl W^T, x>
    lhs = (dl * lin).sum()
    assert abs(lhs - (dwg * w64).sum()) < 1e-11 * abs(lhs) + 1e-12
    assert abs(lhs - (dx * x64).sum()) < 1e-11 * abs(lhs) + 1e-12
    xt = torch.tensor(x64, requires_grad=True)
    wt = torch.tensor(w64, requires_grad=True)
    ((xt @ wt) * torch.tensor(dl)).sum().backward()
    np.testing.assert_allclose(dwg, wt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_expert_rows_bwd_finite_differences():
    H, I, E = 12, 8, 3
    counts = np.array([3, 0, 2], np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(offsets[-1])
    xp = normal((N, H), 1.0, (921, 1), "f32")
    gu = normal((E * H, 2 * I), 0.4, (921, 2), "f32")
    dn = normal((E * I, H), 0.4, (921, 3), "f32")
    dy = normal((N, H), 1.0, (921, 4), "f32")
    dx, dgu = oracle.expert_rows_bwd(xp, dy, offsets, gu, dn, want_gu=True)
    dy64 = dy.astype(np.float64)
    for r in range(N):
        for h in range(H):
            xpp, xpm = xp.copy(), xp.copy()
            xpp[r, h] += np.float32(1e-3)
            xpm[r, h] -= np.float32(1e-3)
            step = float(xpp[r, h]) - float(xpm[r, h])
            fp = (oracle.expert_rows(xpp, offsets, gu, dn, rows=np.array([r])) * dy64[r]).sum()
            fm = (oracle.expert_rows(xpm, offsets, gu, dn, rows=np.array([r])) * dy64[r]).sum()
            assert abs((fp - fm) / step - dx[r, h]) <= 1e-6 * max(1.0, abs(dx[r, h]))
    # d(g|u): perturb the pre-activations through the FFN's definition via torch autograd
    x64, gu64, dn64 = xp.astype(np.float64), gu.astype(np.float64), dn.astype(np.float64)
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        g = torch.tensor(x64[r0:r1] @ gu64[e * H:(e + 1) * H, :I], requires_grad=True)
        u = torch.tensor(x64[r0:r1] @ gu64[e * H:(e + 1) * H, I:], requires_grad=True)
        y = (torch.nn.functional.silu(g) * u) @ torch.tensor(dn64[e * I:(e + 1) * I])
        (y * torch.tensor(dy64[r0:r1])).sum().backward()
        np.testing.assert_allclose(dgu[r0:r1, :I], g.grad.numpy(), rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(dgu[r0:r1, I:], u.grad.numpy(), rtol=1e-10, atol=1e-13)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_expert_weight_grads_autograd_and_empty_experts(dtype):
    H, I, E = 16, 8, 4
    counts = np.array([5, 0, 1, 6], np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(offsets[-1])
    xp = normal((N, H), 1.0, (922, 1), dtype)
    gu = normal((E * H, 2 * I), 0.3, (922, 2), dtype)
    dn = normal((E * I, H), 0.3, (922, 3), dtype)
    dy = normal((N, H), 1.0, (922, 4), dtype)
    for e in range(E):
        dgu, ddn = oracle.expert_weight_grads(xp, dy, offsets, gu, dn, e)
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            assert np.all(dgu == 0) and np.all(ddn == 0)
            continue
        GU = torch.tensor(as64(gu)[e * H:(e + 1) * H], requires_grad=True)
        D = torch.tensor(as64(dn)[e * I:(e + 1) * I], requires_grad=True)
        X = torch.tensor(as64(xp)[r0:r1])
        gu_ = X @ GU
        y = (torch.nn.functional.silu(gu_[:, :I]) * gu_[:, I:]) @ D
        (y * torch.tensor(as64(dy)[r0:r1])).sum().backward()
        np.testing.assert_allclose(dgu, GU.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(ddn, D.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_combine_and_permute_bwd():
    T, H, k, N = 7, 10, 3, 21
    g = np.random.default_rng(5)
    ros = g.permutation(N).astype(np.int32)
    y = normal((N, H), 1.0, (923, 1), "f32")
    w = normal((T, k), 1.0, (923, 2), "f32")
    d_out = normal((T, H), 1.0, (923, 3), "f32")
    d_y, d_w = oracle.combine_bwd(d_out, y, ros, w)
    # finite differences of L = <d_out, combine(y, w)> with respect to w (L is linear in w)
    for t in range(T):
        for j in range(k):
            wp, wm = w.copy(), w.copy()
            wp[t, j] += np.float32(0.5)
            wm[t, j] -= np.float32(0.5)
            step = float(wp[t, j]) - float(wm[t, j])        # the step actually taken in fp32
            fd = ((oracle.combine(y, ros, wp) - oracle.combine(y, ros, wm)) * d_out.astype(np.float64)).sum()
            assert abs(fd / step - d_w[t, j]) < 1e-10 * max(1.0, abs(d_w[t, j]))
    # d_y of slot (t, j) is w[t,j] * d_out[t]: check via the adjoint <d_out, combine(y)> = <d_y, y>
    L = (oracle.combine(y, ros, w) * d_out.astype(np.float64)).sum()
    acc = sum((d_y[t, j] * y[ros[t * k + j]].astype(np.float64)).sum() for t in range(T) for j in range(k))
    assert abs(L - acc) < 1e-10 * abs(L)
    # permute backward: scatter-add of the k rows of every token (numpy add.at as the library)
    dxp = normal((N, H), 1.0, (923, 4), "bf16")
    add = normal((T, H), 1.0, (923, 5), "bf16")
    want = as64(add).copy()
    np.add.at(want, np.repeat(np.arange(T), k), as64(dxp)[ros])
    np.testing.assert_allclose(oracle.permute_bwd(dxp, ros, k, d_x_add=add), want, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("renorm", [True, False])
def test_whole_layer_backward_against_torch_autograd(renorm):
    """Compose the oracle's backward pieces along the layer and compare with torch fp64 autograd of
    the dense per-token formulation (selection fixed to the oracle's)."""
    T, H, I, E, k = 24, 16, 8, 6, 2
    d = make_layer_inputs(T, H, I, E, k, "f32", (924,), w_std=0.3, wg_std=0.3, shared=1, backward=True)
    x, wg, gu, dn = d["x"], d["w_gate"], d["gate_up"], d["down"]
    sgu, sdn, d_out = d["shared_gate_up"], d["shared_down"], d["d_out"]
    # ---- oracle composition
    r = oracle.moe_backward(x, gu, dn, k, d_out, w_gate=wg, renorm=renorm, shared_gate_up=sgu, shared_down=sdn)
    d_x, dwg = r["d_x"], r["d_w_gate"]
    dgu = np.concatenate([r["d_gate_up"][e] for e in range(E)])
    ddn = np.concatenate([r["d_down"][e] for e in range(E)])
    logits = oracle.router_logits(x, wg)
    idx, _ = oracle.router_topk(logits, k, renorm)
    # ---- torch fp64 autograd, dense formulation
    X = torch.tensor(x.astype(np.float64), requires_grad=True)
    WG = torch.tensor(wg.astype(np.float64), requires_grad=True)
    GU = torch.tensor(gu.astype(np.float64), requires_grad=True)
    DN = torch.tensor(dn.astype(np.float64), requires_grad=True)
    SGU = torch.tensor(sgu.astype(np.float64), requires_grad=True)
    SDN = torch.tensor(sdn.astype(np.float64), requires_grad=True)
    L = X @ WG
    S = torch.tensor(idx.astype(np.int64))
    if renorm:
        W = torch.softmax(L.gather(1, S), dim=1)
    else:
        W = torch.softmax(L, dim=1).gather(1, S)

    def ffn(xx, g_u, d_n):
        ii = d_n.shape[0]
        z = xx @ g_u
        return (torch.nn.functional.silu(z[:, :ii]) * z[:, ii:]) @ d_n

    out = ffn(X, SGU, SDN)
    for e in range(E):
        we = (W * (S == e)).sum(dim=1, keepdim=True)
        out = out + we * ffn(X, GU[e * H:(e + 1) * H], DN[e * I:(e + 1) * I])
    (out * torch.tensor(d_out.astype(np.float64))).sum().backward()
    tol = dict(rtol=2e-5, atol=2e-6)
    np.testing.assert_allclose(d_x, X.grad.numpy(), **tol)
    np.testing.assert_allclose(dwg, WG.grad.numpy(), **tol)
    np.testing.assert_allclose(dgu, GU.grad.numpy(), **tol)
    np.testing.assert_allclose(ddn, DN.grad.numpy(), **tol)
    np.testing.assert_allclose(r["d_shared_gate_up"], SGU.grad.numpy(), **tol)
    np.testing.assert_allclose(r["d_shared_down"], SDN.grad.numpy(), **tol)


def test_dropped_slots_contribute_nothing():
    """A slot whose row map is -1 behaves as a slot of weight 0: the combine, its backward and the
    permute backward give the same results as with that slot's weight (and gradient) set to zero."""
    T, H, k, N = 9, 12, 3, 27
    g = np.random.default_rng(6)
    ros = g.permutation(N).astype(np.int32)
    y = normal((N, H), 1.0, (926, 1), "f32")
    w = g.random((T, k)).astype(np.float32)
    d_out = normal((T, H), 1.0, (926, 2), "f32")
    drop = np.zeros(T * k, bool)
    drop[::4] = True
    ros_d = np.where(drop, -1, ros).astype(np.int32)
    w0 = np.where(drop.reshape(T, k), 0.0, w).astype(np.float32)
    np.testing.assert_array_equal(oracle.combine(y, ros_d, w), oracle.combine(y, ros, w0))
    dy_d, dw_d = oracle.combine_bwd(d_out, y, ros_d, w)
    dy_0, dw_0 = oracle.combine_bwd(d_out, y, ros, w0)
    np.testing.assert_array_equal(dy_d, dy_0)
    assert np.all(dw_d.reshape(-1)[drop] == 0.0)
    np.testing.assert_array_equal(dw_d.reshape(-1)[~drop], dw_0.reshape(-1)[~drop])
    dxp = normal((N, H), 1.0, (926, 3), "f32")
    dxp_0 = dxp.copy()
    dxp_0[ros[drop]] = 0.0
    np.testing.assert_array_equal(oracle.permute_bwd(dxp, ros_d, k), oracle.permute_bwd(dxp_0, ros, k))


def test_moe_backward_bf16_inputs_equal_their_fp32_values():
    """bf16 inputs give the same gradients as their (exact) fp32 values."""
    T, H, I, E, k = 10, 16, 8, 4, 2
    d = make_layer_inputs(T, H, I, E, k, "bf16", (927,), w_std=0.3, wg_std=0.3, shared=1, backward=True)
    f = {n: as64(a).astype(np.float32) for n, a in d.items()}
    args = ("x", "gate_up", "down")
    kw = lambda s: dict(w_gate=s["w_gate"], shared_gate_up=s["shared_gate_up"], shared_down=s["shared_down"])
    rb = oracle.moe_backward(*(d[n] for n in args), k, d["d_out"], **kw(d))
    rf = oracle.moe_backward(*(f[n] for n in args), k, f["d_out"], **kw(f))
    for key in ("d_x", "d_w_gate", "d_logits", "d_shared_gate_up", "d_shared_down"):
        np.testing.assert_array_equal(rb[key], rf[key])
    for e in range(E):
        np.testing.assert_array_equal(rb["d_gate_up"][e], rf["d_gate_up"][e])


def test_weight_grad_units_match_full_weight_grads():
    T, H, I, E, k = 40, 24, 12, 3, 2
    d = make_layer_inputs(T, H, I, E, k, "bf16", (928,), w_std=0.3, backward=True)
    counts = np.array([30, 0, 50], np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    xp = normal((80, H), 1.0, (928, 1), "bf16")
    dy = normal((80, H), 1.0, (928, 2), "bf16")
    units = np.array([0, 5, 11, 3])
    for e in range(E):
        dgu, ddn = oracle.expert_weight_grads(xp, dy, offsets, d["gate_up"], d["down"], e)
        g, u, r = oracle.expert_weight_grads_units(xp, dy, offsets, d["gate_up"], d["down"], e, units)
        np.testing.assert_allclose(g, dgu[:, units], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(u, dgu[:, I + units], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(r, ddn[units], rtol=1e-12, atol=1e-14)
        if counts[e] == 0:
            assert not g.any() and not u.any() and not r.any()


@pytest.mark.parametrize("renorm,shared", [(True, 1), (False, 0)])
def test_backward_tokens_match_full_backward(renorm, shared):
    T, H, I, E, k = 30, 16, 8, 6, 3
    d = make_layer_inputs(T, H, I, E, k, "bf16", (929,), w_std=0.3, wg_std=0.3, shared=shared, backward=True)
    kw = dict(w_gate=d["w_gate"], renorm=renorm, shared_gate_up=d.get("shared_gate_up"),
              shared_down=d.get("shared_down"))
    full = oracle.moe_backward(d["x"], d["gate_up"], d["down"], k, d["d_out"], **kw)
    toks = np.array([7, 0, 29, 13])
    part = oracle.moe_backward_tokens(d["x"], d["gate_up"], d["down"], k, d["d_out"], toks, **kw)
    for key in ("d_x", "d_logits", "d_w"):
        np.testing.assert_allclose(part[key], full[key][toks], rtol=1e-12, atol=1e-13)


def test_layer_weight_grad_units_match_full_backward():
    T, H, I, E, k = 40, 16, 8, 6, 2
    d = make_layer_inputs(T, H, I, E, k, "bf16", (930,), w_std=0.3, wg_std=0.3, backward=True)
    full = oracle.moe_backward(d["x"], d["gate_up"], d["down"], k, d["d_out"], w_gate=d["w_gate"])
    idx, w = oracle.router_topk(oracle.router_logits(d["x"], d["w_gate"]), k)
    units = np.array([6, 1, 7])
    for e in range(E):
        g, u, r = oracle.moe_weight_grads_units(d["x"], d["gate_up"], d["down"], idx, w, d["d_out"], e, units)
        np.testing.assert_allclose(g, full["d_gate_up"][e][:, units], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(u, full["d_gate_up"][e][:, I + units], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(r, full["d_down"][e][units], rtol=1e-12, atol=1e-14)
