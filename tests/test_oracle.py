"""Pins of the fp64 oracle to things other than itself.

* Central finite differences of L = sum(O * dO) through the oracle's own forward.
* PyTorch float64 autograd through its scaled-dot-product attention (a library
  routine computing the same function), forward and backward.
* Closed-form identities of softmax attention and special cases with known
  answers (S = 1, causal first query, identical keys, identical values).

The textbook gradient of softmax attention is the method's exact result: the
pages (DASH; zskr.cn explainer section 2.1; gist.science summary section 1)
only change the order in which dQ partials are summed.
"""
import math

import numpy as np
import pytest
import torch

from oracle import ref


def _rand(shape, seed):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape)


def _loss(q, k, v, dout, scale, causal):
    o, _ = ref.attn_fwd(q, k, v, scale, causal)
    return float(np.sum(o * dout))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S,D", [(1, 4), (2, 1), (3, 4), (5, 8), (8, 4)])
def test_backward_matches_finite_differences(S, D, causal):
    B, H = 1, 1
    q, k, v, dout = (_rand((B, H, S, D), 10 + t) for t in range(4))
    scale = 1.0 / math.sqrt(D)
    dq, dk, dv, _, _ = ref.attn_bwd(q, k, v, dout, scale, causal)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy()
            xm = x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name] = xp
            args_m[name] = xm
            fd[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], dout, scale, causal)
                       - _loss(args_m["q"], args_m["k"], args_m["v"], dout, scale, causal)) / (2 * eps)
        err = np.max(np.abs(fd - g))
        assert err <= 1e-7 * max(1.0, np.max(np.abs(fd))), (name, err)


def _torch_ref(q, k, v, dout, scale, causal):
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    o.backward(torch.tensor(dout, dtype=torch.float64))
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,S,D", [(1, 2, 16, 8), (2, 1, 33, 16), (1, 1, 64, 64)])
def test_matches_torch_float64_autograd(B, H, S, D, causal):
    q, k, v, dout = (_rand((B, H, S, D), 20 + t) for t in range(4))
    scale = 1.0 / math.sqrt(D)
    o_t, dq_t, dk_t, dv_t = _torch_ref(q, k, v, dout, scale, causal)
    o, lse = ref.attn_fwd(q, k, v, scale, causal)
    dq, dk, dv, lse2, delta = ref.attn_bwd(q, k, v, dout, scale, causal)
    np.testing.assert_allclose(o, o_t, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=0)
    for a, b in ((dq, dq_t), (dk, dk_t), (dv, dv_t)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11 * max(1.0, np.abs(b).max()))
    # log-sum-exp against its definition evaluated by numpy on the full score matrix
    s = np.einsum("bhid,bhjd->bhij", q, k) * scale
    if causal:
        s = np.where(np.tril(np.ones((S, S), bool)), s, -np.inf)
    np.testing.assert_allclose(lse, np.log(np.sum(np.exp(s), axis=-1)), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_identities(causal):
    B, H, S, D = 2, 2, 24, 8
    q, k, v, dout = (_rand((B, H, S, D), 30 + t) for t in range(4))
    scale = 1.0 / math.sqrt(D)
    o, _ = ref.attn_fwd(q, k, v, scale, causal)
    dq, dk, dv, lse, delta = ref.attn_bwd(q, k, v, dout, scale, causal)
    # sum_j dS_ij = 0 for every row  =>  the keys' dK sum to zero per head
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # sum_j P_ij = 1  =>  the values' dV sum to the queries' dO sum per head
    np.testing.assert_allclose(dv.sum(axis=2), dout.sum(axis=2), atol=1e-12)
    # D_i = sum_j P_ij dP_ij equals <dO_i, O_i>
    np.testing.assert_allclose(delta, np.sum(dout * o, axis=-1), atol=1e-12)


def test_single_key_special_case():
    # S = 1: softmax over one key is 1, so O = V, dV = dO and dQ = dK = 0.
    q, k, v, dout = (_rand((2, 3, 1, 8), 40 + t) for t in range(4))
    for causal in (False, True):
        o, lse = ref.attn_fwd(q, k, v, 0.5, causal)
        np.testing.assert_array_equal(o, v)
        np.testing.assert_allclose(lse[..., 0], 0.5 * np.sum(q * k, axis=-1)[..., 0], rtol=1e-14)
        dq, dk, dv, _, _ = ref.attn_bwd(q, k, v, dout, 0.5, causal)
        assert np.all(dq == 0) and np.all(dk == 0)
        np.testing.assert_array_equal(dv, dout)


def test_causal_first_query():
    # Under the causal mask query 0 sees only key 0: O_0 = V_0 and dQ_0 = 0.
    q, k, v, dout = (_rand((1, 2, 9, 4), 50 + t) for t in range(4))
    o, _ = ref.attn_fwd(q, k, v, 0.5, True)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    dq, _, _, _, _ = ref.attn_bwd(q, k, v, dout, 0.5, True)
    assert np.all(dq[:, :, 0] == 0)


def test_identical_keys_give_zero_dq():
    # All keys equal: every score in a row is equal, P is uniform and dQ_i = scale*k*sum_j dS_ij = 0.
    q, _, v, dout = (_rand((1, 1, 12, 8), 60 + t) for t in range(4))
    k = np.repeat(_rand((1, 1, 1, 8), 64), 12, axis=2)
    o, _ = ref.attn_fwd(q, k, v, 0.35, False)
    np.testing.assert_allclose(o[0, 0], np.repeat(v[0, 0].mean(axis=0, keepdims=True), 12, axis=0), atol=1e-14)
    dq, dk, dv, _, _ = ref.attn_bwd(q, k, v, dout, 0.35, False)
    np.testing.assert_allclose(dq, 0.0, atol=1e-14)


def test_identical_values_give_zero_dq_dk():
    # All values equal: dP_ij = <dO_i, v> = D_i for every j, so dS = 0 and dQ = dK = 0.
    q, k, _, dout = (_rand((1, 1, 10, 8), 70 + t) for t in range(4))
    v = np.repeat(_rand((1, 1, 1, 8), 74), 10, axis=2)
    for causal in (False, True):
        dq, dk, dv, _, _ = ref.attn_bwd(q, k, v, dout, 0.4, causal)
        np.testing.assert_allclose(dq, 0.0, atol=1e-13)
        np.testing.assert_allclose(dk, 0.0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_equals_full(causal):
    B, H, S, D = 1, 1, 40, 16
    q, k, v, dout = (_rand((B, H, S, D), 80 + t) for t in range(4))
    scale = 0.25
    dq, dk, dv, lse, delta = ref.attn_bwd(q, k, v, dout, scale, causal)
    rows, cols = [0, 7, 39], [0, 13, 39]
    sdq, sdk, sdv, slse, sdelta = ref.attn_bwd_sampled(q[0, 0], k[0, 0], v[0, 0], dout[0, 0], scale, causal, rows, cols)
    np.testing.assert_array_equal(sdq, dq[0, 0, rows])
    np.testing.assert_array_equal(sdk, dk[0, 0, cols])
    np.testing.assert_array_equal(sdv, dv[0, 0, cols])
    np.testing.assert_array_equal(slse, lse[0, 0])
    np.testing.assert_array_equal(sdelta, delta[0, 0])


def test_thread_count_does_not_change_bits():
    q, k, v, dout = (_rand((2, 2, 48, 16), 90 + t) for t in range(4))
    a = ref.attn_bwd(q, k, v, dout, 0.25, True, nthreads=1)
    b = ref.attn_bwd(q, k, v, dout, 0.25, True, nthreads=4)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
