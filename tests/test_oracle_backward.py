"""Pins for the oracle's QLoRA backward (CPU only).

The forward Y is linear in X, in A and in B separately, so each gradient is the
adjoint of one linear map: <dY, Y(X)> = <dX, X>, and for the LoRA part
<dY, s X A B> = <dA, A> = <dB, B>.  The forward comes from oracle.matmul, pinned
on its own, so these identities check the backward without restating it."""

import numpy as np

from oracle import backward, matmul


def _case(seed, M=7, N=11, K=13, r=3):
    g = np.random.default_rng(seed)
    return (g.standard_normal((M, N)), g.standard_normal((M, K)), g.standard_normal((N, K)),
            g.standard_normal((K, r)), g.standard_normal((r, N)))


def test_input_gradient_is_the_adjoint_of_the_forward():
    dY, X, Wd, A, B = _case(1)
    s = 2.0
    dX, _, _ = backward.qlora_backward_f64(dY, X, Wd, A, B, s)
    Y = matmul.qlora_forward_f64(X, Wd, A, B, s)
    assert np.isclose(np.sum(dY * Y), np.sum(dX * X), rtol=1e-12, atol=0)


def test_adapter_gradients_are_adjoints_of_the_lora_term():
    dY, X, Wd, A, B = _case(2)
    s = 0.75
    _, dA, dB = backward.qlora_backward_f64(dY, X, Wd, A, B, s)
    lora = matmul.qlora_forward_f64(X, np.zeros_like(Wd), A, B, s)     # s X A B
    assert np.isclose(np.sum(dY * lora), np.sum(dA * A), rtol=1e-12, atol=0)
    assert np.isclose(np.sum(dY * lora), np.sum(dB * B), rtol=1e-12, atol=0)
    assert dA.shape == A.shape and dB.shape == B.shape


def test_finite_differences():
    dY, X, Wd, A, B = _case(3, M=4, N=5, K=6, r=2)
    s = 1.5
    dX, dA, dB = backward.qlora_backward_f64(dY, X, Wd, A, B, s)
    loss = lambda X_, A_, B_: np.sum(dY * matmul.qlora_forward_f64(X_, Wd, A_, B_, s))
    h = 1e-6
    for name, P, grad in (("X", X, dX), ("A", A, dA), ("B", B, dB)):
        E = np.zeros_like(P)
        E.flat[3] = h
        args = {"X": X, "A": A, "B": B}
        up = dict(args, **{name: P + E})
        dn = dict(args, **{name: P - E})
        fd = (loss(up["X"], up["A"], up["B"]) - loss(dn["X"], dn["A"], dn["B"])) / (2 * h)
        assert np.isclose(fd, grad.flat[3], rtol=1e-6, atol=1e-9), name


def test_without_adapter_only_the_base_term():
    dY, X, Wd, _, _ = _case(4)
    dX, dA, dB = backward.qlora_backward_f64(dY, X, Wd)
    assert dA is None and dB is None
    Y = matmul.qlora_forward_f64(X, Wd)
    assert np.isclose(np.sum(dY * Y), np.sum(dX * X), rtol=1e-12, atol=0)
