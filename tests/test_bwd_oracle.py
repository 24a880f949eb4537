"""Pins for the backward-pass oracle (oracle/sage_bwd_oracle.py), each against
something other than the oracle itself.

Sources of truth: torch's float64 autograd of a plainly written attention (a
derivation by the library, not the closed form the oracle writes out), central
finite differences of the loss sum(O * dO), identities of softmax attention
(key-sum of dK is zero; key-sum of dV is the query-sum of dO; a shift of every
key leaves all gradients unchanged), scipy's logsumexp, exact scaling
properties of the INT8 emulation, and a pure-Python loop evaluation of the
emulation on tiny inputs.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle as O
from synthetic import make_custom

RNG = np.random.default_rng(4321)


def _f16(*shape, scale=1.0):
    return (RNG.standard_normal(shape) * scale).astype(np.float16)


def _torch_grads(q, k, v, do, causal, sm):
    """Gradients by torch autograd (float64, CPU) of softmax(sm Q K^T) V."""
    Q, K, V = (torch.tensor(np.asarray(x, np.float64), requires_grad=True) for x in (q, k, v))
    S = sm * Q @ K.transpose(-1, -2)
    if causal:
        n = S.shape[-1]
        S = S.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    Out = torch.softmax(S, dim=-1) @ V
    (Out * torch.tensor(np.asarray(do, np.float64))).sum().backward()
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy(), Out.detach().numpy()


# ---------------------------------------------------------------------------
# exact backward
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(37, 16), (64, 64)])
def test_exact_backward_matches_torch_autograd(causal, N, d):
    q, k, v, do = (_f16(1, 2, N, d) for _ in range(4))
    sm = 1.0 / math.sqrt(d)
    r = O.exact_attention_backward(q, k, v, do, causal=causal, sm_scale=sm)
    gq, gk, gv, out = _torch_grads(q, k, v, do, causal, sm)
    for got, want in ((r["dq"], gq), (r["dk"], gk), (r["dv"], gv), (r["o"], out)):
        assert np.abs(got - want).max() <= 1e-12 * max(1.0, np.abs(want).max())


def test_exact_backward_matches_finite_differences():
    N, d, sm = 9, 5, 0.7
    q, k, v, do = (RNG.standard_normal((1, 1, N, d)) for _ in range(4))

    def loss(q_, k_, v_):
        return float((O.exact_attention(q_, k_, v_, causal=True, sm_scale=sm) * do).sum())

    r = O.exact_attention_backward(q, k, v, do, causal=True, sm_scale=sm)
    h = 1e-6
    for name, idx in [("dq", 0), ("dk", 1), ("dv", 2)]:
        for _ in range(6):
            i, c = int(RNG.integers(N)), int(RNG.integers(d))
            args = [q.copy(), k.copy(), v.copy()]
            args[idx][0, 0, i, c] += h
            up = loss(*args)
            args[idx][0, 0, i, c] -= 2 * h
            dn = loss(*args)
            fd = (up - dn) / (2 * h)
            assert abs(fd - r[name][0, 0, i, c]) <= 1e-7 * max(1.0, abs(fd)), (name, i, c)


@pytest.mark.parametrize("causal", [False, True])
def test_exact_backward_identities(causal):
    N, d = 48, 32
    q, k, v, do = (_f16(2, 1, N, d) for _ in range(4))
    sm = 0.3
    r = O.exact_attention_backward(q, k, v, do, causal=causal, sm_scale=sm)
    # every row of dS sums to zero, so the key-sum of dK vanishes
    assert np.abs(r["dk"].sum(axis=2)).max() <= 1e-12 * np.abs(r["dk"]).max() * N
    # every row of P sums to one, so the key-sum of dV is the query-sum of dO
    assert np.abs(r["dv"].sum(axis=2) - do.astype(np.float64).sum(axis=2)).max() <= 1e-11
    # adding one vector to every key shifts each score row by a constant
    shift = RNG.standard_normal((2, 1, 1, d))
    r2 = O.exact_attention_backward(q, k.astype(np.float64) + shift, v, do, causal=causal, sm_scale=sm)
    for g in ("dq", "dk", "dv"):
        assert np.abs(r2[g] - r[g]).max() <= 1e-10 * max(1.0, np.abs(r[g]).max())
    # the log-sum-exp of the scaled scores (a library routine)
    S = sm * q[0, 0].astype(np.float64) @ k[0, 0].astype(np.float64).T
    if causal:
        S[np.triu(np.ones((N, N), bool), 1)] = -np.inf
    assert np.abs(r["lse"][0, 0] - logsumexp(S, axis=1)).max() <= 1e-12


def test_exact_backward_single_key():
    q, k, v, do = (_f16(1, 1, 1, 8) for _ in range(4))
    r = O.exact_attention_backward(q, k, v, do, causal=False, sm_scale=1.0)
    assert np.array_equal(r["dv"], do.astype(np.float64))
    assert np.abs(r["dq"]).max() == 0.0 and np.abs(r["dk"]).max() == 0.0


# ---------------------------------------------------------------------------
# forward for training: the saved log-sum-exp
# ---------------------------------------------------------------------------

def test_training_forward_lse_on_exactly_representable_codes():
    """With Q and K whose per-block codes are exact (every block holds an
    element of magnitude 127 and integers only, K column means zero) and
    smoothing off, the INT8 forward's scores are the exact scores, so its
    saved log-sum-exp is the exact one up to the fp16 rounding of P that l
    sums (R6): |dL| <= 2^-11 per row."""
    N, d = 200, 64
    qi = RNG.integers(-127, 128, size=(1, 1, N, d)).astype(np.float64)
    ki = RNG.integers(-60, 61, size=(1, 1, N // 2, d)).astype(np.float64)
    ki = np.concatenate([ki, -ki], axis=2)                       # column means exactly zero
    qi[..., ::64, 0] = 127.0                                     # every 128-block and 64-block has max 127
    ki[..., ::64, 0] = 127.0
    ki[..., 32::64, 0] = -127.0
    sm = 1.0 / 4096.0
    q16, k16 = (qi.astype(np.float16), ki.astype(np.float16))
    v16 = _f16(1, 1, N, d)
    fw = O.int8_forward_for_training(q16, k16, v16, causal=True, sm_scale=sm, smooth=False)
    S = sm * qi[0, 0] @ ki[0, 0].T
    S[np.triu(np.ones((N, N), bool), 1)] = -np.inf
    assert np.abs(fw["lse"][0, 0] - logsumexp(S, axis=1)).max() <= 2.0 ** -11


# ---------------------------------------------------------------------------
# INT8 emulation
# ---------------------------------------------------------------------------

def _emulate(q, k, v, do, causal, sm, **kw):
    fw = O.int8_forward_for_training(q, k, v, causal=causal, sm_scale=sm)
    return O.int8_attention_backward(q, k, v, do, fw["o16"], fw["lse"], causal=causal, sm_scale=sm, **kw), fw


def _loop_backward(q16, k16, v16, do16, o16, lse, causal, sm, blk_q=128, blk_k=64):
    """The emulated backward evaluated with Python loops over (query, key) pairs:
    explicit 32x32 tile maxima, round() (ties to even) for every code, integer
    dot products, one scaled partial per tile. The token-block quantizers of Q,
    K_s, V and dO are the forward oracle's (pinned in test_oracle.py)."""
    N, d = q16.shape[2], q16.shape[3]
    qd = O.quant_qk_int8(q16, k16, blk_q=blk_q, blk_k=blk_k, smooth=True)
    vc, vs = O.int8_quant_blocks(v16.astype(np.float32), 1)
    gc, gs = O.int8_quant_blocks(do16.astype(np.float32), 64)
    Qc, Kc = qd["q_codes"][0, 0].astype(int).tolist(), qd["k_codes"][0, 0].astype(int).tolist()
    Vc, Gc = vc[0, 0].astype(int).tolist(), gc[0, 0].astype(int).tolist()
    qs, ks = qd["q_scales"][0, 0].tolist(), qd["k_scales"][0, 0].tolist()
    vsl, gsl = vs[0, 0].tolist(), gs[0, 0].tolist()
    G16, O16 = do16[0, 0].astype(float).tolist(), o16[0, 0].astype(float).tolist()
    Ls = lse[0, 0].tolist()
    P = [[0.0] * N for _ in range(N)]
    dS = [[0.0] * N for _ in range(N)]
    for i in range(N):
        Di = sum(G16[i][c] * O16[i][c] for c in range(d))
        for j in range(N):
            if causal and j > i:
                continue
            s_int = sum(Qc[i][c] * Kc[j][c] for c in range(d))
            p = math.exp(s_int * qs[i // blk_q] * ks[j // blk_k] * sm - Ls[i])
            dp = sum(Gc[i][c] * Vc[j][c] for c in range(d)) * gsl[i // 64] * vsl[j]
            P[i][j] = p
            dS[i][j] = p * (dp - Di)

    def tile_codes(X):
        C = [[0] * N for _ in range(N)]
        scl = {}
        for ti in range(0, N, 32):
            for tj in range(0, N, 32):
                a = max(abs(X[i][j]) for i in range(ti, min(ti + 32, N)) for j in range(tj, min(tj + 32, N)))
                s = float(np.float32(np.float32(a) / np.float32(127.0)))
                scl[ti // 32, tj // 32] = s
                for i in range(ti, min(ti + 32, N)):
                    for j in range(tj, min(tj + 32, N)):
                        C[i][j] = 0 if s == 0 else max(-127, min(127, round(X[i][j] / s)))
        return C, scl

    Pc, Ps = tile_codes(P)
    Sc, Ss = tile_codes(dS)
    dq = np.zeros((N, d)); dk = np.zeros((N, d)); dv = np.zeros((N, d))
    for ti in range(0, N, 32):
        for tj in range(0, N, 32):
            I = range(ti, min(ti + 32, N)); J = range(tj, min(tj + 32, N))
            for c in range(d):
                for i in I:      # dQ: contraction over the tile's keys
                    acc = sum(Sc[i][j] * Kc[j][c] for j in J)
                    dq[i, c] += sm * Ss[ti // 32, tj // 32] * ks[tj // blk_k] * acc
                for j in J:      # dK, dV: contraction over the tile's queries
                    acc_k = sum(Sc[i][j] * Qc[i][c] for i in I)
                    dk[j, c] += sm * Ss[ti // 32, tj // 32] * qs[ti // blk_q] * acc_k
                    acc_v = sum(Pc[i][j] * Gc[i][c] for i in I)
                    dv[j, c] += Ps[ti // 32, tj // 32] * gsl[ti // 64] * acc_v
    return dq, dk, dv


@pytest.mark.parametrize("causal", [False, True])
def test_int8_backward_matches_python_loops(causal):
    N, d = 70, 8                                     # three 32-tiles, the last ragged
    q, k, v = make_custom(1, 1, N, d, seed=11)
    do = _f16(1, 1, N, d)
    sm = 0.35
    r, fw = _emulate(q, k, v, do, causal, sm)
    dq, dk, dv = _loop_backward(q, k, v, do, fw["o16"], fw["lse"], causal, sm)
    for got, want in ((r["dq"][0, 0], dq), (r["dk"][0, 0], dk), (r["dv"][0, 0], dv)):
        assert np.abs(got - want).max() <= 1e-12 * max(1.0, np.abs(want).max())


def test_int8_backward_zero_and_power_of_two_gradients():
    N, d = 96, 32
    q, k, v = make_custom(1, 2, N, d, seed=12)
    do = _f16(1, 2, N, d)
    sm = 1.0 / math.sqrt(d)
    fw = O.int8_forward_for_training(q, k, v, causal=False, sm_scale=sm)
    args = dict(causal=False, sm_scale=sm)
    r = O.int8_attention_backward(q, k, v, do, fw["o16"], fw["lse"], **args)
    z = O.int8_attention_backward(q, k, v, np.zeros_like(do), fw["o16"], fw["lse"], **args)
    assert all(np.abs(z[g]).max() == 0.0 for g in ("dq", "dk", "dv"))
    # doubling dO doubles every scale (codes unchanged) and D: gradients double exactly
    r2 = O.int8_attention_backward(q, k, v, (do.astype(np.float32) * 2).astype(np.float16), fw["o16"],
                                   fw["lse"], **args)
    for g in ("dq", "dk", "dv"):
        assert np.array_equal(r2[g], 2.0 * r[g])


@pytest.mark.parametrize("causal,dist,bar", [(False, "normal", 0.999), (True, "normal", 0.999),
                                             (True, "student_t", 0.98)])
def test_int8_backward_tracks_exact_gradients(causal, dist, bar):
    """The emulated gradients follow the exact ones (a wrong sign, index or
    operand order anywhere would break this): cosine similarity >= 0.999 on
    unit-variance inputs; on heavy-tailed (Student-t) inputs at d = 64 the
    per-block Q and K codes of the scores cost more (dQ about 0.987)."""
    N, d = 256, 64
    q, k, v = make_custom(1, 2, N, d, seed=13, dist=dist)
    do = _f16(1, 2, N, d)
    sm = 1.0 / math.sqrt(d)
    r, _ = _emulate(q, k, v, do, causal, sm)
    ex = O.exact_attention_backward(q, k, v, do, causal=causal, sm_scale=sm)
    for g in ("dq", "dk", "dv"):
        a, b = r[g].ravel(), ex[g].ravel()
        assert a @ b / np.linalg.norm(a) / np.linalg.norm(b) >= bar, g


def test_int8_backward_allowance_is_small():
    N, d = 128, 64
    q, k, v = make_custom(1, 1, N, d, seed=14)
    do = _f16(1, 1, N, d)
    r, _ = _emulate(q, k, v, do, False, 0.125, with_allowance=True)
    assert r["p_flips"] + r["ds_flips"] < 0.01 * N * N
    for g in ("dq", "dk", "dv"):
        assert np.all(r[g + "_allow"] <= 0.05 * r[g + "_mag"] + 1e-30)
