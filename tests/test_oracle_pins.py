"""Pins of the fp64 oracle against things other than itself.

Each test ties the oracle to a library routine, a closed form, an invariant of
the definitions, or finite differences, so that a dropped term, a wrong sign,
a wrong pair index, a wrong frequency exponent or a transposed operand fails at
least one of them.  The definitions pinned are those of the oracle's header:
per-head RMSNorm as static weight times an inverse-RMS scalar ("QK-Normed MLA:
QK normalization without full key caching", abstract), then RoPE ("Rope to Nope
and Back Again", abstract) on the first rotary_dim channels ("Fractional
Rotation, Full Potential? Investigating Performance and Convergence of Partial
RoPE", abstract).
"""

import math
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _case(seed, T, hq, hkv, D, scale=1.0, max_pos=64, wscale=0.1):
    g = np.random.default_rng(seed)
    return dict(
        q=scale * g.standard_normal((T, hq, D)),
        k=scale * g.standard_normal((T, hkv, D)),
        wq=1.0 + wscale * g.standard_normal(D),
        wk=1.0 + wscale * g.standard_normal(D),
        pos=g.integers(0, max_pos, size=T).astype(np.int32),
        dyq=g.standard_normal((T, hq, D)),
        dyk=g.standard_normal((T, hkv, D)),
    )


def _fwd(o, c, R, eps, theta):
    return o.fwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], R, eps, theta)


# --- norm: library routine -------------------------------------------------

@pytest.mark.parametrize("D", [8, 64, 128])
def test_norm_matches_torch_rms_norm(oracle_mod, D):
    """rotary_dim = 0 reduces to RMSNorm with weight; torch's fp64 rms_norm is the
    library routine.  A large eps (0.25) and small values make eps placement and
    the 1/D mean visible."""
    c = _case(1, 5, 3, 2, D, scale=0.4)
    eps = 0.25
    yq, yk = _fwd(oracle_mod, c, 0, eps, 1e4)
    for x, w, y in ((c["q"], c["wq"], yq), (c["k"], c["wk"], yk)):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (D,), torch.from_numpy(w), eps)
        np.testing.assert_allclose(y, ref.numpy(), rtol=1e-13, atol=1e-14)


# --- RoPE: library routines (transformers) ---------------------------------

def _hf_rope(x, pos, R, theta, D):
    """Reference RoPE via transformers' Phi rotary embedding (partial rotary
    factor R/D, frequency denominator R) and apply_rotary_pos_emb (rotate-half
    pairing).  Those compute angles in fp32, hence the loose tolerance."""
    from transformers import PhiConfig
    from transformers.models.phi import modeling_phi as mp

    cfg = PhiConfig(hidden_size=D * 2, num_attention_heads=2,
                    rope_parameters={"rope_type": "default", "rope_theta": float(theta),
                                     "partial_rotary_factor": R / D})
    emb = mp.PhiRotaryEmbedding(cfg)
    xt = torch.from_numpy(x)                        # [T, H, D] fp64
    cos, sin = emb(xt, torch.from_numpy(pos.astype(np.int64))[None, :])  # [1, T, R]
    cos, sin = cos[0].double(), sin[0].double()     # [T, R]
    xr = xt[..., :R].transpose(0, 1)[None]          # [1, H, T, R]
    yr, _ = mp.apply_rotary_pos_emb(xr, xr, cos[None], sin[None], unsqueeze_dim=1)
    y = torch.cat([yr[0].transpose(0, 1), xt[..., R:]], dim=-1)
    return y.numpy()


@pytest.mark.parametrize("D,R,theta", [(64, 64, 1e4), (128, 128, 5e5), (128, 32, 1e6),
                                       (64, 16, 1e6), (16, 8, 10.0)])
def test_rope_matches_transformers(oracle_mod, D, R, theta):
    """Pins pairing (i, i+R/2), rotation sense, frequency theta^(-2i/R) with
    denominator R, and which channels rotate, against transformers' RoPE."""
    c = _case(2, 6, 3, 2, D, max_pos=48)
    c["wq"] = np.ones(D)
    c["wk"] = np.ones(D)
    eps = 0.0 + 1e-30
    yq, yk = _fwd(oracle_mod, c, R, eps, theta)
    nq, nk = _fwd(oracle_mod, c, 0, eps, theta)     # normalised, unrotated
    for n, y in ((nq, yq), (nk, yk)):
        ref = _hf_rope(n, c["pos"], R, theta, D)
        # fp32 angles at positions < 48: |error| <~ 48 * 2^-24 rad per unit norm
        np.testing.assert_allclose(y, ref, rtol=0, atol=2e-5 * np.abs(n).max())


# --- cos/sin definition -----------------------------------------------------

def test_cos_sin_are_fp32_roundings_of_exact_values(oracle_mod):
    """c_i, s_i are cos/sin of pos*theta^(-2i/R) rounded to fp32.  mpmath
    evaluates them at 40 digits; the oracle's fp64 angle carries two roundings,
    so a value may land on the other side of an fp32 rounding boundary only
    rarely: allow at most one fp32 ulp and require >= 99% exact."""
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 40
    exact = total = 0
    for pos, theta, R in [(1, 1e4, 64), (127, 1e4, 64), (4095, 1e6, 64), (8191, 5e5, 128),
                          (131071, 1e6, 32), (0, 1e6, 16)]:
        c, s = oracle_mod.rope_cos_sin(pos, theta, R)
        for i in range(R // 2):
            th = mpmath.power(mpmath.mpf(theta), mpmath.mpf(-2 * i) / R)
            phi = pos * th
            for got, ref in ((c[i], mpmath.cos(phi)), (s[i], mpmath.sin(phi))):
                r32 = np.float32(float(ref))
                g32 = np.float32(got)
                assert float(g32) == got  # the oracle's value is an fp32 value
                d = abs(int(g32.view(np.int32)) - int(r32.view(np.int32)))
                assert d <= 1, (pos, theta, R, i, got, float(ref))
                exact += d == 0
                total += 1
    assert exact >= 0.99 * total


# --- RoPE invariants ---------------------------------------------------------

def test_position_zero_is_identity(oracle_mod):
    """pos = 0 gives c = 1, s = 0 exactly, so the output is the normalised vector
    bit for bit."""
    c = _case(3, 4, 3, 2, 64)
    c["pos"][:] = 0
    y = _fwd(oracle_mod, c, 64, 1e-6, 1e6)
    n = _fwd(oracle_mod, c, 0, 1e-6, 1e6)
    for a, b in zip(y, n):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("D,R", [(64, 64), (128, 32), (128, 128)])
def test_rotation_preserves_pair_norms(oracle_mod, D, R):
    """Each rotated pair (i, i+R/2) keeps its norm up to c^2+s^2 (fp32-rounded
    c, s), and unrotated channels are untouched."""
    c = _case(4, 7, 3, 1, D, max_pos=100000)
    y, _ = _fwd(oracle_mod, c, R, 1e-6, 1e6)
    n, _ = _fwd(oracle_mod, c, 0, 1e-6, 1e6)
    h = R // 2
    for t in range(c["q"].shape[0]):
        cc, ss = oracle_mod.rope_cos_sin(int(c["pos"][t]), 1e6, R)
        assert np.all(np.abs(cc * cc + ss * ss - 1.0) <= 2.0 ** -22)
        ny = y[t, :, :h] ** 2 + y[t, :, h:R] ** 2
        nn = (cc * cc + ss * ss) * (n[t, :, :h] ** 2 + n[t, :, h:R] ** 2)
        np.testing.assert_allclose(ny, nn, rtol=1e-12)
        assert np.array_equal(y[t, :, R:], n[t, :, R:])


@pytest.mark.parametrize("D,R,theta", [(64, 64, 1e4), (128, 32, 1e6), (128, 128, 5e5)])
def test_scores_depend_only_on_relative_position(oracle_mod, D, R, theta):
    """<y_q(m), y_k(n)> is the trigonometric series in (m - n) of the TriAttention
    abstract (Daily Papers "QK-RoPE" search page):
      sum_i (a a' + b b') cos((m-n) t_i) + (a b' - b a') sin((m-n) t_i) + sum_{j>=R} n_j n'_j
    and it is unchanged when both positions shift.  Equal only up to the fp32
    rounding of c, s (floating-point RoPE is not bit-exactly shift invariant)."""
    g = np.random.default_rng(5)
    x = g.standard_normal((1, 1, D))
    kx = g.standard_normal((1, 1, D))
    w = np.ones(D)
    h = R // 2
    nq = oracle_mod.fwd(x, kx, w, w, np.zeros(1, np.int32), 0, 1e-6, theta)[0][0, 0]
    nk = oracle_mod.fwd(kx, x, w, w, np.zeros(1, np.int32), 0, 1e-6, theta)[0][0, 0]
    tol = 1e-6 * np.linalg.norm(nq) * np.linalg.norm(nk)
    for m, n in [(5, 3), (100, 0), (4000, 3999), (77, 1234)]:
        vals = []
        for delta in (0, 1, 1000, 50000):
            pos = np.array([m + delta], np.int32)
            yq = oracle_mod.fwd(x, kx, w, w, pos, R, 1e-6, theta)[0][0, 0]
            pos = np.array([n + delta], np.int32)
            yk = oracle_mod.fwd(kx, x, w, w, pos, R, 1e-6, theta)[0][0, 0]
            vals.append(float(yq @ yk))
        th = theta ** (-2.0 * np.arange(h) / R)
        dlt = (m - n) * th
        a, b, a2, b2 = nq[:h], nq[h:R], nk[:h], nk[h:R]
        series = np.sum((a * a2 + b * b2) * np.cos(dlt) + (a * b2 - b * a2) * np.sin(dlt))
        series += float(nq[R:] @ nk[R:])
        for v in vals:
            assert abs(v - series) <= tol, (m, n, vals, series)


def test_two_channel_case_is_complex_multiplication(oracle_mod):
    """D = R = 2: theta_0 = 1 for every theta, so the output is the normalised
    pair, as a complex number, times exp(i*pos) (with fp32-rounded parts)."""
    import cmath
    g = np.random.default_rng(6)
    q = g.standard_normal((5, 1, 2))
    pos = np.array([0, 1, 7, 4096, 131071], np.int32)
    w = np.array([1.3, 0.7])
    for theta in (1e4, 5e5):
        y = oracle_mod.fwd(q, q, w, w, pos, 2, 1e-6, theta)[0]
        n = oracle_mod.fwd(q, q, w, w, pos, 0, 1e-6, theta)[0]
        for t in range(5):
            e = cmath.exp(1j * float(pos[t]))
            e = complex(float(np.float32(e.real)), float(np.float32(e.imag)))
            z = complex(n[t, 0, 0], n[t, 0, 1]) * e
            assert abs(z - complex(y[t, 0, 0], y[t, 0, 1])) < 1e-15


# --- norm invariants -----------------------------------------------------------

@pytest.mark.parametrize("R", [0, 32, 64])
def test_unit_weight_rms(oracle_mod, R):
    """With w = 1, RMS over all D channels of the output is sqrt(ms/(ms+eps)),
    rotated or not (the mean runs over all D channels, eps inside the root)."""
    c = _case(7, 6, 4, 2, 64, scale=0.3)
    c["wq"] = np.ones(64)
    c["wk"] = np.ones(64)
    eps = 0.0625
    yq, yk = _fwd(oracle_mod, c, R, eps, 1e4)
    for x, y in ((c["q"], yq), (c["k"], yk)):
        ms = np.mean(x * x, axis=-1)
        rms = np.sqrt(np.mean(y * y, axis=-1))
        np.testing.assert_allclose(rms, np.sqrt(ms / (ms + eps)), rtol=3e-7)


def test_scale_law(oracle_mod):
    """y(a*x; eps) = y(x; eps/a^2) exactly in exact arithmetic; with a = 2 and
    eps = 0.25 every input is exact, so fp64 agrees to rounding."""
    c = _case(8, 5, 3, 2, 64, scale=0.5)
    y1 = oracle_mod.fwd(2 * c["q"], 2 * c["k"], c["wq"], c["wk"], c["pos"], 64, 0.25, 1e4)
    y2 = oracle_mod.fwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], 64, 0.0625, 1e4)
    for a, b in zip(y1, y2):
        np.testing.assert_allclose(a, b, rtol=1e-14, atol=1e-15)


def test_weight_is_per_channel_and_shared_across_heads(oracle_mod):
    """A one-hot weight at channel j (pos 0) leaves only channel j non-zero in
    every head; Q uses wq and K uses wk."""
    c = _case(9, 3, 3, 2, 16)
    c["pos"][:] = 0
    c["wq"] = np.zeros(16)
    c["wq"][5] = 1.0
    c["wk"] = np.zeros(16)
    c["wk"][11] = 2.0
    yq, yk = _fwd(oracle_mod, c, 16, 1e-6, 1e4)
    assert np.count_nonzero(np.delete(yq, 5, axis=-1)) == 0
    assert np.count_nonzero(np.delete(yk, 11, axis=-1)) == 0
    assert np.all(yq[..., 5] != 0) and np.all(yk[..., 11] != 0)


# --- layout invariants -------------------------------------------------------

def test_permutations_commute(oracle_mod):
    """Permuting tokens together with their positions, or heads, permutes the
    outputs (and backward outputs) the same way; dw is unchanged."""
    c = _case(10, 9, 4, 2, 32, max_pos=1000)
    a = oracle_mod.bwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], c["dyq"], c["dyk"], 32, 1e-6, 1e4)
    ya = _fwd(oracle_mod, c, 32, 1e-6, 1e4)
    p = np.random.default_rng(0).permutation(9)
    hp = np.array([2, 0, 3, 1])
    cp = {kk: (v[p] if v.ndim >= 1 and v.shape[0] == 9 else v) for kk, v in c.items()}
    cp["q"] = cp["q"][:, hp]
    cp["dyq"] = cp["dyq"][:, hp]
    yb = _fwd(oracle_mod, cp, 32, 1e-6, 1e4)
    b = oracle_mod.bwd(cp["q"], cp["k"], cp["wq"], cp["wk"], cp["pos"], cp["dyq"], cp["dyk"], 32, 1e-6, 1e4)
    assert np.array_equal(yb[0], ya[0][p][:, hp])
    assert np.array_equal(yb[1], ya[1][p])
    assert np.array_equal(b[0], a[0][p][:, hp])
    assert np.array_equal(b[1], a[1][p])
    np.testing.assert_allclose(b[2], a[2], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(b[3], a[3], rtol=1e-13, atol=1e-13)


def test_packed_documents_equal_documents_alone(oracle_mod):
    """Position ids restarting per packed document (Chronicals abstract,
    contribution (4): BFD packing): each document's rows in the packed buffer
    equal the document run alone; dw of the buffer is the sum over documents."""
    lens = [5, 9, 3, 7]
    T = sum(lens)
    g = np.random.default_rng(11)
    q = g.standard_normal((T, 2, 32))
    k = g.standard_normal((T, 1, 32))
    dyq = g.standard_normal((T, 2, 32))
    dyk = g.standard_normal((T, 1, 32))
    w1, w2 = 1 + 0.1 * g.standard_normal(32), 1 + 0.1 * g.standard_normal(32)
    pos = np.concatenate([np.arange(L) for L in lens]).astype(np.int32)
    yq, yk = oracle_mod.fwd(q, k, w1, w2, pos, 32, 1e-6, 1e6)
    _, _, dwq, dwk = oracle_mod.bwd(q, k, w1, w2, pos, dyq, dyk, 32, 1e-6, 1e6)
    sq = np.zeros(32)
    sk = np.zeros(32)
    a = 0
    for L in lens:
        sl = slice(a, a + L)
        p = np.arange(L, dtype=np.int32)
        dq_, dk_ = oracle_mod.fwd(q[sl], k[sl], w1, w2, p, 32, 1e-6, 1e6)
        assert np.array_equal(dq_, yq[sl]) and np.array_equal(dk_, yk[sl])
        r = oracle_mod.bwd(q[sl], k[sl], w1, w2, p, dyq[sl], dyk[sl], 32, 1e-6, 1e6)
        sq += r[2]
        sk += r[3]
        a += L
    np.testing.assert_allclose(dwq, sq, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dwk, sk, rtol=1e-13, atol=1e-13)


# --- backward -----------------------------------------------------------------

def _loss(o, q, k, wq, wk, pos, dyq, dyk, R, eps, theta):
    yq, yk = o.fwd(q, k, wq, wk, pos, R, eps, theta)
    return float(np.sum(dyq * yq) + np.sum(dyk * yk))


@pytest.mark.parametrize("R", [0, 4, 8])
def test_backward_finite_differences(oracle_mod, R):
    """Central differences of L = <dy, y> in fp64 (T=3, H=2, D=8, eps=1e-3,
    step 1e-6) agree with dx and dw to ~1e-7 relative."""
    o = oracle_mod
    g = np.random.default_rng(12 + R)
    T, H, D = 3, 2, 8
    q = g.standard_normal((T, H, D))
    k = g.standard_normal((T, 1, D))
    wq = 1 + 0.3 * g.standard_normal(D)
    wk = 1 + 0.3 * g.standard_normal(D)
    pos = np.array([0, 5, 23], np.int32)
    dyq = g.standard_normal((T, H, D))
    dyk = g.standard_normal((T, 1, D))
    eps = 2.0 ** -10   # exactly representable in fp32
    args = (pos, dyq, dyk, R, eps, 1e4)
    dq, dk, dwq, dwk = o.bwd(q, k, wq, wk, pos, dyq, dyk, R, eps, 1e4)
    hstep = 1e-6

    def fd(arr, setter):
        out = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p = arr.copy()
            p[idx] += hstep
            m = arr.copy()
            m[idx] -= hstep
            out[idx] = (_loss(o, *setter(p), *args) - _loss(o, *setter(m), *args)) / (2 * hstep)
        return out

    nq = fd(q, lambda v: (v, k, wq, wk))
    nk = fd(k, lambda v: (q, v, wq, wk))
    nwq = fd(wq, lambda v: (q, k, v, wk))
    nwk = fd(wk, lambda v: (q, k, wq, v))
    for got, ref in ((dq, nq), (dk, nk), (dwq, nwq), (dwk, nwk)):
        np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-7 * np.abs(ref).max())
        assert np.abs(got).max() > 1e-3     # non-zero gradients


def test_backward_adjoint(oracle_mod):
    """<dy, J v> = <J^T dy, v> with J v from a central difference along v."""
    o = oracle_mod
    g = np.random.default_rng(20)
    T, H, D, R = 4, 3, 16, 8
    q = g.standard_normal((T, H, D))
    k = g.standard_normal((T, 1, D))
    wq = 1 + 0.1 * g.standard_normal(D)
    wk = 1 + 0.1 * g.standard_normal(D)
    pos = g.integers(0, 500, T).astype(np.int32)
    dyq = g.standard_normal((T, H, D))
    dyk = g.standard_normal((T, 1, D))
    vq = g.standard_normal((T, H, D))
    dq, _, _, _ = o.bwd(q, k, wq, wk, pos, dyq, dyk, R, 1e-3, 1e4)
    hs = 1e-6
    yp = o.fwd(q + hs * vq, k, wq, wk, pos, R, 1e-3, 1e4)[0]
    ym = o.fwd(q - hs * vq, k, wq, wk, pos, R, 1e-3, 1e4)[0]
    jv = (yp - ym) / (2 * hs)
    lhs = float(np.sum(dyq * jv))
    rhs = float(np.sum(dq * vq))
    assert abs(lhs - rhs) <= 1e-7 * abs(rhs) + 1e-9


@pytest.mark.parametrize("eps", [0.0, 0.01])
def test_backward_radial_closed_form(oracle_mod, eps):
    """Per row, sum_j x_j dx_j = eps r^3 sum_j u_j x_j with u = w * (R^T dy):
    the gradient is orthogonal to x when eps = 0 (scale invariance)."""
    o = oracle_mod
    g = np.random.default_rng(21)
    T, H, D, R = 5, 2, 32, 32
    q = g.standard_normal((T, H, D))
    k = g.standard_normal((T, 1, D))
    wq = 1 + 0.1 * g.standard_normal(D)
    pos = g.integers(0, 100, T).astype(np.int32)
    dyq = g.standard_normal((T, H, D))
    dyk = g.standard_normal((T, 1, D))
    e = eps if eps > 0 else 1e-38   # smallest positive normal-ish fp32, effectively 0
    dq, _, _, _ = o.bwd(q, k, wq, wq, pos, dyq, dyk, R, e, 1e4)
    for t in range(T):
        for hh in range(H):
            x = q[t, hh]
            r = 1.0 / math.sqrt(np.mean(x * x) + float(np.float32(e)))
            cc, ss = o.rope_cos_sin(int(pos[t]), 1e4, R)
            dy = dyq[t, hh]
            h = R // 2
            gg = dy.copy()
            gg[:h] = dy[:h] * cc + dy[h:R] * ss
            gg[h:R] = dy[h:R] * cc - dy[:h] * ss
            u = wq * gg
            lhs = float(x @ dq[t, hh])
            rhs = float(np.float32(e)) * r ** 3 * float(u @ x)
            assert abs(lhs - rhs) <= 1e-12 * (np.abs(x).max() * np.abs(dq[t, hh]).max() * D)


def test_rope_backward_inverts_forward(oracle_mod):
    """With w = 1 and r ~ 1 (eps -> 0, unit-RMS rows) the RoPE part of the
    backward is the inverse rotation: feeding y back as dy through the
    transpose recovers n up to c^2 + s^2 - 1 (cf. stripping RoPE from keys in
    the cross-model KV transfer abstract of the "byte crossover" search page)."""
    o = oracle_mod
    g = np.random.default_rng(22)
    T, D, R = 6, 64, 64
    x = g.standard_normal((T, 1, D))
    x /= np.sqrt(np.mean(x * x, axis=-1, keepdims=True))   # unit RMS rows: r = 1
    w = np.ones(D)
    pos = g.integers(0, 10000, T).astype(np.int32)
    y = o.fwd(x, x, w, w, pos, R, 1e-30, 1e4)[0]
    for t in range(T):
        cc, ss = o.rope_cos_sin(int(pos[t]), 1e4, R)
        h = R // 2
        dy = y[t, 0]
        gg = np.empty(D)
        gg[:h] = dy[:h] * cc + dy[h:] * ss
        gg[h:] = dy[h:] * cc - dy[:h] * ss
        np.testing.assert_allclose(gg, x[t, 0], atol=1e-6)


# --- bf16 rounding -------------------------------------------------------------

def test_round_bf16_matches_torch_on_fp32_values(oracle_mod):
    """On fp32 inputs one-step rounding equals torch's fp32 -> bf16 cast (round
    to nearest even): random bit patterns plus ties, zeros, subnormals,
    infinities and the largest finite values."""
    g = np.random.default_rng(23)
    bits = g.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0x00000000, 0x80000000, 0x00000001, 0x00008000, 0x00018000,
                        0x3F808000, 0x3F818000, 0x3F80FFFF, 0x7F7FFFFF, 0x7F7F7FFF,
                        0x7F7F8000, 0xFF7F8000, 0x7F800000, 0xFF800000, 0x007FFFFF,
                        0x00800000, 0x3F800000], np.uint32)
    bits = np.concatenate([special, bits])
    f = bits.view(np.float32)
    f = f[~np.isnan(f)]
    got = oracle_mod.round_bf16(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_round_bf16_golden_cases(oracle_mod):
    """Hand-derived cases (tests/golden/bf16_rne_cases.txt), including fp64
    values where rounding through fp32 first would give a different bf16 value."""
    vals, want = [], []
    with open(os.path.join(GOLDEN, "bf16_rne_cases.txt")) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if not line:
                continue
            v, b = line.split()
            vals.append(float.fromhex(v) if "p" in v else float(v))
            want.append(int(b, 16))
    got = oracle_mod.round_bf16(np.array(vals))
    assert [hex(x) for x in got] == [hex(x) for x in want]


# --- convention variants: interleaved pairing, frequency denominator D, no weight

def _gptj_rope(x, pos, R, freq_dim):
    """Interleaved-pair RoPE via transformers' GPT-J helpers: frequencies from
    create_sinusoidal_positions(., freq_dim) (base 10^4, fp32), the first R/2 of
    them applied by apply_rotary_pos_emb / rotate_every_two to channels < R."""
    from transformers.models.gptj import modeling_gptj as mg

    table = mg.create_sinusoidal_positions(int(pos.max()) + 1, freq_dim).double()
    half = freq_dim // 2
    sc = table[torch.from_numpy(pos.astype(np.int64))]         # [T, freq_dim]
    sin, cos = sc[:, : R // 2], sc[:, half: half + R // 2]      # [T, R/2]
    xt = torch.from_numpy(x)[None]                              # [1, T, H, D]
    yr = mg.apply_rotary_pos_emb(xt[..., :R], sin[None], cos[None])
    return torch.cat([yr, xt[..., R:]], dim=-1)[0].numpy()


def _hf_rope_freq_dim(x, pos, R, theta, D):
    """Half-split RoPE with frequencies over the whole head: transformers' Phi
    rotary embedding with partial factor 1 gives theta^(-2i/D); its first R/2
    frequencies drive apply_rotary_pos_emb on channels < R."""
    from transformers import PhiConfig
    from transformers.models.phi import modeling_phi as mp

    cfg = PhiConfig(hidden_size=D * 2, num_attention_heads=2,
                    rope_parameters={"rope_type": "default", "rope_theta": float(theta),
                                     "partial_rotary_factor": 1.0})
    emb = mp.PhiRotaryEmbedding(cfg)
    xt = torch.from_numpy(x)
    cos, sin = emb(xt, torch.from_numpy(pos.astype(np.int64))[None, :])  # [1, T, D]
    h = R // 2
    cos = torch.cat([cos[0, :, :h], cos[0, :, :h]], -1).double()
    sin = torch.cat([sin[0, :, :h], sin[0, :, :h]], -1).double()
    xr = xt[..., :R].transpose(0, 1)[None]
    yr, _ = mp.apply_rotary_pos_emb(xr, xr, cos[None], sin[None], unsqueeze_dim=1)
    return torch.cat([yr[0].transpose(0, 1), xt[..., R:]], dim=-1).numpy()


def _unit_case(seed, D, T=6):
    c = _case(seed, T, 3, 2, D, max_pos=48)
    c["wq"] = np.ones(D)
    c["wk"] = np.ones(D)
    return c


@pytest.mark.parametrize("D,R", [(64, 64), (128, 64), (64, 16), (16, 8)])
def test_interleaved_matches_transformers_gptj(oracle_mod, D, R):
    """Interleaved pairs (2i, 2i+1), rotation sense and the frequency
    denominator R against GPT-J's RoPE (fixed base 10^4)."""
    o = oracle_mod
    c = _unit_case(30, D)
    flags = o.flags_of(interleaved=True)
    yq, yk = o.fwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], R, 1e-30, 1e4, flags=flags)
    nq, nk = _fwd(o, c, 0, 1e-30, 1e4)
    for n, y in ((nq, yq), (nk, yk)):
        ref = _gptj_rope(n, c["pos"], R, R)
        np.testing.assert_allclose(y, ref, rtol=0, atol=2e-5 * np.abs(n).max())


@pytest.mark.parametrize("D,R", [(128, 64), (64, 32), (64, 16)])
def test_freq_head_dim_matches_transformers(oracle_mod, D, R):
    """Frequencies theta^(-2i/D) on a partial rotation, both pairings, against
    the library frequency generators called with the head width."""
    o = oracle_mod
    c = _unit_case(31, D)
    nq, _ = _fwd(o, c, 0, 1e-30, 1e4)
    yq_h = o.fwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], R, 1e-30, 1e4,
                 flags=o.flags_of(freq_head_dim=True))[0]
    yq_i = o.fwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], R, 1e-30, 1e4,
                 flags=o.flags_of(interleaved=True, freq_head_dim=True))[0]
    tol = 2e-5 * np.abs(nq).max()
    np.testing.assert_allclose(yq_h, _hf_rope_freq_dim(nq, c["pos"], R, 1e4, D), rtol=0, atol=tol)
    np.testing.assert_allclose(yq_i, _gptj_rope(nq, c["pos"], R, D), rtol=0, atol=tol)
    # and the two denominators differ here (R < D): the flag is not a no-op
    yq = _fwd(o, c, R, 1e-30, 1e4)[0]
    assert np.abs(yq - yq_h).max() > 1e-3


def test_interleaved_is_channel_permutation_of_half_split(oracle_mod):
    """Moving channel 2i to i and 2i+1 to i+R/2 (tail fixed) turns interleaved
    RoPE into half-split RoPE, in the forward and the backward; the weights
    move with their channels and dw comes back permuted."""
    o = oracle_mod
    D, R = 32, 16
    c = _case(32, 5, 3, 2, D, max_pos=3000)
    perm = np.concatenate([np.arange(0, R, 2), np.arange(1, R, 2), np.arange(R, D)])
    P = lambda a: a[..., perm]
    il = o.flags_of(interleaved=True)
    args_i = (c["q"], c["k"], c["wq"], c["wk"], c["pos"])
    args_h = tuple(P(a) for a in (c["q"], c["k"], c["wq"], c["wk"])) + (c["pos"],)
    yi = o.fwd(*args_i, R, 1e-5, 1e4, flags=il)
    yh = o.fwd(*args_h, R, 1e-5, 1e4)
    for a, b in zip(yi, yh):
        np.testing.assert_allclose(P(a), b, rtol=0, atol=1e-14)
    gi = o.bwd(*args_i, c["dyq"], c["dyk"], R, 1e-5, 1e4, flags=il)
    gh = o.bwd(*args_h, P(c["dyq"]), P(c["dyk"]), R, 1e-5, 1e4)
    for a, b in zip(gi, gh):
        np.testing.assert_allclose(P(a), b, rtol=0, atol=1e-13)


def test_freq_head_dim_is_rescaled_base(oracle_mod):
    """theta^(-2i/D) = (theta^(R/D))^(-2i/R): the flagged oracle at theta agrees
    with the unflagged one at base theta^(R/D) (up to the last bits of pow and
    the fp32 rounding of cos/sin), and at R = D the flag changes nothing."""
    o = oracle_mod
    D = 64
    c = _case(33, 6, 2, 1, D, max_pos=2000)
    fh = o.flags_of(freq_head_dim=True)
    for R in (16, 32):
        a = o.fwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], R, 1e-6, 5e5, flags=fh)
        b = o.fwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], R, 1e-6, 5e5 ** (R / D))
        for x, y in zip(a, b):
            np.testing.assert_allclose(x, y, rtol=0, atol=4e-7 * np.abs(y).max())
    a = o.fwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], D, 1e-6, 5e5, flags=fh)
    b = o.fwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], D, 1e-6, 5e5)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_cos_sin_with_head_dim_denominator(oracle_mod):
    """rope_cos_sin with denominator D evaluates cos/sin of pos*theta^(-2i/D)
    (mpmath at 40 digits), the first R/2 of them."""
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 40
    for pos, theta, R, D in [(777, 1e4, 32, 128), (65535, 1e6, 16, 64)]:
        c, s = oracle_mod.rope_cos_sin(pos, theta, R, freq_denom=D)
        assert len(c) == R // 2
        for i in range(R // 2):
            phi = pos * mpmath.power(mpmath.mpf(theta), mpmath.mpf(-2 * i) / D)
            assert abs(c[i] - float(mpmath.cos(phi))) <= 2 ** -24
            assert abs(s[i] - float(mpmath.sin(phi))) <= 2 ** -24


def test_unit_weight_is_weightless_rms_norm(oracle_mod):
    """A parameter-free QK norm is the weight vector of ones: rotary_dim 0 with
    w = 1 equals torch's rms_norm without a weight."""
    D = 64
    c = _case(34, 4, 3, 2, D, scale=0.7)
    one = np.ones(D)
    eps = 2.0 ** -10   # exactly representable in fp32, as the oracle uses it
    yq, _ = oracle_mod.fwd(c["q"], c["k"], one, one, c["pos"], 0, eps, 1e4)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(c["q"]), (D,), None, eps)
    np.testing.assert_allclose(yq, ref.numpy(), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("flags", [1, 2, 3])
def test_variant_backward_finite_differences(oracle_mod, flags):
    """Central differences of L = <dy, y> for the interleaved and head-width
    frequency variants (T=3, H=2, D=16, R=8, eps=2^-10)."""
    o = oracle_mod
    g = np.random.default_rng(40 + flags)
    T, H, D, R = 3, 2, 16, 8
    q = g.standard_normal((T, H, D))
    k = g.standard_normal((T, 1, D))
    wq = 1 + 0.3 * g.standard_normal(D)
    wk = 1 + 0.3 * g.standard_normal(D)
    pos = np.array([0, 7, 41], np.int32)
    dyq = g.standard_normal((T, H, D))
    dyk = g.standard_normal((T, 1, D))
    eps = 2.0 ** -10
    dq, dk, dwq, dwk = o.bwd(q, k, wq, wk, pos, dyq, dyk, R, eps, 1e4, flags=flags)

    def loss(q_, k_, wq_, wk_):
        yq, yk = o.fwd(q_, k_, wq_, wk_, pos, R, eps, 1e4, flags=flags)
        return float(np.sum(dyq * yq) + np.sum(dyk * yk))

    hs = 1e-6
    for which, arr, got in ((0, q, dq), (1, k, dk), (2, wq, dwq), (3, wk, dwk)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            vals = [q, k, wq, wk]
            p = arr.copy(); p[idx] += hs
            m = arr.copy(); m[idx] -= hs
            vals[which] = p
            lp = loss(*vals)
            vals[which] = m
            num[idx] = (lp - loss(*vals)) / (2 * hs)
        np.testing.assert_allclose(got, num, rtol=1e-6, atol=1e-7 * np.abs(num).max())
        assert np.abs(got).max() > 1e-3


# --- QK-LayerNorm, biases, frequency tables ---------------------------------

LN = 4


@pytest.mark.parametrize("D", [16, 64, 128])
def test_layernorm_matches_torch_layer_norm(oracle_mod, D):
    """ORACLE_LAYERNORM with rotary_dim 0 and biases is torch's fp64
    layer_norm (mean subtracted, biased variance, eps inside the root, weight
    then bias) — the QK-LayerNorm of the Nyonic report abstract."""
    c = _case(50, 5, 3, 2, D, scale=0.6)
    g = np.random.default_rng(51)
    bq, bk = 0.3 * g.standard_normal(D), 0.3 * g.standard_normal(D)
    c["q"] += 0.7   # a non-zero mean, so the centring matters
    eps = 0.25
    yq, yk = oracle_mod.fwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], 0, eps, 1e4, flags=LN,
                            bq=bq, bk=bk)
    for x, w, b, y in ((c["q"], c["wq"], bq, yq), (c["k"], c["wk"], bk, yk)):
        ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (D,), torch.from_numpy(w),
                                             torch.from_numpy(b), eps)
        np.testing.assert_allclose(y, ref.numpy(), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("layernorm", [False, True])
def test_bias_is_added_before_rotation(oracle_mod, layernorm):
    """With biases, the norm output n = w xh + b is what RoPE rotates: torch's
    layer_norm / rms_norm (+ b) followed by transformers' RoPE."""
    D, R = 64, 32
    c = _case(52, 6, 2, 1, D, max_pos=40)
    g = np.random.default_rng(53)
    bq, bk = 0.5 * g.standard_normal(D), 0.5 * g.standard_normal(D)
    eps = 2.0 ** -12
    flags = LN if layernorm else 0
    yq, _ = oracle_mod.fwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], R, eps, 1e4, flags=flags,
                           bq=bq, bk=bk)
    xt = torch.from_numpy(c["q"])
    if layernorm:
        n = torch.nn.functional.layer_norm(xt, (D,), torch.from_numpy(c["wq"]), torch.from_numpy(bq), eps)
    else:
        n = torch.nn.functional.rms_norm(xt, (D,), torch.from_numpy(c["wq"]), eps) + torch.from_numpy(bq)
    ref = _hf_rope(n.numpy(), c["pos"], R, 1e4, D)
    np.testing.assert_allclose(yq, ref, rtol=0, atol=2e-5 * float(np.abs(n.numpy()).max()))


def test_layernorm_invariants(oracle_mod):
    """LayerNorm output is unchanged by adding a constant to the row (up to
    rounding); with w = 1, b = 0, R = 0 each output row has mean 0 and
    mean square var/(var + eps); its input gradient sums to 0 over each row."""
    o = oracle_mod
    D = 32
    c = _case(54, 4, 2, 1, D)
    one = np.ones(D)
    eps = 2.0 ** -8
    y0 = o.fwd(c["q"], c["k"], one, one, c["pos"], 0, eps, 1e4, flags=LN)[0]
    y1 = o.fwd(c["q"] + 3.25, c["k"], one, one, c["pos"], 0, eps, 1e4, flags=LN)[0]
    np.testing.assert_allclose(y1, y0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(y0.mean(axis=-1), 0.0, atol=1e-14)
    var = c["q"].var(axis=-1)
    np.testing.assert_allclose((y0 * y0).mean(axis=-1), var / (var + eps), rtol=1e-12)
    dq = o.bwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], c["dyq"], c["dyk"], 16, eps, 1e4,
               flags=LN)[0]
    np.testing.assert_allclose(dq.sum(axis=-1), 0.0, atol=1e-12)


@pytest.mark.parametrize("flags,R", [(LN, 8), (LN | 1, 8), (0, 8), (LN, 0)])
def test_bias_and_layernorm_backward_finite_differences(oracle_mod, flags, R):
    """Central differences of L = <dy, y> with biases, for LayerNorm (both
    pairings) and RMSNorm: dx, dw and db (T=3, H=2, D=16, eps=2^-10)."""
    o = oracle_mod
    g = np.random.default_rng(60 + flags + R)
    T, H, D = 3, 2, 16
    q = g.standard_normal((T, H, D)) + 0.5
    k = g.standard_normal((T, 1, D))
    wq, wk = 1 + 0.3 * g.standard_normal(D), 1 + 0.3 * g.standard_normal(D)
    bq, bk = 0.4 * g.standard_normal(D), 0.4 * g.standard_normal(D)
    pos = np.array([0, 9, 33], np.int32)
    dyq, dyk = g.standard_normal((T, H, D)), g.standard_normal((T, 1, D))
    eps = 2.0 ** -10
    dq, dk, dwq, dwk, dbq, dbk = o.bwd(q, k, wq, wk, pos, dyq, dyk, R, eps, 1e4, flags=flags,
                                       bias_grads=True)

    def loss(v):
        yq, yk = o.fwd(v[0], v[1], v[2], v[3], pos, R, eps, 1e4, flags=flags, bq=v[4], bk=v[5])
        return float(np.sum(dyq * yq) + np.sum(dyk * yk))

    vals = [q, k, wq, wk, bq, bk]
    hs = 1e-6
    for which, got in enumerate((dq, dk, dwq, dwk, dbq, dbk)):
        arr = vals[which]
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            v = list(vals)
            p = arr.copy(); p[idx] += hs
            m = arr.copy(); m[idx] -= hs
            v[which] = p
            lp = loss(v)
            v[which] = m
            num[idx] = (lp - loss(v)) / (2 * hs)
        np.testing.assert_allclose(got, num, rtol=1e-6, atol=1e-7 * np.abs(num).max())
        assert np.abs(got).max() > 1e-3


@pytest.mark.parametrize("rope", [
    {"rope_type": "linear", "factor": 4.0},
    {"rope_type": "yarn", "factor": 4.0, "original_max_position_embeddings": 1024},
    {"rope_type": "llama3", "factor": 8.0, "low_freq_factor": 1.0, "high_freq_factor": 4.0,
     "original_max_position_embeddings": 1024},
    {"rope_type": "dynamic", "factor": 2.0},
])
def test_frequency_table_matches_transformers_scaled_rope(oracle_mod, rope):
    """RoPE extensions change the per-pair frequencies (and YaRN also scales cos
    and sin): the oracle given transformers' table and attention factor agrees
    with transformers' scaled rotary embedding and apply_rotary_pos_emb."""
    from transformers import LlamaConfig
    from transformers.models.llama import modeling_llama as ml

    D = 64
    cfg = LlamaConfig(hidden_size=2 * D, num_attention_heads=2, max_position_embeddings=4096,
                      rope_parameters=dict(rope, rope_theta=10000.0))
    emb = ml.LlamaRotaryEmbedding(cfg)
    table = emb.inv_freq.double().numpy()
    att = float(emb.attention_scaling)
    c = _unit_case(55, D)
    n = _fwd(oracle_mod, c, 0, 1e-30, 1e4)[0]
    y = oracle_mod.fwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], D, 1e-30, 1e4,
                       inv_freq=table, attention_factor=att)[0]
    xt = torch.from_numpy(n)
    cos, sin = emb(xt, torch.from_numpy(c["pos"].astype(np.int64))[None, :])
    xr = xt.transpose(0, 1)[None]
    yr, _ = ml.apply_rotary_pos_emb(xr, xr, cos.double(), sin.double(), unsqueeze_dim=1)
    ref = yr[0].transpose(0, 1).numpy()
    np.testing.assert_allclose(y, ref, rtol=0, atol=2e-5 * np.abs(n).max() * max(att, 1.0))
    if rope["rope_type"] != "dynamic":   # the table differs from the plain one
        assert np.abs(y - _fwd(oracle_mod, c, D, 1e-30, 1e4)[0]).max() > 1e-3


def test_frequency_table_equal_to_formula_changes_nothing(oracle_mod):
    """A table holding theta^(-2i/R) (the same fp64 pow) gives the default
    result bit for bit, forward and backward."""
    o = oracle_mod
    D, R = 64, 32
    c = _case(56, 5, 3, 1, D, max_pos=100000)
    table = np.array([math.pow(5e5, -2.0 * i / R) for i in range(R // 2)])
    a = o.fwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], R, 1e-6, 5e5, inv_freq=table)
    b = o.fwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], R, 1e-6, 5e5)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    ga = o.bwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], c["dyq"], c["dyk"], R, 1e-6, 5e5,
               inv_freq=table)
    gb = o.bwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], c["dyq"], c["dyk"], R, 1e-6, 5e5)
    for x, y in zip(ga, gb):
        assert np.array_equal(x, y)


def test_position_interpolation_identity(oracle_mod):
    """Linear position interpolation (frequencies theta_i / f) at position f m
    is the plain embedding at position m, up to the rounding of the fp64 angle."""
    o = oracle_mod
    D, R, f = 64, 64, 8
    c = _case(57, 6, 2, 1, D, max_pos=5000)
    table = np.array([math.pow(1e4, -2.0 * i / R) for i in range(R // 2)]) / f
    a = o.fwd(c["q"], c["k"], c["wq"], c["wk"], (c["pos"] * f).astype(np.int32), R, 1e-6, 1e4,
              inv_freq=table)[0]
    b = o.fwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], R, 1e-6, 1e4)[0]
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-6 * np.abs(b).max())


def test_attention_factor_scales_rotated_channels_exactly(oracle_mod):
    """A factor of 2 doubles c and s exactly (a power of two commutes with the
    fp32 rounding), so the rotated channels double bit for bit and the
    unrotated tail is unchanged; the backward's dx scales the same way through
    g = R^T dy on the rotated part."""
    o = oracle_mod
    D, R = 64, 32
    c = _case(58, 4, 2, 1, D, max_pos=3000)
    a = o.fwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], R, 1e-6, 1e4, attention_factor=2.0)[0]
    b = o.fwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], R, 1e-6, 1e4)[0]
    assert np.array_equal(a[..., :R], 2.0 * b[..., :R])
    assert np.array_equal(a[..., R:], b[..., R:])


# --- norm groups and per-head weights ----------------------------------------

HW = 8   # oracle.HEAD_WEIGHTS


def _grouped_norm_torch(x, g, w, b, eps, layernorm):
    """torch fp64 rms_norm / layer_norm over groups of g consecutive heads
    (normalized_shape g*D, no affine), then the [H, D] weight and bias."""
    T, H, D = x.shape
    xt = torch.from_numpy(x).reshape(T, H // g, g * D)
    if layernorm:
        n = torch.nn.functional.layer_norm(xt, (g * D,), None, None, eps)
    else:
        n = torch.nn.functional.rms_norm(xt, (g * D,), None, eps)
    n = n.reshape(T, H, D) * torch.as_tensor(w)
    return n + torch.as_tensor(b) if b is not None else n


def _group_case(seed, T, hq, hkv, D):
    g = np.random.default_rng(seed)
    c = _case(seed, T, hq, hkv, D, max_pos=300)
    c["wq"] = 1.0 + 0.2 * g.standard_normal((hq, D))
    c["wk"] = 1.0 + 0.2 * g.standard_normal((hkv, D))
    c["bq"] = 0.3 * g.standard_normal((hq, D))
    c["bk"] = 0.3 * g.standard_normal((hkv, D))
    # per-head offsets and scales, so that a group's statistics differ from its heads'
    c["q"] = c["q"] * (0.5 + g.random((1, hq, 1))) + 0.4 * g.standard_normal((1, hq, 1))
    c["k"] = c["k"] * (0.5 + g.random((1, hkv, 1))) + 0.4 * g.standard_normal((1, hkv, 1))
    return c


GROUPS = [(6, 2, 3, 2, False), (6, 2, 6, 1, True), (4, 4, 2, 4, False), (8, 2, 1, 1, True),
          (3, 1, 3, 1, False)]


@pytest.mark.parametrize("hq,hkv,gq,gk,layernorm", GROUPS)
def test_norm_groups_match_torch(oracle_mod, hq, hkv, gq, gk, layernorm):
    """Heads in groups of gq (q) and gk (k) share one inverse RMS (QK-Normed
    MLA abstract: one per token and head group; a group of every head is the
    layerwise norm of the SwiftQK abstract): torch's fp64 rms_norm / layer_norm
    over the grouped view with [H, D] weights and biases at rotary_dim 0, and
    then transformers' RoPE on each head at rotary_dim 16."""
    o = oracle_mod
    D = 32
    c = _group_case(70 + hq + gq, 5, hq, hkv, D)
    eps = 0.0625   # exact in fp32, the precision eps is passed in
    flags = HW | (LN if layernorm else 0)
    for R in (0, 16):
        yq, yk = o.fwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], R, eps, 1e4, flags=flags,
                       bq=c["bq"], bk=c["bk"], norm_groups=(gq, gk))
        for x, w, b, gsz, y in ((c["q"], c["wq"], c["bq"], gq, yq), (c["k"], c["wk"], c["bk"], gk, yk)):
            n = _grouped_norm_torch(x, gsz, w, b, eps, layernorm).numpy()
            if R == 0:
                np.testing.assert_allclose(y, n, rtol=1e-13, atol=1e-13)
            else:
                ref = _hf_rope(n, c["pos"], R, 1e4, D)
                np.testing.assert_allclose(y, ref, rtol=0, atol=2e-5 * np.abs(n).max())


def _torch_rope_const(n, cs, R, interleaved):
    """Rotation of the first R channels of n [T, H, D] by the oracle's fp32
    cos/sin values (constants here, so autograd differentiates the norm)."""
    c = torch.from_numpy(np.stack([a for a, _ in cs]))[:, None, :]   # [T, 1, R/2]
    s = torch.from_numpy(np.stack([b for _, b in cs]))[:, None, :]
    h = R // 2
    if interleaved:
        a, b = n[..., 0:R:2], n[..., 1:R:2]
        ya, yb = a * c - b * s, b * c + a * s
        rot = torch.stack([ya, yb], dim=-1).reshape(n.shape[:-1] + (R,))
    else:
        a, b = n[..., :h], n[..., h:R]
        rot = torch.cat([a * c - b * s, b * c + a * s], dim=-1)
    return torch.cat([rot, n[..., R:]], dim=-1)


@pytest.mark.parametrize("hq,hkv,gq,gk,layernorm", GROUPS)
@pytest.mark.parametrize("interleaved", [False, True])
def test_norm_groups_backward_matches_autograd(oracle_mod, hq, hkv, gq, gk, layernorm, interleaved):
    """The grouped backward (dx, [H, D] dw and db) equals torch autograd of the
    torch-built forward (grouped fp64 rms_norm / layer_norm, weights, biases,
    rotation by the oracle's cos/sin) for L = <dy, y>."""
    o = oracle_mod
    D, R, T = 16, 8, 4
    c = _group_case(90 + hq + gk, T, hq, hkv, D)
    eps = 2.0 ** -8
    flags = HW | (LN if layernorm else 0) | (1 if interleaved else 0)
    cs = [o.rope_cos_sin(int(p), 1e4, R) for p in c["pos"]]
    got = o.bwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], c["dyq"], c["dyk"], R, eps, 1e4,
                flags=flags, bias_grads=True, norm_groups=(gq, gk))
    for i, (x, w, b, gsz, dy) in enumerate(((c["q"], c["wq"], c["bq"], gq, c["dyq"]),
                                            (c["k"], c["wk"], c["bk"], gk, c["dyk"]))):
        xt = torch.from_numpy(x).requires_grad_()
        wt = torch.from_numpy(w).requires_grad_()
        bt = torch.from_numpy(b).requires_grad_()
        T_, H, _ = x.shape
        xg = xt.reshape(T_, H // gsz, gsz * D)
        if layernorm:
            n = torch.nn.functional.layer_norm(xg, (gsz * D,), None, None, eps)
        else:
            n = torch.nn.functional.rms_norm(xg, (gsz * D,), None, eps)
        n = n.reshape(T_, H, D) * wt + bt
        y = _torch_rope_const(n, cs, R, interleaved)
        (y * torch.from_numpy(dy)).sum().backward()
        dx, dw, db = got[i], got[2 + i], got[4 + i]
        np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(db, bt.grad.numpy(), rtol=1e-11, atol=1e-12)
        assert np.abs(dx).max() > 1e-3 and np.abs(dw).max() > 1e-3


def test_layerwise_unit_weight_rms(oracle_mod):
    """A group of every head with w = 1 and rotary_dim 0: each token's whole
    output vector has mean square ms/(ms + eps), ms over all H*D inputs (the
    full-hidden-vector norm of the SwiftQK abstract); each head alone does not."""
    o = oracle_mod
    T, H, D, eps = 5, 4, 16, 0.375
    c = _group_case(111, T, H, 1, D)
    one = np.ones((H, D))
    y = o.fwd(c["q"], c["k"], one, np.ones((1, D)), c["pos"], 0, eps, 1e4, flags=HW,
              norm_groups=(H, 1))[0]
    ms = (c["q"] ** 2).mean(axis=(1, 2))
    np.testing.assert_allclose((y ** 2).mean(axis=(1, 2)), ms / (ms + eps), rtol=1e-13)
    per_head = (y ** 2).mean(axis=2)
    assert np.abs(per_head - per_head.mean(axis=1, keepdims=True)).max() > 0.05


def test_group_of_one_with_tiled_weights_is_the_per_head_norm(oracle_mod):
    """Groups of one head and [H, D] weights that repeat one [D] vector give the
    per-head result bit for bit, and the [H, D] weight gradient summed over
    heads is the [D] one."""
    o = oracle_mod
    D, R = 32, 16
    c = _case(112, 6, 4, 2, D, max_pos=5000)
    a = o.fwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], R, 1e-5, 1e4, flags=LN)
    b = o.fwd(c["q"], c["k"], np.tile(c["wq"], (4, 1)), np.tile(c["wk"], (2, 1)), c["pos"], R,
              1e-5, 1e4, flags=LN | HW, norm_groups=(1, 1))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    ga = o.bwd(c["q"], c["k"], c["wq"], c["wk"], c["pos"], c["dyq"], c["dyk"], R, 1e-5, 1e4)
    gb = o.bwd(c["q"], c["k"], np.tile(c["wq"], (4, 1)), np.tile(c["wk"], (2, 1)), c["pos"],
               c["dyq"], c["dyk"], R, 1e-5, 1e4, flags=HW, norm_groups=(1, 1))
    assert np.array_equal(ga[0], gb[0]) and np.array_equal(ga[1], gb[1])
    np.testing.assert_allclose(gb[2].sum(axis=0), ga[2], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gb[3].sum(axis=0), ga[3], rtol=1e-12, atol=1e-12)


# --- Best-Fit-Decreasing packing -----------------------------------------------

def _read_bfd_golden():
    vals = {}
    for line in open(os.path.join(GOLDEN, "bfd_hand_example.txt")):
        line = line.split("#")[0].split()
        if line:
            vals[line[0]] = [int(v) for v in line[1:]]
    return vals


def test_bfd_golden_hand_example(oracle_mod):
    """The hand-worked packing of tests/golden/bfd_hand_example.txt."""
    g = _read_bfd_golden()
    r = oracle_mod.bfd_pack(g["lengths"], g["capacity"][0], 8)
    assert r["status"] == 0 and r["bins"] == g["bins"][0]
    assert r["doc_start"].tolist() == g["doc_start"]
    assert r["cu_seqlens"].tolist() == g["cu_seqlens"]
    assert r["position_ids"].tolist() == g["position_ids"]


def _bfd_lengths(seed, n, cap, kind):
    g = np.random.default_rng(seed)
    if kind == "loguniform":
        return np.clip(np.rint(np.exp(g.uniform(np.log(1), np.log(cap), n))), 1, cap).astype(np.int32)
    if kind == "ties":
        return g.choice([cap // 2, cap // 3, cap // 4, cap // 5 + 1], size=n).astype(np.int32)
    return g.integers(1, cap + 1, size=n).astype(np.int32)


@pytest.mark.parametrize("seed,n,cap,kind", [(1, 200, 1000, "loguniform"), (2, 300, 64, "ties"),
                                             (3, 150, 97, "uniform"), (4, 1, 5, "uniform"),
                                             (5, 0, 16, "uniform")])
def test_bfd_layout_and_best_fit_rule(oracle_mod, seed, n, cap, kind):
    """Every document lies inside one bin; segments (documents, then one filler
    per bin that is not full) tile the buffers in cu_seqlens order; position
    ids count from 0 in every segment; and replaying the documents longest
    first (input order among equals) each one sits in the open bin with the
    least room that fits it (lowest index among equals), or opens the next bin
    exactly when none fits."""
    L = _bfd_lengths(seed, n, cap, kind)
    r = oracle_mod.bfd_pack(L, cap, max(1, n))
    assert r["status"] == 0
    nb, start, cu, pos = r["bins"], r["doc_start"], r["cu_seqlens"], r["position_ids"]
    assert pos.shape == (nb * cap,) and cu[0] == 0 and cu[-1] == nb * cap
    assert np.all(np.diff(cu) > 0)
    for i in range(n):
        assert start[i] // cap == (start[i] + L[i] - 1) // cap
    seg_of_start = {int(c): k for k, c in enumerate(cu[:-1])}
    for i in range(n):
        assert int(start[i]) in seg_of_start
        assert cu[seg_of_start[int(start[i])] + 1] == start[i] + L[i]
    for k in range(len(cu) - 1):
        assert np.array_equal(pos[cu[k]: cu[k + 1]], np.arange(cu[k + 1] - cu[k]))
    fill = np.zeros(nb, np.int64)
    for i in sorted(range(n), key=lambda i: (-int(L[i]), i)):
        b = int(start[i]) // cap
        opened = int((fill > 0).sum())
        fits = [c for c in range(opened) if cap - fill[c] >= L[i]]
        if fits:
            want = min(fits, key=lambda c: (cap - fill[c], c))
        else:
            want = opened
        assert b == want, (i, b, want)
        assert start[i] == b * cap + fill[b]
        fill[b] += L[i]
    assert np.all(fill > 0)


def test_bfd_matches_the_input_generator_packer(oracle_mod):
    """The separately written packer that builds the packed workload
    (workloads/bfd.py) gives the same bins, in the same placement order."""
    from workloads import bfd
    for seed in range(5):
        L = _bfd_lengths(100 + seed, 400, 4096, "loguniform")
        bins = bfd.bfd_bins(L.astype(np.int64), 4096)
        r = oracle_mod.bfd_pack(L, 4096, 400)
        assert r["bins"] == len(bins)
        got = [[] for _ in range(r["bins"])]
        for i in sorted(range(len(L)), key=lambda i: r["doc_start"][i]):
            got[r["doc_start"][i] // 4096].append(int(L[i]))
        assert got == bins


def _opt_bins(L, cap):
    """Fewest bins, by exhaustive search (tiny inputs only)."""
    best = [len(L)]

    def go(i, free):
        if len(free) >= best[0]:
            return
        if i == len(L):
            best[0] = len(free)
            return
        for b in range(len(free)):
            if free[b] >= L[i]:
                free[b] -= L[i]
                go(i + 1, free)
                free[b] += L[i]
        free.append(cap - L[i])
        go(i + 1, free)
        free.pop()

    go(0, [])
    return best[0]


def test_bfd_bound_against_exhaustive_optimum(oracle_mod):
    """BFD uses at most 11/9 OPT + 6/9 bins (the tight bound of the
    decreasing best/first-fit rules), OPT by exhaustive search; and, like
    every any-fit rule, leaves at most one bin at most half full."""
    g = np.random.default_rng(7)
    for trial in range(150):
        n = int(g.integers(1, 8))
        cap = int(g.integers(5, 30))
        L = g.integers(1, cap + 1, size=n).astype(np.int32)
        r = oracle_mod.bfd_pack(L, cap, n)
        opt = _opt_bins(sorted(L.tolist(), reverse=True), cap)
        assert opt <= r["bins"] <= 11 * opt / 9 + 6 / 9, (L, cap, r["bins"], opt)
        fills = np.zeros(r["bins"])
        for i in range(n):
            fills[r["doc_start"][i] // cap] += L[i]
        assert np.sum(fills <= cap / 2) <= 1
    # the heuristic is not optimal on every instance: capacity 10,
    # [4, 4, 3, 3, 3, 3] gives [4, 4], [3, 3, 3], [3]; the optimum is [4, 3, 3] twice
    r = oracle_mod.bfd_pack([4, 4, 3, 3, 3, 3], 10, 6)
    assert r["bins"] == 3 and _opt_bins([4, 4, 3, 3, 3, 3], 10) == 2


def test_bfd_status(oracle_mod):
    assert oracle_mod.bfd_pack([3, 0, 2], 5, 4)["status"] == 2
    assert oracle_mod.bfd_pack([3, 6, 2], 5, 4)["status"] == 2
    assert oracle_mod.bfd_pack([3, 3, 3], 5, 2)["status"] == 1
    assert oracle_mod.bfd_pack([3, 3, 3], 5, 3)["status"] == 0
