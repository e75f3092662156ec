"""Pins for the CPU oracle: checks against facts fixed outside the oracle.

Each test ties one part of the oracle to something other than itself: a
hand-worked example (tests/golden), closed forms, a library routine that
computes the same mathematical object by another route (torch's fp64 scaled
dot-product attention, Python's sort), exact special cases and bounds.

Sources for the rules being pinned ("S2O: Early Stopping for Sparse Attention
via Online Permutation"): the gist.science technical summary, sections
"Classement par Segment" (segments, KV_perm), "2. Règle d'Arrêt Anticipé"
(stop on marginal gain relative to accumulated mass) and "3. Implémentation du
Noyau" (pass 1 dense causal window in the segment, pass 2 history in list
order); the authors' abstract (high-to-low importance, skip the remaining
blocks).
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from long_context_prefill_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _built(oracle_lib):
    return oracle_lib


def f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def tiles_of(p):
    T = p.N // p.tile_m
    return [(b, h, t) for b in range(p.B) for h in range(p.Hq) for t in range(T)]


def run_all(p, Q, K, V, tau):
    """Whole problem through the oracle: O [B,Hq,N,d], n_exec [B,Hq,T], chunks."""
    T = p.N // p.tile_m
    r = oracle.attn_tiles(p, Q, K, V, tiles_of(p), tau, want_lists=True)
    out = r["out"].reshape(p.B, p.Hq, T * p.tile_m, p.d)
    return out, r["n_exec"].reshape(p.B, p.Hq, T), r["chunks"].reshape(p.B, p.Hq, T), r


def widen(a, p):
    return a.astype(np.float64) if p.dtype == 0 else synth.f32_from_bf16_bits(a).astype(np.float64)


def sdpa_fp64(p, Q, K, V):
    """torch's scaled dot-product attention (causal, fp64) as the reference."""
    G = p.Hq // p.Hkv
    q = torch.from_numpy(widen(Q, p))
    k = torch.from_numpy(widen(K, p)).repeat_interleave(G, dim=1)
    v = torch.from_numpy(widen(V, p)).repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=p.scale)
    return o.numpy()


def random_inputs(B, Hq, Hkv, N, d, seed, structure="stripes", dtype="f32", n_stripes=6):
    w = synth.custom_workload(B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, dtype=dtype, structure=structure,
                              n_stripes=n_stripes, seed=seed)
    x = synth.make_inputs(w)
    return x["q"], x["k"], x["v"]


# ---------------------------------------------------------------- geometry ---

@pytest.mark.parametrize("N,S,BM", [(2048, 512, 64), (16384, 4096, 128), (1000 * 4, 384, 4),
                                    (96, 32, 16), (64, 64, 64), (40, 16, 8)])
def test_list_offsets_closed_form(N, S, BM):
    """off(b,h,t) = (b*Hq+h)*L + S*(P*s*(s-1)/2 + (t-s*P)*s), P = S/BM, s = t // P."""
    p = oracle.problem(2, 3, 1, N, 8, "f32", S, BM, min(BM, 4), 1.0)
    T, P = N // BM, S // BM
    L = sum((t * BM // S) * S for t in range(T))
    assert oracle.list_entries(p) == 2 * 3 * L
    for b in (0, 1):
        for h in (0, 2):
            for t in sorted({0, 1, P - 1, P, T // 2, T - 1}):
                s = t // P
                want = (b * 3 + h) * L + S * (P * s * (s - 1) // 2 + (t - s * P) * s)
                assert oracle.list_offset(p, b, h, t) == want
                assert oracle.seg_start(p, t) == s * S


# ------------------------------------------------------- hand-worked golden --

def test_worked_example_golden():
    g = json.load(open(os.path.join(GOLDEN, "ln_weights_worked_example.json")))
    w = np.array([1, 8, 2, 4, 1, 1, 1, 1], dtype=np.float64)
    N, d = 8, 1
    Q = f32(np.ones((1, 1, N, d)))
    K = f32(np.log(w).reshape(1, 1, N, d))
    V = f32(np.arange(N, dtype=np.float64).reshape(1, 1, N, d))
    for bm, key in ((1, "tile_m_1"), (2, "tile_m_2")):
        p = oracle.problem(1, 1, 1, N, d, "f32", 4, bm, 1, 1.0)
        out, n_exec, _, r = run_all(p, Q, K, V, g["inputs"]["tau"])
        want = np.array([float(Fraction(s)) for s in g["expected"][key]["out"]])
        np.testing.assert_allclose(out[0, 0, :, 0], want, rtol=0, atol=g["tolerance"])
        assert n_exec[0, 0].tolist() == g["expected"][key]["n_exec"]
        # the list of every history tile is [1, 3, 2, 0]
        for n, (_, _, t) in enumerate(tiles_of(p)):
            if oracle.seg_start(p, t) == 4:
                assert r["lists"][n, :4].tolist() == [1, 3, 2, 0]


# --------------------------------------------------------- pool and score ---

def test_pool_exact_on_dyadic_inputs():
    """Small integers: every fp32 partial sum is exact, so qbar is the exact mean."""
    rng = np.random.default_rng(1)
    N, d, BM = 64, 8, 16
    Q = f32(rng.integers(-8, 9, size=(1, 2, N, d)))
    p = oracle.problem(1, 2, 1, N, d, "f32", 32, BM, 4, 1.0)
    for h in range(2):
        for t in range(N // BM):
            rows = Q[0, h, t * BM:(t + 1) * BM].astype(np.int64)
            want = [Fraction(int(c), BM) for c in rows.sum(axis=0)]
            got = oracle.pool(p, Q, 0, h, t)
            assert [Fraction(float(x)) for x in got] == want


def test_score_exact_basis_keys_and_gqa_head_mapping():
    """K_g[j] = (g+1)*(j+1)*e_{j mod d}; Q_h rows constant -> s[j] = qbar[j mod d]*(g+1)*(j+1)
    exactly, and query head h must read KV head h // G."""
    Hq, Hkv, N, d, BM, S = 4, 2, 32, 4, 4, 8
    K = np.zeros((1, Hkv, N, d), dtype=np.float32)
    for g in range(Hkv):
        for j in range(N):
            K[0, g, j, j % d] = (g + 1) * (j + 1)
    Q = np.zeros((1, Hq, N, d), dtype=np.float32)
    for h in range(Hq):
        Q[0, h, :, :] = (h + 1) * np.array([1, -2, 3, -4], dtype=np.float32)
    p = oracle.problem(1, Hq, Hkv, N, d, "f32", S, BM, 2, 1.0)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        for t in range(N // BM):
            s = oracle.score_tile(p, Q, K, 0, h, t)
            a = oracle.seg_start(p, t)
            want = [(h + 1) * [1, -2, 3, -4][j % d] * (g + 1) * (j + 1) for j in range(a)]
            assert s.tolist() == want


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_score_within_fp32_error_bound(dtype):
    """|s - dot_fp64(qbar, K_j)| <= d*u*sum|qbar_k K_jk| (u = 2^-24) for the fmaf chain,
    and qbar within BM*u*sum|Q| of the fp64 mean."""
    Q, K, V = random_inputs(1, 2, 1, 256, 32, seed=7, dtype=dtype)
    p = oracle.problem(1, 2, 1, 256, 32, dtype, 64, 16, 8, 1 / np.sqrt(32))
    u = 2.0 ** -24
    Kd, Qd = widen(K, p), widen(Q, p)
    for h in range(2):
        for t in (4, 9, 15):
            qb = oracle.pool(p, Q, 0, h, t).astype(np.float64)
            rows = Qd[0, h, t * 16:(t + 1) * 16]
            assert np.all(np.abs(qb - rows.mean(axis=0)) <= 1.01 * u * np.abs(rows).sum(axis=0))
            s = oracle.score_tile(p, Q, K, 0, h, t).astype(np.float64)
            a = oracle.seg_start(p, t)
            exact = Kd[0, 0, :a] @ qb
            bound = 1.01 * 32 * u * (np.abs(Kd[0, 0, :a]) @ np.abs(qb))
            assert np.all(np.abs(s - exact) <= bound)


# ------------------------------------------------------------------ order ---

def test_order_matches_python_sort_with_ties():
    rng = np.random.default_rng(3)
    for n in (1, 2, 7, 64, 1000):
        s = f32(rng.integers(-3, 4, size=n) * 0.5)  # many exact ties
        s[rng.random(n) < 0.2] = -0.0  # -0.0 ties with +0.0
        want = sorted(range(n), key=lambda j: (-float(s[j]), j))
        assert oracle.order(s).tolist() == want


def test_order_is_a_descending_permutation_with_low_index_ties():
    rng = np.random.default_rng(4)
    s = f32(np.round(rng.standard_normal(5000), 1))
    lst = oracle.order(s)
    seen = np.zeros(len(s), dtype=bool)
    seen[lst] = True
    assert seen.all() and len(lst) == len(s)
    v = s[lst]
    assert np.all(v[:-1] >= v[1:])
    tie = v[:-1] == v[1:]
    assert np.all(lst[:-1][tie] < lst[1:][tie])


def test_lists_and_scores_of_whole_problem_match_per_tile():
    Q, K, V = random_inputs(2, 4, 2, 128, 16, seed=11)
    p = oracle.problem(2, 4, 2, 128, 16, "f32", 32, 8, 4, 0.25)
    scores = oracle.scores_all(p, Q, K)
    lists = oracle.lists_all(p, scores)
    assert len(scores) == oracle.list_entries(p)
    for b, h, t in tiles_of(p):
        off, a = oracle.list_offset(p, b, h, t), oracle.seg_start(p, t)
        s = oracle.score_tile(p, Q, K, b, h, t)
        assert np.array_equal(scores[off:off + a], s)
        assert np.array_equal(lists[off:off + a], oracle.order(s))


# ------------------------------------------- tau = 0 equals dense attention --

GEOMS = [
    # B, Hq, Hkv, N, d, S, BM, BN, dtype
    (1, 1, 1, 256, 16, 64, 16, 8, "f32"),
    (2, 4, 2, 192, 8, 64, 8, 4, "f32"),     # GQA, batch 2
    (1, 2, 1, 200, 8, 48, 8, 8, "bf16"),    # ragged last segment (200 % 48 != 0)
    (1, 1, 1, 64, 4, 16, 1, 1, "f32"),      # one-row tiles, one-key chunks
    (1, 1, 1, 128, 16, 128, 32, 16, "f32"), # one segment: pure pass 1
    (1, 2, 2, 256, 32, 64, 64, 64, "bf16"), # tile = segment
]


@pytest.mark.parametrize("geom", GEOMS)
def test_tau_zero_equals_dense_attention(geom):
    """Order-invariance of softmax attention over keys: with tau = 0 the method visits every
    causal key exactly once, so it must equal dense causal attention (torch fp64 SDPA)."""
    B, Hq, Hkv, N, d, S, BM, BN, dt = geom
    Q, K, V = random_inputs(B, Hq, Hkv, N, d, seed=21 + N, dtype=dt)
    p = oracle.problem(B, Hq, Hkv, N, d, dt, S, BM, BN, 1 / np.sqrt(d))
    out, n_exec, chunks, _ = run_all(p, Q, K, V, 0.0)
    ref = sdpa_fp64(p, Q, K, V)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    T = N // BM
    for t in range(T):
        a = (t * BM // S) * S
        assert np.all(chunks[:, :, t] == a // BN)              # never stops
        assert np.all(n_exec[:, :, t] == ((t + 1) * BM - a) // BN + a // BN)


def test_dense_rows_match_sdpa():
    Q, K, V = random_inputs(1, 4, 2, 160, 16, seed=5, dtype="bf16")
    p = oracle.problem(1, 4, 2, 160, 16, "bf16", 32, 16, 16, 0.3)
    ref = sdpa_fp64(p, Q, K, V)
    for h in range(4):
        np.testing.assert_allclose(oracle.dense_rows(p, Q, K, V, 0, h, 0, 160), ref[0, h],
                                   rtol=0, atol=1e-12)
    outs = oracle.dense_requests(p, Q, K, V, [(0, 1, 10, 20), (0, 3, 100, 160)])
    np.testing.assert_allclose(outs[0], ref[0, 1, 10:20], atol=1e-12)
    np.testing.assert_allclose(outs[1], ref[0, 3, 100:160], atol=1e-12)


def test_bf16_inputs_are_widened_exactly():
    Q, K, V = random_inputs(1, 2, 1, 128, 16, seed=9, dtype="bf16")
    pb = oracle.problem(1, 2, 1, 128, 16, "bf16", 32, 16, 8, 0.25)
    pf = oracle.problem(1, 2, 1, 128, 16, "f32", 32, 16, 8, 0.25)
    Qf, Kf, Vf = (f32(synth.f32_from_bf16_bits(a)) for a in (Q, K, V))
    ob, nb, _, rb = run_all(pb, Q, K, V, 0.05)
    of, nf, _, rf = run_all(pf, Qf, Kf, Vf, 0.05)
    assert np.array_equal(ob, of) and np.array_equal(nb, nf)
    for n, (_, _, t) in enumerate(tiles_of(pb)):
        a = oracle.seg_start(pb, t)
        assert np.array_equal(rb["lists"][n, :a], rf["lists"][n, :a])


# ------------------------------------------------ closed form of the stop rule --

def q_zero_prediction(BM, BN, S, t, tau):
    """Q = 0: every logit and score is 0, so the list is ascending and each key has weight 1.
    Row i's mass after pass 1 is i - a + 1; after chunk c it is i - a + 1 + BN*(c+1) and the
    chunk's gain is BN / that.  The first row has the largest gain, so the tile stops after
    the first chunk c with BN < tau * (r0 + 1 + BN*(c+1)), r0 = t*BM - a."""
    a = (t * BM // S) * S
    C = a // BN
    r0 = t * BM - a
    n = C
    for c in range(C):
        if BN < tau * (r0 + 1 + BN * (c + 1)):
            n = c + 1
            break
    return a, n


@pytest.mark.parametrize("BM,BN,S,N,tau", [
    (16, 8, 64, 256, 0.05), (16, 8, 64, 256, 0.02), (8, 4, 32, 256, 0.1),
    (1, 1, 16, 96, 0.125), (4, 4, 16, 96, 0.2), (16, 16, 32, 256, 1.0), (16, 16, 32, 256, 3.0)])
def test_q_zero_closed_form(BM, BN, S, N, tau):
    d = 4
    rng = np.random.default_rng(BM * 1000 + BN)
    Q = np.zeros((1, 1, N, d), dtype=np.float32)
    K = f32(rng.standard_normal((1, 1, N, d)))
    V = f32(rng.standard_normal((1, 1, N, d)))
    p = oracle.problem(1, 1, 1, N, d, "f32", S, BM, BN, 0.5)
    out, n_exec, chunks, r = run_all(p, Q, K, V, tau)
    for t in range(N // BM):
        a, n = q_zero_prediction(BM, BN, S, t, tau)
        assert chunks[0, 0, t] == n, (t, chunks[0, 0, t], n)
        assert n_exec[0, 0, t] == ((t + 1) * BM - a) // BN + n
        for r_ in range(BM):
            i = t * BM + r_
            keys = list(range(a, i + 1)) + list(range(n * BN))
            np.testing.assert_allclose(out[0, 0, i], V[0, 0, keys].astype(np.float64).mean(axis=0),
                                       rtol=0, atol=1e-12)


def test_gain_equal_to_tau_does_not_stop():
    """BM = BN = 4, Q = 0, tau = 4/33: in the first tile of a segment the first row holds
    mass 1 after pass 1, so chunk c has gain 4 / (1 + 4*(c+1)), equal to tau at c = 7 (both
    sides are the same double 4/33).  The comparison is strict, so the tile also runs chunk 8
    and stops there (9 of 16 chunks); a tau just above 4/33 stops after chunk 7."""
    N, d, S = 128, 4, 64
    Q = np.zeros((1, 1, N, d), dtype=np.float32)
    K = f32(np.ones((1, 1, N, d)))
    V = f32(np.arange(N * d).reshape(1, 1, N, d))
    p = oracle.problem(1, 1, 1, N, d, "f32", S, 4, 4, 1.0)
    t = S // 4
    lst = np.arange(S, dtype=np.int32)
    tau = 4.0 / 33.0
    _, n_exec, c, gstar = oracle.attn_tile(p, Q, K, V, 0, 0, t, lst, tau)
    assert gstar[7] == tau
    assert c == 9 and n_exec == 1 + 9
    _, _, c2, _ = oracle.attn_tile(p, Q, K, V, 0, 0, t, lst, tau * (1 + 2 ** -40))
    assert c2 == 8


def test_tau_at_least_one_runs_exactly_one_chunk():
    """The gain is below 1 because pass 1 always holds positive mass, so tau >= 1 stops after
    the first chunk."""
    Q, K, V = random_inputs(1, 2, 1, 256, 16, seed=31)
    p = oracle.problem(1, 2, 1, 256, 16, "f32", 64, 16, 8, 0.25)
    for tau in (1.0, 7.5):
        _, _, chunks, _ = run_all(p, Q, K, V, tau)
        for t in range(256 // 16):
            assert np.all(chunks[:, :, t] == (1 if t * 16 >= 64 else 0))


# ------------------------------------------------ output given the executed set --

def executed_keys(p, lst, t, i, chunks):
    a = (t * p.tile_m // p.seg_len) * p.seg_len
    return np.array(list(range(a, i + 1)) + list(lst[:chunks * p.tile_n]), dtype=np.int64)


@pytest.mark.parametrize("tau", [3e-2, 0.1, 0.3])
def test_output_is_softmax_restricted_to_executed_keys(tau):
    Q, K, V = random_inputs(1, 2, 1, 256, 16, seed=41, n_stripes=10)
    p = oracle.problem(1, 2, 1, 256, 16, "f32", 64, 16, 8, 0.25)
    out, _, chunks, r = run_all(p, Q, K, V, tau)
    Qd, Kd, Vd = widen(Q, p), widen(K, p), widen(V, p)
    stopped = 0
    for n, (b, h, t) in enumerate(tiles_of(p)):
        c = r["chunks"][n]
        a = oracle.seg_start(p, t)
        stopped += c < a // p.tile_n
        for r_ in range(p.tile_m):
            i = t * p.tile_m + r_
            ks = executed_keys(p, r["lists"][n], t, i, c)
            x = p.scale * (Kd[b, 0, ks] @ Qd[b, h, i])
            w = np.exp(x - x.max())
            np.testing.assert_allclose(out[b, h, i], (w / w.sum()) @ Vd[b, 0, ks], rtol=0, atol=1e-12)
    assert stopped > 0  # the stop rule fired somewhere


def test_constant_and_one_hot_values():
    N, d = 64, 64
    Q, K, _ = random_inputs(1, 1, 1, N, d, seed=51)
    p = oracle.problem(1, 1, 1, N, d, "f32", 16, 8, 4, 0.125)
    Vc = f32(np.tile(np.linspace(-1, 1, d), (1, 1, N, 1)))
    out, _, _, _ = run_all(p, Q, K, Vc, 0.1)
    np.testing.assert_allclose(out, np.broadcast_to(Vc.astype(np.float64), out.shape), atol=1e-12)
    # one-hot V: output row i is the vector of restricted probabilities over keys
    Vh = f32(np.eye(N, d).reshape(1, 1, N, d))
    out, _, _, r = run_all(p, Q, K, Vh, 0.1)
    Qd, Kd = Q.astype(np.float64), K.astype(np.float64)
    for n, (b, h, t) in enumerate(tiles_of(p)):
        for r_ in range(p.tile_m):
            i = t * p.tile_m + r_
            ks = executed_keys(p, r["lists"][n], t, i, r["chunks"][n])
            x = p.scale * (Kd[0, 0, ks] @ Qd[0, 0, i])
            w = np.exp(x - x.max())
            want = np.zeros(d)
            want[ks] = w / w.sum()
            np.testing.assert_allclose(out[0, 0, i], want, atol=1e-12)


# ---------------------------------------------------------- skipped-mass bounds --

def skipped_fraction(p, Qd, Kd, b, h, g, i, ks):
    x = p.scale * (Kd[b, g, :i + 1] @ Qd[b, h, i])
    w = np.exp(x - x.max())
    kept = np.zeros(i + 1, dtype=bool)
    kept[ks] = True
    return w[~kept].sum() / w.sum()


@pytest.mark.parametrize("tau", [3e-3, 3e-2, 0.3])
def test_skipped_mass_bound_b1(tau):
    """Both outputs are convex combinations of value rows, so per coordinate
    |O_s2o - O_dense| <= rho_i * (max_j V_jk - min_j V_jk), rho_i = skipped true mass."""
    Q, K, V = random_inputs(1, 2, 2, 256, 16, seed=61)
    p = oracle.problem(1, 2, 2, 256, 16, "f32", 64, 16, 8, 0.25)
    out, _, _, r = run_all(p, Q, K, V, tau)
    ref = sdpa_fp64(p, Q, K, V)
    Qd, Kd, Vd = widen(Q, p), widen(K, p), widen(V, p)
    for n, (b, h, t) in enumerate(tiles_of(p)):
        for r_ in range(0, p.tile_m, 5):
            i = t * p.tile_m + r_
            ks = executed_keys(p, r["lists"][n], t, i, r["chunks"][n])
            rho = skipped_fraction(p, Qd, Kd, b, h, h, i, ks)
            span = Vd[b, h, :i + 1].max(axis=0) - Vd[b, h, :i + 1].min(axis=0)
            assert np.all(np.abs(out[b, h, i] - ref[b, h, i]) <= rho * span + 1e-12)


@pytest.mark.parametrize("tau", [1e-2, 5e-2, 0.2])
def test_skipped_mass_bound_b2_single_row_tiles(tau):
    """BM = 1: the list follows the row's own logit order, so every later chunk holds no more
    mass than the stopping chunk, which held less than tau * l.  Hence rho < (C - n) * tau."""
    Q, K, V = random_inputs(1, 1, 1, 128, 8, seed=71)
    p = oracle.problem(1, 1, 1, 128, 8, "f32", 32, 1, 4, 0.35)
    out, _, chunks, r = run_all(p, Q, K, V, tau)
    Qd, Kd = widen(Q, p), widen(K, p)
    fired = 0
    for n, (b, h, t) in enumerate(tiles_of(p)):
        a = oracle.seg_start(p, t)
        C, c = a // p.tile_n, r["chunks"][n]
        ks = executed_keys(p, r["lists"][n], t, t, c)
        rho = skipped_fraction(p, Qd, Kd, 0, 0, 0, t, ks)
        if c < C:
            fired += 1
            assert rho < (C - c) * tau * (1 + 1e-5)
        else:
            assert rho == 0.0
    assert fired > 0


def test_force_n_runs_the_requested_chunk_count():
    Q, K, V = random_inputs(1, 1, 1, 256, 16, seed=81)
    p = oracle.problem(1, 1, 1, 256, 16, "f32", 64, 16, 8, 0.25)
    t = 13
    s = oracle.score_tile(p, Q, K, 0, 0, t)
    lst = oracle.order(s)
    for fn in (1, 3, 24):
        out, n_exec, c, gstar = oracle.attn_tile(p, Q, K, V, 0, 0, t, lst, 10.0, force_n=fn)
        assert c == fn and len(gstar) == fn
        Qd, Kd, Vd = widen(Q, p), widen(K, p), widen(V, p)
        for r_ in (0, 15):
            i = t * 16 + r_
            ks = executed_keys(p, lst, t, i, fn)
            x = p.scale * (Kd[0, 0, ks] @ Qd[0, 0, i])
            w = np.exp(x - x.max())
            np.testing.assert_allclose(out[r_], (w / w.sum()) @ Vd[0, 0, ks], atol=1e-12)


# ------------------------------------------------------------ segment lists ---
# One list per (b, h, segment), shared by the segment's tiles and scored against
# the segment's representative query (gist.science summary, "Classement par
# Segment": history keys are scored against a representative query of the
# segment).

@pytest.mark.parametrize("geom", GEOMS)
def test_segment_lists_tau_zero_equals_dense_attention(geom):
    B, Hq, Hkv, N, d, S, BM, BN, dt = geom
    Q, K, V = random_inputs(B, Hq, Hkv, N, d, seed=121 + N, dtype=dt)
    p = oracle.problem(B, Hq, Hkv, N, d, dt, S, BM, BN, 1 / np.sqrt(d), per_segment=True)
    out, _, chunks, _ = run_all(p, Q, K, V, 0.0)
    np.testing.assert_allclose(out, sdpa_fp64(p, Q, K, V), rtol=0, atol=1e-12)


def test_segment_list_layout_and_sharing():
    """Offsets walk (b, h, segment); every tile of a segment uses the same list, equal to
    the order of the segment representative's scores."""
    Q, K, V = random_inputs(2, 4, 2, 200, 16, seed=13)
    S, BM = 48, 8
    p = oracle.problem(2, 4, 2, 200, 16, "f32", S, BM, 8, 0.25, per_segment=True)
    nseg = (200 + S - 1) // S
    L = sum(s * S for s in range(nseg))
    assert oracle.list_entries(p) == 2 * 4 * L
    scores = oracle.scores_all(p, Q, K)
    lists = oracle.lists_all(p, scores)
    T = 200 // BM
    for b in (0, 1):
        for h in (0, 3):
            for t in range(T):
                s = t * BM // S
                off = oracle.list_offset(p, b, h, t)
                assert off == (b * 4 + h) * L + S * s * (s - 1) // 2
                a = oracle.seg_start(p, t)
                sc = oracle.score_tile(p, Q, K, b, h, t)
                assert np.array_equal(scores[off:off + a], sc)
                assert np.array_equal(lists[off:off + a], oracle.order(sc))


def test_segment_representative_is_the_mean_of_its_rows():
    """fp64 mean of the segment's rows, within the two-level fp32 summation bound; the
    last (partial) segment averages only its own tiles."""
    Q, _, _ = random_inputs(1, 2, 1, 200, 16, seed=17, dtype="bf16")
    S, BM = 48, 8
    p = oracle.problem(1, 2, 1, 200, 16, "bf16", S, BM, 8, 0.25, per_segment=True)
    Qd = widen(Q, p)
    u = 2.0 ** -24
    for h in range(2):
        for t in (6, 7, 12, 24):
            s0 = t * BM // S * S
            s1 = min(s0 + S, 200)
            rows = Qd[0, h, s0:s1]
            got = oracle.rep_query(p, Q, 0, h, t).astype(np.float64)
            bound = 4 * (BM + (s1 - s0) // BM) * u * np.abs(rows).mean(axis=0) + 1e-30
            assert np.all(np.abs(got - rows.mean(axis=0)) <= bound)


def test_segment_representative_exact_on_dyadic_inputs():
    """Constant integer rows per tile and a power-of-two tile count: every fp32 operation
    is exact, so the representative equals the exact mean of the tile values."""
    N, d, BM, S = 128, 4, 8, 32
    rng = np.random.default_rng(2)
    vals = rng.integers(-6, 7, size=(N // BM, d)).astype(np.float32)
    Q = np.repeat(vals, BM, axis=0).reshape(1, 1, N, d).astype(np.float32)
    p = oracle.problem(1, 1, 1, N, d, "f32", S, BM, 8, 1.0, per_segment=True)
    for t in range(N // BM):
        first = t * BM // S * (S // BM)
        want = [Fraction(int(x)) for x in vals[first:first + S // BM].astype(np.int64).sum(axis=0)]
        want = [w / (S // BM) for w in want]
        assert [Fraction(float(x)) for x in oracle.rep_query(p, Q, 0, 0, t)] == want


# ------------------------------------------------------- shared (GQA) lists ---
# One list per KV head (per tile or per segment), read by the G query heads of
# the group and ranked against the mean of their representatives: KV_perm's
# index map shared at the granularity at which the heads share K and V
# (gist.science summary, "Classement par Segment").

@pytest.mark.parametrize("geom", GEOMS)
def test_shared_lists_tau_zero_equals_dense_attention(geom):
    B, Hq, Hkv, N, d, S, BM, BN, dt = geom
    Q, K, V = random_inputs(B, Hq, Hkv, N, d, seed=141 + N, dtype=dt)
    for per_segment in (False, True):
        p = oracle.problem(B, Hq, Hkv, N, d, dt, S, BM, BN, 1 / np.sqrt(d), per_segment=per_segment,
                           share_gqa=True)
        out, _, _, _ = run_all(p, Q, K, V, 0.0)
        np.testing.assert_allclose(out, sdpa_fp64(p, Q, K, V), rtol=0, atol=1e-12)


@pytest.mark.parametrize("per_segment", [False, True])
def test_shared_list_layout_and_sharing(per_segment):
    """Offsets walk (b, KV head, list); every query head of a group reads the same list,
    the order of the group representative's scores."""
    B, Hq, Hkv, N, d, S, BM = 2, 4, 2, 200, 16, 48, 8
    Q, K, V = random_inputs(B, Hq, Hkv, N, d, seed=19)
    p = oracle.problem(B, Hq, Hkv, N, d, "f32", S, BM, 8, 0.25, per_segment=per_segment, share_gqa=True)
    ph = oracle.problem(B, Hq, Hkv, N, d, "f32", S, BM, 8, 0.25, per_segment=per_segment)
    L = oracle.list_entries(ph) // (B * Hq)
    assert oracle.list_entries(p) == B * Hkv * L
    scores = oracle.scores_all(p, Q, K)
    lists = oracle.lists_all(p, scores)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            for t in range(N // BM):
                off = oracle.list_offset(p, b, h, t)
                assert off == (b * Hkv + h // G) * L + oracle.list_offset(ph, 0, 0, t)
                a = oracle.seg_start(p, t)
                sc = oracle.score_tile(p, Q, K, b, h, t)
                assert np.array_equal(scores[off:off + a], sc)
                assert np.array_equal(lists[off:off + a], oracle.order(sc))
                assert np.array_equal(oracle.rep_query(p, Q, b, h, t), oracle.rep_query(p, Q, b, h // G * G, t))


def test_shared_representative_exact_on_dyadic_inputs():
    """Constant integer rows per (head, tile), four heads per group and power-of-two
    counts: every fp32 operation is exact, so the representative is the exact mean of
    the group's tile values (per tile) or of its segment means (per segment)."""
    Hq, Hkv, N, d, BM, S = 8, 2, 128, 4, 8, 32
    rng = np.random.default_rng(4)
    vals = rng.integers(-6, 7, size=(Hq, N // BM, d)).astype(np.float32)
    Q = np.repeat(vals, BM, axis=1).reshape(1, Hq, N, d).astype(np.float32)
    G = Hq // Hkv
    for per_segment in (False, True):
        p = oracle.problem(1, Hq, Hkv, N, d, "f32", S, BM, 8, 1.0, per_segment=per_segment, share_gqa=True)
        for h in (0, 5):
            for t in range(N // BM):
                heads = range(h // G * G, h // G * G + G)
                if per_segment:
                    first = t * BM // S * (S // BM)
                    tiles = range(first, first + S // BM)
                else:
                    tiles = [t]
                want = [sum(Fraction(int(vals[hh, tt, k])) for hh in heads for tt in tiles) /
                        (G * len(tiles)) for k in range(d)]
                assert [Fraction(float(x)) for x in oracle.rep_query(p, Q, 0, h, t)] == want


def test_shared_lists_with_one_head_per_group_equal_per_head_lists():
    """G = 1: the shared form is the per-head form, bit for bit."""
    Q, K, V = random_inputs(1, 2, 2, 256, 16, seed=23, dtype="bf16")
    for per_segment in (False, True):
        a = oracle.problem(1, 2, 2, 256, 16, "bf16", 64, 16, 16, 0.25, per_segment=per_segment)
        s = oracle.problem(1, 2, 2, 256, 16, "bf16", 64, 16, 16, 0.25, per_segment=per_segment, share_gqa=True)
        assert oracle.list_entries(a) == oracle.list_entries(s)
        assert np.array_equal(oracle.scores_all(a, Q, K).view(np.uint32), oracle.scores_all(s, Q, K).view(np.uint32))


# ------------------------------------------------------------- block lists ---
# List entries are blocks of BN consecutive keys, scored with the block's mean
# key; pass-2 chunk c is the c-th listed block.  The pages contrast S2O's
# token-level ordering with block-level sparse attention (authors' abstract;
# gist.science summary, "Signification et Revendications"), so the block form is
# the counterpart used for that comparison.

@pytest.mark.parametrize("geom", GEOMS)
def test_block_lists_tau_zero_equals_dense_attention(geom):
    B, Hq, Hkv, N, d, S, BM, BN, dt = geom
    Q, K, V = random_inputs(B, Hq, Hkv, N, d, seed=131 + N, dtype=dt)
    for per_segment in (False, True):
        p = oracle.problem(B, Hq, Hkv, N, d, dt, S, BM, BN, 1 / np.sqrt(d), per_segment=per_segment,
                           block_lists=True)
        out, _, _, _ = run_all(p, Q, K, V, 0.0)
        np.testing.assert_allclose(out, sdpa_fp64(p, Q, K, V), rtol=0, atol=1e-12)


def test_block_list_layout():
    """A block list has a_t / BN entries; offsets walk (b, h, t) over those lengths."""
    S, BM, BN, N = 48, 8, 4, 200
    p = oracle.problem(2, 4, 2, N, 16, "f32", S, BM, BN, 0.25, block_lists=True)
    T = N // BM
    lens = [(t * BM // S) * S // BN for t in range(T)]
    assert oracle.list_entries(p) == 2 * 4 * sum(lens)
    for b, h, t in [(0, 0, 0), (0, 3, 7), (1, 2, 24), (1, 3, T - 1)]:
        assert oracle.list_len(p, t) == lens[t]
        assert oracle.list_offset(p, b, h, t) == (b * 4 + h) * sum(lens) + sum(lens[:t])


def test_block_mean_exact_on_dyadic_inputs():
    """Small integer keys: every fp32 partial sum is exact and BN is a power of two, so the
    block mean is the exact mean."""
    N, d, BN = 256, 8, 16
    rng = np.random.default_rng(4)
    K = rng.integers(-40, 41, size=(1, 2, N, d)).astype(np.float32)
    p = oracle.problem(1, 2, 2, N, d, "f32", 64, 16, BN, 1.0, block_lists=True)
    for g in range(2):
        for c in (0, 3, N // BN - 1):
            want = [Fraction(int(x), BN) for x in K[0, g, c * BN:(c + 1) * BN].astype(np.int64).sum(axis=0)]
            assert [Fraction(float(x)) for x in oracle.pool_block(p, K, 0, g, c)] == want


def test_block_scores_of_block_constant_keys_match_key_scores():
    """Keys constant within each block: the block mean is that key exactly, so each block
    score equals the score of any of its keys, and the block order expanded to keys is the
    key order (ties inside a block go to the lower index in both)."""
    B, Hq, Hkv, N, d, S, BM, BN = 1, 2, 1, 512, 16, 128, 32, 16
    rng = np.random.default_rng(6)
    Kb = (rng.integers(-20, 21, size=(N // BN, d)) / 8).astype(np.float32)  # block sums exact
    K = np.repeat(Kb, BN, axis=0).reshape(1, 1, N, d)
    Q = rng.standard_normal((1, Hq, N, d)).astype(np.float32)
    V = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    pk = oracle.problem(B, Hq, Hkv, N, d, "f32", S, BM, BN, 0.25)
    pb = oracle.problem(B, Hq, Hkv, N, d, "f32", S, BM, BN, 0.25, block_lists=True)
    for h in range(Hq):
        for t in (4, 9, 15):
            sk = oracle.score_tile(pk, Q, K, 0, h, t)
            sb = oracle.score_tile(pb, Q, K, 0, h, t)
            assert np.array_equal(sb, sk[::BN])
            lk = oracle.order(sk)
            lb = oracle.order(sb)
            assert np.array_equal((lb[:, None] * BN + np.arange(BN)).ravel(), lk)
    ok, nk, _, _ = run_all(pk, Q, K, V, 0.01)
    ob, nb, _, _ = run_all(pb, Q, K, V, 0.01)
    assert np.array_equal(ok, ob) and np.array_equal(nk, nb)


@pytest.mark.parametrize("BM,BN,S,N,tau", [(16, 8, 64, 256, 0.05), (8, 4, 32, 256, 0.1),
                                           (16, 16, 32, 256, 1.0)])
def test_block_lists_q_zero_closed_form(BM, BN, S, N, tau):
    """Q = 0: every block scores 0, the block list ascends, so the visited keys and the
    stop follow the same closed form as key lists."""
    d = 4
    rng = np.random.default_rng(BM * 100 + BN)
    Q = np.zeros((1, 1, N, d), dtype=np.float32)
    K = f32(rng.standard_normal((1, 1, N, d)))
    V = f32(rng.standard_normal((1, 1, N, d)))
    p = oracle.problem(1, 1, 1, N, d, "f32", S, BM, BN, 0.5, block_lists=True)
    out, n_exec, chunks, r = run_all(p, Q, K, V, tau)
    for t in range(N // BM):
        a, n = q_zero_prediction(BM, BN, S, t, tau)
        assert np.array_equal(r["lists"][t, :a // BN], np.arange(a // BN))
        assert chunks[0, 0, t] == n and n_exec[0, 0, t] == ((t + 1) * BM - a) // BN + n
        for r_ in (0, BM - 1):
            i = t * BM + r_
            keys = list(range(a, i + 1)) + list(range(n * BN))
            np.testing.assert_allclose(out[0, 0, i], V[0, 0, keys].astype(np.float64).mean(axis=0),
                                       rtol=0, atol=1e-12)


def test_block_scores_exact_on_dyadic_inputs():
    """Constant integer query rows and small integer keys that vary inside each block:
    the pooled query, the block means and every fma step are exact, so each block score is
    the exact dot product of the query with the block's mean key."""
    N, d, BM, BN, S = 256, 8, 16, 16, 64
    rng = np.random.default_rng(8)
    K = rng.integers(-8, 9, size=(1, 1, N, d)).astype(np.float32)
    qrow = rng.integers(-3, 4, size=d).astype(np.float32)
    Q = np.tile(qrow, (1, 1, N, 1)).astype(np.float32)
    p = oracle.problem(1, 1, 1, N, d, "f32", S, BM, BN, 1.0, block_lists=True)
    for t in (4, 8, 15):
        a = t * BM // S * S
        got = oracle.score_tile(p, Q, np.ascontiguousarray(K), 0, 0, t)
        assert len(got) == a // BN
        for c in range(a // BN):
            block = K[0, 0, c * BN:(c + 1) * BN].astype(np.int64)
            want = sum(Fraction(int(qrow[k])) * Fraction(int(block[:, k].sum()), BN) for k in range(d))
            assert Fraction(float(got[c])) == want


# ------------------------------------------------------------------- Q_perm ---
# Inside each segment the query rows are ordered by their score against a shared
# guide vector, and query tiles are formed from that order (gist.science
# summary, "Classement par Segment", Q_perm).  Reading: the guide is the
# segment's mean key; each row keeps its own causal window in pass 1.

QP_GEOMS = [
    # B, Hq, Hkv, N, d, S, BM, BN, dtype
    (1, 1, 1, 256, 16, 64, 16, 8, "f32"),
    (2, 4, 2, 192, 8, 64, 8, 4, "f32"),     # GQA, batch 2
    (1, 2, 1, 200, 8, 48, 8, 8, "bf16"),    # ragged last segment
    (1, 2, 2, 256, 32, 64, 64, 64, "bf16"), # tile = segment
]


@pytest.mark.parametrize("geom", QP_GEOMS)
def test_qperm_tau_zero_equals_dense_attention(geom):
    """Every row still sees exactly its causal prefix, whatever tile it lands in."""
    B, Hq, Hkv, N, d, S, BM, BN, dt = geom
    Q, K, V = random_inputs(B, Hq, Hkv, N, d, seed=151 + N, dtype=dt)
    ref = sdpa_fp64(oracle.problem(B, Hq, Hkv, N, d, dt, S, BM, BN, 1 / np.sqrt(d)), Q, K, V)
    for per_segment in (False, True):
        p = oracle.problem(B, Hq, Hkv, N, d, dt, S, BM, BN, 1 / np.sqrt(d), per_segment=per_segment,
                           qperm=True)
        T = N // BM
        r = oracle.attn_tiles(p, Q, K, V, tiles_of(p), 0.0)
        out = np.empty((B, Hq, N, d))
        for n, (b, h, t) in enumerate(tiles_of(p)):
            out[b, h, r["rows"][n]] = r["out"][n]
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_qperm_rows_partition_each_segment_in_score_order():
    """The tiles of a segment hold every row of it exactly once, in Python's
    (score descending, row ascending) order of the query scores."""
    B, Hq, Hkv, N, d, S, BM = 1, 2, 1, 200, 8, 48, 8
    Q, K, _ = random_inputs(B, Hq, Hkv, N, d, seed=9, dtype="bf16")
    p = oracle.problem(B, Hq, Hkv, N, d, "bf16", S, BM, 8, 0.25, qperm=True)
    for h in range(Hq):
        for s in range((N + S - 1) // S):
            a, e = s * S, min(N, (s + 1) * S)
            sc = oracle.query_scores(p, Q, K, 0, h, s)
            want = a + np.array(sorted(range(e - a), key=lambda i: (-float(sc[i]), i)))
            got = np.concatenate([oracle.tile_rows(p, Q, K, 0, h, t) for t in range(a // BM, e // BM)])
            assert np.array_equal(got, want)


def test_qperm_guide_and_scores_exact_on_dyadic_inputs():
    """Small integer keys and queries with a power-of-two segment: the guide is the
    exact mean key and every query score the exact dot product with it."""
    N, d, S, BM, Hq = 128, 8, 64, 16, 2
    rng = np.random.default_rng(10)
    K = rng.integers(-8, 9, size=(1, 1, N, d)).astype(np.float32)
    Q = rng.integers(-3, 4, size=(1, Hq, N, d)).astype(np.float32)
    p = oracle.problem(1, Hq, 1, N, d, "f32", S, BM, 8, 1.0, qperm=True)
    for s in range(N // S):
        keys = K[0, 0, s * S:(s + 1) * S].astype(np.int64)
        gd = [Fraction(int(keys[:, k].sum()), S) for k in range(d)]
        assert [Fraction(float(x)) for x in oracle.guide(p, K, 0, 0, s)] == gd
        for h in range(Hq):
            sc = oracle.query_scores(p, Q, K, 0, h, s)
            for i in range(0, S, 7):
                want = sum(Fraction(int(Q[0, h, s * S + i, k])) * gd[k] for k in range(d))
                assert Fraction(float(sc[i])) == want


def test_qperm_with_tied_scores_is_the_identity():
    """Keys whose first four dimensions cancel in pairs give a guide that is exactly zero
    there; queries living only in those dimensions then all score exactly 0, so Q_perm
    keeps the row order and reproduces the unpermuted lists, counts and outputs exactly
    (while the attention itself, q . k over those dimensions, is not trivial)."""
    B, Hq, Hkv, N, d, S, BM, BN = 1, 2, 1, 256, 8, 64, 16, 8
    rng = np.random.default_rng(11)
    K = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    K[0, 0, 1::2, :4] = -K[0, 0, 0::2, :4]        # pairs cancel exactly in the running sum
    Q = np.zeros((1, Hq, N, d), np.float32)
    Q[..., :4] = rng.standard_normal((1, Hq, N, 4))
    V = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    p0 = oracle.problem(B, Hq, Hkv, N, d, "f32", S, BM, BN, 0.5)
    p1 = oracle.problem(B, Hq, Hkv, N, d, "f32", S, BM, BN, 0.5, qperm=True)
    for s_ in range(N // S):
        assert not np.any(oracle.guide(p1, K, 0, 0, s_)[:4])
        for h in range(Hq):
            assert not np.any(oracle.query_scores(p1, Q, K, 0, h, s_))
    o0, n0, _, _ = run_all(p0, Q, K, V, 0.02)
    o1, n1, _, _ = run_all(p1, Q, K, V, 0.02)
    assert np.array_equal(o0, o1) and np.array_equal(n0, n1)
    assert np.any(n0 != n0.max())                  # the stop rule did fire somewhere
    s0, s1 = oracle.scores_all(p0, Q, K), oracle.scores_all(p1, Q, K)
    assert np.array_equal(s0, s1[:len(s0)])


def test_qperm_pass1_window_and_layout():
    """Pass 1 of a permuted tile covers key tiles up to its last row; the query orders
    follow every key list, one run of N rows per (b, h)."""
    B, Hq, Hkv, N, d, S, BM, BN = 1, 1, 1, 128, 8, 64, 16, 8
    Q, K, V = random_inputs(B, Hq, Hkv, N, d, seed=12)
    p = oracle.problem(B, Hq, Hkv, N, d, "f32", S, BM, BN, 0.3, qperm=True)
    pk = oracle.problem(B, Hq, Hkv, N, d, "f32", S, BM, BN, 0.3)
    assert oracle.list_entries(p) == oracle.list_entries(pk) + N
    assert oracle.query_list_offset(p, 0, 0, 1) == oracle.list_entries(pk) + S
    r = oracle.attn_tiles(p, Q, K, V, tiles_of(p), 1.0)   # tau >= 1: exactly one pass-2 chunk
    for n, (_, _, t) in enumerate(tiles_of(p)):
        a = t * BM // S * S
        p1 = (int(r["rows"][n].max()) + 1 - a + BN - 1) // BN
        assert r["n_exec"][n] == p1 + (1 if a > 0 else 0)
