"""Pins of the block-causal oracle (forward and gradients) against independent facts.

- the forward equals the per-chunk inference calls of the Rollout model (a
  separate construction of each chunk's keys, through the Tail_H bank);
- the gradients equal central finite differences of sum(dO * O);
- identities of softmax attention: the key gradients of one query sum to
  zero, the value gradients sum to the output gradient;
- closed forms with constant keys (uniform attention);
- block causality: a key receives gradient only from the chunks that read it.
CPU only.
"""
import numpy as np
import pytest

import oracle as orc


def tiny_cfg(**kw):
    base = dict(tokens_per_latent=2, n_heads=2, head_dim=4, n_latents=24, history=2)
    base.update(kw)
    return orc.FFConfig(**base)


def rand_inputs(cfg, seed=0, const_keys=False):
    rng = np.random.default_rng(seed)
    na, nc = orc.n_anchors(cfg), orc.n_chunks(cfg)
    T, L, nh, d = cfg.tokens_per_latent, cfg.chunk_tokens, cfg.n_heads, cfg.head_dim
    Ka = rng.standard_normal((na * T, nh, d))
    Va = rng.standard_normal((na * T, nh, d))
    Q = rng.standard_normal((nc * L, nh, d))
    K = rng.standard_normal((nc * L, nh, d))
    V = rng.standard_normal((nc * L, nh, d))
    dO = rng.standard_normal((nc * L, nh, d))
    if const_keys:
        k0 = rng.standard_normal((1, nh, d))
        Ka[:] = k0
        K[:] = k0
    return Ka, Va, Q, K, V, dO


# --------------------------------------------------------------------------
# Forward: same keys as the per-chunk calls (reading R13, [S] Eq. (2))
# --------------------------------------------------------------------------
CONFIGS = [
    dict(tokens_per_latent=3, n_heads=2, head_dim=8),                              # 81 latents, H = 5
    dict(tokens_per_latent=2, n_heads=1, head_dim=4, n_latents=36, history=2),
    dict(tokens_per_latent=2, n_heads=2, head_dim=4, n_latents=36, w_ctx=11),      # cap binds
    dict(tokens_per_latent=2, n_heads=2, head_dim=4, gamma_rule=orc.GAMMA_CENTER_LR),
    dict(tokens_per_latent=1, n_heads=1, head_dim=4, n_latents=261),               # 65 s clip
]


@pytest.mark.parametrize("kw", CONFIGS)
def test_forward_equals_per_chunk_calls(kw):
    cfg = orc.FFConfig(**kw)
    Ka, Va, Q, K, V, _ = rand_inputs(cfg, seed=1)
    O, LSE = orc.bc_forward(cfg, Ka, Va, Q, K, V)
    ro = orc.Rollout(cfg)
    T, L = cfg.tokens_per_latent, cfg.chunk_tokens
    for blk in orc.planner_blocks(cfg):
        r = slice(blk[0] * T, (blk[-1] + 1) * T)
        ro.publish_anchors(blk[0], Ka[r], Va[r])
    for i in range(orc.n_chunks(cfg)):
        r = slice(i * L, (i + 1) * L)
        Oi, LSEi = ro.render_attend(i, 0, Q[r], K[r], V[r])
        np.testing.assert_allclose(O[r], Oi, rtol=0, atol=1e-12)
        np.testing.assert_allclose(LSE[i], LSEi, rtol=0, atol=1e-12)


def test_key_budget_at_pages_hyper_parameters():
    """H = 5, B_R = 3 and at most 3 anchors give at most 21 = W_ctx key latents."""
    cfg = orc.FFConfig(tokens_per_latent=1, n_heads=1, head_dim=1)
    lat = []
    for i in range(orc.n_chunks(cfg)):
        src = orc.bc_key_sources(cfg, i)
        lat.append(sum(1 if k == "anchor" else 3 for k, _ in src))
    assert max(lat) == 21 and lat[0] == 2 + 3 and lat[5] == 2 + 15 + 3
    # every source is read by some chunk; chunk j's keys by chunks j .. j + H
    m = orc.bc_mask(cfg)
    na = orc.n_anchors(cfg)
    assert m.any(axis=0).all()
    for j in range(orc.n_chunks(cfg)):
        readers = np.nonzero(m[:, na + j])[0].tolist()
        assert readers == list(range(j, min(orc.n_chunks(cfg), j + cfg.history + 1)))


# --------------------------------------------------------------------------
# Gradients
# --------------------------------------------------------------------------
def _loss(cfg, Ka, Va, Q, K, V, dO):
    O, _ = orc.bc_forward(cfg, Ka, Va, Q, K, V)
    return float((dO * O).sum())


@pytest.mark.parametrize("kw", [dict(), dict(w_ctx=8), dict(gamma_rule=orc.GAMMA_CENTER_LR)])
def test_gradients_match_finite_differences(kw):
    cfg = tiny_cfg(**kw)
    Ka, Va, Q, K, V, dO = rand_inputs(cfg, seed=2)
    grads = orc.bc_backward(cfg, Ka, Va, Q, K, V, dO)
    args = [Ka, Va, Q, K, V]
    # bc_backward returns dQ, dK, dV, dKa, dVa
    which = {0: grads[3], 1: grads[4], 2: grads[0], 3: grads[1], 4: grads[2]}
    rng = np.random.default_rng(3)
    eps = 1e-6
    for t in range(5):
        x = args[t]
        for _ in range(12):
            idx = tuple(int(rng.integers(0, s)) for s in x.shape)
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(cfg, *args, dO)
            x[idx] = old - eps
            lm = _loss(cfg, *args, dO)
            x[idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - which[t][idx]) <= 1e-7 + 1e-6 * abs(fd), (t, idx, fd, which[t][idx])


def test_gradient_identities():
    """Per query the softmax weights sum to one: sum_keys dK = 0, sum_keys dV = sum_q dO."""
    cfg = tiny_cfg()
    Ka, Va, Q, K, V, dO = rand_inputs(cfg, seed=4)
    dQ, dK, dV, dKa, dVa = orc.bc_backward(cfg, Ka, Va, Q, K, V, dO)
    np.testing.assert_allclose(dK.sum(0) + dKa.sum(0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dV.sum(0) + dVa.sum(0), dO.sum(0), atol=1e-12)
    for i in range(orc.n_chunks(cfg)):
        dQ1, dK1, dV1, dKa1, dVa1 = orc.bc_backward(cfg, Ka, Va, Q, K, V, dO, chunks=[i])
        L = cfg.chunk_tokens
        np.testing.assert_allclose(dK1.sum(0) + dKa1.sum(0), 0.0, atol=1e-12)
        np.testing.assert_allclose(dV1.sum(0) + dVa1.sum(0), dO[i * L:(i + 1) * L].sum(0), atol=1e-12)


def test_constant_keys_closed_form():
    """Equal keys give uniform weights 1/n: dQ = 0 and dV_j = sum of dO_q / n_q over its readers."""
    cfg = tiny_cfg()
    Ka, Va, Q, K, V, dO = rand_inputs(cfg, seed=5, const_keys=True)
    dQ, dK, dV, dKa, dVa = orc.bc_backward(cfg, Ka, Va, Q, K, V, dO)
    np.testing.assert_allclose(dQ, 0.0, atol=1e-12)
    T, L, H = cfg.tokens_per_latent, cfg.chunk_tokens, cfg.history
    exp_dV = np.zeros_like(dV)
    exp_dVa = np.zeros_like(dVa)
    for i in range(orc.n_chunks(cfg)):
        anchors = orc.gamma(cfg, i)
        chunks = range(max(0, i - H), i + 1)          # uncapped at this W_ctx
        n = len(anchors) * T + len(chunks) * L
        g = dO[i * L:(i + 1) * L].sum(0) / n
        for a in anchors:
            exp_dVa[a * T:(a + 1) * T] += g
        for j in chunks:
            exp_dV[j * L:(j + 1) * L] += g
    np.testing.assert_allclose(dV, exp_dV, atol=1e-12)
    np.testing.assert_allclose(dVa, exp_dVa, atol=1e-12)


def test_block_causality():
    """Output gradient on chunk i reaches only chunk i's queries and its own key sources."""
    cfg = tiny_cfg()
    Ka, Va, Q, K, V, dO = rand_inputs(cfg, seed=6)
    L, T = cfg.chunk_tokens, cfg.tokens_per_latent
    for i in range(orc.n_chunks(cfg)):
        g = np.zeros_like(dO)
        g[i * L:(i + 1) * L] = dO[i * L:(i + 1) * L]
        dQ, dK, dV, dKa, dVa = orc.bc_backward(cfg, Ka, Va, Q, K, V, g)
        rows_q = np.abs(dQ).sum(axis=(1, 2)) > 0
        assert rows_q.tolist() == [i * L <= r < (i + 1) * L for r in range(len(rows_q))]
        read_chunks = set(range(max(0, i - cfg.history), i + 1))
        read_anchors = set(orc.gamma(cfg, i))
        for j in range(orc.n_chunks(cfg)):
            nz = np.abs(dV[j * L:(j + 1) * L]).sum() > 0
            assert nz == (j in read_chunks), (i, j)
        for a in range(orc.n_anchors(cfg)):
            nz = np.abs(dVa[a * T:(a + 1) * T]).sum() > 0
            assert nz == (a in read_anchors), (i, a)


def test_complete_sources_from_a_subset_of_chunks():
    cfg = tiny_cfg()
    Ka, Va, Q, K, V, dO = rand_inputs(cfg, seed=7)
    full = orc.bc_backward(cfg, Ka, Va, Q, K, V, dO)
    # anchor 2 (position 20) is read by chunks 3..7 (positions 9..23); chunk j by j..j+2
    sub_chunks = [3, 4, 5, 6, 7]
    part = orc.bc_backward(cfg, Ka, Va, Q, K, V, dO, chunks=sub_chunks)
    anchors, chunks = orc.bc_complete_sources(cfg, sub_chunks)
    assert chunks == [3, 4, 5, 6, 7] and anchors == [2]
    L, T = cfg.chunk_tokens, cfg.tokens_per_latent
    for j in chunks:
        for f, p in zip(full[1:3], part[1:3]):
            np.testing.assert_allclose(p[j * L:(j + 1) * L], f[j * L:(j + 1) * L], atol=1e-13)
    for a in anchors:
        for f, p in zip(full[3:], part[3:]):
            np.testing.assert_allclose(p[a * T:(a + 1) * T], f[a * T:(a + 1) * T], atol=1e-13)
    np.testing.assert_allclose(part[0][3 * L:], full[0][3 * L:], atol=1e-13)
