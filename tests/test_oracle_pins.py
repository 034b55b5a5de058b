"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these retype the oracle's own formula: each compares it to a value the
pages print (tests/golden), a closed form, a library routine (torch SDPA,
scipy logsumexp), an identity (LSE merge, duplicate keys), or brute-force
enumeration on tiny cases.
"""
import itertools
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle as orc
import synthetic as syn

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def cfg81(**kw):
    base = dict(tokens_per_latent=4, n_heads=2, head_dim=8)
    base.update(kw)
    return orc.FFConfig(**base)


# --------------------------------------------------------------------------
# Worked example of the pages
# --------------------------------------------------------------------------
def test_anchor_positions_and_blocks_match_worked_example(golden):
    g = golden("worked_example_81.txt")
    cfg = cfg81(n_latents=g["n_latents"])
    assert orc.anchor_positions(cfg) == g["anchor_positions"]
    assert orc.n_anchors(cfg) == g["n_anchors"]
    blocks = orc.planner_blocks(cfg)
    assert all(len(b) == g["anchors_per_planner_block"] for b in blocks)
    pos = [[orc.anchor_positions(cfg)[a] for a in b] for b in blocks]
    assert pos == [[0, 10, 20], [30, 40, 50], [60, 70, 80]]


def test_hyper_parameters_match_pages(golden):
    g = golden("worked_example_81.txt")
    cfg = cfg81()
    assert (cfg.planner_block, cfg.chunk_latents, cfg.anchor_stride) == (g["B_P"], g["B_R"], g["Delta"])
    assert (cfg.n_stages, cfg.w_ctx, cfg.history, cfg.planner_history) == (g["S"], g["W_ctx"], g["H"], g["H_P"])


def test_chunks_cover_positions_once(golden):
    g = golden("worked_example_81.txt")
    cfg = cfg81()
    assert orc.n_chunks(cfg) == g["renderer_chunks"]
    seen = []
    for i in range(orc.n_chunks(cfg)):
        p = orc.chunk_positions(cfg, i)
        assert len(p) == g["latents_per_chunk"] and p == list(range(p[0], p[0] + 3))
        seen += p
    assert seen == list(range(g["n_latents"]))


def test_ar_depth_ratio(golden):
    g = golden("worked_example_81.txt")
    d = orc.ar_depth(cfg81())
    assert d["planner_latents_per_step"] == g["planner_latents_per_step"]
    assert d["renderer_latents_per_step"] == g["renderer_latents_per_step"]
    assert d["ratio_per_step"] == 10
    # over the 81-latent clip: 3 planner steps against 27 renderer steps
    assert (d["planner_steps"], d["renderer_steps"]) == (3, 27)


def test_clip_frames_and_long_rollout(golden):
    g = golden("clip_frames.txt")
    # 81 latents <-> 321 frames fixes frames = 4 (L - 1) + 1 (temporal stride 4)
    assert 4 * (g["n_latents"] - 1) + 1 == g["rgb_frames"]
    # 65 s at 16 FPS = 1040 frames -> (1040 - 1) / 4 + 1 = 260.75 -> 261 latents
    L = math.ceil((65 * g["fps"] - 1) / 4 + 1)
    assert L == 261
    cfg = cfg81(n_latents=L)
    assert orc.n_chunks(cfg) == 87 and orc.n_anchors(cfg) == 27
    assert len(orc.planner_blocks(cfg)) == 9
    assert len(orc.schedule(cfg)) == 87 + 4 - 1


# --------------------------------------------------------------------------
# Tail_H bank rule, [S] how it works, Eq. (2)
# --------------------------------------------------------------------------
def _publish_all_anchors(ro, cfg, dtype="f32"):
    for blk in orc.planner_blocks(cfg):
        K, V = syn.anchor_kv(T=cfg.tokens_per_latent, n_heads=cfg.n_heads, head_dim=cfg.head_dim,
                             anchors=blk, dtype=dtype)
        ro.publish_anchors(blk[0], syn.as_f64(K, dtype), syn.as_f64(V, dtype))


def test_tail_h_ids_and_bytes():
    cfg = cfg81(n_stages=2)
    ro = orc.Rollout(cfg)
    _publish_all_anchors(ro, cfg)
    inputs = {}
    for t, diag in enumerate(orc.schedule(cfg)):
        for i, k in diag:
            q, kk, vv = syn.chunk_qkv(T=4, n_heads=2, head_dim=8, chunk=i, stage=k, dtype="bf16")
            inputs[(i, k)] = (kk, vv)
            ro.render_attend(i, k, None, syn.as_f64(kk, "bf16"), syn.as_f64(vv, "bf16"), compute=False)
            ids, Kb, Vb = ro.bank_tail(k)
            # closed form: the last H chunk ids, oldest first
            assert ids == list(range(max(0, i - 4), i + 1))
            assert ids == orc.history_ids_after(cfg, i)
            # contents are exactly the published inputs, in id order
            exp_k = np.concatenate([syn.as_f64(inputs[(c, k)][0], "bf16") for c in ids])
            exp_v = np.concatenate([syn.as_f64(inputs[(c, k)][1], "bf16") for c in ids])
            assert np.array_equal(Kb, exp_k) and np.array_equal(Vb, exp_v)


# --------------------------------------------------------------------------
# Wavefront order
# --------------------------------------------------------------------------
def test_schedule_counts_and_legality(golden):
    cfg = cfg81()
    diags = orc.schedule(cfg)
    assert len(diags) == 27 + 4 - 1 == 30
    calls = [c for d in diags for c in d]
    assert len(calls) == 27 * 4 and len(set(calls)) == 108
    assert all(len(d) <= 4 for d in diags)
    assert orc.is_legal_order(cfg, calls)
    # chunk-major and stage-major orders are also legal, reversed ones are not
    assert orc.is_legal_order(cfg, [(i, k) for i in range(27) for k in range(4)])
    assert orc.is_legal_order(cfg, [(i, k) for k in range(4) for i in range(27)])
    assert not orc.is_legal_order(cfg, [(i, k) for i in range(27) for k in reversed(range(4))])
    assert not orc.is_legal_order(cfg, [(i, k) for i in reversed(range(27)) for k in range(4)])


@pytest.mark.parametrize("nc,S", [(3, 2), (2, 3), (3, 3)])
def test_legal_orders_count_brute_force(nc, S):
    """Brute force: legal orders of an nc x S grid poset = hook-length count of SYT."""
    cfg = orc.FFConfig(tokens_per_latent=1, n_heads=1, head_dim=1, n_latents=3 * nc, n_stages=S)
    calls = [(i, k) for i in range(nc) for k in range(S)]
    n_legal = sum(orc.is_legal_order(cfg, p) for p in itertools.permutations(calls))
    hooks = 1
    for r in range(nc):
        for c in range(S):
            hooks *= (nc - r - 1) + (S - c - 1) + 1
    assert n_legal == math.factorial(nc * S) // hooks


def test_rollout_rejects_out_of_order_calls():
    cfg = cfg81()
    ro = orc.Rollout(cfg)
    z = np.zeros((12, 2, 8))
    with pytest.raises(orc.ContractError):          # anchors of Gamma(0) missing
        ro.render_attend(0, 0, z, z, z, compute=False)
    _publish_all_anchors(ro, cfg)
    with pytest.raises(orc.ContractError):          # chunk 1 before chunk 0
        ro.render_attend(1, 0, z, z, z, compute=False)
    with pytest.raises(orc.ContractError):          # stage 1 before stage 0
        ro.render_attend(0, 1, z, z, z, compute=False)
    ro.render_attend(0, 0, z, z, z, compute=False)
    with pytest.raises(orc.ContractError):          # replay of chunk 0
        ro.render_attend(0, 0, z, z, z, compute=False)
    with pytest.raises(orc.ContractError):          # anchor republished
        K = np.zeros((4, 2, 8))
        ro.publish_anchors(0, K, K)


# --------------------------------------------------------------------------
# Gamma(i) and the W_ctx budget (parity unpinned by the pages; properties only)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("rule", [orc.GAMMA_BRACKET, orc.GAMMA_CENTER_LR])
@pytest.mark.parametrize("L", [81, 261])
def test_gamma_two_sided_and_budget(rule, L):
    cfg = cfg81(n_latents=L, gamma_rule=rule)
    pos = orc.anchor_positions(cfg)
    for i in range(orc.n_chunks(cfg)):
        g = orc.gamma(cfg, i)
        assert g == sorted(set(g)) and 2 <= len(g) <= 3
        ap = [pos[a] for a in g]
        p = orc.chunk_positions(cfg, i)
        if rule == orc.GAMMA_BRACKET:
            # every latent of the chunk has a selected anchor on each side
            assert all(min(ap) <= x <= max(ap) for x in p)
            assert max(ap) - min(ap) <= 2 * cfg.anchor_stride
        else:
            assert len(g) == 2 and ap[0] <= p[1] <= ap[1]
        # key latents never exceed W_ctx = 21, and a full bank reaches 20 or 21
        assert orc.key_latents(cfg, i, min(i, cfg.history)) <= cfg.w_ctx
    lat = [orc.key_latents(cfg, i, cfg.history) for i in range(5, orc.n_chunks(cfg))]
    if rule == orc.GAMMA_BRACKET:
        assert max(lat) == 21 and min(lat) == 20
        three = [i for i in range(orc.n_chunks(cfg)) if len(orc.gamma(cfg, i)) == 3]
        assert three[:3] == [3, 13, 23]
    else:
        assert set(lat) == {20}


def test_w_ctx_cap_drops_oldest_history():
    cfg = cfg81(w_ctx=12, n_stages=1)
    ro = orc.Rollout(cfg)
    _publish_all_anchors(ro, cfg)
    z = np.zeros((12, 2, 8))
    for i in range(7):
        src = ro.key_sources(i, 0)
        lat = sum(1 if s == "anchor" else 3 for s, _ in src)
        assert lat <= 12
        hist = [c for s, c in src if s == "history"]
        assert hist == list(range(i - len(hist), i))   # the newest ones kept
        ro.render_attend(i, 0, z, z, z, compute=False)


# --------------------------------------------------------------------------
# Attention: library routine, closed forms, identities
# --------------------------------------------------------------------------
def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("Lq,Lk,nh,d", [(5, 7, 2, 8), (33, 130, 3, 64), (1, 1, 1, 4)])
def test_attention_vs_torch_sdpa_fp64(Lq, Lk, nh, d):
    Q, K, V = _rand((Lq, nh, d), 1), _rand((Lk, nh, d), 2), _rand((Lk, nh, d), 3)
    O, LSE = orc.attention(Q, K, V, 1.0 / math.sqrt(d))
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2)))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(Q), t(K), t(V))[0].numpy().transpose(1, 0, 2)
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)
    for h in range(nh):
        s = np.einsum("qd,kd->qk", Q[:, h], K[:, h]) / math.sqrt(d)
        np.testing.assert_allclose(LSE[h], logsumexp(s, axis=1), rtol=0, atol=1e-12)


def test_attention_closed_forms():
    d, Lk = 16, 9
    rng = np.random.default_rng(5)
    Q = rng.standard_normal((4, 1, d))
    V = rng.standard_normal((Lk, 1, d))
    k0 = rng.standard_normal((1, 1, d))
    # all keys equal -> O is the mean of V, LSE = s + ln Lk
    K = np.repeat(k0, Lk, axis=0)
    O, LSE = orc.attention(Q, K, V, 0.25)
    np.testing.assert_allclose(O[:, 0], np.broadcast_to(V[:, 0].mean(0), (4, d)), atol=1e-13)
    np.testing.assert_allclose(LSE[0], 0.25 * (Q[:, 0] @ k0[0, 0]) + math.log(Lk), atol=1e-13)
    # constant V -> O is that constant
    O, _ = orc.attention(Q, rng.standard_normal((Lk, 1, d)), np.full((Lk, 1, d), 3.5), 0.25)
    np.testing.assert_allclose(O, 3.5, atol=1e-13)
    # one key -> O = V_0, LSE = s_0
    O, LSE = orc.attention(Q, k0, V[:1], 0.25)
    np.testing.assert_allclose(O[:, 0], np.broadcast_to(V[0, 0], (4, d)), atol=1e-13)
    np.testing.assert_allclose(LSE[0], 0.25 * (Q[:, 0] @ k0[0, 0]), atol=1e-13)
    # zero query -> uniform weights
    O, LSE = orc.attention(np.zeros((2, 1, d)), rng.standard_normal((Lk, 1, d)), V, 0.25)
    np.testing.assert_allclose(O[:, 0], np.broadcast_to(V[:, 0].mean(0), (2, d)), atol=1e-13)
    np.testing.assert_allclose(LSE[0], math.log(Lk), atol=1e-13)
    # one key dominating (orthonormal keys, peaked query) -> O = that V
    K = np.eye(d)[:Lk][:, None, :]
    q = 80.0 * K[6:7]
    O, _ = orc.attention(q, K, V, 1.0)
    np.testing.assert_allclose(O[0, 0], V[6, 0], atol=1e-30 + 1e-12)


def _with_bias(Q, K, bias, scale):
    """Augment head_dim by one so that scale*<Q', K'_j> = scale*<Q,K_j> + bias_j."""
    Qa = np.concatenate([Q, np.ones(Q.shape[:2] + (1,))], axis=2)
    Ka = np.concatenate([K, (np.asarray(bias, dtype=np.float64) / scale).reshape(-1, 1, 1)
                         * np.ones((1, K.shape[1], 1))], axis=2)
    return Qa, Ka


def test_duplicate_key_identity_lemma():
    """n copies of (k, v) equal one copy whose logit is raised by ln n.

    FAST-AR summary page ("Fast Autoregressive Video Diffusion and World
    Models with Temporal Cache Compression and Sparse Attention"), section
    TempCache, Lemma 5.1.
    """
    rng = np.random.default_rng(11)
    d, scale = 8, 0.3
    Q = rng.standard_normal((6, 2, d))
    K = rng.standard_normal((5, 2, d))
    V = rng.standard_normal((5, 2, d))
    n = 4
    Kdup = np.concatenate([K, np.repeat(K[2:3], n - 1, axis=0)])
    Vdup = np.concatenate([V, np.repeat(V[2:3], n - 1, axis=0)])
    O1, L1 = orc.attention(Q, Kdup, Vdup, scale)
    bias = np.zeros(5)
    bias[2] = math.log(n)
    Qa, Ka = _with_bias(Q, K, bias, scale)
    O2, L2 = orc.attention(Qa, Ka, V, scale)
    np.testing.assert_allclose(O1, O2, atol=1e-13)
    np.testing.assert_allclose(L1, L2, atol=1e-13)


def test_shift_and_permutation_invariance():
    rng = np.random.default_rng(12)
    d, scale = 8, 0.4
    Q, K, V = rng.standard_normal((7, 2, d)), rng.standard_normal((11, 2, d)), rng.standard_normal((11, 2, d))
    O, L = orc.attention(Q, K, V, scale)
    perm = rng.permutation(11)
    Op, Lp = orc.attention(Q, K[perm], V[perm], scale)
    np.testing.assert_allclose(O, Op, atol=1e-13)
    np.testing.assert_allclose(L, Lp, atol=1e-13)
    Qa, Ka = _with_bias(Q, K, np.full(11, 2.5), scale)
    Os, Ls = orc.attention(Qa, Ka, V, scale)
    np.testing.assert_allclose(O, Os, atol=1e-13)
    np.testing.assert_allclose(L + 2.5, Ls, atol=1e-12)


def test_lse_merge_of_segments_equals_full():
    rng = np.random.default_rng(13)
    d, scale = 8, 0.35
    Q = rng.standard_normal((9, 2, d))
    segs = [(rng.standard_normal((n, 2, d)), rng.standard_normal((n, 2, d))) for n in (3, 10, 1, 6)]
    O, L = orc.attention(Q, np.concatenate([s[0] for s in segs]), np.concatenate([s[1] for s in segs]), scale)
    parts = [orc.attention(Q, k, v, scale) for k, v in segs]
    Lm = np.logaddexp.reduce(np.stack([p[1] for p in parts]), axis=0)          # [nh, Lq]
    w = np.stack([np.exp(p[1] - Lm) for p in parts])                            # [seg, nh, Lq]
    Om = sum(w[j].T[:, :, None] * parts[j][0] for j in range(len(parts)))
    np.testing.assert_allclose(O, Om, atol=1e-13)
    np.testing.assert_allclose(L, Lm, atol=1e-13)


# --------------------------------------------------------------------------
# The three key sources of a renderer call
# --------------------------------------------------------------------------
def test_key_sources_and_segment_sizes():
    cfg = cfg81(n_stages=1)
    ro = orc.Rollout(cfg)
    _publish_all_anchors(ro, cfg)
    z = np.zeros((12, 2, 8))
    for i in range(orc.n_chunks(cfg)):
        src = ro.key_sources(i, 0)
        kinds = [s for s, _ in src]
        assert kinds == ["anchor"] * len(orc.gamma(cfg, i)) + ["history"] * min(i, 5) + ["own"]
        assert [c for s, c in src if s == "anchor"] == orc.gamma(cfg, i)
        assert [c for s, c in src if s == "history"] == list(range(max(0, i - 5), i))
        Kc, _ = ro.gather_keys(i, 0, z, z)
        assert Kc.shape[0] == 4 * orc.key_latents(cfg, i, min(i, 5))
        ro.render_attend(i, 0, z, z, z, compute=False)


@pytest.mark.parametrize("source", ["anchor0", "anchor1", "hist_oldest", "hist_newest", "own"])
def test_each_source_reaches_the_output(source):
    """A query pointed at one key of one source must return that key's value."""
    cfg = orc.FFConfig(tokens_per_latent=2, n_heads=1, head_dim=64, n_stages=1)
    eye = np.eye(64)
    i = 7
    Ks, Vs = {}, {}
    for c in range(i + 1):                     # one basis direction per recent chunk
        K = np.zeros((6, 1, 64))
        K[0, 0] = eye[c]
        Ks[c], Vs[c] = K, np.full((6, 1, 64), float(c))
    g = orc.gamma(cfg, i)            # positions 21..23 -> anchors at 20 and 30
    ro2 = orc.Rollout(cfg)
    for a in range(orc.n_anchors(cfg)):
        K = np.zeros((2, 1, 64))
        K[0, 0] = eye[40 + a]
        ro2.publish_anchors(a, K, np.full((2, 1, 64), 100.0 + a))
    for c in range(i):
        ro2.render_attend(c, 0, np.zeros((6, 1, 64)), Ks[c], Vs[c], compute=False)
    target = {"anchor0": (eye[40 + g[0]], 100.0 + g[0]), "anchor1": (eye[40 + g[1]], 100.0 + g[1]),
              "hist_oldest": (Ks[i - 5][0, 0], float(i - 5)), "hist_newest": (Ks[i - 1][0, 0], float(i - 1)),
              "own": (Ks[i][0, 0], float(i))}[source]
    Q = np.zeros((6, 1, 64))
    Q[:, 0] = 400.0 * target[0]           # score 50 against 0 for every other key
    O, _ = ro2.render_attend(i, 0, Q, Ks[i], Vs[i])
    np.testing.assert_allclose(O[:, 0, :], target[1], atol=1e-9)


# --------------------------------------------------------------------------
# Planner block attention (readings R11, R12)
# --------------------------------------------------------------------------
def _marker_planner_rollout(cfg, T, d=4):
    """Anchors whose V rows all hold 1 + anchor id; keys all zero."""
    ro = orc.Rollout(cfg)
    return ro, (lambda a: (np.zeros((T, 1, d)), np.full((T, 1, d), 1.0 + a)))


@pytest.mark.parametrize("n_latents,h_p,w_ctx", [(261, 6, 21), (261, 2, 21), (261, 6, 11), (81, 6, 21)])
def test_planner_key_set_closed_form(golden, n_latents, h_p, w_ctx):
    """Zero queries weight every key equally, so O = mean of the key values and
    LSE = ln(number of keys): with one marker value per anchor and a separate
    own value, both identify exactly which anchors block b reads."""
    g = golden("worked_example_81.txt")
    T, d = 2, 4
    cfg = orc.FFConfig(tokens_per_latent=T, n_heads=1, head_dim=d, n_latents=n_latents, planner_history=h_p,
                       w_ctx=w_ctx)
    assert cfg.planner_block == g["B_P"]
    ro = orc.Rollout(cfg)
    blocks = orc.planner_blocks(cfg)
    for b, blk in enumerate(blocks):
        n_own = len(blk) * T
        Q = np.zeros((n_own, 1, d))
        K = np.zeros((n_own, 1, d))
        V = np.full((n_own, 1, d), 1000.0)
        O, LSE = ro.plan_attend(b, Q, K, V)
        # expected key set, written out: the H_P blocks before b, trimmed from
        # the oldest while (their anchors + own latents) exceed W_ctx
        first = max(0, b - h_p)
        while first < b and 3 * (b - first) + len(blk) > w_ctx:
            first += 1
        anchors = [a for x in range(first, b) for a in range(3 * x, 3 * x + 3)]
        n_keys = T * (len(anchors) + len(blk))
        mean = (T * sum(1.0 + a for a in anchors) + n_own * 1000.0) / n_keys
        np.testing.assert_allclose(O, mean, rtol=0, atol=1e-9)
        np.testing.assert_allclose(LSE, math.log(n_keys), rtol=0, atol=1e-12)
        # the cache-extraction call publishes the block with marker values
        Kp = np.zeros((n_own, 1, d))
        Vp = np.concatenate([np.full((T, 1, d), 1.0 + a) for a in blk])
        ro.plan_attend(b, Q, Kp, Vp, publish=True, compute=False)
        for a in blk:
            np.testing.assert_array_equal(ro.anchors[a][1], np.full((T, 1, d), 1.0 + a))


def test_planner_budget_at_pages_hyper_parameters(golden):
    """H_P = 6 blocks of 3 plus the block itself is exactly W_ctx = 21 latents."""
    g = golden("worked_example_81.txt")
    assert g["H_P"] * g["B_P"] + g["B_P"] == g["W_ctx"]
    cfg = orc.FFConfig(tokens_per_latent=2, n_heads=1, head_dim=4, n_latents=261)
    assert orc.planner_key_blocks(cfg, 8) == [2, 3, 4, 5, 6, 7]
    assert orc.planner_key_blocks(cfg, 0) == []


def test_planner_order_contract():
    T, d = 2, 4
    cfg = orc.FFConfig(tokens_per_latent=T, n_heads=1, head_dim=d, n_latents=81)
    ro = orc.Rollout(cfg)
    z = np.zeros((3 * T, 1, d))
    with pytest.raises(orc.ContractError):
        ro.plan_attend(1, z, z, z)                  # block 0 not published
    ro.plan_attend(0, z, z, z)                      # denoising call: publishes nothing
    with pytest.raises(orc.ContractError):
        ro.plan_attend(1, z, z, z)
    with pytest.raises(orc.ContractError):          # renderer chunk 0 needs anchors 0, 1
        ro.render_attend(0, 0, z, z, z)
    ro.plan_attend(0, z, z, z, publish=True)
    with pytest.raises(orc.ContractError):
        ro.plan_attend(0, z, z, z)                  # already published
    ro.render_attend(0, 0, z, z, z)
    with pytest.raises(orc.ContractError):
        ro.plan_attend(3, z, z, z)                  # out of range (3 blocks)


@pytest.mark.parametrize("target", ["oldest", "newest", "own"])
def test_planner_each_source_reaches_the_output(target):
    """A query pointed at one key of one source returns that key's value."""
    T, d = 2, 64
    eye = np.eye(d)
    cfg = orc.FFConfig(tokens_per_latent=T, n_heads=1, head_dim=d, n_latents=261)
    ro = orc.Rollout(cfg)
    b = 7                                           # reads blocks 1..6
    for x in range(b):
        K = np.zeros((3 * T, 1, d))
        V = np.zeros((3 * T, 1, d))
        for j, a in enumerate(range(3 * x, 3 * x + 3)):
            K[j * T, 0] = eye[a]
            V[j * T:(j + 1) * T] = 10.0 + a
        ro.plan_attend(x, np.zeros((3 * T, 1, d)), K, V, publish=True, compute=False)
    Kown = np.zeros((3 * T, 1, d))
    Kown[0, 0] = eye[60]
    Vown = np.full((3 * T, 1, d), 500.0)
    key, val = {"oldest": (eye[3], 13.0), "newest": (eye[20], 30.0), "own": (eye[60], 500.0)}[target]
    Q = np.zeros((3 * T, 1, d))
    Q[:, 0] = 400.0 * key                           # score 50 against 0 for every other key
    O, _ = ro.plan_attend(b, Q, Kown, Vown)
    np.testing.assert_allclose(O[:, 0, :], val, atol=1e-9)
    # block 0's anchors (0..2) are outside the window of block 7
    Q[:, 0] = 400.0 * eye[1]
    O, _ = ro.plan_attend(b, Q, Kown, Vown)
    assert np.all(np.abs(O[:, 0, :] - 1.0 * 11.0) > 1.0)


# --------------------------------------------------------------------------
# The sampled-row path (attention_rows, render_attend / plan_attend with rows=)
# that every full-size GPU parity case compares against
# --------------------------------------------------------------------------
ROW_SETS = {
    "sorted": [0, 3, 4, 17, 31, 32],
    "unsorted": [31, 2, 17, 0, 9],
    "singleton": [13],
    "repeated": [5, 5, 30],
}


@pytest.mark.parametrize("rows", sorted(ROW_SETS))
def test_attention_rows_vs_sdpa_on_the_rows(rows):
    """attention_rows equals torch SDPA (float64, CPU) on exactly the chosen
    query rows, in the order given, and equals the full call restricted to them."""
    r = ROW_SETS[rows]
    Lq, Lk, nh, d = 33, 70, 3, 16
    Q, K, V = _rand((Lq, nh, d), 11), _rand((Lk, nh, d), 12), _rand((Lk, nh, d), 13)
    scale = 1.0 / math.sqrt(d)
    O, LSE = orc.attention_rows(Q, K, V, scale, r)
    assert O.shape == (len(r), nh, d) and LSE.shape == (nh, len(r))
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2)))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(Q[r]), t(K), t(V))[0].numpy().transpose(1, 0, 2)
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)
    for h in range(nh):
        s = Q[r, h] @ K[:, h].T * scale
        np.testing.assert_allclose(LSE[h], logsumexp(s, axis=1), rtol=0, atol=1e-12)
    O_full, LSE_full = orc.attention(Q, K, V, scale)
    np.testing.assert_allclose(O, O_full[r], rtol=0, atol=1e-13)        # BLAS rounding order only
    np.testing.assert_allclose(LSE, LSE_full[:, r], rtol=0, atol=1e-13)


@pytest.mark.parametrize("rows", ["sorted", "unsorted", "singleton"])
def test_render_attend_rows_equal_full_call(rows):
    """Two rollouts in lockstep: the rows= call returns the full call's O rows
    and LSE columns for every call of two stages, and leaves the same banks."""
    cfg = cfg81(n_stages=2)
    r = [x % (3 * cfg.tokens_per_latent) for x in ROW_SETS[rows]]
    full, part = orc.Rollout(cfg), orc.Rollout(cfg)
    _publish_all_anchors(full, cfg)
    _publish_all_anchors(part, cfg)
    for diag in orc.schedule(cfg)[:12]:
        for i, k in diag:
            q, kk, vv = (syn.as_f64(x, "f32") for x in syn.chunk_qkv(
                T=cfg.tokens_per_latent, n_heads=cfg.n_heads, head_dim=cfg.head_dim, chunk=i, stage=k, dtype="f32"))
            O, LSE = full.render_attend(i, k, q, kk, vv)
            Or, LSEr = part.render_attend(i, k, q, kk, vv, rows=r)
            np.testing.assert_allclose(Or, O[r], rtol=0, atol=1e-13)
            np.testing.assert_allclose(LSEr, LSE[:, r], rtol=0, atol=1e-13)
            assert part.bank_tail(k)[0] == full.bank_tail(k)[0]


def test_plan_attend_rows_equal_full_call():
    cfg = cfg81(n_latents=261, n_stages=1)
    T = cfg.tokens_per_latent
    r = [11, 0, 7]
    full, part = orc.Rollout(cfg), orc.Rollout(cfg)
    for b, blk in enumerate(orc.planner_blocks(cfg)):
        q, kk, vv = (syn.as_f64(x, "f32") for x in syn.planner_qkv(
            T=T, n_heads=cfg.n_heads, head_dim=cfg.head_dim, block=b, step=0, n_latents=len(blk), dtype="f32"))
        O, LSE = full.plan_attend(b, q, kk, vv, publish=True)
        Or, LSEr = part.plan_attend(b, q, kk, vv, publish=True, rows=r)
        np.testing.assert_allclose(Or, O[r], rtol=0, atol=1e-13)
        np.testing.assert_allclose(LSEr, LSE[:, r], rtol=0, atol=1e-13)
