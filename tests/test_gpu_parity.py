"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case runs calls in the wavefront order on seeded inputs, compares O and
LSE with the float64 oracle (max-abs 2e-2 for bf16, 1e-4 for fp32, plus a
relative-Frobenius gate) and compares every stage bank's ids and bytes
bit-exactly after every call.  The workspace is filled with NaN first, so a
read of any byte the call should not read (spare ring slot, padding, stale
partials) shows up as a non-finite output.
"""
import numpy as np
import pytest

import oracle as orc
from ffharness import Case, Pair, wavefront

pytestmark = pytest.mark.gpu


def _rollout(case, grouped=False, rows=None, control_from=None, every=1, max_diag=None):
    pr = Pair(case)
    try:
        pr.publish_anchors()
        diags = wavefront(case)
        if max_diag is not None:
            diags = diags[:max_diag]
        for t, diag in enumerate(diags):
            control = control_from is not None and t >= control_from
            if grouped:
                pr.step(diag, grouped=True, rows=rows, control=control)
            else:
                for pair in diag:
                    pr.step([pair], grouped=False, rows=rows, control=control)
        return pr.stats
    finally:
        pr.close()


def test_tiny_fp32_full_rollout():
    """Config: fp32, 2 heads, d=64, T=16, 81 latents, 27 chunks x 4 stages."""
    st = _rollout(Case(T=16, nh=2, d=64, dtype="f32"))
    assert st.calls == 108 and st.bank_checks == 108
    print(f"tiny fp32: max|dO|={st.max_abs:.2e} relF={st.max_rel_fro:.2e} lse={st.max_lse:.2e}")


@pytest.mark.parametrize("rule", [orc.GAMMA_BRACKET, orc.GAMMA_CENTER_LR])
def test_bf16_rollout_multi_tile_ragged(rule):
    """T=200: 600 queries (5 query tiles, ragged), up to 4200 keys (ragged last key tile)."""
    st = _rollout(Case(T=200, nh=2, d=128, S=2, rule=rule), control_from=6)
    assert st.calls == 54
    print(f"bf16 T=200 {rule}: max|dO|={st.max_abs:.2e} relF={st.max_rel_fro:.2e} "
          f"lse={st.max_lse:.2e} control>={st.min_control_ratio:.1f}x")


@pytest.mark.parametrize("n_latents", [3, 9])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_degenerate_short_clips(n_latents, dtype):
    """The shortest clips: one chunk and one anchor (3 latents), three chunks sharing one anchor (9)."""
    st = _rollout(Case(T=16, nh=2, d=128 if dtype == "bf16" else 64, n_latents=n_latents, S=2, dtype=dtype))
    assert st.calls == 2 * (n_latents // 3) and st.bank_checks == st.calls


def test_bf16_head_dim_64_and_peaked_softmax():
    st = _rollout(Case(T=40, nh=3, d=64, S=2, q_scale=8.0))
    assert st.calls == 54
    print(f"bf16 d=64 peaked: max|dO|={st.max_abs:.2e} relF={st.max_rel_fro:.2e}")


def test_bf16_peaked_d128():
    st = _rollout(Case(T=64, nh=2, d=128, S=1, q_scale=8.0), control_from=6)
    print(f"bf16 d=128 peaked: max|dO|={st.max_abs:.2e} relF={st.max_rel_fro:.2e} "
          f"control>={st.min_control_ratio:.1f}x")


def test_grouped_anti_diagonal_long_clip():
    """Grouped launches of whole anti-diagonals (261 latents, 87 chunks, 27 anchors)."""
    st = _rollout(Case(T=24, nh=2, d=128, n_latents=261), grouped=True)
    assert st.calls == 348
    print(f"grouped 261: max|dO|={st.max_abs:.2e} relF={st.max_rel_fro:.2e}")


def test_grouped_bits_equal_single_calls():
    import torch
    case = Case(T=48, nh=3, d=128, S=3)
    outs = {}
    for grouped in (False, True):
        pr = Pair(case, oracle_compute=False)
        try:
            pr.publish_anchors()
            res = {}
            for diag in wavefront(case)[:12]:
                host = [pr.gen(i, k) for i, k in diag]
                from ffharness import to_device
                from chunked_kv_cache_amd import ff
                dev = [[to_device(x, "bf16") for x in h] for h in host]
                o = [torch.empty_like(d[0]) for d in dev]
                if grouped:
                    ff.ff_render_attend_grouped(pr.ctx, [i for i, _ in diag], [k for _, k in diag],
                                                [d[0] for d in dev], [d[1] for d in dev], [d[2] for d in dev], o)
                else:
                    for (i, k), d, oo in zip(diag, dev, o):
                        ff.ff_render_attend(pr.ctx, i, k, d[0], d[1], d[2], oo)
                torch.cuda.synchronize()
                for p, oo in zip(diag, o):
                    res[p] = oo.view(torch.int16).cpu().numpy()
            outs[grouped] = res
        finally:
            pr.close()
    assert outs[False].keys() == outs[True].keys()
    for p in outs[False]:
        assert np.array_equal(outs[False][p], outs[True][p]), p


def test_split_k_path():
    """One head and a short chunk: the grid is tiny, so the key range is split and merged."""
    st = _rollout(Case(T=64, nh=1, d=128, S=1), control_from=6)
    assert st.calls == 27
    print(f"split-K: max|dO|={st.max_abs:.2e} relF={st.max_rel_fro:.2e}")


def test_w_ctx_cap_binding():
    st = _rollout(Case(T=32, nh=2, d=128, S=1, w_ctx=11))
    assert st.calls == 27


def test_minimum_tokens_and_single_history():
    st = _rollout(Case(T=8, nh=2, d=128, S=2, H=1))
    assert st.calls == 54


def _planner_rollout(case, steps=2, rows=None, render_diags=0, control=True):
    """Every planner block in order: `steps` denoising calls, then the
    cache-extraction call that publishes the block; then the first
    `render_diags` anti-diagonals of the renderer on the anchors so published."""
    pr = Pair(case)
    try:
        for b in range(len(orc.planner_blocks(case.cfg))):
            for step in range(steps):
                pr.plan_step(b, step, publish=False, rows=rows, control=control and b > 0 and step == 0)
            pr.plan_step(b, steps, publish=True, rows=rows)
        for diag in wavefront(case)[:render_diags]:
            pr.step(diag, grouped=True, rows=rows)
        return pr.stats
    finally:
        pr.close()


def test_planner_rollout_tiny_fp32():
    """fp32, 2 heads, d=64, T=16, 261 latents: 9 planner blocks x (2 denoising
    calls + the cache-extraction call), then 12 renderer diagonals on them."""
    st = _planner_rollout(Case(T=16, nh=2, d=64, dtype="f32", n_latents=261, S=2), render_diags=12)
    assert st.calls == 27 + 23
    print(f"planner fp32: max|dO|={st.max_abs:.2e} relF={st.max_rel_fro:.2e} lse={st.max_lse:.2e}")


@pytest.mark.parametrize("n_latents", [3, 42])
def test_planner_short_blocks(n_latents):
    """A lone one-anchor block (3 latents), and a last block shorter than B_P
    (42 latents: anchors 0, 10, .., 40 in blocks of 3 and 2)."""
    case = Case(T=16, nh=2, d=128, n_latents=n_latents, S=2)
    n_blocks = len(orc.planner_blocks(case.cfg))
    st = _planner_rollout(case, render_diags=3)
    assert st.calls == 3 * n_blocks + sum(len(d) for d in wavefront(case)[:3])


@pytest.mark.parametrize("h_p", [6, 2])
def test_planner_rollout_bf16_multi_tile(h_p):
    """bf16, T=120 (360 queries: 2 query tiles, ragged), 261 latents: block 8
    reads min(8, H_P) earlier blocks (up to 18 anchors + 3 own = 6720 keys,
    each anchor a ragged 64-key source)."""
    st = _planner_rollout(Case(T=120, nh=2, d=128, n_latents=261, S=2, h_p=h_p), render_diags=4)
    assert st.calls == 27 + 7
    print(f"planner bf16 H_P={h_p}: max|dO|={st.max_abs:.2e} relF={st.max_rel_fro:.2e} "
          f"control>={st.min_control_ratio:.1f}x")


def test_planner_480p_block_sampled_rows():
    """480p shape, 261 latents: blocks 0..8 published through their
    cache-extraction calls; block 8's denoising call reads 6 earlier blocks
    (21 key latents, 4680 queries x 32760 keys), 32 sampled rows per call;
    that call (the one the planner benchmark times) also whole on heads 0 and
    11: every query row against the oracle over the head's 32760 keys."""
    import sys
    case = Case(T=1560, nh=12, d=128, n_latents=261, S=1)
    rows = np.sort(np.random.default_rng(3).choice(3 * 1560, size=32, replace=False))
    pr = Pair(case)
    try:
        for b in range(9):
            if b == 8:
                _, _, whole = pr.plan_step(b, 0, publish=False, rows=rows, control=True, whole_heads=(0, 11))
                for hh, err, relf in whole:
                    print(f"  planner block 8 head {hh}, all rows: max|dO|={err:.2e} relF={relf:.2e}", flush=True,
                          file=sys.stderr)
            pr.plan_step(b, 1, publish=True, rows=rows)
            print(f"  planner block {b} ok", flush=True, file=sys.stderr)
        print(f"planner 480p: max|dO|={pr.stats.max_abs:.2e} relF={pr.stats.max_rel_fro:.2e} "
              f"control>={pr.stats.min_control_ratio:.1f}x")
    finally:
        pr.close()


def test_480p_steps_sampled_rows():
    """480p shape (T=1560, 12 heads, d=128) at stage 0, chunks 0..13: chunk 5 is the
    first 20-latent step (31200 keys), chunk 13 the 21-latent one (32760 keys, three
    anchors).  Outputs on 64 sampled query rows per call, banks bit-exact;
    chunk 5 (the call the step benchmark times) also whole: every query row of
    every head; chunk 13 whole on heads 0 and 11."""
    from ffharness import check_whole_heads, whole_head_reference
    case = Case(T=1560, nh=12, d=128, S=1)
    rows = np.sort(np.random.default_rng(7).choice(3 * 1560, size=64, replace=False))
    pr = Pair(case)
    try:
        pr.publish_anchors()
        for i in range(14):
            heads = range(12) if i == 5 else (0, 11) if i == 13 else ()
            whole = whole_head_reference(pr, i, 0, heads) if heads else {}
            pr.step([(i, 0)], grouped=False, rows=rows, control=i in (5, 13))
            for hh, err, relf in check_whole_heads(pr, whole):
                print(f"480p chunk {i} head {hh}, all rows: max|dO|={err:.2e} relF={relf:.2e}")
        print(f"480p chunks 0..13: max|dO|={pr.stats.max_abs:.2e} relF={pr.stats.max_rel_fro:.2e} "
              f"control>={pr.stats.min_control_ratio:.1f}x")
    finally:
        pr.close()


def test_480p_rollout_grouped_full_size():
    """One-layer 81-latent rollout at the 480p shape (T=1560, 12 heads, d=128):
    9 anchors in 3 planner blocks, then the 30 anti-diagonals of 27 chunks x 4
    stages as grouped launches (108 calls).  Every call: O and LSE on 16
    sampled query rows against the oracle; every stage bank's ids and bytes
    after every call."""
    import sys
    case = Case(T=1560, nh=12, d=128, S=4)
    rows = np.sort(np.random.default_rng(11).choice(3 * 1560, size=16, replace=False))
    pr = Pair(case, device_bank_check=True)
    try:
        pr.publish_anchors()
        for t, diag in enumerate(wavefront(case)):
            pr.step(diag, grouped=True, rows=rows, control=(t == 12))
            print(f"  diagonal {t}: {len(diag)} pairs ok", flush=True, file=sys.stderr)
        assert pr.stats.calls == 108 and pr.stats.bank_checks == 108
        print(f"480p rollout grouped: max|dO|={pr.stats.max_abs:.2e} relF={pr.stats.max_rel_fro:.2e} "
              f"control>={pr.stats.min_control_ratio:.1f}x")
    finally:
        pr.close()


def test_720p_step_sampled_rows():
    """720p / 14B shape (T=3600, 40 heads, d=128): chunks 0..13 at stage 0; chunk 5
    is the 20-latent step (10800 queries x 72000 keys) and chunk 13 the
    21-latent one (75600 keys, three anchors), the largest call of the
    workloads; 8 sampled query rows per call against the oracle, banks exact.
    Chunks 5 (the call the 720p step benchmark times) and 13 are also checked
    whole on heads 0 and 39: all 10800 query rows against the oracle over
    that head's 72000 or 75600 keys."""
    import sys

    from ffharness import check_whole_heads, whole_head_reference
    case = Case(T=3600, nh=40, d=128, S=1)
    rows = np.sort(np.random.default_rng(5).choice(3 * 3600, size=8, replace=False))
    pr = Pair(case, device_bank_check=True)
    try:
        pr.publish_anchors()
        for i in range(14):
            whole = whole_head_reference(pr, i, 0, (0, 39)) if i in (5, 13) else {}
            pr.step([(i, 0)], grouped=False, rows=rows, control=i in (5, 13))
            for hh, err, relf in check_whole_heads(pr, whole):
                print(f"  720p chunk {i} head {hh}, all rows: max|dO|={err:.2e} relF={relf:.2e}", flush=True,
                      file=sys.stderr)
            print(f"  720p chunk {i} ok", flush=True, file=sys.stderr)
        print(f"720p chunks 0..13: max|dO|={pr.stats.max_abs:.2e} relF={pr.stats.max_rel_fro:.2e} "
              f"control>={pr.stats.min_control_ratio:.1f}x")
    finally:
        pr.close()


def test_rewind_and_repeat():
    """ff_stage_bank_rewind, then the same calls again with new inputs (the
    steady-state replay the step benchmark uses): O, LSE and every bank after
    the repeat match the oracle of the state before the first run, and the
    rollout then continues correctly."""
    import copy
    import dataclasses

    from chunked_kv_cache_amd import ff
    case = Case(T=200, nh=2, d=128, S=2)
    pr = Pair(case)
    try:
        pr.publish_anchors()
        diags = wavefront(case)
        for diag in diags[:8]:
            pr.step(diag, grouped=True)
        snap = copy.deepcopy(pr.ro)
        pr.step(diags[8], grouped=True, control=True)
        for _, k in sorted(diags[8], key=lambda p: -p[1]):
            ff.ff_stage_bank_rewind(pr.ctx, k)
        pr.ro = snap
        pr.case = dataclasses.replace(case, seed=5)          # different inputs for the repeat
        pr.step(diags[8], grouped=False, control=True)
        for diag in diags[9:12]:
            pr.step(diag, grouped=True)
        assert pr.stats.calls == sum(len(d) for d in diags[:12]) + len(diags[8])
    finally:
        pr.close()


def test_two_streams_one_stage_each():
    """Stage 0 on one stream, stage 1 on another, (i, 1) after (i, 0) by an
    event: calls of different stages overlap on the GPU and use their own
    partial regions (T = 200: every item is split, so partials are written).
    Every output matches the oracle; the banks end bit-exact."""
    import torch

    import synthetic as syn
    from chunked_kv_cache_amd import ff
    from ffharness import from_device_f64, to_device
    case = Case(T=200, nh=2, d=128, S=2)
    pr = Pair(case)
    try:
        pr.publish_anchors()
        torch.cuda.synchronize()
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        nc = 27
        keep, outs = {}, {}
        for i in range(nc):                      # inputs and NaN-filled outputs, all ready before any call
            for k in (0, 1):
                keep[(i, k)] = [to_device(x, "bf16") for x in pr.gen(i, k)]
                outs[(i, k)] = (torch.full_like(keep[(i, k)][0], float("nan")),
                                torch.full((case.nh, 3 * case.T), float("nan"), dtype=torch.float32,
                                           device="cuda"))
        torch.cuda.synchronize()
        for i in range(nc):
            for k in (0, 1):
                dev, (o, l), s = keep[(i, k)], outs[(i, k)], streams[k]
                if k == 1:
                    s.wait_event(done0)
                ff.ff_render_attend(pr.ctx, i, k, dev[0], dev[1], dev[2], o, l, stream=s)
                if k == 0:
                    done0 = torch.cuda.Event()
                    done0.record(s)
        torch.cuda.synchronize()
        for i in range(nc):
            for k in (0, 1):
                q64, k64, v64 = (syn.as_f64(x, "bf16") for x in pr.gen(i, k))
                O_ref, L_ref = pr.ro.render_attend(i, k, q64, k64, v64)
                pr.inputs[(i, k)] = pr.gen(i, k)[1:]
                o, l = outs[(i, k)]
                pr._compare(from_device_f64(o), l.cpu().numpy().astype(np.float64), O_ref, L_ref, None, 2e-2)
        for k in (0, 1):
            pr.check_bank(k)
        assert pr.stats.calls == 2 * nc
    finally:
        pr.close()


def test_graph_capture_rollout():
    """A whole grouped rollout captured into one HIP graph and replayed three
    times, with eager work and synchronizations between the replays.  The
    renderer calls enqueue kernel launches only (no allocation, memset, copy
    or host wait), so a replay recomputes the rollout from the anchors: every
    replay's outputs, and the stage banks after it, equal the eager rollout's
    bit for bit (items are cut, so the merge kernel is in the graph too)."""
    import torch

    from chunked_kv_cache_amd import ff
    from ffharness import to_device
    case = Case(T=48, nh=2, d=128, S=2, n_latents=21)
    diags = wavefront(case)

    def setup():
        pr = Pair(case, oracle_compute=False)
        pr.publish_anchors()
        ins = {p: [to_device(x, "bf16") for x in pr.gen(*p)] for d in diags for p in d}
        outs = {p: (torch.empty_like(ins[p][0]), torch.empty((case.nh, 3 * case.T), dtype=torch.float32,
                                                               device="cuda")) for p in ins}
        torch.cuda.synchronize()
        return pr, ins, outs

    def rollout(pr, ins, outs):
        for d in diags:
            ff.ff_render_attend_grouped(pr.ctx, [i for i, _ in d], [k for _, k in d], [ins[p][0] for p in d],
                                        [ins[p][1] for p in d], [ins[p][2] for p in d],
                                        [outs[p][0] for p in d], [outs[p][1] for p in d])

    def banks(pr):
        res = []
        for k in range(case.S):
            Ko = torch.empty((case.H * 3 * case.T, case.nh, case.d), dtype=torch.bfloat16, device="cuda")
            Vo = torch.empty_like(Ko)
            ids = ff.ff_bank_tail(pr.ctx, k, Ko, Vo)
            torch.cuda.synchronize()
            res.append((ids, Ko.view(torch.int16).cpu().numpy(), Vo.view(torch.int16).cpu().numpy()))
        return res

    eager, e_ins, e_outs = setup()
    graph, g_ins, g_outs = setup()
    try:
        rollout(eager, e_ins, e_outs)
        torch.cuda.synchronize()
        ref = {p: (o.view(torch.int16).cpu().numpy(), l.cpu().numpy()) for p, (o, l) in e_outs.items()}
        ref_banks = banks(eager)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            rollout(graph, g_ins, g_outs)
        torch.cuda.synchronize()
        for rep in range(3):
            for o, l in g_outs.values():
                o.fill_(float("nan"))
                l.fill_(float("nan"))
            noise = torch.randn(1 << 20, device="cuda").sum()          # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.isfinite(noise)
            for p, (o, l) in g_outs.items():
                assert np.array_equal(o.view(torch.int16).cpu().numpy(), ref[p][0]), (rep, p)
                assert np.array_equal(l.cpu().numpy(), ref[p][1]), (rep, p)
            for (ids, Kb, Vb), (rids, rK, rV) in zip(banks(graph), ref_banks):
                assert ids == rids and np.array_equal(Kb, rK) and np.array_equal(Vb, rV), rep
        del g
    finally:
        eager.close()
        graph.close()


def test_65s_rollout_grouped_full_size():
    """The 65 s rollout at its stated shape: 480p (T = 1560, 12 heads, d = 128),
    261 latents, 27 anchors in 9 planner blocks, 87 chunks x 4 stages = 348
    calls in 90 grouped anti-diagonal launches from the library's schedule.
    Inputs: 8 seeded N(0,1) sets, call (i, k) taking set (i + k) mod 8, so the
    six chunks one call reads from a bank are all different.  Every call: O
    and LSE on 16 sampled query rows of heads 0 and 7 against the oracle run on
    those heads; every stage bank of the diagonal compared bit for bit on the
    device with the input tensors; an anchor-less control on diagonal 40."""
    import sys

    import torch

    import synthetic as syn
    from chunked_kv_cache_amd import ff
    from ffharness import LSE_TOL, RELF_TOL, TOL, Stats, record
    T, nh, d, S, P = 1560, 12, 128, 4, 8
    heads = [0, 7]
    case = Case(T=T, nh=nh, d=d, n_latents=261, S=S)
    cfg_o = orc.FFConfig(tokens_per_latent=T, n_heads=len(heads), head_dim=d, n_latents=261, n_stages=S)
    rows = np.sort(np.random.default_rng(13).choice(3 * T, size=16, replace=False))
    rows_d = torch.as_tensor(rows, device="cuda")
    banks = ff.StageBanks(case.shape(), S, 5)
    banks.workspace.view(torch.int16).fill_(0x7FC0)
    ro = orc.Rollout(cfg_o)
    st = Stats()
    try:
        pool_dev, pool_f64 = [], []
        for j in range(P):
            host = syn.chunk_qkv(T=T, n_heads=nh, head_dim=d, chunk=j, stage=0, seed=3)
            pool_dev.append([torch.from_numpy(x).view(torch.bfloat16).cuda() for x in host])
            pool_f64.append([syn.as_f64(x[:, heads], "bf16") for x in host])
        for b in range(ff.ff_clip_layout(case.shape(), S)["n_planner_blocks"]):
            blk = ff.ff_planner_block(case.shape(), b)
            K, V = syn.anchor_kv(T=T, n_heads=nh, head_dim=d, anchors=blk, seed=3)
            ff.ff_anchor_bank_publish(banks.ctx, blk[0], len(blk), torch.from_numpy(K).view(torch.bfloat16).cuda(),
                                      torch.from_numpy(V).view(torch.bfloat16).cuda())
            ro.publish_anchors(blk[0], syn.as_f64(K[:, heads], "bf16"), syn.as_f64(V[:, heads], "bf16"))
        print("  anchors published", flush=True, file=sys.stderr)
        outs = [torch.empty((3 * T, nh, d), dtype=torch.bfloat16, device="cuda") for _ in range(S)]
        lses = [torch.empty((nh, 3 * T), dtype=torch.float32, device="cuda") for _ in range(S)]
        Ko = torch.empty((5 * 3 * T, nh, d), dtype=torch.bfloat16, device="cuda")
        Vo = torch.empty_like(Ko)
        for t, diag in enumerate(wavefront(case)):
            sets = [(i + k) % P for i, k in diag]
            for o in outs:
                o.fill_(float("nan"))
            ff.ff_render_attend_grouped(banks.ctx, [i for i, _ in diag], [k for _, k in diag],
                                        [pool_dev[s][0] for s in sets], [pool_dev[s][1] for s in sets],
                                        [pool_dev[s][2] for s in sets], [outs[k] for _, k in diag],
                                        [lses[k] for _, k in diag])
            torch.cuda.synchronize()
            for (i, k), s in zip(diag, sets):
                q64, k64, v64 = pool_f64[s]
                ctl = None
                if t == 40:
                    Kc, Vc = ro.gather_keys(i, k, k64, v64)
                    na = T * len(orc.gamma(cfg_o, i))
                    ctl, _ = orc.attention(q64[rows], Kc[na:], Vc[na:], cfg_o.scale)
                O_ref, L_ref = ro.render_attend(i, k, q64, k64, v64, rows=rows)
                O = outs[k][rows_d][:, heads].float().cpu().numpy().astype(np.float64)
                L = lses[k][heads][:, rows_d].cpu().numpy().astype(np.float64)
                assert np.all(np.isfinite(O))
                err = np.abs(O - O_ref).max()
                relf = np.linalg.norm(O - O_ref) / np.linalg.norm(O_ref)
                lerr = np.abs(L - L_ref).max()
                st.max_abs, st.max_rel_fro, st.max_lse = max(st.max_abs, err), max(st.max_rel_fro, relf), \
                    max(st.max_lse, lerr)
                st.max_gate_use = max(st.max_gate_use, err / TOL["bf16"])
                st.calls += 1
                assert err <= TOL["bf16"] and relf <= RELF_TOL["bf16"] and lerr <= LSE_TOL["bf16"], \
                    (i, k, err, relf, lerr)
                if ctl is not None:
                    ratio = np.linalg.norm(O - ctl) / max(np.linalg.norm(O - O_ref), 1e-30)
                    st.min_control_ratio = min(st.min_control_ratio, ratio)
                    assert ratio >= 10.0, ratio
                # stage bank k on the device against the pool tensors it must hold
                ids = ff.ff_bank_tail(banks.ctx, k, Ko, Vo)
                assert ids == ro.bank_tail(k)[0]
                L3 = 3 * T
                for jj, cid in enumerate(ids):
                    src = pool_dev[(cid + k) % P]
                    assert torch.equal(Ko[jj * L3:(jj + 1) * L3].view(torch.int16), src[1].view(torch.int16))
                    assert torch.equal(Vo[jj * L3:(jj + 1) * L3].view(torch.int16), src[2].view(torch.int16))
                st.bank_checks += 1
            if t % 10 == 0:
                print(f"  diagonal {t}: {len(diag)} pairs ok", flush=True, file=sys.stderr)
        assert st.calls == 348 and st.bank_checks == 348
        print(f"65 s rollout grouped: max|dO|={st.max_abs:.2e} relF={st.max_rel_fro:.2e} "
              f"control>={st.min_control_ratio:.1f}x")
    finally:
        record(st)
        banks.close()
