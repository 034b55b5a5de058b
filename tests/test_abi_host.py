"""CPU tests of the C ABI: exports, and the host bookkeeping against the oracle.

libff.so is loaded and its exports are checked against include/ff.h; no
compute call is made on it without a GPU except error paths that return
before any device work.  The success paths (ring metadata, Tail_H ids, the
key-source table handed to the attention kernel, error atomicity) run on
libff_hostcheck.so: the same host source linked against a recording stub.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle as orc
from chunked_kv_cache_amd import ff

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ff.h")


def header_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:ff_status|size_t|void|const char\*)\s+(ff_\w+)\(", src, re.M)))


def test_header_declares_the_boundary():
    fns = header_functions()
    for name in ("ff_anchor_bank_publish", "ff_stage_bank_create", "ff_render_attend", "ff_bank_tail"):
        assert name in fns
    assert sorted(ff.SYMBOLS) == fns


@pytest.mark.parametrize("path", [ff.LIB_PATH, ff.HOSTCHECK_PATH])
def test_library_exports_every_declared_symbol(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(ff_\w+)$", out, re.M))
    missing = [f for f in header_functions() if f not in exported]
    assert not missing, missing
    lib = ff.load(path)                     # loads and binds every prototype
    assert lib.ff_status_str(ff.FF_E_ORDER).startswith(b"order")


def test_product_library_rejects_before_device_work():
    """libff.so validates before touching the GPU, so these run on a CPU host."""
    L = ff.load(ff.LIB_PATH)
    shape = ff.make_shape(n_heads=2, head_dim=128, tokens_per_latent=16)
    need = ff.ff_workspace_bytes(shape, 4, 5, L=L)
    buf, addr = _aligned_buffer(need)
    ctx = ff.ff_stage_bank_create(shape, 4, 5, addr, need, L=L)
    try:
        with pytest.raises(ff.FFError) as e:             # anchors of Gamma(0) missing
            ff.ff_render_attend(ctx, 0, 0, 256, 256, 256, 256, L=L)
        assert e.value.status == ff.FF_E_ANCHOR_MISSING
        with pytest.raises(ff.FFError) as e:
            ff.ff_render_attend(ctx, 1, 0, 256, 256, 256, 256, L=L)
        assert e.value.status == ff.FF_E_ORDER
    finally:
        ff.ff_destroy(ctx, L=L)


def test_profile_families_are_validated():
    """ff_profile_families takes only the bits of the ff_kernel_times families
    (checked on the host, no device work) and holds across enable/disable."""
    L = ff.load(ff.HOSTCHECK_PATH)
    shape = ff.make_shape(n_heads=2, head_dim=128, tokens_per_latent=16)
    need = ff.ff_workspace_bytes(shape, 1, 5, L=L)
    buf, addr = _aligned_buffer(need)
    ctx = ff.ff_stage_bank_create(shape, 1, 5, addr, need, L=L)
    try:
        for fam in (0, ff.PROF_ATTN, ff.PROF_PUBLISH | ff.PROF_MERGE, ff.PROF_ALL):
            ff.ff_profile_families(ctx, fam, L=L)
        with pytest.raises(ff.FFError) as e:
            ff.ff_profile_families(ctx, ff.PROF_ALL + 1, L=L)
        assert e.value.status == ff.FF_E_INVAL
        ff.ff_profile_families(ctx, ff.PROF_ATTN, L=L)
        ff.ff_profile_enable(ctx, True, L=L)
        ff.ff_profile_enable(ctx, False, L=L)
        assert ff.ff_profile_read(ctx, L=L)["attn_launches"] == 0
    finally:
        ff.ff_destroy(ctx, L=L)


# --------------------------------------------------------------------------
# Host-check library (recording stub instead of kernels)
# --------------------------------------------------------------------------
def _aligned_buffer(nbytes):
    raw = np.zeros(nbytes + 512, dtype=np.uint8)
    addr = raw.ctypes.data
    addr = (addr + 255) // 256 * 256
    return raw, addr


class HostCtx:
    def __init__(self, cfg: orc.FFConfig, w_ctx=None, dtype=ff.FF_BF16):
        self.L = ff.load(ff.HOSTCHECK_PATH)
        self.cfg = cfg
        rule = ff.FF_GAMMA_BRACKET if cfg.gamma_rule == orc.GAMMA_BRACKET else ff.FF_GAMMA_CENTER_LR
        self.shape = ff.make_shape(n_heads=cfg.n_heads, head_dim=cfg.head_dim,
                                   tokens_per_latent=cfg.tokens_per_latent, chunk_latents=cfg.chunk_latents,
                                   anchor_stride=cfg.anchor_stride, n_latents=cfg.n_latents,
                                   w_ctx=cfg.w_ctx if w_ctx is None else w_ctx, dtype=dtype, gamma_rule=rule,
                                   planner_latents=cfg.planner_block, planner_history=cfg.planner_history)
        self.need = ff.ff_workspace_bytes(self.shape, cfg.n_stages, cfg.history, L=self.L)
        self.raw, self.ws = _aligned_buffer(self.need)
        self.ctx = ff.ff_stage_bank_create(self.shape, cfg.n_stages, cfg.history, self.ws, self.need, L=self.L)

    def counts(self):
        c = [ctypes.c_int() for _ in range(4)]
        self.L.ffstub_counts(*[ctypes.byref(x) for x in c])
        return [x.value for x in c]

    def last_segments(self, p=0):
        off = (ctypes.c_longlong * ff.FF_MAX_SOURCES)()
        n = (ctypes.c_int * ff.FF_MAX_SOURCES)()
        lk, ns = ctypes.c_int(), ctypes.c_int()
        f = self.L.ffstub_last_segments
        f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                      ctypes.c_void_p]
        k = f(p, self.ws, off, n, ctypes.byref(lk), ctypes.byref(ns))
        return list(off[:k]), list(n[:k]), lk.value, ns.value

    def last_copy_block(self, j):
        f = self.L.ffstub_last_copy_block
        f.restype = ctypes.c_longlong
        f.argtypes = [ctypes.c_int, ctypes.c_void_p]
        return f(j, self.ws)

    def close(self):
        ff.ff_destroy(self.ctx, L=self.L)


def _layout(cfg):
    esz = 2
    T, nh, d = cfg.tokens_per_latent, cfg.n_heads, cfg.head_dim
    al = lambda x: (x + 255) // 256 * 256
    anchor_block = al(2 * nh * T * d * esz)
    slot_block = al(2 * nh * 3 * T * d * esz)
    slot_off = orc.n_anchors(cfg) * anchor_block
    return anchor_block, slot_block, slot_off


FAKE = 1 << 20      # 16-byte aligned stand-in device addresses; the stub never reads them


def _publish_anchors(hc):
    for blk in orc.planner_blocks(hc.cfg):
        ff.ff_anchor_bank_publish(hc.ctx, blk[0], len(blk), FAKE, FAKE, L=hc.L)


@pytest.mark.parametrize("rule", [orc.GAMMA_BRACKET, orc.GAMMA_CENTER_LR])
@pytest.mark.parametrize("L", [81, 261])
def test_gamma_matches_oracle(rule, L):
    cfg = orc.FFConfig(tokens_per_latent=16, n_heads=2, head_dim=64, n_latents=L, gamma_rule=rule)
    hc = HostCtx(cfg)
    try:
        for i in range(orc.n_chunks(cfg)):
            assert ff.ff_gamma(hc.ctx, i, L=hc.L) == orc.gamma(cfg, i)
    finally:
        hc.close()


@pytest.mark.parametrize("rule", [orc.GAMMA_BRACKET, orc.GAMMA_CENTER_LR])
def test_rollout_bookkeeping_matches_oracle(rule):
    cfg = orc.FFConfig(tokens_per_latent=16, n_heads=3, head_dim=128, gamma_rule=rule)
    hc = HostCtx(cfg)
    ro = orc.Rollout(cfg)
    anchor_block, slot_block, slot_off = _layout(cfg)
    z = np.zeros((48, 3, 128))
    c0 = hc.counts()
    try:
        _publish_anchors(hc)
        for blk in orc.planner_blocks(cfg):
            ro.publish_anchors(blk[0], np.zeros((16 * len(blk), 3, 128)), np.zeros((16 * len(blk), 3, 128)))
        for diag in orc.schedule(cfg):
            for i, k in diag:
                plan = ff.ff_key_plan(hc.ctx, i, k, L=hc.L)
                src = ro.key_sources(i, k)
                kinds = {ff.FF_SRC_ANCHOR: "anchor", ff.FF_SRC_HISTORY: "history", ff.FF_SRC_OWN: "own"}
                got = [(kinds[plan.kind[j]], plan.id[j]) for j in range(plan.n_sources)]
                assert got == src
                ntok = [16 if s == "anchor" else 48 for s, _ in src]
                assert list(plan.n_tokens[:plan.n_sources]) == ntok
                assert plan.key_tokens == sum(ntok)
                ff.ff_render_attend(hc.ctx, i, k, FAKE, FAKE, FAKE, FAKE, L=hc.L)
                ro.render_attend(i, k, None, z, z, compute=False)
                # the key table handed to the kernel points at the right blocks
                offs, ntoks, lk, ntiles = hc.last_segments()
                assert ntoks == ntok and lk == sum(ntok)
                assert ntiles == sum((n + 63) // 64 for n in ntok)      # sources padded to 64-key tiles
                for (s, idx), off in zip(src, offs):
                    if s == "anchor":
                        assert off == idx * anchor_block
                    else:
                        assert off == slot_off + (k * 6 + idx % 6) * slot_block
                # the publish went to slot i mod (H+1) of stage k
                assert hc.last_copy_block(0) == slot_off + (k * 6 + i % 6) * slot_block
                assert ff.ff_bank_tail(hc.ctx, k, L=hc.L) == ro.bank_tail(k)[0]
                assert ff.ff_stage_next(hc.ctx, k, L=hc.L) == i + 1
        assert [a - b for a, b in zip(hc.counts(), c0)][:3] == [108, 108, 3]
    finally:
        hc.close()


def test_grouped_calls_match_single_calls_bookkeeping():
    cfg = orc.FFConfig(tokens_per_latent=16, n_heads=2, head_dim=128, n_latents=261)
    hc = HostCtx(cfg)
    c0 = hc.counts()
    try:
        _publish_anchors(hc)
        for diag in orc.schedule(cfg):
            chunks = [i for i, _ in diag]
            stages = [k for _, k in diag]
            n = len(diag)
            ff.ff_render_attend_grouped(hc.ctx, chunks, stages, [FAKE] * n, [FAKE] * n, [FAKE] * n,
                                        [FAKE] * n, L=hc.L)
        for k in range(4):
            assert ff.ff_bank_tail(hc.ctx, k, L=hc.L) == list(range(82, 87))
        assert hc.counts()[0] - c0[0] == 90
    finally:
        hc.close()


def test_error_paths_leave_state_unchanged():
    cfg = orc.FFConfig(tokens_per_latent=16, n_heads=2, head_dim=128)
    hc = HostCtx(cfg)
    L = hc.L
    F = FAKE

    def status(fn, *a):
        try:
            fn(*a, L=L)
            return ff.FF_OK
        except ff.FFError as e:
            return e.status

    try:
        assert status(ff.ff_render_attend, hc.ctx, 0, 0, F, F, F, F) == ff.FF_E_ANCHOR_MISSING
        ff.ff_anchor_bank_publish(hc.ctx, 0, 3, F, F, L=L)
        assert status(ff.ff_anchor_bank_publish, hc.ctx, 2, 1, F, F) == ff.FF_E_ANCHOR_EXISTS
        assert status(ff.ff_anchor_bank_publish, hc.ctx, 8, 2, F, F) == ff.FF_E_RANGE
        assert status(ff.ff_anchor_bank_publish, hc.ctx, 3, 1, F + 8, F) == ff.FF_E_INVAL
        before = hc.counts()
        assert status(ff.ff_render_attend, hc.ctx, 1, 0, F, F, F, F) == ff.FF_E_ORDER      # skips chunk 0
        assert status(ff.ff_render_attend, hc.ctx, 0, 1, F, F, F, F) == ff.FF_E_ORDER      # stage 0 not run
        assert status(ff.ff_render_attend, hc.ctx, 0, 4, F, F, F, F) == ff.FF_E_RANGE
        assert status(ff.ff_render_attend, hc.ctx, 27, 0, F, F, F, F) == ff.FF_E_RANGE
        assert status(ff.ff_render_attend, hc.ctx, 0, 0, 0, F, F, F) == ff.FF_E_INVAL
        assert status(ff.ff_render_attend, hc.ctx, 0, 0, F, F, F, F + 4) == ff.FF_E_INVAL
        assert status(ff.ff_render_attend, hc.ctx, 0, 0, F, F, F, F, F + 2) == ff.FF_E_INVAL   # lse
        assert hc.counts() == before and ff.ff_stage_next(hc.ctx, 0, L=L) == 0
        for i in range(3):
            ff.ff_render_attend(hc.ctx, i, 0, F, F, F, F, L=L)
        # grouped: a pair that depends on another pair of the same call is refused atomically
        assert status(ff.ff_render_attend_grouped, hc.ctx, [0, 0], [1, 2], [F] * 2, [F] * 2, [F] * 2,
                      [F] * 2) == ff.FF_E_ORDER
        assert status(ff.ff_render_attend_grouped, hc.ctx, [0, 1], [1, 1], [F] * 2, [F] * 2, [F] * 2,
                      [F] * 2) == ff.FF_E_ORDER
        assert ff.ff_stage_next(hc.ctx, 1, L=L) == 0
        # rewind: once per publish, and not under a later stage that consumed the chunk
        ff.ff_render_attend(hc.ctx, 0, 1, F, F, F, F, L=L)
        assert status(ff.ff_stage_bank_rewind, hc.ctx, 0) == ff.FF_OK            # chunk 2 of stage 0
        assert ff.ff_stage_next(hc.ctx, 0, L=L) == 2
        assert ff.ff_bank_tail(hc.ctx, 0, L=L) == [0, 1]
        assert status(ff.ff_stage_bank_rewind, hc.ctx, 0) == ff.FF_E_STATE
        ff.ff_render_attend(hc.ctx, 2, 0, F, F, F, F, L=L)
        assert status(ff.ff_stage_bank_rewind, hc.ctx, 1) == ff.FF_OK
        assert status(ff.ff_stage_bank_rewind, hc.ctx, 2) == ff.FF_E_STATE
    finally:
        hc.close()


def test_rewind_after_stage_consumed_is_refused():
    cfg = orc.FFConfig(tokens_per_latent=16, n_heads=2, head_dim=128)
    hc = HostCtx(cfg)
    try:
        _publish_anchors(hc)
        ff.ff_render_attend(hc.ctx, 0, 0, FAKE, FAKE, FAKE, FAKE, L=hc.L)
        ff.ff_render_attend(hc.ctx, 0, 1, FAKE, FAKE, FAKE, FAKE, L=hc.L)
        with pytest.raises(ff.FFError) as e:
            ff.ff_stage_bank_rewind(hc.ctx, 0, L=hc.L)
        assert e.value.status == ff.FF_E_STATE
        ff.ff_stage_bank_rewind(hc.ctx, 1, L=hc.L)
        ff.ff_stage_bank_rewind(hc.ctx, 0, L=hc.L)
        assert [ff.ff_stage_next(hc.ctx, k, L=hc.L) for k in range(4)] == [0, 0, 0, 0]
    finally:
        hc.close()


def test_w_ctx_cap_matches_oracle():
    cfg = orc.FFConfig(tokens_per_latent=16, n_heads=2, head_dim=64, w_ctx=11, n_stages=1)
    hc = HostCtx(cfg)
    ro = orc.Rollout(cfg)
    z = np.zeros((48, 2, 64))
    try:
        _publish_anchors(hc)
        for blk in orc.planner_blocks(cfg):
            ro.publish_anchors(blk[0], np.zeros((16 * len(blk), 2, 64)), np.zeros((16 * len(blk), 2, 64)))
        for i in range(orc.n_chunks(cfg)):
            plan = ff.ff_key_plan(hc.ctx, i, 0, L=hc.L)
            assert plan.key_latents <= 11 or plan.n_sources == len(orc.gamma(cfg, i)) + 1
            assert [plan.id[j] for j in range(plan.n_sources)] == [x for _, x in ro.key_sources(i, 0)]
            ff.ff_render_attend(hc.ctx, i, 0, FAKE, FAKE, FAKE, FAKE, L=hc.L)
            ro.render_attend(i, 0, None, z, z, compute=False)
    finally:
        hc.close()


@pytest.mark.parametrize("bad", [dict(head_dim=96), dict(tokens_per_latent=12), dict(tokens_per_latent=4),
                                 dict(chunk_latents=11), dict(n_latents=82), dict(dtype=7), dict(gamma_rule=5),
                                 dict(n_heads=0)])
def test_unsupported_shapes_are_rejected(bad):
    L = ff.load(ff.HOSTCHECK_PATH)
    kw = dict(n_heads=2, head_dim=128, tokens_per_latent=16)
    kw.update(bad)
    shape = ff.make_shape(**kw)
    assert ff.ff_workspace_bytes(shape, 4, 5, L=L) == 0
    with pytest.raises(ff.FFError) as e:
        ff.ff_stage_bank_create(shape, 4, 5, 256, 1 << 30, L=L)
    assert e.value.status == ff.FF_E_INVAL


def test_history_and_workspace_limits():
    L = ff.load(ff.HOSTCHECK_PATH)
    shape = ff.make_shape(n_heads=2, head_dim=128, tokens_per_latent=16)
    assert ff.ff_workspace_bytes(shape, 4, 9, L=L) == 0
    need = ff.ff_workspace_bytes(shape, 4, 5, L=L)
    with pytest.raises(ff.FFError) as e:
        ff.ff_stage_bank_create(shape, 4, 5, 256, need - 1, L=L)
    assert e.value.status == ff.FF_E_NOSPACE
    with pytest.raises(ff.FFError) as e:
        ff.ff_stage_bank_create(shape, 4, 5, 256 + 16, need, L=L)     # workspace not 256-aligned
    assert e.value.status == ff.FF_E_INVAL


# --------------------------------------------------------------------------
# Planner calls
# --------------------------------------------------------------------------
def _plan_sources(ks: "ff.ff_key_sources"):
    kinds = {ff.FF_SRC_ANCHOR: "anchor", ff.FF_SRC_OWN: "own"}
    return [(kinds[ks.kind[j]], ks.id[j]) for j in range(ks.n_sources)]


@pytest.mark.parametrize("L,h_p,w_ctx", [(261, 6, 21), (261, 2, 21), (261, 6, 11), (81, 6, 21)])
def test_planner_key_plan_and_launch_match_oracle(L, h_p, w_ctx):
    cfg = orc.FFConfig(tokens_per_latent=16, n_heads=2, head_dim=64, n_latents=L, planner_history=h_p,
                       w_ctx=w_ctx)
    hc = HostCtx(cfg)
    ro = orc.Rollout(cfg)
    anchor_block, _, _ = _layout(cfg)
    T = cfg.tokens_per_latent
    z = np.zeros((3 * T, 2, 64))
    try:
        for b, blk in enumerate(orc.planner_blocks(cfg)):
            for publish in (False, True):
                want = ro.plan_key_sources(b)
                ks = ff.ff_plan_key_plan(hc.ctx, b, L=hc.L)
                assert _plan_sources(ks) == want
                assert ks.key_tokens == T * len(want) and ks.key_latents == len(want)
                before = hc.counts()
                ff.ff_plan_attend(hc.ctx, b, FAKE, FAKE, FAKE, FAKE, None, publish=publish, L=hc.L)
                after = hc.counts()
                assert [a - c for a, c in zip(after, before)] == [1, 0, 1, 0]   # attention + anchor-bank copy
                off, n, lk, ntiles = hc.last_segments()
                assert off == [a * anchor_block for _, a in want]
                assert n == [T] * len(want) and lk == T * len(want)
                assert ntiles == len(want) * ((T + 63) // 64)
                assert hc.last_copy_block(0) == blk[0] * anchor_block
                ro.plan_attend(b, z[:len(blk) * T], z[:len(blk) * T], z[:len(blk) * T], publish=publish,
                               compute=False)
    finally:
        hc.close()


def test_planner_order_contract_and_atomicity():
    cfg = orc.FFConfig(tokens_per_latent=16, n_heads=2, head_dim=64, n_latents=81)
    hc = HostCtx(cfg)
    try:
        def status(fn):
            try:
                fn()
                return ff.FF_OK
            except ff.FFError as e:
                return e.status
        plan = lambda b, pub=False: status(lambda: ff.ff_plan_attend(hc.ctx, b, FAKE, FAKE, FAKE, FAKE, None,
                                                                      publish=pub, L=hc.L))
        before = hc.counts()
        assert plan(1) == ff.FF_E_ORDER
        assert plan(3) == ff.FF_E_RANGE and plan(-1) == ff.FF_E_RANGE
        assert status(lambda: ff.ff_plan_attend(hc.ctx, 0, FAKE + 8, FAKE, FAKE, FAKE, L=hc.L)) == ff.FF_E_INVAL
        assert hc.counts() == before                                 # nothing launched
        assert plan(0) == ff.FF_OK                                   # denoising call: publishes nothing
        assert status(lambda: ff.ff_render_attend(hc.ctx, 0, 0, FAKE, FAKE, FAKE, FAKE, L=hc.L)) == \
            ff.FF_E_ANCHOR_MISSING
        assert plan(1) == ff.FF_E_ORDER
        assert plan(0, True) == ff.FF_OK                             # cache-extraction call
        assert plan(0) == ff.FF_E_ANCHOR_EXISTS
        assert status(lambda: ff.ff_anchor_bank_publish(hc.ctx, 0, 3, FAKE, FAKE, L=hc.L)) == \
            ff.FF_E_ANCHOR_EXISTS
        assert status(lambda: ff.ff_render_attend(hc.ctx, 0, 0, FAKE, FAKE, FAKE, FAKE, L=hc.L)) == ff.FF_OK
        # block 1 may also be published by the plain anchor publish after its denoising calls
        assert plan(1) == ff.FF_OK
        ff.ff_anchor_bank_publish(hc.ctx, 3, 3, FAKE, FAKE, L=hc.L)
        assert plan(1) == ff.FF_E_ANCHOR_EXISTS and plan(2) == ff.FF_OK
    finally:
        hc.close()


def test_planner_shape_limits():
    L = ff.load(ff.HOSTCHECK_PATH)
    ok = ff.make_shape(n_heads=2, head_dim=64, tokens_per_latent=16)
    assert ff.ff_workspace_bytes(ok, 4, 5, L=L) > 0
    for kw in (dict(planner_latents=0), dict(planner_history=-1),
               dict(planner_history=9, w_ctx=30)):                   # 30 planner sources > 24
        bad = ff.make_shape(n_heads=2, head_dim=64, tokens_per_latent=16, **kw)
        assert ff.ff_workspace_bytes(bad, 4, 5, L=L) == 0, kw


# --------------------------------------------------------------------------
# The library's own rollout driver pieces: wavefront schedule, planner blocks,
# clip counts (host-only calls of libff.so), pinned to the oracle
# --------------------------------------------------------------------------
@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("n_latents", [81, 261])
def test_wavefront_schedule_matches_oracle(n_latents, S):
    L = ff.load(ff.LIB_PATH)
    shape = ff.make_shape(n_heads=2, head_dim=128, tokens_per_latent=16, n_latents=n_latents)
    cfg = orc.FFConfig(tokens_per_latent=16, n_heads=2, head_dim=128, n_latents=n_latents, n_stages=S)
    counts = ff.ff_clip_layout(shape, S, L=L)
    assert counts == {"n_anchors": orc.n_anchors(cfg), "n_chunks": orc.n_chunks(cfg),
                      "n_planner_blocks": len(orc.planner_blocks(cfg)),
                      "n_diagonals": orc.n_chunks(cfg) + S - 1}
    sched = [ff.ff_wavefront(shape, S, t, L=L) for t in range(counts["n_diagonals"])]
    assert sched == orc.schedule(cfg)
    calls = [p for d in sched for p in d]
    assert orc.is_legal_order(cfg, calls)
    assert sorted(calls) == [(i, k) for i in range(orc.n_chunks(cfg)) for k in range(S)]
    for t in (-1, counts["n_diagonals"]):
        with pytest.raises(ff.FFError) as e:
            ff.ff_wavefront(shape, S, t, L=L)
        assert e.value.status == ff.FF_E_RANGE


@pytest.mark.parametrize("n_latents", [3, 42, 81, 261])
def test_planner_blocks_match_oracle(n_latents):
    L = ff.load(ff.LIB_PATH)
    shape = ff.make_shape(n_heads=2, head_dim=128, tokens_per_latent=16, n_latents=n_latents)
    cfg = orc.FFConfig(tokens_per_latent=16, n_heads=2, head_dim=128, n_latents=n_latents)
    n = ff.ff_clip_layout(shape, L=L)["n_planner_blocks"]
    assert [ff.ff_planner_block(shape, b, L=L) for b in range(n)] == orc.planner_blocks(cfg)
    with pytest.raises(ff.FFError) as e:
        ff.ff_planner_block(shape, n, L=L)
    assert e.value.status == ff.FF_E_RANGE


@pytest.mark.parametrize("S", [1, 4])
def test_wavefront_drives_the_order_contract(S):
    """The product schedule, fed to grouped calls, passes the library's own
    order checks for a whole 261-latent clip (348 calls at S = 4)."""
    cfg = orc.FFConfig(tokens_per_latent=16, n_heads=2, head_dim=128, n_latents=261, n_stages=S)
    hc = HostCtx(cfg)
    try:
        _publish_anchors(hc)
        n = ff.ff_clip_layout(hc.shape, S, L=hc.L)["n_diagonals"]
        calls = 0
        for t in range(n):
            diag = ff.ff_wavefront(hc.shape, S, t, L=hc.L)
            m = len(diag)
            ff.ff_render_attend_grouped(hc.ctx, [i for i, _ in diag], [k for _, k in diag], [FAKE] * m,
                                        [FAKE] * m, [FAKE] * m, [FAKE] * m, L=hc.L)
            calls += m
        assert calls == 87 * S
        for k in range(S):
            assert ff.ff_stage_next(hc.ctx, k, L=hc.L) == 87
    finally:
        hc.close()


def test_partial_regions_are_per_stage():
    """Split-item partials: stage k uses region k and planner calls region S, so
    calls of different stages never share partial slots (concurrent streams)."""
    cfg = orc.FFConfig(tokens_per_latent=16, n_heads=2, head_dim=128, n_stages=3)
    hc = HostCtx(cfg)
    f = hc.L.ffstub_last_part
    f.restype = ctypes.c_longlong
    f.argtypes = [ctypes.c_int, ctypes.c_void_p]
    try:
        _, slot_block, slot_off = _layout(cfg)
        part_off = slot_off + 3 * 6 * slot_block
        part_slot = (512 * 130 * 4 + 255) // 256 * 256      # 512 query rows per item at head_dim 128
        region = 256 * 2 * part_slot
        assert hc.need == part_off + 4 * region
        _publish_anchors(hc)
        for t in range(3):
            diag = ff.ff_wavefront(hc.shape, 3, t, L=hc.L)
            m = len(diag)
            ff.ff_render_attend_grouped(hc.ctx, [i for i, _ in diag], [k for _, k in diag], [FAKE] * m,
                                        [FAKE] * m, [FAKE] * m, [FAKE] * m, L=hc.L)
            assert [f(p, hc.ws) for p in range(m)] == [part_off + k * region for _, k in diag]
    finally:
        hc.close()


# --------------------------------------------------------------------------
# Random call sequences: the library accepts exactly the calls the oracle's
# contract accepts, and the banks then hold the same chunk ids
# --------------------------------------------------------------------------
from hypothesis import HealthCheck, given, settings, strategies as st


@settings(max_examples=60, deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])
@given(st.lists(st.tuples(st.sampled_from(["render", "next", "next", "next", "anchors"]), st.integers(0, 28),
                          st.integers(0, 3)), min_size=1, max_size=120),
       st.sampled_from([orc.GAMMA_BRACKET, orc.GAMMA_CENTER_LR]))
def test_random_call_sequences_match_the_oracle_contract(ops, rule):
    cfg = orc.FFConfig(tokens_per_latent=8, n_heads=1, head_dim=64, n_stages=3, history=2, gamma_rule=rule)
    hc = HostCtx(cfg)
    ro = orc.Rollout(cfg)
    blocks = orc.planner_blocks(cfg)
    z = np.zeros((24, 1, 64))
    try:
        for op, a, b in ops:
            if op == "anchors":
                blk = blocks[a % len(blocks)]
                lib_ok = orc_ok = True
                try:
                    ff.ff_anchor_bank_publish(hc.ctx, blk[0], len(blk), FAKE, FAKE, L=hc.L)
                except ff.FFError as e:
                    lib_ok = False
                    assert e.status == ff.FF_E_ANCHOR_EXISTS
                try:
                    ro.publish_anchors(blk[0], np.zeros((8 * len(blk), 1, 64)), np.zeros((8 * len(blk), 1, 64)))
                except orc.ContractError:
                    orc_ok = False
                assert lib_ok == orc_ok
                continue
            # "render": any chunk (27, 28 and stage 3 are out of range); "next": the
            # chunk the stage expects, which may still lack its anchors or stage k-1
            k = b
            i = ro.next_chunk[k] if op == "next" and k < cfg.n_stages else a
            lib_ok = orc_ok = True
            try:
                ff.ff_render_attend(hc.ctx, i, k, FAKE, FAKE, FAKE, FAKE, L=hc.L)
            except ff.FFError as e:
                lib_ok = False
                assert e.status in (ff.FF_E_ORDER, ff.FF_E_ANCHOR_MISSING, ff.FF_E_RANGE)
            try:
                ro.render_attend(i, k, None, z, z, compute=False)
            except orc.ContractError:
                orc_ok = False
            assert lib_ok == orc_ok, (op, i, k)
            if lib_ok:
                assert ff.ff_bank_tail(hc.ctx, k, L=hc.L) == ro.bank_tail(k)[0]
        for k in range(cfg.n_stages):
            assert ff.ff_bank_tail(hc.ctx, k, L=hc.L) == ro.bank_tail(k)[0]
            assert ff.ff_stage_next(hc.ctx, k, L=hc.L) == ro.next_chunk[k]
    finally:
        hc.close()


@pytest.mark.parametrize("seed", range(6))
def test_random_walks_through_whole_clips(seed):
    """Seeded random walks that mostly attempt each stage's next chunk (with
    anchor blocks published in random order along the way) run deep into the
    clip; at every step the library and the oracle accept the same calls, and
    rewinds are checked against the oracle state before the undone call."""
    import copy
    rng = np.random.default_rng(seed)
    cfg = orc.FFConfig(tokens_per_latent=8, n_heads=1, head_dim=64, n_stages=3, history=2,
                       gamma_rule=[orc.GAMMA_BRACKET, orc.GAMMA_CENTER_LR][seed % 2])
    hc = HostCtx(cfg)
    ro = orc.Rollout(cfg)
    undo = {}
    blocks = orc.planner_blocks(cfg)
    order = list(rng.permutation(len(blocks)))
    z = np.zeros((24, 1, 64))
    accepted = 0
    try:
        for _ in range(400):
            r = rng.random()
            if r < 0.05 and order:
                blk = blocks[order.pop()]
                ff.ff_anchor_bank_publish(hc.ctx, blk[0], len(blk), FAKE, FAKE, L=hc.L)
                ro.publish_anchors(blk[0], np.zeros((8 * len(blk), 1, 64)), np.zeros((8 * len(blk), 1, 64)))
                continue
            k = int(rng.integers(0, 3))
            if r < 0.10:                                      # rewind stage k
                try:
                    ff.ff_stage_bank_rewind(hc.ctx, k, L=hc.L)
                    lib_ok = True
                except ff.FFError as e:
                    lib_ok = False
                    assert e.status == ff.FF_E_STATE
                # the oracle side: allowed once per call, only if stage k+1 has not consumed it
                orc_ok = k in undo and not (k + 1 < cfg.n_stages and ro.next_chunk[k + 1] > ro.next_chunk[k] - 1)
                assert lib_ok == orc_ok
                if orc_ok:                                    # stage k back to before its last call
                    snap = undo.pop(k)
                    ro.banks[k] = snap.banks[k]
                    ro.next_chunk[k] = snap.next_chunk[k]
                continue
            i = ro.next_chunk[k] if r < 0.9 else int(rng.integers(0, 27))
            before = copy.deepcopy(ro)
            try:
                ff.ff_render_attend(hc.ctx, i, k, FAKE, FAKE, FAKE, FAKE, L=hc.L)
                lib_ok = True
            except ff.FFError:
                lib_ok = False
            try:
                ro.render_attend(i, k, None, z, z, compute=False)
                orc_ok = True
            except orc.ContractError:
                orc_ok = False
            assert lib_ok == orc_ok, (i, k)
            if orc_ok:
                accepted += 1
                undo[k] = before
            for kk in range(cfg.n_stages):
                assert ff.ff_bank_tail(hc.ctx, kk, L=hc.L) == ro.bank_tail(kk)[0]
        assert accepted >= 40
    finally:
        hc.close()
