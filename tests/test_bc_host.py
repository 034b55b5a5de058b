"""CPU tests of the block-causal calls of the C ABI against the oracle.

Run on libff_hostcheck.so (the host source linked against a recording stub):
the key plan of every chunk, the source tables handed to the forward's
attention launches, the key ranges and reader runs handed to the backward
kernels, and the argument checks.  No GPU.
"""
import ctypes

import numpy as np
import pytest

import oracle as orc
from chunked_kv_cache_amd import ff

FAKE = 1 << 20      # 16-byte aligned stand-in device addresses; the stub never reads them
KIND = {ff.FF_SRC_ANCHOR: "anchor", ff.FF_SRC_HISTORY: "chunk", ff.FF_SRC_OWN: "chunk"}


def _aligned_buffer(nbytes):
    raw = np.zeros(nbytes + 512, dtype=np.uint8)
    return raw, (raw.ctypes.data + 255) // 256 * 256


class HostBc:
    def __init__(self, cfg: orc.FFConfig, dtype=ff.FF_BF16):
        self.L = ff.load(ff.HOSTCHECK_PATH)
        self.cfg = cfg
        rule = ff.FF_GAMMA_BRACKET if cfg.gamma_rule == orc.GAMMA_BRACKET else ff.FF_GAMMA_CENTER_LR
        self.shape = ff.make_shape(n_heads=cfg.n_heads, head_dim=cfg.head_dim,
                                   tokens_per_latent=cfg.tokens_per_latent, chunk_latents=cfg.chunk_latents,
                                   anchor_stride=cfg.anchor_stride, n_latents=cfg.n_latents, w_ctx=cfg.w_ctx,
                                   dtype=dtype, gamma_rule=rule)
        self.need = ff.ff_bc_workspace_bytes(self.shape, cfg.history, L=self.L)
        assert self.need > 0
        self.raw, self.ws = _aligned_buffer(self.need)
        self.ctx = ff.ff_bc_create(self.shape, cfg.history, self.ws, self.need, L=self.L)

    def counts(self):
        c = [ctypes.c_int() for _ in range(6)]
        self.L.ffstub_counts(*[ctypes.byref(x) for x in c[:4]])
        self.L.ffstub_bc_counts(ctypes.byref(c[4]), ctypes.byref(c[5]))
        return {k: x.value for k, x in zip(("attn", "publish", "anchor", "unpack", "layout", "bwd"), c)}

    def segments(self, p):
        off = (ctypes.c_longlong * ff.FF_MAX_SOURCES)()
        n = (ctypes.c_int * ff.FF_MAX_SOURCES)()
        lk, ns = ctypes.c_int(), ctypes.c_int()
        f = self.L.ffstub_last_segments
        f.argtypes = [ctypes.c_int, ctypes.c_void_p] + [ctypes.c_void_p] * 4
        k = f(p, self.ws, off, n, ctypes.byref(lk), ctypes.byref(ns))
        return list(off[:k]), list(n[:k]), lk.value

    def attn_pairs(self):
        nwg = ctypes.c_int()
        return self.L.ffstub_last_attn_pairs(ctypes.byref(nwg))

    def bc_chunk(self, i):
        v = [ctypes.c_int() for _ in range(4)]
        self.L.ffstub_last_bc_chunk(i, *[ctypes.byref(x) for x in v])
        return tuple(x.value for x in v)

    def bc_readers(self, s):
        i0, n = ctypes.c_int(), ctypes.c_int()
        self.L.ffstub_last_bc_readers(s, ctypes.byref(i0), ctypes.byref(n))
        return i0.value, n.value

    def copy_jobs(self):
        rk, rv = ctypes.c_void_p(), ctypes.c_void_p()
        nseg, Lt = ctypes.c_int(), ctypes.c_int()
        f = self.L.ffstub_last_copy_job
        f.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 4
        n = f(0, ctypes.byref(rk), ctypes.byref(rv), ctypes.byref(nseg), ctypes.byref(Lt))
        jobs = []
        for j in range(n):
            f(j, ctypes.byref(rk), ctypes.byref(rv), ctypes.byref(nseg), ctypes.byref(Lt))
            jobs.append((rk.value, rv.value, nseg.value))
        return jobs, Lt.value

    def close(self):
        ff.ff_bc_destroy(self.ctx, L=self.L)


CONFIGS = [
    dict(tokens_per_latent=16, n_heads=2, head_dim=64),
    dict(tokens_per_latent=16, n_heads=2, head_dim=64, history=2),
    dict(tokens_per_latent=16, n_heads=2, head_dim=64, n_latents=36, w_ctx=11),
    dict(tokens_per_latent=16, n_heads=2, head_dim=128, gamma_rule=orc.GAMMA_CENTER_LR),
    dict(tokens_per_latent=8, n_heads=1, head_dim=64, n_latents=261),
    dict(tokens_per_latent=8, n_heads=1, head_dim=64, n_latents=288, history=8),        # 96 chunks, H max
    dict(tokens_per_latent=8, n_heads=1, head_dim=64, n_latents=60, history=1, w_ctx=5),
    dict(tokens_per_latent=8, n_heads=1, head_dim=64, n_latents=45, anchor_stride=7),  # stride not 10
]


def _plan(ks):
    return [(KIND[ks.kind[j]], ks.id[j]) for j in range(ks.n_sources)]


@pytest.mark.parametrize("kw", CONFIGS)
def test_key_plan_matches_oracle(kw):
    cfg = orc.FFConfig(**kw)
    hb = HostBc(cfg)
    try:
        for i in range(orc.n_chunks(cfg)):
            ks = ff.ff_bc_key_plan(hb.ctx, i, L=hb.L)
            want = orc.bc_key_sources(cfg, i)
            assert _plan(ks) == want
            assert ks.kind[ks.n_sources - 1] == ff.FF_SRC_OWN
            assert ks.key_tokens == sum(cfg.tokens_per_latent if k == "anchor" else cfg.chunk_tokens
                                        for k, _ in want)
    finally:
        hb.close()


@pytest.mark.parametrize("kw", CONFIGS)
def test_forward_launches_match_oracle(kw):
    cfg = orc.FFConfig(**kw)
    hb = HostBc(cfg)
    T, Lq, nh, d = cfg.tokens_per_latent, cfg.chunk_tokens, cfg.n_heads, cfg.head_dim
    al = lambda x: (x + 255) // 256 * 256
    blk_a, blk_c = al(2 * nh * T * d * 2), al(2 * nh * Lq * d * 2)
    na, nc = orc.n_anchors(cfg), orc.n_chunks(cfg)
    kv_chunk = 2 * al(na * blk_a)          # after the anchors' K/V^T and V/K^T blocks
    try:
        before = hb.counts()
        ff.ff_bc_forward(hb.ctx, FAKE, FAKE + 16, FAKE + 32, FAKE + 48, FAKE + 64, FAKE + 80, None, L=hb.L)
        after = hb.counts()
        assert after["layout"] - before["layout"] == 2
        assert after["attn"] - before["attn"] == (nc + 7) // 8
        jobs, Lt = hb.copy_jobs()           # the last copy: every chunk's K, V
        assert jobs == [(FAKE + 48, FAKE + 64, nc)] and Lt == Lq
        first = (nc - 1) // 8 * 8           # chunks of the last attention launch
        assert hb.attn_pairs() == nc - first
        for p in range(nc - first):
            i = first + p
            off, n, lk = hb.segments(p)
            want = orc.bc_key_sources(cfg, i)
            assert off == [a * blk_a if k == "anchor" else kv_chunk + a * blk_c for k, a in want]
            assert n == [T if k == "anchor" else Lq for k, _ in want]
            assert lk == sum(n)
    finally:
        hb.close()


@pytest.mark.parametrize("kw", CONFIGS)
def test_backward_tables_match_oracle(kw):
    cfg = orc.FFConfig(**kw)
    hb = HostBc(cfg)
    na, nc = orc.n_anchors(cfg), orc.n_chunks(cfg)
    mask = orc.bc_mask(cfg)
    try:
        before = hb.counts()
        ff.ff_bc_backward(hb.ctx, *[FAKE + 16 * k for k in range(13)], L=hb.L)
        after = hb.counts()
        assert after["layout"] - before["layout"] == 2 and after["bwd"] - before["bwd"] == 1
        jobs, Lt = hb.copy_jobs()           # chunk operands: K|V^T, V|K^T, Q|Q^T, dO|dO^T
        K, V, Q, dO = FAKE + 48, FAKE + 64, FAKE + 32, FAKE + 112
        assert jobs == [(K, V, nc), (V, K, nc), (Q, Q, nc), (dO, dO, nc)] and Lt == cfg.chunk_tokens
        for i in range(nc):
            a0, n_a, j0, nj = hb.bc_chunk(i)
            src = orc.bc_key_sources(cfg, i)
            assert [("anchor", a) for a in range(a0, a0 + n_a)] == [s for s in src if s[0] == "anchor"]
            assert [("chunk", j) for j in range(j0, j0 + nj)] == [s for s in src if s[0] == "chunk"]
        for s in range(na + nc):
            i0, n = hb.bc_readers(s)
            readers = np.nonzero(mask[:, s])[0].tolist()
            assert list(range(i0, i0 + n)) == readers
    finally:
        hb.close()


def test_argument_checks():
    cfg = orc.FFConfig(tokens_per_latent=16, n_heads=2, head_dim=64)
    hb = HostBc(cfg)
    try:
        def status(fn):
            try:
                fn()
                return ff.FF_OK
            except ff.FFError as e:
                return e.status
        p = [FAKE + 16 * k for k in range(13)]
        assert status(lambda: ff.ff_bc_forward(hb.ctx, *p[:6], L=hb.L)) == ff.FF_OK
        assert status(lambda: ff.ff_bc_forward(hb.ctx, None, *p[1:6], L=hb.L)) == ff.FF_E_INVAL
        assert status(lambda: ff.ff_bc_forward(hb.ctx, *p[:5], FAKE + 8, L=hb.L)) == ff.FF_E_INVAL
        assert status(lambda: ff.ff_bc_forward(hb.ctx, *p[:6], FAKE + 2, L=hb.L)) == ff.FF_E_INVAL
        for k in range(13):             # every backward pointer is required and aligned
            q = list(p)
            q[k] = None
            assert status(lambda: ff.ff_bc_backward(hb.ctx, *q, L=hb.L)) == ff.FF_E_INVAL
        assert status(lambda: ff.ff_bc_key_plan(hb.ctx, orc.n_chunks(cfg), L=hb.L)) == ff.FF_E_RANGE
        # workspace too small; clip over the chunk limit
        with pytest.raises(ff.FFError) as e:
            ff.ff_bc_create(hb.shape, cfg.history, hb.ws, hb.need - 1, L=hb.L)
        assert e.value.status == ff.FF_E_NOSPACE
        big = ff.make_shape(n_heads=2, head_dim=64, tokens_per_latent=16, n_latents=3 * 97)
        assert ff.ff_bc_workspace_bytes(big, 5, L=hb.L) == 0
        ok = ff.make_shape(n_heads=2, head_dim=64, tokens_per_latent=16, n_latents=3 * 96, anchor_stride=10)
        assert ff.ff_bc_workspace_bytes(ok, 5, L=hb.L) > 0
    finally:
        hb.close()


def test_product_library_validates_block_causal_calls_before_device_work():
    """libff.so checks the block-causal calls before touching the GPU, so these run on a CPU host."""
    L = ff.load(ff.LIB_PATH)
    shape = ff.make_shape(n_heads=2, head_dim=128, tokens_per_latent=16)
    need = ff.ff_bc_workspace_bytes(shape, 5, L=L)
    assert need > 0
    raw, addr = _aligned_buffer(need)
    bc = ff.ff_bc_create(shape, 5, addr, need, L=L)
    try:
        with pytest.raises(ff.FFError) as e:
            ff.ff_bc_forward(bc, None, FAKE, FAKE, FAKE, FAKE, FAKE, L=L)
        assert e.value.status == ff.FF_E_INVAL
        with pytest.raises(ff.FFError) as e:        # lse is required by the backward
            ff.ff_bc_backward(bc, *[FAKE] * 6, None, *[FAKE] * 6, L=L)
        assert e.value.status == ff.FF_E_INVAL
        assert ff.ff_bc_key_plan(bc, 26, L=L).key_tokens == 16 * 20
    finally:
        ff.ff_bc_destroy(bc, L=L)
    bad = ff.make_shape(n_heads=2, head_dim=96, tokens_per_latent=16)
    assert ff.ff_bc_workspace_bytes(bad, 5, L=L) == 0
    with pytest.raises(ff.FFError) as e:
        ff.ff_bc_create(bad, 5, addr, need, L=L)
    assert e.value.status == ff.FF_E_INVAL
