"""GPU parity of the block-causal forward and backward against the float64 oracle.

Inputs are the seeded clip tensors of ``synthetic`` (chunk i's Q, K, V are the
renderer inputs of (i, stage 0); dO is drawn from the same family).  The
workspace and every output are filled with NaN first, so an unwritten output
element or a read of a byte the call should not read shows up.

Gates.  O and LSE: as for the renderer call (bf16 max-abs 2e-2 and the
rounding bound, LSE 2e-3; fp32 1e-4).  Gradients: every product term of a
gradient carries one factor rounded to bf16 (P or dS, relative error at most
2^-8) and the output is rounded once more (at most 2^-8 relative), with fp32
accumulation in between; the gates are max|err| <= 2^-5 max|ref| (a few
elements may see both roundings aligned) and relative Frobenius error <= 1e-2
(about 2.5 x 2^-8).  fp32: 1e-4 and 1e-5.  A control compares the same GPU
result with the oracle of a one-chunk-shorter history window and must miss
the gates by 10x.
"""
from dataclasses import dataclass

import numpy as np
import pytest

import oracle as orc
import synthetic as syn
from chunked_kv_cache_amd import ff
from ffharness import LSE_TOL, TOL, bf16_rounding_bound, from_device_f64, to_device

pytestmark = pytest.mark.gpu

GRAD_TOL = {"bf16": (2.0 ** -5, 1e-2), "f32": (1e-4, 1e-5)}   # (max|err| / max|ref|, relative Frobenius)


@dataclass
class BcCase:
    T: int
    nh: int
    d: int
    n_latents: int = 81
    H: int = 5
    w_ctx: int = 21
    rule: str = orc.GAMMA_BRACKET
    dtype: str = "bf16"
    seed: int = 0
    q_scale: float = 1.0
    stride: int = 10

    @property
    def cfg(self):
        return orc.FFConfig(tokens_per_latent=self.T, n_heads=self.nh, head_dim=self.d, n_latents=self.n_latents,
                            history=self.H, w_ctx=self.w_ctx, gamma_rule=self.rule, anchor_stride=self.stride)

    def shape(self):
        return ff.make_shape(n_heads=self.nh, head_dim=self.d, tokens_per_latent=self.T, n_latents=self.n_latents,
                             anchor_stride=self.stride, w_ctx=self.w_ctx,
                             dtype=ff.FF_BF16 if self.dtype == "bf16" else ff.FF_F32,
                             gamma_rule=ff.FF_GAMMA_BRACKET if self.rule == orc.GAMMA_BRACKET
                             else ff.FF_GAMMA_CENTER_LR)

    def inputs(self):
        cfg = self.cfg
        Ka, Va = syn.anchor_kv(T=self.T, n_heads=self.nh, head_dim=self.d, anchors=range(orc.n_anchors(cfg)),
                               seed=self.seed, dtype=self.dtype)
        Q, K, V, dO = syn.clip_tensors(T=self.T, n_heads=self.nh, head_dim=self.d, n_chunks=orc.n_chunks(cfg),
                                       seed=self.seed, dtype=self.dtype, q_scale=self.q_scale)
        return Ka, Va, Q, K, V, dO


def _nan_like(t):
    import torch
    return torch.full_like(t, float("nan"))


def run_gpu(case: BcCase, host, head=None):
    """Forward and backward through the C ABI; returns float64 host arrays
    (of one head only if `head` is given).  Every output must be finite."""
    import torch
    bc = ff.BlockCausal(case.shape(), case.H)
    try:
        if case.dtype == "bf16":
            bc.workspace.view(torch.int16).fill_(0x7FC0)
        else:
            bc.workspace[: bc.ws_bytes // 4 * 4].view(torch.float32).fill_(float("nan"))
        Ka, Va, Q, K, V, dO = (to_device(x, case.dtype) for x in host)
        nc, L = orc.n_chunks(case.cfg), case.cfg.chunk_tokens
        O = _nan_like(Q)
        lse = torch.full((nc, case.nh, L), float("nan"), dtype=torch.float32, device="cuda")
        ff.ff_bc_forward(bc.ctx, Ka, Va, Q, K, V, O, lse)
        dQ, dK, dV, dKa, dVa = _nan_like(Q), _nan_like(K), _nan_like(V), _nan_like(Ka), _nan_like(Va)
        ff.ff_bc_backward(bc.ctx, Ka, Va, Q, K, V, O, lse, dO, dQ, dK, dV, dKa, dVa)
        torch.cuda.synchronize()
        outs = dict(O=O, lse=lse, dQ=dQ, dK=dK, dV=dV, dKa=dKa, dVa=dVa)
        for k, t in outs.items():
            assert bool(torch.isfinite(t).all()), f"non-finite {k} (unwritten element or bad read)"
        if head is not None:
            outs = {k: t[:, head:head + 1, :] for k, t in outs.items()}
        return {k: from_device_f64(t) for k, t in outs.items()}
    finally:
        bc.close()


def grad_err(got, ref):
    m = float(np.abs(ref).max())
    return float(np.abs(got - ref).max()) / m, float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def check(case: BcCase, got, ref_O, ref_lse, ref_grads, rows=slice(None), sources=None, control=None):
    """Compare forward and gradients; `rows` selects query rows, `sources` key rows."""
    tol_max, tol_fro = GRAD_TOL[case.dtype]
    o_err = float(np.abs(got["O"][rows] - ref_O[rows]).max())
    l_err = float(np.nanmax(np.abs(got["lse"] - ref_lse)))
    assert o_err <= TOL[case.dtype], o_err
    assert l_err <= LSE_TOL[case.dtype], l_err
    report = {"O": o_err, "lse": l_err}
    names = ["dQ", "dK", "dV", "dKa", "dVa"]
    for n, ref in zip(names, ref_grads):
        sel = rows if n == "dQ" else (sources or {}).get(n, slice(None))
        if isinstance(sel, list) and not sel:
            continue
        e_max, e_fro = grad_err(got[n][sel], ref[sel])
        assert e_max <= tol_max and e_fro <= tol_fro, (n, e_max, e_fro)
        report[n] = (e_max, e_fro)
        if control is not None and n in ("dQ", "dK"):
            c_max, c_fro = grad_err(got[n][sel], control[names.index(n)][sel])
            assert c_fro >= 10 * tol_fro, (n, "control within gate", c_fro)
    return report


def full_case(case: BcCase, control=False):
    host = case.inputs()
    got = run_gpu(case, host)
    f64 = [syn.as_f64(x, case.dtype) for x in host]
    cfg = case.cfg
    O, LSE = orc.bc_forward(cfg, *f64[:5])
    grads = orc.bc_backward(cfg, *f64)
    ctl = None
    if control:
        import dataclasses
        short = dataclasses.replace(cfg, history=cfg.history - 1)
        ctl = orc.bc_backward(short, *f64)
    if case.dtype == "bf16":
        bound = bf16_rounding_bound(O, float(np.abs(f64[4]).max()))
        assert float(np.abs(got["O"] - O).max()) <= bound
    return check(case, got, O, LSE, grads, control=ctl)


def test_bc_tiny_fp32():
    """fp32, 2 heads, d=64, T=16, 81 latents: 27 chunks, 9 anchors, H=5."""
    r = full_case(BcCase(T=16, nh=2, d=64, dtype="f32"))
    print("bc tiny fp32:", r)


@pytest.mark.parametrize("rule", [orc.GAMMA_BRACKET, orc.GAMMA_CENTER_LR])
def test_bc_bf16_multi_tile_ragged(rule):
    """T=200: 600 queries per chunk (3 dQ tiles of 256, ragged), 200-key anchors (ragged 64-key tiles)."""
    r = full_case(BcCase(T=200, nh=2, d=128, n_latents=36, rule=rule), control=True)
    print(f"bc bf16 T=200 {rule}:", r)


def test_bc_bf16_w_ctx_cap_and_short_history():
    r = full_case(BcCase(T=72, nh=2, d=128, n_latents=36, w_ctx=11, H=3))
    print("bc bf16 capped:", r)


def test_bc_bf16_head_dim_64_peaked():
    r = full_case(BcCase(T=40, nh=3, d=64, n_latents=24, H=2, q_scale=4.0))
    print("bc bf16 d=64 peaked:", r)


@pytest.mark.parametrize("case", [
    BcCase(T=8, nh=1, d=128, n_latents=24, H=1, dtype="f32"),          # fp32 at d=128, one history chunk
    BcCase(T=64, nh=2, d=128, n_latents=30, H=1, rule=orc.GAMMA_CENTER_LR),   # whole 64-query tiles
    BcCase(T=8, nh=4, d=64, n_latents=12, H=5),                        # smallest tiles, bank never full
    BcCase(T=24, nh=2, d=128, n_latents=45, H=8, w_ctx=30, stride=7),  # H = 8, anchor stride 7
    BcCase(T=16, nh=2, d=128, n_latents=3),                            # one chunk, one anchor
    BcCase(T=16, nh=2, d=128, n_latents=6),                            # two chunks, one anchor
], ids=["f32_d128_H1", "bf16_center_lr_H1", "bf16_T8", "bf16_H8_stride7", "bf16_1chunk", "bf16_2chunks"])
def test_bc_small_edge_cases(case):
    r = full_case(case)
    print(f"bc edge {case.dtype} T={case.T} d={case.d} H={case.H}:", r)


def test_bc_context_reused_across_calls():
    """Two forward + backward passes with different inputs on one context: the
    workspace is scratch, so the second result depends on its own inputs only."""
    import torch
    cases = [BcCase(T=64, nh=2, d=128, n_latents=24, H=2, seed=s) for s in (3, 4)]
    bc = ff.BlockCausal(cases[0].shape(), cases[0].H)
    try:
        bc.workspace.view(torch.int16).fill_(0x7FC0)
        for case in cases:
            host = case.inputs()
            Ka, Va, Q, K, V, dO = (to_device(x, case.dtype) for x in host)
            nc, L = orc.n_chunks(case.cfg), case.cfg.chunk_tokens
            O = _nan_like(Q)
            lse = torch.full((nc, case.nh, L), float("nan"), dtype=torch.float32, device="cuda")
            ff.ff_bc_forward(bc.ctx, Ka, Va, Q, K, V, O, lse)
            grads = [_nan_like(x) for x in (Q, K, V, Ka, Va)]
            ff.ff_bc_backward(bc.ctx, Ka, Va, Q, K, V, O, lse, dO, *grads)
            torch.cuda.synchronize()
            f64 = [syn.as_f64(x, case.dtype) for x in host]
            O_ref, LSE_ref = orc.bc_forward(case.cfg, *f64[:5])
            refs = orc.bc_backward(case.cfg, *f64)
            got = dict(O=from_device_f64(O), lse=from_device_f64(lse),
                       **{n: from_device_f64(g) for n, g in zip(("dQ", "dK", "dV", "dKa", "dVa"), grads)})
            check(case, got, O_ref, LSE_ref, refs)
    finally:
        bc.close()


def test_bc_forward_equals_inference_calls():
    """Chunk i's forward rows equal ff_render_attend(i, 0) on the same bytes, bit for bit."""
    import torch
    case = BcCase(T=200, nh=2, d=128, n_latents=36)
    host = case.inputs()
    got = run_gpu(case, host)
    banks = ff.StageBanks(case.shape(), 1, case.H)
    try:
        Ka, Va, Q, K, V, _ = (to_device(x, case.dtype) for x in host)
        T, L = case.T, case.cfg.chunk_tokens
        for blk in orc.planner_blocks(case.cfg):
            r = slice(blk[0] * T, (blk[-1] + 1) * T)
            ff.ff_anchor_bank_publish(banks.ctx, blk[0], len(blk), Ka[r].contiguous(), Va[r].contiguous())
        for i in range(orc.n_chunks(case.cfg)):
            r = slice(i * L, (i + 1) * L)
            O = torch.empty_like(Q[r])
            lse = torch.empty((case.nh, L), dtype=torch.float32, device="cuda")
            ff.ff_render_attend(banks.ctx, i, 0, Q[r].contiguous(), K[r].contiguous(), V[r].contiguous(), O, lse)
            torch.cuda.synchronize()
            assert np.array_equal(from_device_f64(O), got["O"][r]), i
            assert np.array_equal(from_device_f64(lse), got["lse"][i]), i
    finally:
        banks.close()


def test_bc_480p_sampled():
    """480p clip (T=1560, 12 heads, d=128, 81 latents) run whole on the GPU; one head checked
    on query chunks 0..5 and 26, which complete the gradients of chunks 0 and 26 and anchor 0."""
    case = BcCase(T=1560, nh=12, d=128)
    cfg = case.cfg
    host = case.inputs()
    h = 5
    mine = run_gpu(case, host, head=h)
    one = [syn.as_f64(x[:, h:h + 1, :], case.dtype) for x in host]
    del host
    cfg1 = orc.FFConfig(tokens_per_latent=case.T, n_heads=1, head_dim=case.d)
    chunks = [0, 1, 2, 3, 4, 5, 26]
    O, LSE = orc.bc_forward(cfg1, *one[:5], chunks=chunks)
    grads = orc.bc_backward(cfg1, *one, chunks=chunks)
    anchors, srcs = orc.bc_complete_sources(cfg, chunks)
    assert srcs == [0, 26] and anchors == [0]
    T, L = case.T, cfg.chunk_tokens
    rows = np.concatenate([np.arange(i * L, (i + 1) * L) for i in chunks])
    key_rows = np.concatenate([np.arange(j * L, (j + 1) * L) for j in srcs])
    anc_rows = np.concatenate([np.arange(a * T, (a + 1) * T) for a in anchors])
    r = check(case, mine, O, LSE, grads, rows=rows,
              sources={"dK": key_rows, "dV": key_rows, "dKa": anc_rows, "dVa": anc_rows})
    print("bc 480p head 5:", r)


def test_bc_720p_last_chunk():
    """720p clip (T=3600, 40 heads, d=128, 81 latents: 10800-query chunks, 72000 keys) run whole
    on the GPU; one head checked on chunk 26, which alone completes the gradients of its own keys."""
    case = BcCase(T=3600, nh=40, d=128)
    cfg = case.cfg
    host = case.inputs()
    h = 17
    mine = run_gpu(case, host, head=h)
    one = [syn.as_f64(x[:, h:h + 1, :], case.dtype) for x in host]
    del host
    cfg1 = orc.FFConfig(tokens_per_latent=case.T, n_heads=1, head_dim=case.d)
    chunks = [26]
    O, LSE = orc.bc_forward(cfg1, *one[:5], chunks=chunks)
    grads = orc.bc_backward(cfg1, *one, chunks=chunks)
    anchors, srcs = orc.bc_complete_sources(cfg, chunks)
    assert srcs == [26] and anchors == []
    L = cfg.chunk_tokens
    rows = np.arange(26 * L, 27 * L)
    r = check(case, mine, O, LSE, grads, rows=rows, sources={"dK": rows, "dV": rows, "dKa": [], "dVa": []})
    print("bc 720p head 17 chunk 26:", r)
