"""Side-by-side driver for GPU parity tests: HIP path (through the C ABI) and
the CPU oracle consume the same seeded bytes and are compared call by call."""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

import oracle as orc
import synthetic as syn
from chunked_kv_cache_amd import ff

TOL = {"bf16": 2e-2, "f32": 1e-4}          # O max-abs gates (N(0,1) workloads, |O| << 1)


def bf16_rounding_bound(O_ref: np.ndarray, V_keys: float) -> float:
    """Worst-case |dO| of the bf16 path from its two roundings: each softmax
    weight p is rounded to bf16 before the PV product (relative error <= 2^-9,
    so |dO| <= 2^-9 max|V|) and O is rounded to bf16 (<= half an ulp, which is
    <= 2^-8 |O|).  fp32 accumulation adds far less; 10% margin."""
    return 1.1 * (2.0 ** -8 * float(np.abs(O_ref).max()) + 2.0 ** -9 * float(V_keys))


LSE_TOL = {"bf16": 2e-3, "f32": 1e-4}
RELF_TOL = {"bf16": 1e-2, "f32": 1e-5}     # relative Frobenius (diagnostic gate)


def wavefront(case: "Case"):
    """The library's own anti-diagonal schedule (ff_wavefront), which drives the
    GPU rollouts; a CPU test pins it to the oracle's schedule."""
    shape = case.shape()
    n = ff.ff_clip_layout(shape, case.S)["n_diagonals"]
    return [ff.ff_wavefront(shape, case.S, t) for t in range(n)]


def whole_head_reference(pr: "Pair", i: int, k: int, heads):
    """Oracle O and LSE of call (i, k) on every query row of the given heads,
    from the oracle's state before the call (one head's keys at a time, so
    full-size calls stay cheap).  Returns {head: (O [Lq, 1, d], LSE [1, Lq])}."""
    c = pr.case
    bank = {cid: (Kb, Vb) for cid, Kb, Vb in pr.ro.banks[k]}
    q, kk, vv = pr.gen(i, k)
    out = {}
    for hh in heads:
        one = lambda x: syn.as_f64(x[:, hh:hh + 1], c.dtype)
        ks, vs = [], []
        for kind, idx in pr.ro.key_sources(i, k):
            if kind == "own":
                ks.append(one(kk))
                vs.append(one(vv))
            else:
                Ks, Vs = pr.ro.anchors[idx] if kind == "anchor" else bank[idx]
                ks.append(Ks[:, hh:hh + 1])
                vs.append(Vs[:, hh:hh + 1])
        out[hh] = orc.attention(one(q), np.concatenate(ks), np.concatenate(vs), pr.cfg.scale)
    return out


def check_whole_heads(pr: "Pair", refs) -> list:
    """Compare the last step's device output with whole_head_reference(); returns
    (head, max |dO|, relative Frobenius) per head."""
    res = []
    dt = pr.case.dtype
    for hh, (O_ref, L_ref) in refs.items():
        o, l = pr.last_outs[0]
        O = from_device_f64(o[:, hh:hh + 1])
        L = l[hh:hh + 1].cpu().numpy().astype(np.float64)
        err = np.abs(O - O_ref).max()
        relf = np.linalg.norm(O - O_ref) / np.linalg.norm(O_ref)
        assert err <= TOL[dt] and relf <= RELF_TOL[dt] and np.abs(L - L_ref).max() <= LSE_TOL[dt], (hh, err, relf)
        res.append((hh, err, relf))
    return res


def to_device(x: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def from_device_f64(t) -> np.ndarray:
    import torch
    return t.float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 else \
        t.cpu().numpy().astype(np.float64)


@dataclass
class Case:
    T: int
    nh: int
    d: int
    n_latents: int = 81
    S: int = 4
    H: int = 5
    w_ctx: int = 21
    dtype: str = "bf16"
    rule: str = orc.GAMMA_BRACKET
    seed: int = 0
    q_scale: float = 1.0
    h_p: int = 6

    @property
    def cfg(self) -> orc.FFConfig:
        return orc.FFConfig(tokens_per_latent=self.T, n_heads=self.nh, head_dim=self.d, n_latents=self.n_latents,
                            n_stages=self.S, history=self.H, w_ctx=self.w_ctx, gamma_rule=self.rule,
                            planner_history=self.h_p)

    def shape(self) -> ff.ff_shape:
        return ff.make_shape(n_heads=self.nh, head_dim=self.d, tokens_per_latent=self.T, n_latents=self.n_latents,
                             w_ctx=self.w_ctx, dtype=ff.FF_BF16 if self.dtype == "bf16" else ff.FF_F32,
                             gamma_rule=ff.FF_GAMMA_BRACKET if self.rule == orc.GAMMA_BRACKET
                             else ff.FF_GAMMA_CENTER_LR, planner_history=self.h_p)


@dataclass
class Stats:
    max_abs: float = 0.0
    max_rel_fro: float = 0.0
    max_lse: float = 0.0
    min_control_ratio: float = math.inf
    max_gate_use: float = 0.0              # max over calls of (O max-abs error) / (its gate)
    calls: int = 0
    bank_checks: int = 0


class Pair:
    """GPU context + oracle rollout driven in lockstep."""

    def __init__(self, case: Case, poison_workspace: bool = True, oracle_compute: bool = True,
                 device_bank_check: bool = False):
        import torch
        self.case = case
        self.cfg = case.cfg
        self.banks = ff.StageBanks(case.shape(), case.S, case.H)
        if poison_workspace:
            # NaN everywhere the kernels must not read (spare slots, padding, partials)
            if case.dtype == "bf16":
                self.banks.workspace.view(torch.int16).fill_(0x7FC0)
            else:
                self.banks.workspace[: self.banks.ws_bytes // 4 * 4].view(torch.float32).fill_(float("nan"))
        self.ro = orc.Rollout(self.cfg)
        self.inputs = {}
        self.vmax = {}                       # max |V| per key source, for the rounding bound
        self.stats = Stats()
        self.oracle_compute = oracle_compute
        # full-size cases: compare bank bytes on the device against the exact
        # input tensors (kept while they can still be in a bank)
        self.device_bank_check = device_bank_check
        self.dev_inputs = {}

    @property
    def ctx(self):
        return self.banks.ctx

    def publish_anchors(self):
        c = self.case
        for blk in orc.planner_blocks(self.cfg):
            K, V = syn.anchor_kv(T=c.T, n_heads=c.nh, head_dim=c.d, anchors=blk, seed=c.seed, dtype=c.dtype)
            ff.ff_anchor_bank_publish(self.ctx, blk[0], len(blk), to_device(K, c.dtype), to_device(V, c.dtype))
            V64 = syn.as_f64(V, c.dtype)
            self.ro.publish_anchors(blk[0], syn.as_f64(K, c.dtype), V64)
            for j, a in enumerate(blk):
                self.vmax[("anchor", a)] = float(np.abs(V64[j * c.T:(j + 1) * c.T]).max())

    def gen(self, i, k):
        c = self.case
        return syn.chunk_qkv(T=c.T, n_heads=c.nh, head_dim=c.d, chunk=i, stage=k, seed=c.seed, dtype=c.dtype,
                             q_scale=c.q_scale)

    def step(self, pairs: Sequence[tuple], grouped: bool, rows: Optional[np.ndarray] = None,
             check_bank: bool = True, control: bool = False):
        """Run pairs [(i, k), ...] on the GPU (one grouped call or one call each), then the oracle."""
        import torch
        c = self.case
        host = [self.gen(i, k) for i, k in pairs]
        dev = [[to_device(x, c.dtype) for x in h] for h in host]
        tdt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
        outs = [torch.full_like(d[0], float("nan"), dtype=tdt) for d in dev]
        lses = [torch.full((c.nh, 3 * c.T), float("nan"), dtype=torch.float32, device="cuda") for _ in dev]
        controls = []
        if control:
            for (i, k), h in zip(pairs, host):
                controls.append(self._control(i, k, h, rows))
        if grouped:
            ff.ff_render_attend_grouped(self.ctx, [i for i, _ in pairs], [k for _, k in pairs],
                                        [d[0] for d in dev], [d[1] for d in dev], [d[2] for d in dev], outs, lses)
        else:
            for (i, k), d, o, l in zip(pairs, dev, outs, lses):
                ff.ff_render_attend(self.ctx, i, k, d[0], d[1], d[2], o, l)
        torch.cuda.synchronize()
        self.last_outs = list(zip(outs, lses))          # the whole outputs of the last step, on the device
        results = []
        for j, ((i, k), h) in enumerate(zip(pairs, host)):
            q64, k64, v64 = (syn.as_f64(x, c.dtype) for x in h)
            self.vmax[("history", (i, k))] = float(np.abs(v64).max())
            vkeys = max(self.vmax[("anchor", x)] if kind == "anchor" else self.vmax[("history", (x, k))]
                        for kind, x in self.ro.key_sources(i, k))
            O_ref, L_ref = self.ro.render_attend(i, k, q64, k64, v64, rows=rows, compute=self.oracle_compute)
            if self.device_bank_check:
                self.dev_inputs[(i, k)] = (dev[j][1], dev[j][2])
                self.dev_inputs.pop((i - c.H - 1, k), None)
            else:
                self.inputs[(i, k)] = (h[1], h[2])
            if self.oracle_compute:
                O = from_device_f64(outs[j])
                L = lses[j].cpu().numpy().astype(np.float64)
                if rows is not None:
                    O, L = O[rows], L[:, rows]
                tol = TOL[c.dtype]
                if c.dtype == "bf16":
                    # stress cases with |O| >> 1 (peaked softmax): gate on the rounding bound
                    tol = max(tol, bf16_rounding_bound(O_ref, vkeys))
                self._compare(O, L, O_ref, L_ref, controls[j] if control else None, tol)
                results.append((O, O_ref))
            if check_bank:
                self.check_bank(k)
        return results

    def plan_step(self, b: int, step: int, publish: bool, rows: Optional[np.ndarray] = None,
                  control: bool = False, whole_heads=()):
        """One planner call of block b at denoising step `step` on the GPU, then the oracle.
        `whole_heads`: heads whose every query row is also compared (one head's
        keys at a time); returns (head, max |dO|, relative Frobenius) per such head
        as a third value."""
        import torch
        c = self.case
        blk = orc.planner_blocks(self.cfg)[b]
        n = len(blk) * c.T
        host = syn.planner_qkv(T=c.T, n_heads=c.nh, head_dim=c.d, block=b, step=step, n_latents=len(blk),
                               seed=c.seed, dtype=c.dtype, q_scale=c.q_scale)
        dq, dk, dv = (to_device(x, c.dtype) for x in host)
        tdt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
        out = torch.full_like(dq, float("nan"), dtype=tdt)
        lse = torch.full((c.nh, n), float("nan"), dtype=torch.float32, device="cuda")
        ff.ff_plan_attend(self.ctx, b, dq, dk, dv, out, lse, publish=publish)
        torch.cuda.synchronize()
        q64, k64, v64 = (syn.as_f64(x, c.dtype) for x in host)
        srcs = self.ro.plan_key_sources(b)
        vkeys = max([self.vmax[("anchor", a)] for kind, a in srcs if kind == "anchor"] +
                    [float(np.abs(v64).max())])
        ctrl = None
        if control:
            qc = q64 if rows is None else q64[rows]
            ctrl, _ = orc.attention(qc, k64, v64, self.cfg.scale)        # own latents only
        whole = []
        if whole_heads:
            O_all = from_device_f64(out)
            L_all = lse.cpu().numpy().astype(np.float64)
            for hh in whole_heads:
                h1 = lambda x: np.asarray(x)[:, hh:hh + 1]
                ks = [h1(self.ro.anchors[a][0]) for kind, a in srcs if kind == "anchor"] + [h1(k64)]
                vs = [h1(self.ro.anchors[a][1]) for kind, a in srcs if kind == "anchor"] + [h1(v64)]
                Oh, Lh = orc.attention(h1(q64), np.concatenate(ks), np.concatenate(vs), self.cfg.scale)
                Og = O_all[:, hh:hh + 1]
                err = float(np.abs(Og - Oh).max())
                relf = float(np.linalg.norm(Og - Oh) / np.linalg.norm(Oh))
                dl = float(np.abs(L_all[hh:hh + 1] - Lh).max())
                assert err <= TOL[c.dtype] and relf <= RELF_TOL[c.dtype] and dl <= LSE_TOL[c.dtype], (hh, err, relf, dl)
                whole.append((hh, err, relf))
        O_ref, L_ref = self.ro.plan_attend(b, q64, k64, v64, publish=publish, rows=rows)
        O = from_device_f64(out)
        L = lse.cpu().numpy().astype(np.float64)
        if rows is not None:
            O, L = O[rows], L[:, rows]
        tol = TOL[c.dtype]
        if c.dtype == "bf16":
            tol = max(tol, bf16_rounding_bound(O_ref, vkeys))
        self._compare(O, L, O_ref, L_ref, ctrl, tol)
        if publish:
            for j, a in enumerate(blk):
                self.vmax[("anchor", a)] = float(np.abs(v64[j * c.T:(j + 1) * c.T]).max())
        if whole_heads:
            return O, O_ref, whole
        return O, O_ref

    def _control(self, i, k, host, rows):
        """Negative control: the oracle with the anchor sources dropped."""
        c = self.case
        Kc, Vc = self.ro.gather_keys(i, k, syn.as_f64(host[1], c.dtype), syn.as_f64(host[2], c.dtype))
        n_anchor_tok = c.T * len(orc.gamma(self.cfg, i))
        q = syn.as_f64(host[0], c.dtype)
        if rows is not None:
            q = q[rows]
        O, _ = orc.attention(q, Kc[n_anchor_tok:], Vc[n_anchor_tok:], self.cfg.scale)
        return O

    def _compare(self, O, L, O_ref, L_ref, O_ctrl, tol):
        dt = self.case.dtype
        assert np.all(np.isfinite(O)), "non-finite output"
        err = np.abs(O - O_ref).max()
        relf = np.linalg.norm(O - O_ref) / np.linalg.norm(O_ref)
        lerr = np.abs(L - L_ref).max()
        st = self.stats
        st.max_abs = max(st.max_abs, err)
        st.max_rel_fro = max(st.max_rel_fro, relf)
        st.max_lse = max(st.max_lse, lerr)
        st.max_gate_use = max(st.max_gate_use, err / tol)
        st.calls += 1
        assert err <= tol, f"O max-abs {err:.3e} > {tol:.3e}"
        assert relf <= RELF_TOL[dt], f"O rel-Frobenius {relf:.3e} > {RELF_TOL[dt]}"
        assert lerr <= LSE_TOL[dt], f"LSE max-abs {lerr:.3e} > {LSE_TOL[dt]}"
        if O_ctrl is not None:
            ratio = np.linalg.norm(O - O_ctrl) / max(np.linalg.norm(O - O_ref), 1e-30)
            st.min_control_ratio = min(st.min_control_ratio, ratio)
            assert ratio >= 10.0, f"GPU only {ratio:.1f}x closer to the oracle than to the anchor-less control"

    def check_bank(self, k):
        """B_k ids and bytes must equal the oracle's bank and the generated bits exactly."""
        import torch
        c = self.case
        ids_ref, K_ref, V_ref = self.ro.bank_tail(k)
        n = len(ids_ref)
        tdt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
        Ko = torch.empty((max(n, 1) * 3 * c.T, c.nh, c.d), dtype=tdt, device="cuda")
        Vo = torch.empty_like(Ko)
        ids = ff.ff_bank_tail(self.ctx, k, Ko, Vo)
        assert ids == ids_ref
        if n == 0:
            return
        torch.cuda.synchronize()
        if self.device_bank_check:
            L = 3 * c.T
            for j, cid in enumerate(ids):
                kin, vin = self.dev_inputs[(cid, k)]
                assert torch.equal(Ko[j * L:(j + 1) * L].view(torch.int16), kin.view(torch.int16))
                assert torch.equal(Vo[j * L:(j + 1) * L].view(torch.int16), vin.view(torch.int16))
            self.stats.bank_checks += 1
            return
        kbits = np.concatenate([self.inputs[(i, k)][0] for i in ids])
        vbits = np.concatenate([self.inputs[(i, k)][1] for i in ids])
        view = (lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)) if c.dtype == "bf16" else \
            (lambda t: t.cpu().numpy())
        assert np.array_equal(view(Ko), kbits) and np.array_equal(view(Vo), vbits)
        assert np.array_equal(from_device_f64(Ko), K_ref) and np.array_equal(from_device_f64(Vo), V_ref)
        self.stats.bank_checks += 1

    def close(self):
        record(self.stats)
        self.banks.close()


# Error statistics of every parity case of the session; conftest writes them
# to the file named by FF_PARITY_SUMMARY (if set) when the session ends.
RECORDS: List[tuple] = []


def record(stats: "Stats", label: Optional[str] = None) -> None:
    import os
    name = label or os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    if stats.calls:
        RECORDS.append((name, stats))
