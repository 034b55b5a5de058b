"""CPU float64 oracle for FlashForward's renderer attention step and its banks.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module; only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it.  It shares no code with the HIP library: it reads
plain numpy arrays (the seeded bytes from ``synthetic``, widened to float64 by
the caller) and computes everything from the definitions below, slowly and in
the order the pages give.

Pages cited (title, then the part of the page):
  [S] "In-Flight KV Cache with Clean Anchors for Faster Autoregressive Video
      Diffusion" -- Korean summary page ("FlashForward가 디노이징 중 KV 캐시를
      재사용해 자기회귀 영상 생성을 가속한다"), sections 무엇인가 (what it is),
      어떻게 동작하나 (how it works, Eq. (2)), 무엇과 다른가 (how it differs),
      어떻게 쓰나 (how it is used), 전제와 한계 (assumptions and limits).
  [A] "In-Flight KV Cache with Clean Anchors for Faster Autoregressive Video
      Diffusion" -- abstract page with Korean notes.
  [C] "In-Flight KV Cache 与 Clean Anchors：更快的自回归视频扩散" -- Chinese notes,
      section 方法 (method).

Readings taken where the pages are silent:
  R1  Gamma(i) is never written out.  Default "bracket": every anchor whose
      position lies in [D*floor(first/D), D*ceil(last/D)] for the chunk's first
      and last latent positions (two-sided for every latent of the chunk).
      Alternative "center_lr": the anchor at or left of the chunk's middle
      latent and the next one to its right.
  R2  W_ctx counts key latents per renderer call; past it the oldest history
      chunks are dropped first (never binding at the pages' hyper-parameters).
  R3  Before the bank fills, B_k^(i) holds the i chunks published so far.
  R4  No mask: every query attends every key of the three sources.
  R5  Attention of call i reads B_k^(i) (history only) plus the chunk's own
      in-flight K/V; the publish of (i, K, V) follows and defines B_k^(i+1).
  R6  Softmax scale is 1/sqrt(head_dim).
  R7  Anchors are published once each, in planner blocks, and never evicted.
  R8  Call (i, k) also requires (i, k-1) to have run (the same-stage /
      previous-stage dependency of the wavefront schedule).
  R11 Planner block b attends the clean anchor KV of the previous min(b, H_P)
      planner blocks (H_P counts blocks: 6 x 3 + 3 = 21 = W_ctx) plus its own
      in-flight K/V, with no mask inside; past W_ctx the oldest blocks are
      dropped first.  The cache-extraction forward is the planner call whose
      own K/V becomes the block's published anchor KV.
  R12 Planner blocks run in order: block b needs blocks 0..b-1 published and
      block b not yet published.

Parity status per function is stated in each docstring.  gamma() and the W_ctx
cap are "parity unpinned": no page prints the rule, so they are pinned only by
the properties the pages do state (two-sided, budget 21) and by our reading.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

GAMMA_BRACKET = "bracket"
GAMMA_CENTER_LR = "center_lr"


class ContractError(RuntimeError):
    """A call that the state contract forbids (order, missing anchor, range)."""


# ---------------------------------------------------------------------------
# Configuration  ([S] how it differs: B_P = B_R = 3, D = 10, S = 4, W_ctx = 21,
# H = 5, H_P = 6; 81 latent positions in the worked example)
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class FFConfig:
    tokens_per_latent: int          # T (patch tokens of one latent frame)
    n_heads: int
    head_dim: int
    n_latents: int = 81             # latent positions of the clip
    chunk_latents: int = 3          # B_R
    planner_block: int = 3          # B_P
    anchor_stride: int = 10         # D (Delta)
    n_stages: int = 4               # S
    history: int = 5                # H
    planner_history: int = 6        # H_P, in planner blocks (reading R11)
    w_ctx: int = 21                 # context budget in latents
    gamma_rule: str = GAMMA_BRACKET

    @property
    def scale(self) -> float:
        """Reading R6: 1/sqrt(head_dim)."""
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def chunk_tokens(self) -> int:
        return self.chunk_latents * self.tokens_per_latent


def anchor_positions(cfg: FFConfig) -> List[int]:
    """Latent positions of the clean anchors: 0, D, 2D, ... inside the clip.

    [S] how it differs: for 81 latents the planner makes anchors at
    {0, 10, ..., 80}, nine in all.
    """
    return list(range(0, cfg.n_latents, cfg.anchor_stride))


def n_anchors(cfg: FFConfig) -> int:
    return len(anchor_positions(cfg))


def planner_blocks(cfg: FFConfig) -> List[List[int]]:
    """Anchor ids grouped by planner block, in generation order.

    [S] how it differs: anchors are produced B_P = 3 at a time; after each
    completed block one cache-extraction forward publishes its clean KV.
    """
    ids = list(range(n_anchors(cfg)))
    return [ids[b:b + cfg.planner_block] for b in range(0, len(ids), cfg.planner_block)]


def planner_key_blocks(cfg: FFConfig, b: int) -> List[int]:
    """Planner blocks whose clean anchor KV planner block b attends, oldest first.

    [S] how it differs: planner history H_P = 6; [S] training paragraph: a
    planner block attends causally to the clean KV of earlier blocks (reading
    R11: the last min(b, H_P) blocks, oldest dropped first past W_ctx).
    """
    blocks = planner_blocks(cfg)
    if not 0 <= b < len(blocks):
        raise ValueError("planner block out of range")
    hist = list(range(max(0, b - cfg.planner_history), b))
    while hist and sum(len(blocks[x]) for x in hist) + len(blocks[b]) > cfg.w_ctx:
        hist = hist[1:]
    return hist


def n_chunks(cfg: FFConfig) -> int:
    """[S] how it differs: 81 positions are rendered as 27 chunks of 3 latents."""
    if cfg.n_latents % cfg.chunk_latents:
        raise ValueError("n_latents must be a multiple of chunk_latents")
    return cfg.n_latents // cfg.chunk_latents


def chunk_positions(cfg: FFConfig, i: int) -> List[int]:
    """Latent positions covered by renderer chunk i (consecutive, B_R of them)."""
    return list(range(cfg.chunk_latents * i, cfg.chunk_latents * (i + 1)))


def gamma(cfg: FFConfig, i: int) -> List[int]:
    """Anchor ids that renderer chunk i conditions on.  PARITY UNPINNED (reading R1).

    [S] how it differs / how it is used: chunk i reads the left/right clean
    anchor KV selected by Gamma(i); [A] abstract: the anchors give two-sided
    conditioning.  The rule itself is not printed.
    """
    D = cfg.anchor_stride
    pos = chunk_positions(cfg, i)
    na = n_anchors(cfg)
    if cfg.gamma_rule == GAMMA_BRACKET:
        lo = (pos[0] // D) * D
        hi = -(-pos[-1] // D) * D          # ceil to a multiple of D
        return [a for a in range(na) if lo <= a * D <= hi]
    if cfg.gamma_rule == GAMMA_CENTER_LR:
        mid = pos[len(pos) // 2]
        left = mid // D
        return [a for a in (left, left + 1) if a < na]
    raise ValueError(f"unknown gamma rule {cfg.gamma_rule!r}")


def history_ids_after(cfg: FFConfig, i: int) -> List[int]:
    """Chunk ids that B_k holds after chunks 0..i were published at stage k.

    [S] how it works, Eq. (2): Tail_H keeps only the H most recent chunks.
    """
    return list(range(max(0, i - cfg.history + 1), i + 1))


def schedule(cfg: FFConfig) -> List[List[Tuple[int, int]]]:
    """Anti-diagonal wavefront: step t runs the pairs (chunk t-k, stage k).

    [S] how it works: the same-stage dependency lets one GPU per stage run a
    wavefront where different chunks sit at different stages at once; [A]
    abstract: after a chunk finishes stage k its stage-k cache is ready for the
    next chunk.
    """
    nc, S = n_chunks(cfg), cfg.n_stages
    return [[(t - k, k) for k in range(S) if 0 <= t - k < nc] for t in range(nc + S - 1)]


def ar_depth(cfg: FFConfig) -> Dict[str, float]:
    """Autoregressive depth of the two roles.

    [S] how it differs: one planner transition advances B_P*D latents, one
    renderer transition B_R latents, so the planner's AR depth is about 1/10.
    """
    planner_step = cfg.planner_block * cfg.anchor_stride
    renderer_step = cfg.chunk_latents
    return {
        "planner_latents_per_step": planner_step,
        "renderer_latents_per_step": renderer_step,
        "ratio_per_step": planner_step / renderer_step,
        "planner_steps": len(planner_blocks(cfg)),
        "renderer_steps": n_chunks(cfg),
    }


# ---------------------------------------------------------------------------
# Attention: the plain definition of softmax attention, float64.
# ---------------------------------------------------------------------------
def attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of every query over every key, per head (reading R4).

    Q [Lq, nh, d], K [Lk, nh, d], V [Lk, nh, dv] (float64).  Returns O [Lq, nh, dv] and
    the natural-log LSE [nh, Lq].  Per head h and query q:
        s_j = scale * <Q_q, K_j>,  m = max_j s_j,  p_j = exp(s_j - m),
        l = sum_j p_j,  O_q = sum_j p_j V_j / l,  LSE_q = m + ln l.
    [S] how it works, Eq. (2): the renderer forward reads A_Gamma(i) and B_k^(i)
    together with its own chunk; attention over their union is this definition.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Lq, nh, _ = Q.shape
    O = np.empty((Lq, nh, V.shape[2]), dtype=np.float64)
    LSE = np.empty((nh, Lq), dtype=np.float64)
    for h in range(nh):
        s = scale * (Q[:, h, :] @ K[:, h, :].T)            # [Lq, Lk]
        m = s.max(axis=1)
        p = np.exp(s - m[:, None])
        l = p.sum(axis=1)
        O[:, h, :] = (p @ V[:, h, :]) / l[:, None]
        LSE[h] = m + np.log(l)
    return O, LSE


def attention_rows(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                   rows: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """attention() restricted to the query rows ``rows`` (same definition)."""
    O, LSE = attention(np.asarray(Q)[np.asarray(rows)], K, V, scale)
    return O, LSE


# ---------------------------------------------------------------------------
# The rollout state: anchor bank A, stage banks B_0..B_{S-1}, call record.
# ---------------------------------------------------------------------------
@dataclass
class Rollout:
    """Model of the renderer state contract.

    [S] what it is: the design question is what each chunk publishes, at which
    noise level, and when later chunks may consume it.  State = clean anchor
    KV (A) + one history bank per stage (B_k) + which (chunk, stage) calls ran.
    """
    cfg: FFConfig
    anchors: Dict[int, Tuple[np.ndarray, np.ndarray]] = field(default_factory=dict)
    banks: List[List[Tuple[int, np.ndarray, np.ndarray]]] = field(default_factory=list)
    next_chunk: List[int] = field(default_factory=list)

    def __post_init__(self):
        self.banks = [[] for _ in range(self.cfg.n_stages)]
        self.next_chunk = [0] * self.cfg.n_stages

    # -- anchors -----------------------------------------------------------
    def publish_anchors(self, first: int, K: np.ndarray, V: np.ndarray) -> None:
        """Store clean anchor KV for anchors first..first+n-1 (reading R7).

        K, V: [n*T, nh, d].  [S] how it differs: one cache-extraction forward per
        completed planner block publishes that block's clean anchor KV.
        """
        T = self.cfg.tokens_per_latent
        n, rem = divmod(K.shape[0], T)
        if rem or n < 1 or K.shape != V.shape:
            raise ContractError("anchor K/V must be n*T tokens")
        if first < 0 or first + n > n_anchors(self.cfg):
            raise ContractError("anchor id out of range")
        for a in range(first, first + n):
            if a in self.anchors:
                raise ContractError(f"anchor {a} already published")
        for j, a in enumerate(range(first, first + n)):
            self.anchors[a] = (np.array(K[j * T:(j + 1) * T], copy=True),
                               np.array(V[j * T:(j + 1) * T], copy=True))

    # -- the renderer call -------------------------------------------------
    def check_call(self, i: int, k: int) -> None:
        """Raise ContractError unless (i, k) may run now (readings R3, R8)."""
        cfg = self.cfg
        if not (0 <= k < cfg.n_stages) or not (0 <= i < n_chunks(cfg)):
            raise ContractError("chunk or stage out of range")
        if self.next_chunk[k] != i:
            raise ContractError(f"stage {k} expects chunk {self.next_chunk[k]}, got {i}")
        if k > 0 and self.next_chunk[k - 1] <= i:
            raise ContractError(f"chunk {i} has not run stage {k - 1}")
        for a in gamma(cfg, i):
            if a not in self.anchors:
                raise ContractError(f"anchor {a} of Gamma({i}) not published")

    def key_sources(self, i: int, k: int) -> List[Tuple[str, int]]:
        """Ordered key sources of call (i, k): anchors, history (oldest first), own.

        [S] how it works, Eq. (2): F_R(x, c, tau_k; A_Gamma(i), B_k^(i)).
        W_ctx cap (reading R2): drop the oldest history chunks while the key
        latent count exceeds W_ctx.
        """
        cfg = self.cfg
        anc = gamma(cfg, i)
        hist = [cid for cid, _, _ in self.banks[k]]
        while hist and len(anc) + cfg.chunk_latents * (len(hist) + 1) > cfg.w_ctx:
            hist = hist[1:]
        return [("anchor", a) for a in anc] + [("history", c) for c in hist] + [("own", i)]

    def gather_keys(self, i: int, k: int, K_own: np.ndarray, V_own: np.ndarray):
        """Concatenate the key/value rows of key_sources(i, k) in that order."""
        bank = {cid: (Kb, Vb) for cid, Kb, Vb in self.banks[k]}
        ks, vs = [], []
        for kind, idx in self.key_sources(i, k):
            if kind == "anchor":
                Ka, Va = self.anchors[idx]
            elif kind == "history":
                Ka, Va = bank[idx]
            else:
                Ka, Va = K_own, V_own
            ks.append(Ka)
            vs.append(Va)
        return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)

    def render_attend(self, i: int, k: int, Q: np.ndarray, K: np.ndarray, V: np.ndarray,
                      rows: Optional[Sequence[int]] = None, compute: bool = True):
        """One renderer call: attention over the three sources, then Tail_H publish.

        [S] how it works, Eq. (2): (v_hat, K, V) = F_R(x, c, tau_k; A_Gamma(i),
        B_k^(i)) and B_k^(i+1) = Tail_H(B_k^(i) U (i, K, V)); [S] what it is /
        how it works: no cache-update-only forward -- the K/V this call already
        has is what is published (reading R5 for the order).
        Returns (O, LSE) over all rows, or over ``rows`` if given; (None, None)
        when ``compute`` is False (bank bookkeeping only).
        """
        self.check_call(i, k)
        cfg = self.cfg
        O = LSE = None
        if compute:
            Kc, Vc = self.gather_keys(i, k, K, V)
            if rows is None:
                O, LSE = attention(Q, Kc, Vc, cfg.scale)
            else:
                O, LSE = attention_rows(Q, Kc, Vc, cfg.scale, rows)
        # Tail_H: append (i, K, V), keep the last H.
        bank = self.banks[k] + [(i, np.array(K, copy=True), np.array(V, copy=True))]
        self.banks[k] = bank[-cfg.history:]
        self.next_chunk[k] = i + 1
        return O, LSE

    # -- the planner call -------------------------------------------------
    def check_plan(self, b: int) -> None:
        """Raise ContractError unless planner block b may run now (reading R12)."""
        blocks = planner_blocks(self.cfg)
        if not 0 <= b < len(blocks):
            raise ContractError("planner block out of range")
        for x in range(b):
            for a in blocks[x]:
                if a not in self.anchors:
                    raise ContractError(f"planner block {x} (anchor {a}) not published")
        for a in blocks[b]:
            if a in self.anchors:
                raise ContractError(f"anchor {a} of planner block {b} already published")

    def plan_key_sources(self, b: int) -> List[Tuple[str, int]]:
        """Ordered key sources of planner block b: earlier blocks' anchors, then its own latents."""
        blocks = planner_blocks(self.cfg)
        return ([("anchor", a) for x in planner_key_blocks(self.cfg, b) for a in blocks[x]] +
                [("own", a) for a in blocks[b]])

    def plan_attend(self, b: int, Q: np.ndarray, K: np.ndarray, V: np.ndarray, publish: bool = False,
                    rows: Optional[Sequence[int]] = None, compute: bool = True):
        """One planner call: block b attends its key sources; optionally publishes.

        [S] how it differs: anchors are made B_P at a time and, once a block is
        complete, one cache-extraction forward publishes its clean anchor KV;
        [S] training paragraph: planner blocks attend causally to earlier
        blocks' clean KV (readings R11, R12).  Q, K, V: [len(block)*T, nh, d].
        With ``publish`` the call is the cache-extraction forward: K, V become
        the block's anchors.  Returns (O, LSE) like render_attend.
        """
        self.check_plan(b)
        cfg = self.cfg
        blocks = planner_blocks(cfg)
        O = LSE = None
        if compute:
            ks, vs = [], []
            for kind, a in self.plan_key_sources(b):
                if kind == "anchor":
                    Ka, Va = self.anchors[a]
                    ks.append(Ka)
                    vs.append(Va)
            ks.append(np.asarray(K))
            vs.append(np.asarray(V))
            Kc, Vc = np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)
            if rows is None:
                O, LSE = attention(Q, Kc, Vc, cfg.scale)
            else:
                O, LSE = attention_rows(Q, Kc, Vc, cfg.scale, rows)
        if publish:
            self.publish_anchors(blocks[b][0], K, V)
        return O, LSE

    def bank_tail(self, k: int):
        """Chunk ids (oldest first) and concatenated K, V of B_k."""
        bank = self.banks[k]
        ids = [cid for cid, _, _ in bank]
        if not bank:
            return ids, None, None
        return ids, np.concatenate([b[1] for b in bank], 0), np.concatenate([b[2] for b in bank], 0)


def is_legal_order(cfg: FFConfig, calls: Sequence[Tuple[int, int]]) -> bool:
    """True when every call (i, k) finds (i-1, k) and (i, k-1) already done.

    [S] how it works: same-stage dependency; [A] abstract: stage-k cache of
    chunk i is ready for chunk i+1 once chunk i finishes stage k.
    """
    done = set()
    for i, k in calls:
        if (i > 0 and (i - 1, k) not in done) or (k > 0 and (i, k - 1) not in done) or (i, k) in done:
            return False
        done.add((i, k))
    return True


def key_latents(cfg: FFConfig, i: int, k_history: int) -> int:
    """Key latents of a call with ``k_history`` history chunks, after the W_ctx cap."""
    anc = len(gamma(cfg, i))
    h = k_history
    while h and anc + cfg.chunk_latents * (h + 1) > cfg.w_ctx:
        h -= 1
    return anc + cfg.chunk_latents * (h + 1)
