"""CPU float64 oracle of the block-causal renderer attention and its gradients.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module; only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it.  It shares no code with the HIP library.

Page cited: [S] "In-Flight KV Cache with Clean Anchors for Faster
Autoregressive Video Diffusion" -- Korean summary page, the training
paragraph of section 어떻게 동작하나 (how it works) and Eq. (2) there.
The training paragraph says that a renderer target attends the clean anchor
KV that Gamma(i) allows and the previous H chunks at its own noise level, and
that in self-rollout distillation the renderer runs as one block-causal
forward over the clip instead of per-chunk cache updates, so that gradients
reach earlier chunks from later ones and the planner from the renderer.

Readings taken where the pages leave a step open:
  R13 The block-causal forward at one stage gives chunk i's queries exactly
      the keys of the inference call (i, k) once its bank is in steady state:
      the anchors of Gamma(i), chunks max(0, i-H) .. i-1 of the same stage
      (oldest dropped first past W_ctx, reading R2), and chunk i itself, with
      no mask inside a source (reading R4).  Chunk i's output therefore equals
      the per-chunk call's output on the same K/V (Eq. (2)).
  R14 The gradients are those of the scalar sum(dO * O) with respect to Q, K,
      V of every chunk and K, V of the anchors (the path into the planner);
      the LSE is an output only.

Layouts (token-major, float64 here):
  Ka, Va  [N_a*T, nh, d]      anchor a = rows a*T .. a*T + T - 1
  Q, K, V, O, dO  [N_c*3T, nh, d]   chunk i = rows i*3T .. i*3T + 3T - 1
  LSE     [N_c, nh, 3T]       natural logarithm
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

from .flashforward import FFConfig, attention, gamma, n_anchors, n_chunks


def bc_key_sources(cfg: FFConfig, i: int) -> List[Tuple[str, int]]:
    """Key sources of chunk i in the block-causal forward (reading R13).

    ("anchor", a) for a in Gamma(i) ascending, then ("chunk", j) for the
    history chunks oldest first, then ("chunk", i) for the chunk itself.
    """
    if not 0 <= i < n_chunks(cfg):
        raise ValueError("chunk out of range")
    anc = gamma(cfg, i)
    hist = list(range(max(0, i - cfg.history), i))
    while hist and len(anc) + cfg.chunk_latents * (len(hist) + 1) > cfg.w_ctx:
        hist = hist[1:]
    return [("anchor", a) for a in anc] + [("chunk", j) for j in hist] + [("chunk", i)]


def source_rows(cfg: FFConfig, kind: str, idx: int) -> slice:
    """Token rows of one source in the anchor arrays or the chunk arrays."""
    n = cfg.tokens_per_latent if kind == "anchor" else cfg.chunk_tokens
    return slice(idx * n, (idx + 1) * n)


def bc_mask(cfg: FFConfig) -> np.ndarray:
    """Which sources each chunk's queries attend: bool [N_c, N_a + N_c].

    Column a < N_a is anchor a, column N_a + j is chunk j.
    """
    na, nc = n_anchors(cfg), n_chunks(cfg)
    m = np.zeros((nc, na + nc), dtype=bool)
    for i in range(nc):
        for kind, idx in bc_key_sources(cfg, i):
            m[i, idx if kind == "anchor" else na + idx] = True
    return m


def bc_keys(cfg: FFConfig, i: int, Ka, Va, K, V) -> Tuple[np.ndarray, np.ndarray]:
    """Chunk i's keys and values, concatenated in bc_key_sources order."""
    ks, vs = [], []
    for kind, idx in bc_key_sources(cfg, i):
        src_k, src_v = (Ka, Va) if kind == "anchor" else (K, V)
        r = source_rows(cfg, kind, idx)
        ks.append(np.asarray(src_k[r], dtype=np.float64))
        vs.append(np.asarray(src_v[r], dtype=np.float64))
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


def _chunk_list(cfg: FFConfig, chunks: Optional[Sequence[int]]) -> List[int]:
    return list(range(n_chunks(cfg))) if chunks is None else [int(c) for c in chunks]


def bc_forward(cfg: FFConfig, Ka, Va, Q, K, V, chunks: Optional[Sequence[int]] = None):
    """O [N_c*3T, nh, d] and LSE [N_c, nh, 3T] of the block-causal forward.

    Each chunk's rows are softmax attention over its own key set (the
    definition in ``attention``).  With ``chunks`` only those chunks are
    computed; the other rows of O and LSE are NaN.
    """
    L = cfg.chunk_tokens
    Q = np.asarray(Q, dtype=np.float64)
    nh = Q.shape[1]
    O = np.full((Q.shape[0], nh, np.asarray(V).shape[2]), np.nan)
    LSE = np.full((n_chunks(cfg), nh, L), np.nan)
    for i in _chunk_list(cfg, chunks):
        Kc, Vc = bc_keys(cfg, i, Ka, Va, K, V)
        rows = slice(i * L, (i + 1) * L)
        O[rows], LSE[i] = attention(Q[rows], Kc, Vc, cfg.scale)
    return O, LSE


def bc_backward(cfg: FFConfig, Ka, Va, Q, K, V, dO, chunks: Optional[Sequence[int]] = None):
    """Gradients of sum(dO * O) for the block-causal forward (reading R14).

    Returns dQ, dK, dV (shaped like Q) and dKa, dVa (shaped like Ka), summing
    the contributions of the query chunks ``chunks`` (all by default).  Per
    chunk and head, with S = scale Q Kc^T and P = softmax(S) row by row:
        dVc = P^T dO,  dP = dO Vc^T,
        dS = P * (dP - rowsum(P * dP))      (Jacobian of the softmax),
        dQ = scale dS Kc,  dKc = scale dS^T Q,
    and dKc, dVc are added back into the rows of the sources they came from.
    """
    L = cfg.chunk_tokens
    Q = np.asarray(Q, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    nh = Q.shape[1]
    dQ = np.zeros_like(Q)
    dK = np.zeros(np.shape(K), dtype=np.float64)
    dV = np.zeros(np.shape(V), dtype=np.float64)
    dKa = np.zeros(np.shape(Ka), dtype=np.float64)
    dVa = np.zeros(np.shape(Va), dtype=np.float64)
    for i in _chunk_list(cfg, chunks):
        Kc, Vc = bc_keys(cfg, i, Ka, Va, K, V)
        rows = slice(i * L, (i + 1) * L)
        dKc = np.zeros_like(Kc)
        dVc = np.zeros_like(Vc)
        for h in range(nh):
            q, g = Q[rows, h, :], dO[rows, h, :]
            s = cfg.scale * (q @ Kc[:, h, :].T)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            P = e / e.sum(axis=1, keepdims=True)
            dVc[:, h, :] = P.T @ g
            dP = g @ Vc[:, h, :].T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dQ[rows, h, :] = cfg.scale * (dS @ Kc[:, h, :])
            dKc[:, h, :] = cfg.scale * (dS.T @ q)
        off = 0
        for kind, idx in bc_key_sources(cfg, i):
            r = source_rows(cfg, kind, idx)
            n = r.stop - r.start
            tk, tv = (dKa, dVa) if kind == "anchor" else (dK, dV)
            tk[r] += dKc[off:off + n]
            tv[r] += dVc[off:off + n]
            off += n
    return dQ, dK, dV, dKa, dVa


def bc_complete_sources(cfg: FFConfig, chunks: Sequence[int]) -> Tuple[List[int], List[int]]:
    """Anchors and chunks whose gradients are complete from the query chunks ``chunks``.

    A source's dK/dV is complete when every chunk that attends it is included.
    """
    m = bc_mask(cfg)
    na = n_anchors(cfg)
    inc = np.zeros(m.shape[0], dtype=bool)
    inc[list(chunks)] = True
    done = [c for c in range(m.shape[1]) if m[:, c].any() and not (m[:, c] & ~inc).any()]
    return [c for c in done if c < na], [c - na for c in done if c >= na]
