"""The oracle pins must fail when a plausible mistake is planted in the oracle.

Each case copies ``oracle/``, ``synthetic/`` and the pin tests into a temporary
directory, edits one line of the copied oracle, and runs the pins there in a
subprocess.  The repository's own oracle is never modified.  CPU only.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FF = "flashforward.py"
BC = "block_causal.py"
PINS = ("test_oracle_pins.py", "test_oracle_bc_pins.py")

MUTATIONS = {
    "tail_keeps_H_plus_1": ("self.banks[k] = bank[-cfg.history:]", "self.banks[k] = bank[-(cfg.history + 1):]"),
    "tail_keeps_oldest": ("self.banks[k] = bank[-cfg.history:]", "self.banks[k] = bank[:cfg.history]"),
    "scale_one_over_d": ("return 1.0 / math.sqrt(self.head_dim)", "return 1.0 / self.head_dim"),
    "lse_without_max": ("LSE[h] = m + np.log(l)", "LSE[h] = np.log(l)"),
    "own_chunk_dropped": ('+ [("own", i)]', ""),
    "gamma_right_anchor_floor": ("hi = -(-pos[-1] // D) * D", "hi = (pos[-1] // D) * D"),
    "wrong_head_of_K": ("s = scale * (Q[:, h, :] @ K[:, h, :].T)", "s = scale * (Q[:, h, :] @ K[:, (h + 1) % nh, :].T)"),
    "history_reversed": ("hist = [cid for cid, _, _ in self.banks[k]]",
                         "hist = [cid for cid, _, _ in self.banks[k]][::-1]"),
    "no_stage_dependency": ("if k > 0 and self.next_chunk[k - 1] <= i:", "if False:"),
    "cap_drops_newest": ("hist = hist[1:]", "hist = hist[:-1]"),
    "anchor_grid_shifted": ("return list(range(0, cfg.n_latents, cfg.anchor_stride))",
                            "return list(range(cfg.anchor_stride, cfg.n_latents, cfg.anchor_stride))"),
    "softmax_sign": ("p = np.exp(s - m[:, None])", "p = np.exp(m[:, None] - s)"),
    "planner_window_short": ("hist = list(range(max(0, b - cfg.planner_history), b))",
                             "hist = list(range(max(0, b - cfg.planner_history + 1), b))"),
    "planner_window_long": ("hist = list(range(max(0, b - cfg.planner_history), b))",
                            "hist = list(range(max(0, b - cfg.planner_history - 1), b))"),
    "planner_own_dropped": ("            ks.append(np.asarray(K))\n            vs.append(np.asarray(V))\n", ""),
    "planner_no_order_check": ("        for x in range(b):\n            for a in blocks[x]:", "        for x in range(0):\n            for a in blocks[x]:"),
    "planner_publish_shifted": ("self.publish_anchors(blocks[b][0], K, V)", "self.publish_anchors(blocks[b][-1], K, V)"),
    # the sampled-row path of the full-size GPU comparisons
    "rows_select_keys": ("O, LSE = attention(np.asarray(Q)[np.asarray(rows)], K, V, scale)",
                         "O, LSE = attention(Q, np.asarray(K)[np.asarray(rows)], np.asarray(V)[np.asarray(rows)], "
                         "scale)"),
    "rows_sorted_silently": ("O, LSE = attention(np.asarray(Q)[np.asarray(rows)], K, V, scale)",
                             "O, LSE = attention(np.asarray(Q)[np.sort(np.asarray(rows))], K, V, scale)"),
    "render_rows_ignored": ("                O, LSE = attention_rows(Q, Kc, Vc, cfg.scale, rows)\n        # Tail_H",
                            "                O, LSE = attention(Q, Kc, Vc, cfg.scale)\n        # Tail_H"),
    # block-causal forward and gradients (oracle/block_causal.py)
    "bc_window_long": ("hist = list(range(max(0, i - cfg.history), i))",
                       "hist = list(range(max(0, i - cfg.history - 1), i))", BC),
    "bc_own_chunk_dropped": (' + [("chunk", i)]', "", BC),
    "bc_cap_drops_newest": ("hist = hist[1:]", "hist = hist[:-1]", BC),
    "bc_no_softmax_jacobian_term": ("dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))", "dS = P * dP", BC),
    "bc_dk_unscaled": ("dKc[:, h, :] = cfg.scale * (dS.T @ q)", "dKc[:, h, :] = dS.T @ q", BC),
    "bc_dq_from_values": ("dQ[rows, h, :] = cfg.scale * (dS @ Kc[:, h, :])",
                          "dQ[rows, h, :] = cfg.scale * (dS @ Vc[:, h, :])", BC),
    "bc_dv_from_queries": ("dVc[:, h, :] = P.T @ g", "dVc[:, h, :] = P.T @ q", BC),
    "bc_scatter_misaligned": ("            off += n\n", "", BC),
    "bc_anchor_grads_to_chunks": ('tk, tv = (dKa, dVa) if kind == "anchor" else (dK, dV)',
                                  'tk, tv = (dK, dV) if kind == "anchor" else (dKa, dVa)', BC),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new, target = (MUTATIONS[name] + (FF,))[:3]
    for d in ("oracle", "synthetic"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("__pycache__"))
    (tmp_path / "tests").mkdir()
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tmp_path / "tests" / "golden")
    for f in ("conftest.py",) + PINS:
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    src_path = tmp_path / "oracle" / target
    src = src_path.read_text()
    assert old in src, f"mutation {name} no longer applies"
    src_path.write_text(src.replace(old, new))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        *[str(tmp_path / "tests" / f) for f in PINS]],
                       cwd=tmp_path, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"pins did not catch mutation {name}:\n{r.stdout[-2000:]}"
