"""GPU test of ff_render_attend_static_scratch, the renderer call that
allocates nothing: its partials live in the library's fixed device array.

Twin contexts receive the same seeded calls, one through ff_render_attend
(partials in the workspace) and one through the fixed-scratch entry point;
outputs, LSE and bank bytes must be identical, and both match the oracle.
Two call sequences in a row, the second with a smaller shape, so the second
runs on the array as the first left it.  Every item is split (few heads, short
chunks), so the partial slots are written and read on every call.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import synthetic as syn
from chunked_kv_cache_amd import ff
from ffharness import Case, Pair, from_device_f64, to_device, wavefront

pytestmark = pytest.mark.gpu


def _twin_rollout(case, n_diag):
    ref, fixed = Pair(case), Pair(case)
    try:
        ref.publish_anchors()
        fixed.publish_anchors()
        calls = 0
        for diag in wavefront(case)[:n_diag]:
            for i, k in diag:
                host = ref.gen(i, k)
                dev = [to_device(x, "bf16") for x in host]
                outs = [torch.full_like(dev[0], float("nan")) for _ in range(2)]
                lses = [torch.full((case.nh, 3 * case.T), float("nan"), dtype=torch.float32, device="cuda")
                        for _ in range(2)]
                ff.ff_render_attend(ref.ctx, i, k, dev[0], dev[1], dev[2], outs[0], lses[0])
                ff.ff_render_attend_static_scratch(fixed.ctx, i, k, dev[0], dev[1], dev[2], outs[1], lses[1])
                torch.cuda.synchronize()
                assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), (i, k)
                assert torch.equal(lses[0], lses[1]), (i, k)
                q64, k64, v64 = (syn.as_f64(x, "bf16") for x in host)
                O_ref, L_ref = fixed.ro.render_attend(i, k, q64, k64, v64)
                fixed.inputs[(i, k)] = (host[1], host[2])
                fixed._compare(from_device_f64(outs[1]), lses[1].cpu().numpy().astype(np.float64), O_ref, L_ref,
                               None, 2e-2)
                fixed.check_bank(k)
                calls += 1
        return calls
    finally:
        ref.close()
        fixed.close()


def test_static_scratch_matches_workspace_call_twice():
    big = Case(T=200, nh=4, d=128, S=2)          # 600 queries x 4 heads: 12 items, all split
    small = Case(T=64, nh=2, d=128, S=2)         # 192 queries x 2 heads: 2 items, all split
    assert _twin_rollout(big, 8) == 15
    assert _twin_rollout(small, 8) == 15


def test_static_scratch_rejects_before_device_work():
    """Order violations are rejected before the scratch is touched."""
    case = Case(T=64, nh=2, d=128, S=2)
    pr = Pair(case)
    try:
        x = torch.zeros((3 * case.T, case.nh, case.d), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(ff.FFError) as e:
            ff.ff_render_attend_static_scratch(pr.ctx, 0, 0, x, x, x, x)
        assert e.value.status == ff.FF_E_ANCHOR_MISSING
        pr.publish_anchors()
        with pytest.raises(ff.FFError) as e:
            ff.ff_render_attend_static_scratch(pr.ctx, 1, 0, x, x, x, x)
        assert e.value.status == ff.FF_E_ORDER
    finally:
        pr.close()
