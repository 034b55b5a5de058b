"""Python binding of the C ABI in include/ff.h (argument marshalling only).

Every function here has the name of the C entry point it calls and does
nothing but check and convert arguments: torch tensors become device
pointers, the current torch stream becomes the hipStream_t, and a non-zero
status becomes an ``FFError``.  All work runs in libff.so.  If libff.so has not
been built the import fails; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libff.so")
HOSTCHECK_PATH = os.path.join(PKG, "libff_hostcheck.so")

FF_OK, FF_E_INVAL, FF_E_ORDER, FF_E_ANCHOR_MISSING, FF_E_ANCHOR_EXISTS = 0, -1, -2, -3, -4
FF_E_RANGE, FF_E_NOSPACE, FF_E_HIP, FF_E_STATE = -5, -6, -7, -8
FF_BF16, FF_F32 = 0, 1
FF_GAMMA_BRACKET, FF_GAMMA_CENTER_LR = 0, 1
FF_SRC_ANCHOR, FF_SRC_HISTORY, FF_SRC_OWN = 0, 1, 2
FF_MAX_SOURCES = 32


class ff_shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_heads", "head_dim", "tokens_per_latent", "chunk_latents", "anchor_stride",
        "n_latents", "w_ctx", "dtype", "gamma_rule", "planner_latents", "planner_history")]


class ff_key_sources(ctypes.Structure):
    _fields_ = [("n_sources", ctypes.c_int32),
                ("kind", ctypes.c_int32 * FF_MAX_SOURCES),
                ("id", ctypes.c_int32 * FF_MAX_SOURCES),
                ("n_tokens", ctypes.c_int32 * FF_MAX_SOURCES),
                ("key_tokens", ctypes.c_int32),
                ("key_latents", ctypes.c_int32)]


class ff_clip_counts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_anchors", "n_chunks", "n_planner_blocks", "n_diagonals")]


class ff_kernel_times(ctypes.Structure):
    _fields_ = [("attn_launches", ctypes.c_int64), ("attn_ms", ctypes.c_double),
                ("merge_launches", ctypes.c_int64), ("merge_ms", ctypes.c_double),
                ("publish_launches", ctypes.c_int64), ("publish_ms", ctypes.c_double),
                ("anchor_launches", ctypes.c_int64), ("anchor_ms", ctypes.c_double),
                ("layout_launches", ctypes.c_int64), ("layout_ms", ctypes.c_double),
                ("bwd_pre_launches", ctypes.c_int64), ("bwd_pre_ms", ctypes.c_double),
                ("bwd_dq_launches", ctypes.c_int64), ("bwd_dq_ms", ctypes.c_double),
                ("bwd_dk_launches", ctypes.c_int64), ("bwd_dk_ms", ctypes.c_double),
                ("bwd_dv_launches", ctypes.c_int64), ("bwd_dv_ms", ctypes.c_double)]


class FFError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


_VP = ctypes.c_void_p
_I = ctypes.c_int
_SIGS = {
    "ff_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(ff_shape), _I, _I]),
    "ff_stage_bank_create": (_I, [ctypes.POINTER(ff_shape), _I, _I, _VP, ctypes.c_size_t, ctypes.POINTER(_VP)]),
    "ff_destroy": (None, [_VP]),
    "ff_anchor_bank_publish": (_I, [_VP, _I, _I, _VP, _VP, _VP]),
    "ff_render_attend": (_I, [_VP, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP]),
    "ff_render_attend_static_scratch": (_I, [_VP, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP]),
    "ff_render_attend_grouped": (_I, [_VP, _I, ctypes.POINTER(_I), ctypes.POINTER(_I), ctypes.POINTER(_VP),
                                      ctypes.POINTER(_VP), ctypes.POINTER(_VP), ctypes.POINTER(_VP),
                                      ctypes.POINTER(_VP), _VP]),
    "ff_plan_attend": (_I, [_VP, _I, _VP, _VP, _VP, _VP, _VP, _I, _VP]),
    "ff_plan_key_plan": (_I, [_VP, _I, ctypes.POINTER(ff_key_sources)]),
    "ff_bank_tail": (_I, [_VP, _I, ctypes.POINTER(_I), ctypes.POINTER(_I), _VP, _VP, _VP]),
    "ff_gamma": (_I, [_VP, _I, ctypes.POINTER(_I), ctypes.POINTER(_I)]),
    "ff_key_plan": (_I, [_VP, _I, _I, ctypes.POINTER(ff_key_sources)]),
    "ff_stage_next": (_I, [_VP, _I, ctypes.POINTER(_I)]),
    "ff_stage_bank_rewind": (_I, [_VP, _I]),
    "ff_clip_layout": (_I, [ctypes.POINTER(ff_shape), _I, ctypes.POINTER(ff_clip_counts)]),
    "ff_planner_block": (_I, [ctypes.POINTER(ff_shape), _I, ctypes.POINTER(_I), ctypes.POINTER(_I)]),
    "ff_wavefront": (_I, [ctypes.POINTER(ff_shape), _I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I),
                          ctypes.POINTER(_I)]),
    "ff_profile_enable": (_I, [_VP, _I]),
    "ff_profile_read": (_I, [_VP, ctypes.POINTER(ff_kernel_times)]),
    "ff_profile_families": (_I, [_VP, ctypes.c_uint]),
    "ff_bc_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(ff_shape), _I]),
    "ff_bc_create": (_I, [ctypes.POINTER(ff_shape), _I, _VP, ctypes.c_size_t, ctypes.POINTER(_VP)]),
    "ff_bc_destroy": (None, [_VP]),
    "ff_bc_forward": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "ff_bc_backward": (_I, [_VP] + [_VP] * 14),
    "ff_bc_key_plan": (_I, [_VP, _I, ctypes.POINTER(ff_key_sources)]),
    "ff_bc_profile_enable": (_I, [_VP, _I]),
    "ff_bc_profile_read": (_I, [_VP, ctypes.POINTER(ff_kernel_times)]),
    "ff_status_str": (ctypes.c_char_p, [_I]),
}
SYMBOLS = tuple(_SIGS)


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{os.path.basename(path)} is not built; run `python -m chunked_kv_cache_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = load()
    return _lib


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream, *tensors) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    for t in tensors:
        if t is not None and not isinstance(t, int) and t.is_cuda:
            import torch
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _check(st: int, L) -> None:
    if st != FF_OK:
        raise FFError(st, L.ff_status_str(st).decode())


def make_shape(*, n_heads, head_dim, tokens_per_latent, chunk_latents=3, anchor_stride=10, n_latents=81,
               w_ctx=21, dtype=FF_BF16, gamma_rule=FF_GAMMA_BRACKET, planner_latents=3,
               planner_history=6) -> ff_shape:
    return ff_shape(n_heads, head_dim, tokens_per_latent, chunk_latents, anchor_stride, n_latents, w_ctx,
                    dtype, gamma_rule, planner_latents, planner_history)


def ff_workspace_bytes(shape: ff_shape, n_stages: int, history: int, L=None) -> int:
    L = L or lib()
    return int(L.ff_workspace_bytes(ctypes.byref(shape), n_stages, history))


def ff_stage_bank_create(shape: ff_shape, n_stages: int, history: int, workspace, workspace_bytes: int,
                         L=None) -> int:
    L = L or lib()
    out = _VP()
    _check(L.ff_stage_bank_create(ctypes.byref(shape), n_stages, history, _ptr(workspace), workspace_bytes,
                                  ctypes.byref(out)), L)
    return out.value


def ff_destroy(ctx: int, L=None) -> None:
    (L or lib()).ff_destroy(ctx)


def ff_anchor_bank_publish(ctx, first_anchor, n_anchors, K, V, stream=None, L=None) -> None:
    L = L or lib()
    _check(L.ff_anchor_bank_publish(ctx, first_anchor, n_anchors, _ptr(K), _ptr(V), _stream(stream, K)), L)


def ff_render_attend(ctx, chunk, stage, Q, K, V, O, lse=None, stream=None, L=None) -> None:
    L = L or lib()
    _check(L.ff_render_attend(ctx, chunk, stage, _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(lse),
                              _stream(stream, Q)), L)


def ff_render_attend_static_scratch(ctx, chunk, stage, Q, K, V, O, lse=None, stream=None, L=None) -> None:
    L = L or lib()
    _check(L.ff_render_attend_static_scratch(ctx, chunk, stage, _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(lse),
                                             _stream(stream, Q)), L)


def ff_render_attend_grouped(ctx, chunks: Sequence[int], stages: Sequence[int], Q, K, V, O, lse=None,
                             stream=None, L=None) -> None:
    L = L or lib()
    n = len(chunks)
    arr = lambda xs: (_VP * n)(*[_ptr(x) for x in xs])
    lse_arr = None if lse is None else arr(lse)
    _check(L.ff_render_attend_grouped(ctx, n, (_I * n)(*chunks), (_I * n)(*stages), arr(Q), arr(K), arr(V),
                                      arr(O), lse_arr, _stream(stream, Q[0])), L)


def ff_plan_attend(ctx, block, Q, K, V, O, lse=None, publish=False, stream=None, L=None) -> None:
    L = L or lib()
    _check(L.ff_plan_attend(ctx, block, _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(lse), 1 if publish else 0,
                            _stream(stream, Q)), L)


def ff_plan_key_plan(ctx, block, L=None) -> ff_key_sources:
    L = L or lib()
    out = ff_key_sources()
    _check(L.ff_plan_key_plan(ctx, block, ctypes.byref(out)), L)
    return out


def ff_bank_tail(ctx, stage, K_out=None, V_out=None, stream=None, L=None, history_max=8):
    L = L or lib()
    n = _I()
    ids = (_I * history_max)()
    _check(L.ff_bank_tail(ctx, stage, ctypes.byref(n), ids, _ptr(K_out), _ptr(V_out),
                          _stream(stream, K_out, V_out)), L)
    return list(ids[:n.value])


def ff_gamma(ctx, chunk, L=None):
    L = L or lib()
    n = _I()
    ids = (_I * 3)()
    _check(L.ff_gamma(ctx, chunk, ctypes.byref(n), ids), L)
    return list(ids[:n.value])


def ff_key_plan(ctx, chunk, stage, L=None) -> ff_key_sources:
    L = L or lib()
    out = ff_key_sources()
    _check(L.ff_key_plan(ctx, chunk, stage, ctypes.byref(out)), L)
    return out


def ff_stage_next(ctx, stage, L=None) -> int:
    L = L or lib()
    n = _I()
    _check(L.ff_stage_next(ctx, stage, ctypes.byref(n)), L)
    return n.value


def ff_stage_bank_rewind(ctx, stage, L=None) -> None:
    L = L or lib()
    _check(L.ff_stage_bank_rewind(ctx, stage), L)


def ff_clip_layout(shape: ff_shape, n_stages: int = 1, L=None) -> dict:
    L = L or lib()
    out = ff_clip_counts()
    _check(L.ff_clip_layout(ctypes.byref(shape), n_stages, ctypes.byref(out)), L)
    return {f: getattr(out, f) for f, _ in ff_clip_counts._fields_}


def ff_planner_block(shape: ff_shape, block: int, L=None):
    L = L or lib()
    first, n = _I(), _I()
    _check(L.ff_planner_block(ctypes.byref(shape), block, ctypes.byref(first), ctypes.byref(n)), L)
    return list(range(first.value, first.value + n.value))


def ff_wavefront(shape: ff_shape, n_stages: int, t: int, L=None):
    L = L or lib()
    n = _I()
    chunks, stages = (_I * n_stages)(), (_I * n_stages)()
    _check(L.ff_wavefront(ctypes.byref(shape), n_stages, t, ctypes.byref(n), chunks, stages), L)
    return [(chunks[j], stages[j]) for j in range(n.value)]


def ff_profile_enable(ctx, on: bool, L=None) -> None:
    L = L or lib()
    _check(L.ff_profile_enable(ctx, 1 if on else 0), L)


# Kernel families of ff_kernel_times (bits of ff_profile_families).
PROF_ATTN, PROF_MERGE, PROF_PUBLISH, PROF_ANCHOR, PROF_LAYOUT = 1, 2, 4, 8, 16
PROF_BWD_PRE, PROF_BWD_DQ, PROF_BWD_DK, PROF_BWD_DV = 32, 64, 128, 256
PROF_ALL = 511


def ff_profile_families(ctx, families: int, L=None) -> None:
    L = L or lib()
    _check(L.ff_profile_families(ctx, families), L)


def ff_profile_read(ctx, L=None) -> dict:
    L = L or lib()
    t = ff_kernel_times()
    _check(L.ff_profile_read(ctx, ctypes.byref(t)), L)
    return {f: getattr(t, f) for f, _ in ff_kernel_times._fields_}


class StageBanks:
    """Owns one context and its torch-allocated workspace (device memory only)."""

    def __init__(self, shape: ff_shape, n_stages: int, history: int, device="cuda"):
        import torch
        self.shape, self.n_stages, self.history = shape, n_stages, history
        self.ws_bytes = ff_workspace_bytes(shape, n_stages, history)
        if self.ws_bytes == 0:
            raise FFError(FF_E_INVAL, "unsupported shape")
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.ctx = ff_stage_bank_create(shape, n_stages, history, self.workspace, self.ws_bytes)

    def close(self):
        if getattr(self, "ctx", None):
            ff_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------------------
# Block-causal attention over a clip (training form)
# ---------------------------------------------------------------------------
def ff_bc_workspace_bytes(shape: ff_shape, history: int, L=None) -> int:
    L = L or lib()
    return int(L.ff_bc_workspace_bytes(ctypes.byref(shape), history))


def ff_bc_create(shape: ff_shape, history: int, workspace, workspace_bytes: int, L=None) -> int:
    L = L or lib()
    out = _VP()
    _check(L.ff_bc_create(ctypes.byref(shape), history, _ptr(workspace), workspace_bytes, ctypes.byref(out)), L)
    return out.value


def ff_bc_destroy(bc, L=None) -> None:
    L = L or lib()
    L.ff_bc_destroy(bc)


def ff_bc_forward(bc, Ka, Va, Q, K, V, O, lse=None, stream=None, L=None) -> None:
    L = L or lib()
    _check(L.ff_bc_forward(bc, _ptr(Ka), _ptr(Va), _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(lse),
                           _stream(stream, Q, O)), L)


def ff_bc_backward(bc, Ka, Va, Q, K, V, O, lse, dO, dQ, dK, dV, dKa, dVa, stream=None, L=None) -> None:
    L = L or lib()
    _check(L.ff_bc_backward(bc, _ptr(Ka), _ptr(Va), _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(lse), _ptr(dO),
                            _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dKa), _ptr(dVa), _stream(stream, Q, dQ)), L)


def ff_bc_key_plan(bc, chunk, L=None) -> ff_key_sources:
    L = L or lib()
    out = ff_key_sources()
    _check(L.ff_bc_key_plan(bc, chunk, ctypes.byref(out)), L)
    return out


def ff_bc_profile_enable(bc, on: bool, L=None) -> None:
    L = L or lib()
    _check(L.ff_bc_profile_enable(bc, 1 if on else 0), L)


def ff_bc_profile_read(bc, L=None) -> dict:
    L = L or lib()
    t = ff_kernel_times()
    _check(L.ff_bc_profile_read(bc, ctypes.byref(t)), L)
    return {f: getattr(t, f) for f, _ in ff_kernel_times._fields_}


class BlockCausal:
    """Owns one block-causal context and its torch-allocated workspace."""

    def __init__(self, shape: ff_shape, history: int, device="cuda"):
        import torch
        self.shape, self.history = shape, history
        self.ws_bytes = ff_bc_workspace_bytes(shape, history)
        if self.ws_bytes == 0:
            raise FFError(FF_E_INVAL, "unsupported shape")
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.ctx = ff_bc_create(shape, history, self.workspace, self.ws_bytes)

    def close(self):
        if getattr(self, "ctx", None):
            ff_bc_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
