"""Python binding for libpa.so, the paged decode-attention library (C ABI in include/pa.h).

The functions below carry the C entry points' names and only marshal
arguments: torch tensors supply device pointers, and the current torch stream
supplies the HIP stream.  Every step of the computation runs in the library's
HIP kernels; there is no fallback.  If libpa.so has not been built, importing
works but every call raises RuntimeError; so does a libpa.so built from
sources other than the ones beside it (build.py embeds their hash).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_OK = 0
PA_ERR_INVALID_ARG = -1
PA_ERR_UNSUPPORTED = -2
PA_ERR_WORKSPACE = -3
PA_ERR_HIP = -4
PA_F16 = 1
PA_FP8_E4M3 = 2

EXPORTS = ("pa_pool_bytes", "pa_pool_create", "pa_pool_set_scales", "pa_pool_destroy", "pa_write_kv",
           "pa_decode_split_tokens", "pa_decode_workspace_bytes", "pa_decode",
           "pa_append_decode", "pa_decode_partial", "pa_decode_merge", "pa_decode_plan",
           "pa_cascade_plan", "pa_decode_run", "pa_prefill_plan", "pa_prefill_run",
           "pa_decode_noalloc", "pa_status_string")


class PaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {pa_status_string(status)} ({status})")
        self.status = status


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("max_context_len", ctypes.c_int32), ("num_items", ctypes.c_int32),
                ("num_merges", ctypes.c_int32), ("num_slots", ctypes.c_int32),
                ("max_piece_tokens", ctypes.c_int32), ("num_prefix_items", ctypes.c_int32),
                ("num_members", ctypes.c_int32), ("shared_newest", ctypes.c_int32),
                ("num_prefill_items", ctypes.c_int32), ("num_q_rows", ctypes.c_int32),
                ("mixed_decode_waves", ctypes.c_int32), ("decode_wave_heads", ctypes.c_int32),
                ("plan_bytes", ctypes.c_size_t),
                ("workspace_bytes", ctypes.c_size_t)]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libpa.so (once) and declares every exported signature."""
    global _lib
    if _lib is not None:
        return _lib
    from . import build as _build

    _build.check_current(path)
    lib = ctypes.CDLL(path)
    lib.pa_pool_bytes.restype = ctypes.c_size_t
    lib.pa_pool_bytes.argtypes = [ctypes.POINTER(PoolDesc)]
    lib.pa_pool_create.restype = _I
    lib.pa_pool_create.argtypes = [ctypes.POINTER(PoolDesc), _P, _P, ctypes.POINTER(_P)]
    lib.pa_pool_set_scales.restype = _I
    lib.pa_pool_set_scales.argtypes = [_P, _I, ctypes.c_float, ctypes.c_float]
    lib.pa_pool_destroy.restype = _I
    lib.pa_pool_destroy.argtypes = [_P]
    lib.pa_write_kv.restype = _I
    lib.pa_write_kv.argtypes = [_P, _I, _P, _P, _P, _I, _P]
    lib.pa_decode_split_tokens.restype = _I
    lib.pa_decode_split_tokens.argtypes = [_P, _I, _I, _I]
    lib.pa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.pa_decode_workspace_bytes.argtypes = [_P, _I, _I, _I]
    lib.pa_decode.restype = _I
    lib.pa_decode.argtypes = [_P, _I, _P, _P, _P, _I, _P, _I, _I, _I, ctypes.c_float, _P,
                              ctypes.c_size_t, _P]
    for name in ("pa_append_decode", "pa_decode_partial"):
        fn = getattr(lib, name)
        fn.restype = _I
        fn.argtypes = [_P, _I, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, ctypes.c_float, _P,
                       ctypes.c_size_t, _P]
    lib.pa_decode_merge.restype = _I
    lib.pa_decode_merge.argtypes = [_P, _P, _P, _I, _I, _I, _P, ctypes.c_size_t, _P]
    lib.pa_decode_plan.restype = _I
    lib.pa_decode_plan.argtypes = [_P, _P, _I, _I, _P, ctypes.c_size_t, ctypes.POINTER(PlanInfo)]
    lib.pa_cascade_plan.restype = _I
    lib.pa_cascade_plan.argtypes = [_P, _P, _I, _P, _P, _I, _I, _P, ctypes.c_size_t,
                                    ctypes.POINTER(PlanInfo)]
    lib.pa_prefill_plan.restype = _I
    lib.pa_prefill_plan.argtypes = [_P, _P, _P, _I, _I, _P, ctypes.c_size_t, ctypes.POINTER(PlanInfo)]
    lib.pa_prefill_run.restype = _I
    lib.pa_prefill_run.argtypes = [_P, _I, ctypes.POINTER(PlanInfo), _P, ctypes.c_size_t, _P, _P,
                                   _P, _I, ctypes.c_float, _P, ctypes.c_size_t, _P]
    lib.pa_decode_run.restype = _I
    lib.pa_decode_run.argtypes = [_P, _I, ctypes.POINTER(PlanInfo), _P, ctypes.c_size_t, _P, _P,
                                  _P, _P, _P, _I, ctypes.c_float, _P, ctypes.c_size_t, _P]
    lib.pa_decode_noalloc.restype = _I
    lib.pa_decode_noalloc.argtypes = [_P, _I, _P, _P, _P, _I, _P, _I, _I, _I, ctypes.c_float, _P]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_status_string.argtypes = [_I]
    _lib = lib
    return lib


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _check(status: int, what: str) -> None:
    if status != PA_OK:
        raise PaError(status, what)


def _expect(t: torch.Tensor, dtype, shape, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name}: want contiguous {dtype} {tuple(shape)}, got {t.dtype} "
                         f"{tuple(t.shape)} contiguous={t.is_contiguous()}")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def pa_status_string(status: int) -> str:
    return load_library().pa_status_string(int(status)).decode()


def pa_pool_bytes(desc: PoolDesc) -> int:
    return int(load_library().pa_pool_bytes(ctypes.byref(desc)))


def pa_pool_create(desc: PoolDesc, k_pool, v_pool) -> int:
    handle = _P()
    _check(load_library().pa_pool_create(ctypes.byref(desc), _ptr(k_pool), _ptr(v_pool),
                                         ctypes.byref(handle)), "pa_pool_create")
    return handle.value


def pa_pool_set_scales(handle, layer, k_scale, v_scale) -> None:
    _check(load_library().pa_pool_set_scales(handle, layer, float(k_scale), float(v_scale)),
           "pa_pool_set_scales")


def pa_pool_destroy(handle: int) -> None:
    _check(load_library().pa_pool_destroy(handle), "pa_pool_destroy")


def pa_write_kv(handle, layer, k_new, v_new, slot_mapping, n_tokens, stream=None) -> None:
    _check(load_library().pa_write_kv(handle, layer, _ptr(k_new), _ptr(v_new), _ptr(slot_mapping),
                                      n_tokens, _stream(stream)), "pa_write_kv")


def pa_decode_split_tokens(handle, batch, num_q_heads, max_context_len) -> int:
    return int(load_library().pa_decode_split_tokens(handle, batch, num_q_heads, max_context_len))


def pa_decode_workspace_bytes(handle, batch, num_q_heads, max_context_len) -> int:
    return int(load_library().pa_decode_workspace_bytes(handle, batch, num_q_heads,
                                                        max_context_len))


def pa_decode(handle, layer, q, out, block_tables, max_blocks_per_seq, context_lens, batch,
              num_q_heads, max_context_len, scale, workspace, workspace_bytes, stream=None):
    _check(load_library().pa_decode(handle, layer, _ptr(q), _ptr(out), _ptr(block_tables),
                                    max_blocks_per_seq, _ptr(context_lens), batch, num_q_heads,
                                    max_context_len, float(scale), _ptr(workspace),
                                    int(workspace_bytes), _stream(stream)), "pa_decode")


def pa_decode_noalloc(handle, layer, q, out, block_tables, max_blocks_per_seq, context_lens, batch,
                      num_q_heads, max_context_len, scale, stream=None):
    _check(load_library().pa_decode_noalloc(handle, layer, _ptr(q), _ptr(out), _ptr(block_tables),
                                            max_blocks_per_seq, _ptr(context_lens), batch,
                                            num_q_heads, max_context_len, float(scale),
                                            _stream(stream)), "pa_decode_noalloc")


def _new_kv_call(name, handle, layer, q, k_new, v_new, out, block_tables, max_blocks_per_seq,
                 context_lens, batch, num_q_heads, max_context_len, scale, workspace,
                 workspace_bytes, stream):
    fn = getattr(load_library(), name)
    _check(fn(handle, layer, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(block_tables),
              max_blocks_per_seq, _ptr(context_lens), batch, num_q_heads, max_context_len,
              float(scale), _ptr(workspace), int(workspace_bytes), _stream(stream)), name)


def pa_append_decode(handle, layer, q, k_new, v_new, out, block_tables, max_blocks_per_seq,
                     context_lens, batch, num_q_heads, max_context_len, scale, workspace,
                     workspace_bytes, stream=None):
    _new_kv_call("pa_append_decode", handle, layer, q, k_new, v_new, out, block_tables,
                 max_blocks_per_seq, context_lens, batch, num_q_heads, max_context_len, scale,
                 workspace, workspace_bytes, stream)


def pa_decode_partial(handle, layer, q, k_new, v_new, out, block_tables, max_blocks_per_seq,
                      context_lens, batch, num_q_heads, max_context_len, scale, workspace,
                      workspace_bytes, stream=None):
    _new_kv_call("pa_decode_partial", handle, layer, q, k_new, v_new, out, block_tables,
                 max_blocks_per_seq, context_lens, batch, num_q_heads, max_context_len, scale,
                 workspace, workspace_bytes, stream)


def pa_decode_merge(handle, out, context_lens, batch, num_q_heads, max_context_len, workspace,
                    workspace_bytes, stream=None):
    _check(load_library().pa_decode_merge(handle, _ptr(out), _ptr(context_lens), batch,
                                          num_q_heads, max_context_len, _ptr(workspace),
                                          int(workspace_bytes), _stream(stream)),
           "pa_decode_merge")


def pa_decode_plan(handle, context_lens_host, num_q_heads):
    """Host schedule for int32 host lengths: returns (PlanInfo, int32 numpy plan)."""
    import numpy as np

    lens = np.ascontiguousarray(context_lens_host, dtype=np.int32)
    info = PlanInfo()
    lib = load_library()
    ptr = lens.ctypes.data_as(_P) if lens.size else None
    _check(lib.pa_decode_plan(handle, ptr, int(lens.shape[0]), num_q_heads, None, 0,
                              ctypes.byref(info)), "pa_decode_plan")
    plan = np.zeros(max(1, info.plan_bytes // 4), dtype=np.int32)
    _check(lib.pa_decode_plan(handle, ptr, int(lens.shape[0]), num_q_heads,
                              plan.ctypes.data_as(_P), plan.nbytes, ctypes.byref(info)),
           "pa_decode_plan")
    return info, plan


def pa_cascade_plan(handle, context_lens_host, prefix_group_host, prefix_len_host, num_q_heads):
    """Shared-prefix schedule: returns (PlanInfo, int32 numpy plan)."""
    import numpy as np

    lens = np.ascontiguousarray(context_lens_host, dtype=np.int32)
    grp = np.ascontiguousarray(prefix_group_host, dtype=np.int32)
    plen = np.ascontiguousarray(prefix_len_host, dtype=np.int32)
    if grp.shape != lens.shape:
        raise ValueError("prefix_group must have one entry per sequence")
    info = PlanInfo()
    lib = load_library()
    args = (lens.ctypes.data_as(_P) if lens.size else None, int(lens.shape[0]),
            grp.ctypes.data_as(_P) if grp.size else None,
            plen.ctypes.data_as(_P) if plen.size else None, int(plen.shape[0]), num_q_heads)
    _check(lib.pa_cascade_plan(handle, *args, None, 0, ctypes.byref(info)), "pa_cascade_plan")
    plan = np.zeros(max(1, info.plan_bytes // 4), dtype=np.int32)
    _check(lib.pa_cascade_plan(handle, *args, plan.ctypes.data_as(_P), plan.nbytes,
                               ctypes.byref(info)), "pa_cascade_plan")
    return info, plan


def _nbytes(t, nbytes):
    if nbytes is not None:
        return int(nbytes)
    return t.numel() * t.element_size() if isinstance(t, torch.Tensor) else 0


def pa_decode_run(handle, layer, info, plan_dev, q, k_new, v_new, out, block_tables,
                  max_blocks_per_seq, scale, workspace, workspace_bytes, stream=None,
                  plan_dev_bytes=None):
    """plan_dev_bytes defaults to the size of plan_dev when it is a tensor."""
    _check(load_library().pa_decode_run(handle, layer, ctypes.byref(info), _ptr(plan_dev),
                                        _nbytes(plan_dev, plan_dev_bytes), _ptr(q), _ptr(k_new),
                                        _ptr(v_new), _ptr(out), _ptr(block_tables),
                                        max_blocks_per_seq, float(scale), _ptr(workspace),
                                        int(workspace_bytes), _stream(stream)), "pa_decode_run")


def pa_prefill_plan(handle, query_start_host, seq_lens_host, num_q_heads):
    """Chunked-prefill / mixed-step schedule: returns (PlanInfo, int32 numpy plan)."""
    import numpy as np

    qs = np.ascontiguousarray(query_start_host, dtype=np.int32)
    lens = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    if qs.shape != (lens.shape[0] + 1,):
        raise ValueError("query_start must have batch + 1 entries")
    info = PlanInfo()
    lib = load_library()
    args = (qs.ctypes.data_as(_P), lens.ctypes.data_as(_P) if lens.size else None,
            int(lens.shape[0]), num_q_heads)
    _check(lib.pa_prefill_plan(handle, *args, None, 0, ctypes.byref(info)), "pa_prefill_plan")
    plan = np.zeros(max(1, info.plan_bytes // 4), dtype=np.int32)
    _check(lib.pa_prefill_plan(handle, *args, plan.ctypes.data_as(_P), plan.nbytes,
                               ctypes.byref(info)), "pa_prefill_plan")
    return info, plan


def pa_prefill_run(handle, layer, info, plan_dev, q, out, block_tables, max_blocks_per_seq, scale,
                   workspace, workspace_bytes, stream=None, plan_dev_bytes=None):
    """plan_dev_bytes defaults to the size of plan_dev when it is a tensor."""
    _check(load_library().pa_prefill_run(handle, layer, ctypes.byref(info), _ptr(plan_dev),
                                         _nbytes(plan_dev, plan_dev_bytes), _ptr(q), _ptr(out),
                                         _ptr(block_tables), max_blocks_per_seq, float(scale),
                                         _ptr(workspace), int(workspace_bytes), _stream(stream)),
           "pa_prefill_run")


class Plan:
    """A host schedule (pa_decode_plan, or pa_cascade_plan when prefix groups are
    given) and its device copy."""

    def __init__(self, handle, context_lens_host, num_q_heads, device="cuda",
                 prefix_group=None, prefix_len=None, query_start=None):
        if query_start is not None:
            self.info, self.host = pa_prefill_plan(handle, query_start, context_lens_host,
                                                   num_q_heads)
        elif prefix_group is None:
            self.info, self.host = pa_decode_plan(handle, context_lens_host, num_q_heads)
        else:
            self.info, self.host = pa_cascade_plan(handle, context_lens_host, prefix_group,
                                                   prefix_len, num_q_heads)
        self.dev = torch.from_numpy(self.host).to(device)
        n = self.info.workspace_bytes
        self.workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
# a torch-owning convenience wrapper
# ---------------------------------------------------------------------------
class Pool:
    """K and V pools in torch device memory plus the library handle.

    Memory is allocated with torch (uint8 buffers); `fill` initialises it
    (NaN by default so that any slot that is read without being written
    shows up in the output).
    """

    def __init__(self, num_layers, num_blocks, num_kv_heads=8, head_dim=128, block_size=16,
                 device="cuda", fill=float("nan"), dtype=PA_F16):
        self.desc = PoolDesc(num_layers, num_blocks, block_size, num_kv_heads, head_dim, dtype)
        nbytes = pa_pool_bytes(self.desc)
        if nbytes == 0:
            raise ValueError("invalid pool geometry")
        shape = (num_layers, num_blocks, num_kv_heads, block_size, head_dim)
        self.dtype = dtype
        if dtype == PA_FP8_E4M3:
            # raw E4M3 codes; NaN is 0x7f
            self.k = torch.empty(nbytes, dtype=torch.uint8, device=device).view(shape)
            self.v = torch.empty(nbytes, dtype=torch.uint8, device=device).view(shape)
            if fill is not None:
                code = 0x7F if fill != fill else 0
                self.k.fill_(code)
                self.v.fill_(code)
        else:
            self.k = torch.empty(nbytes // 2, dtype=torch.float16, device=device).view(shape)
            self.v = torch.empty(nbytes // 2, dtype=torch.float16, device=device).view(shape)
            if fill is not None:
                self.k.fill_(fill)
                self.v.fill_(fill)
        self.handle = pa_pool_create(self.desc, self.k, self.v)
        self.num_layers, self.num_blocks = num_layers, num_blocks
        self.num_kv_heads, self.head_dim, self.block_size = num_kv_heads, head_dim, block_size

    def set_scales(self, layer, k_scale, v_scale):
        pa_pool_set_scales(self.handle, layer, k_scale, v_scale)

    def close(self):
        if getattr(self, "handle", None):
            pa_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def write(self, layer, k_new, v_new, slot_mapping, stream=None):
        n = int(slot_mapping.shape[0])
        shape = (n, self.num_kv_heads, self.head_dim)
        _expect(k_new, torch.float16, shape, "k_new")
        _expect(v_new, torch.float16, shape, "v_new")
        _expect(slot_mapping, torch.int32, (n,), "slot_mapping")
        pa_write_kv(self.handle, layer, k_new, v_new, slot_mapping, n, stream)

    def plan(self, context_lens_host, num_q_heads=None, prefix_group=None, prefix_len=None):
        return Plan(self.handle, context_lens_host, num_q_heads or 4 * self.num_kv_heads,
                    self.k.device, prefix_group, prefix_len)

    def run(self, layer, plan, q, out, block_tables, scale, k_new=None, v_new=None, stream=None):
        """pa_decode_run on a Plan from plan()."""
        batch = plan.info.batch
        _expect(q, torch.float16, (batch, plan.info.num_q_heads, self.head_dim), "q")
        _expect(out, torch.float16, (batch, plan.info.num_q_heads, self.head_dim), "out")
        _expect(block_tables, torch.int32, (batch, block_tables.shape[1]), "block_tables")
        if (k_new is None) != (v_new is None):
            raise ValueError("k_new and v_new go together")
        if k_new is not None:
            _expect(k_new, torch.float16, (batch, self.num_kv_heads, self.head_dim), "k_new")
            _expect(v_new, torch.float16, (batch, self.num_kv_heads, self.head_dim), "v_new")
        pa_decode_run(self.handle, layer, plan.info, plan.dev, q, k_new, v_new, out, block_tables,
                      int(block_tables.shape[1]), scale, plan.workspace, plan.info.workspace_bytes,
                      stream)
        return out

    def prefill_plan(self, query_start, seq_lens, num_q_heads=None):
        """pa_prefill_plan from host int32 query_start [batch + 1] and seq_lens [batch]."""
        return Plan(self.handle, seq_lens, num_q_heads or 4 * self.num_kv_heads, self.k.device,
                    query_start=query_start)

    def prefill_run(self, layer, plan, q, out, block_tables, scale, stream=None):
        """pa_prefill_run on a Plan from prefill_plan(); q/out [num_q_rows, Hq, d] F16."""
        rows = plan.info.num_q_rows
        _expect(q, torch.float16, (rows, plan.info.num_q_heads, self.head_dim), "q")
        _expect(out, torch.float16, (rows, plan.info.num_q_heads, self.head_dim), "out")
        _expect(block_tables, torch.int32, (plan.info.batch, block_tables.shape[1]), "block_tables")
        pa_prefill_run(self.handle, layer, plan.info, plan.dev, q, out, block_tables,
                       int(block_tables.shape[1]), scale, plan.workspace,
                       plan.info.workspace_bytes, stream)
        return out

    def split_tokens(self, batch, num_q_heads, max_context_len):
        return pa_decode_split_tokens(self.handle, batch, num_q_heads, max_context_len)

    def workspace_bytes(self, batch, num_q_heads, max_context_len):
        return pa_decode_workspace_bytes(self.handle, batch, num_q_heads, max_context_len)

    def workspace(self, batch, num_q_heads, max_context_len, device="cuda"):
        n = self.workspace_bytes(batch, num_q_heads, max_context_len)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=device), n

    def _check_decode(self, q, out, block_tables, context_lens, max_context_len):
        batch, hq, d = q.shape
        _expect(q, torch.float16, (batch, hq, self.head_dim), "q")
        _expect(out, torch.float16, (batch, hq, self.head_dim), "out")
        _expect(block_tables, torch.int32, (batch, block_tables.shape[1]), "block_tables")
        _expect(context_lens, torch.int32, (batch,), "context_lens")
        if max_context_len > block_tables.shape[1] * self.block_size:
            raise ValueError("max_context_len exceeds the table width")
        return batch, hq, int(block_tables.shape[1])

    def decode(self, layer, q, out, block_tables, context_lens, max_context_len, scale,
               workspace=None, stream=None, phases=False, k_new=None, v_new=None):
        """pa_decode, or pa_append_decode when k_new/v_new ([batch, Hkv, d]) are given;
        phases=True issues the same work as pa_decode_partial + pa_decode_merge."""
        batch, hq, width = self._check_decode(q, out, block_tables, context_lens, max_context_len)
        if (k_new is None) != (v_new is None):
            raise ValueError("k_new and v_new go together")
        if k_new is not None:
            _expect(k_new, torch.float16, (batch, self.num_kv_heads, self.head_dim), "k_new")
            _expect(v_new, torch.float16, (batch, self.num_kv_heads, self.head_dim), "v_new")
        if workspace is None:
            workspace = self.workspace(batch, hq, max_context_len, q.device)
        ws, ws_bytes = workspace
        if phases:
            pa_decode_partial(self.handle, layer, q, k_new, v_new, out, block_tables, width,
                              context_lens, batch, hq, max_context_len, scale, ws, ws_bytes, stream)
            pa_decode_merge(self.handle, out, context_lens, batch, hq, max_context_len, ws,
                            ws_bytes, stream)
        elif k_new is not None:
            pa_append_decode(self.handle, layer, q, k_new, v_new, out, block_tables, width,
                             context_lens, batch, hq, max_context_len, scale, ws, ws_bytes, stream)
        else:
            pa_decode(self.handle, layer, q, out, block_tables, width, context_lens, batch, hq,
                      max_context_len, scale, ws, ws_bytes, stream)
        return out
