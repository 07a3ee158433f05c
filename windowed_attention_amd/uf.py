"""ctypes binding of libuf (include/uf.h): argument marshalling only.

Every function here has the name of the C entry point it calls and does
nothing but convert arguments: torch tensors become device pointers,
sizes and strides; streams become their hipStream_t handles.  All work
happens in the HIP library.  If libuf.so has not been built, importing this
module raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

# UF_LIBRARY_PATH names another build of the same C ABI to load instead (the tests use it for
# a host-only build of the host side under sanitizers).
_LIB_PATH = os.environ.get("UF_LIBRARY_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libuf.so")

UF_OK = 0
UF_ERR_INVALID_ARG = -1
UF_ERR_SHAPE = -2
UF_ERR_DTYPE = -3
UF_ERR_CAPACITY = -4
UF_ERR_STATE = -5
UF_ERR_HIP = -6
UF_ERR_UNSUPPORTED = -7
UF_BF16 = 0
UF_FP8_E4M3 = 1
UF_APPEND_OVERWRITE_NEWEST = 1
UF_APPEND_COMMIT_ONLY = 2
UF_TILE = 128
UF_MAX_APPEND_FRAMES = 64
UF_STATIC_SCRATCH_BYTES = 32 << 20

EXPORTED = [
    "uf_kvcache_storage_bytes", "uf_attn_workspace_bytes", "uf_kvcache_create", "uf_kvcache_destroy",
    "uf_kvcache_reset", "uf_kvcache_set_window", "uf_kvcache_append", "uf_kvcache_plan_append",
    "uf_kvcache_window", "uf_attn_step", "uf_attn_step_static", "uf_block_mask_workspace_bytes",
    "uf_block_mask_topk",
    "uf_status_string", "uf_last_error",
]


class uf_tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("n_tokens", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("stride_token", ctypes.c_int64), ("stride_head", ctypes.c_int64)]


class uf_kvcache_desc(ctypes.Structure):
    _fields_ = [("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("tokens_per_frame", ctypes.c_int32), ("window_frames", ctypes.c_int32),
                ("anchor_frames", ctypes.c_int32), ("k_storage", ctypes.c_void_p),
                ("v_storage", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("kv_dtype", ctypes.c_int32),
                ("q_scale", ctypes.c_float), ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
                ("block_grid_h", ctypes.c_int32), ("block_grid_w", ctypes.c_int32),
                ("max_q_heads", ctypes.c_int32), ("max_q_tokens", ctypes.c_int32),
                ("heads_per_wg", ctypes.c_int32), ("splits", ctypes.c_int32), ("pipeline", ctypes.c_int32)]


class uf_block_mask(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("n_heads", ctypes.c_int32), ("n_q_blocks", ctypes.c_int32),
                ("n_k_blocks", ctypes.c_int32), ("stride_head", ctypes.c_int64),
                ("stride_qblock", ctypes.c_int64)]


class uf_window_info(ctypes.Structure):
    _fields_ = [("frames_appended", ctypes.c_int64), ("n_keys", ctypes.c_int32),
                ("anchor_keys", ctypes.c_int32), ("ring_keys", ctypes.c_int32),
                ("ring_capacity_keys", ctypes.c_int32), ("ring_rotation_keys", ctypes.c_int32),
                ("last_append_frames", ctypes.c_int32), ("active_frames", ctypes.c_int32)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class uf_append_plan(ctypes.Structure):
    _fields_ = [("n_frames", ctypes.c_int32), ("first_row", ctypes.c_int32 * UF_MAX_APPEND_FRAMES),
                ("window_after", uf_window_info)]


class uf_topk_params(ctypes.Structure):
    _fields_ = [("top_k", ctypes.c_int32), ("local_blocks", ctypes.c_int32)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run `python -m windowed_attention_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER
    sig = {
        "uf_kvcache_storage_bytes": (ctypes.c_size_t, [P(uf_kvcache_desc)]),
        "uf_attn_workspace_bytes": (ctypes.c_size_t, [P(uf_kvcache_desc)]),
        "uf_kvcache_create": (ctypes.c_int, [P(uf_kvcache_desc), P(ctypes.c_void_p)]),
        "uf_kvcache_destroy": (ctypes.c_int, [ctypes.c_void_p]),
        "uf_kvcache_reset": (ctypes.c_int, [ctypes.c_void_p]),
        "uf_kvcache_set_window": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]),
        "uf_kvcache_append": (ctypes.c_int, [ctypes.c_void_p, P(uf_tensor), P(uf_tensor), ctypes.c_int32,
                                             ctypes.c_uint32, ctypes.c_void_p]),
        "uf_kvcache_plan_append": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32,
                                                  P(uf_append_plan)]),
        "uf_kvcache_window": (ctypes.c_int, [ctypes.c_void_p, P(uf_window_info)]),
        "uf_attn_step": (ctypes.c_int, [P(uf_tensor), ctypes.c_void_p, P(uf_block_mask), P(uf_tensor),
                                        ctypes.c_void_p]),
        "uf_attn_step_static": (ctypes.c_int, [P(uf_tensor), ctypes.c_void_p, P(uf_block_mask), P(uf_tensor),
                                               ctypes.c_void_p]),
        "uf_block_mask_workspace_bytes": (ctypes.c_size_t, [P(uf_kvcache_desc), ctypes.c_int32, ctypes.c_int32]),
        "uf_block_mask_topk": (ctypes.c_int, [P(uf_tensor), ctypes.c_void_p, P(uf_topk_params), ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
        "uf_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "uf_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


class UfError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = _lib.uf_last_error().decode()
        super().__init__(f"{where}: {_lib.uf_status_string(status).decode()} ({detail})")


def _check(status: int, where: str) -> int:
    if status != UF_OK:
        raise UfError(status, where)
    return status


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def tensor_of(t) -> uf_tensor:
    """uf_tensor view of a torch bf16 tensor [tokens, heads, head_dim] (last dim contiguous)."""
    import torch
    if t.dtype != torch.bfloat16 or t.dim() != 3 or t.stride(2) != 1:
        raise ValueError("expected a bf16 tensor [tokens, heads, head_dim] with contiguous head_dim")
    return uf_tensor(t.data_ptr(), UF_BF16, t.shape[0], t.shape[1], t.shape[2], t.stride(0), t.stride(1))


def mask_of(m) -> uf_block_mask:
    """uf_block_mask view of a torch uint8 tensor [heads, q_blocks, k_blocks] (last dim contiguous)."""
    import torch
    if m.dtype != torch.uint8 or m.dim() != 3 or m.stride(2) != 1:
        raise ValueError("expected a uint8 tensor [heads, q_blocks, k_blocks] with contiguous k_blocks")
    return uf_block_mask(m.data_ptr(), m.shape[0], m.shape[1], m.shape[2], m.stride(0), m.stride(1))


# -- the C entry points, same names -------------------------------------------------------------

def uf_kvcache_storage_bytes(desc: uf_kvcache_desc) -> int:
    return _lib.uf_kvcache_storage_bytes(ctypes.byref(desc))


def uf_attn_workspace_bytes(desc: uf_kvcache_desc) -> int:
    return _lib.uf_attn_workspace_bytes(ctypes.byref(desc))


def uf_kvcache_create(desc: uf_kvcache_desc) -> int:
    handle = ctypes.c_void_p()
    _check(_lib.uf_kvcache_create(ctypes.byref(desc), ctypes.byref(handle)), "uf_kvcache_create")
    return handle.value


def uf_kvcache_destroy(handle: int) -> None:
    _check(_lib.uf_kvcache_destroy(handle), "uf_kvcache_destroy")


def uf_kvcache_reset(handle: int) -> None:
    _check(_lib.uf_kvcache_reset(handle), "uf_kvcache_reset")


def uf_kvcache_set_window(handle: int, active_frames: int) -> None:
    _check(_lib.uf_kvcache_set_window(handle, active_frames), "uf_kvcache_set_window")


def uf_kvcache_append(handle: int, k_new, v_new, n_frames: int, flags: int = 0, stream=None) -> None:
    kt = None if k_new is None else ctypes.byref(tensor_of(k_new))
    vt = None if v_new is None else ctypes.byref(tensor_of(v_new))
    s = None if flags & UF_APPEND_COMMIT_ONLY else _stream_handle(stream)
    _check(_lib.uf_kvcache_append(handle, kt, vt, n_frames, flags, s), "uf_kvcache_append")


def uf_kvcache_plan_append(handle: int, n_frames: int, flags: int = 0) -> uf_append_plan:
    plan = uf_append_plan()
    _check(_lib.uf_kvcache_plan_append(handle, n_frames, flags, ctypes.byref(plan)), "uf_kvcache_plan_append")
    return plan


def uf_kvcache_window(handle: int) -> uf_window_info:
    info = uf_window_info()
    _check(_lib.uf_kvcache_window(handle, ctypes.byref(info)), "uf_kvcache_window")
    return info


def uf_attn_step(q, handle: int, block_mask, out, stream=None) -> None:
    m = None if block_mask is None else ctypes.byref(mask_of(block_mask))
    _check(_lib.uf_attn_step(ctypes.byref(tensor_of(q)), handle, m, ctypes.byref(tensor_of(out)),
                             _stream_handle(stream)), "uf_attn_step")


def uf_attn_step_static(q, handle: int, block_mask, out, stream=None) -> None:
    m = None if block_mask is None else ctypes.byref(mask_of(block_mask))
    _check(_lib.uf_attn_step_static(ctypes.byref(tensor_of(q)), handle, m, ctypes.byref(tensor_of(out)),
                                    _stream_handle(stream)), "uf_attn_step_static")


def uf_block_mask_workspace_bytes(desc: uf_kvcache_desc, n_q_tokens: int, n_q_heads: int) -> int:
    return _lib.uf_block_mask_workspace_bytes(ctypes.byref(desc), n_q_tokens, n_q_heads)


def uf_block_mask_topk(q, handle: int, top_k: int, local_blocks: int, mask, scores, workspace,
                       stream=None) -> None:
    """mask: uint8 [Hq, q_tiles, k_tiles] contiguous; scores: float32 of that shape or None;
    workspace: a device tensor of at least uf_block_mask_workspace_bytes bytes."""
    import torch
    if mask.dtype != torch.uint8 or not mask.is_contiguous():
        raise ValueError("mask must be a contiguous uint8 tensor")
    if scores is not None and (scores.dtype != torch.float32 or not scores.is_contiguous()):
        raise ValueError("scores must be a contiguous float32 tensor")
    params = uf_topk_params(top_k, local_blocks)
    _check(_lib.uf_block_mask_topk(ctypes.byref(tensor_of(q)), handle, ctypes.byref(params), mask.data_ptr(),
                                   None if scores is None else scores.data_ptr(), workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), _stream_handle(stream)),
           "uf_block_mask_topk")


def uf_status_string(status: int) -> str:
    return _lib.uf_status_string(status).decode()


def uf_last_error() -> str:
    return _lib.uf_last_error().decode()


def raw_lib():
    """The loaded ctypes library (for calls with hand-built, possibly invalid, arguments)."""
    return _lib


class KVCache:
    """A rolling KV cache whose device memory is held by torch tensors.

    Storage, workspace and the handle's lifetime are tied to this object;
    every method calls one C entry point.
    """

    def __init__(self, n_kv_heads: int, head_dim: int, tokens_per_frame: int, window_frames: int,
                 anchor_frames: int = 0, device="cuda", workspace: bool = True, kv_dtype: int = UF_BF16,
                 q_scale: float = 1.0, k_scale: float = 1.0, v_scale: float = 1.0, block_grid=(0, 0),
                 max_q_heads: int = 0, max_q_tokens: int = 0, heads_per_wg: int = 0, splits: int = 0,
                 k_storage=None, v_storage=None, workspace_bytes: int = None, pipeline: int = 0):
        """k_storage / v_storage: caller-made device tensors of the storage's shape
        [n_kv_heads, (anchor_frames + window_frames) * tokens_per_frame, head_dim] (bf16, or uint8
        for FP8), e.g. views into larger buffers; allocated here when not given.
        workspace_bytes: size of the workspace allocated here (default: uf_attn_workspace_bytes)."""
        import torch
        desc = uf_kvcache_desc(n_kv_heads, head_dim, tokens_per_frame, window_frames, anchor_frames,
                               None, None, None, 0, kv_dtype, q_scale, k_scale, v_scale,
                               block_grid[0], block_grid[1], max_q_heads, max_q_tokens, heads_per_wg, splits,
                               pipeline)
        nbytes = uf_kvcache_storage_bytes(desc)
        if nbytes == 0:
            _check(_lib.uf_kvcache_create(ctypes.byref(desc), ctypes.byref(ctypes.c_void_p())), "KVCache")
        rows = (anchor_frames + window_frames) * tokens_per_frame
        tdt = torch.uint8 if kv_dtype == UF_FP8_E4M3 else torch.bfloat16
        shape = (n_kv_heads, rows, head_dim)
        for t in (k_storage, v_storage):
            if t is not None and (tuple(t.shape) != shape or t.dtype != tdt or not t.is_contiguous()):
                raise ValueError(f"storage must be a contiguous {tdt} tensor of shape {shape}")
        self.k_storage = torch.empty(shape, dtype=tdt, device=device) if k_storage is None else k_storage
        self.v_storage = torch.empty_like(self.k_storage) if v_storage is None else v_storage
        ws_bytes = (uf_attn_workspace_bytes(desc) if workspace_bytes is None else workspace_bytes) if workspace else 0
        self.workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=device)
        desc.k_storage = self.k_storage.data_ptr()
        desc.v_storage = self.v_storage.data_ptr()
        desc.workspace = self.workspace.data_ptr() if ws_bytes else None
        desc.workspace_bytes = ws_bytes
        self.desc = desc
        self.handle = uf_kvcache_create(desc)

    def append(self, k_new, v_new, n_frames: int, flags: int = 0, stream=None):
        uf_kvcache_append(self.handle, k_new, v_new, n_frames, flags, stream)

    def plan_append(self, n_frames: int, flags: int = 0):
        return uf_kvcache_plan_append(self.handle, n_frames, flags)

    def window(self):
        return uf_kvcache_window(self.handle)

    def set_window(self, active_frames: int):
        uf_kvcache_set_window(self.handle, active_frames)

    def reset(self):
        uf_kvcache_reset(self.handle)

    def attn_step(self, q, out, block_mask=None, stream=None):
        uf_attn_step(q, self.handle, block_mask, out, stream)
        return out

    def attn_step_static(self, q, out, block_mask=None, stream=None):
        uf_attn_step_static(q, self.handle, block_mask, out, stream)
        return out

    def block_mask_topk(self, q, top_k: int, local_blocks: int = 0, mask=None, scores=None, workspace=None,
                        stream=None):
        """Top-k block mask of q against the current window (uf_block_mask_topk).

        mask / scores / workspace are allocated here when not given; returns mask."""
        import torch
        n_q, hq = q.shape[0], q.shape[1]
        n_qb = -(-n_q // UF_TILE)
        n_kb = -(-self.window().n_keys // UF_TILE)
        if mask is None:
            mask = torch.empty((hq, n_qb, n_kb), dtype=torch.uint8, device=q.device)
        if workspace is None:
            nbytes = uf_block_mask_workspace_bytes(self.desc, n_q, hq)
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
        uf_block_mask_topk(q, self.handle, top_k, local_blocks, mask, scores, workspace, stream)
        return mask

    def close(self):
        if self.handle:
            uf_kvcache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
