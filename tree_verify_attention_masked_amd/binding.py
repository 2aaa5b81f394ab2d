"""ctypes binding of libspectree (include/spectree.h) for PyTorch tensors.

Argument marshalling only: shapes are read from the tensors, outputs and
workspaces are allocated with torch on the tensors' device, and the raw device
pointers plus torch's current HIP stream are handed to the C ABI.  Every step
of the computation runs in the library's HIP kernels; if the library is not
built this module raises instead of computing anything another way.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspectree.so")
HEADER_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "spectree.h")

SPEC_OK = 0
SPEC_ERR_INVALID_ARG = -1
SPEC_ERR_UNSUPPORTED = -2
SPEC_ERR_WORKSPACE = -3
SPEC_ERR_HIP = -4
SPEC_F32 = 0
SPEC_BF16 = 1

DEV_ERRORS = {1: "parent", 2: "block", 4: "length", 8: "token", 16: "nonfinite", 32: "empty", 64: "path",
              128: "timeout"}

_c_i32p = ctypes.c_void_p
_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t

_SIGNATURES = {
    "spec_status_string": (ctypes.c_char_p, [_i]),
    "spec_version": (_i, []),
    "spec_tree_attn_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "spec_tree_attn": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i,
                            ctypes.c_float, _i, _vp, _vp, _sz, _vp]),
    "spec_tree_reject_workspace_size": (_sz, [_i, _i, _i]),
    "spec_sequoia_tree": (_i, [ctypes.c_void_p, _i, _i, _i, ctypes.c_void_p, ctypes.c_void_p]),
    "spec_tree_reject_plan": (_i, [_i, _i, _i, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]),
    "spec_tree_reject_max_resident": (ctypes.c_int64, []),
    "spec_tree_reject": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, ctypes.c_float, _i, ctypes.c_uint64,
                              ctypes.c_uint64, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "spec_kv_compact": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _vp, _vp]),
    "spec_tree_kv_write": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i,
                                ctypes.c_float, _i, _vp]),
    "spec_tree_write_attn_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "spec_tree_write_attn": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i,
                                  ctypes.c_float, ctypes.c_float, _i, _vp, _vp, _sz, _vp]),
    "spec_tree_truncate": (_i, [_vp, _vp, _i, _i, _i, ctypes.c_float, _i, ctypes.c_float, _vp, _vp]),
    "spec_tree_reject_compact": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, ctypes.c_float, _i, ctypes.c_uint64,
                                      ctypes.c_uint64, _vp, _vp, _vp, _vp, _vp, _sz,
                                      _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "spec_tree_reject_truncated_workspace_size": (_sz, [_i, _i, _i, _i]),
    "spec_tree_reject_truncated_plan": (_i, [_i, _i, _i, _i, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]),
    "spec_tree_reject_truncated": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, ctypes.c_float, _i, ctypes.c_float, _i,
                                        ctypes.c_uint64, ctypes.c_uint64, _vp, _vp, _vp, _vp, _vp, _sz,
                                        _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "spec_tree_reject_compact_noalloc": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, ctypes.c_float, _i, ctypes.c_uint64,
                                              ctypes.c_uint64, _vp, _vp, _vp, _vp,
                                              _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
}

_lib = None


class SpecError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = load_library().spec_status_string(code).decode()
        super().__init__(f"{where}: {msg} ({code})")
        self.code = code


def load_library():
    """Load libspectree.so (built in-tree by tree_verify_attention_masked_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m tree_verify_attention_masked_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def header_functions() -> list:
    """Names of the functions include/spectree.h declares."""
    with open(HEADER_PATH) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z_]+)\s*\(", text)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    if t.dtype == torch.float32:
        return SPEC_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(rc, where):
    if rc != SPEC_OK:
        raise SpecError(rc, where)


def spec_tree_attn_workspace_size(B, T, Hq, Hkv, D, max_blocks_per_seq, dtype_code) -> int:
    return int(load_library().spec_tree_attn_workspace_size(B, T, Hq, Hkv, D, max_blocks_per_seq, dtype_code))


def spec_tree_attn(q, k_cache, v_cache, block_table, prefix_lens, parent, scale=None, out=None,
                   status=None, workspace=None):
    """Tree-masked verify attention.  q [B,T,Hq,D], caches [num_blocks,Hkv,16,D] -> out [B,T,Hq,D]."""
    lib = load_library()
    _need(q, "q", ndim=4)
    _need(k_cache, "k_cache", dtype=q.dtype, ndim=4)
    _need(v_cache, "v_cache", dtype=q.dtype, ndim=4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(prefix_lens, "prefix_lens", torch.int32, 1)
    _need(parent, "parent", torch.int32, 2)
    B, T, Hq, D = q.shape
    nb, Hkv, bs, D2 = k_cache.shape
    if v_cache.shape != k_cache.shape or D2 != D:
        raise ValueError("k_cache / v_cache / q shapes disagree")
    if tuple(parent.shape) != (B, T) or prefix_lens.shape[0] != B or block_table.shape[0] != B:
        raise ValueError("parent / prefix_lens / block_table shapes disagree with q")
    code = _dtype_code(q)
    mb = block_table.shape[1]
    if scale is None:
        scale = 1.0 / (D ** 0.5)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", q.dtype)
    if status is not None:
        _need(status, "status", torch.int32, 1)
    ws = int(lib.spec_tree_attn_workspace_size(B, T, Hq, Hkv, D, mb, code))
    if workspace is None and ws > 0:  # zero-filled: its header holds split arrival counters
        workspace = torch.zeros(ws, dtype=torch.uint8, device=q.device)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.spec_tree_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(prefix_lens),
                            _ptr(parent), _ptr(out), B, T, Hq, Hkv, D, bs, mb, nb, float(scale), code,
                            _ptr(status), _ptr(workspace), wsz, _stream(q.device))
    _check(rc, "spec_tree_attn")
    return out


def spec_tree_reject(target_logits, draft_probs, draft_tokens, parent, temperature, without_replacement=False,
                     seed=0, offset=0, accepted_nodes=None, out_tokens=None, num_accepted=None, status=None,
                     workspace=None):
    """Tree rejection sampling.  Returns (accepted_nodes [B,T], out_tokens [B,T], num_accepted [B])."""
    lib = load_library()
    _need(target_logits, "target_logits", torch.float32, 3)
    _need(draft_tokens, "draft_tokens", torch.int32, 2)
    _need(parent, "parent", torch.int32, 2)
    B, T, V = target_logits.shape
    if draft_probs is not None:
        _need(draft_probs, "draft_probs", torch.float32, 3)
        if tuple(draft_probs.shape) != (B, T, V):
            raise ValueError("draft_probs shape disagrees with target_logits")
    if tuple(draft_tokens.shape) != (B, T) or tuple(parent.shape) != (B, T):
        raise ValueError("draft_tokens / parent shapes disagree with target_logits")
    dev = target_logits.device
    if accepted_nodes is None:
        accepted_nodes = torch.empty((B, T), dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, T), dtype=torch.int32, device=dev)
    if num_accepted is None:
        num_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    if status is not None:
        _need(status, "status", torch.int32, 1)
    ws = int(lib.spec_tree_reject_workspace_size(B, T, V))
    if workspace is None and ws > 0:  # zero-filled: its header holds the exit counter and the call epoch
        workspace = torch.zeros(ws, dtype=torch.uint8, device=dev)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.spec_tree_reject(_ptr(target_logits), _ptr(draft_probs), _ptr(draft_tokens), _ptr(parent),
                              B, T, V, float(temperature), int(bool(without_replacement)),
                              int(seed) & (2 ** 64 - 1), int(offset) & (2 ** 64 - 1),
                              _ptr(accepted_nodes), _ptr(out_tokens), _ptr(num_accepted), _ptr(status),
                              _ptr(workspace), wsz, _stream(dev))
    _check(rc, "spec_tree_reject")
    return accepted_nodes, out_tokens, num_accepted


def spec_kv_compact(k_cache, v_cache, block_table, prefix_lens, accepted_nodes, num_accepted, new_lens=None,
                    status=None):
    """In-place compaction of the paged KV cache to the accepted path.  Returns new_lens [B]."""
    lib = load_library()
    _need(k_cache, "k_cache", ndim=4)
    _need(v_cache, "v_cache", k_cache.dtype, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(prefix_lens, "prefix_lens", torch.int32, 1)
    _need(accepted_nodes, "accepted_nodes", torch.int32, 2)
    _need(num_accepted, "num_accepted", torch.int32, 1)
    nb, Hkv, bs, D = k_cache.shape
    B, T = accepted_nodes.shape
    if new_lens is None:
        new_lens = torch.empty((B,), dtype=torch.int32, device=k_cache.device)
    if status is not None:
        _need(status, "status", torch.int32, 1)
    rc = lib.spec_kv_compact(_ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(prefix_lens),
                             _ptr(accepted_nodes), _ptr(num_accepted), _ptr(new_lens), B, T, Hkv, D, bs,
                             block_table.shape[1], nb, _dtype_code(k_cache), _ptr(status),
                             _stream(k_cache.device))
    _check(rc, "spec_kv_compact")
    return new_lens


def spec_tree_reject_compact(target_logits, draft_probs, draft_tokens, parent, temperature, k_cache, v_cache,
                             block_table, prefix_lens, without_replacement=False, seed=0, offset=0,
                             accepted_nodes=None, out_tokens=None, num_accepted=None, new_lens=None, status=None,
                             workspace=None):
    """spec_tree_reject, then compaction of the KV cache along the accepted path, in one launch.
    Returns (accepted_nodes [B,T], out_tokens [B,T], num_accepted [B], new_lens [B])."""
    lib = load_library()
    _need(target_logits, "target_logits", torch.float32, 3)
    _need(draft_tokens, "draft_tokens", torch.int32, 2)
    _need(parent, "parent", torch.int32, 2)
    _need(k_cache, "k_cache", ndim=4)
    _need(v_cache, "v_cache", k_cache.dtype, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(prefix_lens, "prefix_lens", torch.int32, 1)
    B, T, V = target_logits.shape
    if draft_probs is not None:
        _need(draft_probs, "draft_probs", torch.float32, 3)
        if tuple(draft_probs.shape) != (B, T, V):
            raise ValueError("draft_probs shape disagrees with target_logits")
    if tuple(draft_tokens.shape) != (B, T) or tuple(parent.shape) != (B, T):
        raise ValueError("draft_tokens / parent shapes disagree with target_logits")
    nb, Hkv, bs, D = k_cache.shape
    dev = target_logits.device
    if accepted_nodes is None:
        accepted_nodes = torch.empty((B, T), dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, T), dtype=torch.int32, device=dev)
    if num_accepted is None:
        num_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    if new_lens is None:
        new_lens = torch.empty((B,), dtype=torch.int32, device=dev)
    if status is not None:
        _need(status, "status", torch.int32, 1)
    ws = int(lib.spec_tree_reject_workspace_size(B, T, V))
    if workspace is None and ws > 0:  # zero-filled: its header holds the exit counter and the call epoch
        workspace = torch.zeros(ws, dtype=torch.uint8, device=dev)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.spec_tree_reject_compact(_ptr(target_logits), _ptr(draft_probs), _ptr(draft_tokens), _ptr(parent),
                                      B, T, V, float(temperature), int(bool(without_replacement)),
                                      int(seed) & (2 ** 64 - 1), int(offset) & (2 ** 64 - 1),
                                      _ptr(accepted_nodes), _ptr(out_tokens), _ptr(num_accepted), _ptr(status),
                                      _ptr(workspace), wsz, _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                      _ptr(prefix_lens), _ptr(new_lens), Hkv, D, bs, block_table.shape[1], nb,
                                      _dtype_code(k_cache), _stream(dev))
    _check(rc, "spec_tree_reject_compact")
    return accepted_nodes, out_tokens, num_accepted, new_lens


def spec_tree_reject_truncated(target_logits, draft_probs, draft_tokens, parent, temperature, top_k, top_p=1.0,
                               without_replacement=False, seed=0, offset=0, k_cache=None, v_cache=None,
                               block_table=None, prefix_lens=None, accepted_nodes=None, out_tokens=None,
                               num_accepted=None, new_lens=None, status=None, workspace=None):
    """spec_tree_reject against the target truncated to top_k (1..64), then top_p, applied to the rows the walk
    visits; with k_cache given, also the compaction of spec_tree_reject_compact.
    Returns (accepted_nodes [B,T], out_tokens [B,T], num_accepted [B], new_lens [B] or None)."""
    lib = load_library()
    _need(target_logits, "target_logits", torch.float32, 3)
    _need(draft_tokens, "draft_tokens", torch.int32, 2)
    _need(parent, "parent", torch.int32, 2)
    B, T, V = target_logits.shape
    if draft_probs is not None:
        _need(draft_probs, "draft_probs", torch.float32, 3)
        if tuple(draft_probs.shape) != (B, T, V):
            raise ValueError("draft_probs shape disagrees with target_logits")
    if tuple(draft_tokens.shape) != (B, T) or tuple(parent.shape) != (B, T):
        raise ValueError("draft_tokens / parent shapes disagree with target_logits")
    dev = target_logits.device
    compact = k_cache is not None
    nb = Hkv = bs = D = mb = 0
    code = SPEC_F32
    if compact:
        _need(k_cache, "k_cache", ndim=4)
        _need(v_cache, "v_cache", k_cache.dtype, 4)
        _need(block_table, "block_table", torch.int32, 2)
        _need(prefix_lens, "prefix_lens", torch.int32, 1)
        nb, Hkv, bs, D = k_cache.shape
        mb = block_table.shape[1]
        code = _dtype_code(k_cache)
        if new_lens is None:
            new_lens = torch.empty((B,), dtype=torch.int32, device=dev)
    if accepted_nodes is None:
        accepted_nodes = torch.empty((B, T), dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, T), dtype=torch.int32, device=dev)
    if num_accepted is None:
        num_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    if status is not None:
        _need(status, "status", torch.int32, 1)
    ws = int(lib.spec_tree_reject_truncated_workspace_size(B, T, V, int(top_k)))
    if workspace is None and ws > 0:  # zero-filled: its header holds the exit counter and the call epoch
        workspace = torch.zeros(ws, dtype=torch.uint8, device=dev)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.spec_tree_reject_truncated(_ptr(target_logits), _ptr(draft_probs), _ptr(draft_tokens), _ptr(parent),
                                        B, T, V, float(temperature), int(top_k), float(top_p),
                                        int(bool(without_replacement)), int(seed) & (2 ** 64 - 1),
                                        int(offset) & (2 ** 64 - 1), _ptr(accepted_nodes), _ptr(out_tokens),
                                        _ptr(num_accepted), _ptr(status), _ptr(workspace), wsz,
                                        _ptr(k_cache) if compact else None, _ptr(v_cache) if compact else None,
                                        _ptr(block_table) if compact else None,
                                        _ptr(prefix_lens) if compact else None,
                                        _ptr(new_lens) if compact else None, Hkv, D, bs, mb, nb, code, _stream(dev))
    _check(rc, "spec_tree_reject_truncated")
    return accepted_nodes, out_tokens, num_accepted, new_lens


def spec_tree_reject_truncated_workspace_size(B, T, V, top_k) -> int:
    return int(load_library().spec_tree_reject_truncated_workspace_size(B, T, V, top_k))


def spec_tree_reject_truncated_plan(B, T, V, top_k, max_resident_workgroups):
    """(team size, length of the members' first lists) of the truncating sampler on a device holding
    `max_resident_workgroups` of its workgroups at once (host only)."""
    team, kc = ctypes.c_int(0), ctypes.c_int(0)
    rc = load_library().spec_tree_reject_truncated_plan(B, T, V, int(top_k), int(max_resident_workgroups),
                                                        ctypes.byref(team), ctypes.byref(kc))
    _check(rc, "spec_tree_reject_truncated_plan")
    return team.value, kc.value


def spec_tree_reject_compact_noalloc(target_logits, draft_probs, draft_tokens, parent, temperature, k_cache,
                                     v_cache, block_table, prefix_lens, accepted_nodes, out_tokens, num_accepted,
                                     new_lens, without_replacement=False, seed=0, offset=0, status=None):
    """spec_tree_reject_compact on the library's static workspace: the caller passes every output (nothing is
    allocated here or in the call).  Returns (accepted_nodes, out_tokens, num_accepted, new_lens)."""
    lib = load_library()
    _need(target_logits, "target_logits", torch.float32, 3)
    _need(draft_tokens, "draft_tokens", torch.int32, 2)
    _need(parent, "parent", torch.int32, 2)
    _need(k_cache, "k_cache", ndim=4)
    _need(v_cache, "v_cache", k_cache.dtype, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(prefix_lens, "prefix_lens", torch.int32, 1)
    B, T, V = target_logits.shape
    if draft_probs is not None:
        _need(draft_probs, "draft_probs", torch.float32, 3)
        if tuple(draft_probs.shape) != (B, T, V):
            raise ValueError("draft_probs shape disagrees with target_logits")
    if tuple(draft_tokens.shape) != (B, T) or tuple(parent.shape) != (B, T):
        raise ValueError("draft_tokens / parent shapes disagree with target_logits")
    for t, name, shape in ((accepted_nodes, "accepted_nodes", (B, T)), (out_tokens, "out_tokens", (B, T)),
                           (num_accepted, "num_accepted", (B,)), (new_lens, "new_lens", (B,))):
        _need(t, name, torch.int32, len(shape))
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}")
    if status is not None:
        _need(status, "status", torch.int32, 1)
    nb, Hkv, bs, D = k_cache.shape
    rc = lib.spec_tree_reject_compact_noalloc(_ptr(target_logits), _ptr(draft_probs), _ptr(draft_tokens),
                                              _ptr(parent), B, T, V, float(temperature), int(bool(without_replacement)),
                                              int(seed) & (2 ** 64 - 1), int(offset) & (2 ** 64 - 1),
                                              _ptr(accepted_nodes), _ptr(out_tokens), _ptr(num_accepted), _ptr(status),
                                              _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(prefix_lens),
                                              _ptr(new_lens), Hkv, D, bs, block_table.shape[1], nb,
                                              _dtype_code(k_cache), _stream(target_logits.device))
    _check(rc, "spec_tree_reject_compact_noalloc")
    return accepted_nodes, out_tokens, num_accepted, new_lens


def spec_tree_kv_write(k_new, v_new, q, k_cache, v_cache, block_table, prefix_lens, parent, rope_theta,
                       status=None):
    """Write every tree node's K/V rows into the paged cache at slot prefix + node, the keys and (if q is
    given) the queries rotated in place for position prefix + depth.  Returns nothing."""
    lib = load_library()
    _need(k_new, "k_new", ndim=4)
    _need(v_new, "v_new", k_new.dtype, 4)
    _need(k_cache, "k_cache", k_new.dtype, 4)
    _need(v_cache, "v_cache", k_new.dtype, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(prefix_lens, "prefix_lens", torch.int32, 1)
    _need(parent, "parent", torch.int32, 2)
    B, T, Hkv, D = k_new.shape
    if tuple(v_new.shape) != (B, T, Hkv, D):
        raise ValueError("v_new shape disagrees with k_new")
    Hq = 0
    if q is not None:
        _need(q, "q", k_new.dtype, 4)
        if q.shape[0] != B or q.shape[1] != T or q.shape[3] != D:
            raise ValueError("q shape disagrees with k_new")
        Hq = q.shape[2]
    nb, _, bs, _ = k_cache.shape
    if status is not None:
        _need(status, "status", torch.int32, 1)
    rc = lib.spec_tree_kv_write(_ptr(k_new), _ptr(v_new), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                _ptr(prefix_lens), _ptr(parent), _ptr(status), B, T, Hq, Hkv, D, bs,
                                block_table.shape[1], nb, float(rope_theta), _dtype_code(k_new),
                                _stream(k_new.device))
    _check(rc, "spec_tree_kv_write")


def spec_tree_write_attn_workspace_size(B, T, Hq, Hkv, D, max_blocks_per_seq, dtype_code) -> int:
    return int(load_library().spec_tree_write_attn_workspace_size(B, T, Hq, Hkv, D, max_blocks_per_seq, dtype_code))


def spec_tree_write_attn(k_new, v_new, q, k_cache, v_cache, block_table, prefix_lens, parent, rope_theta,
                         scale=None, out=None, status=None, workspace=None):
    """spec_tree_kv_write and spec_tree_attn in one launch: the tree's K/V rows into the cache (keys rotated for
    position prefix + depth), then attention with the queries rotated the same way (q itself is not modified).
    k_new, v_new [B,T,Hkv,D], q [B,T,Hq,D], caches [num_blocks,Hkv,16,D] (bf16) -> out [B,T,Hq,D]."""
    lib = load_library()
    _need(q, "q", ndim=4)
    _need(k_new, "k_new", q.dtype, 4)
    _need(v_new, "v_new", q.dtype, 4)
    _need(k_cache, "k_cache", q.dtype, 4)
    _need(v_cache, "v_cache", q.dtype, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(prefix_lens, "prefix_lens", torch.int32, 1)
    _need(parent, "parent", torch.int32, 2)
    B, T, Hq, D = q.shape
    nb, Hkv, bs, D2 = k_cache.shape
    if v_cache.shape != k_cache.shape or D2 != D:
        raise ValueError("k_cache / v_cache / q shapes disagree")
    if tuple(k_new.shape) != (B, T, Hkv, D) or tuple(v_new.shape) != (B, T, Hkv, D):
        raise ValueError("k_new / v_new shapes disagree with q and the cache")
    if tuple(parent.shape) != (B, T) or prefix_lens.shape[0] != B or block_table.shape[0] != B:
        raise ValueError("parent / prefix_lens / block_table shapes disagree with q")
    code = _dtype_code(q)
    mb = block_table.shape[1]
    if scale is None:
        scale = 1.0 / (D ** 0.5)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", q.dtype)
    if status is not None:
        _need(status, "status", torch.int32, 1)
    ws = int(lib.spec_tree_write_attn_workspace_size(B, T, Hq, Hkv, D, mb, code))
    if workspace is None:  # zero-filled: its header holds the work counter and the write flags
        workspace = torch.zeros(max(ws, 1), dtype=torch.uint8, device=q.device)
    wsz = workspace.numel() * workspace.element_size()
    rc = lib.spec_tree_write_attn(_ptr(k_new), _ptr(v_new), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(block_table), _ptr(prefix_lens), _ptr(parent), _ptr(out), B, T, Hq, Hkv, D,
                                  bs, mb, nb, float(rope_theta), float(scale), code, _ptr(status), _ptr(workspace),
                                  wsz, _stream(q.device))
    _check(rc, "spec_tree_write_attn")
    return out


def spec_sequoia_tree(accept, n, max_depth):
    """(parent array [n] int32 as a numpy array, expected tokens per step) of the Sequoia-optimal tree of n nodes
    and depth <= max_depth for a per-rank acceptance vector (host only, no GPU)."""
    import numpy as np

    acc = np.ascontiguousarray(np.asarray(accept, dtype=np.float64).ravel())
    parent = np.zeros(int(n), dtype=np.int32)
    val = ctypes.c_double(0.0)
    rc = load_library().spec_sequoia_tree(acc.ctypes.data_as(ctypes.c_void_p) if acc.size else None, int(acc.size),
                                          int(n), int(max_depth), parent.ctypes.data_as(ctypes.c_void_p),
                                          ctypes.byref(val))
    _check(rc, "spec_sequoia_tree")
    return parent, val.value


def spec_tree_reject_plan(B, T, V, max_resident_workgroups):
    """(team size, slice length) the sampler uses on a device holding `max_resident_workgroups` of its
    workgroups at once (host only)."""
    team, sl = ctypes.c_int(0), ctypes.c_int(0)
    rc = load_library().spec_tree_reject_plan(B, T, V, int(max_resident_workgroups), ctypes.byref(team),
                                              ctypes.byref(sl))
    _check(rc, "spec_tree_reject_plan")
    return team.value, sl.value


def spec_tree_reject_max_resident() -> int:
    """Workgroups of the sampler kernel the current GPU holds at once."""
    return int(load_library().spec_tree_reject_max_resident())


def spec_status_string(code: int) -> str:
    return load_library().spec_status_string(code).decode()


def spec_version() -> int:
    return int(load_library().spec_version())


def spec_tree_truncate(target_logits, temperature, top_k=0, top_p=1.0, out=None, status=None):
    """Top-k / top-p truncation of [B, T, V] float32 target logits: dropped entries become -inf.  In place
    when out is None (returns target_logits), else into out (a disjoint [B, T, V] float32 tensor)."""
    lib = load_library()
    _need(target_logits, "target_logits", torch.float32, 3)
    B, T, V = target_logits.shape
    if out is None:
        out = target_logits
    else:
        _need(out, "out", torch.float32, 3)
        if tuple(out.shape) != (B, T, V):
            raise ValueError("out shape disagrees with target_logits")
    if status is not None:
        _need(status, "status", torch.int32, 1)
    rc = lib.spec_tree_truncate(_ptr(target_logits), _ptr(out), B, T, V, float(temperature), int(top_k),
                                float(top_p), _ptr(status), _stream(target_logits.device))
    _check(rc, "spec_tree_truncate")
    return out
