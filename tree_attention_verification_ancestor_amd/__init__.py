"""Python binding of the tav C ABI (``include/tav.h``): tree-attention
verification on AMD MI355X.

Argument marshalling only: every function checks tensor placement, dtype and
layout, allocates outputs and workspaces with torch when the caller passes
none, and calls the C entry point of the same name on the current HIP stream.
All arithmetic runs in the library's HIP kernels. If ``libtav.so`` has not
been built, every call raises; there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os
import re
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# TAV_LIBRARY names another build of the library (a sanitized host build, say)
LIB_PATH = os.environ.get("TAV_LIBRARY") or os.path.join(_HERE, "libtav.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "tav.h")

OK = 0
ERR_ARG = 1
ERR_UNSUPPORTED = 2
ERR_WORKSPACE = 3
ERR_LAUNCH = 4

FLAG_BAD_PARENT = 0x1
FLAG_BAD_BLOCK = 0x2
FLAG_NONFINITE_LOGITS = 0x4
FLAG_CAPACITY = 0x8
FLAG_BAD_TOKEN = 0x10
FLAG_SYNC_TIMEOUT = 0x20
FLAG_ATTN_RANGE = 0x40

BLOCK = 16


class TavError(RuntimeError):
    """A tav entry point returned a non-OK status."""

    def __init__(self, name: str, status: int):
        super().__init__(f"{name}: {status_string(status)} (status {status})")
        self.status = status


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_U64 = ctypes.c_uint64
_F32 = ctypes.c_float
_F64 = ctypes.c_double
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "tav_abi_version": (_I32, []),
    "tav_status_string": (ctypes.c_char_p, [_I32]),
    "tree_mask_build": (_I32, [_P, _I32, _I32, _P, _P, _P, _P]),
    "tree_attn_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "tav_attn_plan": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P]),
    "tav_sampler_plan": (_I32, [_I32, _I32, _I32, _P]),
    "tav_sampler_plan_for": (_I32, [_I32, _I32, _I32, _I32, _P, _P]),
    "tree_attn_verify": (_I32, [_P, _P, _P, _P, _P, _I32, _P, _I32, _P, _I32, _P, _I32, _I32,
                                _I32, _I32, _I32, _I32, _F32, _P, _P, _SZ, _P, _P]),
    "tree_attn_verify_tree": (_I32, [_P, _P, _P, _P, _P, _I32, _P, _I32, _P, _I32, _P, _P, _P,
                                     _I32, _I32, _I32, _I32, _I32, _I32, _F32, _P, _P, _SZ, _P,
                                     _P]),
    "spec_verify_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "spec_verify_sample": (_I32, [_P, _P, _P, _P, _I32, _I32, _I32, _F64, _U64, _U64, _P, _P,
                                  _P, _P, _SZ, _P, _P]),
    "spec_verify_sample_wor": (_I32, [_P, _P, _P, _P, _I32, _I32, _I32, _F64, _U64, _U64, _P, _P,
                                  _P, _P, _SZ, _P, _P]),
    "spec_verify_sample_probe": (_I32, [_P, _P, _P, _P, _I32, _I32, _I32, _F64, _U64, _U64, _P,
                                        _P, _P, _P, _P, _P, _P, _SZ, _P, _P]),
    "spec_verify_sample_noalloc": (_I32, [_P, _P, _P, _P, _I32, _I32, _I32, _F64, _U64, _U64,
                                          _P, _P, _P, _P, _P]),
    "spec_verify_sample_commit": (_I32, [_P, _P, _P, _P, _I32, _I32, _I32, _F64, _U64, _U64,
                                         _I32, _P, _P, _P, _P, _P, _I32, _P, _I32, _P, _P, _P,
                                         _I32, _I32, _I32, _P, _P, _P, _SZ, _P, _P]),
    "kv_commit_path": (_I32, [_P, _P, _P, _P, _I32, _P, _I32, _P, _P, _P, _I32, _I32, _I32,
                              _I32, _I32, _P, _P, _P, _P]),
    "kv_commit_inplace": (_I32, [_P, _P, _I32, _P, _I32, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                 _P, _P, _P, _P]),
    "tree_expand_workspace_bytes": (_SZ, [_I64, _I32, _I32]),
    "tree_expand_topk": (_I32, [_P, _I64, _I32, _I32, _F64, _P, _P, _P, _P, _SZ, _P, _P]),
    "tree_expand_sample": (_I32, [_P, _I64, _I32, _I32, _F64, _U64, _U64, _P, _P, _P, _P, _SZ, _P, _P]),
    "tree_select_topm": (_I32, [_P, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P, _P]),
    "tree_widths_by_entropy": (_I32, [_P, _I32, _I32, _I32, _I32, _P, _P, _P]),
    "tree_topology_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "tree_topology_dp": (_I32, [_P, _I32, _I32, _I32, _P, _P, _P, _P, _SZ, _P]),
    "tav_model_speedup": (ctypes.c_double, [_F64, _F64, _F64, _I32]),
    "tav_verify_speedup": (ctypes.c_double, [_F64, _F64, _I32, _F64, _F64, _I32, _I32, _F64,
                                             _F64, _F64, _F64, _F64, _F64, _P]),
    "tav_best_chain_length": (_I32, [_F64, _F64, _F64, _I32, _P]),
    "tav_fit_alpha": (ctypes.c_double, [_P, _P, _I32]),
    "tav_philox_uniforms": (_I32, [_U64, _U64, _I32, _I32, _P, _P]),
    "tav_target_probs": (_I32, [_P, _I64, _I32, _F64, _P, _P, _P]),
}


def lib() -> ctypes.CDLL:
    """The loaded ``libtav.so``; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def header_functions(path: str = HEADER_PATH):
    """Names of the functions ``include/tav.h`` declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


def abi_version() -> int:
    return int(lib().tav_abi_version())


def status_string(status: int) -> str:
    return lib().tav_status_string(int(status)).decode()


# ---------------------------------------------------------------------------
# marshalling helpers

def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(name: str, status: int):
    if status != OK:
        raise TavError(name, status)


def _need(t: torch.Tensor, name: str, dtypes, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_I32T = (torch.int32,)
_U32T = (torch.int32, torch.uint32)
_MASKT = (torch.int64, torch.uint64)


def prepare(name: str, *args):
    """A zero-argument callable that calls C entry point ``name`` with
    ``args`` converted once (tensors become their device pointers, streams
    their handles). For tight loops over the same buffers; the caller keeps
    the tensors alive and has checked them with the functions below."""
    fn = getattr(lib(), name)
    conv = []
    for a in args:
        if isinstance(a, torch.Tensor):
            conv.append(ctypes.c_void_p(a.data_ptr()))
        elif isinstance(a, torch.cuda.Stream):
            conv.append(ctypes.c_void_p(a.cuda_stream))
        else:
            conv.append(a)
    conv = tuple(conv)

    def call():
        _check(name, fn(*conv))
    return call


def new_flags(device=None) -> torch.Tensor:
    """A zeroed device word for ``dev_flags``."""
    return torch.zeros(1, dtype=torch.int32, device=device or "cuda")


# ---------------------------------------------------------------------------
# entry points

def tree_mask_build(parent: torch.Tensor, mask: Optional[torch.Tensor] = None,
                    depth: Optional[torch.Tensor] = None, dev_flags: Optional[torch.Tensor] = None,
                    stream=None, want_depth: bool = True):
    """parent int32 [B, N] -> (mask int64 [B, N, ceil(N/64)], depth int32 [B, N] or None)."""
    _need(parent, "parent", _I32T)
    B, N = parent.shape
    W = (N + 63) // 64
    dev = parent.device
    if mask is None:
        mask = torch.empty((B, N, W), dtype=torch.int64, device=dev)
    _need(mask, "mask", _MASKT, (B, N, W), dev)
    if depth is None and want_depth:
        depth = torch.empty((B, N), dtype=torch.int32, device=dev)
    if depth is not None:
        _need(depth, "depth", _I32T, (B, N), dev)
    _check("tree_mask_build", lib().tree_mask_build(_ptr(parent), B, N, _ptr(mask), _ptr(depth),
                                                    _ptr(dev_flags), _stream(stream)))
    return mask, depth


def attn_plan(B, N, Hq, Hkv, D, max_prefix_len, cus, per_cu):
    """tree_attn_verify's work decomposition on a device of ``cus`` compute
    units holding ``per_cu`` workgroups each (host only): a dict with the
    waves per workgroup, row blocks, splits, and the most block-table entries
    a split stages against the capacity of its LDS copy."""
    plan = (ctypes.c_int32 * 5)()
    _check("tav_attn_plan", lib().tav_attn_plan(B, N, Hq, Hkv, D, max_prefix_len, cus, per_cu,
                                                ctypes.cast(plan, ctypes.c_void_p)))
    return {"waves": plan[0], "row_blocks": plan[1], "splits": plan[2],
            "max_split_blocks": plan[3], "capacity": plan[4]}


def sampler_plan(B, V, greedy=False):
    """spec_verify_sample's layout for B sequences of vocabulary V on the
    current device (needs one): entries per thread, workgroups per sequence,
    groups walking at once, vocabulary entries per workgroup, and the
    sequences each group walks in turn."""
    plan = (ctypes.c_int32 * 4)()
    _check("tav_sampler_plan", lib().tav_sampler_plan(B, V, int(bool(greedy)),
                                                      ctypes.cast(plan, ctypes.c_void_p)))
    return {"entries_per_thread": plan[0], "workgroups_per_sequence": plan[1], "groups": plan[2],
            "chunk": plan[3], "sequences_per_group": -(-B // plan[2])}


def sampler_plan_for(B, V, cus, per_cu, greedy=False):
    """``sampler_plan``'s rule on a device of ``cus`` compute units holding
    ``per_cu`` workgroups at once of each walk kernel (4, 8, 16 and 28
    entries per thread, then greedy verification); host only."""
    occ = (ctypes.c_int32 * 5)(*per_cu)
    plan = (ctypes.c_int32 * 4)()
    _check("tav_sampler_plan_for", lib().tav_sampler_plan_for(
        B, V, int(bool(greedy)), cus, ctypes.cast(occ, ctypes.c_void_p),
        ctypes.cast(plan, ctypes.c_void_p)))
    return {"entries_per_thread": plan[0], "workgroups_per_sequence": plan[1], "groups": plan[2],
            "chunk": plan[3], "sequences_per_group": -(-B // plan[2])}


def tree_attn_workspace_bytes(B, N, Hq, Hkv, D, max_prefix_len) -> int:
    return int(lib().tree_attn_workspace_bytes(B, N, Hq, Hkv, D, max_prefix_len))


def new_attn_workspace(B, N, Hq, Hkv, D, max_prefix_len, device=None) -> torch.Tensor:
    """A zero-filled workspace for ``tree_attn_verify`` (each call leaves it zeroed)."""
    n = tree_attn_workspace_bytes(B, N, Hq, Hkv, D, max_prefix_len)
    return torch.zeros(max(1, n), dtype=torch.uint8, device=device or "cuda")


def tree_attn_verify(q, k_tree, v_tree, k_cache, v_cache, block_table, prefix_len,
                     max_prefix_len: int, mask, scale: Optional[float] = None,
                     out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     dev_flags: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Tree attention of one layer; returns out fp32 [B, N, Hq, D]."""
    _need(q, "q", _BF16)
    B, N, Hq, D = q.shape
    dev = q.device
    Hkv = k_tree.shape[2]
    _need(k_tree, "k_tree", _BF16, (B, N, Hkv, D), dev)
    _need(v_tree, "v_tree", _BF16, (B, N, Hkv, D), dev)
    nblk = k_cache.shape[0]
    _need(k_cache, "k_cache", _BF16, (nblk, Hkv, BLOCK, D), dev)
    _need(v_cache, "v_cache", _BF16, (nblk, Hkv, D, BLOCK), dev)
    _need(block_table, "block_table", _I32T, None, dev)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    _need(prefix_len, "prefix_len", _I32T, (B,), dev)
    _need(mask, "mask", _MASKT, (B, N, (N + 63) // 64), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, N, Hq, D), dtype=torch.float32, device=dev)
    _need(out, "out", (torch.float32,), (B, N, Hq, D), dev)
    need = tree_attn_workspace_bytes(B, N, Hq, Hkv, D, max_prefix_len)
    if workspace is None and need > 0:
        workspace = new_attn_workspace(B, N, Hq, Hkv, D, max_prefix_len, dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("tree_attn_verify", lib().tree_attn_verify(
        _ptr(q), _ptr(k_tree), _ptr(v_tree), _ptr(k_cache), _ptr(v_cache), nblk,
        _ptr(block_table), block_table.shape[1], _ptr(prefix_len), int(max_prefix_len),
        _ptr(mask), B, N, Hq, Hkv, D, BLOCK, float(scale), _ptr(out), _ptr(workspace), ws_bytes,
        _ptr(dev_flags), _stream(stream)))
    return out


def tree_attn_verify_tree(q, k_tree, v_tree, k_cache, v_cache, block_table, prefix_len,
                          max_prefix_len: int, parent, scale: Optional[float] = None,
                          out: Optional[torch.Tensor] = None, mask_out=None, depth_out=None,
                          workspace: Optional[torch.Tensor] = None,
                          dev_flags: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Tree attention with the mask built in the launch from parent [B, N];
    optionally also writes the mask and depths into mask_out, depth_out."""
    _need(q, "q", _BF16)
    B, N, Hq, D = q.shape
    dev = q.device
    Hkv = k_tree.shape[2]
    _need(k_tree, "k_tree", _BF16, (B, N, Hkv, D), dev)
    _need(v_tree, "v_tree", _BF16, (B, N, Hkv, D), dev)
    nblk = k_cache.shape[0]
    _need(k_cache, "k_cache", _BF16, (nblk, Hkv, BLOCK, D), dev)
    _need(v_cache, "v_cache", _BF16, (nblk, Hkv, D, BLOCK), dev)
    _need(block_table, "block_table", _I32T, None, dev)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    _need(prefix_len, "prefix_len", _I32T, (B,), dev)
    _need(parent, "parent", _I32T, (B, N), dev)
    if mask_out is not None:
        _need(mask_out, "mask_out", _MASKT, (B, N, (N + 63) // 64), dev)
    if depth_out is not None:
        _need(depth_out, "depth_out", _I32T, (B, N), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, N, Hq, D), dtype=torch.float32, device=dev)
    _need(out, "out", (torch.float32,), (B, N, Hq, D), dev)
    need = tree_attn_workspace_bytes(B, N, Hq, Hkv, D, max_prefix_len)
    if workspace is None and need > 0:
        workspace = new_attn_workspace(B, N, Hq, Hkv, D, max_prefix_len, dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("tree_attn_verify_tree", lib().tree_attn_verify_tree(
        _ptr(q), _ptr(k_tree), _ptr(v_tree), _ptr(k_cache), _ptr(v_cache), nblk,
        _ptr(block_table), block_table.shape[1], _ptr(prefix_len), int(max_prefix_len),
        _ptr(parent), _ptr(mask_out), _ptr(depth_out), B, N, Hq, Hkv, D, BLOCK, float(scale),
        _ptr(out), _ptr(workspace), ws_bytes, _ptr(dev_flags), _stream(stream)))
    return out


def spec_verify_workspace_bytes(B, N, V) -> int:
    return int(lib().spec_verify_workspace_bytes(B, N, V))


def new_sampler_workspace(B, N, V, device=None) -> torch.Tensor:
    """A zero-filled workspace for ``spec_verify_sample`` (each call leaves it zeroed)."""
    n = spec_verify_workspace_bytes(B, N, V)
    if n == 0:
        raise ValueError(f"spec_verify_sample does not support B={B}, N={N}, V={V}")
    return torch.zeros(n, dtype=torch.uint8, device=device or "cuda")


def _verify_sample(name, target_logits, draft_logits, parent, token, temperature, seed, offset,
                   path, n_accepted, out_tokens, workspace, dev_flags, stream):
    _need(target_logits, "target_logits", (torch.float32,))
    B, N, V = target_logits.shape
    dev = target_logits.device
    if draft_logits is not None or temperature != 0:
        _need(draft_logits, "draft_logits", (torch.float32,), (B, N, V), dev)
    _need(parent, "parent", _I32T, (B, N), dev)
    _need(token, "token", _I32T, (B, N), dev)
    if path is None:
        path = torch.empty((B, N), dtype=torch.int32, device=dev)
    if n_accepted is None:
        n_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    _need(path, "path", _I32T, (B, N), dev)
    _need(n_accepted, "n_accepted", _I32T, (B,), dev)
    _need(out_tokens, "out_tokens", _I32T, (B, N), dev)
    if workspace is None:
        workspace = new_sampler_workspace(B, N, V, dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(name, getattr(lib(), name)(
        _ptr(target_logits), _ptr(draft_logits), _ptr(parent), _ptr(token), B, N, V,
        float(temperature), int(seed), int(offset), _ptr(path), _ptr(n_accepted),
        _ptr(out_tokens), _ptr(workspace), ws_bytes, _ptr(dev_flags), _stream(stream)))
    return path, n_accepted, out_tokens


def spec_verify_sample(target_logits, draft_logits, parent, token, temperature: float = 1.0,
                       seed: int = 0, offset: int = 0, path=None, n_accepted=None,
                       out_tokens=None, workspace=None, dev_flags=None, stream=None):
    """Rejection-sampling walk with siblings tested against q_u each time
    (drawn i.i.d.), or greedy verification at temperature 0 (then
    draft_logits may be None); returns (path [B,N], n_accepted [B], out_tokens [B,N])."""
    return _verify_sample("spec_verify_sample", target_logits, draft_logits, parent, token,
                          temperature, seed, offset, path, n_accepted, out_tokens, workspace,
                          dev_flags, stream)


def spec_verify_sample_probe(target_logits, draft_logits, parent, token,
                             temperature: float = 1.0, seed: int = 0, offset: int = 0,
                             workspace=None, dev_flags=None, stream=None):
    """``spec_verify_sample`` that also returns the softmax values the walk
    decides with: (path, n_accepted, out_tokens, p_rows [B,N,V] fp64,
    q_rows [B,N,V] fp64, child_pq [B,N,2] fp64). Rows of nodes the walk does
    not visit (and q rows of visited leaves) are NaN."""
    _need(target_logits, "target_logits", (torch.float32,))
    B, N, V = target_logits.shape
    dev = target_logits.device
    _need(draft_logits, "draft_logits", (torch.float32,), (B, N, V), dev)
    _need(parent, "parent", _I32T, (B, N), dev)
    _need(token, "token", _I32T, (B, N), dev)
    path = torch.empty((B, N), dtype=torch.int32, device=dev)
    n_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    out_tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    p_rows = torch.full((B, N, V), float("nan"), dtype=torch.float64, device=dev)
    q_rows = torch.full((B, N, V), float("nan"), dtype=torch.float64, device=dev)
    child_pq = torch.full((B, N, 2), float("nan"), dtype=torch.float64, device=dev)
    if workspace is None:
        workspace = new_sampler_workspace(B, N, V, dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("spec_verify_sample_probe", lib().spec_verify_sample_probe(
        _ptr(target_logits), _ptr(draft_logits), _ptr(parent), _ptr(token), B, N, V,
        float(temperature), int(seed), int(offset), _ptr(path), _ptr(n_accepted),
        _ptr(out_tokens), _ptr(p_rows), _ptr(q_rows), _ptr(child_pq), _ptr(workspace), ws_bytes,
        _ptr(dev_flags), _stream(stream)))
    return path, n_accepted, out_tokens, p_rows, q_rows, child_pq


def spec_verify_sample_noalloc(target_logits, draft_logits, parent, token,
                               temperature: float = 1.0, seed: int = 0, offset: int = 0,
                               path=None, n_accepted=None, out_tokens=None, dev_flags=None,
                               stream=None):
    """``spec_verify_sample`` on the library's fixed per-device scratch: no
    workspace argument and no allocation inside the call (pass preallocated
    outputs to allocate nothing at all). Calls on one device must not overlap
    in time."""
    _need(target_logits, "target_logits", (torch.float32,))
    B, N, V = target_logits.shape
    dev = target_logits.device
    if draft_logits is not None or temperature != 0:
        _need(draft_logits, "draft_logits", (torch.float32,), (B, N, V), dev)
    _need(parent, "parent", _I32T, (B, N), dev)
    _need(token, "token", _I32T, (B, N), dev)
    if path is None:
        path = torch.empty((B, N), dtype=torch.int32, device=dev)
    if n_accepted is None:
        n_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    _need(path, "path", _I32T, (B, N), dev)
    _need(n_accepted, "n_accepted", _I32T, (B,), dev)
    _need(out_tokens, "out_tokens", _I32T, (B, N), dev)
    _check("spec_verify_sample_noalloc", lib().spec_verify_sample_noalloc(
        _ptr(target_logits), _ptr(draft_logits), _ptr(parent), _ptr(token), B, N, V,
        float(temperature), int(seed), int(offset), _ptr(path), _ptr(n_accepted),
        _ptr(out_tokens), _ptr(dev_flags), _stream(stream)))
    return path, n_accepted, out_tokens


def spec_verify_sample_wor(target_logits, draft_logits, parent, token,
                           temperature: float = 1.0, seed: int = 0, offset: int = 0, path=None,
                           n_accepted=None, out_tokens=None, workspace=None, dev_flags=None,
                           stream=None):
    """As ``spec_verify_sample`` for siblings drawn from q_u without
    replacement: a rejected sibling's token leaves q_u (the rest
    renormalised) before the next sibling is tried."""
    return _verify_sample("spec_verify_sample_wor", target_logits, draft_logits, parent, token,
                          temperature, seed, offset, path, n_accepted, out_tokens, workspace,
                          dev_flags, stream)


def kv_commit_path(k_tree, v_tree, path, n_accepted, block_table, prefix_len, k_cache, v_cache,
                   commit_slots=None, new_prefix_len=None, dev_flags=None, stream=None):
    """Commit the accepted path in place; returns (commit_slots [B,N], new_prefix_len [B])."""
    _need(k_tree, "k_tree", _BF16)
    B, N, Hkv, D = k_tree.shape
    dev = k_tree.device
    _need(v_tree, "v_tree", _BF16, (B, N, Hkv, D), dev)
    _need(path, "path", _I32T, (B, N), dev)
    _need(n_accepted, "n_accepted", _I32T, (B,), dev)
    _need(block_table, "block_table", _I32T, None, dev)
    _need(prefix_len, "prefix_len", _I32T, (B,), dev)
    nblk = k_cache.shape[0]
    _need(k_cache, "k_cache", _BF16, (nblk, Hkv, BLOCK, D), dev)
    _need(v_cache, "v_cache", _BF16, (nblk, Hkv, D, BLOCK), dev)
    if commit_slots is None:
        commit_slots = torch.empty((B, N), dtype=torch.int32, device=dev)
    if new_prefix_len is None:
        new_prefix_len = torch.empty((B,), dtype=torch.int32, device=dev)
    _check("kv_commit_path", lib().kv_commit_path(
        _ptr(k_tree), _ptr(v_tree), _ptr(path), _ptr(n_accepted), nblk, _ptr(block_table),
        block_table.shape[1], _ptr(prefix_len), _ptr(k_cache), _ptr(v_cache), B, N, Hkv, D,
        BLOCK, _ptr(commit_slots), _ptr(new_prefix_len), _ptr(dev_flags), _stream(stream)))
    return commit_slots, new_prefix_len


def spec_verify_sample_commit(target_logits, draft_logits, parent, token, k_tree, v_tree,
                              block_table, prefix_len, k_cache, v_cache,
                              temperature: float = 1.0, seed: int = 0, offset: int = 0,
                              without_replacement: bool = False, path=None, n_accepted=None,
                              out_tokens=None, commit_slots=None, new_prefix_len=None,
                              workspace=None, dev_flags=None, stream=None):
    """The walk and the KV commit of its accepted paths in one launch; returns
    (path, n_accepted, out_tokens, commit_slots, new_prefix_len), the outputs
    of spec_verify_sample (or its without-replacement form) followed by
    kv_commit_path."""
    _need(target_logits, "target_logits", (torch.float32,))
    B, N, V = target_logits.shape
    dev = target_logits.device
    if draft_logits is not None or temperature != 0:
        _need(draft_logits, "draft_logits", (torch.float32,), (B, N, V), dev)
    _need(parent, "parent", _I32T, (B, N), dev)
    _need(token, "token", _I32T, (B, N), dev)
    _need(k_tree, "k_tree", _BF16)
    _, _, Hkv, D = k_tree.shape
    _need(k_tree, "k_tree", _BF16, (B, N, Hkv, D), dev)
    _need(v_tree, "v_tree", _BF16, (B, N, Hkv, D), dev)
    _need(block_table, "block_table", _I32T, None, dev)
    _need(prefix_len, "prefix_len", _I32T, (B,), dev)
    nblk = k_cache.shape[0]
    _need(k_cache, "k_cache", _BF16, (nblk, Hkv, BLOCK, D), dev)
    _need(v_cache, "v_cache", _BF16, (nblk, Hkv, D, BLOCK), dev)
    outs = []
    for t, shape in ((path, (B, N)), (n_accepted, (B,)), (out_tokens, (B, N)),
                     (commit_slots, (B, N)), (new_prefix_len, (B,))):
        if t is None:
            t = torch.empty(shape, dtype=torch.int32, device=dev)
        _need(t, "output", _I32T, shape, dev)
        outs.append(t)
    if workspace is None:
        workspace = new_sampler_workspace(B, N, V, dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("spec_verify_sample_commit", lib().spec_verify_sample_commit(
        _ptr(target_logits), _ptr(draft_logits), _ptr(parent), _ptr(token), B, N, V,
        float(temperature), int(seed), int(offset), int(bool(without_replacement)),
        _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]), _ptr(k_tree), _ptr(v_tree), nblk,
        _ptr(block_table), block_table.shape[1], _ptr(prefix_len), _ptr(k_cache), _ptr(v_cache),
        Hkv, D, BLOCK, _ptr(outs[3]), _ptr(outs[4]), _ptr(workspace), ws_bytes,
        _ptr(dev_flags), _stream(stream)))
    return tuple(outs)


def kv_commit_inplace(path, n_accepted, block_table, prefix_len, k_cache, v_cache,
                      commit_slots=None, new_prefix_len=None, dev_flags=None, stream=None):
    """Zero-copy rollback (the tree's rows already at positions L..L+N-1 of
    the cache); returns (commit_slots [B,N], new_prefix_len [B])."""
    _need(path, "path", _I32T)
    B, N = path.shape
    dev = path.device
    _need(n_accepted, "n_accepted", _I32T, (B,), dev)
    _need(block_table, "block_table", _I32T, None, dev)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    _need(prefix_len, "prefix_len", _I32T, (B,), dev)
    _need(k_cache, "k_cache", _BF16, None, dev)
    nblk, Hkv, _, D = k_cache.shape
    _need(k_cache, "k_cache", _BF16, (nblk, Hkv, BLOCK, D), dev)
    _need(v_cache, "v_cache", _BF16, (nblk, Hkv, D, BLOCK), dev)
    if commit_slots is None:
        commit_slots = torch.empty((B, N), dtype=torch.int32, device=dev)
    if new_prefix_len is None:
        new_prefix_len = torch.empty((B,), dtype=torch.int32, device=dev)
    _check("kv_commit_inplace", lib().kv_commit_inplace(
        _ptr(path), _ptr(n_accepted), nblk, _ptr(block_table), block_table.shape[1],
        _ptr(prefix_len), _ptr(k_cache), _ptr(v_cache), B, N, Hkv, D, BLOCK,
        _ptr(commit_slots), _ptr(new_prefix_len), _ptr(dev_flags), _stream(stream)))
    return commit_slots, new_prefix_len


def tree_expand_workspace_bytes(R: int, V: int, k: int) -> int:
    return int(lib().tree_expand_workspace_bytes(R, V, k))


def tree_expand_topk(draft_logits, k: int, temperature: float = 1.0, top_token=None,
                     top_logq=None, entropy=None, workspace=None, dev_flags=None, stream=None):
    """Top-k draft tokens, their log q and the entropy of every row of
    draft_logits fp32 [R, V]; returns (top_token int32 [R, k], top_logq
    float64 [R, k], entropy float64 [R])."""
    return _expand(draft_logits, k, temperature, top_token, top_logq, entropy, workspace,
                   dev_flags, stream, None)


def _expand(draft_logits, k, temperature, top_token, top_logq, entropy, workspace, dev_flags,
            stream, sample):
    _need(draft_logits, "draft_logits", (torch.float32,))
    if draft_logits.dim() != 2:
        raise ValueError("draft_logits must be [R, V]")
    R, V = draft_logits.shape
    dev = draft_logits.device
    if top_token is None:
        top_token = torch.empty((R, k), dtype=torch.int32, device=dev)
    if top_logq is None:
        top_logq = torch.empty((R, k), dtype=torch.float64, device=dev)
    if entropy is None:
        entropy = torch.empty((R,), dtype=torch.float64, device=dev)
    _need(top_token, "top_token", _I32T, (R, k), dev)
    _need(top_logq, "top_logq", (torch.float64,), (R, k), dev)
    _need(entropy, "entropy", (torch.float64,), (R,), dev)
    if workspace is None:
        n = tree_expand_workspace_bytes(R, V, k)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    if sample is None:
        _check("tree_expand_topk", lib().tree_expand_topk(
            _ptr(draft_logits), R, V, int(k), float(temperature), _ptr(top_token),
            _ptr(top_logq), _ptr(entropy), _ptr(workspace), ws_bytes, _ptr(dev_flags),
            _stream(stream)))
    else:
        seed, offset = sample
        _check("tree_expand_sample", lib().tree_expand_sample(
            _ptr(draft_logits), R, V, int(k), float(temperature), int(seed), int(offset),
            _ptr(top_token), _ptr(top_logq), _ptr(entropy), _ptr(workspace), ws_bytes,
            _ptr(dev_flags), _stream(stream)))
    return top_token, top_logq, entropy


def tree_expand_sample(draft_logits, k: int, temperature: float = 1.0, seed: int = 0,
                       offset: int = 0, top_token=None, top_logq=None, entropy=None,
                       workspace=None, dev_flags=None, stream=None):
    """As ``tree_expand_topk`` with the k tokens of each row drawn from q
    without replacement (Gumbel top-k on Philox draws of (seed, offset))."""
    return _expand(draft_logits, k, temperature, top_token, top_logq, entropy, workspace,
                   dev_flags, stream, (seed, offset))


def philox_uniforms(seed: int, offset: int, B: int, N: int, out=None, device=None, stream=None):
    """fp32 [B, N, 2]: (acceptance, resampling) uniform of every node."""
    if out is None:
        out = torch.empty((B, N, 2), dtype=torch.float32, device=device or "cuda")
    _need(out, "out", (torch.float32,), (B, N, 2))
    _check("tav_philox_uniforms", lib().tav_philox_uniforms(int(seed), int(offset), B, N,
                                                            _ptr(out), _stream(stream)))
    return out


def target_probs(logits: torch.Tensor, temperature: float = 1.0, out=None, dev_flags=None,
                 stream=None) -> torch.Tensor:
    """fp64 softmax(logits / T) over the last axis, with the sampler's device softmax."""
    _need(logits, "logits", (torch.float32,))
    V = logits.shape[-1]
    rows = logits.numel() // V
    if out is None:
        out = torch.empty(logits.shape, dtype=torch.float64, device=logits.device)
    _need(out, "out", (torch.float64,), tuple(logits.shape), logits.device)
    _check("tav_target_probs", lib().tav_target_probs(_ptr(logits), rows, V, float(temperature),
                                                      _ptr(out), _ptr(dev_flags),
                                                      _stream(stream)))
    return out


def tree_select_topm(parent, token, logq, M: int, out_parent=None, out_token=None, out_src=None,
                     dev_flags=None, stream=None):
    """Keep the M best nodes of each candidate tree by cumulative log q;
    returns (out_parent [B,M], out_token [B,M], out_src [B,M])."""
    _need(parent, "parent", _I32T)
    B, Nc = parent.shape
    dev = parent.device
    _need(token, "token", _I32T, (B, Nc), dev)
    _need(logq, "logq", (torch.float64,), (B, Nc), dev)
    if out_parent is None:
        out_parent = torch.empty((B, M), dtype=torch.int32, device=dev)
    if out_token is None:
        out_token = torch.empty((B, M), dtype=torch.int32, device=dev)
    if out_src is None:
        out_src = torch.empty((B, M), dtype=torch.int32, device=dev)
    for t, n in ((out_parent, "out_parent"), (out_token, "out_token"), (out_src, "out_src")):
        _need(t, n, _I32T, (B, M), dev)
    _check("tree_select_topm", lib().tree_select_topm(
        _ptr(parent), _ptr(token), _ptr(logq), B, Nc, int(M), _ptr(out_parent), _ptr(out_token),
        _ptr(out_src), _ptr(dev_flags), _stream(stream)))
    return out_parent, out_token, out_src


def tree_widths_by_entropy(entropy, w_min: int, w_max: int, width=None, dev_flags=None,
                           stream=None):
    """Branching widths from the entropy rank of each frontier node;
    entropy fp64 [B, F] -> width int32 [B, F]."""
    _need(entropy, "entropy", (torch.float64,))
    B, F = entropy.shape
    dev = entropy.device
    if width is None:
        width = torch.empty((B, F), dtype=torch.int32, device=dev)
    _need(width, "width", _I32T, (B, F), dev)
    _check("tree_widths_by_entropy", lib().tree_widths_by_entropy(
        _ptr(entropy), B, F, int(w_min), int(w_max), _ptr(width), _ptr(dev_flags),
        _stream(stream)))
    return width


def tree_topology_dp(p_rank, n: int, depth: int, device=None, stream=None):
    """The n-node topology of largest expected accepted count under
    acceptance by sibling rank (p_rank: K floats, host). Returns (parent
    int32 [n], rank int32 [n], value fp64 [1]) on the device."""
    K = len(p_rank)
    dev = device or torch.device("cuda")
    p = (ctypes.c_double * K)(*[float(x) for x in p_rank])
    parent = torch.empty((n,), dtype=torch.int32, device=dev)
    rank = torch.empty((n,), dtype=torch.int32, device=dev)
    value = torch.empty((1,), dtype=torch.float64, device=dev)
    need = int(lib().tree_topology_workspace_bytes(K, n, depth))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check("tree_topology_dp", lib().tree_topology_dp(
        ctypes.cast(p, ctypes.c_void_p), K, n, depth, _ptr(parent), _ptr(rank), _ptr(value),
        _ptr(ws), need, _stream(stream)))
    return parent, rank, value


def verify_speedup(expected_emitted, draft_ratio, layers, layer_params, head_params, batch, n,
                   attn_verify_us, sampler_verify_us, attn_decode_us, sampler_decode_us,
                   hbm_gbs, mfma_tflops):
    """tav_verify_speedup (host): (speedup, alpha, T_decode us, T_verify us)."""
    out = (ctypes.c_double * 3)()
    s = lib().tav_verify_speedup(float(expected_emitted), float(draft_ratio), int(layers),
                                 float(layer_params), float(head_params), int(batch), int(n),
                                 float(attn_verify_us), float(sampler_verify_us),
                                 float(attn_decode_us), float(sampler_decode_us), float(hbm_gbs),
                                 float(mfma_tflops), ctypes.cast(out, ctypes.c_void_p))
    return float(s), out[0], out[1], out[2]


def model_speedup(expected_emitted: float, draft_ratio: float, alpha: float, n: int) -> float:
    """E[emitted] / (T_draft/T_decode + 1 + alpha * N) (NaN on bad input)."""
    return float(lib().tav_model_speedup(float(expected_emitted), float(draft_ratio),
                                         float(alpha), int(n)))


def best_chain_length(p: float, draft_ratio: float, alpha: float, n_max: int):
    """(N, speedup) of the best chain length under the model; N = 0 on bad input."""
    s = ctypes.c_double(float("nan"))
    n = int(lib().tav_best_chain_length(float(p), float(draft_ratio), float(alpha), int(n_max),
                                        ctypes.byref(s)))
    return n, s.value


def fit_alpha(n_values, t_us) -> float:
    """Per-position verification overhead from times t_us measured at tree
    sizes n_values (the first must be 1)."""
    n = (ctypes.c_int32 * len(n_values))(*[int(x) for x in n_values])
    t = (ctypes.c_double * len(t_us))(*[float(x) for x in t_us])
    return float(lib().tav_fit_alpha(n, t, len(n_values)))
