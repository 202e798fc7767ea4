"""Softmax, Philox uniforms and the rejection-sampling walk (float64).

The walk and Philox live in plain C (``csrc/walk.c``) so that statistical pins
can run a million trials in seconds; this module loads that library and adds
the softmax definition used by tests.

Sources on the pages (restated, see ``csrc/walk.c`` for the full list):
  * radar-34b blog, section 2: acceptance with probability min(1, p/q), and
    redraw from the normalised positive part of p - q on rejection;
  * LLM Primer VI ch. 9, section 9.1: N+1 target distributions per pass, so a
    fully accepted path emits a bonus token;
  * jisaku.com glossary, SpecInfer paragraph: root-down, depth-first decisions.
"""

from __future__ import annotations

import ctypes
import dataclasses
import os

import numpy as np

from . import build as _build

NEAR_EPS = 1e-6

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        P = ctypes.c_void_p
        lib.oracle_verify_walk.restype = ctypes.c_int
        lib.oracle_verify_walk.argtypes = [P, P, P, P, ctypes.c_int64, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_double, ctypes.c_uint64,
                                           ctypes.c_uint64, ctypes.c_double, ctypes.c_int32,
                                           P, P, P, P, P, P, P, P]
        lib.oracle_verify_walk_u.restype = ctypes.c_int
        lib.oracle_verify_walk_u.argtypes = [P, P, P, P, ctypes.c_int64, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_double, ctypes.c_uint64,
                                             ctypes.c_uint64, ctypes.c_double, ctypes.c_int32,
                                             P, P, P, P, P, P, P, P, P]
        lib.oracle_uniform_table.restype = None
        lib.oracle_uniform_table.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                             ctypes.c_int32, P]
        lib.oracle_philox_words.restype = None
        lib.oracle_philox_words.argtypes = [P, ctypes.c_int64, ctypes.c_uint64,
                                            ctypes.c_uint64, P]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def softmax(logits: np.ndarray, temperature: float = 1.0) -> np.ndarray:
    """p = softmax(logits / T) along the last axis, float64 (max-subtracted).

    radar-34b blog section 2 names the target and draft distributions p and q;
    this is how both are formed from logits."""
    z = np.asarray(logits, dtype=np.float64) / float(temperature)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def philox4x64_10(counters: np.ndarray, key=(0, 0)) -> np.ndarray:
    """Philox4x64-10 output words for uint64 counters [n, 4] under ``key``."""
    ctr = np.ascontiguousarray(counters, dtype=np.uint64).reshape(-1, 4)
    out = np.empty_like(ctr)
    _load().oracle_philox_words(_ptr(ctr), ctr.shape[0], int(key[0]), int(key[1]), _ptr(out))
    return out


def node_uniforms(seed: int, offset: int, B: int, N: int) -> np.ndarray:
    """float64 [B, N, 2]: (acceptance uniform, resampling uniform) per node."""
    u = np.empty((B, N, 2), dtype=np.float64)
    _load().oracle_uniform_table(int(seed), int(offset), int(B), int(N), _ptr(u))
    return u


@dataclasses.dataclass
class WalkResult:
    path: np.ndarray         # int32 [B, N], accepted nodes from the root, -1 padded
    n_accepted: np.ndarray   # int32 [B]
    out_tokens: np.ndarray   # int32 [B, N], emitted tokens (n_accepted + 1), -1 padded
    draws: np.ndarray        # int32 [B], uniforms that decided something
    near: np.ndarray         # int32 [B], draws within NEAR_EPS of their boundary
    first_near: np.ndarray   # int32 [B], accepted count at the first near draw, or -1
    min_margin: np.ndarray   # float64 [B]


_ERRORS = {1: "bad parent array", 2: "token out of range", 3: "non-finite logits",
           4: "bad argument", 5: "out of memory"}


def verify_walk(target_logits, draft_logits, parent, token, temperature: float = 1.0,
                seed: int = 0, offset: int = 0, near_eps: float = NEAR_EPS,
                without_replacement: bool = False, uniforms=None) -> WalkResult:
    """Root-down rejection-sampling walk for a batch of trees.

    target_logits, draft_logits: float32 [B, N, V]; row u of the draft is the
    distribution node u's children were drawn from. parent, token: int [B, N].

    Sibling rule: by default every child of u is tested with q_u, which is
    lossless when siblings are independent draws from q_u. With
    ``without_replacement`` a rejected child's token then leaves q_u (its
    entry zeroed, the rest renormalised by their sum) before the next sibling
    is tried, which is lossless when siblings are drawn from q_u without
    replacement. The rejection step itself (radar-34b blog section 2) is the
    same under both: the residual is the normalised positive part of the
    current p minus the current q.
    uniforms: None (Philox from seed and offset, the default) or float64
    [B, N, 2], node i's (acceptance, resampling) uniforms, for tests that
    integrate over them.
    Raises ValueError on an invalid tree, token or logit row.
    """
    tl = np.ascontiguousarray(target_logits, dtype=np.float32)
    dl = np.ascontiguousarray(draft_logits, dtype=np.float32)
    par = np.ascontiguousarray(parent, dtype=np.int32)
    tok = np.ascontiguousarray(token, dtype=np.int32)
    B, N, V = tl.shape
    if dl.shape != tl.shape or par.shape != (B, N) or tok.shape != (B, N):
        raise ValueError("shape mismatch")
    path = np.empty((B, N), np.int32)
    n_acc = np.empty(B, np.int32)
    out_tok = np.empty((B, N), np.int32)
    draws = np.zeros(B, np.int32)
    near = np.zeros(B, np.int32)
    first_near = np.full(B, -1, np.int32)
    min_margin = np.full(B, np.inf)
    bad = np.zeros(1, np.int64)
    utab = None
    if uniforms is not None:
        utab = np.ascontiguousarray(uniforms, dtype=np.float64)
        if utab.shape != (B, N, 2):
            raise ValueError("uniforms must be [B, N, 2]")
    rc = _load().oracle_verify_walk_u(_ptr(tl), _ptr(dl), _ptr(par), _ptr(tok), B, N, V,
                                      float(temperature), int(seed), int(offset),
                                      float(near_eps), 1 if without_replacement else 0,
                                      None if utab is None else _ptr(utab), _ptr(path),
                                      _ptr(n_acc), _ptr(out_tok), _ptr(draws), _ptr(near),
                                      _ptr(first_near), _ptr(min_margin), _ptr(bad))
    if rc:
        raise ValueError(f"oracle walk: {_ERRORS.get(rc, rc)} (sequence {int(bad[0])})")
    return WalkResult(path, n_acc, out_tok, draws, near, first_near, min_margin)


def verify_greedy(target_logits, parent, token) -> WalkResult:
    """Greedy (temperature 0) verification of a batch of trees.

    LLM Primer VI ch. 9, section 9.1: the longest prefix of candidates that
    matches the target's own choice is accepted, and at the first mismatch
    the engine commits to the target's choice. Read on a tree, root-down
    (jisaku.com glossary, SpecInfer paragraph): at node u the target's choice
    is the argmax of target row u (the lowest token id among equal maxima);
    the first child of u, in ascending node index, whose token is that choice
    is accepted and the walk moves there; if none is, the choice is emitted
    and the walk stops. At a leaf the choice is the bonus token. Every step
    emits accepted + 1 tokens; no uniform is drawn.

    target_logits float32 [B, N, V]; parent, token int [B, N]. Raises
    ValueError on an invalid tree or token, or on a visited row whose
    maximum is not finite or that holds a NaN.
    """
    tl = np.asarray(target_logits, dtype=np.float32)
    par = np.asarray(parent)
    tok = np.asarray(token)
    B, N, V = tl.shape
    path = np.full((B, N), -1, np.int32)
    n_acc = np.zeros(B, np.int32)
    out_tok = np.full((B, N), -1, np.int32)
    for b in range(B):
        if par[b, 0] != -1 or any(not (0 <= par[b, i] < i) for i in range(1, N)):
            raise ValueError(f"oracle greedy: bad parent array (sequence {b})")
        if any(not (0 <= tok[b, i] < V) for i in range(1, N)):
            raise ValueError(f"oracle greedy: token out of range (sequence {b})")
        u, m = 0, 0
        path[b, 0] = 0
        while True:
            row = tl[b, u]
            if np.isnan(row).any() or not np.isfinite(row.max()):
                raise ValueError(f"oracle greedy: non-finite logits (sequence {b})")
            x = int(np.argmax(row))            # first index of the maximum
            out_tok[b, m] = x
            hit = next((c for c in range(1, N) if par[b, c] == u and tok[b, c] == x), None)
            if hit is None:
                break
            m += 1
            path[b, m] = hit
            u = hit
        n_acc[b] = m
    zeros = np.zeros(B, np.int32)
    return WalkResult(path, n_acc, out_tok, zeros, zeros.copy(), np.full(B, -1, np.int32),
                      np.full(B, np.inf))
