"""spec_verify_sample_noalloc (the sampler with the library's fixed scratch
instead of a workspace) against spec_verify_sample on the same inputs:
bit-exact paths, accepted counts and tokens, on calls in a row whose sizes
shrink, so the second call runs on scratch the first one used."""

import ctypes

import numpy as np
import pytest
import torch

import tree_attention_verification_ancestor_amd as tav
from gpu_helpers import device, say
from synth import make_workload
from synth.device import to_numpy, upload

pytestmark = pytest.mark.gpu

_P, _I32, _U64, _F64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_double


def _noalloc(d, B, N, V, T, seed, offset, flags):
    fn = tav.lib().spec_verify_sample_noalloc
    fn.restype = _I32
    fn.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32, _F64, _U64, _U64, _P, _P, _P, _P, _P]
    dev = d["target_logits"].device
    path = torch.full((B, N), -7, dtype=torch.int32, device=dev)
    n_acc = torch.full((B,), -7, dtype=torch.int32, device=dev)
    toks = torch.full((B, N), -7, dtype=torch.int32, device=dev)
    dl = d["draft_logits"]
    st = fn(d["target_logits"].data_ptr(), None if dl is None else dl.data_ptr(),
            d["parent"].data_ptr(), d["token"].data_ptr(), B, N, V, T, seed, offset,
            path.data_ptr(), n_acc.data_ptr(), toks.data_ptr(), flags.data_ptr(),
            torch.cuda.current_stream().cuda_stream)
    assert st == tav.OK, tav.status_string(st)
    return path, n_acc, toks


def _check(w, T, seed, offset):
    dev = device()
    d = upload(w, dev)
    flags = tav.new_flags(dev)
    B, N, V = w.B, w.N, w.V
    got = _noalloc(d, B, N, V, T, seed, offset, flags)
    ref = tav.spec_verify_sample(d["target_logits"], d["draft_logits"], d["parent"], d["token"],
                                 T, seed, offset, dev_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    for g, r in zip(got, ref):
        np.testing.assert_array_equal(to_numpy(g), to_numpy(r))
    return to_numpy(got[1])


def test_noalloc_matches_workspace_call_on_shrinking_inputs():
    say("noalloc: llama70b (B=8, N=64, V=128256), then a smaller batch")
    acc = _check(make_workload("llama70b"), 1.0, 0, 0)
    say(f"  accepted {acc.tolist()}")
    acc = _check(make_workload("tiny", N=40, B=5, V=5000, tree="random", seed=5), 0.8, 3, 9)
    say(f"  second call, smaller: accepted {acc.tolist()}")
    # greedy (temperature 0) through the same scratch, smaller still
    acc = _check(make_workload("tiny", N=12, B=3, V=3000, tree="random", seed=6), 0.0, 0, 0)
    say(f"  greedy: accepted {acc.tolist()}")


def test_noalloc_repeated_calls_leave_scratch_reusable():
    say("noalloc: 20 calls in a row on one stream, offsets 0..19")
    w = make_workload("tiny", N=64, B=16, V=20000, tree="random", seed=8)
    for off in range(20):
        _check(w, 1.0, 11, off)
