"""The C-ABI library loads and exports every declared entry point, and its
host-side argument checks reject bad calls before touching the GPU (CPU only).
"""

import ctypes

import pytest

import tree_attention_verification_ancestor_amd as tav


def test_library_exports_every_declared_function():
    names = tav.header_functions()
    assert set(names) >= {"tree_mask_build", "tree_attn_verify", "spec_verify_sample",
                          "spec_verify_sample_wor", "kv_commit_path", "tree_attn_workspace_bytes",
                          "spec_verify_workspace_bytes", "tav_philox_uniforms",
                          "tav_target_probs", "tav_status_string", "tav_abi_version"}
    lib = tav.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(tav._SIGNATURES)


def test_abi_version_and_status_strings():
    assert tav.abi_version() == 1
    for code in range(5):
        assert tav.status_string(code)
    assert "unknown" in tav.status_string(99)


P = ctypes.c_void_p
FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: every case fails its checks first


def test_mask_build_rejects_bad_arguments():
    lib = tav.lib()
    assert lib.tree_mask_build(None, 1, 5, FAKE, None, None, None) == tav.ERR_ARG
    assert lib.tree_mask_build(FAKE, 0, 5, FAKE, None, None, None) == tav.ERR_ARG
    assert lib.tree_mask_build(FAKE, 1, 0, FAKE, None, None, None) == tav.ERR_ARG
    assert lib.tree_mask_build(FAKE, 1, 257, FAKE, None, None, None) == tav.ERR_UNSUPPORTED
    assert lib.tree_mask_build(FAKE, 1, 5, ctypes.c_void_p(0x10004), None, None, None) == tav.ERR_ARG


def _attn(**kw):
    args = dict(q=FAKE, k_tree=FAKE, v_tree=FAKE, k_cache=FAKE, v_cache=FAKE, num_blocks=10,
                block_table=FAKE, max_blocks=4, prefix_len=FAKE, max_prefix_len=64, mask=FAKE,
                B=1, N=5, Hq=8, Hkv=2, D=128, block_size=16, scale=0.088, out=FAKE,
                workspace=None, ws_bytes=0, dev_flags=None, stream=None)
    args.update(kw)
    return tav.lib().tree_attn_verify(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), tav.ERR_ARG), (dict(out=None), tav.ERR_ARG), (dict(B=0), tav.ERR_ARG),
    (dict(N=0), tav.ERR_ARG), (dict(scale=0.0), tav.ERR_ARG), (dict(scale=float("nan")), tav.ERR_ARG),
    (dict(max_prefix_len=-1), tav.ERR_ARG), (dict(num_blocks=0), tav.ERR_ARG),
    (dict(D=96), tav.ERR_UNSUPPORTED), (dict(Hq=7), tav.ERR_UNSUPPORTED),
    (dict(block_size=32), tav.ERR_UNSUPPORTED), (dict(N=300), tav.ERR_UNSUPPORTED),
    (dict(N=256, Hq=64, Hkv=2), tav.ERR_UNSUPPORTED),
    (dict(num_blocks=(1 << 31) - 1, Hq=8, Hkv=4), tav.ERR_UNSUPPORTED),
    (dict(q=ctypes.c_void_p(0x10008)), tav.ERR_ARG),
])
def test_attention_rejects_bad_arguments(kw, code):
    assert _attn(**kw) == code


def _sample(fn="spec_verify_sample", **kw):
    args = dict(tl=FAKE, dl=FAKE, parent=FAKE, token=FAKE, B=2, N=5, V=1000, T=1.0, seed=0,
                offset=0, path=FAKE, n_acc=FAKE, out_tok=FAKE, ws=FAKE, ws_bytes=1 << 20,
                flags=None, stream=None)
    args.update(kw)
    return getattr(tav.lib(), fn)(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(tl=None), tav.ERR_ARG), (dict(path=None), tav.ERR_ARG), (dict(B=0), tav.ERR_ARG),
    (dict(V=0), tav.ERR_ARG), (dict(T=float("nan")), tav.ERR_ARG), (dict(T=-1.0), tav.ERR_ARG),
    (dict(T=float("inf")), tav.ERR_ARG), (dict(N=257), tav.ERR_UNSUPPORTED),
    # the draft rows are required unless the temperature is 0 (greedy)
    (dict(dl=None), tav.ERR_ARG), (dict(dl=None, T=0.0, tl=None), tav.ERR_ARG),
    (dict(V=(1 << 21) + 1), tav.ERR_UNSUPPORTED),
])
@pytest.mark.parametrize("fn", ["spec_verify_sample", "spec_verify_sample_wor"])
def test_sampler_rejects_bad_arguments(fn, kw, code):
    assert _sample(fn, **kw) == code


def _attn_tree(**kw):
    args = dict(q=FAKE, k_tree=FAKE, v_tree=FAKE, k_cache=FAKE, v_cache=FAKE, num_blocks=10,
                block_table=FAKE, max_blocks=4, prefix_len=FAKE, max_prefix_len=64, parent=FAKE,
                mask_out=None, depth_out=None, B=1, N=5, Hq=8, Hkv=2, D=128, block_size=16,
                scale=0.088, out=FAKE, workspace=None, ws_bytes=0, dev_flags=None, stream=None)
    args.update(kw)
    return tav.lib().tree_attn_verify_tree(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(parent=None), tav.ERR_ARG), (dict(q=None), tav.ERR_ARG), (dict(B=0), tav.ERR_ARG),
    (dict(scale=0.0), tav.ERR_ARG), (dict(D=96), tav.ERR_UNSUPPORTED),
    (dict(N=300), tav.ERR_UNSUPPORTED), (dict(parent=ctypes.c_void_p(0x10002)), tav.ERR_ARG),
    (dict(mask_out=ctypes.c_void_p(0x10004)), tav.ERR_ARG),
    (dict(depth_out=ctypes.c_void_p(0x10002)), tav.ERR_ARG),
])
def test_attention_from_parents_rejects_bad_arguments(kw, code):
    assert _attn_tree(**kw) == code


def _sample_commit(**kw):
    args = dict(tl=FAKE, dl=FAKE, parent=FAKE, token=FAKE, B=2, N=5, V=1000, T=1.0, seed=0,
                offset=0, wor=0, path=FAKE, n_acc=FAKE, out_tok=FAKE, k_tree=FAKE, v_tree=FAKE,
                num_blocks=10, block_table=FAKE, max_blocks=4, prefix_len=FAKE, k_cache=FAKE,
                v_cache=FAKE, Hkv=2, D=128, block_size=16, slots=FAKE, new_len=FAKE, ws=FAKE,
                ws_bytes=1 << 20, flags=None, stream=None)
    args.update(kw)
    return tav.lib().spec_verify_sample_commit(*args.values())


@pytest.mark.parametrize("kw,code", [
    # the commit's checks
    (dict(k_cache=None), tav.ERR_ARG), (dict(slots=None), tav.ERR_ARG),
    (dict(num_blocks=0), tav.ERR_ARG), (dict(wor=2), tav.ERR_ARG),
    (dict(D=80), tav.ERR_UNSUPPORTED), (dict(block_size=8), tav.ERR_UNSUPPORTED),
    (dict(k_tree=ctypes.c_void_p(0x10008)), tav.ERR_ARG),
    # then the walk's
    (dict(tl=None), tav.ERR_ARG), (dict(path=None), tav.ERR_ARG), (dict(V=0), tav.ERR_ARG),
    (dict(T=-1.0), tav.ERR_ARG), (dict(dl=None), tav.ERR_ARG),
    (dict(V=(1 << 21) + 1), tav.ERR_UNSUPPORTED),
])
def test_sample_commit_rejects_bad_arguments(kw, code):
    assert _sample_commit(**kw) == code


def _commit(**kw):
    args = dict(k_tree=FAKE, v_tree=FAKE, path=FAKE, n_acc=FAKE, num_blocks=10,
                block_table=FAKE, max_blocks=4, prefix_len=FAKE, k_cache=FAKE, v_cache=FAKE,
                B=1, N=5, Hkv=2, D=128, block_size=16, slots=FAKE, new_len=FAKE, flags=None,
                stream=None)
    args.update(kw)
    return tav.lib().kv_commit_path(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(path=None), tav.ERR_ARG), (dict(k_cache=None), tav.ERR_ARG), (dict(B=0), tav.ERR_ARG),
    (dict(num_blocks=0), tav.ERR_ARG), (dict(D=80), tav.ERR_UNSUPPORTED),
    (dict(block_size=8), tav.ERR_UNSUPPORTED), (dict(N=1000), tav.ERR_UNSUPPORTED),
])
def test_commit_rejects_bad_arguments(kw, code):
    assert _commit(**kw) == code


def _inplace(**kw):
    args = dict(path=FAKE, n_acc=FAKE, num_blocks=10, block_table=FAKE, max_blocks=4,
                prefix_len=FAKE, k_cache=FAKE, v_cache=FAKE, B=1, N=5, Hkv=2, D=128,
                block_size=16, slots=FAKE, new_len=FAKE, flags=None, stream=None)
    args.update(kw)
    return tav.lib().kv_commit_inplace(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(path=None), tav.ERR_ARG), (dict(v_cache=None), tav.ERR_ARG), (dict(B=0), tav.ERR_ARG),
    (dict(max_blocks=0), tav.ERR_ARG), (dict(D=80), tav.ERR_UNSUPPORTED),
    (dict(block_size=32), tav.ERR_UNSUPPORTED), (dict(N=257), tav.ERR_UNSUPPORTED),
    (dict(B=70000), tav.ERR_UNSUPPORTED), (dict(k_cache=ctypes.c_void_p(0x10008)), tav.ERR_ARG),
])
def test_inplace_commit_rejects_bad_arguments(kw, code):
    assert _inplace(**kw) == code


def _expand(**kw):
    args = dict(x=FAKE, R=4, V=1000, k=4, T=1.0, tok=FAKE, logq=FAKE, ent=FAKE, ws=FAKE,
                ws_bytes=1 << 20, flags=None, stream=None)
    args.update(kw)
    return tav.lib().tree_expand_topk(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), tav.ERR_ARG), (dict(ent=None), tav.ERR_ARG), (dict(R=0), tav.ERR_ARG),
    (dict(k=0), tav.ERR_ARG), (dict(k=1001), tav.ERR_ARG), (dict(T=0.0), tav.ERR_ARG),
    (dict(k=17, V=5000), tav.ERR_UNSUPPORTED), (dict(V=(1 << 21) + 1), tav.ERR_UNSUPPORTED),
    (dict(ws=None), tav.ERR_WORKSPACE), (dict(ws_bytes=10), tav.ERR_WORKSPACE),
])
def test_expand_rejects_bad_arguments(kw, code):
    assert _expand(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), tav.ERR_ARG), (dict(R=0), tav.ERR_ARG), (dict(k=0), tav.ERR_ARG),
    (dict(T=0.0), tav.ERR_ARG), (dict(k=17, V=5000), tav.ERR_UNSUPPORTED),
    (dict(ws=None), tav.ERR_WORKSPACE),
])
def test_sampled_expand_rejects_bad_arguments(kw, code):
    args = dict(x=FAKE, R=4, V=1000, k=4, T=1.0, seed=1, offset=2, tok=FAKE, logq=FAKE, ent=FAKE,
                ws=FAKE, ws_bytes=1 << 20, flags=None, stream=None)
    args.update(kw)
    assert tav.lib().tree_expand_sample(*args.values()) == code


def test_expand_workspace_sizes():
    lib = tav.lib()
    assert lib.tree_expand_workspace_bytes(0, 100, 4) == 0
    assert lib.tree_expand_workspace_bytes(3, 100, 17) == 0
    assert lib.tree_expand_workspace_bytes(3, 16384, 4) < lib.tree_expand_workspace_bytes(3, 16385, 4)


def _select(**kw):
    args = dict(parent=FAKE, token=FAKE, logq=FAKE, B=2, Nc=100, M=64, op=FAKE, ot=FAKE,
                src=FAKE, flags=None, stream=None)
    args.update(kw)
    return tav.lib().tree_select_topm(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(parent=None), tav.ERR_ARG), (dict(logq=None), tav.ERR_ARG), (dict(src=None), tav.ERR_ARG),
    (dict(B=0), tav.ERR_ARG), (dict(M=0), tav.ERR_ARG), (dict(M=101), tav.ERR_ARG),
    (dict(Nc=1025, M=10), tav.ERR_UNSUPPORTED),
    (dict(logq=ctypes.c_void_p(0x10004)), tav.ERR_ARG),
])
def test_select_rejects_bad_arguments(kw, code):
    assert _select(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(h=None), tav.ERR_ARG), (dict(w=None), tav.ERR_ARG), (dict(B=0), tav.ERR_ARG),
    (dict(F=0), tav.ERR_ARG), (dict(lo=-1), tav.ERR_ARG), (dict(lo=3, hi=2), tav.ERR_ARG),
    (dict(F=1025), tav.ERR_UNSUPPORTED), (dict(h=ctypes.c_void_p(0x10004)), tav.ERR_ARG),
])
def test_widths_reject_bad_arguments(kw, code):
    args = dict(h=FAKE, B=2, F=16, lo=1, hi=4, w=FAKE, flags=None, stream=None)
    args.update(kw)
    assert tav.lib().tree_widths_by_entropy(*args.values()) == code


def test_helpers_reject_bad_arguments():
    lib = tav.lib()
    assert lib.tav_philox_uniforms(0, 0, 1, 1, None, None) == tav.ERR_ARG
    assert lib.tav_philox_uniforms(0, 0, 0, 1, FAKE, None) == tav.ERR_ARG
    assert lib.tav_target_probs(None, 1, 10, 1.0, FAKE, None, None) == tav.ERR_ARG
    assert lib.tav_target_probs(FAKE, 1, 10, 0.0, FAKE, None, None) == tav.ERR_ARG


def test_attention_plan_keeps_every_split_within_its_block_table_copy():
    """Every split of tree_attn_verify's plan stages at most the LDS copy's
    capacity of block-table entries, tree tiles counted in the balance of the
    splits (host arithmetic only, swept over batch, tree size, group size and
    prefix length, for devices from one CU to a full MI355X)."""
    worst = 0
    for cus, per_cu in ((256, 1), (256, 2), (8, 1), (1, 1)):
        for B in (1, 4, 8, 64, 128):
            for N in (1, 5, 16, 64, 128, 192, 256):
                for G in (1, 8, 16):
                    if G * N > 4096:
                        continue
                    for L in (0, 1, 63, 64, 8192, 32767, 32768, 65472, 65536, 131072, 1 << 20):
                        p = tav.attn_plan(B, N, 8 * G, 8, 128, L, cus, per_cu)
                        assert p["max_split_blocks"] <= p["capacity"], (cus, per_cu, B, N, G, L, p)
                        worst = max(worst, p["max_split_blocks"])
    assert worst == 2048   # the bound is reached, so the sweep does test it


def test_attention_plan_case_that_once_overflowed():
    """B=64, N=192, Hq=Hkv=8, prefix up to 65472: one split used to take 513
    prefix tiles (2052 block-table entries for a 2048-entry copy)."""
    p = tav.attn_plan(64, 192, 8, 8, 128, 65472, 256, 1)
    assert p["max_split_blocks"] <= p["capacity"] == 2048
    assert p["splits"] >= 2


def test_attention_plan_takes_four_row_waves_where_splits_dominate():
    """On a 256-CU device: 64 tree nodes, 32 query heads on 8 KV heads (256
    query rows per KV head), 4096-token prefix. At batch one the 8-row-wave
    form makes 128 workgroups (16 splits at most) and at batch 2 and 4 it
    needs 16 and 8 splits, so the plan takes four row waves in two key sets
    (two row blocks, half the splits); from batch 8 on it fills the device
    with 4 splits or fewer and keeps eight row waves. Above 256 rows (the
    70B-shaped layer, 512 rows) only the split cap switches: batch one and
    one KV head of batch 8 (16 splits) switch, batch 2 (8 splits) does not."""
    rb = lambda *a: (lambda p: (p["row_blocks"], p["splits"]))(tav.attn_plan(*a, 256, 1))
    assert rb(1, 64, 32, 8, 128, 4096) == (2, 16)
    assert rb(2, 64, 32, 8, 128, 4096) == (2, 8)
    assert rb(4, 64, 32, 8, 128, 4096) == (2, 4)
    for B in (8, 32):
        assert rb(B, 64, 32, 8, 128, 4096)[0] == 1, B
    assert rb(1, 64, 64, 8, 128, 8192) == (4, 8)
    assert rb(8, 64, 8, 1, 128, 8192) == (4, 8)
    assert rb(2, 64, 64, 8, 128, 8192) == (2, 8)
    assert rb(8, 64, 64, 8, 128, 8192) == (2, 2)
    # splits the block-table bound forces on a full device do not switch:
    # a 1M-token prefix at batch 4 (70B-shaped) and at batch 32 (8B-shaped)
    p = tav.attn_plan(4, 64, 64, 8, 128, 1 << 20, 256, 1)
    assert p["row_blocks"] == 2 and p["splits"] > 16, p
    p = tav.attn_plan(32, 64, 32, 8, 128, 1 << 20, 256, 1)
    assert p["row_blocks"] == 1 and p["splits"] > 8, p
    # the two GPU parity cases of this form (ragged second row block)
    assert tav.attn_plan(1, 40, 32, 8, 64, 2000, 256, 1)["row_blocks"] == 2
    assert tav.attn_plan(1, 60, 32, 8, 128, 2600, 256, 1)["row_blocks"] == 2
    # at most 128 rows: the 4-row-wave form, as before
    assert tav.attn_plan(1, 16, 64, 8, 128, 4096, 256, 1)["row_blocks"] == 1
    assert tav.attn_plan(1, 16, 64, 8, 128, 4096, 256, 1)["waves"] == 8


def test_attention_plan_rejects_bad_arguments():
    lib = tav.lib()
    plan = (ctypes.c_int32 * 5)()
    assert lib.tav_attn_plan(1, 5, 8, 2, 128, 64, 256, 1, None) == tav.ERR_ARG
    assert lib.tav_attn_plan(1, 5, 8, 2, 128, 64, 0, 1, ctypes.cast(plan, P)) == tav.ERR_ARG
    assert lib.tav_attn_plan(1, 5, 8, 2, 96, 64, 256, 1, ctypes.cast(plan, P)) == tav.ERR_UNSUPPORTED


def test_sampler_plan_rejects_bad_arguments():
    lib = tav.lib()
    plan = (ctypes.c_int32 * 4)()
    assert lib.tav_sampler_plan(8, 1000, 0, None) == tav.ERR_ARG
    assert lib.tav_sampler_plan(0, 1000, 0, ctypes.cast(plan, P)) == tav.ERR_ARG
    assert lib.tav_sampler_plan(8, 0, 0, ctypes.cast(plan, P)) == tav.ERR_ARG
    assert lib.tav_sampler_plan(8, 1000, 2, ctypes.cast(plan, P)) == tav.ERR_ARG
    assert lib.tav_sampler_plan(8, (1 << 21) + 1, 0, ctypes.cast(plan, P)) == tav.ERR_UNSUPPORTED


def test_sampler_plan_for_rejects_bad_arguments():
    lib = tav.lib()
    plan = (ctypes.c_int32 * 4)()
    occ = (ctypes.c_int32 * 5)(1, 1, 1, 1, 1)
    bad = (ctypes.c_int32 * 5)(1, -1, 1, 1, 1)
    pp, po, pb = (ctypes.cast(x, P) for x in (plan, occ, bad))
    assert lib.tav_sampler_plan_for(8, 1000, 0, 256, po, None) == tav.ERR_ARG
    assert lib.tav_sampler_plan_for(8, 1000, 0, 256, None, pp) == tav.ERR_ARG
    assert lib.tav_sampler_plan_for(8, 1000, 0, 0, po, pp) == tav.ERR_ARG
    assert lib.tav_sampler_plan_for(8, 1000, 0, 256, pb, pp) == tav.ERR_ARG
    assert lib.tav_sampler_plan_for(0, 1000, 0, 256, po, pp) == tav.ERR_ARG
    assert lib.tav_sampler_plan_for(8, 1000, 3, 256, po, pp) == tav.ERR_ARG
    assert lib.tav_sampler_plan_for(8, (1 << 21) + 1, 0, 256, po, pp) == tav.ERR_UNSUPPORTED
    # nothing resident: no layout fits
    zero = (ctypes.c_int32 * 5)(0, 0, 0, 0, 0)
    assert lib.tav_sampler_plan_for(8, 1000, 0, 256, ctypes.cast(zero, P), pp) == tav.ERR_LAUNCH


@pytest.mark.parametrize("B,entries,groups", [
    (1, 4, 1), (4, 4, 4), (8, 8, 8), (16, 16, 16), (32, 16, 16), (64, 16, 16),
    (96, 16, 16), (128, 28, 28), (256, 28, 28)])
def test_sampler_plan_for_the_70b_vocabulary(B, entries, groups):
    """The layout rule on a 256-CU device holding one walk workgroup per CU,
    over a 128256-token vocabulary: 4 entries per thread up to batch 4, 8 at
    batch 8, 16 up to batch 96, and 28 (16 in registers, 12 in LDS) where it
    cuts the sequences per group by more than a third."""
    p = tav.sampler_plan_for(B, 128256, 256, (1, 1, 1, 1, 1))
    assert (p["entries_per_thread"], p["groups"]) == (entries, groups), p
    assert p["workgroups_per_sequence"] == -(-128256 // (512 * entries))
    g = tav.sampler_plan_for(B, 128256, 256, (1, 1, 1, 1, 1), greedy=True)
    assert g["entries_per_thread"] == 8


def test_sampler_plan_for_covers_the_vocabulary():
    """Over a sweep of batches, vocabularies and device shapes: the chunks
    are whole 16-byte runs that cover the vocabulary with no workgroup past
    its capacity, no more groups than sequences, and no more workgroups
    than the device holds at once."""
    for cus in (1, 8, 80, 256):
        for occ in ((1, 1, 1, 1, 1), (2, 2, 1, 1, 2), (2, 1, 1, 0, 1)):
            for B in (1, 2, 3, 5, 8, 17, 64, 100, 128, 300):
                for V in (1, 3, 1000, 4097, 20001, 32000, 128256, 151936, 1 << 21):
                    for greedy in (False, True):
                        try:
                            p = tav.sampler_plan_for(B, V, cus, occ, greedy=greedy)
                        except tav.TavError as e:
                            assert e.status == tav.ERR_LAUNCH
                            continue
                        E, wpg, ng, chunk = (p["entries_per_thread"], p["workgroups_per_sequence"],
                                             p["groups"], p["chunk"])
                        assert E in ((8,) if greedy else (4, 8, 16, 28))
                        assert chunk % 4 == 0 and chunk <= 512 * E
                        assert wpg * chunk >= V and (wpg - 1) * chunk < V
                        assert 1 <= ng <= B
                        i = 4 if greedy else (4, 8, 16, 28).index(E)
                        assert ng * wpg <= occ[i] * cus


def test_noalloc_sampler_rejects_bad_arguments_before_any_device_work():
    lib = tav.lib()
    fn = lib.spec_verify_sample_noalloc
    base = dict(tl=FAKE, dl=FAKE, parent=FAKE, token=FAKE, B=2, N=5, V=1000, T=1.0, seed=0,
                offset=0, path=FAKE, n_acc=FAKE, out_tok=FAKE, flags=None, stream=None)
    for kw, code in [(dict(tl=None), tav.ERR_ARG), (dict(B=0), tav.ERR_ARG),
                     (dict(T=-1.0), tav.ERR_ARG), (dict(N=257), tav.ERR_UNSUPPORTED),
                     (dict(V=(1 << 21) + 1), tav.ERR_UNSUPPORTED), (dict(dl=None), tav.ERR_ARG)]:
        args = dict(base)
        args.update(kw)
        assert fn(*args.values()) == code, kw


def test_topology_rejects_bad_arguments_on_the_host():
    lib = tav.lib()
    bad = (ctypes.c_double * 2)(0.5, 1.5)
    ok = (ctypes.c_double * 2)(0.5, 0.5)
    cast = lambda a: ctypes.cast(a, P)
    assert lib.tree_topology_dp(cast(bad), 2, 4, 3, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == tav.ERR_ARG
    assert lib.tree_topology_dp(None, 2, 4, 3, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == tav.ERR_ARG
    # no 8-node tree of depth 2 with 2 children per node (at most 1 + 2 + 4)
    assert lib.tree_topology_dp(cast(ok), 2, 8, 2, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == tav.ERR_UNSUPPORTED
    assert lib.tree_topology_dp(cast(ok), 17, 8, 2, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == tav.ERR_UNSUPPORTED
    assert lib.tree_topology_dp(cast(ok), 2, 7, 2, FAKE, FAKE, FAKE, None, 0, None) == tav.ERR_WORKSPACE
    assert lib.tree_topology_workspace_bytes(4, 64, 6) == 6 * 6 * 64 * 2
