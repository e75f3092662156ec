"""CPU checks of the C ABI: the library loads, exports what include/s2o.h declares,
and its host-side geometry and validation behave as documented.  No compute call
is made (there is no GPU here); every error path returns before anything is
enqueued."""

import ctypes
import os
import re

import numpy as np
import pytest

import long_context_prefill_amd as s2o
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "s2o.h")

pytestmark = pytest.mark.skipif(not os.path.exists(s2o.LIB_PATH), reason="libs2o.so not built")

INVALID, UNSUPPORTED, WORKSPACE = -1, -2, -3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(s2o.EXPORTS), names
    L = s2o.lib()
    for n in names:
        assert getattr(L, n) is not None


def base_problem(**kw):
    args = dict(batch=1, heads_q=4, heads_kv=2, seq_len=1024, head_dim=128, dtype=1,
                seg_len=256, tile_m=128, tile_n=64, scale=None, causal=True)
    args.update(kw)
    return s2o.problem(**args)


@pytest.mark.parametrize("N,S,BM,B,Hq", [(1024, 256, 128, 1, 4), (2048, 512, 64, 2, 3),
                                         (1000 * 64 // 64 * 64, 384, 64, 1, 2),
                                         (131072, 8192, 128, 1, 32), (640, 1024, 128, 1, 1)])
def test_list_layout_matches_oracle_walk(N, S, BM, B, Hq):
    """The library's closed-form offsets agree with the oracle's tile-by-tile walk."""
    p = base_problem(batch=B, heads_q=Hq, heads_kv=1, seq_len=N, seg_len=S, tile_m=BM)
    assert s2o.check_problem(p) == 0
    po = oracle.problem(B, Hq, 1, N, 128, "bf16", S, BM, 64, 1.0)
    assert s2o.list_entries(p) == oracle.list_entries(po)
    T = N // BM
    for b in range(B):
        for h in {0, Hq - 1}:
            for t in sorted({0, T // 3, T // 2, T - 1}):
                assert s2o.list_offset(p, b, h, t) == oracle.list_offset(po, b, h, t)
    assert s2o.list_offset(p, B, 0, 0) == -1
    assert s2o.list_offset(p, 0, 0, T) == -1


@pytest.mark.parametrize("N,S,BM,B,Hq", [(1024, 256, 128, 1, 4), (2048, 512, 64, 2, 3),
                                         (64 * 63, 384, 64, 1, 2), (131072, 8192, 128, 1, 32)])
def test_segment_list_layout_matches_oracle_walk(N, S, BM, B, Hq):
    p = base_problem(batch=B, heads_q=Hq, heads_kv=1, seq_len=N, seg_len=S, tile_m=BM,
                     lists="segment")
    assert s2o.check_problem(p) == 0
    po = oracle.problem(B, Hq, 1, N, 128, "bf16", S, BM, 64, 1.0, per_segment=True)
    assert s2o.list_entries(p) == oracle.list_entries(po)
    T = N // BM
    for b in range(B):
        for h in {0, Hq - 1}:
            for t in sorted({0, T // 3, T // 2, T - 1}):
                assert s2o.list_offset(p, b, h, t) == oracle.list_offset(po, b, h, t)


@pytest.mark.parametrize("lists", ["tile_blocks", "segment_blocks"])
@pytest.mark.parametrize("N,S,BM,B,Hq", [(1024, 256, 128, 1, 4), (2048, 512, 64, 2, 3),
                                         (64 * 63, 384, 64, 1, 2), (131072, 8192, 128, 1, 32)])
def test_block_list_layout_matches_oracle_walk(N, S, BM, B, Hq, lists):
    p = base_problem(batch=B, heads_q=Hq, heads_kv=1, seq_len=N, seg_len=S, tile_m=BM, lists=lists)
    assert s2o.check_problem(p) == 0
    po = oracle.problem(B, Hq, 1, N, 128, "bf16", S, BM, 64, 1.0, per_segment=lists.startswith("segment"),
                        block_lists=True)
    assert s2o.list_entries(p) == oracle.list_entries(po)
    T = N // BM
    for b in range(B):
        for h in {0, Hq - 1}:
            for t in sorted({0, T // 3, T // 2, T - 1}):
                assert s2o.list_offset(p, b, h, t) == oracle.list_offset(po, b, h, t)


@pytest.mark.parametrize("lists", ["tile", "segment", "tile_blocks", "segment_blocks"])
@pytest.mark.parametrize("N,S,BM,B,Hq,Hkv", [(1024, 256, 128, 1, 4, 2), (2048, 512, 64, 2, 6, 2),
                                             (64 * 63, 384, 64, 1, 2, 1), (131072, 8192, 128, 1, 32, 8)])
def test_shared_list_layout_matches_oracle_walk(N, S, BM, B, Hq, Hkv, lists):
    """Shared lists: one run per (b, KV head), read by every query head of the group."""
    p = base_problem(batch=B, heads_q=Hq, heads_kv=Hkv, seq_len=N, seg_len=S, tile_m=BM, lists=lists,
                     share_gqa=True)
    assert s2o.check_problem(p) == 0
    po = oracle.problem(B, Hq, Hkv, N, 128, "bf16", S, BM, 64, 1.0, per_segment=lists.startswith("segment"),
                        block_lists=lists.endswith("blocks"), share_gqa=True)
    ph = base_problem(batch=B, heads_q=Hq, heads_kv=Hkv, seq_len=N, seg_len=S, tile_m=BM, lists=lists)
    assert s2o.list_entries(p) == oracle.list_entries(po) == s2o.list_entries(ph) // (Hq // Hkv)
    T, G = N // BM, Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            for t in sorted({0, T // 3, T // 2, T - 1}):
                off = s2o.list_offset(p, b, h, t)
                assert off == oracle.list_offset(po, b, h, t) == s2o.list_offset(p, b, h // G * G, t)


def test_workspace_sizes():
    p = base_problem()
    assert s2o.score_workspace_bytes(p) == 1 * 4 * (1024 // 128) * 128 * 4
    # every list fits one workgroup's LDS (at most 4096 entries): sorted in place
    assert s2o.build_index_workspace_bytes(p) == 0
    # longer lists: (key, position) pairs and their scratch copy, 16 bytes per entry
    p = base_problem(seq_len=16384, seg_len=4096)
    assert s2o.build_index_workspace_bytes(p) >= 16 * s2o.list_entries(p)
    # many lists: the scratch is one slot per overflow workgroup (1024 x the
    # longest list) once that is smaller than a copy of every list
    p = s2o.problem(1, 32, 8, 131072, 128, 1, 8192, 128, 64)
    n, longest = s2o.list_entries(p), 15 * 8192
    ws = s2o.build_index_workspace_bytes(p)
    assert 8 * n + 8 * 1024 * longest <= ws < 8 * n + 8 * 1024 * longest + n  # + histograms and queues
    assert ws < 9 * n
    # block lists: the mean key of every block joins the pooled queries
    p = base_problem(lists="tile_blocks")
    assert s2o.score_workspace_bytes(p) == 1 * 4 * 8 * 128 * 4 + 1 * 2 * (1024 // 64) * 128 * 4
    assert s2o.list_entries(p) == s2o.list_entries(base_problem()) // 64


@pytest.mark.parametrize("field,value,code", [
    ("batch", 0, INVALID), ("heads_q", 3, INVALID), ("seq_len", 1000, INVALID),
    ("seg_len", 200, INVALID), ("head_dim", 96, UNSUPPORTED), ("tile_m", 256, UNSUPPORTED),
    ("tile_n", 32, UNSUPPORTED), ("dtype", 7, INVALID), ("causal", 2, INVALID),
    ("scale", float("nan"), INVALID), ("scale", 0.0, INVALID), ("scale", -0.125, INVALID),
    ("scale", float("inf"), INVALID), ("tile_m", 96, INVALID), ("list_granularity", 16, INVALID), ("list_granularity", -1, INVALID),
    ("list_granularity", 4 | 8, UNSUPPORTED),  # query permutation with shared lists
    ("seq_len", 1 << 23, UNSUPPORTED)])  # one head's K at d = 128 would span 2^31 bytes
def test_problem_validation(field, value, code):
    p = base_problem()
    setattr(p, field, value)
    assert s2o.check_problem(p) == code
    assert s2o.lib().s2o_list_entries(ctypes.byref(p)) == -1


def _call(name, *args):
    return getattr(s2o.lib(), name)(*args)


def test_entry_points_reject_bad_arguments_before_launch():
    """Every case returns its documented status synchronously; nothing reaches HIP."""
    L = s2o.lib()
    p = base_problem()
    pb = ctypes.byref(p)
    nul = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x100000)  # never dereferenced: validation fails first
    odd = ctypes.c_void_p(0x100004)
    n = s2o.list_entries(p)
    # null pointers
    assert L.s2o_attn_fwd(pb, nul, fake, fake, fake, 0.0, fake, nul, nul) == INVALID
    assert L.dense_attn_fwd(pb, fake, fake, fake, nul, nul) == INVALID
    assert L.s2o_score(pb, fake, nul, fake, fake, 1 << 30, nul) == INVALID
    assert L.s2o_build_index(pb, nul, fake, fake, 1 << 40, nul) == INVALID
    # misaligned tensors
    assert L.s2o_attn_fwd(pb, odd, fake, fake, fake, 0.0, fake, nul, nul) == INVALID
    # bad tau
    assert L.s2o_attn_fwd(pb, fake, fake, fake, fake, -1e-3, fake, nul, nul) == INVALID
    assert L.s2o_attn_fwd(pb, fake, fake, fake, fake, float("nan"), fake, nul, nul) == INVALID
    # workspace missing, too small or misaligned (lists long enough to need one)
    pl = base_problem(seq_len=16384, seg_len=4096)
    plb = ctypes.byref(pl)
    need = s2o.build_index_workspace_bytes(pl)
    assert need > 0
    assert L.s2o_build_index(plb, fake, fake, nul, need, nul) == WORKSPACE
    assert L.s2o_build_index(plb, fake, fake, fake, need - 1, nul) == WORKSPACE
    assert L.s2o_build_index(plb, fake, fake, ctypes.c_void_p(0x100080), need, nul) == WORKSPACE
    assert L.s2o_score(pb, fake, fake, fake, fake, s2o.score_workspace_bytes(p) - 4, nul) == WORKSPACE
    # causal = 0 is dense-only
    pc = base_problem(causal=False)
    assert L.s2o_score(ctypes.byref(pc), fake, fake, fake, fake, 1 << 30, nul) == UNSUPPORTED
    assert L.s2o_build_index(ctypes.byref(pc), fake, fake, fake, 1 << 40, nul) == UNSUPPORTED
    assert L.s2o_attn_fwd(ctypes.byref(pc), fake, fake, fake, fake, 0.0, fake, nul, nul) == UNSUPPORTED
    # unsupported head dim
    pd = base_problem(head_dim=96)
    assert L.dense_attn_fwd(ctypes.byref(pd), fake, fake, fake, fake, nul) == UNSUPPORTED
    # null problem
    assert L.s2o_check_problem(None) == INVALID
    assert n > 0


def test_status_strings():
    L = s2o.lib()
    for code in (0, -1, -2, -3, -4):
        assert len(L.s2o_status_string(code)) > 0
    assert L.s2o_status_string(99) == b"unknown status"


def test_python_binding_raises_without_device_tensors():
    import torch
    p = base_problem()
    q = torch.zeros(1, 4, 1024, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        s2o.dense_attn_fwd(p, q, q[:, :2].contiguous(), q[:, :2].contiguous())


@pytest.mark.parametrize("lists", ["tile", "segment", "tile_blocks"])
def test_query_permutation_layout_and_validation(lists):
    """Q_perm appends one run of N query-order entries per (b, h) after every key list."""
    N, S, BM, B, Hq = 2048, 512, 128, 2, 3
    p = base_problem(batch=B, heads_q=Hq, heads_kv=1, seq_len=N, seg_len=S, tile_m=BM, lists=lists,
                     qperm=True)
    assert s2o.check_problem(p) == 0
    po = oracle.problem(B, Hq, 1, N, 128, "bf16", S, BM, 64, 1.0, per_segment=lists.startswith("segment"),
                        block_lists=lists.endswith("blocks"), qperm=True)
    pk = base_problem(batch=B, heads_q=Hq, heads_kv=1, seq_len=N, seg_len=S, tile_m=BM, lists=lists)
    assert s2o.list_entries(p) == oracle.list_entries(po) == s2o.list_entries(pk) + B * Hq * N
    for b, h, t in [(0, 0, 5), (1, 2, 15)]:
        assert s2o.list_offset(p, b, h, t) == s2o.list_offset(pk, b, h, t) == oracle.list_offset(po, b, h, t)
    # fp32 inputs and segments beyond the in-LDS query sort are not compiled
    assert s2o.check_problem(base_problem(dtype=0, qperm=True)) == UNSUPPORTED
    assert s2o.check_problem(base_problem(seq_len=32768, seg_len=16384, qperm=True)) == UNSUPPORTED


def test_score_noalloc_rejects_problems_above_its_static_workspace():
    """s2o_score_noalloc validates the problem and its workspace size on the host
    and returns before touching the GPU: an invalid problem is INVALID_ARG, one
    whose score workspace exceeds the static array is WORKSPACE, and the header's
    limit is the one the binding states."""
    text = open(HEADER).read()
    m = re.search(r"#define S2O_SCORE_NOALLOC_MAX_WORKSPACE \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == s2o.SCORE_NOALLOC_MAX_WORKSPACE
    L = s2o.lib()
    fake, nul = ctypes.c_void_p(1 << 20), ctypes.c_void_p(0)
    big = base_problem(batch=8, heads_q=32, heads_kv=8, seq_len=131072, seg_len=8192)
    assert s2o.score_workspace_bytes(big) > s2o.SCORE_NOALLOC_MAX_WORKSPACE
    assert L.s2o_score_noalloc(ctypes.byref(big), fake, fake, fake, nul) == WORKSPACE
    bad = base_problem(seq_len=1000)
    assert L.s2o_score_noalloc(ctypes.byref(bad), fake, fake, fake, nul) == INVALID
    head = base_problem(batch=1, heads_q=32, heads_kv=8, seq_len=131072, seg_len=8192)
    for lists in ("tile", "segment", "tile_blocks"):
        for qperm in (False, True):
            p = base_problem(batch=1, heads_q=32, heads_kv=8, seq_len=131072, seg_len=8192, lists=lists,
                             qperm=qperm)
            assert s2o.score_workspace_bytes(p) <= s2o.SCORE_NOALLOC_MAX_WORKSPACE, (lists, qperm)
    assert s2o.score_workspace_bytes(head) > 0
