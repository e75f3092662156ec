"""Re-entrancy through the C ABI: two different problems (per-tile lists at
d = 128 and per-segment block lists at d = 64) run the whole path on two
streams at once, each several times, and every result equals the same
problem run alone, bit for bit.  The library keeps no state between calls
and every buffer is the caller's, so concurrent calls on different streams do
not interact."""

import pytest
import torch

import long_context_prefill_amd as s2o
from long_context_prefill_amd import synth
from parity_util import say, to_device

pytestmark = pytest.mark.gpu

TAU = 1e-3
ROUNDS = 3


def _problem(name, Hq, Hkv, N, d, lists, seed):
    w = synth.custom_workload(B=1, Hq=Hq, Hkv=Hkv, N=N, d=d, dtype="bf16", tile_m=128, tile_n=64,
                              seg_len=1024, structure="stripes+band", n_stripes=N // 100, seed=seed, name=name)
    x = synth.make_inputs(w)
    q, k, v = (to_device(x[n]) for n in ("q", "k", "v"))
    p = s2o.problem(w.B, w.Hq, w.Hkv, w.N, w.d, 1, w.seg_len, w.tile_m, w.tile_n, w.scale, lists=lists)
    return p, q, k, v


def _run(p, q, k, v, ws):
    """The whole path into fresh outputs; workspaces from ws (allocated beforehand)."""
    scores = s2o.s2o_score(p, q, k, ws["scores"], ws["ws_score"])
    idx = s2o.s2o_build_index(p, scores, ws["idx"], ws["ws_sort"])
    o, ex = s2o.s2o_attn_fwd(p, q, k, v, idx, TAU, out=ws["o"], exec_tiles=ws["ex"])
    od = s2o.dense_attn_fwd(p, q, k, v, out=ws["od"])
    return scores, idx, o, ex, od


def _buffers(p, q):
    n = max(s2o.list_entries(p), 1)
    return {"scores": torch.empty(n, dtype=torch.float32, device="cuda"),
            "idx": torch.empty(n, dtype=torch.int32, device="cuda"),
            "ws_score": torch.empty(max(s2o.score_workspace_bytes(p), 1), dtype=torch.uint8, device="cuda"),
            "ws_sort": torch.empty(max(s2o.build_index_workspace_bytes(p), 1), dtype=torch.uint8, device="cuda"),
            "o": torch.empty_like(q), "od": torch.empty_like(q),
            "ex": torch.empty((p.batch, p.heads_q, p.seq_len // p.tile_m), dtype=torch.int32, device="cuda")}


def _bits(res):
    scores, idx, o, ex, od = res
    return [scores.view(torch.int32).clone(), idx.clone(), o.view(torch.int16).clone(), ex.clone(),
            od.view(torch.int16).clone()]


def test_two_streams_at_once_equal_each_problem_alone():
    probs = [_problem("streams_a", 8, 2, 8192, 128, "tile", 41),
             _problem("streams_b", 4, 1, 6144, 64, "segment_blocks", 42)]
    bufs = [_buffers(p, q) for p, q, _, _ in probs]
    say("streams: each problem alone")
    want = []
    for (p, q, k, v), ws in zip(probs, bufs):
        want.append(_bits(_run(p, q, k, v, ws)))
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    for r in range(ROUNDS):
        for ws in bufs:  # sentinels, so a result that was not rewritten cannot pass
            for key in ("scores", "o", "od"):
                ws[key].fill_(float("nan"))
            ws["idx"].fill_(-1)
            ws["ex"].fill_(-1)
        torch.cuda.synchronize()
        say(f"streams: round {r}, both problems at once")
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        outs = []
        for (p, q, k, v), ws, s in zip(probs, bufs, streams):
            with torch.cuda.stream(s):
                outs.append(_run(p, q, k, v, ws))
        torch.cuda.synchronize()
        for i, (res, ref) in enumerate(zip(outs, want)):
            for name, got, exp in zip(("scores", "idx", "out", "exec_tiles", "dense out"), _bits(res), ref):
                assert torch.equal(got, exp), (i, name, r)
