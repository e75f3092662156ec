"""The whole path captured in one HIP graph and replayed through the C ABI:
s2o_score (or s2o_score_noalloc), s2o_build_index, s2o_attn_fwd and
dense_attn_fwd.  The library allocates nothing, clears no memory with memset
nodes and enqueues only on the caller's stream, so the calls can be captured.
Every replay, with the program's own eager work and synchronisations between
replays and the outputs overwritten with sentinels before each, must equal the
eager calls bit for bit (the kernels are deterministic)."""

import pytest
import torch

import long_context_prefill_amd as s2o
from long_context_prefill_amd import synth
from parity_util import say, to_device

pytestmark = pytest.mark.gpu

TAU = 1e-3
REPLAYS = 3

# (lists, qperm, share_gqa, noalloc score)
CASES = [("tile", False, False, False), ("tile", False, False, True), ("segment", False, False, False),
         ("tile_blocks", False, False, False), ("tile", True, False, False), ("segment", False, True, False)]


def _case_id(c):
    lists, qperm, share, noalloc = c
    return lists + ("_qperm" if qperm else "") + ("_shared" if share else "") + ("_noalloc" if noalloc else "")


class Buffers:
    """Outputs and workspaces of one run of the path (allocated before any capture)."""

    def __init__(self, p, q):
        self.scores = torch.empty(max(s2o.list_entries(p), 1), dtype=torch.float32, device="cuda")
        self.idx = torch.empty(max(s2o.list_entries(p), 1), dtype=torch.int32, device="cuda")
        self.ws_score = torch.empty(max(s2o.score_workspace_bytes(p), 1), dtype=torch.uint8, device="cuda")
        self.ws_sort = torch.empty(max(s2o.build_index_workspace_bytes(p), 1), dtype=torch.uint8, device="cuda")
        self.o = torch.empty_like(q)
        self.od = torch.empty_like(q)
        self.ex = torch.empty((p.batch, p.heads_q, p.seq_len // p.tile_m), dtype=torch.int32, device="cuda")

    def poison(self):
        self.scores.fill_(float("nan"))
        self.idx.fill_(-1)
        self.o.fill_(float("nan"))
        self.od.fill_(float("nan"))
        self.ex.fill_(-1)

    def results(self):
        return (self.scores.view(torch.int32), self.idx, self.o.view(torch.int16), self.od.view(torch.int16),
                self.ex)


def run_path(p, q, k, v, buf, noalloc):
    if noalloc:
        s2o.s2o_score_noalloc(p, q, k, buf.scores)
    else:
        s2o.s2o_score(p, q, k, buf.scores, buf.ws_score)
    s2o.s2o_build_index(p, buf.scores, buf.idx, buf.ws_sort)
    s2o.s2o_attn_fwd(p, q, k, v, buf.idx, TAU, out=buf.o, exec_tiles=buf.ex)
    s2o.dense_attn_fwd(p, q, k, v, out=buf.od)


@pytest.mark.parametrize("case", CASES, ids=_case_id)
def test_pipeline_replays_in_a_hip_graph(case):
    lists, qperm, share, noalloc = case
    w = synth.custom_workload(B=1, Hq=4, Hkv=1, N=4096, d=128, dtype="bf16", tile_m=128, tile_n=64,
                              seg_len=1024, structure="stripes+band", n_stripes=40, seed=71, name="graph_4k")
    x = synth.make_inputs(w)
    q, k, v = (to_device(x[n]) for n in ("q", "k", "v"))
    p = s2o.problem(w.B, w.Hq, w.Hkv, w.N, w.d, 1, w.seg_len, w.tile_m, w.tile_n, w.scale, lists=lists,
                    qperm=qperm, share_gqa=share)
    if noalloc:
        assert s2o.score_workspace_bytes(p) <= s2o.SCORE_NOALLOC_MAX_WORKSPACE
    say(f"graph capture: {_case_id(case)}")

    eager = Buffers(p, q)
    run_path(p, q, k, v, eager, noalloc)
    torch.cuda.synchronize()
    want = [t.clone() for t in eager.results()]
    assert int(eager.ex.min()) > 0

    cap = Buffers(p, q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream, as capture requires
        run_path(p, q, k, v, cap, noalloc)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_path(p, q, k, v, cap, noalloc)
    torch.cuda.synchronize()

    names = ("scores", "idx", "out", "dense out", "exec_tiles")
    for r in range(REPLAYS):
        cap.poison()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(names, cap.results(), want):
            assert torch.equal(got, ref), (name, r)
        # the program's own eager work between replays
        run_path(p, q, k, v, eager, noalloc)
        torch.cuda.synchronize()
        for name, got, ref in zip(names, eager.results(), want):
            assert torch.equal(got, ref), (name, "eager", r)
    say(f"graph capture: {_case_id(case)}: {REPLAYS} replays equal the eager calls")
