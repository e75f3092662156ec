"""s2o_score_noalloc (static device workspace) against s2o_score (caller
workspace) through the C ABI: bit-identical scores on two calls in a row, the
second on a smaller problem, for per-tile and per-segment lists."""

import numpy as np
import pytest
import torch

import long_context_prefill_amd as s2o
from long_context_prefill_amd import synth
from parity_util import say, to_device

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, N, seed):
    w = synth.custom_workload(B=B, Hq=Hq, Hkv=Hkv, N=N, d=128, dtype="bf16", tile_m=128, tile_n=64,
                              seg_len=1024, structure="stripes+band", n_stripes=N // 100, seed=seed,
                              name=f"noalloc_{N}")
    x = synth.make_inputs(w)
    return w, to_device(x["q"]), to_device(x["k"])


@pytest.mark.parametrize("lists", ["tile", "segment"])
def test_noalloc_scores_equal_the_workspace_entry_point(lists):
    cases = [(2, 8, 2, 8192, 5), (1, 4, 1, 4096, 6)]  # the second call is the smaller problem
    for B, Hq, Hkv, N, seed in cases:
        w, q, k = _inputs(B, Hq, Hkv, N, seed)
        p = s2o.problem(B, Hq, Hkv, N, 128, 1, w.seg_len, 128, 64, w.scale, lists=lists)
        assert 0 < s2o.score_workspace_bytes(p) <= s2o.SCORE_NOALLOC_MAX_WORKSPACE
        say(f"noalloc {lists} lists, B={B} Hq={Hq} N={N}")
        ref = s2o.s2o_score(p, q, k)
        got = torch.full_like(ref, float("nan"))
        s2o.s2o_score_noalloc(p, q, k, got)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), (lists, N)
        assert np.isfinite(got.cpu().numpy()).all()
