"""index_score_topk_noalloc (the indexer call for callers that cannot allocate)
against index_score_topk with a workspace, through the C ABI: two calls in a row
on one GPU, the second with a smaller input, must give the same selections (and
these agree with the oracle's)."""
import numpy as np
import pytest
import torch

from long_context_sparse_19_amd.configs import DECODE, RAGGED, scaled_down
from long_context_sparse_19_amd.inputs import make_inputs
from oracle import oracle as O
from tests import parity as P

pytestmark = pytest.mark.gpu


def _case(w):
    from long_context_sparse_19_amd import _lib, device as D
    inp = make_inputs(w, with_attention=False)
    d = D.upload(inp)
    D.compress(d)
    ws = D.Workspaces(d)
    D.score_topk(d, ws)                                   # with a workspace
    ref = ws.sel.clone()
    got = torch.full_like(ref, -7)
    _lib.index_score_topk_noalloc(d.seqs, d.q_idx, d.gates, d.pooled, d.top_k, got)
    torch.cuda.synchronize()
    return inp, d, ref.cpu().numpy(), got.cpu().numpy()


@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
def test_noalloc_matches_the_workspace_call_twice():
    for w in (scaled_down(DECODE, 4 * 33000 + 4, batch=2), scaled_down(RAGGED, 4 * 3000, batch=3, min_blocks=200)):
        inp, d, ref, got = _case(w)
        assert np.array_equal(got, ref), w.name
        pooled, sigma, *_ = O.compress(inp)
        vals = O.pooled_values(np.asarray(d.pooled.data.cpu().numpy()), d.pooled.scale.cpu().numpy().astype(np.float64))
        ids, scores = O.score_select(inp, vals, w.top_k)
        for r in range(w.n_rows):
            P.check_selection(got[r], ids[r], scores[r], int(inp.q_pos[r]) // 4, w.top_k)
