"""The context handle (cachetune_create / cachetune_prepare_scoring): score
calls that take the twiddle and trigonometric tables from a prepared handle
give the same scores, bit for bit, as calls that rebuild them in their
workspace; once prepared, a call launches no table build and its workspace
query no longer counts the tables.  Covers the fp16 pass, the redo pass for
values beyond the fp16 range (its per-block range flags are written, not
cleared, by every call), and ragged lengths sharing tables."""
import numpy as np
import pytest
import torch

from gpu_util import need_gpu, to_dev

pytestmark = pytest.mark.gpu

SEED = 20260600


def _chunks(syn, ns, L, H, D, wide=False):
    out = []
    for b, n in enumerate(ns):
        k = syn.chunk(SEED, syn.K, 50 + b, L, n, H, D, "bf16")
        v = syn.chunk(SEED, syn.V, 50 + b, L, n, H, D, "bf16")
        if wide and b == 1:  # values beyond the fp16 range in one problem (exact in bf16)
            k = k.copy()
            k[1, 7] = (k[1, 7].astype(np.uint32) + (17 << 7)).astype(np.uint16)
        out.append((to_dev(k), to_dev(v)))
    return out


@pytest.mark.parametrize("alpha", [(1, 16), (1, 32)])
def test_prepared_tables_give_identical_scores(syn, alpha):
    ct = need_gpu()
    ns, L, H, D = [2048, 1500, 2048, 777], 3, 8, 128
    chunks = _chunks(syn, ns, L, H, D, wide=True)
    ws_before = ct.cachetune_score_chunk_ws(ns, L, H, D, alpha)
    s0, l0 = ct.cachetune_score_chunk(chunks, L, H, D, alpha=alpha, want_layers=True)
    s0b, _ = ct.cachetune_score_chunk(chunks, L, H, D, alpha=alpha)
    torch.cuda.synchronize()
    assert torch.equal(s0, s0b)
    ct.cachetune_prepare_scoring(ns, alpha)
    ws_after = ct.cachetune_score_chunk_ws(ns, L, H, D, alpha)
    assert ws_after < ws_before
    ct.cachetune_timing_read("twiddle")
    ct.cachetune_timing_enable(True)
    s1, l1 = ct.cachetune_score_chunk(chunks, L, H, D, alpha=alpha, want_layers=True)
    torch.cuda.synchronize()
    ct.cachetune_timing_enable(False)
    assert ct.cachetune_timing_read("twiddle")[1] == 0
    assert torch.equal(s0, s1) and torch.equal(l0, l1)
    # data within the fp16 range right after a call on data outside it (whose
    # tiles took the bf16 pass, which rounds differently): nothing carries
    # over, so this call equals the same call made after one on in-range data
    clean = _chunks(syn, ns, L, H, D, wide=False)
    c_a, _ = ct.cachetune_score_chunk(clean, L, H, D, alpha=alpha)
    c_b, _ = ct.cachetune_score_chunk(clean, L, H, D, alpha=alpha)
    torch.cuda.synchronize()
    assert torch.equal(c_a, c_b)
    assert torch.isfinite(c_a).all() and not torch.equal(c_a, s1)
