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


def test_check_indices_counts_broken_entries():
    """cachetune_check_indices reads an index array without trusting it: the
    selection's own arrays pass, and planted entries (out of range, negative,
    repeated, descending) are each counted once; values are never followed."""
    ct = need_gpu()
    import numpy as np
    n_per_chunk = [300, 2048, 7]
    g = torch.Generator(device="cuda").manual_seed(5)
    score = torch.rand(sum(n_per_chunk), generator=g, device="cuda", dtype=torch.float32)
    k, ranking, sel, comp = ct.cachetune_select_topr(score, n_per_chunk, r=(15, 100))
    # each chunk's lists are ascending local indices below its length
    assert ct.cachetune_check_indices(ranking[:300], 300, ascending=False) == 0
    o_s = o_c = 0
    for n, kb in zip(n_per_chunk, k):
        assert ct.cachetune_check_indices(sel[o_s:o_s + kb], n) == 0
        assert ct.cachetune_check_indices(comp[o_c:o_c + n - kb], n) == 0
        o_s += kb
        o_c += n - kb
    idx = torch.tensor([0, 3, 5, 5, 12, -1, 7, 2, 9], dtype=torch.int32, device="cuda")
    # ascending: 5 (repeat), 12 (>= 10), -1 (< 0), 2 (below 7) -> 4
    assert ct.cachetune_check_indices(idx, 10) == 4
    # range only: 12 and -1
    assert ct.cachetune_check_indices(idx, 10, ascending=False) == 2
    assert ct.cachetune_check_indices(idx[:0], 10) == 0
    # a long array across many blocks: every 1000th entry out of range
    big = torch.arange(300_000, dtype=torch.int32, device="cuda")
    big[::1000] = 400_000
    want = int(np.count_nonzero(np.arange(300_000) % 1000 == 0))
    assert ct.cachetune_check_indices(big, 300_000, ascending=False) == want
