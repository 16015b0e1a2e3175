"""The attention entry point that allocates nothing
(cachetune_recompute_attn_noalloc), for callers that cannot allocate: its
workspace is the library's own per-device scratch array.  Its outputs must
equal those of cachetune_recompute_attn with a caller-allocated workspace,
bit for bit (same kernels, same arithmetic), on two calls in a row -- the
second with smaller shapes, so that it runs on what the first left in the
shared scratch -- and shapes whose workspace exceeds the scratch are refused
with an error before any work is enqueued."""
import numpy as np
import pytest
import torch

from gpu_util import need_gpu, to_dev

pytestmark = pytest.mark.gpu

SEED = 20260600


def _case(syn, T, H, Hq, D, n_q, seed_off):
    rng = np.random.default_rng(seed_off)
    k = syn.rows(SEED + seed_off, syn.K, 0, 1, T, H, D, np.arange(T), "bf16")
    v = syn.rows(SEED + seed_off, syn.V, 0, 1, T, H, D, np.arange(T), "bf16")
    qpos = np.sort(rng.choice(T, n_q, replace=False)).astype(np.int32)
    q = syn.rows(SEED + seed_off, syn.Q, 0, 1, T, Hq, D, qpos, "bf16")
    return to_dev(q), to_dev(qpos), to_dev(k), to_dev(v)


def test_noalloc_matches_workspace_call_twice(syn):
    ct = need_gpu()
    import ctypes
    # first call: keys split over several segments (partials + merge); second:
    # fewer rows, shorter context, one segment, another head dim
    cases = [(9000, 8, 32, 128, 700, 1), (1500, 2, 8, 64, 90, 2)]
    for T, H, Hq, D, n_q, so in cases:
        q, qpos, k, v = _case(syn, T, H, Hq, D, n_q, so)
        ref, ref_lse = ct.cachetune_recompute_attn(q, qpos, k, v, 1.0 / np.sqrt(D), 500000.0, want_lse=True)
        out = torch.full_like(ref, float("nan"))
        lse = torch.full_like(ref_lse, float("nan"))
        ct.cachetune_recompute_attn_noalloc(q, qpos, k, v, 1.0 / np.sqrt(D), 500000.0, out, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (T, H, Hq, D, n_q)
        assert torch.equal(lse, ref_lse), (T, H, Hq, D, n_q)
    # shapes above the scratch are refused, with the output untouched
    need = ct.cachetune_recompute_attn_ws(20573, 32, 136643, 8, 128)
    assert need > 256 << 20
    qb = torch.zeros((1, 32, 128), dtype=torch.bfloat16, device="cuda")
    kb = torch.zeros((2, 8, 128), dtype=torch.bfloat16, device="cuda")
    lib = ct.lib()
    st = lib.cachetune_recompute_attn_noalloc(ct.handle(), ctypes.c_void_p(qb.data_ptr()), ctypes.c_void_p(qpos.data_ptr()), 20573,
                                              32, ctypes.c_void_p(kb.data_ptr()), ctypes.c_void_p(kb.data_ptr()), 136643,
                                              8, 128, ct.CT_BF16, 0.088, 500000.0, 0, ctypes.c_void_p(qb.data_ptr()),
                                              None, None)
    assert st == ct.CT_E_WORKSPACE
    assert b"no-alloc" in lib.cachetune_last_error()
