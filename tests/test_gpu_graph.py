"""HIP-graph replay and the two-stream schedule of the hot path.

* The step captured once (scoring, top-r, per layer assembly and attention,
  through the C ABI on torch's capture stream) and replayed several times,
  with eager work and synchronisations in between, gives bit-identical
  results to the eager step every time.
* The two-stream step (each layer's assembly on a side stream into one of
  two buffers, overlapping the previous layer's attention) gives the serial
  step's outputs bit for bit, eager and replayed.
* The assembly-only path (neighbouring layers' assemblies on two streams
  into two buffers) gives every layer's serial assembly bit for bit, eager
  and replayed."""
import math

import numpy as np
import pytest
import torch

from gpu_util import need_gpu, to_dev

pytestmark = pytest.mark.gpu
SEED = 20260611


def _request(ct, syn, L):
    """Inputs and buffers of a small two-chunk request (two assembled-cache
    buffers, one output per layer) and its calls."""
    ns, H, Hq, D, theta, n_sfx = [512, 300], 2, 8, 64, 500000.0, 16
    chunks = [(to_dev(syn.chunk(SEED, syn.K, b, L, n, H, D, "bf16")), to_dev(syn.chunk(SEED, syn.V, b, L, n, H, D, "bf16")))
              for b, n in enumerate(ns)]
    offs = [0, ns[0]]
    T_c = sum(ns)
    T = T_c + n_sfx
    ks = [(15 * n) // 100 for n in ns]
    score = torch.empty(T_c, dtype=torch.float32, device="cuda")
    sel = torch.empty(sum(ks), dtype=torch.int32, device="cuda")
    comp = torch.empty(T_c - sum(ks), dtype=torch.int32, device="cuda")
    ws = torch.empty(ct.cachetune_score_chunk_ws(ns, L, H, D, (1, 16)), dtype=torch.uint8, device="cuda")
    rec = [[(to_dev(syn.rows(SEED, syn.K, b, l, n, H, D, np.arange(ks[b]), "bf16")),
             to_dev(syn.rows(SEED, syn.V, b, l, n, H, D, np.arange(ks[b]), "bf16"))) for b, n in enumerate(ns)]
           for l in range(L)]
    sfx = [(to_dev(syn.rows(SEED, syn.K, syn.SUFFIX_CHUNK, l, n_sfx, H, D, np.arange(n_sfx), "bf16")),
            to_dev(syn.rows(SEED, syn.V, syn.SUFFIX_CHUNK, l, n_sfx, H, D, np.arange(n_sfx), "bf16"))) for l in range(L)]
    n_q = 40
    qpos = to_dev(np.sort(np.random.default_rng(1).choice(T, n_q, replace=False)).astype(np.int32))
    q = [to_dev(syn.rows(SEED, syn.Q, 0, l, T, Hq, D, np.arange(n_q), "bf16")) for l in range(L)]
    asm = [(torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda"),
            torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")) for _ in range(2)]
    out = [torch.empty((n_q, Hq, D), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    attn_ws = torch.empty(max(256, ct.cachetune_recompute_attn_ws(n_q, Hq, T, H, D)), dtype=torch.uint8,
                          device="cuda")
    so, co = [0, ks[0]], [0, ns[0] - ks[0]]
    places = [[ct.make_place(chunks[b][0][l], chunks[b][1][l], n, ks[b], offs[b], sel=sel[so[b]:],
                             comp=comp[co[b]:], k_rec=rec[l][b][0], v_rec=rec[l][b][1])
               for b, n in enumerate(ns)] for l in range(L)]

    def select():
        ct.cachetune_score_chunk(chunks, L, H, D, score=score, ws=ws)
        ct.cachetune_select_topr(score, ns, r=(15, 100), sel=sel, comp=comp, want_ranking=False)

    def assemble(l, b):
        ct.cachetune_assemble_rope(places[l], asm[b][0], asm[b][1], H, D, theta, k_sfx=sfx[l][0],
                                   v_sfx=sfx[l][1], n_sfx=n_sfx, sfx_offset=T_c)

    # the places hold raw device pointers: the tensors they point into must
    # live as long as the calls (a captured graph replays them later)
    assemble.sources = (chunks, rec, sel, comp)

    def attend(l, b):
        ct.cachetune_recompute_attn(q[l], qpos, asm[b][0], asm[b][1], 1.0 / math.sqrt(D), theta, out=out[l],
                                    ws=attn_ws)

    return score, sel, comp, asm, out, select, assemble, attend


def _replays_match(step, outputs, clobber):
    """Capture ``step`` in a HIP graph on a side stream, replay it three
    times with the outputs clobbered by eager work in between, and compare
    every replay with the eager step's outputs."""
    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in outputs]
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        step()
    for rep in range(3):
        for t in clobber:  # clobber the outputs with eager work between replays
            t.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outputs, want)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager step"
    return want


def test_step_graph_replays_match_eager(syn):
    ct = need_gpu()
    L = 2
    score, sel, comp, asm, out, select, assemble, attend = _request(ct, syn, L)

    def step():
        select()
        for l in range(L):
            assemble(l, 0)
            attend(l, 0)

    _replays_match(step, (score, sel, comp, *asm[0], *out), (score, *asm[0], *out))


def test_two_stream_step_matches_serial(syn):
    """The two-stream schedule (each layer's assembly on a side stream into
    one of two buffers, the attention on the current stream) gives the
    serial step's per-layer outputs bit for bit, eager and replayed from a
    HIP graph."""
    from non_prefix_kv_token_amd.schedule import run_layers

    ct = need_gpu()
    L = 5  # both buffers reused more than once
    score, sel, comp, asm, out, select, assemble, attend = _request(ct, syn, L)

    select()
    for l in range(L):
        assemble(l, 0)
        attend(l, 0)
    torch.cuda.synchronize()
    want = [t.clone() for t in out]
    for t in (*asm[0], *asm[1], *out):
        t.fill_(-1)
    side = torch.cuda.Stream()

    def step():
        select()
        run_layers(L, assemble, attend, side)

    got = _replays_match(step, out, (*asm[0], *asm[1], *out))
    for l in range(L):
        assert torch.equal(got[l], want[l]), f"layer {l}: two-stream output differs from the serial step"


@pytest.mark.parametrize("L", [1, 4, 5])
def test_two_stream_assemblies_match_serial(syn, L):
    """``run_assemblies`` (even layers on the current stream into buffer 0,
    odd ones on a side stream into buffer 1): after the step each buffer
    holds the last layer assembled into it, equal bit for bit to that
    layer's serial assembly, eager and replayed from a HIP graph."""
    from non_prefix_kv_token_amd.schedule import run_assemblies

    ct = need_gpu()
    score, sel, comp, asm, out, select, assemble, attend = _request(ct, syn, L)
    select()
    want = {}
    for l in range(L):
        assemble(l, 0)
        torch.cuda.synchronize()
        want[l % 2] = (asm[0][0].clone(), asm[0][1].clone())  # the last layer of each parity
    for t in (*asm[0], *asm[1]):
        t.fill_(-1)
    side = torch.cuda.Stream()

    def step():
        select()
        run_assemblies(L, assemble, side)

    bufs = [t for b in range(min(L, 2)) for t in asm[b]]
    got = _replays_match(step, bufs, bufs)
    for b in range(min(L, 2)):
        assert torch.equal(got[2 * b], want[b][0]) and torch.equal(got[2 * b + 1], want[b][1]), \
            f"buffer {b}: two-stream assembly differs from the serial one"
