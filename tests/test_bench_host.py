"""Host arithmetic of bench.py's reported work figures (no GPU).

The band projection's issued matrix-core work per step follows the kernel's
per-block dispatch: 64-bin blocks take the radix-4 pass (36 MFMAs per 64
tokens per 64-channel wave) where the transform length is a multiple of 128,
else the folded pass (48 per 32 folded columns), and a block with at most 32
bins left runs unfolded (8 per 16 tokens, padded to 32).  At the 8 x 2048
Llama-3-8B shapes the count is checked against the hardware: rocprofv3's
SQ_INSTS_MFMA for one k_band_bf16<2> dispatch there reads 9.437e6
(profiles/counters_stalls_band_gram_assembly_llama3-8b-8x2048.md)."""
import types

import bench

FLOPS_PER_MFMA = 32 * 32 * 16 * 2


def _flops(ns, L, H, D, alpha, dtype="bf16"):
    w = types.SimpleNamespace(ns=list(ns), L=L, H=H, D=D, alpha=alpha, dtype=dtype)
    return bench.Workload.band_mfma_flops(w)


def test_band_mfma_count_matches_the_counter_at_8x2048():
    flops = _flops([2048] * 8, 32, 8, 128, (1, 16))
    mfmas = flops / FLOPS_PER_MFMA
    assert mfmas == 9_437_184  # 512 problems x 2 channel blocks x 8 waves x 32 k-steps x 36
    assert abs(mfmas - 9.437e6) / 9.437e6 < 1e-3


def test_band_mfma_count_per_pass():
    # one layer, K and V, 64 channels (one wave per block)
    per_kv = lambda ns, alpha: _flops(ns, 1, 1, 64, alpha) / FLOPS_PER_MFMA / 2
    # 1024 tokens, 64 bins: one radix-4 block, 36 x 1024 / 64
    assert per_kv([1024], (1, 8)) == 576
    # 700 tokens, 43 bins: one folded block, 48 x ceil(350 / 32)
    assert per_kv([700, 1024], (1, 8)) == 576 + 48 * 11
    # 300 tokens (320 padded), 18 bins in a launch of 64-bin blocks: one 32-bin block
    assert per_kv([300, 1024], (1, 8)) == 576 + 8 * 320 // 16
    # 1152 tokens, 144 bins: two radix-4 blocks and a 16-bin block
    assert per_kv([1152], (1, 4)) == 2 * 36 * 1152 // 64 + 8 * 1152 // 16
    # every chunk at most 32 bins: 32-bin blocks throughout
    assert per_kv([512, 600], (1, 16)) == 8 * 512 // 16 + 8 * 608 // 16
