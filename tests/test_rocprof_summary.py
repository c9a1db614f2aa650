"""Host logic of the profile summary tool (no GPU): the exact MFMA count it predicts for
the bf16 prefill kernel, which pins the meaning of the MFMA op counter."""
import math

import workloads as W
from exact_tiled_attention_08_amd.rocprof_summary import kernel_mfma_count


def _w(B, H, N, d, causal):
    return W.Workload(0, "t", B, H, N, N, d, W.torch.bfloat16, causal)


def test_noncausal_count_is_padded_tiles_times_both_products():
    # every wave sees every key tile: S and PV once per tile (the first S in the prologue,
    # the last PV alone in the final step)
    for d, bc in ((128, 96), (64, 128)):
        w = _w(2, 3, 512, d, False)
        nt = math.ceil(512 / bc)
        per_wave = nt * ((bc // 32) * (d // 16) + (d // 32) * (bc // 16))
        assert kernel_mfma_count(w) == 2 * 3 * 2 * 8 * per_wave


def test_causal_count_covers_the_causal_flops_and_is_at_most_noncausal():
    for N in (256, 1000, 8192):
        c = kernel_mfma_count(_w(1, 1, N, 128, True))
        n = kernel_mfma_count(_w(1, 1, N, 128, False))
        assert c <= n
        # causal work (2 products, 2 flop per MAC) over 32768 flop per MFMA, plus padding
        assert c * 32768 >= 4 * N * (N + 1) / 2 * 128


def test_ragged_rows_past_nq_issue_nothing():
    # N = 40: one workgroup, only wave 0 and wave 1 hold rows
    w = _w(1, 1, 40, 128, False)
    assert kernel_mfma_count(w) == 2 * (24 + 24)
