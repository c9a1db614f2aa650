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


def test_after_marker_keeps_the_timed_dispatches(tmp_path):
    """A synthetic kernel-trace database: warm-up launches, a one-workgroup marker, the timed
    launches, then more launches of the same kernel (a later measurement); --after-marker
    0:3 keeps exactly the three timed ones."""
    import sqlite3
    from exact_tiled_attention_08_amd.rocprof_summary import summarise
    db = str(tmp_path / "t.db")
    con = sqlite3.connect(db)
    con.execute("create table kernels (name text, duration int, grid_x int, workgroup_x int, "
                "lds_size int, vgpr_count int, accum_vgpr_count int, dispatch_id int)")
    k = "void fa::(anonymous namespace)::fwd_bf16_kernel<128, 96, true, false, false>(fa::FwdParams)"
    m = "fa::(anonymous namespace)::mfma_probe_kernel(float*, int)"
    rows = [(k, 900, 512 * 1024, 512, 0, 0, 0, i) for i in range(5)]            # warm-up
    rows += [(m, 10, 256, 256, 0, 0, 0, 5)]                                     # marker
    rows += [(k, 500 + i, 512 * 1024, 512, 0, 0, 0, 6 + i) for i in range(3)]   # timed
    rows += [(m, 99, 256 * 2048, 256, 0, 0, 0, 9)]                              # a big probe
    rows += [(k, 700, 512 * 1024, 512, 0, 0, 0, 10 + i) for i in range(4)]      # later use
    rows += [(m, 10, 256, 256, 0, 0, 0, 14)]                                    # next leg
    rows += [("fa::other_kernel", 5, 256, 256, 0, 0, 0, 15)]
    con.executemany("insert into kernels values (?,?,?,?,?,?,?,?)", rows)
    con.commit()
    con.close()
    by, _ = summarise([db], "fwd_bf16", after=(0, 3))
    (ent,) = by.values()
    assert ent["d"] == [500, 501, 502]
    # a kernel that only the next leg launches is not part of this leg's window
    by, _ = summarise([db], "fa::", after=(0, 3))
    assert all("other_kernel" not in name for name, _ in by)
    by, _ = summarise([db], "other_kernel", after=(1, 3))
    assert [e["d"] for e in by.values()] == [[5]]
