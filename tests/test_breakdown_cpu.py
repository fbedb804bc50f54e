"""CPU check of the trace breakdown's arithmetic on a hand-made trace."""
import numpy as np

from persistent_megakernel_wg_amd import breakdown as bd


def _put(tr, cu, i, hw0, layer, start, staged, end):
    tr[cu, i, bd.TR["HW0"]] = hw0
    tr[cu, i, bd.TR["HW1"]] = layer << 16
    tr[cu, i, bd.TR["START"]] = start & 0xFFFFFFFF
    tr[cu, i, bd.TR["STAGED"]] = staged & 0xFFFFFFFF
    tr[cu, i, bd.TR["SIGNAL"]] = end & 0xFFFFFFFF


def test_stage_spans_add_up_to_the_step():
    # two CUs, one layer: QKV (epi 0) then O (epi 1); stamps in 10 ns ticks
    # near the 32-bit wrap, to exercise the modular arithmetic
    base = 0xFFFFFF00
    tr = np.zeros((2, 2, 16), np.uint32)
    gemv = 1
    _put(tr, 0, 0, gemv | (0 << 8), 0, base, base + 100, base + 300)
    _put(tr, 1, 0, gemv | (0 << 8), 0, base + 10, base + 120, base + 400)
    _put(tr, 0, 1, gemv | (1 << 8), 0, (base + 300) & 0xFFFFFFFF, (base + 500) & 0xFFFFFFFF,
         (base + 700) & 0xFFFFFFFF)
    _put(tr, 1, 1, gemv | (1 << 8), 0, (base + 400) & 0xFFFFFFFF, (base + 520) & 0xFFFFFFFF,
         (base + 900) & 0xFFFFFFFF)
    res = bd.analyse(tr)
    assert abs(res["step_us"] - 9.0) < 1e-9
    q, o = res["by_stage"]["qkv"], res["by_stage"]["o"]
    # QKV: staged median 1.1 us from the start, last end 4.0 us
    assert abs(q["handover_us"] - 1.1) < 1e-9 and abs(q["work_us"] - 2.9) < 1e-9
    # O: staged median 5.1 us, previous stage ended at 4.0, last end 9.0
    assert abs(o["handover_us"] - 1.1) < 1e-9 and abs(o["work_us"] - 3.9) < 1e-9
    assert abs(sum(v["total_us"] for v in res["by_stage"].values()) - res["step_us"]) < 1e-9
    assert "| qkv |" in bd.report(res, "test")
