"""Full-size GPU parity: the workloads at their real shapes, in the launch
configuration bench.py times (default plan), against the CPU oracle."""
import numpy as np
import pytest

from oracle import DecoderOracle
from persistent_megakernel_wg_amd import synth
from test_gpu_decode import kv_rows_close

pytestmark = pytest.mark.gpu

TOL = 1e-2


def rel_l2(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / np.linalg.norm(b))


def _greedy_case(name, steps, keep_f64=True):
    from persistent_megakernel_wg_amd.engine import Engine
    s = synth.SHAPES[name]
    print("case %s: %d greedy steps from position %d" % (name, steps, s.prefill), flush=True)
    w = synth.make_weights(s)
    kc, vc = synth.make_kv_cache(s)
    tok = synth.make_tokens(s)
    eng = Engine(s, w, kc, vc)
    try:
        lgs, toks = eng.generate(tok, s.prefill, steps, logits=True)
        kg, vg = eng.read_kv()
    finally:
        eng.close()
    orc = DecoderOracle(s, w, keep_f64=keep_f64)
    k_ref, v_ref = kc.copy(), vc.copy()
    t = tok
    worst = 0.0
    for i in range(steps):
        ref_lg, ref_nx = orc.step(t, s.prefill + i, k_ref, v_ref)
        err = rel_l2(lgs[i][0], ref_lg[0])
        worst = max(worst, err)
        print("  step %d: rel_l2 %.3e token %d / oracle %d" % (i, err, toks[i][0], ref_nx[0]), flush=True)
        if toks[i][0] != ref_nx[0]:
            top = np.sort(ref_lg[0])[-2:]
            pytest.fail("step %d: token %d vs oracle %d (oracle top-2 margin %.3e)"
                        % (i, toks[i][0], ref_nx[0], top[1] - top[0]))
        assert err <= TOL, (i, err)
        t = ref_nx
    print("  worst rel_l2 %.3e" % worst, flush=True)
    # appended rows within one bf16 step; the rest of the cache untouched
    span = slice(s.prefill, s.prefill + steps)
    for got, ref in ((kg, k_ref), (vg, v_ref)):
        assert kv_rows_close(got[:, :, :, span], ref[:, :, :, span])
        assert np.array_equal(got[:, :, :, :s.prefill], ref[:, :, :, :s.prefill])


@pytest.mark.timeout(900)
def test_llama1b_ctx128_32_greedy_steps(need_gpu):
    _greedy_case("llama1b_ctx128", 32)


@pytest.mark.timeout(900)
def test_llama1b_ctx8192_4_steps(need_gpu):
    _greedy_case("llama1b_ctx8192", 4)


@pytest.mark.timeout(900)
def test_llama8b_ctx2048_1_step(need_gpu):
    _greedy_case("llama8b_ctx2048", 1, keep_f64=False)


@pytest.mark.timeout(1100)
def test_moe_b8_ctx2048_2_steps_sampled(need_gpu):
    """The batch-8 MoE shape at full size: two device-chained greedy steps,
    checked against the oracle on two of the eight sequences (the sequences
    of a step are independent, so each is a full check of its own outputs)."""
    from persistent_megakernel_wg_amd.engine import Engine
    s = synth.SHAPES["moe_b8_ctx2048"]
    steps, sample = 2, [0, 5]
    print("case %s: %d greedy steps from position %d, sequences %s checked"
          % (s.name, steps, s.prefill, sample), flush=True)
    w = synth.make_weights(s)
    kc, vc = synth.make_kv_cache(s)
    tok = synth.make_tokens(s)
    print("  inputs generated", flush=True)
    eng = Engine(s, w, kc, vc)
    try:
        lgs, toks = eng.generate(tok, s.prefill, steps, logits=True)
        kg, vg = eng.read_kv()
    finally:
        eng.close()
    print("  device steps done", flush=True)
    orc = DecoderOracle(s, w, keep_f64=False)
    k_ref, v_ref = kc.copy(), vc.copy()
    t = tok.copy()
    for i in range(steps):
        ref_lg, ref_nx = orc.step(t, s.prefill + i, k_ref, v_ref, seqs=sample)
        for b in sample:
            err = rel_l2(lgs[i][b], ref_lg[b])
            print("  step %d seq %d: rel_l2 %.3e token %d / oracle %d"
                  % (i, b, err, toks[i][b], ref_nx[b]), flush=True)
            assert err <= TOL, (i, b, err)
            assert toks[i][b] == ref_nx[b], (i, b)
        t = toks[i].copy()
    span = slice(s.prefill, s.prefill + steps)
    for got, ref in ((kg, k_ref), (vg, v_ref)):
        for b in sample:
            assert kv_rows_close(got[:, b, :, span], ref[:, b, :, span])
        assert np.array_equal(got[:, :, :, :s.prefill], ref[:, :, :, :s.prefill])
