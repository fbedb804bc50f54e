"""Multi-step resident decode (mk_decode_steps): N greedy steps in one launch.

Bar: bitwise equal to N single-step launches chained on the device (the same
kernels and plan; the step boundary only moves inside the kernel): tokens,
logits of every step and the appended K/V rows; and token-identical to the
oracle's greedy sequence.  Cases cover the short-context plan, split
attention (the merge tickets and partials are reused by every step of the
launch), one CU (the whole launch on one workgroup), the mixture-of-experts
decoder (one launch per step) and the argument checks."""
import numpy as np
import pytest

from oracle import DecoderOracle, greedy_decode
from persistent_megakernel_wg_amd import synth
from test_gpu_decode import TIGHT, _say, rel_l2

pytestmark = pytest.mark.gpu


def _engine(shape, w, kc, vc, **opts):
    from persistent_megakernel_wg_amd import binding as B
    from persistent_megakernel_wg_amd.engine import Engine
    return Engine(shape, w, kc, vc, plan=B.plan_opts(**opts) if opts else None)


def _reset_kv(eng, kc, vc):
    i16 = eng.torch.int16
    eng.k_cache.view(i16).copy_(eng.torch.from_numpy(kc.view(np.int16)))
    eng.v_cache.view(i16).copy_(eng.torch.from_numpy(vc.view(np.int16)))


def _resident_case(shape, steps, oracle_check=True, **opts):
    _say("case %s: %d steps in one launch from position %d, opts %s" % (shape.name, steps, shape.prefill, opts))
    w = synth.make_weights(shape)
    kc, vc = synth.make_kv_cache(shape)
    tok = synth.make_tokens(shape)
    eng = _engine(shape, w, kc, vc, **opts)
    try:
        lg1, tk1 = eng.generate(tok, shape.prefill, steps, logits=True)
        kv1 = eng.read_kv()
        _reset_kv(eng, kc, vc)
        lg2, tk2 = eng.generate_resident(tok, shape.prefill, steps, logits=True)
        kv2 = eng.read_kv()
    finally:
        eng.close()
    for s in range(steps):
        assert np.array_equal(tk2[s], tk1[s]), (s, tk2[s], tk1[s])
        assert np.array_equal(lg2[s], lg1[s]), s
    assert np.array_equal(kv2[0], kv1[0]) and np.array_equal(kv2[1], kv1[1])
    _say("  bitwise equal to %d chained single-step launches; tokens %s" % (steps, [int(t[0]) for t in tk2]))
    if oracle_check:
        _, ref = greedy_decode(shape, w, kc.copy(), vc.copy(), tok, shape.prefill, steps,
                               oracle=DecoderOracle(shape, w))
        for s in range(steps):
            assert np.array_equal(tk2[s], ref[s]), (s, tk2[s], ref[s])
        _say("  token-identical to the oracle's greedy sequence")


def test_resident_tiny_8_steps(need_gpu):
    _resident_case(synth.SHAPES["tiny"], 8)


def test_resident_tiny_split_attention(need_gpu):
    _resident_case(synth.SHAPES["tiny"], 6, attn_block=64)


def test_resident_tiny_one_cu(need_gpu):
    _resident_case(synth.SHAPES["tiny"], 4, n_cus=1)


def test_resident_tiny_to_the_last_position(need_gpu):
    # the launch's last step writes the cache's last row
    s = synth.SHAPES["tiny"]
    _resident_case(s.replace(prefill=s.max_seq - 5), 5, attn_block=64)


def test_resident_split_k_o_projection(need_gpu):
    # the O row blocks' tickets and partials are reused by every step
    s = synth.SHAPES["tiny"].replace(n_q_heads=8)
    _resident_case(s, 6, o_split=1)
    _resident_case(s, 4, o_split=1, n_cus=3)


def test_resident_moe_tiny(need_gpu):
    _resident_case(synth.SHAPES["moe_tiny"], 3)


@pytest.mark.timeout(600)
def test_resident_llama1b_ctx128_32_steps(need_gpu):
    # the headline shape: 32 steps in one launch against 32 launches
    _resident_case(synth.SHAPES["llama1b_ctx128"], 32, oracle_check=True)


def test_resident_moe_tiny_ready_queue(need_gpu):
    # the down projection's ready-queue counters alternate between steps:
    # each step's expert sums clear the next step's
    _resident_case(synth.SHAPES["moe_tiny"], 4, edn_queue=2)
    _resident_case(synth.SHAPES["moe_tiny"], 3, edn_queue=4, n_cus=3, egu_balance=-1)


def test_resident_argument_checks(need_gpu):
    from persistent_megakernel_wg_amd import binding as B
    s = synth.SHAPES["tiny"]
    w = synth.make_weights(s)
    kc, vc = synth.make_kv_cache(s)
    eng = _engine(s, w, kc, vc)
    try:
        out = eng.torch.zeros(4, dtype=eng.torch.int32, device=eng.dev)
        for pos, n in ((s.max_seq - 2, 3), (0, 0), (-1, 1)):
            with pytest.raises(B.MkError) as e:
                B.mk_decode_steps(eng.ctx, eng.tokens.data_ptr(), pos, n, out.data_ptr())
            assert e.value.status == -1
    finally:
        eng.close()
