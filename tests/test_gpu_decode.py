"""GPU parity of the megakernel decode step against the CPU oracle.

Bar (per step and sequence): logits within relative L2 error 1e-2 of the
oracle, the same greedy token, and appended K/V rows within one bf16 step.
Every case prints its name and shape first, so a failing run names it."""
import os

import numpy as np
import pytest

from oracle import DecoderOracle, bf16_to_f64
from persistent_megakernel_wg_amd import synth

pytestmark = pytest.mark.gpu

TOL = 1e-2       # contract
TIGHT = 1e-4     # fp32 accumulation over these sizes stays far below this


def rel_l2(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / np.linalg.norm(b))


def _engine(shape, w, kc, vc, **opts):
    from persistent_megakernel_wg_amd import binding as B
    from persistent_megakernel_wg_amd.engine import Engine
    return Engine(shape, w, kc, vc, plan=B.plan_opts(**opts) if opts else None)


def _say(msg):
    print(msg, flush=True)


def kv_rows_close(got_bits, ref_bits):
    """Appended rows agree within one bf16 step of the larger magnitude, plus
    a floor of TIGHT times the row's RMS.

    Both sides round the same pre-rounding value to bf16, but that value
    differs between the float32 path and the float64 oracle by the
    accumulated rounding of every earlier stage: an absolute error of the
    order of (relative error) * RMS of the row, since each element is a dot
    product whose rounding scales with the norms, not with the element.  Near
    zero or a rounding boundary that difference can exceed one step of the
    element.  The floor holds it to TIGHT, the relative error the logits are
    held to.  The worst excess over one step is printed for every call."""
    a, b = bf16_to_f64(got_bits), bf16_to_f64(ref_bits)
    big = np.maximum(np.abs(a), np.abs(b))
    step = np.exp2(np.floor(np.log2(np.maximum(big, 1e-30))) - 7)
    rms = np.sqrt(np.mean(b * b, axis=-1, keepdims=True))
    excess = (np.abs(a - b) - step) / rms
    bad = excess > TIGHT
    print("kv rows: worst excess over one bf16 step %.3e of the row RMS (floor %.0e); "
          "%d of %d beyond one step" % (float(np.max(excess)), TIGHT, int((excess > 0).sum()), excess.size),
          flush=True)
    return not bad.any()


def _check_kv(shape, kg, vg, k_ref, v_ref, pos):
    # appended rows within one bf16 step, every other row untouched
    for got, ref in ((kg, k_ref), (vg, v_ref)):
        assert kv_rows_close(got[:, :, :, pos], ref[:, :, :, pos])
        mask = np.ones(shape.max_seq, bool)
        mask[pos] = False
        assert np.array_equal(got[:, :, :, mask], ref[:, :, :, mask])


def _one_step_case(shape, pos=None, tok=None, **opts):
    _say("case %s pos=%s opts=%s" % (shape.name, pos, opts))
    w = synth.make_weights(shape)
    kc, vc = synth.make_kv_cache(shape, prefill=pos)
    tok = synth.make_tokens(shape) if tok is None else np.array([tok], np.int32)
    p = shape.prefill if pos is None else pos
    eng = _engine(shape, w, kc, vc, **opts)
    try:
        lg, nx = eng.step(tok, p)
        kg, vg = eng.read_kv()
    finally:
        eng.close()
    k_ref, v_ref = kc.copy(), vc.copy()
    ref_lg, ref_nx = DecoderOracle(shape, w).step(tok, p, k_ref, v_ref)
    err = rel_l2(lg[0], ref_lg[0])
    _say("  rel_l2 %.3e  next %d / oracle %d" % (err, nx[0], ref_nx[0]))
    assert err <= TOL and err <= TIGHT
    assert nx[0] == ref_nx[0]
    _check_kv(shape, kg, vg, k_ref, v_ref, p)


def test_tiny_step_default_plan(need_gpu):
    _one_step_case(synth.SHAPES["tiny"])


def test_tiny_step_split_attention(need_gpu):
    # two KV blocks per group: the last-arriving tile merges the partials
    _one_step_case(synth.SHAPES["tiny"], attn_block=64)


def test_tiny_step_few_cus_one_chunk(need_gpu):
    # several items per wave and per CU, single-chunk down projection
    _one_step_case(synth.SHAPES["tiny"], n_cus=7, mlp_chunks=1)


def test_tiny_step_two_chunks_odd_cus(need_gpu):
    _one_step_case(synth.SHAPES["tiny"], n_cus=37, mlp_chunks=2, attn_block=64)


def test_tiny_step_generic_kernel(need_gpu):
    # the kernel built for every shape, on the shape that has its own kernel
    _one_step_case(synth.SHAPES["tiny"], generic_kernel=1)
    _one_step_case(synth.SHAPES["tiny"], generic_kernel=1, attn_block=64, n_cus=37)


def test_tiny_step_four_chunks(need_gpu):
    # first / middle / last down-projection accumulations
    _one_step_case(synth.SHAPES["tiny"], mlp_chunks=4)


@pytest.mark.parametrize("n_cus", [1, 7, 256])
def test_tiny_gate_up_per_chunk_and_over_every_chunk(need_gpu, n_cus):
    # gate/up of every chunk in one instruction per CU (items chunk by chunk,
    # each written to its chunk's rows) against one instruction per chunk
    for chunks in (2, 4):
        _one_step_case(synth.SHAPES["tiny"], n_cus=n_cus, mlp_chunks=chunks, gu_all=1)
        _one_step_case(synth.SHAPES["tiny"], n_cus=n_cus, mlp_chunks=chunks, gu_all=-1)


@pytest.mark.parametrize("heads", [(4, 4, 64), (8, 2, 64), (8, 1, 64), (4, 2, 128), (4, 1, 128)])
def test_tiny_step_head_layouts(need_gpu, heads):
    # every attention code path: 1, 2, 4, 8 query heads per KV group, Dh 64/128
    h, g, dh = heads
    s = synth.SHAPES["tiny"].replace(n_q_heads=h, n_kv_heads=g, head_dim=dh)
    _one_step_case(s)                                  # one query head per tile
    _one_step_case(s, attn_block=64)                   # ... with split KV blocks
    _one_step_case(s, attn_heads=h // g)               # whole groups per tile
    _one_step_case(s, attn_heads=h // g, attn_block=64)


@pytest.mark.parametrize("block", [24, 40])
def test_tiny_position_blocks_of_eight_row_multiples(need_gpu, block):
    # blocks that are not multiples of 64 positions: block boundaries inside
    # a KV page, a last block holding the new position, 4 and 8 rows per unit
    for h, g, dh in ((4, 2, 64), (8, 2, 64), (4, 1, 128)):
        s = synth.SHAPES["tiny"].replace(n_q_heads=h, n_kv_heads=g, head_dim=dh)
        _one_step_case(s, attn_block=block)
        _one_step_case(s, attn_block=block, attn_heads=h // g)
        _one_step_case(s, attn_block=block, pos=block)  # the new row opens a block


@pytest.mark.parametrize("n_cus", [1, 3, 256])
def test_tiny_split_k_o_projection(need_gpu, n_cus):
    # O tiles per (row block, KV group), each waiting only for its group's
    # attention; the block's last ticket adds x and the partials in group
    # order (the first layer's residual is the embedding row); and the
    # whole-row O tiles of the same shape
    s = synth.SHAPES["tiny"].replace(n_q_heads=8)
    _one_step_case(s, n_cus=n_cus, o_split=1)
    _one_step_case(s, n_cus=n_cus, o_split=-1)
    _one_step_case(s.replace(head_dim=128, n_q_heads=4), n_cus=n_cus, o_split=1, attn_block=64)


def test_tiny_step_one_cu(need_gpu):
    # the whole decoder on one workgroup: split residual tiles, long queue
    _one_step_case(synth.SHAPES["tiny"], n_cus=1)


def test_tiny_empty_cache_position_zero(need_gpu):
    # attention over the single new row returns its value row
    _one_step_case(synth.SHAPES["tiny"], pos=0)


def test_tiny_last_position(need_gpu):
    s = synth.SHAPES["tiny"]
    _one_step_case(s, pos=s.max_seq - 1, attn_block=64)


def test_tiny_greedy_chain_on_device(need_gpu):
    from persistent_megakernel_wg_amd.engine import Engine
    s = synth.SHAPES["tiny"]
    _say("case tiny greedy 8 steps")
    w = synth.make_weights(s)
    kc, vc = synth.make_kv_cache(s)
    tok = synth.make_tokens(s)
    eng = Engine(s, w, kc, vc)
    try:
        lgs, toks = eng.generate(tok, s.prefill, 8, logits=True)
    finally:
        eng.close()
    orc = DecoderOracle(s, w)
    k_ref, v_ref = kc.copy(), vc.copy()
    t = tok
    for i in range(8):
        ref_lg, ref_nx = orc.step(t, s.prefill + i, k_ref, v_ref)
        assert rel_l2(lgs[i][0], ref_lg[0]) <= TIGHT
        assert toks[i][0] == ref_nx[0], (i, toks[i][0], ref_nx[0])
        t = ref_nx


def test_tiny_repeat_is_bitwise_deterministic(need_gpu):
    from persistent_megakernel_wg_amd.engine import Engine
    s = synth.SHAPES["tiny"]
    w = synth.make_weights(s)
    kc, vc = synth.make_kv_cache(s)
    tok = synth.make_tokens(s)
    eng = Engine(s, w, kc, vc)
    try:
        outs = [eng.step(tok, s.prefill)[0] for _ in range(5)]
    finally:
        eng.close()
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_cooperative_launch_matches_plain(need_gpu, monkeypatch):
    # MK_COOP=1 at context creation selects the cooperative launch; the
    # kernel and plan are the same, so the step is bitwise the same
    from persistent_megakernel_wg_amd.engine import Engine
    s = synth.SHAPES["tiny"]
    _say("case tiny cooperative vs plain launch")
    w = synth.make_weights(s)
    outs = []
    for coop in ("0", "1"):
        monkeypatch.setenv("MK_COOP", coop)
        kc, vc = synth.make_kv_cache(s)
        eng = Engine(s, w, kc, vc)
        try:
            outs.append(eng.step(synth.make_tokens(s), s.prefill))
        finally:
            eng.close()
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])


def test_abi_errors(need_gpu):
    from persistent_megakernel_wg_amd import binding as B
    from persistent_megakernel_wg_amd.engine import Engine
    s = synth.SHAPES["tiny"]
    w = synth.make_weights(s)
    kc, vc = synth.make_kv_cache(s)
    eng = Engine(s, w, kc, vc)
    try:
        with pytest.raises(B.MkError) as e:
            B.mk_decode_step(eng.ctx, eng.tokens.data_ptr(), s.max_seq, eng.next.data_ptr())
        assert e.value.status == -1
        with pytest.raises(B.MkError) as e:
            B.mk_decode_step(eng.ctx, 0, 3, eng.next.data_ptr())
        assert e.value.status == -1
    finally:
        eng.close()
    B.mk_destroy(None)


def test_watchdog_turns_a_stuck_wait_into_an_error(need_gpu):
    from persistent_megakernel_wg_amd import binding as B
    from persistent_megakernel_wg_amd.engine import Engine
    s = synth.SHAPES["tiny"]
    _say("case watchdog (one wait target raised by one)")
    w = synth.make_weights(s)
    kc, vc = synth.make_kv_cache(s)
    tok = synth.make_tokens(s)
    eng = Engine(s, w, kc, vc, plan=B.plan_opts(debug_corrupt_target=1, watchdog_ms=200))
    try:
        eng.tokens.copy_(eng.torch.from_numpy(tok))
        eng.launch(s.prefill)
        with pytest.raises(B.MkError) as e:
            eng.sync()
        assert e.value.status == -6
        # the context is usable again with a correct plan
        eng.rebuild_plan()
        _, nx = eng.step(tok, s.prefill)
        k_ref, v_ref = kc.copy(), vc.copy()
        _, ref_nx = DecoderOracle(s, w).step(tok, s.prefill, k_ref, v_ref)
        assert nx[0] == ref_nx[0]
    finally:
        eng.close()
