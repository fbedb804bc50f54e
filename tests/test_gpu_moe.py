"""GPU parity of the batched megakernel (the parallel-block mixture-of-experts
decoder, B sequences per step) against the CPU oracle.

Bar, per step and per sequence: logits within relative L2 error 1e-2 of the
oracle (and within 1e-4: the fp32 path stays far below the contract here),
the same greedy token, appended K/V rows within one bf16 step, every other
cache row untouched.  Every case prints its name, shape and plan options first.
"""
import numpy as np
import pytest

from oracle import DecoderOracle
from persistent_megakernel_wg_amd import synth
from test_gpu_decode import TIGHT, TOL, _check_kv, _say, rel_l2

pytestmark = pytest.mark.gpu

TINY = synth.SHAPES["moe_tiny"]


def _engine(shape, w, kc, vc, **opts):
    from persistent_megakernel_wg_amd import binding as B
    from persistent_megakernel_wg_amd.engine import Engine
    return Engine(shape, w, kc, vc, plan=B.plan_opts(**opts) if opts else None)


def _moe_case(shape, pos=None, **opts):
    _say("case %s B=%d E=%d k=%d Fe=%d H=%d G=%d Dh=%d pos=%s opts=%s"
         % (shape.name, shape.batch, shape.n_experts, shape.top_k, shape.expert_ffn,
            shape.n_q_heads, shape.n_kv_heads, shape.head_dim, pos, opts))
    w = synth.make_weights(shape)
    kc, vc = synth.make_kv_cache(shape, prefill=pos)
    tok = synth.make_tokens(shape)
    p = shape.prefill if pos is None else pos
    eng = _engine(shape, w, kc, vc, **opts)
    try:
        lg, nx = eng.step(tok, p)
        kg, vg = eng.read_kv()
        info = eng.plan_info()
    finally:
        eng.close()
    _say("  plan: %d instructions, kernel %d" % (info["n_instr"], info["kernel_variant"]))
    k_ref, v_ref = kc.copy(), vc.copy()
    tr = {}
    ref_lg, ref_nx = DecoderOracle(shape, w).step(tok, p, k_ref, v_ref, trace=tr)
    _say("  sequence 0 experts per layer: %s" % [list(map(int, e)) for e in tr["router_ids"]])
    for b in range(shape.batch):
        err = rel_l2(lg[b], ref_lg[b])
        _say("  seq %d: rel_l2 %.3e next %d / oracle %d" % (b, err, nx[b], ref_nx[b]))
        assert err <= TOL and err <= TIGHT, (b, err)
        assert nx[b] == ref_nx[b], b
    _check_kv(shape, kg, vg, k_ref, v_ref, p)


def test_moe_tiny_default_plan(need_gpu):
    _moe_case(TINY)


def test_moe_tiny_split_attention_few_cus(need_gpu):
    # two KV blocks per (sequence, group): the last-arriving tile merges
    _moe_case(TINY, n_cus=16, attn_block=64)


def test_moe_tiny_three_cus(need_gpu):
    # long queues: several expert gate/up and down instructions per CU and layer
    _moe_case(TINY, n_cus=3)


def test_moe_tiny_one_cu(need_gpu):
    _moe_case(TINY, n_cus=1, attn_block=64)


@pytest.mark.parametrize("batch", [1, 3, 5])
def test_moe_tiny_ragged_batch(need_gpu, batch):
    _moe_case(TINY.replace(batch=batch))


@pytest.mark.parametrize("top_k", [1, 8])
def test_moe_tiny_top_k(need_gpu, top_k):
    # one expert per token; every expert for every token (k = E)
    _moe_case(TINY.replace(top_k=top_k))


def test_moe_tiny_staging_groups(need_gpu):
    # wide experts: the routed intermediates of a layer need several
    # staging groups in the down projection
    _moe_case(TINY.replace(expert_ffn=2048, top_k=4, n_experts=16))


def test_moe_tiny_generic_attention(need_gpu):
    # the batched kernel with per-instruction attention dispatch: one query
    # head per tile, and a head_dim 64 layout
    _moe_case(TINY, attn_heads=1)
    _moe_case(TINY.replace(n_q_heads=8, n_kv_heads=1, head_dim=64))
    _moe_case(TINY.replace(n_q_heads=8, n_kv_heads=1, head_dim=64), attn_block=64)


def test_moe_tiny_position_zero_and_last(need_gpu):
    _moe_case(TINY, pos=0)
    _moe_case(TINY, pos=TINY.max_seq - 1, attn_block=64)


@pytest.mark.parametrize("kw,opts", [({}, {}), ({"batch": 3}, {}), ({"batch": 1}, {}),
                                     ({}, {"n_cus": 1, "attn_block": 64}), ({}, {"n_cus": 37})])
def test_moe_tiny_matrix_core_lm_head(need_gpu, kw, opts):
    # the LM head as v_mfma_f32_16x16x32_bf16 tiles of 16 rows (the input as
    # bf16 high + low parts, fp32 accumulation): padded row blocks, ragged
    # batches, one CU (16 blocks through one workgroup) and odd CU counts
    _moe_case(TINY.replace(**kw), mfma=1, **opts)


@pytest.mark.parametrize("queue,opts", [(2, {}), (2, {"n_cus": 1, "attn_block": 64}), (4, {"n_cus": 3}),
                                        (1, {"n_cus": 3}), (1, {"n_cus": 37}), (-1, {}), (-1, {"n_cus": 37})])
def test_moe_tiny_ready_queue(need_gpu, queue, opts):
    # the expert down projection with a 1/queue share of its units handed out
    # at run time (chunks to whichever CU asks first), and with none
    _moe_case(TINY, edn_queue=queue, **opts)
    _moe_case(TINY.replace(expert_ffn=2048, top_k=4, n_experts=16), edn_queue=queue, **opts)


@pytest.mark.parametrize("balance,opts", [(1, {}), (-1, {}), (1, {"n_cus": 1, "attn_block": 64}),
                                          (1, {"n_cus": 3}), (-1, {"n_cus": 3}), (1, {"n_cus": 37, "edn_queue": -1})])
def test_moe_tiny_gate_up_shares(need_gpu, balance, opts):
    # gate/up items as weighted shares of the layer's (expert, row) items
    # (share boundaries inside an expert, CUs with no items) and as even row
    # slices of every expert
    _moe_case(TINY, egu_balance=balance, **opts)
    _moe_case(TINY.replace(expert_ffn=2048, top_k=4, n_experts=16), egu_balance=balance, **opts)
    _moe_case(TINY.replace(batch=1, top_k=1), egu_balance=balance, **opts)


def test_moe_tiny_greedy_chain_on_device(need_gpu):
    from persistent_megakernel_wg_amd.engine import Engine
    s = TINY
    steps = 6
    _say("case moe_tiny greedy %d steps" % steps)
    w = synth.make_weights(s)
    kc, vc = synth.make_kv_cache(s)
    tok = synth.make_tokens(s)
    eng = Engine(s, w, kc, vc)
    try:
        lgs, toks = eng.generate(tok, s.prefill, steps, logits=True)
    finally:
        eng.close()
    orc = DecoderOracle(s, w)
    k_ref, v_ref = kc.copy(), vc.copy()
    t = tok
    for i in range(steps):
        ref_lg, ref_nx = orc.step(t, s.prefill + i, k_ref, v_ref)
        for b in range(s.batch):
            assert rel_l2(lgs[i][b], ref_lg[b]) <= TIGHT, (i, b)
        assert np.array_equal(toks[i], ref_nx), (i, toks[i], ref_nx)
        t = ref_nx


def test_moe_tiny_repeat_is_bitwise_deterministic(need_gpu):
    from persistent_megakernel_wg_amd.engine import Engine
    s = TINY
    w = synth.make_weights(s)
    kc, vc = synth.make_kv_cache(s)
    tok = synth.make_tokens(s)
    eng = Engine(s, w, kc, vc)
    try:
        outs = [eng.step(tok, s.prefill)[0] for _ in range(4)]
    finally:
        eng.close()
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
