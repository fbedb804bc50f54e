"""GPU parity of the method's tie rules, on planted exact ties.

* Greedy argmax: the lowest index wins among equal logits.  Two rows of the
  LM head are set to the row that holds the oracle's maximum (that row itself
  is replaced by the row of the smallest logit), so the maximum appears at
  exactly two indices j1 < j2.  Identical rows give bitwise identical logits
  on both sides, so the oracle must answer j1 and so must the kernel.  The
  pairs are placed so that each level of the kernel's reduction decides the
  tie: inside one wave's two rows of an iteration (or one 1 KiB unit holding
  two rows), across one wave's iterations, across the waves of one CU (the
  lower index on the higher wave) and across the CUs' argmax slots.
* Mixture-of-experts router: identical router rows give identical logits,
  and the top-k takes the lower expert id on ties.

Expected tokens come from the oracle on the planted weights; the row layout
of the LM-head tiles (rows split evenly over 256 CUs, items dealt to the six
compute waves round-robin, two items per iteration) only chooses where the
ties are planted.
"""
import numpy as np
import pytest

from oracle import DecoderOracle
from persistent_megakernel_wg_amd import synth
from test_gpu_decode import TIGHT, _say, rel_l2

pytestmark = pytest.mark.gpu

N_CUS = 256
WAVES = 6


def _tile_rows(vocab, rpu, cu):
    """First row of the LM-head tile of `cu` (items split evenly over N_CUS)."""
    n = vocab // rpu
    return (n * cu // N_CUS) * rpu


def _cases(vocab, rpu):
    """(name, j1, j2) pairs, j1 < j2, one per level of the reduction."""
    r0 = _tile_rows(vocab, rpu, 10)
    if rpu == 1:
        # item t = row r0 + t; wave w takes t = w, w+6 (one iteration), w+12, ...
        return [("one iteration of one wave", r0 + 1, r0 + 1 + WAVES),
                ("two iterations of one wave", r0 + 2, r0 + 2 + 2 * WAVES),
                ("two waves, lower row on the higher wave", r0 + WAVES - 1, r0 + WAVES),
                ("two CUs", _tile_rows(vocab, rpu, 3) + 7, _tile_rows(vocab, rpu, 200) + 3)]
    # rpu == 2: item t = rows r0 + 2t (lanes 0-31) and r0 + 2t + 1 (lanes 32-63)
    return [("one unit (two half-wave rows)", r0 + 4, r0 + 5),
            ("two items of one wave", r0, r0 + 2 * WAVES),
            ("two waves, lower row on the higher wave", r0 + 2, r0 + 2 * WAVES),
            ("two CUs", _tile_rows(vocab, rpu, 3) + 1, _tile_rows(vocab, rpu, 250) + 9)]


def _argmax_ties(shape):
    import torch
    from persistent_megakernel_wg_amd import binding as B
    from persistent_megakernel_wg_amd.engine import Engine
    assert not shape.tied_embedding  # the LM head is edited, the embedding is not
    w = synth.make_weights(shape)
    kc, vc = synth.make_kv_cache(shape)
    tok = synth.make_tokens(shape)
    pos = shape.prefill
    base = w["lm_head"].copy()
    lg0, nx0 = DecoderOracle(shape, w, keep_f64=False).step(tok, pos, kc.copy(), vc.copy())
    r_max, r_min = int(nx0[0]), int(np.argmin(lg0[0]))
    rpu = 2 if shape.hidden == 256 else 1
    eng = Engine(shape, w, kc, vc, plan=B.plan_opts(n_cus=N_CUS))
    try:
        dev_lm = eng.tensors["lm_head"].view(torch.int16)
        for name, j1, j2 in _cases(shape.vocab, rpu):
            assert r_min not in (j1, j2)
            lm = base.copy()
            if r_max not in (j1, j2):
                lm[r_max] = base[r_min]
            lm[j1] = base[r_max]
            lm[j2] = base[r_max]
            w2 = dict(w)
            w2["lm_head"] = lm
            ref_lg, ref_nx = DecoderOracle(shape, w2, keep_f64=False).step(tok, pos, kc.copy(), vc.copy())
            _say("case %s ties %s: rows %d and %d (oracle max was row %d); oracle picks %d"
                 % (shape.name, name, j1, j2, r_max, ref_nx[0]))
            assert ref_lg[0][j1] == ref_lg[0][j2] == np.max(ref_lg[0])
            assert ref_nx[0] == j1
            dev_lm.copy_(torch.from_numpy(lm.view(np.int16)))
            eng.rebuild_plan(B.plan_opts(n_cus=N_CUS))
            lg, nx = eng.step(tok, pos)
            err = rel_l2(lg[0], ref_lg[0])
            _say("  device picks %d; logits %r %r; rel_l2 %.3e" % (nx[0], lg[0][j1], lg[0][j2], err))
            assert lg[0][j1] == lg[0][j2]
            assert err <= TIGHT
            assert nx[0] == j1, (name, nx[0], j1)
    finally:
        eng.close()


def test_argmax_ties_half_wave_rows(need_gpu):
    # the small decoder's 512 B rows: two rows per 1 KiB unit
    _argmax_ties(synth.SHAPES["tiny"].replace(tied_embedding=False))


@pytest.mark.timeout(600)
def test_argmax_ties_llama1b_rows(need_gpu):
    # the Llama-3.2-1B LM head (4 KiB rows), the headline kernel
    _argmax_ties(synth.SHAPES["llama1b_ctx128"].replace(tied_embedding=False))


@pytest.mark.parametrize("pattern", ["all_equal", "pairs_equal"])
def test_router_ties_take_lower_expert(need_gpu, pattern):
    from persistent_megakernel_wg_amd.engine import Engine
    s = synth.SHAPES["moe_tiny"]
    _say("case moe_tiny router ties: %s" % pattern)
    w = synth.make_weights(s)
    r = w["router"].copy()
    if pattern == "all_equal":
        r[:] = r[:, :1, :]                 # every expert's logit equal: top-k = 0..k-1
    else:
        r[:, 1::2, :] = r[:, 0::2, :]      # experts 2i and 2i+1 tie
    w["router"] = r
    kc, vc = synth.make_kv_cache(s)
    tok = synth.make_tokens(s)
    eng = Engine(s, w, kc, vc)
    try:
        lg, nx = eng.step(tok, s.prefill)
    finally:
        eng.close()
    tr = {}
    ref_lg, ref_nx = DecoderOracle(s, w).step(tok, s.prefill, kc.copy(), vc.copy(), trace=tr)
    ids = [list(map(int, e)) for e in tr["router_ids"]]
    _say("  oracle experts of sequence 0 per layer: %s" % ids)
    if pattern == "all_equal":
        assert all(e == list(range(s.top_k)) for e in ids)
    for b in range(s.batch):
        err = rel_l2(lg[b], ref_lg[b])
        _say("  seq %d: rel_l2 %.3e next %d / oracle %d" % (b, err, nx[b], ref_nx[b]))
        assert err <= TIGHT, (b, err)
        assert nx[b] == ref_nx[b], b
