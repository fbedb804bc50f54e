"""mk_decode_step_noalloc (the step with its scratch in the fixed per-GPU
array) against mk_decode_step (the context's own arena), through the C ABI.

Two no-allocation calls run back to back on one stream: first the batch-8
mixture-of-experts decoder (the larger scratch), then the small dense decoder
at an earlier position (a smaller input), so the second call starts from the
array as the first left it.  Each must match what mk_decode_step returned for
the same context and input: the same tokens, logits within TIGHT (the kernels
and plans are the same, so they are expected to be bitwise equal, which is
printed), the same appended K/V rows.
"""
import numpy as np
import pytest

from persistent_megakernel_wg_amd import synth
from test_gpu_decode import TIGHT, _say, rel_l2

pytestmark = pytest.mark.gpu


def _ctx(name, **kw):
    from persistent_megakernel_wg_amd.engine import Engine
    s = synth.SHAPES[name].replace(**kw)
    w = synth.make_weights(s)
    kc, vc = synth.make_kv_cache(s)
    eng = Engine(s, w, kc, vc)
    eng.tokens.copy_(eng.torch.from_numpy(synth.make_tokens(s)))
    return eng


def test_noalloc_matches_decode_step_on_two_calls(need_gpu):
    import torch
    from persistent_megakernel_wg_amd import binding as B
    cases = [("moe_tiny", 64), ("tiny", 40)]
    engs = [_ctx(n) for n, _ in cases]
    try:
        ref = []
        for eng, (name, pos) in zip(engs, cases):
            info = eng.plan_info()
            _say("case %s pos %d: scratch %d bytes" % (name, pos, info["scratch_bytes"]))
            assert 0 < info["scratch_bytes"] <= B.NOALLOC_SCRATCH_BYTES
            B.mk_decode_step(eng.ctx, eng.tokens.data_ptr(), pos, eng.next.data_ptr(),
                             eng.logits.data_ptr(), torch.cuda.current_stream().cuda_stream)
            B.mk_sync(eng.ctx)
            ref.append((eng.logits.cpu().numpy().copy(), eng.next.cpu().numpy().copy(), eng.read_kv()))
        assert ref[0][1].size > ref[1][1].size  # the second input is the smaller one
        outs = []
        stream = torch.cuda.current_stream().cuda_stream
        for eng, (name, pos) in zip(engs, cases):
            eng.logits.zero_()
            eng.next.fill_(-1)
        for eng, (name, pos) in zip(engs, cases):
            B.mk_decode_step_noalloc(eng.ctx, eng.tokens.data_ptr(), pos, eng.next.data_ptr(),
                                     eng.logits.data_ptr(), stream)
        for eng in engs:
            B.mk_sync(eng.ctx)
            outs.append((eng.logits.cpu().numpy().copy(), eng.next.cpu().numpy().copy(), eng.read_kv()))
        for (name, pos), (lg0, nx0, kv0), (lg1, nx1, kv1) in zip(cases, ref, outs):
            errs = [rel_l2(lg1[b], lg0[b]) for b in range(lg0.shape[0])]
            _say("  %s: tokens %s / %s, worst rel_l2 %.3e, bitwise equal: %s"
                 % (name, nx1.tolist(), nx0.tolist(), max(errs), bool(np.array_equal(lg1, lg0))))
            assert np.array_equal(nx1, nx0)
            assert max(errs) <= TIGHT
            assert np.array_equal(kv1[0], kv0[0]) and np.array_equal(kv1[1], kv0[1])
    finally:
        for eng in engs:
            eng.close()


def test_noalloc_rejects_a_plan_beyond_the_array(need_gpu):
    from persistent_megakernel_wg_amd import binding as B
    # 1024 attention blocks per (sequence, KV group): the split partials
    # alone exceed the array
    eng = _ctx("moe_tiny", max_seq=131072)
    try:
        need = eng.plan_info()["scratch_bytes"]
        _say("case moe_tiny max_seq 131072: scratch %d bytes" % need)
        assert need > B.NOALLOC_SCRATCH_BYTES
        with pytest.raises(B.MkError) as e:
            B.mk_decode_step_noalloc(eng.ctx, eng.tokens.data_ptr(), 64, eng.next.data_ptr())
        assert e.value.status == -4 and "limit" in str(e.value)
    finally:
        eng.close()
