"""Host-side tests of libmk.so: exported symbols, the planner and its verifier,
and argument checking.  No GPU needed (no compute call is made)."""
import ctypes
import json
import os
import re

import pytest

from persistent_megakernel_wg_amd import binding as B
from persistent_megakernel_wg_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DENSE = ["tiny", "llama1b_ctx128", "llama1b_ctx8192", "llama8b_ctx2048"]


def _cfg(name, **kw):
    return B.config_from_shape(synth.SHAPES[name].replace(**kw))


def test_library_exports_every_declared_entry_point():
    lib = B.load_library()
    with open(os.path.join(ROOT, "include", "mk.h")) as fh:
        header = fh.read()
    declared = set(re.findall(r"^(?:mk_status|const char \*)\s*(mk_\w+)\s*\(", header, re.M))
    assert declared == set(B.EXPORTS)
    for name in declared:
        assert getattr(lib, name) is not None


@pytest.mark.parametrize("name", DENSE)
def test_default_plan_verifies(name):
    s = synth.SHAPES[name]
    summ, rep = B.mk_plan_check(B.config_from_shape(s), 256)
    r = json.loads(rep)
    assert summ["n_cus"] == 256 and len(r["queue_lengths"]) == 256
    assert summ["weight_bytes"] == synth.weight_bytes_per_step(s)
    # the shape-specific kernels: 1B, 8B, the small test decoder
    assert summ["kernel_variant"] == {"tiny": 4, "llama1b_ctx128": 1, "llama1b_ctx8192": 2,
                                      "llama8b_ctx2048": 3}[name]
    # one query head per attention tile at short contexts, whole groups at long ones
    nblk = -(-s.max_seq // summ["attn_block"])
    per_block = s.n_q_heads if name in ("tiny", "llama1b_ctx128") else s.n_kv_heads
    assert summ["attn_tiles"] == per_block * nblk
    # default: the fewest chunks of at most 4096 values
    assert summ["mlp_chunks"] == {"tiny": 1, "llama1b_ctx128": 2, "llama1b_ctx8192": 2,
                                  "llama8b_ctx2048": 4}[name]
    assert summ["lds_bytes"] <= 160 * 1024
    # every CU streams about the same number of bytes (the tiny decoder has
    # fewer rows than there are CUs, so it cannot be balanced)
    if name != "tiny":
        assert summ["max_cu_bytes"] <= 1.25 * summ["min_cu_bytes"]


@pytest.mark.parametrize("name,n_cus,opts", [
    ("tiny", 1, {}), ("tiny", 7, {"mlp_chunks": 1}), ("tiny", 37, {"attn_block": 64}),
    ("tiny", 256, {"mlp_chunks": 2, "attn_block": 64}),
    ("llama1b_ctx128", 100, {"attn_block": 64}), ("llama1b_ctx8192", 256, {"attn_block": 128}),
    ("llama8b_ctx2048", 128, {}),
    ("tiny", 64, {"attn_heads": 2, "attn_block": 64}), ("llama1b_ctx128", 256, {"attn_heads": 4}),
    ("llama1b_ctx128", 256, {"attn_heads": 2, "attn_block": 64}),
])
def test_plan_variants_verify(name, n_cus, opts):
    B.mk_plan_check(_cfg(name), n_cus, B.plan_opts(**opts))


@pytest.mark.parametrize("name,kw,n_cus", [
    ("tiny", {"n_q_heads": 8}, 1), ("tiny", {"n_q_heads": 8}, 3), ("tiny", {"n_q_heads": 8}, 256),
    ("tiny", {"head_dim": 128}, 5), ("llama1b_ctx128", {}, 256), ("llama1b_ctx128", {}, 17),
    ("llama1b_ctx8192", {}, 256), ("llama8b_ctx2048", {}, 256),
])
def test_split_k_o_projection_plans_verify(name, kw, n_cus):
    # O tiles per (row block, KV group), the block's last ticket merging x and
    # the group partials; against whole-row O tiles of the same shape
    split, rep = B.mk_plan_check(_cfg(name, **kw), n_cus, B.plan_opts(o_split=1))
    whole, _ = B.mk_plan_check(_cfg(name, **kw), n_cus, B.plan_opts(o_split=-1))
    assert split["weight_bytes"] == whole["weight_bytes"]


@pytest.mark.parametrize("kw", [{}, {"n_kv_heads": 1, "n_q_heads": 8}])
def test_split_k_o_projection_needs_groups_and_a_gemv_width(kw):
    # tiny: two groups of 2 x 64 = 128 inputs (no GEMV path for K = 128); one
    # KV group: nothing to split
    with pytest.raises(B.MkError) as e:
        B.mk_plan_check(_cfg("tiny", **kw), 64, B.plan_opts(o_split=1))
    assert e.value.status == -4


def test_verifier_rejects_a_wrong_counter_target():
    with pytest.raises(B.MkError) as e:
        B.mk_plan_check(_cfg("tiny"), 64, B.plan_opts(debug_corrupt_target=1))
    assert e.value.status == -1 and "waits for" in str(e.value)


@pytest.mark.parametrize("kw,status", [
    ({"head_dim": 96}, -4), ({"n_kv_heads": 3}, -1), ({"batch": 2}, -4),
    ({"n_experts": 4, "top_k": 2, "expert_ffn": 512}, -4), ({"hidden": 384}, -4),
    ({"n_layers": 0}, -1),
])
def test_unsupported_or_bad_shapes_are_rejected(kw, status):
    with pytest.raises(B.MkError) as e:
        B.mk_plan_check(_cfg("tiny", **kw), 64)
    assert e.value.status == status


@pytest.mark.parametrize("opts", [{"attn_block": 100}, {"mlp_chunks": 3}, {"attn_block": 1024},
                                  {"attn_heads": 3}])
def test_bad_plan_options_are_rejected(opts):
    with pytest.raises(B.MkError):
        B.mk_plan_check(_cfg("tiny"), 64, B.plan_opts(**opts))


def test_null_arguments():
    lib = B.load_library()
    assert lib.mk_destroy(None) == 0
    out = ctypes.c_void_p()
    assert lib.mk_create(None, None, 0, ctypes.byref(out)) == -1
    assert "required" in B.mk_last_error()
    assert lib.mk_build_plan(None, None) == -1
    assert lib.mk_decode_step(None, None, 0, None, None, None) == -1
    assert lib.mk_sync(None) == -1


# ------------------------------------------------------------ batched (MoE)
MOE = ["moe_tiny", "moe_b8_ctx2048"]


def moe_fixed_bytes(s):
    """Weight bytes of one batched step that do not depend on the routing:
    attention and router projections, norms, the LM head, B embedding rows."""
    d, L = s.hidden, s.n_layers
    per_layer = 2 * ((s.q_dim + 2 * s.kv_dim) * d + d * s.q_dim + s.n_experts * d + d)
    return L * per_layer + 2 * s.vocab * d + 2 * d + 2 * d * s.batch


@pytest.mark.parametrize("name", MOE)
def test_moe_default_plan_verifies(name):
    s = synth.SHAPES[name]
    summ, rep = B.mk_plan_check(B.config_from_shape(s), 256)
    assert summ["weight_bytes"] == moe_fixed_bytes(s)
    # the kernel built for 4 heads/group, Dh 128, with the matrix-core LM head
    # (the default); without it, the same shape's vector-ALU kernel
    assert summ["kernel_variant"] == 2
    assert B.mk_plan_check(B.config_from_shape(s), 256, B.plan_opts(mfma=-1))[0]["kernel_variant"] == 1
    assert summ["lds_bytes"] == 159744 and summ["n_pages"] == 5
    hpg = s.n_q_heads // s.n_kv_heads
    assert summ["attn_block"] * hpg <= 512      # scores of one tile fit the scratch
    nblk = -(-s.max_seq // summ["attn_block"])
    assert summ["attn_tiles"] == s.batch * s.n_kv_heads * nblk
    # every CU holds a slice of every expert: the same bytes per CU up to
    # the attention tiles and the rounding of the slices (the tiny shape has
    # fewer attention tiles and router rows than CUs)
    if name != "moe_tiny":
        assert summ["max_cu_bytes"] <= 1.25 * summ["min_cu_bytes"]


def test_moe_fixed_bytes_of_the_large_shape():
    # attention + router + LM head + norms of the 24-layer batch-8 shape
    assert moe_fixed_bytes(synth.SHAPES["moe_b8_ctx2048"]) == 778_178_560


@pytest.mark.parametrize("n_cus,kw,opts", [
    (1, {}, {"attn_block": 64}), (3, {}, {}), (16, {}, {"attn_block": 64}), (37, {"batch": 3}, {}),
    (256, {"batch": 1}, {}), (256, {"top_k": 1}, {}), (256, {"top_k": 8}, {}),
    (64, {"expert_ffn": 2048, "top_k": 4, "n_experts": 16}, {}), (256, {}, {"attn_heads": 1}),
    (256, {"n_q_heads": 8, "n_kv_heads": 1, "head_dim": 64}, {"attn_block": 64}),
    (100, {"n_experts": 64, "top_k": 8}, {}),
])
def test_moe_plan_variants_verify(n_cus, kw, opts):
    summ, _ = B.mk_plan_check(_cfg("moe_tiny", **kw), n_cus, B.plan_opts(**opts))
    assert summ["n_cus"] == n_cus


def test_moe_plan_for_the_large_shape_on_fewer_cus():
    B.mk_plan_check(_cfg("moe_b8_ctx2048"), 80)


@pytest.mark.parametrize("gu_all", [-1, 1])
def test_gate_up_over_every_chunk_plans_verify(gu_all):
    # one gate/up instruction per CU over every chunk removes chunks - 1
    # instructions per CU and layer; the verifier checks the chunk geometry,
    # the output rows and the packed copies
    for name, chunks, cus in (("tiny", 2, (1, 7, 256)), ("tiny", 4, (1, 7, 256)),
                              ("llama1b_ctx128", 0, (37, 256)), ("llama8b_ctx2048", 0, (64, 256))):
        for n_cus in cus:
            on, _ = B.mk_plan_check(_cfg(name), n_cus, B.plan_opts(mlp_chunks=chunks, gu_all=gu_all))
            off, _ = B.mk_plan_check(_cfg(name), n_cus, B.plan_opts(mlp_chunks=chunks, gu_all=-1))
            assert on["weight_bytes"] == off["weight_bytes"]
            if gu_all > 0:
                L = synth.SHAPES[name].n_layers
                assert off["n_instr"] - on["n_instr"] == L * (on["mlp_chunks"] - 1) * min(n_cus, 256)


@pytest.mark.parametrize("queue", [-1, 1, 2, 4, 8, 16])
def test_moe_ready_queue_plans_verify(queue):
    for n_cus in (1, 3, 256):
        B.mk_plan_check(_cfg("moe_tiny"), n_cus, B.plan_opts(edn_queue=queue))
    B.mk_plan_check(_cfg("moe_b8_ctx2048"), 256, B.plan_opts(edn_queue=queue))


@pytest.mark.parametrize("balance", [-1, 1])
def test_moe_gate_up_share_plans_verify(balance):
    # weighted shares (the verifier checks that a layer's shares tile its
    # items exactly) and even row slices
    for n_cus in (1, 3, 37, 256):
        B.mk_plan_check(_cfg("moe_tiny"), n_cus, B.plan_opts(egu_balance=balance))
    B.mk_plan_check(_cfg("moe_tiny", expert_ffn=2048, top_k=4, n_experts=16), 64, B.plan_opts(egu_balance=balance))
    summ, _ = B.mk_plan_check(_cfg("moe_b8_ctx2048"), 256, B.plan_opts(egu_balance=balance))
    assert summ["weight_bytes"] == moe_fixed_bytes(synth.SHAPES["moe_b8_ctx2048"])


@pytest.mark.parametrize("name,kw,n_cus", [
    ("moe_tiny", {}, 256), ("moe_tiny", {}, 1), ("moe_tiny", {"batch": 3}, 37), ("moe_b8_ctx2048", {}, 256),
])
def test_moe_matrix_core_lm_head_plans_verify(name, kw, n_cus):
    # LM-head tiles of 16 rows in MFMA fragment order (same bytes streamed,
    # rows padded to whole blocks), run by the kernel variant that has them
    mf, _ = B.mk_plan_check(_cfg(name, **kw), n_cus, B.plan_opts(mfma=1))
    vec, _ = B.mk_plan_check(_cfg(name, **kw), n_cus, B.plan_opts(mfma=-1))
    assert mf["weight_bytes"] == vec["weight_bytes"]
    assert mf["kernel_variant"] == 2 and vec["kernel_variant"] == 1


@pytest.mark.parametrize("kw", [
    {"top_k": 9, "n_experts": 16}, {"top_k": 4, "n_experts": 3}, {"batch": 9},
    {"expert_ffn": 768}, {"hidden": 4096, "n_q_heads": 32}, {"n_experts": 65},
    {"expert_ffn": 4096}, {"parallel_block": False},
])
def test_unsupported_moe_shapes_are_rejected(kw):
    with pytest.raises(B.MkError) as e:
        B.mk_plan_check(_cfg("moe_tiny", **kw), 64)
    assert e.value.status == -4


def test_moe_bad_plan_options_are_rejected():
    for opts in ({"attn_block": 256}, {"attn_heads": 3}, {"attn_block": 96}):
        with pytest.raises(B.MkError):
            B.mk_plan_check(_cfg("moe_tiny"), 64, B.plan_opts(**opts))


@pytest.mark.parametrize("name", DENSE + ["moe_tiny", "moe_b8_ctx2048"])
def test_noalloc_scratch_fits_the_fixed_array(name):
    # the no-allocation entry point runs every workload's plan in the fixed
    # per-GPU array; its size in the header matches the binding's constant
    with open(os.path.join(ROOT, "include", "mk.h")) as fh:
        m = re.search(r"#define MK_NOALLOC_SCRATCH_BYTES \((\d+)u \* 1024u \* 1024u\)", fh.read())
    assert m and int(m.group(1)) << 20 == B.NOALLOC_SCRATCH_BYTES
    summ, _ = B.mk_plan_check(B.config_from_shape(synth.SHAPES[name]), 256)
    assert 0 < summ["scratch_bytes"] <= B.NOALLOC_SCRATCH_BYTES
