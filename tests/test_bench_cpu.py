"""CPU checks of bench.py's contract: the algorithmic bytes behind
roofline.achieved, counted here from the matrix shapes, and the refusal of
more than one GPU (before anything touches a device)."""
import os
import subprocess
import sys

from persistent_megakernel_wg_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_llama1b_algorithmic_bytes_from_the_architecture():
    s = synth.SHAPES["llama1b_ctx128"]
    d, q, kv, f, v, L = 2048, 32 * 64, 8 * 64, 8192, 128256, 16
    assert (s.hidden, s.n_q_heads * s.head_dim, s.n_kv_heads * s.head_dim, s.ffn, s.vocab, s.n_layers) == \
        (d, q, kv, f, v, L)
    bf16 = 2
    per_layer = bf16 * (d * q + 2 * d * kv + q * d + 3 * d * f)   # Wq, Wk, Wv, Wo, gate, up, down
    norms = bf16 * d * (2 * L + 1)                                 # two per layer and the final one
    weights = L * per_layer + bf16 * v * d + norms + bf16 * d      # + tied LM head + one embedding row
    assert weights == 2_471_632_896
    assert synth.weight_bytes_per_step(s) == weights
    # KV: read positions [0, P) of every layer and group, K and V; write row P
    row = 2 * s.head_dim * bf16
    for p in (128, 143, 159):
        assert synth.kv_bytes_per_step(s, p) == L * s.n_kv_heads * row * (p + 1)
    # the 32 timed steps run at P = 128 ... 159
    mean = sum(synth.kv_bytes_per_step(s, p) for p in range(128, 160)) / 32
    assert weights + mean == 2_476_367_872


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_moe_fixed_bytes_from_the_architecture():
    # bench.py's algorithmic bytes for the MoE shape: the plan's routing-
    # independent weight bytes plus 6 * d * Fe per selected expert and layer
    from persistent_megakernel_wg_amd import binding as B
    s = synth.SHAPES["moe_b8_ctx2048"]
    d, q, kv, E, Fe, V, L, nb = 2048, 16 * 128, 4 * 128, 64, 1024, 65536, 24, 8
    assert (s.hidden, s.n_q_heads * s.head_dim, s.n_kv_heads * s.head_dim, s.n_experts, s.expert_ffn,
            s.vocab, s.n_layers, s.batch) == (d, q, kv, E, Fe, V, L, nb)
    bf16 = 2
    attn = bf16 * (d * q + 2 * d * kv + q * d)   # Wq, Wk, Wv, Wo
    router = bf16 * E * d
    fixed = L * (attn + router) + bf16 * V * d + bf16 * d * (L + 1) + bf16 * nb * d
    #        layers                untied LM head   one norm per layer + final   embedding rows
    assert fixed == 778_178_560
    summ, _ = B.mk_plan_check(B.config_from_shape(s), 256)
    assert summ["weight_bytes"] == fixed
