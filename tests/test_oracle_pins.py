"""Pins of the CPU oracle against facts that do not come from the oracle itself:
closed forms, invariants, special cases that reduce to library routines, and
brute force on tiny shapes."""
import math

import numpy as np
import pytest
import torch

from oracle import (DecoderOracle, attend, bf16_to_f64, f64_to_bf16, greedy,
                    rms_norm, rope, silu, softmax, top_k_ids)
from persistent_megakernel_wg_amd import synth


# ----------------------------------------------------------------- bf16 rounding
def test_bf16_round_nearest_even_cases():
    # Hand-derived: bf16 keeps 7 fraction bits, so the spacing above 1.0 is 2^-7.
    cases = {
        1.0: 0x3F80,
        1.0 + 2.0 ** -8: 0x3F80,             # exact tie -> even (fraction 0)
        1.0 + 3 * 2.0 ** -8: 0x3F82,         # exact tie -> even (fraction 2)
        1.0 + 2.0 ** -8 + 2.0 ** -20: 0x3F81,  # just above the tie -> up
        -2.0: 0xC000,
        0.0: 0x0000,
        3.140625: 0x4049,                    # exactly representable
    }
    for val, bits in cases.items():
        assert int(f64_to_bf16(np.array([val]))[0]) == bits, val
    assert bf16_to_f64(np.array([0x4049], dtype=np.uint16))[0] == 3.140625


def test_bf16_matches_torch_conversion():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(10000).astype(np.float32) * 3
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f64_to_bf16(x.astype(np.float64)), ref)
    assert np.array_equal(bf16_to_f64(ref), torch.from_numpy(ref.view(np.int16)).view(
        torch.bfloat16).to(torch.float64).numpy())


# ---------------------------------------------------------------------- RMSNorm
@pytest.mark.parametrize("c", [0.5, -3.0, 1e-3])
def test_rms_norm_of_constant_vector(c):
    d, eps = 256, 1e-5
    g = np.linspace(0.5, 1.5, d)
    n = rms_norm(np.full(d, c), g, eps)
    np.testing.assert_allclose(n, g * c / math.sqrt(c * c + eps), rtol=1e-14)


def test_rms_norm_matches_torch():
    rng = np.random.default_rng(1)
    x, g = rng.standard_normal(2048), rng.standard_normal(2048)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (2048,), torch.from_numpy(g),
                                       eps=1e-5).numpy()
    np.testing.assert_allclose(rms_norm(x, g, 1e-5), ref, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------------- RoPE
def test_rope_position_zero_is_identity():
    v = np.random.default_rng(2).standard_normal((3, 64))
    np.testing.assert_array_equal(rope(v, 0, 500000.0), v)


def test_rope_equals_complex_rotation():
    # Pair (j, j + Dh/2) as the complex number v_j + i v_{j+Dh/2}, multiplied by
    # exp(i * pos * theta^(-2j/Dh)).
    rng = np.random.default_rng(3)
    dh, theta = 8, 10000.0
    v = rng.standard_normal(dh)
    for pos in (1, 7, 1234):
        z = v[:dh // 2] + 1j * v[dh // 2:]
        rot = np.array([z[j] * complex(math.cos(pos * theta ** (-2 * j / dh)),
                                       math.sin(pos * theta ** (-2 * j / dh)))
                        for j in range(dh // 2)])
        np.testing.assert_allclose(rope(v, pos, theta),
                                   np.concatenate([rot.real, rot.imag]), rtol=1e-12,
                                   atol=1e-12)


def test_rope_preserves_pair_norms_and_is_relative():
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for pos in (3, 100, 8191):
        r = rope(q, pos, 500000.0)
        np.testing.assert_allclose(r[:32] ** 2 + r[32:] ** 2, q[:32] ** 2 + q[32:] ** 2,
                                   rtol=1e-12)
    # <R_m q, R_n k> depends only on m - n
    a = rope(q, 40, 1e4) @ rope(k, 15, 1e4)
    b = rope(q, 1040, 1e4) @ rope(k, 1015, 1e4)
    assert abs(a - b) < 1e-9 * max(1.0, abs(a))


def test_rope_matches_transformers_llama_rotary():
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import (LlamaRotaryEmbedding,
                                                          apply_rotary_pos_emb)
    cfg = LlamaConfig(hidden_size=256, num_attention_heads=4, head_dim=64,
                      rope_theta=500000.0, max_position_embeddings=4096)
    rot = LlamaRotaryEmbedding(cfg)
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 4, 1, 64))
    k = rng.standard_normal((1, 2, 1, 64))
    for pos in (0, 5, 2047):
        x = torch.zeros(1, 1, 64, dtype=torch.float64)
        cos, sin = rot(x, torch.tensor([[pos]]))
        qr, kr = apply_rotary_pos_emb(torch.from_numpy(q), torch.from_numpy(k),
                                      cos.double(), sin.double())
        # the library builds its frequencies in float32: allow that error
        np.testing.assert_allclose(rope(q, pos, 500000.0), qr.numpy(), atol=2e-4 * (1 + pos / 512))
        np.testing.assert_allclose(rope(k, pos, 500000.0), kr.numpy(), atol=2e-4 * (1 + pos / 512))


# -------------------------------------------------------------------- attention
def test_attention_single_position_returns_v():
    rng = np.random.default_rng(7)
    q, k, v = rng.standard_normal(64), rng.standard_normal((1, 64)), rng.standard_normal((1, 64))
    np.testing.assert_array_equal(attend(q, k, v), v[0])


def test_attention_equal_keys_returns_mean_of_values():
    rng = np.random.default_rng(8)
    q = rng.standard_normal(64)
    keys = np.tile(rng.standard_normal(64), (9, 1))
    vals = rng.standard_normal((9, 64))
    np.testing.assert_allclose(attend(q, keys, vals), vals.mean(axis=0), rtol=1e-12)


def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(9)
    q, keys, vals = rng.standard_normal(64), rng.standard_normal((33, 64)), rng.standard_normal((33, 64))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None, None], torch.from_numpy(keys)[None, None],
        torch.from_numpy(vals)[None, None])[0, 0, 0].numpy()
    np.testing.assert_allclose(attend(q, keys, vals), ref, rtol=1e-12, atol=1e-14)


def test_softmax_shift_invariant():
    s = np.random.default_rng(10).standard_normal(50)
    np.testing.assert_allclose(softmax(s), softmax(s + 123.0), rtol=1e-12)
    assert abs(softmax(s).sum() - 1) < 1e-14


# ------------------------------------------------------------- silu / selection
def test_silu_values():
    z = np.linspace(-20, 20, 81)
    np.testing.assert_allclose(silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(),
                               rtol=1e-13, atol=1e-300)
    assert silu(np.array([0.0]))[0] == 0.0


def test_greedy_lowest_index_on_ties_and_planted_max():
    x = np.zeros(4096)
    x[[17, 900, 4000]] = 2.5
    assert greedy(x) == 17
    x[3333] = 2.6
    assert greedy(x) == 3333


def test_top_k_ties_to_lower_id():
    r = np.array([0.1, 0.9, 0.5, 0.9, -1.0, 0.5, 0.2, 0.9])
    assert list(top_k_ids(r, 4)) == [1, 3, 7, 2]


# ------------------------------------------------------------ decoder structure
def _tiny(**kw):
    return synth.SHAPES["tiny"].replace(**kw)


def test_zero_layer_matrices_pass_embedding_through():
    s = _tiny()
    w = synth.make_weights(s)
    for name in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
        w[name] = np.zeros_like(w[name])
    kc, vc = synth.make_kv_cache(s)
    tok = synth.make_tokens(s)
    logits, nxt = DecoderOracle(s, w).step(tok, s.prefill, kc, vc)
    e = bf16_to_f64(w["embed"])
    x = e[tok[0]]
    expect = e @ (x / np.sqrt(np.mean(x * x) + s.rms_eps))
    np.testing.assert_allclose(logits[0], expect, rtol=1e-12, atol=1e-12)
    assert nxt[0] == tok[0]          # tied head: the input row has the largest logit
    # the appended rows are bf16 zeros (either sign)
    assert not (kc[:, :, :, s.prefill] & 0x7FFF).any()
    assert not (vc[:, :, :, s.prefill] & 0x7FFF).any()


def test_gqa_head_to_kv_group_mapping():
    # Two KV heads whose cached values are +1 and -1 everywhere: query heads 0,1
    # must read +1 and heads 2,3 must read -1 (o = Wo . o_heads with Wo = I).
    s = _tiny(n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64)
    w = synth.make_weights(s)
    w["wv"] = np.zeros_like(w["wv"])   # new value rows are 0
    w["wk"] = np.zeros_like(w["wk"])   # all scores 0: uniform weights
    eye = np.zeros((1, 256, 256), dtype=np.uint16)
    eye[0][np.arange(256), np.arange(256)] = 0x3F80
    w["wo"] = eye
    kc = np.zeros((1, 1, 2, s.max_seq, 64), dtype=np.uint16)
    vc = np.zeros_like(kc)
    p = 10
    vc[0, 0, 0, :p] = 0x3F80        # +1
    vc[0, 0, 1, :p] = 0xBF80        # -1
    tr = {}
    DecoderOracle(s, w).step(np.array([5]), p, kc, vc, trace=tr)
    o = tr["attn_out"][0].reshape(4, 64)
    # uniform weights over p rows of +-1 and the new zero row
    np.testing.assert_allclose(o[:2], p / (p + 1.0), rtol=1e-14)
    np.testing.assert_allclose(o[2:], -p / (p + 1.0), rtol=1e-14)


def test_batch_rows_are_independent():
    s = _tiny(batch=2)
    w = synth.make_weights(s)
    kc, vc = synth.make_kv_cache(s)
    toks = np.array([11, 2222], dtype=np.int32)
    lg, nx = DecoderOracle(s, w).step(toks, s.prefill, kc.copy(), vc.copy())
    s1 = _tiny()
    for b in range(2):
        k1 = kc[:, b:b + 1].copy()
        v1 = vc[:, b:b + 1].copy()
        lg1, nx1 = DecoderOracle(s1, w).step(toks[b:b + 1], s.prefill, k1, v1)
        np.testing.assert_array_equal(lg1[0], lg[b])


# ---------------------------------------------------------------- brute force
def _loops_decode(s, w, kc, vc, tok, pos):
    """Whole decode step with explicit Python loops (tiny shapes only)."""
    f = lambda a: [float(v) for v in bf16_to_f64(a).reshape(-1)]
    d, H, G, dh, F = s.hidden, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn
    x = f(w["embed"][tok])

    def mv(mat, vec, rows, cols):
        flat = f(mat)
        return [sum(flat[r * cols + c] * vec[c] for c in range(cols)) for r in range(rows)]

    def norm(vec, gain):
        ms = sum(v * v for v in vec) / len(vec)
        inv = 1.0 / math.sqrt(ms + s.rms_eps)
        return [gain[i] * vec[i] * inv for i in range(len(vec))]

    def rot(vec):
        half = dh // 2
        out = list(vec)
        for j in range(half):
            ang = pos * s.rope_theta ** (-2.0 * j / dh)
            a, b = vec[j], vec[j + half]
            out[j] = a * math.cos(ang) - b * math.sin(ang)
            out[j + half] = b * math.cos(ang) + a * math.sin(ang)
        return out

    for l in range(s.n_layers):
        n = norm(x, f(w["attn_norm"][l]))
        q = mv(w["wq"][l], n, H * dh, d)
        k = mv(w["wk"][l], n, G * dh, d)
        v = mv(w["wv"][l], n, G * dh, d)
        for g in range(G):
            kr = rot(k[g * dh:(g + 1) * dh])
            kc[l, 0, g, pos] = f64_to_bf16(np.array(kr))
            vc[l, 0, g, pos] = f64_to_bf16(np.array(v[g * dh:(g + 1) * dh]))
        o = []
        for h in range(H):
            g = h // (H // G)
            qh = rot(q[h * dh:(h + 1) * dh])
            keys = [f(kc[l, 0, g, p]) for p in range(pos + 1)]
            vals = [f(vc[l, 0, g, p]) for p in range(pos + 1)]
            sc = [sum(qh[i] * kk[i] for i in range(dh)) / math.sqrt(dh) for kk in keys]
            mx = max(sc)
            ex = [math.exp(t - mx) for t in sc]
            tot = sum(ex)
            o += [sum(ex[p] * vals[p][i] for p in range(pos + 1)) / tot for i in range(dh)]
        att = mv(w["wo"][l], o, d, H * dh)
        h_ = [x[i] + att[i] for i in range(d)]
        n2 = norm(h_, f(w["mlp_norm"][l]))
        gt = mv(w["w_gate"][l], n2, F, d)
        up = mv(w["w_up"][l], n2, F, d)
        mid = [gt[i] / (1.0 + math.exp(-gt[i])) * up[i] for i in range(F)]
        dn = mv(w["w_down"][l], mid, d, F)
        x = [h_[i] + dn[i] for i in range(d)]
    n = norm(x, f(w["final_norm"]))
    return mv(w["lm_head"], n, s.vocab, d)


def test_brute_force_micro_decoder():
    s = synth.ModelShape("micro", n_layers=2, hidden=8, n_q_heads=2, n_kv_heads=1,
                         head_dim=4, ffn=16, vocab=32, prefill=5, max_seq=8,
                         rope_theta=10000.0)
    w = synth.make_weights(s, std=0.5)
    kc, vc = synth.make_kv_cache(s)
    kc2, vc2 = kc.copy(), vc.copy()
    lg, _ = DecoderOracle(s, w).step(np.array([7]), 5, kc, vc)
    ref = _loops_decode(s, w, kc2, vc2, 7, 5)
    np.testing.assert_allclose(lg[0], ref, rtol=1e-10, atol=1e-12)
    assert np.array_equal(kc, kc2) and np.array_equal(vc, vc2)


# ------------------------------------------------------------------------ MoE
def _moe_shape(**kw):
    base = dict(n_layers=1, hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16, ffn=0,
                vocab=128, prefill=6, max_seq=16, batch=2, tied_embedding=False,
                n_experts=4, top_k=2, expert_ffn=32, parallel_block=True)
    base.update(kw)
    return synth.ModelShape("moe_small", **base)


def test_moe_single_expert_is_dense_swiglu():
    s = _moe_shape(n_experts=1, top_k=1)
    w = synth.make_weights(s, std=0.2)
    orc = DecoderOracle(s, w)
    n = np.random.default_rng(11).standard_normal(64)
    wg, wu, wd = (bf16_to_f64(w[k][0, 0]) for k in ("e_gate", "e_up", "e_down"))
    dense = wd @ (silu(wg @ n) * (wu @ n))
    np.testing.assert_allclose(orc.moe(n, 0), dense, rtol=1e-13)


def test_moe_identical_experts_ignore_routing():
    s = _moe_shape()
    w = synth.make_weights(s, std=0.2)
    for k in ("e_gate", "e_up", "e_down"):
        w[k][:] = w[k][:, :1]
    orc = DecoderOracle(s, w)
    n = np.random.default_rng(12).standard_normal(64)
    wg, wu, wd = (bf16_to_f64(w[k][0, 0]) for k in ("e_gate", "e_up", "e_down"))
    np.testing.assert_allclose(orc.moe(n, 0), wd @ (silu(wg @ n) * (wu @ n)), rtol=1e-12)


def test_moe_planted_router_selects_and_weights():
    s = _moe_shape()
    w = synth.make_weights(s, std=0.2)
    # router rows e = c_e * n_hat direction: logits are known multiples
    n = np.ones(64)
    coef = np.array([0.25, 1.0, -0.5, 0.75])  # in bf16 exactly
    w["router"] = np.stack([f64_to_bf16(np.full(64, c / 64.0)) for c in coef])[None]
    tr = {}
    orc = DecoderOracle(s, w)
    out = orc.moe(n, 0, tr)
    assert list(tr["router_ids"][0]) == [1, 3]
    e1, e3 = math.exp(1.0), math.exp(0.75)
    np.testing.assert_allclose(tr["router_w"][0], [e1 / (e1 + e3), e3 / (e1 + e3)], rtol=1e-12)
    parts = []
    for e in (1, 3):
        wg, wu, wd = (bf16_to_f64(w[k][0, e]) for k in ("e_gate", "e_up", "e_down"))
        parts.append(wd @ (silu(wg @ n) * (wu @ n)))
    np.testing.assert_allclose(out, tr["router_w"][0][0] * parts[0] + tr["router_w"][0][1] * parts[1],
                               rtol=1e-12)


def test_parallel_block_branches_read_the_same_norm():
    # x_out - x is additive over the two branches only if both read RMSNorm(x).
    s = _moe_shape(batch=1)
    w = synth.make_weights(s, std=0.2)
    kc, vc = synth.make_kv_cache(s)
    tok = np.array([3])

    def delta(wmod):
        tr = {}
        DecoderOracle(s, wmod).step(tok, s.prefill, kc.copy(), vc.copy(), trace=tr)
        return tr["x_out"][0] - tr["x_in"][0]

    both = delta(w)
    w_attn = dict(w)
    w_attn["e_down"] = np.zeros_like(w["e_down"])
    w_moe = dict(w)
    w_moe["wo"] = np.zeros_like(w["wo"])
    np.testing.assert_allclose(both, delta(w_attn) + delta(w_moe), rtol=1e-11, atol=1e-14)
