"""Cross-checks of the whole oracle decode step on the tiny decoder against
implementations that share nothing with it: one assembled here from PyTorch's
library routines, and the Llama model of HF ``transformers`` (float64, CPU)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import DecoderOracle, bf16_to_f64, f64_to_bf16
from persistent_megakernel_wg_amd import synth


def _inputs(shape):
    w = synth.make_weights(shape)
    kc, vc = synth.make_kv_cache(shape)
    tok = synth.make_tokens(shape)
    return w, kc, vc, tok


def _t(bits):
    return torch.from_numpy(bf16_to_f64(bits))


def _torch_library_step(s, w, kc, vc, tok, pos):
    """Decode step built from torch.nn.functional routines and the rotary helper
    of transformers; rounds the appended K/V rows to bf16 with torch's cast."""
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb
    # float64 angles for the library's rotate-half helper (its own rotary module
    # forms the angles in float32)
    inv_freq = s.rope_theta ** (-torch.arange(0, s.head_dim, 2, dtype=torch.float64) / s.head_dim)
    emb = torch.cat([pos * inv_freq, pos * inv_freq])[None, None]
    cos, sin = emb.cos(), emb.sin()
    x = _t(w["embed"][tok])[None]                              # [1, d]
    kc_t, vc_t = kc.copy(), vc.copy()
    for l in range(s.n_layers):
        n = F.rms_norm(x, (s.hidden,), _t(w["attn_norm"][l]), eps=s.rms_eps)
        q = F.linear(n, _t(w["wq"][l])).view(1, s.n_q_heads, 1, s.head_dim)
        k = F.linear(n, _t(w["wk"][l])).view(1, s.n_kv_heads, 1, s.head_dim)
        v = F.linear(n, _t(w["wv"][l])).view(1, s.n_kv_heads, 1, s.head_dim)
        q, k = apply_rotary_pos_emb(q, k, cos, sin)
        k16 = k.float().to(torch.bfloat16)
        v16 = v.float().to(torch.bfloat16)
        kc_t[l, 0, :, pos] = k16[0, :, 0].view(torch.int16).numpy().view(np.uint16)
        vc_t[l, 0, :, pos] = v16[0, :, 0].view(torch.int16).numpy().view(np.uint16)
        keys = _t(kc_t[l, 0, :, :pos + 1])[None]               # [1, G, P+1, Dh]
        vals = _t(vc_t[l, 0, :, :pos + 1])[None]
        o = F.scaled_dot_product_attention(q, keys, vals, enable_gqa=True)
        h = x + F.linear(o.reshape(1, -1), _t(w["wo"][l]))
        n2 = F.rms_norm(h, (s.hidden,), _t(w["mlp_norm"][l]), eps=s.rms_eps)
        mid = F.silu(F.linear(n2, _t(w["w_gate"][l]))) * F.linear(n2, _t(w["w_up"][l]))
        x = h + F.linear(mid, _t(w["w_down"][l]))
    n = F.rms_norm(x, (s.hidden,), _t(w["final_norm"]), eps=s.rms_eps)
    return F.linear(n, _t(w["lm_head"]))[0].numpy(), kc_t, vc_t


def test_oracle_matches_torch_library_decoder():
    s = synth.SHAPES["tiny"]
    w, kc, vc, tok = _inputs(s)
    ref_logits, ref_k, ref_v = _torch_library_step(s, w, kc, vc, int(tok[0]), s.prefill)
    logits, nxt = DecoderOracle(s, w).step(tok, s.prefill, kc, vc)
    np.testing.assert_allclose(logits[0], ref_logits, rtol=1e-9, atol=1e-11)
    assert np.array_equal(kc, ref_k) and np.array_equal(vc, ref_v)
    assert nxt[0] == int(np.argmax(ref_logits.astype(np.float32)))


def test_oracle_matches_transformers_llama():
    from transformers import DynamicCache, LlamaConfig, LlamaForCausalLM
    s = synth.SHAPES["tiny"]
    w, kc, vc, tok = _inputs(s)
    cfg = LlamaConfig(hidden_size=s.hidden, intermediate_size=s.ffn,
                      num_attention_heads=s.n_q_heads, num_key_value_heads=s.n_kv_heads,
                      head_dim=s.head_dim, vocab_size=s.vocab, rms_norm_eps=s.rms_eps,
                      rope_theta=s.rope_theta, tie_word_embeddings=True,
                      num_hidden_layers=s.n_layers, max_position_embeddings=s.max_seq,
                      attention_bias=False, mlp_bias=False)
    model = LlamaForCausalLM(cfg).double().eval()
    sd = {"model.embed_tokens.weight": _t(w["embed"]), "model.norm.weight": _t(w["final_norm"])}
    names = {"self_attn.q_proj": "wq", "self_attn.k_proj": "wk", "self_attn.v_proj": "wv",
             "self_attn.o_proj": "wo", "mlp.gate_proj": "w_gate", "mlp.up_proj": "w_up",
             "mlp.down_proj": "w_down"}
    for l in range(s.n_layers):
        for hf, ours in names.items():
            sd[f"model.layers.{l}.{hf}.weight"] = _t(w[ours][l])
        sd[f"model.layers.{l}.input_layernorm.weight"] = _t(w["attn_norm"][l])
        sd[f"model.layers.{l}.post_attention_layernorm.weight"] = _t(w["mlp_norm"][l])
    missing, unexpected = model.load_state_dict(sd, strict=False)
    assert not unexpected and all("lm_head" in m or "rotary" in m for m in missing)
    model.lm_head.weight = model.model.embed_tokens.weight
    cache = DynamicCache(config=cfg)
    P = s.prefill
    for l in range(s.n_layers):
        cache.update(_t(kc[l, :, :, :P]), _t(vc[l, :, :, :P]), l)
    with torch.no_grad():
        out = model(input_ids=torch.tensor([[int(tok[0])]]), past_key_values=cache,
                    position_ids=torch.tensor([[P]]), use_cache=True)
    hf_logits = out.logits[0, -1].numpy()
    logits, nxt = DecoderOracle(s, w).step(tok, P, kc, vc)
    # The oracle rounds the new key/value rows to bf16 before attending; the
    # library attends to them unrounded. That single rounding bounds the gap.
    rel = np.linalg.norm(logits[0] - hf_logits) / np.linalg.norm(hf_logits)
    assert rel < 2e-3, rel
    assert nxt[0] == int(np.argmax(hf_logits))
    # appended rows: the library's rotated key / value rounded to bf16, within
    # one bf16 step (the library forms rotary angles in float32, and layer 1
    # sees layer 0's rounding); the torch-library test above checks them exactly
    for l in range(s.n_layers):
        layer = cache.layers[l]
        for mine, lib in ((kc, layer.keys), (vc, layer.values)):
            a = f64_to_bf16(lib[0, :, P].numpy())
            b = mine[l, 0, :, P]
            if l == 0:
                d = np.abs(a.astype(np.int32) - b.astype(np.int32))
                assert d.max() <= 1 and np.mean(d != 0) < 0.02
            else:
                va, vb = bf16_to_f64(a), bf16_to_f64(b)
                assert np.linalg.norm(va - vb) <= 5e-3 * np.linalg.norm(vb)
