"""Pins for the oracle's decode glue (not gpu): closed forms for SiLU,
RMSNorm and the one-token attention stand-in, and the MLP block against a
composition of independently pinned pieces on a case with known structure."""
import math

import numpy as np

from oracle import (derive, Derived, rmsnorm_bf16, silu, attention_1tok, mlp_block,
                    decode_layer, bf16_rne, gemv)
from synth.inputs import weight_f32, act_bf16, bf16_values


def test_silu_closed_forms():
    assert silu(np.array([0.0]))[0] == 0.0
    z = np.linspace(-8, 8, 101)
    # silu(z) - silu(-z) = z (sigmoid(z) + sigmoid(-z) = 1)
    assert np.allclose(silu(z) - silu(-z), z, rtol=0, atol=1e-14)
    assert abs(silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16


def test_rmsnorm_closed_forms():
    c = 3.0
    x = np.full((1, 16), c)
    # mean(x^2) = c^2 -> c / sqrt(c^2 + eps)
    assert np.all(rmsnorm_bf16(x, 1e-5) == bf16_rne(np.array(c / math.sqrt(c * c + 1e-5))))
    x = np.array([[3.0, -4.0]])      # rms = sqrt(12.5)
    ref = bf16_rne(x / math.sqrt(12.5 + 1e-5))
    assert np.array_equal(rmsnorm_bf16(x), ref)


def test_attention_stand_in_gqa_mapping():
    n_heads, n_kv, hd = 8, 2, 4
    v = np.arange(n_kv * hd, dtype=np.float64)[None, :]
    a = attention_1tok(v, n_heads, n_kv, hd)[0]
    for h in range(n_heads):
        grp = h // 4
        assert np.array_equal(a[h * hd:(h + 1) * hd], v[0, grp * hd:(grp + 1) * hd])


def test_mlp_block_zero_down_is_identity():
    hidden, ffn = 64, 160
    g = derive(weight_f32(ffn, hidden, 1).numpy())
    u = derive(weight_f32(ffn, hidden, 2).numpy())
    dn = derive(weight_f32(hidden, ffn, 3).numpy())
    zero = Derived(dn.s1, dn.s2, np.zeros_like(dn.g1), dn.h1, np.zeros_like(dn.g2), dn.h2)
    x = bf16_values(act_bf16(2, hidden, 4))
    assert np.array_equal(mlp_block(x, g, u, zero), x)


def test_mlp_block_gate_sign_structure():
    # all planes +1 with equal scales make gate == up: z = bf16(silu(t) * t) >= 0
    hidden, ffn = 32, 48
    rng = np.random.default_rng(5)
    f = lambda n: rng.uniform(0.01, 0.03, n).astype(np.float16)
    gs, hs = f(ffn), f(hidden)
    mk = lambda o, i, g, h: Derived(np.zeros((o, i), bool), np.zeros((o, i), bool), g, h, g, h)
    gate, up = mk(ffn, hidden, gs, hs), mk(ffn, hidden, gs, hs)
    dn = mk(hidden, ffn, f(hidden), f(ffn))
    x = bf16_values(act_bf16(1, hidden, 6))
    n = rmsnorm_bf16(x)
    t = gemv(gate, n)
    z = bf16_rne(silu(t) * t)
    assert np.all(z >= 0)
    ref = bf16_rne(x + gemv(dn, z))
    assert np.array_equal(mlp_block(x, gate, up, dn), ref)


def test_decode_layer_without_attention_is_mlp_block():
    hidden, ffn = 64, 96
    mats = {"gate": derive(weight_f32(ffn, hidden, 7).numpy()),
            "up": derive(weight_f32(ffn, hidden, 8).numpy()),
            "down": derive(weight_f32(hidden, ffn, 9).numpy())}
    x = bf16_values(act_bf16(1, hidden, 10))
    cfg = {"n_heads": 4, "n_kv_heads": 2, "head_dim": 16, "rms_eps": 1e-5}
    assert np.array_equal(decode_layer(x, mats, cfg), mlp_block(x, mats["gate"], mats["up"], mats["down"]))
