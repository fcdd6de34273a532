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


# ---------------------------------------------------------------------------
# The attention half of decode_layer (RMSNorm -> v -> bf16 -> one-token
# attention -> o -> residual -> bf16), pinned on layers whose effective
# weights have a known structure.
# ---------------------------------------------------------------------------
def _select_layer(out, inp, sel, scale):
    """Two paths whose effective weight is scale[i] at column sel[i] and 0
    elsewhere: g_1 = g_2 = scale/2, h_1 = h_2 = 1, B_1 = +1 everywhere and
    B_2 = +1 only at sel[i] (so g_1 B_1 + g_2 B_2 is scale or 0), exact in
    float64 for fp16 scales."""
    s1 = np.zeros((out, inp), bool)
    s2 = np.ones((out, inp), bool)
    s2[np.arange(out), sel] = False
    half = (np.asarray(scale, np.float64) / 2).astype(np.float16)
    assert np.array_equal(half.astype(np.float64) * 2, np.asarray(scale, np.float64))
    one = np.ones(inp, np.float16)
    return Derived(s1, s2, half, one, half.copy(), one.copy())


def _zero_layer(d):
    return Derived(d.s1, d.s2, np.zeros_like(d.g1), d.h1, np.zeros_like(d.g2), d.h2)


def _attention_case(seed=21):
    H, n_heads, n_kv, hd, F = 64, 8, 2, 8, 48
    kv = n_kv * hd
    rng = np.random.default_rng(seed)
    sel_v = rng.permutation(H)[:kv]
    sel_k = rng.permutation(H)[:kv]
    sel_o = rng.permutation(H)
    # fp16 scales whose products with bf16 values need more than 8 bits
    c_v = (rng.uniform(0.3, 0.9, kv) * 2048).round().astype(np.float16) / np.float16(2048)
    c_k = (rng.uniform(0.3, 0.9, kv) * 2048).round().astype(np.float16) / np.float16(2048)
    d_o = (rng.uniform(0.5, 1.5, H) * 1024).round().astype(np.float16) / np.float16(1024)
    mats = {
        "q": derive(weight_f32(H, H, seed + 1).numpy()),
        "k": _select_layer(kv, H, sel_k, c_k),
        "v": _select_layer(kv, H, sel_v, c_v),
        "o": _select_layer(H, H, sel_o, d_o),
        "gate": derive(weight_f32(F, H, seed + 2).numpy()),
        "up": derive(weight_f32(F, H, seed + 3).numpy()),
        # zero down scales: the MLP half returns its input unchanged
        "down": _zero_layer(derive(weight_f32(H, F, seed + 4).numpy())),
    }
    cfg = {"n_heads": n_heads, "n_kv_heads": n_kv, "head_dim": hd, "rms_eps": 1e-5}
    x = bf16_values(act_bf16(2, H, seed + 5))
    parts = dict(H=H, n_heads=n_heads, n_kv=n_kv, hd=hd, sel_v=sel_v, sel_k=sel_k, sel_o=sel_o,
                 c_v=c_v.astype(np.float64), c_k=c_k.astype(np.float64), d_o=d_o.astype(np.float64))
    return x, mats, cfg, parts


def _expected_attention_half(x, p, use_k=False, round_v=True, group=lambda h, rep, n_kv: h // rep,
                             round_o=False, resid_from_norm=False):
    """The attention half written out element by element from the structure
    of the layers; the keyword arguments switch on plausible mistakes."""
    n = rmsnorm_bf16(x)
    B, H = x.shape
    sel, c = (p["sel_k"], p["c_k"]) if use_k else (p["sel_v"], p["c_v"])
    kv = p["n_kv"] * p["hd"]
    v = np.empty((B, kv))
    for b in range(B):
        for i in range(kv):
            v[b, i] = c[i] * n[b, sel[i]]
    if round_v:
        v = bf16_rne(v)
    rep = p["n_heads"] // p["n_kv"]
    a = np.empty((B, H))
    for b in range(B):
        for hh in range(p["n_heads"]):
            grp = group(hh, rep, p["n_kv"])
            for dd in range(p["hd"]):
                a[b, hh * p["hd"] + dd] = v[b, grp * p["hd"] + dd]
    o = np.empty((B, H))
    for b in range(B):
        for i in range(H):
            o[b, i] = p["d_o"][i] * a[b, p["sel_o"][i]]
    if round_o:
        o = bf16_rne(o)
    base = n if resid_from_norm else x
    return bf16_rne(base + o)


def test_decode_layer_zero_o_is_mlp_block():
    # o scales of zero: the attention half adds nothing and the layer is its MLP block
    x, mats, cfg, _ = _attention_case(31)
    mats["o"] = _zero_layer(derive(weight_f32(64, 64, 77).numpy()))
    mats["down"] = derive(weight_f32(64, 48, 78).numpy())
    assert np.array_equal(decode_layer(x, mats, cfg), mlp_block(x, mats["gate"], mats["up"], mats["down"]))


def test_decode_layer_attention_half_selection_structure():
    x, mats, cfg, p = _attention_case()
    # the structured layers give the intended effective weights
    n = rmsnorm_bf16(x)
    vv = gemv(mats["v"], n)
    assert np.array_equal(vv, p["c_v"][None, :] * n[:, p["sel_v"]])
    want = _expected_attention_half(x, p)
    assert np.array_equal(decode_layer(x, mats, cfg), want)
    # each plausible mistake changes the result on this case
    mistakes = {
        "k used for v": dict(use_k=True),
        "v not rounded to bf16": dict(round_v=False),
        "wrong key/value group": dict(group=lambda h, rep, n_kv: h % n_kv),
        "o rounded before the residual add": dict(round_o=True),
        "residual taken from the normalised input": dict(resid_from_norm=True),
    }
    for name, kw in mistakes.items():
        assert not np.array_equal(_expected_attention_half(x, p, **kw), want), name


def test_decode_layer_gqa_one_group_per_head():
    # as many key/value heads as query heads: head h reads group h
    x, mats, cfg, p = _attention_case(41)
    H, hd = p["H"], p["hd"]
    n_heads = H // hd
    kvsel = np.random.default_rng(3).permutation(H)
    cv = np.full(H, 0.75, np.float16)
    mats["k"] = _select_layer(H, H, kvsel, cv)
    mats["v"] = _select_layer(H, H, kvsel, cv)
    cfg = dict(cfg, n_heads=n_heads, n_kv_heads=n_heads)
    n = rmsnorm_bf16(x)
    a = bf16_rne(0.75 * n[:, kvsel])     # attention output = v, column for column
    want = bf16_rne(x + p["d_o"][None, :] * a[:, p["sel_o"]])
    assert np.array_equal(decode_layer(x, mats, cfg), want)
