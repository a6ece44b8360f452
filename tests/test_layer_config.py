"""Per-layer config resolution (host-only C ABI) against the oracle's Python
`re` version of the same rules, on rule sets covering exact keys, pattern
keys, rule order, keys that are not patterns, keys that do not compile, the
unquantized fallback and fused layers. No GPU involved."""
import itertools

import pytest

import autoround_signsgd_rounding_amd as ar
import oracle as O

DEF = (4, 128, False)
RULES = [
    (r"model\.layers\.\d+\.mlp\..*", {"bits": 8}),
    ("model.layers.0.mlp.down_proj", {"bits": 2, "group_size": 64}),
    (r"model\.layers\.(1|2)\.self_attn\.[qkv]_proj", {"bits": 3, "sym": True}),
    ("model.layers.0.mlp", {"bits": 8}),
    ("lm_head", {"group_size": 32}),
    ("layers.(", {"bits": 2}),                         # does not compile: skipped
    (r"embed.*", {"sym": True}),
    (r"model\.layers\.[0-9]{2}\..*", {"group_size": -1}),
    ("m.q_proj", {"bits": 8}), ("m.k_proj", {"bits": 8}), ("m.v_proj", {"bits": 4}),
    ("e.experts.0.w1", {"bits": 3}), ("e.experts.1.w1", {"bits": 3}),
    (r"model\.layers\.4", {"bits": 2}),                 # matches a prefix of longer names only
]
NAMES = [
    "model.layers.0.mlp.down_proj", "model.layers.0.mlp.up_proj", "model.layers.1.mlp.gate_proj",
    "model.layers.1.self_attn.q_proj", "model.layers.2.self_attn.v_proj",
    "model.layers.3.self_attn.k_proj", "model.layers.12.self_attn.o_proj",
    "x.model.layers.1.self_attn.q_proj", "model.layers.0.mlp", "modelXlayersX0Xmlp", "lm_head",
    "embed_tokens", "norm", "layers.(", "layers.7", "m.q_proj", "e.experts.0.w1",
    "model.layers.4.self_attn.o_proj", "model.layers.4",
]


@pytest.mark.parametrize("quantized", [True, False])
def test_resolution_matches_oracle(quantized):
    for name in NAMES:
        want = O.resolve_layer_config(RULES, DEF, quantized, name)
        got = ar.resolve_layer_config(RULES, DEF, quantized, name)
        assert got == tuple(want), (name, got, want)


def test_rule_order_and_subsets():
    """Every ordered pair of rules, every name: the first matching pattern
    decides, and exact keys beat patterns wherever they stand."""
    for r1, r2 in itertools.permutations(RULES[:8], 2):
        for name in NAMES:
            assert ar.resolve_layer_config([r1, r2], DEF, True, name) == \
                tuple(O.resolve_layer_config([r1, r2], DEF, True, name)), (r1, r2, name)


def test_no_rules():
    assert ar.resolve_layer_config([], DEF, True, "a") == DEF
    assert ar.resolve_layer_config([], DEF, False, "a") == (16, -1, True)


def test_fused_layers():
    assert ar.resolve_fused_config(RULES, DEF, True, "m.qk", ["m.q_proj", "m.k_proj"]) == \
        O.resolve_fused_config(RULES, DEF, True, "m.qk", ["m.q_proj", "m.k_proj"])
    with pytest.raises(ar.ArError):
        ar.resolve_fused_config(RULES, DEF, True, "m.qkv_proj",
                                ["m.q_proj", "m.k_proj", "m.v_proj"])
    with pytest.raises(ValueError):
        O.resolve_fused_config(RULES, DEF, True, "m.qkv_proj",
                               ["m.q_proj", "m.k_proj", "m.v_proj"])
    for layer in ("e.experts", "f.experts"):
        assert ar.resolve_fused_config(RULES, DEF, True, layer) == \
            tuple(O.resolve_fused_config(RULES, DEF, True, layer)), layer
    # two keys start with this name and disagree: both sides reject it
    with pytest.raises(ar.ArError):
        ar.resolve_fused_config(RULES, DEF, True, "model.layers.0.mlp")
    with pytest.raises(ValueError):
        O.resolve_fused_config(RULES, DEF, True, "model.layers.0.mlp")
    bad = RULES + [("e.experts.2.w1", {"bits": 2})]
    with pytest.raises(ar.ArError):
        ar.resolve_fused_config(bad, DEF, True, "e.experts")


def test_fused_layer_with_empty_sub_layer_list():
    """An explicit empty sub-layer list has no config to agree on: both sides
    reject it ([SGLang] "4. FusedMoE와 Fused QKV 처리" requires one config
    shared by the sub-layers), while no list at all (None) is the fused-expert
    rule, which collects the sub-layers from the rule keys."""
    rules = [("experts.0", {"bits": 8}), ("experts.1", {"bits": 8})]
    with pytest.raises(ValueError):
        O.resolve_fused_config(rules, DEF, True, "experts", [])
    with pytest.raises(ar.ArError):
        ar.resolve_fused_config(rules, DEF, True, "experts", [])
    assert ar.resolve_fused_config(rules, DEF, True, "experts") == \
        tuple(O.resolve_fused_config(rules, DEF, True, "experts")) == (8, 128, False)


def test_null_arguments():
    import ctypes
    out = ar.ArLayerQConfig()
    d = ar.ArLayerQConfig(4, 128, 0)
    assert ar.lib.ar_resolve_layer_config(None, 1, ctypes.byref(d), 1, b"x",
                                          ctypes.byref(out)) == 1
    assert ar.lib.ar_resolve_layer_config(None, 0, None, 1, b"x", ctypes.byref(out)) == 1
    assert ar.lib.ar_resolve_layer_config(None, 0, ctypes.byref(d), 1, None,
                                          ctypes.byref(out)) == 1
    assert ar.lib.ar_resolve_layer_config(None, 0, ctypes.byref(d), 1, b"x",
                                          ctypes.byref(out)) == 0
