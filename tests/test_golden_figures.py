"""The figures the model doc states, against the arithmetic they imply.
Fixture: tests/golden/model_doc_figures.json (each entry cites its section)."""
import json
import math
import os

from global_attention_mimo_amd import synth

FIG = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "model_doc_figures.json")))


def val(name):
    return FIG[name]["value"]


def test_value_scale_is_the_stated_square_root():
    # MiMoV2FlashConfig: 0.707 approximates sqrt(hidden_size / (heads * v_head_dim)).
    exact = math.sqrt(val("hidden_size") / (val("num_attention_heads") * val("v_head_dim")))
    assert abs(exact - val("attention_value_scale")) < 5e-4


def test_window_129_is_128_previous_tokens_plus_self():
    # Key features says a 128-token window, the config says sliding_window=129:
    # 128 earlier keys plus the query's own key.
    assert val("sliding_window") == val("window_tokens") + 1


def test_layer_pattern_is_5_to_1():
    types = synth.hybrid_layer_types(val("num_hidden_layers"))
    swa, ga = types.count(0), types.count(1)
    assert (swa, ga) == (40, 8)
    assert swa * val("swa_to_ga_ratio")[1] == ga * val("swa_to_ga_ratio")[0]


def _kv_rows(L, layers):
    # Cached positions per sequence per layer: GA keeps all L, SWA keeps the
    # last sliding_window-1 (the ring); the new token is the extra key.
    ring = val("sliding_window") - 1
    return sum(L if t == 1 else min(L, ring) for t in layers)


def test_kv_cache_reduction_about_six():
    layers = synth.hybrid_layer_types(val("num_hidden_layers"))
    all_ga = [1] * len(layers)
    ratios = {L: _kv_rows(L, all_ga) / _kv_rows(L, layers) for L in (4096, val("native_context"), val("extended_context"))}
    # "about 1/6": within 3% of 6 at the native and extended context lengths,
    # never above 6, and increasing towards 6 with length.
    for L in (val("native_context"), val("extended_context")):
        assert abs(ratios[L] - val("kv_cache_reduction")) / 6 < 0.03, ratios
    assert all(r < 6 for r in ratios.values())
    assert ratios[4096] < ratios[val("native_context")] < ratios[val("extended_context")]
    assert abs(ratios[val("native_context")] - 48 * 32768 / (8 * 32768 + 40 * 128)) < 1e-12
