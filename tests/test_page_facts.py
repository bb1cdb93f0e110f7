"""The synthetic workloads carry the structure the pages fix (tests/golden/page_facts.json)."""
import json
import os

import synth

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def fact(name):
    return FACTS[name]["value"]


def test_format_constants():
    assert synth.GROUP == fact("group_size")
    w = synth.affine_weights(fact("weight_code_bits"), 2, 128, cfg=1, set_id=0)
    assert w.scales.shape == (2, 128 // fact("group_size"))
    r = synth.affine_weights(fact("router_code_bits"), 2, 128, cfg=1, set_id=0)
    assert r.wq.shape == (2, 128 * fact("router_code_bits") // 32)


def test_moe_workloads_follow_the_pages():
    for name in ("c3_moe_decode", "c4_moe_prefill"):
        c = synth.CONFIGS[name]
        assert c["top_k"] == fact("top_k")
        assert c["layers"] == fact("layers")
        assert c["H"] % fact("group_size") == 0 and c["I"] % fact("group_size") == 0
    assert synth.CONFIGS["c4_moe_prefill"]["T"] <= fact("prefill_chunk_max_tokens")
    assert synth.CONFIGS["c4_chunk"]["M"] <= fact("prefill_chunk_max_tokens")


def test_moe_shapes_fit_the_stated_parameter_counts():
    # shape sanity only: the FFN parameters of the synthetic layer stack stay
    # below the stated totals (attention and embeddings make up the rest)
    c = synth.CONFIGS["c3_moe_decode"]
    H, I, Is, E, L, k = c["H"], c["I"], c["Is"], c["E"], c["layers"], c["top_k"]
    expert = 3 * H * I
    per_layer_total = E * expert + 3 * H * Is + E * H
    per_layer_active = k * expert + 3 * H * Is + E * H
    assert 0.8 * fact("total_params_billion") * 1e9 < L * per_layer_total < fact("total_params_billion") * 1e9
    assert L * per_layer_active < fact("active_params_billion") * 1e9
