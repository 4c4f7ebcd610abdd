"""Printed values of the pages (tests/golden/, each entry cited there) against the dimension
presets and the oracle's cache layout."""
import json
import os

import mla_synth as S
import oracle.mla_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "deepseek_v2_mla_printed_values.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_presets_match_printed_hyper_parameters():
    g = _golden()
    for key, dims in (("v2", S.V2), ("v2_lite", S.V2_LITE)):
        for f in ("d_model", "n_h", "d_h", "d_c", "d_cq", "d_hr"):
            assert getattr(dims, f) == g[key][f], (key, f)


def test_cache_matches_printed_gqa_equivalence():
    """GQA with g groups caches 2 * g * d_h values per token and layer (one key and one value
    per group); the oracle's latent entry must equal that at the printed g."""
    g = _golden()["kv_cache_equivalent_gqa_groups"]["groups"]
    for dims in (S.V2, S.V2_LITE):
        assert O.cache_values_per_token(dims) == 2 * g * dims.d_h
