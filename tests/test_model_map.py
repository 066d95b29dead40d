"""CPU: layer maps of the whole-model composition (summary page §C.3: an
independent first layer, then groups of G = 4, or 7 groups of 8 and one of 4)."""
import pytest

from sparse_attention_token_absorb_amd.model import METHODS, LayerMap


def test_layer_maps_of_the_pages():
    lm4 = LayerMap.grouped(61, 4)
    lm8 = LayerMap.grouped(61, 8)
    assert lm4.independent == (0,) and lm4.group_sizes() == [4] * 15
    assert lm8.independent == (0,) and lm8.group_sizes() == [8] * 7 + [4]
    for lm in (lm4, lm8):
        layers = list(lm.independent) + [l for grp in lm.groups for l in grp]
        assert layers == list(range(61))  # every layer exactly once, in order


def test_layer_map_edges():
    assert LayerMap.grouped(1, 4).groups == ()
    assert LayerMap.grouped(5, 4, independent=0).group_sizes() == [4, 1]
    with pytest.raises(ValueError):
        LayerMap.grouped(4, 0)
    assert METHODS == ("dsa", "latentindex", "hs", "indexcache")
