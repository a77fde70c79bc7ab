"""The Python binding's argument checks, without a GPU: the C ABI takes bare
pointers, so the binding refuses tensors whose dtype, element count or
layout would make libblock read or write past them, before any call."""
import pytest
import torch

from transformer_decoder_block_amd import binding as L
from transformer_decoder_block_amd import synth


def cfg(name):
    return L.make_config(synth.WORKLOADS[name] if name in synth.WORKLOADS
                         else synth.SMALL[name])


def raises(status, fn):
    with pytest.raises(L.BlockError) as e:
        fn()
    assert e.value.status == status, str(e.value)


def test_wrong_dtype_shape_layout_and_host_memory_are_refused():
    shp = (2, 5, 8)
    raises(L.BLK_E_DTYPE, lambda: L.check_tensor("x", torch.zeros(shp), shp, L.BLK_BF16))
    raises(L.BLK_E_DTYPE, lambda: L.check_tensor(
        "mask", torch.ones((2, 5), dtype=torch.bool), (2, 5), L.BLK_I32))
    raises(L.BLK_E_DTYPE, lambda: L.check_tensor(
        "mask", torch.ones((2, 5), dtype=torch.int64), (2, 5), L.BLK_I32))
    raises(L.BLK_E_SHAPE, lambda: L.check_tensor(
        "x", torch.zeros((2, 5, 7), dtype=torch.bfloat16), shp, L.BLK_BF16))
    raises(L.BLK_E_SHAPE, lambda: L.check_tensor(
        "x", torch.zeros((2, 8, 5), dtype=torch.bfloat16).transpose(1, 2), shp, L.BLK_BF16))
    # right dtype, count and layout, but host memory
    raises(L.BLK_E_NULL, lambda: L.check_tensor(
        "x", torch.zeros(shp, dtype=torch.bfloat16), shp, L.BLK_BF16))
    raises(L.BLK_E_NULL, lambda: L.check_tensor("x", None, shp, L.BLK_BF16))


@pytest.mark.parametrize("name", list(synth.WORKLOADS) + list(synth.SMALL))
def test_weight_shapes_match_the_generated_weights(name):
    """Every weight the configuration reads has the shape the input
    generator draws, and nothing the generator draws is left unchecked."""
    w = synth.WORKLOADS.get(name) or synth.SMALL[name]
    shapes = {k: v for k, v in synth.weight_shapes(w).items()
              if k not in ("xielu_alpha_p", "xielu_alpha_n")}
    need = L.weight_shapes(L.make_config(w))
    for n, s in need.items():
        assert tuple(shapes[n]) == s, n
    assert set(need) == set(shapes), set(shapes) ^ set(need)


def test_tap_shapes_cover_every_tap():
    c = cfg("afmoe_small")
    assert set(L.tap_shapes(c, 2, 3)) == set(L.TAP_NAMES)
