"""GPU parity with the modes in a chosen chain order (tt_linear_desc.chain_perm)
against the fp64 oracle, on both contraction orders.

The pages leave the order of the modes in the chain open; their rank table
for the compressed encoder (project page, results) caps the Q/K/V ranks as
(12,30,30,30,12) for modes (12,8,8) x (12,8,8), i.e. the end cores carry the
12-wide modes: output modes in listed order, then the input modes reversed
(chain_perm (0,1,2,5,4,3)).  W's row and column indices stay the listed
mixed-radix ones, so the results must match the oracle's weight for the same
permutation.  Same bounds as elsewhere (1e-5 fp32, 2e-2 bf16 rel-L2 per
tensor; dead-slice gradients exactly 0).
"""

import numpy as np
import pytest
import torch

import synth
from test_gpu_tt_linear import MERGED, SEQUENTIAL, _check, _run

pytestmark = pytest.mark.gpu

MIRRORED = (0, 1, 2, 5, 4, 3)


@pytest.mark.parametrize("path,T", [(MERGED, 300), (SEQUENTIAL, 3)])
@pytest.mark.parametrize("li", [0, 4, 5])
def test_mirrored_layout_config2(li, path, T):
    base = synth.config_layers(2, 30)[li]
    spec = synth.LayerSpec(base.name, base.out_modes, base.in_modes, 30, chain_perm=MIRRORED)
    layer = synth.make_tt_layer(2, 700 + li, spec, T, 0.40, "bf16")
    _check(spec, layer, "bf16", path=path)


@pytest.mark.parametrize("path,T", [(MERGED, 200), (SEQUENTIAL, 5)])
def test_mirrored_layout_config1_fp32(path, T):
    base = synth.config_layers(1)[4]
    spec = synth.LayerSpec(base.name, base.out_modes, base.in_modes, 30, chain_perm=MIRRORED)
    layer = synth.make_tt_layer(1, 710, spec, T, 0.25, "f32")
    _check(spec, layer, "f32", path=path)


PERMS = [
    (1, 0, 3, 2),  # both blocks reversed, outputs first
    (3, 2, 0, 1),  # inputs first, output block reversed
    (2, 3, 1, 0),  # inputs first, input block reversed
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("path,T", [(MERGED, 130), (SEQUENTIAL, 4)])
@pytest.mark.parametrize("perm", PERMS)
def test_small_chains_in_any_block_order(perm, path, T, dtype):
    spec = synth.LayerSpec("perm", (2, 3), (3, 4), 5, chain_perm=perm)
    layer = synth.make_tt_layer(720, sum(perm), spec, T, 0.3, dtype)
    _check(spec, layer, dtype, path=path)


@pytest.mark.parametrize("path,T", [(MERGED, 150), (SEQUENTIAL, 6)])
def test_longer_chain_permuted(path, T):
    spec = synth.LayerSpec("perm6", (2, 3, 2), (3, 2, 4), 6, chain_perm=(1, 2, 0, 4, 5, 3))
    layer = synth.make_tt_layer(730, 0, spec, T, 0.34, "f32")
    _check(spec, layer, "f32", path=path)


def test_identity_permutation_is_bitwise_the_default():
    spec = synth.config_layers(2, 30)[0]
    perm_spec = synth.LayerSpec(spec.name, spec.out_modes, spec.in_modes, 30, chain_perm=(0, 1, 2, 3, 4, 5))
    layer = synth.make_tt_layer(2, 740, spec, 257, 0.40, "bf16")
    a = _run(spec, layer, "bf16")
    b = _run(perm_spec, layer, "bf16")
    for u, v in zip([a[0], a[1]] + a[2], [b[0], b[1]] + b[2]):
        assert np.array_equal(u, v)
