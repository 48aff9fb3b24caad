"""The no-allocation backward, tt_linear_bwd_noalloc, called through the C
ABI, against tt_linear_bwd with a caller-provided scratch buffer.

Both run the same kernels with the same plan, so dX and every dG must agree
bitwise.  Two calls in a row go through the library's one scratch array, the
second with fewer tokens (a ragged tail) and then a different layer shape, so
a call that read what the previous call left there would show.
"""

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _layer(cfg, li, rank, T, dtype):
    import tensor_train_compressed_tt_amd as ttc

    spec = synth.config_layers(cfg, rank)[li]
    L = synth.make_tt_layer(cfg, 700 + li, spec, T, 0.4, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    mod = ttc.TTLinear(spec.out_modes, spec.in_modes, spec.ranks, tdt, spec.in_first)
    if dtype == "bf16":
        x = torch.from_numpy(L["x_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
        dy = torch.from_numpy(L["dy_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        x = torch.from_numpy(L["x"]).to(dev)
        dy = torch.from_numpy(L["dy"]).to(dev)
    cores = [torch.from_numpy(c).to(dev) for c in L["cores"]]
    D = [torch.from_numpy(v).to(dev) for v in L["D"]]
    return mod, x, dy, cores, D


def _both(mod, x, dy, cores, D):
    import tensor_train_compressed_tt_amd as ttc

    T = int(x.shape[0])
    _, saved = mod.forward(x, cores, D)
    sb, cb = mod.workspace(T)
    assert cb <= ttc.NOALLOC_SCRATCH_BYTES
    G = [c.data_ptr() for c in cores]
    Dp = [v.data_ptr() for v in D]
    stream = torch.cuda.current_stream().cuda_stream
    scratch = torch.empty(max(cb, 256), dtype=torch.uint8, device=x.device)
    dx_ref = torch.empty((T, mod.n_in), dtype=x.dtype, device=x.device)
    dG_ref = [torch.empty(s, dtype=torch.float32, device=x.device) for s in mod.core_shapes]
    ttc.tt_linear_bwd(mod.desc, T, x.data_ptr(), dy.data_ptr(), G, Dp, saved.data_ptr(), sb, dx_ref.data_ptr(),
                      [g.data_ptr() for g in dG_ref], scratch.data_ptr(), cb, stream)
    dx = torch.full((T, mod.n_in), float("nan"), dtype=x.dtype, device=x.device)
    dG = [torch.full(s, float("nan"), dtype=torch.float32, device=x.device) for s in mod.core_shapes]
    ttc.tt_linear_bwd_noalloc(mod.desc, T, x.data_ptr(), dy.data_ptr(), G, Dp, saved.data_ptr(), sb,
                              dx.data_ptr(), [g.data_ptr() for g in dG], stream)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx_ref), "dX differs"
    for k, (a, b) in enumerate(zip(dG, dG_ref)):
        assert torch.equal(a, b), f"dG{k} differs"


def test_noalloc_backward_matches_backward_with_scratch():
    # FFN1 768 -> 3072, bf16, rank 30, 8192 tokens; then 777 tokens of the
    # same layer; then a fp32 768 -> 768 layer at rank 64 (another plan)
    _both(*_layer(2, 4, 30, 8192, "bf16"))
    _both(*_layer(2, 4, 30, 777, "bf16"))
    _both(*_layer(1, 0, 64, 1000, "f32"))


def test_noalloc_refuses_oversized_scratch():
    import tensor_train_compressed_tt_amd as ttc

    mod, x, dy, cores, D = _layer(4, 4, 64, 64, "bf16")
    T = 16384  # config-4 FFN1 at full size: its scratch exceeds the array
    _, cb = mod.workspace(T)
    assert cb > ttc.NOALLOC_SCRATCH_BYTES
    with pytest.raises(ttc.TTCError) as e:
        ttc.tt_linear_bwd_noalloc(mod.desc, T, x.data_ptr(), dy.data_ptr(), [c.data_ptr() for c in cores],
                                  [v.data_ptr() for v in D], x.data_ptr(), 1 << 30, None,
                                  [c.data_ptr() for c in cores], 0)
    assert e.value.code == 6
