"""The allocation-free packed layer, moge_layer_forward_packed_noalloc, against
moge_layer_forward_packed with a caller-owned workspace: the same bits for every
output, on two calls in a row with the second one smaller (the fixed scratch array
keeps the first call's contents), and its size limit."""
import numpy as np
import pytest

from synth import inputs as S
from synth.configs import C1
from tests.gpu_util import dims_of, layer_inputs, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _outputs(lib, cfg, T, dt):
    import torch
    e = lambda shape, t: torch.empty(shape, dtype=t, device="cuda")
    return dict(y=e((T, cfg.d), dt), logits=e((T, cfg.N), torch.float32),
                idx=e((T, cfg.K), torch.int32), gate=e((T, cfg.K), torch.float32),
                gc=e((cfg.M,), torch.int32))


def _call(lib, dims, dw, packed, bias, out, ws=None):
    kw = dict(logits_out=out["logits"], topk_idx_out=out["idx"], topk_gate_out=out["gate"],
              group_counts_out=out["gc"])
    if ws is None:
        lib.layer_forward_packed_noalloc(dims, dw["x"], dw["w_router"], bias, packed, out["y"], **kw)
    else:
        lib.layer_forward_packed(dims, dw["x"], dw["w_router"], bias, packed, out["y"], ws, **kw)


def test_noalloc_layer_equals_workspace_layer(lib):
    import torch
    cfg = C1
    # 456 tokens with a Zipf-biased router, then 64 plain tokens: the second call
    # is smaller and finds the first one's intermediates in the scratch array
    cases = [(456, S.zipf_bias(cfg.N, 1.2)), (64, None)]
    _, dw = layer_inputs(cfg, 64)
    dims0 = dims_of(lib, cfg, 64)
    packed = torch.empty(lib.packed_weights_size(dims0), dtype=torch.uint8, device="cuda")
    lib.pack_weights(dims0, dw["w_gate"], dw["w_up"], dw["w_down"], dw["ws_gate"], dw["ws_up"],
                     dw["ws_down"], packed)
    for T, bias_h in cases:
        _, dw = layer_inputs(cfg, T)
        dims = dims_of(lib, cfg, T)
        assert lib.workspace_size(dims) <= lib.NOALLOC_SCRATCH_BYTES
        bias = to_dev(bias_h, "f32") if bias_h is not None else None
        ref = _outputs(lib, cfg, T, dw["x"].dtype)
        got = _outputs(lib, cfg, T, dw["x"].dtype)
        ws = torch.empty(lib.workspace_size(dims), dtype=torch.uint8, device="cuda")
        say("noalloc layer", T, "bias" if bias_h is not None else "no bias")
        _call(lib, dims, dw, packed, bias, ref, ws)
        _call(lib, dims, dw, packed, bias, got)
        torch.cuda.synchronize()
        for k in ref:
            np.testing.assert_array_equal(to_host(got[k]), to_host(ref[k]), err_msg=f"T={T} {k}")
        assert (to_host(got["gc"]) == T * cfg.kp).all()


def test_noalloc_rejects_dims_beyond_the_scratch_array(lib):
    import torch
    cfg = C1
    T = 4096
    dims = dims_of(lib, cfg, T)
    assert lib.workspace_size(dims) > lib.NOALLOC_SCRATCH_BYTES
    x = torch.empty((T, cfg.d), dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    packed = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(lib.MogeError) as ei:
        lib.layer_forward_packed_noalloc(dims, x, x, None, packed, y)
    assert ei.value.status == 2   # MOGE_ERR_UNSUPPORTED, before anything is enqueued
    assert "scratch" in str(ei.value)
