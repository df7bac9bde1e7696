"""The layer call under HIP stream capture.

The library never allocates, never synchronises and never reads device data on
the host, so one layer call can be captured into a graph.  The graph is replayed
several times with eager work and synchronisations between the replays, and every
replay must give the eager call's output bit for bit.  Covered: the row-major,
packed and int8-weight layers, and the packed layer at the prefill sizes (256-row
tiles; at 16384 tokens the persistent gate/up tiles whose round counters the
routing kernel of the same call zeroes)."""
import numpy as np
import pytest

from synth import inputs as S
from synth.configs import C0, C1, C2, C3, C4
from tests.gpu_util import dims_of, layer_inputs, say, to_host


def _replays_equal_eager(cfg, T, y, idx, call):
    import torch
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        call()
    torch.cuda.synchronize()
    y_ref, idx_ref = to_host(y), to_host(idx)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        call()
    torch.cuda.synchronize()
    other = torch.from_numpy(S.make_x(cfg, T=T, seed=11).view(np.int16)
                             if cfg.dtype == "bf16" else S.make_x(cfg, T=T, seed=11)).cuda()
    for rep in range(4):
        y.zero_()
        idx.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host(y), y_ref, err_msg=f"replay {rep}")
        np.testing.assert_array_equal(to_host(idx), idx_ref, err_msg=f"replay {rep}")
        # eager work between replays
        _ = float(other.float().square().sum().item())


def _buffers(lib, cfg, T, dw):
    import torch
    dims = dims_of(lib, cfg, T)
    ws = torch.empty(lib.workspace_size(dims), dtype=torch.uint8, device="cuda")
    y = torch.empty((T, cfg.d), dtype=dw["x"].dtype, device="cuda")
    idx = torch.empty((T, dims.K), dtype=torch.int32, device="cuda")
    return dims, ws, y, idx


@pytest.mark.gpu
@pytest.mark.parametrize("cfg,T", [(C0, 64), (C1, 64), (C2, 456)])
def test_layer_graph_replays_equal_eager(lib, cfg, T):
    inp, dw = layer_inputs(cfg, T)
    dims, ws, y, idx = _buffers(lib, cfg, T, dw)

    def call():
        lib.layer_forward(dims, dw["x"], dw["w_router"], dw["router_bias"], dw["w_gate"],
                          dw["w_up"], dw["w_down"], dw["ws_gate"], dw["ws_up"], dw["ws_down"],
                          y, ws, topk_idx_out=idx)

    say("graph capture, row-major weights", cfg.name, T)
    _replays_equal_eager(cfg, T, y, idx, call)


@pytest.mark.gpu
@pytest.mark.parametrize("kind,cfg,T", [("packed", C1, 64), ("packed", C2, 456),
                                        ("packed", C3, 4096), ("packed", C4, 16384),
                                        ("int8", C1, 64), ("int8", C2, 456)])
def test_packed_and_int8_layer_graph_replays_equal_eager(lib, kind, cfg, T):
    import torch
    inp, dw = layer_inputs(cfg, T)
    dims, ws, y, idx = _buffers(lib, cfg, T, dw)
    if kind == "packed":
        buf = torch.empty(lib.packed_weights_size(dims), dtype=torch.uint8, device="cuda")
        lib.pack_weights(dims, dw["w_gate"], dw["w_up"], dw["w_down"], dw["ws_gate"],
                         dw["ws_up"], dw["ws_down"], buf)
        forward = lib.layer_forward_packed
    else:
        buf = torch.empty(lib.w8_weights_size(dims), dtype=torch.uint8, device="cuda")
        lib.quantize_weights_w8(dims, dw["w_gate"], dw["w_up"], dw["w_down"], dw["ws_gate"],
                                dw["ws_up"], dw["ws_down"], buf)
        forward = lib.layer_forward_w8
    torch.cuda.synchronize()

    def call():
        forward(dims, dw["x"], dw["w_router"], dw["router_bias"], buf, y, ws, topk_idx_out=idx)

    say("graph capture,", kind, "weights", cfg.name, T)
    _replays_equal_eager(cfg, T, y, idx, call)
