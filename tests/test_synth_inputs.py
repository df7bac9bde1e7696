"""The seeded input generator: determinism, thread independence, bf16 rounding."""
import numpy as np
import torch

from synth import inputs as S
from synth.configs import C0, C1


def test_deterministic_and_thread_independent(monkeypatch):
    shape = (3, S.CHUNK // 2 + 7)          # spans several chunks
    a = S.normal_tensor(shape, 0.02, 0, 2, "bf16")
    b = S.normal_tensor(shape, 0.02, 0, 2, "bf16")
    np.testing.assert_array_equal(a, b)
    monkeypatch.setattr(S, "_threads", lambda: 1)
    c = S.normal_tensor(shape, 0.02, 0, 2, "bf16")
    np.testing.assert_array_equal(a, c)
    d = S.normal_tensor(shape, 0.02, 1, 2, "bf16")
    assert (a != d).mean() > 0.9


def test_bf16_rounding_matches_torch():
    v = np.random.Generator(np.random.PCG64(5)).standard_normal(100000).astype(np.float32) * 3
    v[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]  # exact ties
    ours = S.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(S.bf16_bits_to_f32(ours),
                                  torch.from_numpy(v).to(torch.bfloat16).float().numpy())


def test_shapes_and_scale():
    inp = S.make_layer_inputs(C0)
    assert inp.x.shape == (64, 256) and inp.x.dtype == np.float32
    assert inp.w_gate.shape == (16, 128, 256) and inp.w_down.shape == (16, 256, 128)
    assert inp.ws_gate.shape == (256, 256) and inp.ws_down.shape == (256, 256)
    assert abs(inp.w_gate.std() - 0.02) < 0.001 and abs(inp.w_router.std() - 0.1) < 0.005
    s = S.make_scores(C1, T=32)
    assert s.shape == (32, 64) and s.dtype == np.float32


def test_first_rows_do_not_depend_on_T():
    a = S.make_layer_inputs(C0, T=10).x
    b = S.make_layer_inputs(C0, T=64).x
    np.testing.assert_array_equal(a, b[:10])


def test_tie_scores_have_signed_zeros():
    v = S.tie_scores(50, 16, 0)
    z = v[v == 0]
    assert (np.signbit(z)).any() and (~np.signbit(z)).any()
