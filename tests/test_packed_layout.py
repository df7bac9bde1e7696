"""The packed weight layout: the numpy definition is a permutation of the six
weight tensors with the size the library reports; the GPU pack kernel writes
exactly it; the packed layer gives the row-major layer's results bit for bit."""
import numpy as np
import pytest

import sparse_moe_layer_moge_amd as moge
from synth.configs import C0, C1, C2
from tests import packed_ref


def _dims(cfg, T):
    return moge.make_dims(T, cfg.d, cfg.N, cfg.M, cfg.kp, cfg.inter, cfg.I_s,
                          moge.MOGE_BF16 if cfg.dtype == "bf16" else moge.MOGE_F32)


def test_layout_is_a_permutation_with_reported_size():
    # distinct values everywhere: every source element lands exactly once
    N, I, d, Is = 3, 32, 64, 64
    n = 2 * N * I * d + N * d * I + 3 * Is * d
    vals = np.arange(n, dtype=np.int64)
    o = 0
    def take(*shape):
        nonlocal o
        k = int(np.prod(shape))
        a = vals[o:o + k].reshape(shape)
        o += k
        return a
    wg, wu, wd = take(N, I, d), take(N, I, d), take(N, d, I)
    sg, su, sd = take(Is, d), take(Is, d), take(d, Is)
    p = packed_ref.pack(wg, wu, wd, sg, su, sd)
    assert p.size == n and np.array_equal(np.sort(p), vals)
    dims = moge.make_dims(1, d, N, 1, 1, I, Is, moge.MOGE_BF16)
    assert moge.packed_weights_size(dims) == 2 * n
    # first tile: gate rows 0..15 of expert 0, elements 0..31, chunk l = (l%16, l//16)
    tile = p[:512].reshape(64, 8)
    for l in range(64):
        assert list(tile[l]) == list(wg[0, l % 16, 8 * (l // 16): 8 * (l // 16) + 8])
    # second tile: up rows, same positions
    assert list(p[512:520]) == list(wu[0, 0, 0:8])


def test_down_layout_first_block():
    d, I = 64, 32
    w = np.arange(d * I).reshape(1, d, I)
    p = packed_ref.pack(np.zeros((1, 32, 64), int), np.zeros((1, 32, 64), int), w)
    down = p[2 * 32 * 64:]
    t0 = down[:512].reshape(64, 8)          # rows 0..15, step 0
    t1 = down[512:1024].reshape(64, 8)      # rows 16..31, step 0
    for l in range(64):
        assert list(t0[l]) == list(w[0, l % 16, 8 * (l // 16): 8 * (l // 16) + 8])
        assert list(t1[l]) == list(w[0, 16 + l % 16, 8 * (l // 16): 8 * (l // 16) + 8])


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["C0", "C1"])
def test_gpu_pack_matches_definition(lib, name):
    import torch
    from tests.gpu_util import layer_inputs, say, to_host
    cfg = {"C0": C0, "C1": C1}[name]
    inp, dw = layer_inputs(cfg, 8)
    dims = _dims(cfg, 8)
    packed = torch.empty(moge.packed_weights_size(dims), dtype=torch.uint8, device="cuda")
    say("pack", name)
    moge.pack_weights(dims, dw["w_gate"], dw["w_up"], dw["w_down"], dw["ws_gate"], dw["ws_up"],
                      dw["ws_down"], packed)
    torch.cuda.synchronize()
    ref = packed_ref.pack(inp.w_gate, inp.w_up, inp.w_down, inp.ws_gate, inp.ws_up, inp.ws_down)
    got = to_host(packed).view(ref.dtype)
    assert got.shape == ref.shape
    assert np.array_equal(got, ref)


@pytest.mark.gpu
@pytest.mark.parametrize("name,T,given", [("C0", 64, True), ("C0", 37, False), ("C1", 64, True),
                                          ("C1", 64, False), ("C2", 456, True), ("C1", 9, False)])
def test_packed_layer_equals_row_major_layer(lib, name, T, given):
    import torch
    from synth import inputs as S
    from tests.gpu_util import layer_inputs, say, to_dev, to_host
    cfg = {"C0": C0, "C1": C1, "C2": C2}[name]
    inp, dw = layer_inputs(cfg, T)
    dims = _dims(cfg, T)
    packed = torch.empty(moge.packed_weights_size(dims), dtype=torch.uint8, device="cuda")
    moge.pack_weights(dims, dw["w_gate"], dw["w_up"], dw["w_down"], dw["ws_gate"], dw["ws_up"],
                      dw["ws_down"], packed)
    ws = torch.empty(moge.workspace_size(dims), dtype=torch.uint8, device="cuda")
    logits_in = to_dev(S.make_scores(cfg, T=T), "f32") if given else None
    ya = torch.empty((T, cfg.d), dtype=dw["x"].dtype, device="cuda")
    yb = torch.empty_like(ya)
    say("packed vs row-major", name, T, given)
    moge.layer_forward(dims, dw["x"], dw["w_router"], dw["router_bias"], dw["w_gate"], dw["w_up"],
                       dw["w_down"], dw["ws_gate"], dw["ws_up"], dw["ws_down"], ya, ws,
                       logits_in=logits_in)
    moge.layer_forward_packed(dims, dw["x"], dw["w_router"], dw["router_bias"], packed, yb, ws,
                              logits_in=logits_in)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(ya), to_host(yb))


# ----------------------------------------------------------------------------
# int8 expert weights
# ----------------------------------------------------------------------------

def test_w8_layout_first_tiles_and_size():
    rng = np.random.Generator(np.random.PCG64(5))
    N, I, d, Is = 2, 64, 128, 64
    q = lambda *s: rng.integers(-127, 128, size=s).astype(np.int8)
    f = lambda *s: rng.random(s).astype(np.float32)
    qg, qu, qd, qsg, qsu, qsd = q(N, I, d), q(N, I, d), q(N, d, I), q(Is, d), q(Is, d), q(d, Is)
    sg, su, sd, ssg, ssu, ssd = f(N, I), f(N, I), f(N, d), f(Is), f(Is), f(d)
    buf = packed_ref.w8_buffer(qg, sg, qu, su, qd, sd, qsg, ssg, qsu, ssu, qsd, ssd)
    dims = moge.make_dims(1, d, N, 1, 1, I, Is, moge.MOGE_BF16)
    assert moge.w8_weights_size(dims) == buf.size
    codes = buf.view(np.int8)
    # first tile: gate rows 0..15 of expert 0, elements 0..63; chunk l = row l%16,
    # elements 16*(l//16) .. +15
    t0 = codes[:1024].reshape(64, 16)
    t1 = codes[1024:2048].reshape(64, 16)
    for l in range(64):
        assert list(t0[l]) == list(qg[0, l % 16, 16 * (l // 16): 16 * (l // 16) + 16])
        assert list(t1[l]) == list(qu[0, l % 16, 16 * (l // 16): 16 * (l // 16) + 16])
    # second step of block 0 follows: elements 64..127
    t2 = codes[2048:3072].reshape(64, 16)
    assert list(t2[5]) == list(qg[0, 5, 64:80])
    # down part of expert 0: tiles of rows 0..15 and 16..31, step 0
    off, _ = packed_ref.w8_regions(d, N, I, Is)
    o = off["routed_down"][0]
    d0 = codes[o:o + 1024].reshape(64, 16)
    d1 = codes[o + 1024:o + 2048].reshape(64, 16)
    for l in range(64):
        assert list(d0[l]) == list(qd[0, l % 16, 16 * (l // 16): 16 * (l // 16) + 16])
        assert list(d1[l]) == list(qd[0, 16 + l % 16, 16 * (l // 16): 16 * (l // 16) + 16])
    # scales sit where the regions say, as float32
    o = off["s_down"][0]
    np.testing.assert_array_equal(buf[o:o + 4 * N * d].view(np.float32).reshape(N, d), sd)
    # the unpacking inverts the packing
    u = packed_ref.w8_unpack(buf, d, N, I, Is)
    for e in range(N):
        np.testing.assert_array_equal(u["q_gate"][e], qg[e])
        np.testing.assert_array_equal(u["q_up"][e], qu[e])
        np.testing.assert_array_equal(u["q_down"][e], qd[e])
    np.testing.assert_array_equal(u["qs_gate"], qsg)
    np.testing.assert_array_equal(u["qs_down"], qsd)
    np.testing.assert_array_equal(u["ss_up"], ssu)


def test_w8_size_rejects_unsupported_dims():
    assert moge.w8_weights_size(moge.make_dims(1, 96, 4, 1, 1, 64, 0, moge.MOGE_BF16)) == 0
    assert moge.w8_weights_size(moge.make_dims(1, 128, 4, 1, 1, 96, 0, moge.MOGE_BF16)) == 0
    assert moge.w8_weights_size(moge.make_dims(1, 128, 4, 1, 1, 64, 0, moge.MOGE_F32)) == 0
    assert moge.w8_weights_size(moge.make_dims(1, 128, 4, 1, 1, 64, 0, moge.MOGE_BF16)) > 0
