"""The C-ABI library loads on the CPU, exports every function include/moge.h
declares, and rejects bad arguments on the host before touching the GPU.
No call here reaches a kernel launch: every call either fails validation or has
T = 0 (which enqueues nothing)."""
import ctypes

import pytest

import sparse_moe_layer_moge_amd as moge
from sparse_moe_layer_moge_amd import lib

FAKE = 0x10000          # aligned, never dereferenced (validation fails or T = 0)
MIS = 0x10002           # misaligned


def dims(**kw):
    base = dict(T=64, d=5120, N=64, M=8, k_per_group=1, inter=1344, shared_inter=5376,
                dtype=moge.MOGE_BF16)
    base.update(kw)
    return moge.make_dims(**base)


def test_every_declared_function_is_exported():
    names = moge.header_functions()
    assert {"moge_route", "moge_permute", "moge_expert_ffn", "moge_combine",
            "moge_layer_forward", "moge_workspace_size", "moge_last_error",
            "moge_abi_version"} <= set(names)
    raw = ctypes.CDLL(moge.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert lib.moge_abi_version() == 1


def test_workspace_size():
    w = moge.workspace_size(dims())
    assert w > 0 and w % 256 == 0
    assert moge.workspace_size(dims(T=4096)) > w
    assert moge.workspace_size(dims(N=63)) == 0        # N % M != 0
    assert moge.workspace_size(dims(d=100)) == 0       # d % 32 != 0
    assert lib.moge_workspace_size(None) == 0


def test_noalloc_scratch_covers_the_documented_batch():
    # include/moge.h: at the Pangu-Pro shape the fixed scratch array of the
    # allocation-free entry point holds the workspace of up to 645 tokens
    assert moge.NOALLOC_SCRATCH_BYTES == 128 << 20
    assert moge.workspace_size(dims(T=645)) <= moge.NOALLOC_SCRATCH_BYTES
    assert moge.workspace_size(dims(T=646)) > moge.NOALLOC_SCRATCH_BYTES


def route(d, logits=FAKE, probs=None, idx=FAKE, gate=FAKE):
    return lib.moge_route(ctypes.byref(d) if d is not None else None, logits, probs, idx, gate,
                          None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(N=63), 1, "multiple of M"),
    (dict(k_per_group=9), 1, "exceeds the group size"),
    (dict(k_per_group=0), 1, "out of range"),
    (dict(T=-1), 1, "out of range"),
    (dict(dtype=7), 1, "dtype"),
    (dict(N=512, M=8), 2, "N=512"),
    (dict(N=128, M=128, k_per_group=1), 2, "K=M*k_per_group"),
    (dict(d=5100), 2, "multiples of 32"),
    (dict(inter=1000), 2, "multiples of 32"),
    (dict(shared_inter=100), 2, "multiples of 32"),
    # buffers addressed with 32-bit offsets: activations, one expert's packed gate/up
    # pair (2 * inter * d), the shared experts' gate/up pair
    (dict(T=1 << 20), 2, "exceeds 4 GiB"),
    (dict(d=32768, inter=40960, shared_inter=0), 2, "exceeds 4 GiB"),
    (dict(d=32768, inter=64, shared_inter=40960), 2, "exceeds 4 GiB"),
])
def test_invalid_dims(kw, status, msg):
    assert route(dims(**kw)) == status
    assert msg in moge.last_error()


def test_null_dims_and_pointers():
    assert route(None) == 1 and "dims is NULL" in moge.last_error()
    assert route(dims(), logits=None) == 1 and "logits is NULL" in moge.last_error()
    assert route(dims(), idx=None) == 1 and "topk_idx" in moge.last_error()
    assert route(dims(), logits=MIS) == 1 and "aligned" in moge.last_error()


def test_zero_tokens_is_ok_and_enqueues_nothing():
    assert route(dims(T=0)) == 0
    assert moge.last_error() == ""


def test_workspace_checks():
    d = dims(T=0)
    need = moge.workspace_size(d)
    args = [FAKE] * 7
    # moge_permute: ws NULL / too small / misaligned
    st = lib.moge_permute(ctypes.byref(d), FAKE, FAKE, *args[:5], None, None, need, None)
    assert st == 3 and "NULL" in moge.last_error()
    st = lib.moge_permute(ctypes.byref(d), FAKE, FAKE, *args[:5], None, FAKE, need - 1, None)
    assert st == 3 and "need" in moge.last_error()
    st = lib.moge_permute(ctypes.byref(d), FAKE, FAKE, *args[:5], None, FAKE + 16, need, None)
    assert st == 1 and "256-byte" in moge.last_error()
    st = lib.moge_permute(ctypes.byref(d), FAKE, FAKE, *args[:5], None, FAKE, need, None)
    assert st == 0


def test_layer_forward_pointer_rules():
    d = dims(T=0)
    need = moge.workspace_size(d)
    P = FAKE

    def call(**over):
        a = dict(x=P, w_router=P, bias=None, wg=P, wu=P, wd=P, sg=P, su=P, sd=P, lin=None, y=P,
                 lout=None, iout=None, gout=None, gcout=None, ws=P, wsb=need)
        a.update(over)
        return lib.moge_layer_forward(ctypes.byref(d), a["x"], a["w_router"], a["bias"], a["wg"],
                                      a["wu"], a["wd"], a["sg"], a["su"], a["sd"], a["lin"],
                                      a["y"], a["lout"], a["iout"], a["gout"], a["gcout"],
                                      a["ws"], a["wsb"], None)
    assert call() == 0
    assert call(w_router=None) == 1                       # needed without logits_in
    assert call(w_router=None, lin=P) == 0                # not needed with logits_in
    assert call(sg=None) == 1                             # shared experts configured
    d.shared_inter = 0
    need0 = moge.workspace_size(d)
    assert call(sg=None, su=None, sd=None, wsb=need0) == 0
    assert call(y=MIS) == 1
    assert call(wsb=0) == 3


def test_expert_ffn_and_combine_validation():
    d = dims(T=0)
    need = moge.workspace_size(d)
    assert lib.moge_expert_ffn(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need,
                               None) == 0
    assert lib.moge_expert_ffn(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need,
                               None) == 1
    assert lib.moge_combine(ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, None) == 0
    assert lib.moge_combine(ctypes.byref(d), FAKE, FAKE, FAKE, MIS, FAKE, None) == 1


def test_w8_entry_points_validation():
    d = dims(T=0)
    need = moge.workspace_size(d)
    wsize = moge.w8_weights_size(d)
    assert wsize > 0 and wsize % 256 == 0
    P = FAKE

    def fwd(dd, **over):
        a = dict(x=P, w_router=P, bias=None, w8=P, lin=None, y=P, ws=P, wsb=need)
        a.update(over)
        return lib.moge_layer_forward_w8(ctypes.byref(dd), a["x"], a["w_router"], a["bias"],
                                         a["w8"], a["lin"], a["y"], None, None, None, None,
                                         a["ws"], a["wsb"], None)
    assert fwd(d) == 0
    assert fwd(d, w8=None) == 1 and "w8 is NULL" in moge.last_error()
    assert fwd(d, w8=FAKE + 16) == 1 and "256-byte" in moge.last_error()
    assert fwd(d, wsb=0) == 3
    assert fwd(dims(T=0, dtype=moge.MOGE_F32)) == 2 and "bf16" in moge.last_error()
    assert fwd(dims(T=0, inter=1312)) == 2 and "multiples of 64" in moge.last_error()
    assert fwd(dims(T=0, d=5088)) == 2 and "multiples of 64" in moge.last_error()

    # pack: codes must be 16-byte aligned, the buffer large enough (no call here
    # passes validation: these entry points launch kernels whatever T is)
    codes = [P] * 3 + [P] * 3 + [P] * 3 + [P] * 3
    st = lib.moge_pack_weights_w8(ctypes.byref(d), MIS, *codes[1:], P, wsize, None)
    assert st == 1 and "q_gate" in moge.last_error()
    st = lib.moge_pack_weights_w8(ctypes.byref(d), *codes, P, wsize - 1, None)
    assert st == 1 and "need" in moge.last_error()
    st = lib.moge_pack_weights_w8(ctypes.byref(d), *codes[:6], None, *codes[7:], P, wsize, None)
    assert st == 1 and "qs_gate" in moge.last_error()
    # quantise
    st = lib.moge_quantize_weights_w8(ctypes.byref(d), P, P, MIS, P, P, P, P, wsize, None)
    assert st == 1 and "w_down" in moge.last_error()
    st = lib.moge_quantize_weights_w8(ctypes.byref(d), P, P, P, P, P, P, P, 0, None)
    assert st == 1 and "need" in moge.last_error()
    st = lib.moge_quantize_weights_w8(ctypes.byref(dims(T=0, dtype=moge.MOGE_F32)), P, P, P, P,
                                      P, P, P, wsize, None)
    assert st == 2
