"""The packed expert-weight layout written out with numpy reshapes, from its
definition in include/moge.h (fragment tile = 16 rows x 32 contraction elements,
chunk l = row l % 16, elements 8*(l/16)..8*(l/16)+7)."""
import numpy as np


def _gu(g, u):
    """gate/up part of one expert: g, u are [I, d]."""
    I, d = g.shape
    nb, ns = I // 16, d // 32
    def tiles(w):                       # [b, r, s, q, j] -> [b, s, q, r, j]
        return w.reshape(nb, 16, ns, 4, 8).transpose(0, 2, 3, 1, 4)
    return np.stack([tiles(g), tiles(u)], axis=2).reshape(-1)   # [b, s, t, q, r, j]


def _down(w):
    """down part of one expert: w is [d, I]."""
    d, I = w.shape
    nb, ns = d // 32, I // 32
    t = w.reshape(nb, 2, 16, ns, 4, 8)                           # [b, t, r, s, q, j]
    return t.transpose(0, 3, 1, 4, 2, 5).reshape(-1)             # [b, s, t, q, r, j]


def pack(w_gate, w_up, w_down, ws_gate=None, ws_up=None, ws_down=None):
    parts = [_gu(w_gate[e], w_up[e]) for e in range(w_gate.shape[0])]
    parts += [_down(w_down[e]) for e in range(w_down.shape[0])]
    if ws_gate is not None and ws_gate.shape[0] > 0:
        parts += [_gu(ws_gate, ws_up), _down(ws_down)]
    return np.concatenate(parts)


# ---------------------------------------------------------------------------
# int8 expert weights: code tiles of 16 rows x 64 contraction elements, chunk l =
# row l % 16, elements 16*(l/16)..16*(l/16)+15; regions 256-byte aligned, then the
# float32 scales (definition in include/moge.h)
# ---------------------------------------------------------------------------

def _w8_gu(g, u):
    """code tiles of one gate/up pair: g, u are [I, d]."""
    I, d = g.shape
    nb, ns = I // 16, d // 64
    def tiles(w):                       # [b, r, s, q, j] -> [b, s, q, r, j]
        return w.reshape(nb, 16, ns, 4, 16).transpose(0, 2, 3, 1, 4)
    return np.stack([tiles(g), tiles(u)], axis=2).reshape(-1)   # [b, s, t, q, r, j]


def _w8_down(w):
    """code tiles of one down matrix: w is [d, I]."""
    d, I = w.shape
    nb, ns = d // 32, I // 64
    t = w.reshape(nb, 2, 16, ns, 4, 16)                          # [b, t, r, s, q, j]
    return t.transpose(0, 3, 1, 4, 2, 5).reshape(-1)             # [b, s, t, q, r, j]


def _w8_gu_inv(flat, I, d):
    nb, ns = I // 16, d // 64
    a = flat.reshape(nb, ns, 2, 4, 16, 16)                       # [b, s, t, q, r, j]
    def rows(t):
        return a[:, :, t].transpose(0, 3, 1, 2, 4).reshape(I, d)  # [b, r, s, q, j]
    return rows(0), rows(1)


def _w8_down_inv(flat, d, I):
    nb, ns = d // 32, I // 64
    a = flat.reshape(nb, ns, 2, 4, 16, 16)                       # [b, s, t, q, r, j]
    return a.transpose(0, 2, 4, 1, 3, 5).reshape(d, I)           # [b, t, r, s, q, j]


def _al(n):
    return (n + 255) // 256 * 256


def w8_regions(d, N, I, Is):
    """byte offsets of the regions and the total size"""
    sizes = [("routed_gu", N * 2 * I * d), ("routed_down", N * d * I), ("shared_gu", 2 * Is * d),
             ("shared_down", d * Is), ("s_gate", 4 * N * I), ("s_up", 4 * N * I),
             ("s_down", 4 * N * d), ("ss_gate", 4 * Is), ("ss_up", 4 * Is),
             ("ss_down", 4 * d if Is > 0 else 0)]
    off, o = {}, 0
    for name, n in sizes:
        off[name] = (o, n)
        o += _al(n)
    return off, o


def w8_buffer(q_gate, s_gate, q_up, s_up, q_down, s_down, qs_gate=None, ss_gate=None,
              qs_up=None, ss_up=None, qs_down=None, ss_down=None):
    """the whole int8 weight buffer (uint8) from codes [.., rows, K] and scales [.., rows]"""
    N, I, d = q_gate.shape
    Is = 0 if qs_gate is None else qs_gate.shape[0]
    off, total = w8_regions(d, N, I, Is)
    buf = np.zeros(total, dtype=np.uint8)

    def put(name, arr):
        o, n = off[name]
        b = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        assert b.size == n
        buf[o:o + n] = b
    put("routed_gu", np.concatenate([_w8_gu(q_gate[e], q_up[e]) for e in range(N)]))
    put("routed_down", np.concatenate([_w8_down(q_down[e]) for e in range(N)]))
    put("s_gate", s_gate.astype(np.float32))
    put("s_up", s_up.astype(np.float32))
    put("s_down", s_down.astype(np.float32))
    if Is > 0:
        put("shared_gu", _w8_gu(qs_gate, qs_up))
        put("shared_down", _w8_down(qs_down))
        put("ss_gate", ss_gate.astype(np.float32))
        put("ss_up", ss_up.astype(np.float32))
        put("ss_down", ss_down.astype(np.float32))
    return buf


def w8_unpack(buf, d, N, I, Is, experts=None):
    """codes and scales back out of an int8 weight buffer (uint8); `experts`
    limits the routed parts returned (default: all)."""
    off, _ = w8_regions(d, N, I, Is)
    experts = range(N) if experts is None else experts

    def part(name, o_extra, n, dtype=np.int8):
        o, _ = off[name]
        return buf[o + o_extra:o + o_extra + n].view(dtype)
    out = {"q_gate": {}, "q_up": {}, "q_down": {}}
    for e in experts:
        g, u = _w8_gu_inv(part("routed_gu", e * 2 * I * d, 2 * I * d), I, d)
        out["q_gate"][e], out["q_up"][e] = g, u
        out["q_down"][e] = _w8_down_inv(part("routed_down", e * d * I, d * I), d, I)
    out["s_gate"] = part("s_gate", 0, 4 * N * I, np.float32).reshape(N, I)
    out["s_up"] = part("s_up", 0, 4 * N * I, np.float32).reshape(N, I)
    out["s_down"] = part("s_down", 0, 4 * N * d, np.float32).reshape(N, d)
    if Is > 0:
        out["qs_gate"], out["qs_up"] = _w8_gu_inv(part("shared_gu", 0, 2 * Is * d), Is, d)
        out["qs_down"] = _w8_down_inv(part("shared_down", 0, d * Is), d, Is)
        out["ss_gate"] = part("ss_gate", 0, 4 * Is, np.float32)
        out["ss_up"] = part("ss_up", 0, 4 * Is, np.float32)
        out["ss_down"] = part("ss_down", 0, 4 * d, np.float32)
    return out
