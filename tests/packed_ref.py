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
