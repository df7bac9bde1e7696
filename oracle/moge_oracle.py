"""CPU oracle for the MoGE (Mixture of Grouped Experts) expert-layer forward pass.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It is plain, slow numpy in float64; it
shares no code with the GPU library and imports nothing from it.

Sources (cited by page title and section, never by line):
  [TW1]  TechWalker, "华为发布Pangu Pro MoE：全球首个72B参数稀疏语言模型，专为昇腾NPU
         优化设计", section 一 (创新架构: 混合分组专家的智慧设计).
  [TW2]  same page, section 二 (硬件协同设计) - layer shape: hidden 5120, 64 routed
         and 4 shared experts.
  [TW6]  same page, section 六 (专家特性分析) - no co-activation inside a group.
  [RC]   Reportify concept page "分组混合专家模型", bullet list 技术创新细节.
  [MK]   mokono.cn, "盘古Pro MoE", 核心亮点 item 1 (分组专家机制): 8 groups of 8,
         one expert per group, 4 shared experts kept.
  [TW3]  TechWalker page, section 三 (推理性能优化) - quantised deployment of the
         experts (expert-aware quantisation).
  [CS]   CSDN page (hwcomputing.csdn.net) - W8A8 deployment within 1.2% accuracy.

What the pages fix (restated):
  * The N routed experts are split evenly into M groups of G = N/M experts; each
    group sits on one device [TW1].
  * Scores of all N experts go through one softmax over all N experts first; only
    then is a top-K' taken inside every group, K' = K/M, so every token uses
    exactly K' experts of each group and all groups carry the same load; the
    imbalance score (busiest minus idlest device load) is then always zero [TW1, RC].
  * Shared experts are always active, besides the routed ones [MK, TW2].

Readings where the pages are silent (each listed in the design notes as well):
  R1 selection keys on the float32 router scores; softmax is strictly increasing,
     so in exact arithmetic this is the same set as keying on probabilities.
  R2 equal scores inside a group: the lower expert index wins; +0.0 == -0.0.
  R3 gate = the global softmax probability of the chosen expert, not renormalised.
  R4 groups are the contiguous index blocks [g*G, (g+1)*G).
  R5 slot order in idx[T,K]: group-major, then (score desc, index asc) in a group.
  R6 expert FFN = SwiGLU: down( silu(x Wg^T) * (x Wu^T) ), no biases.
  R7 shared experts are ungated (weight 1) and summed; S SwiGLUs of width I are the
     same as one SwiGLU of width S*I with the weights concatenated.
  R8 permuted row order = expert ascending, then token ascending (stable).
  R9 imbalance score = (max_g load_g - min_g load_g) / T, load_g = number of
     (token, expert) assignments that land in group g.
  R10 y[t] = shared(x_t) + sum_k gate[t,k] * FFN_{idx[t,k]}(x_t), k in slot order.
  Q1 int8 expert weights (the weight half of [CS]'s W8A8): symmetric, one float32
     scale per output row, s = max|w| / 127, q = rint(w / s) ties to even, clamped
     to [-127, 127], each step in float32; a zero row gets s = 0, q = 0.  The layer
     then uses the weights s * q exactly; activations stay as they are.

Parity pins: see the oracle tests (brute force, closed forms, invariants, special
cases).  Every function here is pinned by at least one of them.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np


# ----------------------------------------------------------------------------
# dtype handling (the oracle's own; it does not reuse the input generator's)
# ----------------------------------------------------------------------------

def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a layer tensor: float32 arrays are widened; bf16
    tensors arrive as uint16 bit patterns = the high half of a float32 word;
    "f64" values (dequantised int8 weights) are taken as they are."""
    if dtype == "f64":
        return np.asarray(a, dtype=np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# S0: router scores  [TW1: each expert gets a score per token]
# ----------------------------------------------------------------------------

def router_logits(x64: np.ndarray, w_router64: np.ndarray,
                  bias: Optional[np.ndarray] = None) -> np.ndarray:
    """logits[t, e] = sum_j x[t, j] * W_r[e, j] (+ b[e]), in float64."""
    l = x64 @ w_router64.T
    if bias is not None:
        l = l + np.asarray(bias, dtype=np.float64)[None, :]
    return l


# ----------------------------------------------------------------------------
# S1: global softmax over all N experts  [TW1: softmax over every expert first]
# ----------------------------------------------------------------------------

def softmax(logits: np.ndarray) -> np.ndarray:
    """p[t, e] = exp(l[t,e] - max_e' l[t,e']) / sum_e'' exp(l[t,e''] - max), float64."""
    l = np.asarray(logits, dtype=np.float64)
    if not np.all(np.isfinite(l)):
        raise ValueError("router scores must be finite")
    m = l.max(axis=1, keepdims=True)
    e = np.exp(l - m)
    return e / e.sum(axis=1, keepdims=True)


# ----------------------------------------------------------------------------
# S2: per-group top-K'  [TW1, RC: every group independently keeps its top K']
# ----------------------------------------------------------------------------

def group_topk(scores: np.ndarray, M: int, kp: int) -> np.ndarray:
    """idx[t, g*kp + j] = the j-th best expert of group g for token t.

    Experts are split into M contiguous groups of G = N/M (R4).  Inside a group the
    order is score descending, lower index first on equal scores (R2, R5)."""
    s = np.asarray(scores)
    T, N = s.shape
    if N % M != 0:
        raise ValueError("N must be a multiple of M")
    G = N // M
    if not 1 <= kp <= G:
        raise ValueError("kp must be in [1, N/M]")
    idx = np.empty((T, M * kp), dtype=np.int32)
    for g in range(M):
        block = s[:, g * G:(g + 1) * G]
        # a stable sort on the negated score keeps the lower index first among
        # equal scores; -0.0 and +0.0 compare equal, as in IEEE comparison.
        order = np.argsort(-block, axis=1, kind="stable")[:, :kp]
        idx[:, g * kp:(g + 1) * kp] = order + g * G
    return idx


def global_topk(scores: np.ndarray, K: int) -> np.ndarray:
    """The conventional router the pages compare against: top-K over all N experts,
    ignoring where experts live [TW1].  Same tie rule.  (= group_topk with M=1.)"""
    return group_topk(scores, 1, K)


def route(logits_f32: np.ndarray, M: int, kp: int) -> Dict[str, np.ndarray]:
    """Routing of one batch: probabilities, selected experts and their gates.

    Selection keys on the float32 scores (R1); probabilities are the float64
    softmax of those same scores; gate = probability of the chosen expert (R3)."""
    l32 = np.asarray(logits_f32, dtype=np.float32)
    p = softmax(l32.astype(np.float64))
    idx = group_topk(l32, M, kp)
    gate = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    return {"probs": p, "idx": idx, "gate": gate}


# ----------------------------------------------------------------------------
# S3: permutation into expert-contiguous order, group loads, imbalance score
# ----------------------------------------------------------------------------

def permute(idx: np.ndarray, N: int, M: int) -> Dict[str, np.ndarray]:
    """Expert-contiguous order of the (token, slot) pairs.

    pair p = t*K + k refers to expert idx[t, k].  Rows are ordered by expert, then
    by token (R8): sorted_pair[row] = p, pair_row[p] = row.  counts[e] = rows of
    expert e, offsets = exclusive prefix sum (N+1 entries), group_counts[g] = rows
    whose expert is in group g."""
    idx = np.asarray(idx, dtype=np.int64)
    T, K = idx.shape
    flat = idx.reshape(-1)
    counts = np.zeros(N, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(N + 1, dtype=np.int64)
    for e in range(N):
        offsets[e + 1] = offsets[e] + counts[e]
    # counting sort, visiting pairs in increasing p = t*K + k: within one expert
    # the rows come out in token order (an expert appears at most once per token).
    fill = offsets[:N].copy()
    sorted_pair = np.empty(T * K, dtype=np.int64)
    for p in range(T * K):
        e = flat[p]
        sorted_pair[fill[e]] = p
        fill[e] += 1
    pair_row = np.empty(T * K, dtype=np.int64)
    pair_row[sorted_pair] = np.arange(T * K)
    G = N // M
    group_counts = np.array([counts[g * G:(g + 1) * G].sum() for g in range(M)],
                            dtype=np.int64)
    return {"counts": counts.astype(np.int32), "offsets": offsets.astype(np.int32),
            "group_counts": group_counts.astype(np.int32),
            "sorted_pair": sorted_pair.astype(np.int32),
            "pair_row": pair_row.astype(np.int32)}


def imbalance_score(group_loads: Sequence[int], T: int) -> float:
    """(busiest group load - idlest group load) / T  (R9, [TW1])."""
    g = np.asarray(group_loads, dtype=np.int64)
    return float(g.max() - g.min()) / float(T) if T > 0 else 0.0


def group_loads_of(idx: np.ndarray, N: int, n_groups: int) -> np.ndarray:
    """Load of each of n_groups contiguous expert blocks for a routing result."""
    G = N // n_groups
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    return np.bincount(flat // G, minlength=n_groups).astype(np.int64)


# ----------------------------------------------------------------------------
# S4-S6: SwiGLU expert FFNs (R6, R7)
# ----------------------------------------------------------------------------

def silu(a: np.ndarray) -> np.ndarray:
    """silu(a) = a * sigmoid(a) = a / (1 + exp(-a)), float64."""
    return a / (1.0 + np.exp(-a))


def swiglu(X: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """FFN(X) = (silu(X Wg^T) * (X Wu^T)) Wd^T for X[r,d], Wg/Wu[I,d], Wd[d,I]."""
    return (silu(X @ Wg.T) * (X @ Wu.T)) @ Wd.T


def expert_ffn(x_perm64: np.ndarray, offsets: np.ndarray, w_gate, w_up, w_down,
               dtype: str) -> np.ndarray:
    """y_perm rows of expert e = SwiGLU_e(x_perm rows offsets[e]:offsets[e+1]).

    Weights are widened one expert at a time to bound host memory."""
    N = len(offsets) - 1
    y = np.zeros((x_perm64.shape[0], w_down.shape[1]), dtype=np.float64)
    for e in range(N):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        y[lo:hi] = swiglu(x_perm64[lo:hi], to_f64(w_gate[e], dtype),
                          to_f64(w_up[e], dtype), to_f64(w_down[e], dtype))
    return y


def shared_experts(x64: np.ndarray, ws_gate, ws_up, ws_down, dtype: str) -> np.ndarray:
    """Always-on shared experts as one SwiGLU of the concatenated width (R7)."""
    return swiglu(x64, to_f64(ws_gate, dtype), to_f64(ws_up, dtype), to_f64(ws_down, dtype))


# ----------------------------------------------------------------------------
# S7: gate-weighted combine back to token order (R10)
# ----------------------------------------------------------------------------

def combine(y_perm64: np.ndarray, pair_row: np.ndarray, gate: np.ndarray,
            shared_out64: Optional[np.ndarray], T: int, K: int) -> np.ndarray:
    """y[t] = shared[t] + sum_{k=0..K-1} gate[t,k] * y_perm[pair_row[t*K+k]]."""
    d = y_perm64.shape[1]
    y = np.zeros((T, d), dtype=np.float64) if shared_out64 is None else shared_out64.copy()
    for k in range(K):
        rows = np.asarray(pair_row, dtype=np.int64).reshape(T, K)[:, k]
        y += np.asarray(gate, dtype=np.float64)[:, k:k + 1] * y_perm64[rows]
    return y


# ----------------------------------------------------------------------------
# the whole layer
# ----------------------------------------------------------------------------

def layer(x, w_router, router_bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down,
          M: int, kp: int, dtype: str, logits_f32: Optional[np.ndarray] = None,
          tokens: Optional[np.ndarray] = None,
          wdtype: Optional[str] = None) -> Dict[str, np.ndarray]:
    """MoGE layer forward: scores -> global softmax -> per-group top-K' ->
    expert-contiguous permutation -> routed SwiGLU experts -> shared experts ->
    gate-weighted combine.

    logits_f32: router scores to route on; when None they are computed here from
    x and w_router in float64 and rounded to float32 for the selection (R1).
    tokens: optional subset of token indices; routing covers all T tokens, the
    permutation / FFN / combine only the listed ones (rows of y follow `tokens`).
    wdtype: dtype of the expert and shared weights when it differs from the
    activations' ("f64" for dequantised int8 weights); the router uses `dtype`."""
    wdtype = dtype if wdtype is None else wdtype
    x = np.asarray(x)
    T = x.shape[0]
    N = w_gate.shape[0]
    K = M * kp
    out: Dict[str, np.ndarray] = {}
    if logits_f32 is None:
        l64 = router_logits(to_f64(x, dtype), to_f64(w_router, dtype), router_bias)
        out["logits64"] = l64
        logits_f32 = l64.astype(np.float32)
    r = route(logits_f32, M, kp)
    out.update(r)
    out["logits"] = np.asarray(logits_f32, dtype=np.float32)
    perm_all = permute(r["idx"], N, M)
    out.update({k: perm_all[k] for k in ("counts", "offsets", "group_counts")})
    out["sorted_pair"], out["pair_row"] = perm_all["sorted_pair"], perm_all["pair_row"]

    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    sub_idx = r["idx"][tok]
    sub = permute(sub_idx, N, M)            # permutation of the selected tokens' pairs
    x_sel = to_f64(x[tok], dtype)
    token_of_row = sub["sorted_pair"].astype(np.int64) // K
    x_perm = x_sel[token_of_row]
    y_perm = expert_ffn(x_perm, sub["offsets"], w_gate, w_up, w_down, wdtype)
    sh = shared_experts(x_sel, ws_gate, ws_up, ws_down, wdtype)
    out["shared"] = sh
    out["y"] = combine(y_perm, sub["pair_row"], r["gate"][tok], sh, len(tok), K)
    out["tokens"] = tok
    return out


# ----------------------------------------------------------------------------
# Weight-only int8 expert weights (Q1; [TW3], [CS])
# ----------------------------------------------------------------------------

W8_QMAX = 127


def w8_quantize(w, dtype: str):
    """int8 codes q[..., rows, K] and float32 scales s[..., rows] of weights w
    (rows along the second-to-last axis, the contraction along the last).

    s = fl32(max_k |w[k]| / 127); q[k] = rint(fl32(w[k] / s)), ties to even,
    clamped to [-127, 127]; a row of zeros gets s = 0 and q = 0 (Q1)."""
    w32 = to_f64(w, dtype).astype(np.float32)           # exact for bf16 and float32
    absmax = np.max(np.abs(w32), axis=-1)
    s = (absmax / np.float32(W8_QMAX)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint(w32 / s[..., None])                  # float32 division, then ties-to-even
    q = np.where(s[..., None] > 0, np.clip(r, -W8_QMAX, W8_QMAX), 0).astype(np.int8)
    return q, s


class W8Weights:
    """The float64 weights s[..., r] * q[..., r, k] of int8 codes, widened one
    leading index (one expert) at a time when indexed, or whole via np.asarray."""

    def __init__(self, q: np.ndarray, s: np.ndarray):
        self.q = np.asarray(q, dtype=np.int8)
        self.s = np.asarray(s, dtype=np.float32)
        if self.s.shape != self.q.shape[:-1]:
            raise ValueError("one scale per row of codes")
        self.shape = self.q.shape

    def __getitem__(self, e):
        return self.q[e].astype(np.float64) * self.s[e].astype(np.float64)[..., None]

    def __array__(self, dtype=None, copy=None):
        a = self.q.astype(np.float64) * self.s.astype(np.float64)[..., None]
        return a if dtype is None else a.astype(dtype)


def layer_w8(x, w_router, router_bias, q_gate, s_gate, q_up, s_up, q_down, s_down,
             qs_gate, ss_gate, qs_up, ss_up, qs_down, ss_down, M: int, kp: int,
             dtype: str = "bf16", logits_f32: Optional[np.ndarray] = None,
             tokens: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """The MoGE layer with int8 expert and shared weights: `layer` on the weights
    s * q (Q1).  The activations and the router keep `dtype`."""
    return layer(x, w_router, router_bias, W8Weights(q_gate, s_gate), W8Weights(q_up, s_up),
                 W8Weights(q_down, s_down), W8Weights(qs_gate, ss_gate),
                 W8Weights(qs_up, ss_up), W8Weights(qs_down, ss_down), M=M, kp=kp,
                 dtype=dtype, logits_f32=logits_f32, tokens=tokens, wdtype="f64")
