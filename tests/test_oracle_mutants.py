"""Each test plants one plausible mistake in the CPU oracle (monkeypatched, CPU
only) and checks that at least one oracle pin then fails.  This shows the pins
are strong enough to catch a dropped term, a wrong sign, a wrong index or tie
rule, or a transposed operand."""
import numpy as np
import pytest

from oracle import moge_oracle as O
import tests.test_oracle_pins as P


def _fails(fn, *args):
    with pytest.raises((AssertionError, ValueError)):
        fn(*args)


def test_mutant_tie_goes_to_highest_index(monkeypatch):
    real = O.group_topk

    def mutant(scores, M, kp):
        s = np.asarray(scores)
        N = s.shape[1]
        G = N // M
        idx = real(s, M, kp)
        for g in range(M):
            block = s[:, g * G:(g + 1) * G][:, ::-1]
            order = np.argsort(-block, axis=1, kind="stable")[:, :kp]
            idx[:, g * kp:(g + 1) * kp] = (G - 1 - order) + g * G
        return idx
    monkeypatch.setattr(O, "group_topk", mutant)
    _fails(P.test_group_topk_brute_force, 8, 2, 2)
    _fails(P.test_routing_golden_example)


def test_mutant_strided_groups(monkeypatch):
    def mutant(scores, M, kp):
        s = np.asarray(scores)
        T, N = s.shape
        idx = np.empty((T, M * kp), dtype=np.int32)
        for g in range(M):
            members = np.arange(g, N, M)              # e % M == g instead of blocks
            order = np.argsort(-s[:, members], axis=1, kind="stable")[:, :kp]
            idx[:, g * kp:(g + 1) * kp] = members[order]
        return idx
    monkeypatch.setattr(O, "group_topk", mutant)
    _fails(P.test_exactly_kp_per_group_and_distinct)
    _fails(P.test_group_topk_brute_force, 12, 4, 2)


def test_mutant_renormalised_gates(monkeypatch):
    real = O.route

    def mutant(l, M, kp):
        r = real(l, M, kp)
        r["gate"] = r["gate"] / r["gate"].sum(1, keepdims=True)
        return r
    monkeypatch.setattr(O, "route", mutant)
    _fails(P.test_routing_golden_example)
    _fails(P.test_layer_equals_dense_brute_force, 1)


def test_mutant_router_bias_dropped(monkeypatch):
    real = O.router_logits
    monkeypatch.setattr(O, "router_logits", lambda x, w, bias=None: real(x, w, None))
    _fails(P.test_router_scores_golden_example)


def test_mutant_router_bias_sign_flipped(monkeypatch):
    real = O.router_logits
    monkeypatch.setattr(O, "router_logits",
                        lambda x, w, bias=None: real(x, w, None if bias is None else -np.asarray(bias)))
    _fails(P.test_router_scores_golden_example)


def test_mutant_router_bias_after_softmax(monkeypatch):
    # the bias added to the probabilities after the softmax instead of the scores
    real_logits, real_softmax = O.router_logits, O.softmax
    held = {}

    def logits(x, w, bias=None):
        held["b"] = None if bias is None else np.asarray(bias, dtype=np.float64)
        return real_logits(x, w, None)

    def softmax(l):
        p = real_softmax(l)
        return p if held.get("b") is None else p + held["b"][None, :]
    monkeypatch.setattr(O, "router_logits", logits)
    monkeypatch.setattr(O, "softmax", softmax)
    _fails(P.test_router_scores_golden_example)


def test_mutant_router_bias_wrong_index(monkeypatch):
    real = O.router_logits
    monkeypatch.setattr(O, "router_logits",
                        lambda x, w, bias=None: real(x, w, None if bias is None
                                                     else np.asarray(bias)[::-1].copy()))
    _fails(P.test_router_scores_golden_example)


def test_mutant_silu_sign(monkeypatch):
    monkeypatch.setattr(O, "silu", lambda a: a / (1.0 + np.exp(a)))
    _fails(P.test_silu_closed_forms)
    _fails(P.test_swiglu_closed_form_scalar)


def test_mutant_transposed_down(monkeypatch):
    def mutant(X, Wg, Wu, Wd):
        return (O.silu(X @ Wg.T) * (X @ Wu.T)) @ Wd      # Wd not transposed
    monkeypatch.setattr(O, "swiglu", mutant)
    _fails(P.test_swiglu_closed_form_asymmetric)


def test_mutant_transposed_gate(monkeypatch):
    def mutant(X, Wg, Wu, Wd):
        return (O.silu(X @ Wg) * (X @ Wu.T)) @ Wd.T      # Wg not transposed
    monkeypatch.setattr(O, "swiglu", mutant)
    _fails(P.test_swiglu_closed_form_asymmetric)


def test_mutant_gate_and_up_swapped(monkeypatch):
    def mutant(X, Wg, Wu, Wd):
        return (O.silu(X @ Wu.T) * (X @ Wg.T)) @ Wd.T
    monkeypatch.setattr(O, "swiglu", mutant)
    _fails(P.test_swiglu_closed_form_scalar)


def test_mutant_shared_dropped(monkeypatch):
    real = O.combine
    monkeypatch.setattr(O, "combine", lambda y, pr, g, sh, T, K: real(y, pr, g, None, T, K))
    _fails(P.test_layer_equals_dense_brute_force, 1)
    _fails(P.test_combine_closed_form)


def test_mutant_one_slot_dropped(monkeypatch):
    real = O.combine
    monkeypatch.setattr(O, "combine",
                        lambda y, pr, g, sh, T, K: real(y, pr, np.where(np.arange(K) == K - 1, 0.0, g), sh, T, K))
    _fails(P.test_layer_equals_dense_brute_force, 2)


def test_mutant_softmax_without_max_shift(monkeypatch):
    def mutant(l):
        e = np.exp(np.asarray(l, dtype=np.float64))
        return e / e.sum(1, keepdims=True)
    monkeypatch.setattr(O, "softmax", mutant)
    with np.errstate(over="ignore", invalid="ignore"):
        _fails(P.test_softmax_shift_invariant_and_large_scores)


def test_mutant_permutation_token_major(monkeypatch):
    real = O.permute

    def mutant(idx, N, M):
        r = real(idx, N, M)
        T, K = np.asarray(idx).shape
        r["sorted_pair"] = np.arange(T * K, dtype=np.int32)
        r["pair_row"] = np.arange(T * K, dtype=np.int32)
        return r
    monkeypatch.setattr(O, "permute", mutant)
    _fails(P.test_permute_matches_python_sort)


def test_mutant_group_count_off_by_one(monkeypatch):
    real = O.permute

    def mutant(idx, N, M):
        r = real(idx, N, M)
        G = N // M
        r["group_counts"] = np.array([r["counts"][g * G:(g + 1) * G - 1].sum() for g in range(M)],
                                     dtype=np.int32)
        return r
    monkeypatch.setattr(O, "permute", mutant)
    _fails(P.test_group_loads_equal_imbalance_zero)


def test_mutant_w8_truncating_codes(monkeypatch):
    def mutant(w, dtype):
        w32 = O.to_f64(w, dtype).astype(np.float32)
        s = (np.max(np.abs(w32), axis=-1) / np.float32(127)).astype(np.float32)
        with np.errstate(divide="ignore", invalid="ignore"):
            r = np.trunc(w32 / s[..., None])
        return np.where(s[..., None] > 0, np.clip(r, -127, 127), 0).astype(np.int8), s
    monkeypatch.setattr(O, "w8_quantize", mutant)
    _fails(P.test_w8_quantize_golden_rows)
    _fails(P.test_w8_quantize_error_bound_and_range, "f32")


def test_mutant_w8_scale_over_128(monkeypatch):
    real = O.w8_quantize

    def mutant(w, dtype):
        q, s = real(w, dtype)
        w32 = O.to_f64(w, dtype).astype(np.float32)
        s = (np.max(np.abs(w32), axis=-1) / np.float32(128)).astype(np.float32)
        with np.errstate(divide="ignore", invalid="ignore"):
            r = np.rint(w32 / s[..., None])
        return np.where(s[..., None] > 0, np.clip(r, -127, 127), 0).astype(np.int8), s
    monkeypatch.setattr(O, "w8_quantize", mutant)
    _fails(P.test_w8_quantize_error_bound_and_range, "f32")


def test_mutant_w8_scale_along_contraction(monkeypatch):
    class Mutant(O.W8Weights):
        def __getitem__(self, e):
            q = self.q[e].astype(np.float64)
            s = self.s[e].astype(np.float64)
            k = q.shape[-1]
            # scales applied along the contraction index instead of the output row
            return q * np.resize(s, k)[None, :]

        def __array__(self, dtype=None, copy=None):
            return np.stack([self[i] for i in range(self.q.shape[0])]) if self.q.ndim == 3 \
                else self.q.astype(np.float64) * np.resize(self.s, self.q.shape[-1])[None, :]
    monkeypatch.setattr(O, "W8Weights", Mutant)
    _fails(P.test_w8_layer_is_the_layer_on_exactly_quantisable_weights)
