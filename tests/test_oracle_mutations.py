"""Planted mistakes in the oracle (on the CPU) must each fail at least one pin.

Each mutation replaces one oracle step with a plausible wrong version; the
pins of test_oracle_pins are then run and at least one must fail.
"""

import numpy as np
import pytest

import oracle
from oracle import hxq_oracle as H
import test_oracle_bound_pins as BP
import test_oracle_pins as P

PINS = [
    lambda: P.test_u8_matches_bruteforce(7, 12, 3),
    lambda: P.test_pk12_matches_bruteforce(6, 16, 3),
    P.test_bf16_activations_bruteforce,
    P.test_constant_index_closed_form,
    P.test_constant_index_pk12_closed_form,
    P.test_empty_sidecar_difference,
    P.test_one_hot_reconstructs_columns,
    P.test_cross_format_special_case,
    P.test_pk12_golden_bytes,
    P.test_bf16_round_matches_library_cast,
    lambda: P.test_bwd_u8_matches_bruteforce(7, 12, 3),
    lambda: P.test_bwd_pk12_matches_bruteforce(6, 16, 3),
    P.test_bwd_golden_hand_example,
    P.test_bwd_constant_index_closed_form,
    P.test_bwd_one_hot_rows_give_weight_rows,
    lambda: P.test_bwd_adjoint_of_forward("u8"),
    lambda: P.test_bwd_adjoint_of_forward("pk12"),
    lambda: BP.test_bound_u8_bruteforce(7, 12, 3),
    lambda: BP.test_bound_u8_bruteforce(6, 6, 4),
    lambda: BP.test_bound_pk12_bruteforce(6, 16, 3),
    BP.test_bound_bf16_activations_bruteforce,
    lambda: BP.test_bound_bwd_u8_bruteforce(7, 12, 3),
    lambda: BP.test_bound_bwd_u8_bruteforce(6, 6, 4),
    BP.test_bound_sidecar_add_bruteforce,
    BP.test_bound_golden_hand_example,
    BP.test_bound_bwd_golden_hand_example,
    BP.test_bound_sidecar_golden_hand_example,
]


def _transposed_forward(W, X, bias=None):
    Y = (X[:, : W.shape[0]] @ W[:, : X.shape[0]]) if W.shape[0] != W.shape[1] else X @ W
    if bias is not None:
        Y = Y + np.asarray(bias, np.float32).astype(np.float64)[None, :]
    return Y


def _no_bias_forward(W, X, bias=None):
    return X @ W.T


def _swapped_sidecar(W, rows, cols, deltas):
    out = np.array(W, dtype=np.float64, copy=True)
    r = np.asarray(cols, np.int64) % W.shape[0]
    c = np.asarray(rows, np.int64) % W.shape[1]
    if r.size:
        np.add.at(out, (r, c), np.asarray(deltas, np.float32).astype(np.float64))
    return out


def _sidecar_overwrites_duplicates(W, rows, cols, deltas):
    out = np.array(W, dtype=np.float64, copy=True)
    r = np.asarray(rows, np.int64)
    if r.size:
        out[r, np.asarray(cols, np.int64)] += np.asarray(deltas, np.float32).astype(np.float64)
    return out


def _unpack_nibble_swapped(packed, N, K):
    T = (K + 3) // 4
    p = np.asarray(packed, np.uint8).reshape(N, T, 3).astype(np.int64)
    a = p[:, :, 0] | ((p[:, :, 1] >> 4) << 8)
    b = (p[:, :, 1] & 0xF) | (p[:, :, 2] << 4)
    idx = np.empty((N, 2 * T), np.int64)
    idx[:, 0::2] = a
    idx[:, 1::2] = b
    return idx[:, : K // 2]


def _dequant_pk12_components_swapped(codebook2, idx2, K):
    c = np.asarray(codebook2, np.float32).astype(np.float64)[:, ::-1]
    return c[idx2].reshape(idx2.shape[0], K)


def _bf16_truncate(v):
    u = np.ascontiguousarray(v, np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    return u.view(np.float32)


def _bf16_bits_low_half(bits):
    return np.asarray(bits, np.uint16).astype(np.float32).astype(np.float64)


def _bwd_rows_reversed(W, DY):
    return DY @ W[::-1]


def _bwd_forward_orientation(W, DY):
    # the forward's operand order: only defined when W is square
    return DY @ W.T


def _bwd_columns_shifted(W, DY):
    return np.roll(DY @ W, 1, axis=1)


def _bwd_sign_lost(W, DY):
    return DY @ np.abs(W)


def _bound_scaled(W, X):
    return 1000.0 * (np.abs(X) @ np.abs(W).T)


def _bound_untransposed(W, X):
    # only defined when W is square
    return np.abs(X) @ np.abs(W)


def _bound_abs_x_only(W, X):
    return np.abs(X) @ W.T


def _bound_abs_w_only(W, X):
    return X @ np.abs(W).T


def _bound_plus_one(W, X):
    return np.abs(X) @ np.abs(W).T + 1.0


_real_fwd_u8 = H.hxq_linear_fwd_u8


def _fwd_u8_bound_plus_bias(codebook, indices, rows, cols, deltas, x, x_dtype, bias, m_rows=None,
                            want_bound=True):
    Y, B = _real_fwd_u8(codebook, indices, rows, cols, deltas, x, x_dtype, bias, m_rows, want_bound)
    if B is not None and bias is not None:
        B = B + np.abs(np.asarray(bias, np.float32).astype(np.float64))[None, :]
    return Y, B


def _fwd_u8_bound_abs_before_sidecar(codebook, indices, rows, cols, deltas, x, x_dtype, bias, m_rows=None,
                                     want_bound=True):
    # |C[idx]| + |deltas| instead of |C[idx] + deltas|
    Y, _ = _real_fwd_u8(codebook, indices, rows, cols, deltas, x, x_dtype, bias, m_rows, False)
    W = np.abs(H.dequant_u8(codebook, H.unpack_u8(indices)))
    W = H.apply_sidecar(W, rows, cols, np.abs(np.asarray(deltas, np.float32)))
    X = H.activations_f64(x, x_dtype)
    if m_rows is not None:
        X = X[np.asarray(m_rows, np.int64)]
    return Y, np.abs(X) @ W.T


def _bound_bwd_scaled(W, DY):
    return 1000.0 * (np.abs(DY) @ np.abs(W))


def _bound_bwd_transposed(W, DY):
    # the forward's orientation: only defined when W is square
    return np.abs(DY) @ np.abs(W).T


def _bound_bwd_abs_dy_only(W, DY):
    return np.abs(DY) @ W


_real_sidecar_add = H.hxq_sidecar_add


def _sidecar_add_bound_summed_first(rows, cols, deltas, x, x_dtype, N):
    # |S| |x| with the repeated coordinates summed before the absolute value
    Z, _ = _real_sidecar_add(rows, cols, deltas, x, x_dtype, N)
    X = H.activations_f64(x, x_dtype)
    S = np.zeros((N, X.shape[1]))
    np.add.at(S, (np.asarray(rows, np.int64), np.asarray(cols, np.int64)),
              np.asarray(deltas, np.float32).astype(np.float64))
    return Z, np.abs(X) @ np.abs(S).T


def _sidecar_add_bound_scaled(rows, cols, deltas, x, x_dtype, N):
    Z, B = _real_sidecar_add(rows, cols, deltas, x, x_dtype, N)
    return Z, 2.0 * B


MUTATIONS = {
    "transposed_weight": ("linear_forward", _transposed_forward),
    "dropped_bias": ("linear_forward", _no_bias_forward),
    "sidecar_row_col_swapped": ("apply_sidecar", _swapped_sidecar),
    "sidecar_duplicates_not_summed": ("apply_sidecar", _sidecar_overwrites_duplicates),
    "pk12_nibbles_swapped": ("unpack_pk12", _unpack_nibble_swapped),
    "pk12_pair_components_swapped": ("dequant_pk12", _dequant_pk12_components_swapped),
    "bf16_truncation": ("bf16_round_f32", _bf16_truncate),
    "bf16_upcast_wrong": ("bf16_bits_to_f64", _bf16_bits_low_half),
    "bwd_rows_reversed": ("linear_backward_x", _bwd_rows_reversed),
    "bwd_forward_orientation": ("linear_backward_x", _bwd_forward_orientation),
    "bwd_columns_shifted": ("linear_backward_x", _bwd_columns_shifted),
    "bwd_sign_lost": ("linear_backward_x", _bwd_sign_lost),
    "bound_scaled": ("error_bound", _bound_scaled),
    "bound_untransposed": ("error_bound", _bound_untransposed),
    "bound_abs_x_only": ("error_bound", _bound_abs_x_only),
    "bound_abs_w_only": ("error_bound", _bound_abs_w_only),
    "bound_plus_one": ("error_bound", _bound_plus_one),
    "bound_plus_bias": ("hxq_linear_fwd_u8", _fwd_u8_bound_plus_bias),
    "bound_abs_before_sidecar": ("hxq_linear_fwd_u8", _fwd_u8_bound_abs_before_sidecar),
    "bound_bwd_scaled": ("error_bound_bwd", _bound_bwd_scaled),
    "bound_bwd_transposed": ("error_bound_bwd", _bound_bwd_transposed),
    "bound_bwd_abs_dy_only": ("error_bound_bwd", _bound_bwd_abs_dy_only),
    "sidecar_bound_summed_first": ("hxq_sidecar_add", _sidecar_add_bound_summed_first),
    "sidecar_bound_scaled": ("hxq_sidecar_add", _sidecar_add_bound_scaled),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    fn_name, bad = MUTATIONS[name]
    monkeypatch.setattr(H, fn_name, bad)
    monkeypatch.setattr(oracle, fn_name, bad)
    failures = 0
    for pin in PINS:
        try:
            pin()
        except Exception:  # an AssertionError or a shape error both count as caught
            failures += 1
    assert failures > 0, "planted mistake %s passed every pin" % name
