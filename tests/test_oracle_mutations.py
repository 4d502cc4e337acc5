"""Planted mistakes: each test patches one plausible error into the oracle (CPU only) and checks that
an existing pin fails.  This is how we know the pins bind every step."""
import math

import numpy as np
import pytest

from oracle import tq_oracle as O
from tests import test_oracle_codebook as CB
from tests import test_oracle_codec as CC


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_search_off_by_one_is_caught(monkeypatch):
    # the quantise_scalar bug class of [AB] §2: ties to the lower cell
    monkeypatch.setattr(O, "quantise", lambda y, t: np.searchsorted(t, y, side="left").astype(np.int64))
    _fails(CC.test_search_equals_linear_count_at_and_around_every_threshold, 3)


def test_missing_normalisation_is_caught(monkeypatch):
    monkeypatch.setattr(O, "rotate", lambda u, s: (u * s) @ O.hadamard(u.shape[-1]))
    _fails(CB.test_rotated_unit_vector_coordinates_follow_beta_model, 64)


def test_wrong_hadamard_order_is_caught(monkeypatch):
    real = O.hadamard
    monkeypatch.setattr(O, "hadamard", lambda d: real(d)[::-1].copy())
    _fails(CB.test_hadamard_natural_order_closed_form, 8)


def test_unconverged_codebook_is_caught(monkeypatch):
    real = O.lloyd_max
    monkeypatch.setattr(O, "lloyd_max", lambda d, b, **k: real(d, b, max_iter=2))
    _fails(CB.test_lloyd_max_centroid_and_midpoint_conditions, 128, 4)


def test_wrong_density_exponent_is_caught(monkeypatch):
    monkeypatch.setattr(O, "beta_alpha", lambda d: (d - 2) / 2.0)
    _fails(CB.test_lloyd_max_one_bit_closed_form, 64)


def _patched_scores(sign=1.0, denom="m", transpose=False):
    def scores(q, rec, s, centroids, S=None):
        q_rot = O.query_rotate(q, s)
        y_hat = centroids[np.asarray(rec["idx"])]
        n16 = np.asarray(rec["n16"], dtype=np.float64)
        base = q_rot @ y_hat.T
        if S is None:
            return base * n16[None, :]
        S = np.asarray(S, dtype=np.float64)
        m = S.shape[0]
        p = q_rot @ (S if transpose else S.T)
        pm = 2.0 * np.asarray(rec["sigma"], dtype=np.float64) - 1.0
        r16 = np.asarray(rec["r16"], dtype=np.float64)
        k = m if denom == "m" else q_rot.shape[-1]
        return (base + sign * math.sqrt(math.pi / 2) / k * r16[None, :] * (p @ pm.T)) * n16[None, :]
    return scores


def test_qjl_sign_error_is_caught(monkeypatch):
    monkeypatch.setattr(O, "scores", _patched_scores(sign=-1.0))
    _fails(CC.test_qjl_scores_reduce_error_on_average_and_use_every_term)


def test_qjl_wrong_normaliser_is_caught(monkeypatch):
    monkeypatch.setattr(O, "scores", _patched_scores(denom="d"))   # m = 256 != d = 128 there
    _fails(CC.test_qjl_scores_reduce_error_on_average_and_use_every_term)


def test_qjl_estimator_missing_root_is_caught(monkeypatch):
    def bad(q, e, S):
        S = np.asarray(S, dtype=np.float64)
        z = S @ e
        return (math.pi / 2) / S.shape[0] * float(np.linalg.norm(e)) * float((S @ q) @ np.where(z >= 0, 1.0, -1.0))
    monkeypatch.setattr(O, "qjl_estimate", bad)
    _fails(CC.test_qjl_estimator_unbiased_and_variance_closed_form)


def test_wrong_bit_order_is_caught(monkeypatch):
    real = O.pack_bits
    monkeypatch.setattr(O, "pack_bits", lambda v, b: np.packbits(
        ((np.asarray(v)[:, :, None] >> np.arange(b)[None, None, :]) & 1).astype(np.uint8)
        .reshape(np.asarray(v).shape[0], -1), axis=1, bitorder="big"))
    _fails(CC.test_pack_bits_closed_form_and_round_trip)


def test_softmax_over_wrong_axis_is_caught(monkeypatch):
    real = O.softmax
    monkeypatch.setattr(O, "softmax", lambda x, axis=-1: real(x, axis=0))
    _fails(CC.test_attention_rotated_equals_dense)


# ---- randomized Hadamard sketch and the QJL decode correction ----------------------------------
from tests import test_oracle_rht as RH  # noqa: E402


def test_rht_without_second_signs_is_caught(monkeypatch):
    monkeypatch.setattr(O, "rht_matrix", lambda seed, head, d: O.hadamard(d).astype(np.float16))
    _fails(RH.test_rht_matrix_is_hadamard_times_second_signs)


def test_rht_signs_from_the_rotation_tag_are_caught(monkeypatch):
    monkeypatch.setattr(O, "rht_signs", lambda seed, head, d: O.head_signs(seed, head, d))
    _fails(RH.test_rht_signs_balanced_and_distinct_from_rotation_signs)


def test_correction_without_sqrt_is_caught(monkeypatch):
    def corr(sigma, r16, S):
        S = np.asarray(S, dtype=np.float64)
        pm = 2.0 * np.asarray(sigma, dtype=np.float64) - 1.0
        return (math.pi / 2.0) / S.shape[0] * np.asarray(r16, dtype=np.float64)[:, None] * (pm @ S)
    monkeypatch.setattr(O, "qjl_correction", corr)
    _fails(RH.test_correction_closed_form_on_a_hadamard_column)


def test_correction_through_S_instead_of_S_transpose_is_caught(monkeypatch):
    def corr(sigma, r16, S):
        S = np.asarray(S, dtype=np.float64)
        pm = 2.0 * np.asarray(sigma, dtype=np.float64) - 1.0
        return math.sqrt(math.pi / 2.0) / S.shape[0] * np.asarray(r16, dtype=np.float64)[:, None] * (pm @ S.T)
    monkeypatch.setattr(O, "qjl_correction", corr)
    _fails(RH.test_correction_closed_form_on_a_hadamard_column)
