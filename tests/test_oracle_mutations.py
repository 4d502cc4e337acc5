"""Planted mistakes: each test patches one plausible error into the oracle (CPU only) and checks that
an existing pin fails.  This is how we know the pins bind every step."""
import math

import numpy as np
import pytest

from oracle import tq_oracle as O
from tests import test_oracle_codebook as CB
from tests import test_oracle_codec as CC
from tests import test_oracle_sketch as SKP


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


# ---- SpectralQuant oracle ---------------------------------------------------------------------
from oracle import sq_oracle as SQ
from tests import test_oracle_sq as SP


def test_sq_projection_through_the_transpose_is_caught(monkeypatch):
    monkeypatch.setattr(SQ, "project", lambda x, model: np.asarray(x, dtype=np.float64) @ model["U"].T)
    _fails(SP.test_codec_distortion_is_the_gaussian_rate_distortion_of_its_allocation, False)


def test_sq_scale_by_variance_instead_of_deviation_is_caught(monkeypatch):
    real = SQ.calibrate
    def calibrate(*a, **k):
        m = real(*a, **k)
        m["sigma"] = m["sigma"] ** 2
        return m
    monkeypatch.setattr(SQ, "calibrate", calibrate)
    _fails(SP.test_codec_distortion_is_the_gaussian_rate_distortion_of_its_allocation, True)


def test_sq_waterfill_to_the_smallest_distortion_is_caught(monkeypatch):
    def waterfill(lam_sem, total, b_tail, b_max=8):
        bits = np.full(len(lam_sem), b_tail, dtype=np.int64)
        for _ in range(total - int(bits.sum())):
            k = int(np.argmin(np.where(bits < b_max, lam_sem * 4.0 ** -bits, np.inf)))
            bits[k] += 1
        return bits
    monkeypatch.setattr(SQ, "waterfill", waterfill)
    _fails(SP.test_waterfill_is_uniform_at_ratio_at_most_4_and_optimal_otherwise)


def test_sq_tail_at_the_semantic_width_is_caught(monkeypatch):
    real = SQ.calibrate
    def calibrate(x, b, b_tail, **k):
        return real(x, b, b, **k)
    monkeypatch.setattr(SQ, "calibrate", calibrate)
    _fails(SP.test_storage_bits_match_the_pages)


def test_sq_inverted_gap_ratio_is_caught(monkeypatch):
    def effective_dim(lam, gamma=10.0, d_eff_max=0):
        d_eff = min(max(SQ.participation_ratio(lam), 1), len(lam))
        if gamma > 0:
            for k in range(1, d_eff):
                if lam[k] / lam[k - 1] > gamma:
                    d_eff = k
                    break
        return min(d_eff, d_eff_max) if d_eff_max > 0 else d_eff
    monkeypatch.setattr(SQ, "effective_dim", effective_dim)
    _fails(SP.test_gap_criterion_trims_a_spurious_dimension_and_the_cap_applies)


def test_sq_centred_covariance_is_caught(monkeypatch):
    def covariance(x_cal):
        x = np.asarray(x_cal, dtype=np.float64)
        x = x - x.mean(axis=0)
        return x.T @ x / x.shape[0]
    monkeypatch.setattr(SQ, "covariance", covariance)
    _fails(SP.test_covariance_is_not_centred)


def test_sq_msb_first_fields_are_caught(monkeypatch):
    def pack(idx, bits, rec_bytes):
        n, d = idx.shape
        out = np.zeros((n, rec_bytes * 8), dtype=np.uint8)
        pos = 0
        for k in range(d):
            w = int(bits[k])
            for i in range(w):
                out[:, pos + i] = (idx[:, k] >> (w - 1 - i)) & 1
            pos += w
        return np.packbits(out, axis=1, bitorder="little")
    monkeypatch.setattr(SQ, "pack", pack)
    _fails(SP.test_index_is_the_nearest_centroid_and_records_round_trip)


def test_sq_unconverged_codebook_is_caught(monkeypatch):
    real = SQ.gauss_lloyd_max.__wrapped__
    monkeypatch.setattr(SQ, "gauss_lloyd_max", lambda b, **k: real(b, max_iter=2))
    _fails(SP.test_gauss_codebook_matches_max_1960_table)


def test_sq_ties_to_the_lower_cell_are_caught(monkeypatch):
    real = SQ.encode
    def encode(x, model):
        r = real(x, model)
        for w in np.unique(model["bits"]):
            cols = model["bits"] == w
            t, _ = SQ.gauss_lloyd_max(int(w))
            r["idx"][:, cols] = np.sum(r["u"][:, cols, None] > t[None, None, :], axis=2)
        return r
    monkeypatch.setattr(SQ, "encode", encode)
    _fails(SP.test_index_counts_thresholds_with_ties_to_the_upper_cell)


# ---- Fmag oracle ------------------------------------------------------------------------------
from oracle import fmag_oracle as FM
from tests import test_oracle_fmag as FP


def test_fmag_conjugated_spectrum_is_caught(monkeypatch):
    real = FM.rfft
    monkeypatch.setattr(FM, "rfft", lambda x: np.conj(real(x)))
    _fails(FP.test_transform_is_the_written_out_dft_and_its_real_inverse, 16)


def test_fmag_min_max_over_2_to_the_b_levels_is_caught(monkeypatch):
    real = FM.encode
    def encode(x, b, p):
        r = real(x, b, p)
        span = (r["hi"] - r["lo"])[:, None]
        r["q"] = np.minimum(np.floor((r["mag"] - r["lo"][:, None]) / span * (1 << b) + 0.5).astype(np.int64),
                            (1 << b) - 1)
        return r
    monkeypatch.setattr(FM, "encode", encode)
    _fails(FP.test_min_max_quantiser_exact_points_and_bound)


def test_fmag_phase_truncated_instead_of_rounded_is_caught(monkeypatch):
    real = FM.encode
    def encode(x, b, p):
        r = real(x, b, p)
        if r["pidx"] is not None:
            P = 1 << p
            r["pidx"] = np.floor((r["phase"] + math.pi) / (2 * math.pi) * P).astype(np.int64) % P
        return r
    monkeypatch.setattr(FM, "encode", encode)
    _fails(FP.test_phase_levels_and_bound, 6)


def test_fmag_inverse_without_the_half_spectrum_weights_is_caught(monkeypatch):
    monkeypatch.setattr(FM, "irfft", lambda X, d: np.fft.ifft(np.concatenate([X, np.zeros((X.shape[0], d - X.shape[1]))], axis=1), n=d).real)
    _fails(FP.test_transform_is_the_written_out_dft_and_its_real_inverse, 16)


def test_sq_sketch_with_the_residual_sign_flipped_is_caught(monkeypatch):
    real = SQ.sketch_of
    def sketch_of(z, idx, model):
        r = real(z, idx, model)
        r["sigma_bits"] = 1 - r["sigma_bits"]
        return r
    monkeypatch.setattr(SQ, "sketch_of", sketch_of)
    _fails(SP.test_sketch_bits_and_norm_written_out)


def test_sq_correction_without_the_sqrt_is_caught(monkeypatch):
    real = SQ.scores
    def scores(q, idx, model, sigma_bits=None, r16=None):
        out = real(q, idx, model, sigma_bits, r16)
        if model.get("m"):
            base = real(q, idx, {k: v for k, v in model.items() if k != "m"})
            out = base + (out - base) * math.sqrt(2 / math.pi) * (math.pi / 2)
        return out
    monkeypatch.setattr(SQ, "scores", scores)
    _fails(SP.test_selective_qjl_estimate_is_close_to_unbiased)


def test_half_precision_sketch_residual_is_caught(monkeypatch):
    def half(e, S, tol=O.FLAG_TOL):
        eh = (np.asarray(e, dtype=np.float64) * 2.0 ** 14).astype(np.float16).astype(np.float64) / 2.0 ** 14
        z = eh @ np.asarray(S, dtype=np.float64).T
        return {"z": z, "sigma": z >= 0.0, "sflag": np.abs(z) < tol}
    monkeypatch.setattr(O, "sketch", half)
    _fails(SKP.test_sketch_takes_the_exact_residual)


def test_sketch_of_the_negated_residual_is_caught(monkeypatch):
    real = O.sketch
    monkeypatch.setattr(O, "sketch", lambda e, S, tol=O.FLAG_TOL: real(-np.asarray(e), S, tol))
    _fails(SKP.test_encoded_sketch_by_brute_force_at_d8)


def test_sketch_sign_of_zero_negative_is_caught(monkeypatch):
    real = O.sketch
    def neg0(e, S, tol=O.FLAG_TOL):
        r = real(e, S, tol)
        r["sigma"] = r["z"] > 0.0
        return r
    monkeypatch.setattr(O, "sketch", neg0)
    _fails(SKP.test_sketch_of_a_small_case_written_out)
