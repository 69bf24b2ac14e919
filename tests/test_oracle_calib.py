"""Pins of the oracle's heavy-channel calibration ("Double Sparsity", section
"offline calibration": K-, Q- and QK-outlier criteria; LeanK section 1.1: the
importance of a channel is the L2 norm of the product of its query column and
its key column).  Each pin checks the oracle against a definition written out
here in numpy, or against a planted answer that the criteria fix."""
import numpy as np
import pytest

import oracle

def _f16(rng, *shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float16)

def test_norms_match_the_written_out_products():
    rng = np.random.default_rng(1)
    B, Hkv, G, N, W, d = 2, 2, 3, 37, 5, 16
    K = _f16(rng, B, Hkv, N, d)
    q = _f16(rng, B, W, Hkv * G, d)
    _, nrm = oracle.calibrate(K, oracle.CALIB_QK, 4, qwin=q)
    Kd, qd = K.astype(np.float64), q.astype(np.float64)
    for g in range(Hkv):
        for c in range(d):
            kn = sum(np.sum(Kd[b, g, :, c] ** 2) for b in range(B))
            qn = sum(np.sum(qd[b, :, g * G:(g + 1) * G, c] ** 2) for b in range(B))
            # the product matrices themselves: rows (window query, head), columns tokens
            fro2 = 0.0
            for b in range(B):
                qcol = qd[b, :, g * G:(g + 1) * G, c].reshape(-1)
                fro2 += np.sum(np.outer(qcol, Kd[b, g, :, c]) ** 2)
            np.testing.assert_allclose(nrm[g, 0, c], kn, rtol=1e-12)
            np.testing.assert_allclose(nrm[g, 1, c], qn, rtol=1e-12)
            np.testing.assert_allclose(nrm[g, 2, c], np.sqrt(fro2), rtol=1e-12)

def test_planted_columns_separate_the_three_criteria():
    # column 3: large K, tiny q; column 5: large q, tiny K; column 7: both
    # moderately large.  K-outlier picks 3, Q-outlier 5, QK-outlier 7.
    rng = np.random.default_rng(2)
    B, Hkv, G, N, W, d = 1, 2, 2, 64, 8, 16
    K = rng.standard_normal((B, Hkv, N, d))
    q = rng.standard_normal((B, W, Hkv * G, d))
    K[..., 3] *= 8.0
    q[..., 3] *= 0.01
    q[..., 5] *= 8.0
    K[..., 5] *= 0.01
    K[..., 7] *= 3.0
    q[..., 7] *= 3.0
    K, q = K.astype(np.float16), q.astype(np.float16)
    assert oracle.calibrate(K, oracle.CALIB_K, 1, qwin=q)[0].tolist() == [[3], [3]]
    assert oracle.calibrate(K, oracle.CALIB_Q, 1, qwin=q)[0].tolist() == [[5], [5]]
    assert oracle.calibrate(K, oracle.CALIB_QK, 1, qwin=q)[0].tolist() == [[7], [7]]

def test_equal_scores_go_to_the_lower_column_and_output_is_ascending():
    K = np.ones((1, 1, 10, 16), np.float16)
    chan, _ = oracle.calibrate(K, oracle.CALIB_K, 5)
    assert chan.tolist() == [[0, 1, 2, 3, 4]]
    # columns 9 and 2 identical and largest, then 12: ties to the lower column
    rng = np.random.default_rng(3)
    K = _f16(rng, 1, 1, 30, 16, scale=0.1)
    K[..., 9] = 1.0
    K[..., 2] = 1.0
    K[..., 12] = 0.9
    assert oracle.calibrate(K, oracle.CALIB_K, 1)[0].tolist() == [[2]]
    assert oracle.calibrate(K, oracle.CALIB_K, 3)[0].tolist() == [[2, 9, 12]]

def test_query_norm_sums_the_group_heads_only():
    # only query head 1 (group 0 of G = 2) has an outlier at channel 9
    rng = np.random.default_rng(4)
    B, Hkv, G, W, d = 1, 2, 2, 4, 16
    q = rng.standard_normal((B, W, Hkv * G, d)) * 0.1
    q[:, :, 1, 9] = 5.0
    q = q.astype(np.float16)
    K = np.ones((B, Hkv, 8, d), np.float16)
    chan, _ = oracle.calibrate(K, oracle.CALIB_Q, 1, qwin=q)
    assert chan[0, 0] == 9 and chan[1, 0] != 9

def test_keep_table_reads_the_query_at_the_kept_channel():
    # stored column c of KV head g is query channel keep[g][c] (LeanK section 2.2)
    rng = np.random.default_rng(5)
    B, Hkv, W, d_q, d_k = 1, 2, 3, 32, 8
    q = rng.standard_normal((B, W, Hkv, d_q)) * 0.1
    q[..., 20] = 4.0
    q = q.astype(np.float16)
    K = np.ones((B, Hkv, 4, d_k), np.float16)
    keep = np.array([[1, 2, 3, 20, 4, 5, 6, 7], [0, 1, 2, 3, 4, 5, 6, 7]], np.int32)
    chan, _ = oracle.calibrate(K, oracle.CALIB_Q, 1, qwin=q, keep=keep)
    assert chan[0, 0] == 3 and chan[1, 0] != 3

def test_selection_is_the_sorted_definition():
    rng = np.random.default_rng(6)
    K = _f16(rng, 3, 4, 50, 32)
    K[:, :, :, 17] = K[:, :, :, 4]  # an exact tie between columns 4 and 17
    q = _f16(rng, 3, 2, 8, 32)
    for crit in (oracle.CALIB_K, oracle.CALIB_Q, oracle.CALIB_QK):
        for r in (1, 8, 31, 32):
            chan, nrm = oracle.calibrate(K, crit, r, qwin=q)
            for g in range(4):
                s = nrm[g, 2]
                order = sorted(range(32), key=lambda c: (-s[c], c))
                assert chan[g].tolist() == sorted(order[:r])

def test_only_the_first_n_tok_tokens_count():
    rng = np.random.default_rng(7)
    K = _f16(rng, 1, 1, 20, 8)
    K2 = K.copy()
    K2[:, :, 12:, 6] = 100.0
    a = oracle.calibrate(K, oracle.CALIB_K, 2, n_tok=12)
    b = oracle.calibrate(K2, oracle.CALIB_K, 2, n_tok=12)
    assert a[0].tolist() == b[0].tolist()
    np.testing.assert_array_equal(a[1], b[1])

def test_bad_arguments_and_non_finite_inputs_are_rejected():
    K = np.ones((1, 1, 4, 8), np.float16)
    with pytest.raises(ValueError):
        oracle.calibrate(K, oracle.CALIB_K, 9)
    with pytest.raises(ValueError):
        oracle.calibrate(K, 3, 2)
    K[0, 0, 1, 2] = np.inf
    with pytest.raises(ValueError):
        oracle.calibrate(K, oracle.CALIB_K, 2)


def test_channel_overlap_hand_worked():
    """The overlap of two channel tables ("Double Sparsity", section "offline
    calibration", offline against online outlier channels), worked by hand:
    head 0 shares {3, 4} of 4 channels, head 1 all 4 (another order), head 2
    none; a table with a repeated channel counts it once ({1, 2, 3} against
    {1, 2, 9}: 2 of r = 4)."""
    a = [[1, 2, 3, 4], [5, 6, 7, 8], [0, 10, 20, 30]]
    b = [[4, 3, 9, 10], [8, 7, 6, 5], [1, 11, 21, 31]]
    np.testing.assert_array_equal(oracle.channel_overlap(a, b), [0.5, 1.0, 0.0])
    np.testing.assert_array_equal(oracle.channel_overlap([[1, 1, 2, 3]], [[1, 2, 2, 9]]), [0.5])
    np.testing.assert_array_equal(oracle.channel_overlap(b, a), [0.5, 1.0, 0.0])
    with pytest.raises(ValueError):
        oracle.channel_overlap(a, [[1, 2, 3, 4]])
