"""Pins for the CPU oracle (runs on the CPU; no GPU).

The oracle is the plain per-token recurrence.  These tests tie it to things
other than itself: the pages' chunkwise-parallel and one-token matrix forms,
closed forms of special cases, exact invariants of the method, and algebraic
properties (linearity, column independence, resumability).  Dimensions are
often chosen with dk != dv so that a transposed state index cannot pass.
"""
import numpy as np
import pytest

import oracle
from pins import (block_doubling_inverse, chunk_form, chunk_form_unit,
                  matrix_step, rel_err, transition_form_unit)


def rand_case(rng, B, T, H, dk, dv, s0=True, unit=True):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = -np.log1p(np.exp(rng.standard_normal((B, T, H))))     # -softplus
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    S0 = 0.1 * rng.standard_normal((B, H, dk, dv)) if s0 else None
    return q, k, v, g, beta, S0


# --- the pages' chunkwise-parallel form -------------------------------------

@pytest.mark.parametrize("C", [1, 5, 16, 64])
@pytest.mark.parametrize("T", [1, 37, 100, 130])
def test_oracle_matches_chunk_form(C, T):
    rng = np.random.default_rng(1000 + 7 * C + T)
    q, k, v, g, beta, S0 = rand_case(rng, 2, T, 2, 12, 7)
    O, S_T = oracle.prefill(q, k, v, g, beta, S0)
    Oc, Sc = chunk_form(q, k, v, g, beta, S0, C)
    assert rel_err(O, Oc) < 1e-12
    assert rel_err(S_T, Sc) < 1e-12


def test_oracle_matches_chunk_form_full_head_size_slow_decay():
    # dk = dv = 128 as on the page, with a slow decay so that the state carries
    # far across chunk boundaries (the workloads' decay forgets within tokens).
    rng = np.random.default_rng(5)
    q, k, v, g, beta, S0 = rand_case(rng, 1, 150, 1, 128, 128)
    g = g * 0.01
    O, S_T = oracle.prefill(q, k, v, g, beta, S0)
    Oc, Sc = chunk_form(q, k, v, g, beta, S0, 64)
    assert rel_err(O, Oc) < 1e-12
    assert rel_err(S_T, Sc) < 1e-12


def test_chunk_form_is_chunk_size_invariant():
    rng = np.random.default_rng(11)
    q, k, v, g, beta, S0 = rand_case(rng, 1, 200, 1, 16, 9)
    ref = chunk_form(q, k, v, g, beta, S0, 1)
    for C in (16, 64):
        O, S = chunk_form(q, k, v, g, beta, S0, C)
        assert rel_err(O, ref[0]) < 1e-12 and rel_err(S, ref[1]) < 1e-12


def test_block_doubling_inverse_is_exact():
    # the page's exact triangular inverse agrees with a library triangular solve
    rng = np.random.default_rng(3)
    for n in (16, 64):
        k = rng.standard_normal((n, 32))
        k /= np.linalg.norm(k, axis=1, keepdims=True)
        N = np.tril(0.5 * (k @ k.T), -1)
        M = np.eye(n) + N
        Tinv = block_doubling_inverse(M)
        assert np.max(np.abs(Tinv @ M - np.eye(n))) < 1e-13
        from scipy.linalg import solve_triangular
        ref = solve_triangular(M, np.eye(n), lower=True, unit_diagonal=True)
        assert np.max(np.abs(Tinv - ref)) < 1e-13


# --- the one-token matrix form ----------------------------------------------

def test_decode_step_matches_matrix_form():
    rng = np.random.default_rng(4)
    dk, dv = 10, 6
    q, k, v, g, beta, _ = rand_case(rng, 1, 1, 3, dk, dv)
    S = 0.1 * rng.standard_normal((1, 3, dk, dv))
    o, S1 = oracle.decode(q[0], k[0], v[0], g[0], beta[0], S)
    for h in range(3):
        om, Sm = matrix_step(q[0, 0, h], k[0, 0, h], v[0, 0, h], g[0, 0, h],
                             beta[0, 0, h], S[0, h])
        assert rel_err(o[0, h], om) < 1e-14
        assert rel_err(S1[0, h], Sm) < 1e-14


def test_decode_layout_equals_prefill_layout():
    # decode steps [steps, B, H, d] and a prefill over the same tokens
    # [B, T, H, d] are the same recurrence: bit-identical
    rng = np.random.default_rng(8)
    q, k, v, g, beta, S0 = rand_case(rng, 3, 9, 2, 8, 5)
    O, S_T = oracle.prefill(q, k, v, g, beta, S0)
    tr = lambda x: np.ascontiguousarray(np.swapaxes(x, 0, 1))
    o, S = oracle.decode(tr(q), tr(k), tr(v), tr(g), tr(beta), S0)
    assert np.array_equal(tr(o), O) and np.array_equal(S, S_T)


# --- brute force and closed forms -------------------------------------------

def test_transition_matrix_brute_force():
    rng = np.random.default_rng(9)
    q, k, v, g, beta, S0 = rand_case(rng, 1, 40, 1, 9, 4, unit=False)
    O, S_T = oracle.prefill(q, k, v, g, beta, S0)
    Ob, Sb = transition_form_unit(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0],
                                  beta[0, :, 0], S0[0, 0])
    assert rel_err(O[0, :, 0], Ob) < 1e-12 and rel_err(S_T[0, 0], Sb) < 1e-12


def test_projection_invariant_reads_back_written_value():
    # g = 0, beta = 1, unit keys: after writing (k_t, v_t) the state returns v_t
    # for k_t (S_t^T k_t = v_t); querying with q_t = k_t makes o_t = v_t.
    rng = np.random.default_rng(12)
    q, k, v, g, beta, S0 = rand_case(rng, 1, 60, 2, 16, 11)
    O, _ = oracle.prefill(k, k, v, np.zeros_like(g), np.ones_like(beta), S0)
    assert np.max(np.abs(O - v)) < 1e-12


def test_orthonormal_keys_closed_form():
    # g = 0, beta = 1, orthonormal keys (successive projections onto orthogonal
    # complements): S_t = (I - K_t^T K_t) S0 + K_t^T V_t with K_t the first t keys.
    rng = np.random.default_rng(13)
    dk, dv, T = 24, 10, 20
    Kq, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    K = Kq[:, :T].T                                   # [T, dk], orthonormal rows
    V = rng.standard_normal((T, dv))
    Q = rng.standard_normal((T, dk))
    S0 = rng.standard_normal((dk, dv))
    O, S_T = oracle.prefill(Q[None, :, None], K[None, :, None], V[None, :, None],
                            np.zeros((1, T, 1)), np.ones((1, T, 1)), S0[None, None])
    for t in range(T):
        Kt, Vt = K[:t + 1], V[:t + 1]
        St = (np.eye(dk) - Kt.T @ Kt) @ S0 + Kt.T @ Vt
        assert np.max(np.abs(O[0, t, 0] - St.T @ Q[t])) < 1e-12
    assert np.max(np.abs(S_T[0, 0] - ((np.eye(dk) - K.T @ K) @ S0 + K.T @ V))) < 1e-12


def test_beta_zero_is_pure_decay():
    rng = np.random.default_rng(14)
    q, k, v, g, beta, S0 = rand_case(rng, 1, 30, 2, 7, 5)
    O, S_T = oracle.prefill(q, k, v, g, np.zeros_like(beta), S0)
    G = np.cumsum(g, axis=1)                                 # [1, T, H]
    for h in range(2):
        for t in range(30):
            ref = np.exp(G[0, t, h]) * (S0[0, h].T @ q[0, t, h])
            assert np.max(np.abs(O[0, t, h] - ref)) < 1e-14
        assert rel_err(S_T[0, h], np.exp(G[0, -1, h]) * S0[0, h]) < 1e-13


def test_full_decay_keeps_only_the_current_token():
    # exp(g) = 0: S_t = beta_t k_t v_t^T and o_t = beta_t (q_t . k_t) v_t
    rng = np.random.default_rng(15)
    q, k, v, g, beta, S0 = rand_case(rng, 1, 12, 3, 9, 6)
    g = np.full_like(g, -1e4)                                 # exp underflows to 0
    O, S_T = oracle.prefill(q, k, v, g, beta, S0)
    qk = np.einsum("bthd,bthd->bth", q, k)
    assert np.max(np.abs(O - (beta * qk)[..., None] * v)) < 1e-14
    for h in range(3):
        ref = beta[0, -1, h] * np.outer(k[0, -1, h], v[0, -1, h])
        assert np.max(np.abs(S_T[0, h] - ref)) < 1e-14


def test_single_token_from_zero_state():
    rng = np.random.default_rng(16)
    q, k, v, g, beta, _ = rand_case(rng, 4, 1, 2, 8, 8)
    O, S_T = oracle.prefill(q, k, v, g, beta, None)
    qk = np.einsum("bthd,bthd->bth", q, k)
    assert np.max(np.abs(O - (beta * qk)[..., None] * v)) < 1e-15
    ref = beta[:, 0, :, None, None] * np.einsum("bhi,bhj->bhij", k[:, 0], v[:, 0])
    assert np.max(np.abs(S_T - ref)) < 1e-15


def test_zero_length_sequence_returns_initial_state():
    rng = np.random.default_rng(17)
    q, k, v, g, beta, S0 = rand_case(rng, 1, 10, 2, 8, 4)
    cu = np.array([0, 4, 4, 10])
    S0_3 = 0.1 * rng.standard_normal((3, 2, 8, 4))
    _, S_T = oracle.prefill(q, k, v, g, beta, S0_3, cu_seqlens=cu)
    assert np.array_equal(S_T[1], S0_3[1])


# --- algebraic properties ---------------------------------------------------

def test_linear_in_values_and_state_jointly():
    rng = np.random.default_rng(18)
    q, k, v, g, beta, S0 = rand_case(rng, 1, 50, 2, 10, 6)
    v2 = rng.standard_normal(v.shape)
    S02 = rng.standard_normal(S0.shape)
    O1, S1 = oracle.prefill(q, k, v, g, beta, S0)
    O2, S2 = oracle.prefill(q, k, v2, g, beta, S02)
    O3, S3 = oracle.prefill(q, k, 2.0 * v - 3.0 * v2, g, beta, 2.0 * S0 - 3.0 * S02)
    assert rel_err(O3, 2 * O1 - 3 * O2) < 1e-12
    assert rel_err(S3, 2 * S1 - 3 * S2) < 1e-12


def test_output_scales_exactly_with_q():
    # O is linear in q; a power-of-two scale (the page's q x 1024) is exact in fp64
    rng = np.random.default_rng(19)
    q, k, v, g, beta, S0 = rand_case(rng, 1, 40, 2, 12, 8)
    O, S_T = oracle.prefill(q, k, v, g, beta, S0)
    O2, S_T2 = oracle.prefill(1024.0 * q, k, v, g, beta, S0)
    assert np.array_equal(O2, 1024.0 * O) and np.array_equal(S_T2, S_T)


def test_value_columns_are_independent():
    rng = np.random.default_rng(20)
    q, k, v, g, beta, S0 = rand_case(rng, 1, 33, 1, 9, 6)
    O, S_T = oracle.prefill(q, k, v, g, beta, S0)
    v2, S02 = v.copy(), S0.copy()
    v2[..., 2] += rng.standard_normal(v2[..., 2].shape)
    S02[..., 2] += 1.0
    Ob, Sb = oracle.prefill(q, k, v2, g, beta, S02)
    keep = [0, 1, 3, 4, 5]
    assert np.array_equal(O[..., keep], Ob[..., keep])
    assert np.array_equal(S_T[..., keep], Sb[..., keep])
    assert not np.array_equal(O[..., 2], Ob[..., 2])


def test_split_and_resume_equals_one_run():
    rng = np.random.default_rng(21)
    q, k, v, g, beta, S0 = rand_case(rng, 2, 70, 2, 8, 8)
    O, S_T = oracle.prefill(q, k, v, g, beta, S0)
    O1, S1 = oracle.prefill(q[:, :23], k[:, :23], v[:, :23], g[:, :23], beta[:, :23], S0)
    O2, S2 = oracle.prefill(q[:, 23:], k[:, 23:], v[:, 23:], g[:, 23:], beta[:, 23:], S1)
    assert np.array_equal(np.concatenate([O1, O2], axis=1), O)
    assert np.array_equal(S2, S_T)


def test_packed_batch_equals_separate_calls():
    rng = np.random.default_rng(22)
    lens = [5, 17, 1, 40]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta, _ = rand_case(rng, 1, int(cu[-1]), 3, 8, 6)
    S0 = 0.1 * rng.standard_normal((len(lens), 3, 8, 6))
    O, S_T = oracle.prefill(q, k, v, g, beta, S0, cu_seqlens=cu)
    for n, (s, e) in enumerate(zip(cu[:-1], cu[1:])):
        On, Sn = oracle.prefill(q[:, s:e], k[:, s:e], v[:, s:e], g[:, s:e],
                                beta[:, s:e], S0[n:n + 1])
        assert np.array_equal(O[:, s:e], On) and np.array_equal(S_T[n], Sn[0])
    Oc, Sc = chunk_form(q, k, v, g, beta, S0, 16, cu_seqlens=cu)
    assert rel_err(O, Oc) < 1e-12 and rel_err(S_T, Sc) < 1e-12


def test_thread_count_does_not_change_bits():
    rng = np.random.default_rng(23)
    q, k, v, g, beta, S0 = rand_case(rng, 3, 20, 4, 8, 8)
    a = oracle.prefill(q, k, v, g, beta, S0, nthreads=1)
    b = oracle.prefill(q, k, v, g, beta, S0, nthreads=7)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_bad_arguments_are_rejected():
    rng = np.random.default_rng(24)
    q, k, v, g, beta, S0 = rand_case(rng, 1, 10, 1, 4, 4)
    with pytest.raises(ValueError):
        oracle.prefill(q, k, v, g, beta, S0[:, :, :3])
    with pytest.raises(ValueError):   # cu_seqlens that does not end at T
        oracle.prefill(q, k, v, g, beta, None, cu_seqlens=np.array([0, 4, 9]))


def test_chunk_form_unit_matches_transition_form_with_padding_only_tail():
    # a single partial block (the speculative-verify shape: 16 real rows of 64)
    rng = np.random.default_rng(25)
    q, k, v, g, beta, S0 = rand_case(rng, 1, 16, 1, 128, 128)
    a = chunk_form_unit(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0],
                        S0[0, 0], 64)
    b = transition_form_unit(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0],
                             beta[0, :, 0], S0[0, 0])
    assert rel_err(a[0], b[0]) < 1e-12 and rel_err(a[1], b[1]) < 1e-12


# --- per-token states (the rewindable verify form) --------------------------

def test_token_states_equal_the_prompt_form_on_every_prefix():
    # the state after token t equals the pages' chunk form run on the prefix
    # through t (an independent NumPy implementation), in packed batches
    rng = np.random.default_rng(31)
    lens = [3, 16, 0, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta, _ = rand_case(rng, 1, int(cu[-1]), 2, 7, 5)
    S0 = 0.1 * rng.standard_normal((len(lens), 2, 7, 5))
    O, S_T, S_tok = oracle.prefill(q, k, v, g, beta, S0, cu_seqlens=cu, states=True)
    assert S_tok.shape == (1, int(cu[-1]), 2, 7, 5)
    for n, (s, e) in enumerate(zip(cu[:-1], cu[1:])):
        for t in range(s, e):
            for h in range(2):
                _, Sp = chunk_form_unit(q[0, s:t + 1, h], k[0, s:t + 1, h], v[0, s:t + 1, h],
                                        g[0, s:t + 1, h], beta[0, s:t + 1, h], S0[n, h], 5)
                assert rel_err(S_tok[0, t, h], Sp) < 1e-12


def test_token_states_follow_the_matrix_form():
    # the pages' one-token matrix form, iterated, gives every emitted state
    rng = np.random.default_rng(32)
    q, k, v, g, beta, S0 = rand_case(rng, 2, 12, 2, 6, 9)
    O, S_T, S_tok = oracle.prefill(q, k, v, g, beta, S0, states=True)
    for b in range(2):
        for h in range(2):
            S = S0[b, h]
            for t in range(12):
                o, S = matrix_step(q[b, t, h], k[b, t, h], v[b, t, h], g[b, t, h], beta[b, t, h], S)
                assert rel_err(S_tok[b, t, h], S) < 1e-12
                assert rel_err(O[b, t, h], o) < 1e-12


def test_token_states_keep_outputs_and_final_state():
    rng = np.random.default_rng(33)
    q, k, v, g, beta, S0 = rand_case(rng, 2, 10, 3, 8, 8)
    O, S_T = oracle.prefill(q, k, v, g, beta, S0)
    O2, S_T2, S_tok = oracle.prefill(q, k, v, g, beta, S0, states=True)
    assert np.array_equal(O, O2) and np.array_equal(S_T, S_T2)
    assert np.array_equal(S_tok[:, -1], S_T)


# --- the gated RMS norm on the output (the norm that follows the recurrence) ---

def test_gated_rmsnorm_closed_form_two_columns():
    # Hand-computed: rows of two values, so mean(o^2) = (o0^2 + o1^2) / 2; gates
    # at +-ln 3, where sigmoid is 3/4 and 1/4; distinct weights per column.
    l3 = np.log(3.0)
    o = np.array([[3.0, 4.0], [-1.0, 0.0]])
    z = np.array([[l3, -l3], [l3, l3]])
    w = np.array([2.0, 0.5])
    y = oracle.gated_rmsnorm(o, z, w, 0.0)
    r = 1.0 / np.sqrt(12.5)
    expect = np.array([[2.0 * 3.0 * r * 0.75 * l3, 0.5 * 4.0 * r * (-0.25 * l3)],
                       [2.0 * -1.0 * np.sqrt(2.0) * 0.75 * l3, 0.0]])
    assert rel_err(y, expect) < 1e-14
    # eps sits inside the root, added to the mean square: 12.5 + 12.5 = 25
    y = oracle.gated_rmsnorm(o[:1], z[:1], w, 12.5)
    assert rel_err(y, np.array([[2.0 * 3.0 / 5.0 * 0.75 * l3, 0.5 * 4.0 / 5.0 * (-0.25 * l3)]])) < 1e-14


def test_gated_rmsnorm_rows_have_unit_rms_once_the_gate_is_divided_out():
    from scipy.special import expit
    rng = np.random.default_rng(31)
    o = rng.standard_normal((9, 128)) * rng.uniform(1e-3, 10.0, (9, 1))
    z = rng.standard_normal((9, 128))
    y = oracle.gated_rmsnorm(o, z, np.ones(128), 0.0)
    unit = y / (z * expit(z))
    assert np.allclose(np.sqrt(np.mean(unit ** 2, axis=-1)), 1.0, rtol=1e-13, atol=0)
    assert np.allclose(unit * np.sqrt(np.mean(o ** 2, axis=-1, keepdims=True)), o,
                       rtol=1e-13, atol=1e-300)


def test_gated_rmsnorm_gate_limits():
    rng = np.random.default_rng(32)
    o = rng.standard_normal((3, 16))
    w = rng.uniform(0.5, 1.5, 16)
    # a strongly negative gate shuts the output, zero gate gives exactly zero
    assert np.abs(oracle.gated_rmsnorm(o, np.full_like(o, -60.0), w, 1e-6)).max() < 1e-20
    assert np.all(oracle.gated_rmsnorm(o, np.zeros_like(o), w, 1e-6) == 0.0)
    # a strongly positive gate passes x * 1: y = w o / rms(o) * z
    z = np.full_like(o, 40.0)
    y = oracle.gated_rmsnorm(o, z, w, 0.0)
    rms = np.sqrt(np.mean(o ** 2, axis=-1, keepdims=True))
    assert rel_err(y, w * o / rms * 40.0) < 1e-15


def test_gated_norm_of_the_output_is_invariant_to_the_pages_q_rescale():
    # The Qwen3.5-9B-npu page rescales q by 1024 inside the recurrence and the
    # norm's eps by 1024^2 and states that nothing changes: O is linear in q, so
    # mean(O^2) scales by 1024^2 and the norm's output does not change.
    rng = np.random.default_rng(33)
    q, k, v, g, beta, S0 = rand_case(rng, 1, 40, 2, 128, 128)
    z = rng.standard_normal((1, 40, 2, 128))
    w = rng.uniform(0.5, 1.5, 128)
    eps = 1e-3
    O, _ = oracle.prefill(q, k, v, g, beta, S0)
    O2, _ = oracle.prefill(1024.0 * q, k, v, g, beta, S0)
    y = oracle.gated_rmsnorm(O, z, w, eps)
    assert rel_err(oracle.gated_rmsnorm(O2, z, w, eps * 1024.0 ** 2), y) < 1e-12
    # ... and eps matters here, so the check above is not vacuous
    assert rel_err(oracle.gated_rmsnorm(O2, z, w, eps), y) > 1e-4


def test_gated_rmsnorm_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.gated_rmsnorm(np.ones((2, 4)), np.ones((2, 3)), np.ones(4), 1e-6)
    with pytest.raises(ValueError):
        oracle.gated_rmsnorm(np.ones((2, 4)), np.ones((2, 4)), np.ones(4), -1.0)


# --- the block's pre-operations (conv FIFO, silu, L2 norm, gates) --------------

def preop_case(rng, B, T, H, d, K=4, N=None):
    x = [rng.standard_normal((B, T, H, d)) for _ in range(3)]
    a = rng.standard_normal((B, T, H))
    b = rng.standard_normal((B, T, H))
    w = rng.standard_normal((3, H, d, K)) * 0.5
    st = rng.standard_normal((N or B, 3, H, K - 1, d))
    return x, a, b, w, st


def test_preop_conv_is_numpy_correlate_over_state_and_rows():
    from scipy.special import expit
    rng = np.random.default_rng(51)
    x, a, b, w, st = preop_case(rng, 1, 9, 2, 6)
    _, _, v, _, _, _ = oracle.preop(*x, a, b, w, st, eps=0.0)
    for h in range(2):
        for c in range(6):
            full = np.concatenate([st[0, 2, h, :, c], x[2][0, :, h, c]])
            conv = np.correlate(full, w[2, h, c], mode="valid")       # 9 outputs
            assert np.allclose(v[0, :, h, c], conv * expit(conv), rtol=1e-13, atol=1e-15)


def test_preop_one_hot_taps():
    from scipy.special import expit
    rng = np.random.default_rng(52)
    x, a, b, w, st = preop_case(rng, 1, 7, 1, 5)
    # the newest tap alone: q is silu(x) normalised
    w1 = np.zeros_like(w); w1[..., 3] = 1.0
    q, _, v, _, _, _ = oracle.preop(*x, a, b, w1, st, eps=0.0)
    y = x[0] * expit(x[0])
    assert rel_err(q, y / np.linalg.norm(y, axis=-1, keepdims=True)) < 1e-14
    assert rel_err(v, x[2] * expit(x[2])) < 1e-14
    # the oldest tap alone: v_t = silu(x_{t-3}), the first three from the FIFO
    w0 = np.zeros_like(w); w0[..., 0] = 1.0
    _, _, v, _, _, _ = oracle.preop(*x, a, b, w0, st, eps=0.0)
    src = np.concatenate([st[0, 2, 0], x[2][0, :, 0]], axis=0)[:7]
    assert rel_err(v[0, :, 0], src * expit(src)) < 1e-14


def test_preop_q_and_k_have_unit_norm():
    rng = np.random.default_rng(53)
    x, a, b, w, st = preop_case(rng, 2, 11, 3, 16)
    q, k, _, _, _, _ = oracle.preop(*x, a, b, w, st, eps=0.0)
    assert np.allclose(np.linalg.norm(q, axis=-1), 1.0, rtol=1e-13, atol=0)
    assert np.allclose(np.linalg.norm(k, axis=-1), 1.0, rtol=1e-13, atol=0)


def test_preop_gates_closed_forms():
    rng = np.random.default_rng(54)
    x, a, b, w, st = preop_case(rng, 1, 4, 1, 4)
    a[0, :, 0] = [0.0, np.log(np.e - 1.0), -30.0, 30.0]
    b[0, :, 0] = [0.0, np.log(3.0), -np.log(3.0), 40.0]
    _, _, _, g, beta, _ = oracle.preop(*x, a, b, w, st)
    assert rel_err(g[0, :, 0], [-np.log(2.0), -1.0, -np.exp(-30.0), -30.0]) < 1e-12
    assert rel_err(beta[0, :, 0], [0.5, 0.75, 0.25, 1.0]) < 1e-15


def test_preop_fifo_after_short_and_long_calls():
    rng = np.random.default_rng(55)
    x, a, b, w, st = preop_case(rng, 1, 6, 2, 4)
    # one token: the FIFO keeps its two newest rows and appends the token
    sl = lambda t, n: t[:, :n]
    out = oracle.preop(*(sl(xx, 1) for xx in x), sl(a, 1), sl(b, 1), w, st)
    s_out = out[5]
    for s in range(3):
        assert np.array_equal(s_out[0, s, :, :2], st[0, s, :, 1:])
        assert np.array_equal(s_out[0, s, :, 2], x[s][0, 0])
    # six tokens: the FIFO is the last three rows
    s_out = oracle.preop(*x, a, b, w, st)[5]
    for s in range(3):
        assert np.array_equal(s_out[0, s], np.moveaxis(x[s][0, 3:], 0, 1))


@pytest.mark.parametrize("cut", [1, 2, 3, 7])
def test_preop_split_and_resume_equals_one_call(cut):
    rng = np.random.default_rng(56 + cut)
    x, a, b, w, st = preop_case(rng, 1, 12, 2, 8)
    whole = oracle.preop(*x, a, b, w, st)
    p1 = oracle.preop(*(xx[:, :cut] for xx in x), a[:, :cut], b[:, :cut], w, st)
    p2 = oracle.preop(*(xx[:, cut:] for xx in x), a[:, cut:], b[:, cut:], w, p1[5])
    for i in range(5):
        assert np.array_equal(np.concatenate([p1[i], p2[i]], axis=1), whole[i])
    assert np.array_equal(p2[5], whole[5])


def test_preop_packed_batch_equals_separate_calls():
    rng = np.random.default_rng(57)
    lens = [5, 0, 2, 9]
    T = sum(lens)
    x, a, b, w, _ = preop_case(rng, 1, T, 2, 8)
    st = rng.standard_normal((len(lens), 3, 2, 3, 8))
    cu = np.concatenate([[0], np.cumsum(lens)])
    packed = oracle.preop(*x, a, b, w, st, cu_seqlens=cu)
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        one = oracle.preop(*(xx[:, s:e] for xx in x), a[:, s:e], b[:, s:e], w, st[n:n + 1])
        for i in range(5):
            assert np.array_equal(packed[i][:, s:e], one[i])
        assert np.array_equal(packed[5][n], one[5][0])
