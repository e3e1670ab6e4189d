"""GPU parity of gdn_prefill_states (the prompt form keeping the state after
every token, for rolling a verify pass back to any accepted prefix) against the
fp64 oracle's per-token states, through the C ABI.

Tolerances as for the prompt form: per-slice normwise error <= 2e-3 for bf16
inputs (with a bf16 output's own rounding allowed elementwise) and <= 1e-5 for
fp32 inputs; every emitted state is one slice.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrence_02_amd import inputs
from linear_attention_recurrence_02_amd.binding import gdn_chunk_prefill, gdn_prefill_states
from metrics import TOL_BF16, TOL_F32, bf16_output_ok, spans_of, worst_slice_error

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def run_states(w, **kw):
    O, S_tok = gdn_prefill_states(w.q, w.k, w.v, w.g, w.beta, w.S0, w.cu_seqlens, **kw)
    torch.cuda.synchronize()
    return O, S_tok


def check(w, O, S_tok, Or, Str, label):
    """O and every per-token state of a (sub)workload against the oracle."""
    spans = spans_of(w.q.shape[0], w.q.shape[1], w.cu_seqlens)
    H = w.q.shape[2]
    eo = worst_slice_error(O, Or, spans, H)
    es = worst_slice_error(S_tok, Str)
    say(f"[{label}] worst slice error O={eo:.3e} S_tok={es:.3e}")
    if w.q.dtype == torch.float32:
        assert eo <= TOL_F32 and es <= TOL_F32, (eo, es)
    else:
        ok, ratio = bf16_output_ok(O, Or, TOL_BF16, spans, H)
        assert ok, f"bf16 O exceeds bound by x{ratio:.3f} (raw {eo:.3e})"
        assert es <= TOL_BF16, es


def test_token_states_verify_blocks_full():
    # 32 verify blocks of 16 tokens from snapshotted states: every token's state
    w = inputs.verify_workload(32, 16, 16, device=DEV)
    snap = w.S0.clone()
    O, S_tok = run_states(w)
    assert torch.equal(w.S0, snap), "S0 must be left untouched"
    Or, _, Str = oracle.prefill(w.q, w.k, w.v, w.g, w.beta, w.S0, cu_seqlens=w.cu_seqlens,
                                states=True)
    check(w, O, S_tok, Or, Str, "verify states")


def test_token_states_verify_workload_sampled_sequences():
    # the full verify workload (256 x 16 tokens x 16 heads: 4 GiB of states);
    # sampled sequences in full against the oracle
    w = inputs.verify_blocks(device=DEV)
    O, S_tok = run_states(w)
    cu = w.cu_seqlens.cpu().numpy()
    for n in (0, 97, 255):
        s, e = int(cu[n]), int(cu[n + 1])
        sl = lambda x: x[:, s:e]
        Or, _, Str = oracle.prefill(sl(w.q), sl(w.k), sl(w.v), sl(w.g), sl(w.beta),
                                    w.S0[n:n + 1], states=True)
        sub = inputs.Workload("verify", sl(w.q), sl(w.k), sl(w.v), sl(w.g), sl(w.beta),
                              w.S0[n:n + 1])
        check(sub, sl(O), S_tok[:, s:e], Or, Str, f"verify seq {n}")


def test_token_states_fp32_and_final_state_matches_prompt_form():
    w = inputs.prefill_workload(2, 70, 3, chunk=16, io_dtype=torch.float32, seed=3,
                                device=DEV)
    O, S_tok = run_states(w)
    Or, Sr, Str = oracle.prefill(w.q, w.k, w.v, w.g, w.beta, w.S0, states=True)
    check(w, O, S_tok, Or, Str, "fp32 states")
    _, S_T = gdn_chunk_prefill(w.q, w.k, w.v, w.g, w.beta, w.S0, None, 16)
    torch.cuda.synchronize()
    e = worst_slice_error(S_tok[:, -1], S_T.cpu())
    say(f"[fp32 states] last state vs prompt form: {e:.3e}")
    assert e <= TOL_F32


def test_token_states_bf16_long_sequences_and_prompt_form():
    # several chunks' worth of tokens, bf16; the last state also against the
    # prompt form's S_T
    w = inputs.prefill_workload(1, 300, 4, chunk=64, seed=4, device=DEV)
    O, S_tok = run_states(w)
    Or, Sr, Str = oracle.prefill(w.q, w.k, w.v, w.g, w.beta, w.S0, states=True)
    check(w, O, S_tok, Or, Str, "bf16 long states")
    _, S_T = gdn_chunk_prefill(w.q, w.k, w.v, w.g, w.beta, w.S0, None, 64)
    torch.cuda.synchronize()
    assert worst_slice_error(S_tok[:, -1], Sr) <= TOL_BF16
    assert worst_slice_error(S_T, Sr) <= TOL_BF16


def test_token_states_empty_sequences_and_zero_state():
    lens = [0, 5, 0, 17]
    w = inputs.varlen_workload(lens, H=2, s0=False, seed=5, device=DEV)
    O, S_tok = run_states(w)
    Or, _, Str = oracle.prefill(w.q, w.k, w.v, w.g, w.beta, None, cu_seqlens=w.cu_seqlens,
                                states=True)
    check(w, O, S_tok, Or, Str, "empty seqs")
    # no token rows at all
    z = inputs.prefill_workload(2, 0, 2, seed=6, device=DEV)
    O0, S0t = run_states(z)
    assert O0.numel() == 0 and S0t.numel() == 0


def test_token_states_launch_forms_agree_bit_for_bit():
    # The kernel loads a token's inputs two tokens ahead when a launch's
    # workgroups (two per sequence and head) fit on the CUs at once, four per
    # CU, and in the token's own iteration otherwise.  The same sequences run
    # both ways give the same states bit for bit, and outputs within one bf16
    # rounding of each other.
    H = 16
    n_small = 4 * torch.cuda.get_device_properties(0).multi_processor_count // (2 * H)
    big = inputs.verify_workload(n_small + 8, 16, H, seed=9, device=DEV)   # packed, B = 1
    n = n_small * 16
    small = inputs.Workload("verify_head", *(x[:, :n] for x in (big.q, big.k, big.v, big.g, big.beta)),
                            big.S0[:n_small], big.cu_seqlens[:n_small + 1], big.chunk, {})
    Ob, Sb = run_states(big)
    Os, Ss = run_states(small)
    assert torch.equal(Ss, Sb[:, :n])
    d = (Os.float() - Ob[:, :n].float()).abs()
    assert d.max().item() <= 2.0 ** -8 * Ob[:, :n].float().abs().max().item()
    say(f"[launch forms] {n} tokens: states equal, outputs differ in {(d > 0).sum().item()} elements")
