"""GPU parity of gdn_chunk_prefill_segmented (the prompt form with each
sequence cut into segments walked in parallel, joined by a scan of the
segments' affine state maps) against the fp64 oracle, through the C ABI.

Same bar as the prompt form: per-slice normwise error <= 2e-3 for bf16 inputs
(with the bf16 output's own rounding allowed elementwise) and <= 1e-5 for fp32
inputs.
"""
import pytest
import torch

import oracle
from linear_attention_recurrence_02_amd import inputs
from linear_attention_recurrence_02_amd.binding import (gdn_chunk_prefill,
                                                        gdn_chunk_prefill_segmented)
from metrics import TOL_BF16, TOL_F32, bf16_output_ok, spans_of, worst_slice_error

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def check(w, O, S_T, label, S0=None):
    Or, Sr = oracle.prefill(w.q, w.k, w.v, w.g, w.beta, w.S0 if S0 is None else S0,
                            w.cu_seqlens)
    spans = spans_of(w.q.shape[0], w.q.shape[1], w.cu_seqlens)
    H = w.q.shape[2]
    eo, es = worst_slice_error(O, Or, spans, H), worst_slice_error(S_T, Sr)
    say(f"[{label}] worst slice error O={eo:.3e} S_T={es:.3e}")
    if w.q.dtype == torch.float32:
        assert eo <= TOL_F32 and es <= TOL_F32, (eo, es)
    else:
        ok, ratio = bf16_output_ok(O, Or, TOL_BF16, spans, H)
        assert ok, ratio
        assert es <= TOL_BF16, es


@pytest.mark.parametrize("L", [256, 512])
def test_long_workload_segmented(L):
    # 1 x 4096 tokens x 16 heads in 16 segments of 256 tokens (256 segment-heads,
    # one workgroup each) or 8 of 512 (128 segment-heads, whose prompt-kernel
    # runs split each unit's value columns over two workgroups)
    w = inputs.long_prefill(device=DEV)
    O, S_T = gdn_chunk_prefill_segmented(w.q, w.k, w.v, w.g, w.beta, w.S0, 64, L)
    torch.cuda.synchronize()
    check(w, O, S_T, f"long, segments of {L}")


@pytest.mark.parametrize("T,L", [(1000, 64), (1000, 256), (1000, 384), (1000, 512), (2100, 64)])
def test_slow_decay_carries_state_across_segments(T, L):
    # decay slow enough that the state entering each segment matters; the last
    # segment is partial.  Segment counts 16, 4, 3, 2 and 33: the scan's
    # step count P - 1 both odd and even
    w = inputs.prefill_workload(2, T, 2, chunk=64, seed=81, device=DEV)
    w.g.mul_(0.02)
    O, S_T = gdn_chunk_prefill_segmented(w.q, w.k, w.v, w.g, w.beta, w.S0, 64, L)
    torch.cuda.synchronize()
    check(w, O, S_T, f"slow decay, T={T}, segments of {L}")


def test_fp32_vector_kernel_segments():
    w = inputs.prefill_workload(2, 300, 3, chunk=16, io_dtype=torch.float32, seed=82, device=DEV)
    O, S_T = gdn_chunk_prefill_segmented(w.q, w.k, w.v, w.g, w.beta, w.S0, 16, 64)
    torch.cuda.synchronize()
    check(w, O, S_T, "fp32, segments of 64")


def test_zero_state_and_in_place_state():
    w = inputs.prefill_workload(1, 700, 2, chunk=64, s0=False, seed=83, device=DEV)
    O, S_T = gdn_chunk_prefill_segmented(w.q, w.k, w.v, w.g, w.beta, None, 64, 128)
    torch.cuda.synchronize()
    check(w, O, S_T, "zero S0")
    w = inputs.prefill_workload(1, 700, 2, chunk=64, seed=84, device=DEV)
    S = w.S0.clone()
    O, S_T = gdn_chunk_prefill_segmented(w.q, w.k, w.v, w.g, w.beta, S, 64, 128, S_T=S)
    torch.cuda.synchronize()
    assert S_T.data_ptr() == S.data_ptr()
    check(w, O, S_T, "in place", S0=w.S0)


def test_one_segment_is_the_plain_form():
    w = inputs.prefill_workload(2, 200, 2, chunk=64, seed=85, device=DEV)
    O1, S1 = gdn_chunk_prefill_segmented(w.q, w.k, w.v, w.g, w.beta, w.S0, 64, 256)
    O2, S2 = gdn_chunk_prefill(w.q, w.k, w.v, w.g, w.beta, w.S0, None, 64)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(S1, S2)


# packed batches: empty sequences, sequences shorter than a segment, partial last
# segments and sequences of several segments side by side
PACKED = [1000, 0, 37, 300, 129, 64]


@pytest.mark.parametrize("L", [64, 128, 256])
def test_packed_batch_segmented(L):
    w = inputs.varlen_workload(PACKED, H=3, seed=86, device=DEV)
    w.g.mul_(0.05)      # slow decay, so that the entering states matter
    O, S_T = gdn_chunk_prefill_segmented(w.q, w.k, w.v, w.g, w.beta, w.S0, 64, L,
                                         cu_seqlens=w.cu_seqlens)
    torch.cuda.synchronize()
    check(w, O, S_T, f"packed {PACKED}, segments of {L}")


def test_packed_zero_and_in_place_state():
    w = inputs.varlen_workload(PACKED, H=2, s0=False, seed=87, device=DEV)
    O, S_T = gdn_chunk_prefill_segmented(w.q, w.k, w.v, w.g, w.beta, None, 64, 128,
                                         cu_seqlens=w.cu_seqlens)
    torch.cuda.synchronize()
    check(w, O, S_T, "packed, zero S0")
    w = inputs.varlen_workload(PACKED, H=2, seed=88, device=DEV)
    S = w.S0.clone()
    O, S_T = gdn_chunk_prefill_segmented(w.q, w.k, w.v, w.g, w.beta, S, 64, 128,
                                         cu_seqlens=w.cu_seqlens, S_T=S)
    torch.cuda.synchronize()
    assert S_T.data_ptr() == S.data_ptr()
    check(w, O, S_T, "packed, in place", S0=w.S0)


def test_packed_fp32_vector_kernel():
    w = inputs.varlen_workload([90, 0, 33, 5], H=2, chunk=16, io_dtype=torch.float32,
                               seed=89, device=DEV)
    O, S_T = gdn_chunk_prefill_segmented(w.q, w.k, w.v, w.g, w.beta, w.S0, 16, 32,
                                         cu_seqlens=w.cu_seqlens)
    torch.cuda.synchronize()
    check(w, O, S_T, "packed fp32, segments of 32")


def test_packed_long_sequence_among_short_ones():
    # one 4096-token sequence with 15 short ones: the serving case the packed
    # form is for
    w = inputs.varlen_workload([4096] + [16] * 15, H=4, seed=90, device=DEV)
    O, S_T = gdn_chunk_prefill_segmented(w.q, w.k, w.v, w.g, w.beta, w.S0, 64, 256,
                                         cu_seqlens=w.cu_seqlens)
    torch.cuda.synchronize()
    check(w, O, S_T, "one long among short, segments of 256")
