"""gdn_chunk_prefill_segmented_noalloc (the segmented prompt form on the
library's own per-GPU scratch, for callers that cannot allocate) against the
workspace form gdn_chunk_prefill_segmented, through the C ABI: two calls in a
row on the same scratch, the second with a smaller input.  Both forms run the
same kernels in the same order, so their outputs must be equal bit for bit;
each is also held to the usual bar against the fp64 oracle."""
import pytest
import torch

import oracle
from linear_attention_recurrence_02_amd import inputs
from linear_attention_recurrence_02_amd.binding import (GDN_ERR_SCRATCH, GdnError,
                                                        gdn_chunk_prefill_segmented,
                                                        gdn_chunk_prefill_segmented_noalloc)
from metrics import TOL_BF16, bf16_output_ok, spans_of, worst_slice_error

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def both_forms(w, L):
    On, Sn = gdn_chunk_prefill_segmented_noalloc(w.q, w.k, w.v, w.g, w.beta, w.S0, w.chunk, L,
                                                 cu_seqlens=w.cu_seqlens)
    torch.cuda.synchronize()
    Ow, Sw = gdn_chunk_prefill_segmented(w.q, w.k, w.v, w.g, w.beta, w.S0, w.chunk, L,
                                         cu_seqlens=w.cu_seqlens)
    torch.cuda.synchronize()
    return On, Sn, Ow, Sw


def check_oracle(w, O, S_T, label):
    Or, Sr = oracle.prefill(w.q, w.k, w.v, w.g, w.beta, w.S0, cu_seqlens=w.cu_seqlens)
    spans = spans_of(w.q.shape[0], w.q.shape[1], w.cu_seqlens)
    H = w.q.shape[2]
    ok, ratio = bf16_output_ok(O, Or, TOL_BF16, spans, H)
    es = worst_slice_error(S_T, Sr)
    say(f"[{label}] O bound ratio {ratio:.3f}, S_T {es:.3e}")
    assert ok and es <= TOL_BF16, (ratio, es)


def test_noalloc_equals_workspace_form_on_two_calls():
    # 1 x 4096 tokens x 16 heads in 256-token segments: 256 segment-heads, the
    # most the scratch holds at this shape
    w1 = inputs.long_prefill(device=DEV)
    say("noalloc call 1: long workload, segment_len 256")
    On, Sn, Ow, Sw = both_forms(w1, 256)
    assert torch.equal(On, Ow) and torch.equal(Sn, Sw)
    check_oracle(w1, On, Sn, "noalloc long")
    # a smaller packed batch on the same scratch, whose earlier contents must
    # not leak into the result
    w2 = inputs.varlen_workload([700, 130, 0, 33], H=4, seed=3, device=DEV)
    say("noalloc call 2: packed 700/130/0/33 tokens x 4 heads, segment_len 128")
    On, Sn, Ow, Sw = both_forms(w2, 128)
    assert torch.equal(On, Ow) and torch.equal(Sn, Sw)
    check_oracle(w2, On, Sn, "noalloc packed")


def test_noalloc_refuses_calls_beyond_its_scratch():
    w = inputs.prefill_workload(1, 4096, 32, seed=4, device=DEV)
    O = torch.full_like(w.v, 7.0)
    with pytest.raises(GdnError) as e:
        gdn_chunk_prefill_segmented_noalloc(w.q, w.k, w.v, w.g, w.beta, w.S0, 64, 256, O=O)
    assert e.value.status == GDN_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((O == 7.0).all()), "a refused call must enqueue nothing"
