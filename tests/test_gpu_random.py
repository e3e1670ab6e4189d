"""GPU parity on seeded random configurations of the prompt form, through the C
ABI, against the fp64 oracle: uniform and packed batches (with empty and
one-token sequences), 1 to 16 heads, chunk 16/32/64, bf16 and fp32 inputs, O
in the io dtype or (bf16) in fp32, with and without S0, in place or not, and
the launch's own, the whole or the split column form.  The configurations
reach every prompt-form kernel (vector, 16-token, 64-token whole and split).
The bar is the one of every other parity test."""
import random

import pytest
import torch

import oracle
from linear_attention_recurrence_02_amd import inputs
from linear_attention_recurrence_02_amd.binding import (GDN_COLUMNS_SPLIT, GDN_COLUMNS_WHOLE,
                                                        gdn_chunk_prefill)
from metrics import TOL_BF16, TOL_F32, bf16_output_ok, spans_of, worst_slice_error

pytestmark = pytest.mark.gpu
DEV = "cuda"


def config(i):
    rng = random.Random(1000 + i)
    c = dict(packed=rng.random() < 0.4, H=rng.choice([1, 2, 3, 5, 8, 16]),
             dt=rng.choice([torch.bfloat16, torch.bfloat16, torch.float32]),
             chunk=rng.choice([16, 32, 64, 64]),
             cols=rng.choice([None, GDN_COLUMNS_WHOLE, GDN_COLUMNS_SPLIT]),
             s0=rng.random() < 0.7)
    c["out32"] = c["dt"] == torch.bfloat16 and rng.random() < 0.3
    c["inplace"] = c["s0"] and rng.random() < 0.3
    if c["packed"]:
        c["lengths"] = [rng.choice([0, 1, 7, 16, 17, 63, 64, 65, 100, 200, 333])
                        for _ in range(rng.randint(1, 6))]
    else:
        c["B"], c["T"] = rng.randint(1, 4), rng.choice([1, 5, 16, 31, 64, 65, 129, 250])
    return c


@pytest.mark.parametrize("i", range(60))
def test_random_configuration(i):
    c = config(i)
    H, dt, chunk = c["H"], c["dt"], c["chunk"]
    if c["packed"]:
        w = inputs.varlen_workload(c["lengths"], H=H, chunk=chunk, io_dtype=dt, s0=c["s0"],
                                   seed=i, device=DEV)
    else:
        w = inputs.prefill_workload(c["B"], c["T"], H, chunk=chunk, io_dtype=dt, s0=c["s0"],
                                    seed=i, device=DEV)
    S = w.S0.clone() if c["inplace"] else None
    O, S_T = gdn_chunk_prefill(w.q, w.k, w.v, w.g, w.beta, S if c["inplace"] else w.S0,
                               w.cu_seqlens, chunk, S_T=S, columns=c["cols"],
                               out_dtype=torch.float32 if c["out32"] else None)
    torch.cuda.synchronize()
    Or, Sr = oracle.prefill(w.q, w.k, w.v, w.g, w.beta, w.S0, cu_seqlens=w.cu_seqlens)
    spans = spans_of(w.q.shape[0], w.q.shape[1], w.cu_seqlens)
    eo = worst_slice_error(O, Or, spans, H) if O.numel() else 0.0
    es = worst_slice_error(S_T, Sr)
    print(f"[{c}] O {eo:.2e} S_T {es:.2e}", flush=True)
    if dt == torch.float32:
        assert eo <= TOL_F32 and es <= TOL_F32, (eo, es)
    elif c["out32"]:
        assert eo <= TOL_BF16 and es <= TOL_BF16, (eo, es)
    else:
        if O.numel():
            ok, ratio = bf16_output_ok(O, Or, TOL_BF16, spans, H)
            assert ok, ratio
        assert es <= TOL_BF16, es
