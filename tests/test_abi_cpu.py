"""C-ABI checks that need no GPU: the library loads, exports every function
include/gdn.h declares, and rejects malformed calls with the documented status
before anything is enqueued (every call below fails validation, so no HIP call
is made)."""
import ctypes
import os
import re

import pytest

from linear_attention_recurrence_02_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

A = 0x10000          # fake, 16-byte aligned device addresses (never dereferenced)
MB = 1 << 20


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def test_header_declares_expected_calls():
    assert declared_functions() == sorted(binding.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.gdn_version() == 1
    for s in range(5):
        assert lib.gdn_status_string(s)
    assert b"unknown" in lib.gdn_status_string(99)


def prefill(lib, q=A, k=A + 64 * MB, v=A + 128 * MB, dtype=1, g=A + 192 * MB,
            beta=A + 200 * MB, S0=A + 256 * MB, cu=None, N=2, T=64, H=2, dk=128,
            dv=128, chunk=64, O=A + 512 * MB, S_T=A + 768 * MB):
    return lib.gdn_chunk_prefill(q, k, v, dtype, g, beta, S0, cu, N, T, H, dk, dv, chunk,
                                 O, S_T, None)


def decode(lib, q=A, k=A + MB, v=A + 2 * MB, dtype=1, g=A + 3 * MB, beta=A + 4 * MB,
           S=A + 8 * MB, B=4, H=2, dk=128, dv=128, o=A + 64 * MB):
    return lib.gdn_decode_step(q, k, v, dtype, g, beta, S, B, H, dk, dv, o, None)


def test_prefill_rejects_null_and_bad_sizes(lib):
    assert prefill(lib, q=None) == binding.GDN_ERR_INVALID_ARG
    assert prefill(lib, O=None) == binding.GDN_ERR_INVALID_ARG
    assert prefill(lib, S_T=None) == binding.GDN_ERR_INVALID_ARG
    assert prefill(lib, N=-1) == binding.GDN_ERR_INVALID_ARG
    assert prefill(lib, T=-5) == binding.GDN_ERR_INVALID_ARG
    assert prefill(lib, H=0) == binding.GDN_ERR_INVALID_ARG


def test_prefill_rejects_unsupported(lib):
    assert prefill(lib, dk=64) == binding.GDN_ERR_UNSUPPORTED
    assert prefill(lib, dv=256) == binding.GDN_ERR_UNSUPPORTED
    assert prefill(lib, chunk=48) == binding.GDN_ERR_UNSUPPORTED
    assert prefill(lib, chunk=128) == binding.GDN_ERR_UNSUPPORTED
    assert prefill(lib, dtype=7) == binding.GDN_ERR_UNSUPPORTED


def test_prefill_rejects_misaligned(lib):
    assert prefill(lib, q=A + 2) == binding.GDN_ERR_INVALID_ARG
    assert prefill(lib, S_T=A + 768 * MB + 4) == binding.GDN_ERR_INVALID_ARG
    assert prefill(lib, g=A + 192 * MB + 1) == binding.GDN_ERR_INVALID_ARG


def test_prefill_aliasing_rules(lib):
    assert prefill(lib, O=A) == binding.GDN_ERR_ALIAS                   # O over q
    assert prefill(lib, O=A + 256 * MB) == binding.GDN_ERR_ALIAS        # O over S0
    assert prefill(lib, S_T=A + 256 * MB + 4096) == binding.GDN_ERR_ALIAS  # partial S0
    assert prefill(lib, S_T=A + 64 * MB) == binding.GDN_ERR_ALIAS       # S_T over k
    # an empty batch is accepted without enqueueing anything
    assert prefill(lib, N=0) == binding.GDN_OK
    assert prefill(lib, N=0, S_T=A + 256 * MB) == binding.GDN_OK        # S_T == S0


def states(lib, q=A, k=A + 64 * MB, v=A + 128 * MB, dtype=1, g=A + 192 * MB,
           beta=A + 200 * MB, S0=A + 256 * MB, cu=None, N=2, T=64, H=2, dk=128,
           dv=128, O=A + 512 * MB, S_tok=A + 1024 * MB):
    return lib.gdn_prefill_states(q, k, v, dtype, g, beta, S0, cu, N, T, H, dk, dv, O,
                                  S_tok, None)


def test_prefill_states_validation(lib):
    assert states(lib, S_tok=None) == binding.GDN_ERR_INVALID_ARG
    assert states(lib, v=None) == binding.GDN_ERR_INVALID_ARG
    assert states(lib, H=0) == binding.GDN_ERR_INVALID_ARG
    assert states(lib, dk=64) == binding.GDN_ERR_UNSUPPORTED
    assert states(lib, dtype=5) == binding.GDN_ERR_UNSUPPORTED
    assert states(lib, S_tok=A + 1024 * MB + 8) == binding.GDN_ERR_INVALID_ARG
    # S_tok holds 2 x 64 token rows x 2 heads x 64 KiB = 16 MiB
    assert states(lib, S_tok=A + 256 * MB) == binding.GDN_ERR_ALIAS      # over S0
    assert states(lib, S_tok=A + 120 * MB) == binding.GDN_ERR_ALIAS      # over k, v
    assert states(lib, O=A + 1030 * MB) == binding.GDN_ERR_ALIAS         # O over S_tok
    assert states(lib, N=0) == binding.GDN_OK
    assert states(lib, N=0, S_tok=None, q=None, k=None, v=None, O=None) == binding.GDN_OK


def test_prefill_ex_validation(lib):
    def ex(inverse, columns=binding.GDN_COLUMNS_DEFAULT, **kw):
        args = dict(q=A, k=A + 64 * MB, v=A + 128 * MB, dtype=1, g=A + 192 * MB,
                    beta=A + 200 * MB, S0=A + 256 * MB, cu=None, N=2, T=64, H=2, dk=128,
                    dv=128, chunk=64, O=A + 512 * MB, S_T=A + 768 * MB)
        args.update(kw)
        a = args
        return lib.gdn_chunk_prefill_ex(a["q"], a["k"], a["v"], a["dtype"], a["g"], a["beta"],
                                        a["S0"], a["cu"], a["N"], a["T"], a["H"], a["dk"],
                                        a["dv"], a["chunk"], inverse, columns, a["O"], a["S_T"],
                                        None)
    assert ex(3) == binding.GDN_ERR_UNSUPPORTED
    assert ex(-1) == binding.GDN_ERR_UNSUPPORTED
    assert ex(binding.GDN_INVERSE_DEFAULT, 3) == binding.GDN_ERR_UNSUPPORTED
    assert ex(binding.GDN_INVERSE_DEFAULT, -1) == binding.GDN_ERR_UNSUPPORTED
    assert ex(binding.GDN_INVERSE_DOUBLING, q=None) == binding.GDN_ERR_INVALID_ARG
    assert ex(binding.GDN_INVERSE_SUBSTITUTION, O=A) == binding.GDN_ERR_ALIAS
    assert ex(binding.GDN_INVERSE_DEFAULT, binding.GDN_COLUMNS_SPLIT, O=A) == binding.GDN_ERR_ALIAS
    for inv in (binding.GDN_INVERSE_DEFAULT, binding.GDN_INVERSE_SUBSTITUTION,
                binding.GDN_INVERSE_DOUBLING):
        for col in (binding.GDN_COLUMNS_DEFAULT, binding.GDN_COLUMNS_WHOLE,
                    binding.GDN_COLUMNS_SPLIT):
            assert ex(inv, col, N=0) == binding.GDN_OK


def test_prefill_segmented_validation(lib):
    W = A + 2048 * MB
    ws = lib.gdn_chunk_prefill_segmented_workspace
    need = ws(1, None, 2, 1000, 2, 256)
    # 2 x 4 segments x 2 heads x 64 KiB three times, plus the segments' offsets
    # and each sequence's first segment (256-byte aligned parts)
    assert need == 3 * 16 * 65536 + 256 + 256
    assert ws(1, None, 2, 1000, 2, 0) == -1
    assert ws(7, None, 2, 1000, 2, 256) == -1
    # a packed batch of N sequences and T rows is sized for N + ceil(T / L) segments
    packed = ws(1, A, 3, 2000, 2, 256)
    assert packed == 3 * (3 + 8) * 2 * 65536 + 256 + 256
    # the rows (B * T, or T when packed) must fit the int32 segment offsets
    assert ws(1, None, 2, 1 << 30, 1, 1 << 20) == -1
    assert ws(1, None, 1, (1 << 30) - 1, 1, 1 << 20) > 0
    assert ws(1, A, 2, 1 << 31, 1, 1 << 20) == -1

    def seg(**kw):
        a = dict(q=A, k=A + 64 * MB, v=A + 128 * MB, dtype=1, g=A + 192 * MB, beta=A + 200 * MB,
                 S0=A + 256 * MB, cu=None, B=2, T=1000, H=2, chunk=64, L=256, ws=W, wsb=need,
                 O=A + 512 * MB, S_T=A + 768 * MB)
        a.update(kw)
        return lib.gdn_chunk_prefill_segmented(a["q"], a["k"], a["v"], a["dtype"], a["g"],
                                               a["beta"], a["S0"], a["cu"], a["B"], a["T"],
                                               a["H"], 128, 128, a["chunk"], a["L"], a["ws"],
                                               a["wsb"], a["O"], a["S_T"], None)
    assert seg(L=100) == binding.GDN_ERR_INVALID_ARG               # not a multiple of chunk
    assert seg(ws=None) == binding.GDN_ERR_INVALID_ARG
    assert seg(wsb=need - 1) == binding.GDN_ERR_INVALID_ARG
    assert seg(ws=W + 16) == binding.GDN_ERR_INVALID_ARG            # not 256-byte aligned
    assert seg(ws=A + 128 * MB + 4096) == binding.GDN_ERR_ALIAS    # workspace over v
    assert seg(q=None) == binding.GDN_ERR_INVALID_ARG
    assert seg(B=0) == binding.GDN_OK
    # packed: the workspace must hold the packed bound and must not cover the offsets
    cu = A + 1500 * MB
    assert seg(cu=cu, B=3, T=2000, wsb=packed - 1) == binding.GDN_ERR_INVALID_ARG
    assert seg(cu=cu, B=3, T=2000, wsb=packed, ws=cu - 256) == binding.GDN_ERR_ALIAS


def test_prefill_segmented_noalloc_validation(lib):
    """The no-allocation segmented form checks its arguments like the workspace
    form and refuses, before any device work, a call whose workspace would not
    fit its scratch."""
    scratch = lib.gdn_noalloc_scratch_bytes()
    assert scratch == 48 * MB + 64 * 1024

    def seg(**kw):
        a = dict(q=A, k=A + 64 * MB, v=A + 128 * MB, dtype=1, g=A + 192 * MB, beta=A + 200 * MB,
                 S0=A + 256 * MB, cu=None, B=2, T=1000, H=2, chunk=64, L=256,
                 O=A + 512 * MB, S_T=A + 768 * MB)
        a.update(kw)
        return lib.gdn_chunk_prefill_segmented_noalloc(
            a["q"], a["k"], a["v"], a["dtype"], a["g"], a["beta"], a["S0"], a["cu"], a["B"],
            a["T"], a["H"], 128, 128, a["chunk"], a["L"], a["O"], a["S_T"], None)
    assert seg(L=100) == binding.GDN_ERR_INVALID_ARG               # not a multiple of chunk
    assert seg(q=None) == binding.GDN_ERR_INVALID_ARG
    assert seg(chunk=48) == binding.GDN_ERR_UNSUPPORTED
    assert seg(B=0) == binding.GDN_OK
    # 16 heads of 4096 tokens in 256-token segments fit (256 segment-heads) ...
    fits = lib.gdn_chunk_prefill_segmented_workspace(1, None, 1, 4096, 16, 256)
    assert 0 < fits <= scratch
    # ... 32 heads do not: refused with its own status, nothing enqueued
    assert lib.gdn_chunk_prefill_segmented_workspace(1, None, 1, 4096, 32, 256) > scratch
    assert seg(B=1, T=4096, H=32) == binding.GDN_ERR_SCRATCH
    assert b"scratch" in lib.gdn_status_string(binding.GDN_ERR_SCRATCH)


def gated(lib, q=A, k=A + 64 * MB, v=A + 128 * MB, dtype=1, g=A + 192 * MB,
          beta=A + 200 * MB, S0=A + 256 * MB, cu=None, N=2, T=64, H=2, dk=128,
          dv=128, chunk=64, z=A + 1024 * MB, w=A + 1100 * MB, eps=1e-6, Y=A + 512 * MB,
          S_T=A + 768 * MB):
    return lib.gdn_chunk_prefill_gated(q, k, v, dtype, g, beta, S0, cu, N, T, H, dk, dv,
                                       chunk, z, w, eps, Y, S_T, None)


def test_prefill_gated_validation(lib):
    # the prompt form's own rules still hold
    assert gated(lib, q=None) == binding.GDN_ERR_INVALID_ARG
    assert gated(lib, chunk=48) == binding.GDN_ERR_UNSUPPORTED
    assert gated(lib, Y=A) == binding.GDN_ERR_ALIAS                     # Y over q
    # the gate, the weights and eps
    assert gated(lib, z=None) == binding.GDN_ERR_INVALID_ARG
    assert gated(lib, w=None) == binding.GDN_ERR_INVALID_ARG
    assert gated(lib, z=A + 1024 * MB + 8) == binding.GDN_ERR_INVALID_ARG
    assert gated(lib, w=A + 1100 * MB + 2) == binding.GDN_ERR_INVALID_ARG
    assert gated(lib, eps=-1e-6) == binding.GDN_ERR_INVALID_ARG
    assert gated(lib, eps=float("nan")) == binding.GDN_ERR_INVALID_ARG
    assert gated(lib, eps=float("inf")) == binding.GDN_ERR_INVALID_ARG
    # Y holds 2 x 64 rows x 2 heads x 256 B = 64 KiB
    assert gated(lib, z=A + 512 * MB + 1024) == binding.GDN_ERR_ALIAS    # z under Y
    assert gated(lib, w=A + 512 * MB + 64) == binding.GDN_ERR_ALIAS     # w under Y
    assert gated(lib, w=A + 768 * MB + 64) == binding.GDN_ERR_ALIAS     # w under S_T
    assert gated(lib, N=0) == binding.GDN_OK
    assert gated(lib, T=0, z=None, q=None, k=None, v=None, g=None, beta=None,
                 Y=None, N=0) == binding.GDN_OK


def preop(lib, xq=A, xk=A + 8 * MB, xv=A + 16 * MB, dtype=1, a=A + 24 * MB, b=A + 25 * MB,
          w=A + 26 * MB, si=A + 27 * MB, so=A + 27 * MB, cu=None, N=2, T=64, H=2, dk=128,
          dv=128, K=4, eps=1e-6, q=A + 32 * MB, k=A + 40 * MB, v=A + 48 * MB, g=A + 56 * MB,
          beta=A + 57 * MB):
    return lib.gdn_preop(xq, xk, xv, dtype, a, b, w, si, so, cu, N, T, H, dk, dv, K, eps, q, k,
                         v, g, beta, None)


def test_preop_validation(lib):
    assert preop(lib, xq=None) == binding.GDN_ERR_INVALID_ARG
    assert preop(lib, w=None) == binding.GDN_ERR_INVALID_ARG
    assert preop(lib, si=None) == binding.GDN_ERR_INVALID_ARG
    assert preop(lib, K=3) == binding.GDN_ERR_UNSUPPORTED
    assert preop(lib, dk=64) == binding.GDN_ERR_UNSUPPORTED
    assert preop(lib, dtype=9) == binding.GDN_ERR_UNSUPPORTED
    assert preop(lib, eps=-1.0) == binding.GDN_ERR_INVALID_ARG
    assert preop(lib, xk=A + 8 * MB + 8) == binding.GDN_ERR_INVALID_ARG
    assert preop(lib, w=A + 26 * MB + 4) == binding.GDN_ERR_INVALID_ARG
    # 2 x 64 rows x 2 heads x 256 B = 64 KiB per token tensor
    assert preop(lib, q=A + 1024) == binding.GDN_ERR_ALIAS              # q over xq
    assert preop(lib, k=A + 32 * MB + 4096) == binding.GDN_ERR_ALIAS    # k over q
    assert preop(lib, g=A + 24 * MB) == binding.GDN_ERR_ALIAS           # g over a
    assert preop(lib, so=A + 27 * MB + 256) == binding.GDN_ERR_ALIAS    # partial state overlap
    assert preop(lib, q=A + 27 * MB) == binding.GDN_ERR_ALIAS           # q over state_in
    assert preop(lib, N=0) == binding.GDN_OK
    assert preop(lib, N=0, xq=None, xk=None, xv=None, a=None, b=None, w=None, si=None,
                 so=None, q=None, k=None, v=None, g=None, beta=None) == binding.GDN_OK


def test_prefill_preop_validation(lib):
    def pp(**kw):
        a = dict(xq=A, xk=A + 8 * MB, xv=A + 16 * MB, dtype=1, a=A + 24 * MB, b=A + 25 * MB,
                 w=A + 26 * MB, si=A + 27 * MB, so=A + 27 * MB, eps=1e-6, S0=A + 28 * MB,
                 cu=None, N=2, T=64, H=2, dk=128, dv=128, K=4, chunk=64, O=A + 32 * MB,
                 S_T=A + 40 * MB)
        a.update(kw)
        return lib.gdn_chunk_prefill_preop(a["xq"], a["xk"], a["xv"], a["dtype"], a["a"],
                                           a["b"], a["w"], a["si"], a["so"], a["eps"], a["S0"],
                                           a["cu"], a["N"], a["T"], a["H"], a["dk"], a["dv"],
                                           a["K"], a["chunk"], a["O"], a["S_T"], None)
    assert pp(xq=None) == binding.GDN_ERR_INVALID_ARG
    assert pp(w=None) == binding.GDN_ERR_INVALID_ARG
    assert pp(si=None) == binding.GDN_ERR_INVALID_ARG
    assert pp(S_T=None) == binding.GDN_ERR_INVALID_ARG
    assert pp(dtype=0) == binding.GDN_ERR_UNSUPPORTED                   # fp32: bf16 only
    assert pp(dtype=2) == binding.GDN_ERR_UNSUPPORTED                   # no fp32 O here
    assert pp(chunk=32) == binding.GDN_ERR_UNSUPPORTED
    assert pp(K=3) == binding.GDN_ERR_UNSUPPORTED
    assert pp(dk=64) == binding.GDN_ERR_UNSUPPORTED
    assert pp(eps=-1.0) == binding.GDN_ERR_INVALID_ARG
    assert pp(eps=float("nan")) == binding.GDN_ERR_INVALID_ARG
    assert pp(w=A + 26 * MB + 4) == binding.GDN_ERR_INVALID_ARG         # misaligned
    assert pp(si=A + 27 * MB + 8, so=A + 27 * MB + 8) == binding.GDN_ERR_INVALID_ARG
    # 2 x 64 rows x 2 heads x 256 B = 64 KiB per token tensor
    assert pp(O=A + 4096) == binding.GDN_ERR_ALIAS                      # O over xq
    assert pp(O=A + 26 * MB) == binding.GDN_ERR_ALIAS                   # O over conv_w
    assert pp(S_T=A + 27 * MB) == binding.GDN_ERR_ALIAS                 # S_T over the FIFO
    assert pp(so=A + 27 * MB + 256) == binding.GDN_ERR_ALIAS            # FIFO partly in place
    assert pp(so=A + 24 * MB) == binding.GDN_ERR_ALIAS                  # new FIFO over a
    assert pp(so=A + 40 * MB) == binding.GDN_ERR_ALIAS                  # new FIFO over S_T
    assert pp(N=0) == binding.GDN_OK
    assert pp(N=0, so=A + 29 * MB) == binding.GDN_OK                    # out of place
    assert pp(N=0, T=0, xq=None, xk=None, xv=None, a=None, b=None, w=None, si=None,
              so=None, O=None) == binding.GDN_OK


def test_decode_rejects_bad_calls(lib):
    assert decode(lib, S=None) == binding.GDN_ERR_INVALID_ARG
    assert decode(lib, B=-1) == binding.GDN_ERR_INVALID_ARG
    assert decode(lib, dk=64) == binding.GDN_ERR_UNSUPPORTED
    assert decode(lib, dtype=3) == binding.GDN_ERR_UNSUPPORTED
    assert decode(lib, S=A + 8 * MB + 8) == binding.GDN_ERR_INVALID_ARG
    assert decode(lib, o=A + 8 * MB) == binding.GDN_ERR_ALIAS            # o over S
    assert decode(lib, S=A) == binding.GDN_ERR_ALIAS                     # S over q
    assert decode(lib, B=0) == binding.GDN_OK


def test_decode_ex_validation(lib):
    def ex(hint, **kw):
        a = dict(q=A, k=A + MB, v=A + 2 * MB, dtype=1, g=A + 3 * MB, beta=A + 4 * MB,
                 S=A + 8 * MB, B=4, H=2, dk=128, dv=128, o=A + 64 * MB)
        a.update(kw)
        return lib.gdn_decode_step_ex(a["q"], a["k"], a["v"], a["dtype"], a["g"], a["beta"],
                                      a["S"], a["B"], a["H"], a["dk"], a["dv"], hint, a["o"],
                                      None)
    # an unknown hint is refused before any other check or launch
    assert ex(2) == binding.GDN_ERR_UNSUPPORTED
    assert ex(-1) == binding.GDN_ERR_UNSUPPORTED
    # the rest validates exactly as gdn_decode_step
    for hint in (binding.GDN_STATE_CACHED, binding.GDN_STATE_STREAMING):
        assert ex(hint, S=None) == binding.GDN_ERR_INVALID_ARG
        assert ex(hint, dk=64) == binding.GDN_ERR_UNSUPPORTED
        assert ex(hint, o=A + 8 * MB) == binding.GDN_ERR_ALIAS
        assert ex(hint, B=0) == binding.GDN_OK


def test_decode_preop_validation(lib):
    def dp(**kw):
        a = dict(xq=A, xk=A + MB, xv=A + 2 * MB, dtype=1, a=A + 3 * MB, b=A + 4 * MB,
                 w=A + 5 * MB, si=A + 6 * MB, so=A + 6 * MB, eps=1e-6, z=None, nw=None,
                 neps=1e-6, S=A + 16 * MB, B=4, H=2, dk=128, dv=128, hint=0, o=A + 64 * MB)
        a.update(kw)
        return lib.gdn_decode_step_preop(a["xq"], a["xk"], a["xv"], a["dtype"], a["a"], a["b"],
                                         a["w"], a["si"], a["so"], a["eps"], a["z"], a["nw"],
                                         a["neps"], a["S"], a["B"], a["H"], a["dk"], a["dv"],
                                         a["hint"], a["o"], None)
    assert dp(hint=2) == binding.GDN_ERR_UNSUPPORTED
    assert dp(dtype=3) == binding.GDN_ERR_UNSUPPORTED
    assert dp(dk=64) == binding.GDN_ERR_UNSUPPORTED
    assert dp(w=None) == binding.GDN_ERR_INVALID_ARG
    assert dp(si=None) == binding.GDN_ERR_INVALID_ARG
    assert dp(eps=-1.0) == binding.GDN_ERR_INVALID_ARG
    assert dp(eps=float("inf")) == binding.GDN_ERR_INVALID_ARG
    assert dp(xq=A + 8) == binding.GDN_ERR_INVALID_ARG                  # misaligned
    assert dp(o=A + 16 * MB) == binding.GDN_ERR_ALIAS                   # o over S
    assert dp(S=A) == binding.GDN_ERR_ALIAS                             # S over xq
    assert dp(so=A + 6 * MB + 256) == binding.GDN_ERR_ALIAS             # FIFO partly in place
    assert dp(so=A + 3 * MB) == binding.GDN_ERR_ALIAS                   # new FIFO over a
    assert dp(B=0) == binding.GDN_OK
    assert dp(so=A + 8 * MB, B=0) == binding.GDN_OK                     # out of place
    # the gated norm: z needs norm_w and a finite eps >= 0; outputs apart from z
    assert dp(z=A + 7 * MB) == binding.GDN_ERR_INVALID_ARG              # no norm_w
    assert dp(z=A + 7 * MB, nw=A + 7 * MB + 65536, neps=-1.0) == binding.GDN_ERR_INVALID_ARG
    assert dp(z=A + 7 * MB + 8, nw=A + 7 * MB + 65536) == binding.GDN_ERR_INVALID_ARG
    assert dp(z=A + 64 * MB, nw=A + 7 * MB) == binding.GDN_ERR_ALIAS    # o over z
    assert dp(z=A + 7 * MB, nw=A + 7 * MB + 65536, B=0) == binding.GDN_OK


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(1, 4, 1, 128)
    g = torch.zeros(1, 4, 1)
    with pytest.raises(ValueError):
        binding.gdn_chunk_prefill(x, x, x, g, g)


def test_package_import_does_not_load_library():
    import subprocess
    import sys
    code = ("import sys, linear_attention_recurrence_02_amd as m; "
            "assert 'linear_attention_recurrence_02_amd.binding' not in sys.modules")
    subprocess.run([sys.executable, "-c", code], check=True, cwd=ROOT)
