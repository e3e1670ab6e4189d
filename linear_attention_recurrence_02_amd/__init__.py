"""libgdn: gated delta-rule linear attention (Gated DeltaNet) on AMD MI355X.

The compute lives in ``libgdn.so``, a C-ABI library of hand-written HIP
kernels for gfx950 (sources in ``csrc/``, ABI in ``include/gdn.h``).  This
package is its thin Python binding: it marshals torch tensors into pointers,
sizes and the current HIP stream, and nothing else.  Importing the package
does not load the library; the first call does, and it raises if the library
has not been built.
"""
from . import inputs  # noqa: F401  (seeded workloads; no method arithmetic)

__all__ = ["gdn_chunk_prefill", "gdn_decode_step", "gdn_status_string",
           "gdn_version", "load_library", "inputs"]


def __getattr__(name):
    if name in ("gdn_chunk_prefill", "gdn_decode_step", "gdn_status_string",
                "gdn_version", "load_library", "GdnError"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
