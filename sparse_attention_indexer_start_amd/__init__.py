"""MI355X-native DSA decode-time candidate selection.

The compute path is the HIP library ``libdsa_select.so`` (built from
``csrc/``); :mod:`.binding` marshals arguments to its C ABI.  The library is
loaded on first use and a missing library raises: there is no fallback.
"""
from . import workloads  # noqa: F401

__all__ = ["workloads"]
