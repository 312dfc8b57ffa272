"""MI355X-native routed low-bit MoE expert layer (libmoeq + Python binding).

The compute path is the HIP library ``libmoeq.so`` (C ABI in
``include/moeq.h``); the ``moeq`` submodule only marshals torch tensors into
it.  Importing works without the library; the first call that needs it
raises if it has not been built (``python -m bit_quantized_moe_token_amd.build``).
"""

from ._lib import MoeqError, lib  # noqa: F401

__all__ = ["MoeqError", "lib"]
