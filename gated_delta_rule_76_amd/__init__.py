"""MI355X-native Kimi Delta Attention (KDA) layer: chunked prefill, decode step
and varlen packing in hand-written HIP for gfx950, behind a C ABI
(``include/kda.h``).  The Python side only marshals arguments; importing the
package does not load the library -- the first call does, and fails loudly if
it has not been built.
"""

__all__ = ["prefill", "decode_step", "prefill_workspace_size", "PrefillCall", "KdaError"]


def __getattr__(name):
    if name in __all__:
        from . import kda as _kda
        return getattr(_kda, name)
    raise AttributeError(name)
