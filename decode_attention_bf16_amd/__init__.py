"""MI355X (gfx950) decode attention over a bf16 KV cache: MLA absorbed latent form
and GQA/MQA/MHA grouped form, as hand-written HIP kernels behind a C ABI.

Importing the package is cheap; the shared library is loaded on the first call
of ``mla_decode`` / ``gqa_decode`` and fails loudly if it is missing.
"""
from . import costmodel  # noqa: F401

__all__ = ["costmodel", "mla_decode", "gqa_decode", "mla_decode_workspace_size",
           "gqa_decode_workspace_size", "library_path"]


def __getattr__(name):
    if name in ("mla_decode", "gqa_decode", "mla_decode_workspace_size",
                "gqa_decode_workspace_size", "library_path", "load_library", "DecodeAttentionError"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
