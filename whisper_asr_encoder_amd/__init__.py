"""MI355X-native Whisper-large-v3 encoder and block-verification attention.

The compute path is the HIP library ``libedda.so`` (kernels in ``csrc/``); the
binding in ``_lib`` only marshals tensors and streams into its C ABI. Importing
this package loads nothing: ``whisper_asr_encoder_amd.lib()`` loads the library
and raises if it was not built.
"""


def lib():
    from . import _lib
    return _lib.load()
