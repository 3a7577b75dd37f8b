"""Domino head drafting loop for MI355X (gfx950).

The compute lives in ``libdomino_head.so`` (hand-written HIP kernels behind a C
ABI declared in include/domino_head.h); this package is its Python binding.
"""
from .binding import (  # noqa: F401
    DOMINO_BF16, DOMINO_F32, EXEC_AUTO, EXEC_PERSISTENT, EXEC_STEPWISE, EXEC_STREAM_W2, EXEC_PLAIN_LAUNCH, EXEC_POSITION_BATCHED, LBASE_BF16, MARKOV, FOLD_EMBED, FLAG_BAD_TOKEN, FLAG_SYNC_TIMEOUT,
    LIB_PATH, SYMBOLS, DominoError, DominoHead, accept_len, load_library, verify, verify_noalloc,
    verify_workspace_size,
)
from .tensors import device_tensor, head_weights_to_device  # noqa: F401
