"""MI355X-native KIVI-style quantized KV cache with decode attention over the codes.

The compute path is the HIP library libkvq.so (include/kvq.h); this package is its thin
Python binding. Importing it without the built library raises ImportError.
"""
from .cache import (  # noqa: F401
    KVQCache,
    KVQError,
    kvq_append,
    kvq_append_decode_attend,
    kvq_cache_bytes,
    kvq_decode_attend,
    kvq_decode_attend_multi,
    kvq_decode_attend_noalloc,
    kvq_encode,
    kvq_encode_block,
    kvq_layout,
    kvq_prefill,
    kvq_probe,
    kvq_workspace_bytes,
    make_config,
)
from ._lib import LIB_PATH  # noqa: F401
