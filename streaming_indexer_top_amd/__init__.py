"""MI355X-native Compressed Sparse Attention lightning-indexer top-k.

``topk`` scores every causally usable compressed key for each query with the
lightning indexer and returns the query's top-k keys, through the C-ABI
library ``libcsa_indexer.so`` and its gfx950 HIP kernels.  ``sparse_attention``
is the CSA consumer of the selection: softmax attention of each query row
over its selected entries.  ``inputs`` holds the seeded synthetic input
generators.
"""
from .binding import (CsaError, abi_version, library_path, load_library,  # noqa: F401
                      profile_collect, profile_enable, sparse_attention, topk,
                      topk_noalloc, workspace_size)
