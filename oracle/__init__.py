"""CPU oracle for the CSA lightning-indexer top-k (test infrastructure only)."""
from .oracle import build, compile_source, n_valid, open_library, row_scores, topk  # noqa: F401
