"""MI355X-native Compressed Sparse Attention lightning-indexer top-k."""
