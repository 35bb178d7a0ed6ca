"""CPU oracle for paged-KV attention with prefix reuse (test infrastructure only;
the product path never imports it)."""
from .pkv_oracle import *  # noqa: F401,F403
from .prefix_index import ChainHashPrefixCache, OutOfBlocks, RadixTree  # noqa: F401
