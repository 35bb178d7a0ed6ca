"""Plain Python model of the host-side prefix index that feeds the hot path.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: the product path never
imports it. Two matchers from the pages, written for readability:

* ChainHashPrefixCache - page A §05: every full KV block is identified by its
  parent block's identity, its own token IDs and optional extra keys (a LoRA
  id, a multimodal input hash); identical token prefixes give the identical
  chain, and a new request reuses blocks up to the first miss and allocates
  new blocks from there. Page A §06: a per-tenant salt is part of the cache
  identifier, so equal prompts of different tenants never share blocks.
  Page A §02 and page B "PagedAttention": blocks are allocated only when
  tokens need them, and blocks no longer used go back to a pool that other
  requests draw from.
* RadixTree - page A §03: the token paths of finished requests are kept in a
  radix tree that stores a common prefix once; a new request finds its longest
  matching path and computes only the rest; page A §04: new KV is inserted
  after a request, and under memory pressure leaves are removed first,
  least recently used first, so shared interior prefixes stay; page B
  "RadixAttention": the tree of one shared system prompt with per-user
  branches, managed by LRU.

Where the pages leave a step open, the plainest reading is taken (each is
listed with its reason in the design notes of this repository):

* identities are exact: this model keys blocks by the full nested tuple
  (parent identity, token IDs, extra); a hash of it only names it;
* only full blocks are published and matched (a partly filled block belongs
  to its request);
* when every token of a request is cached, the last block is still computed,
  so that at least one token goes through the model;
* blocks are taken from a FIFO free list first, then by evicting the least
  recently released cached block; a request releases its blocks tail first,
  so a chain loses its last blocks before its first ones;
* the radix tree matches in units of ``page`` tokens (1 for the pages'
  token-level examples, the block size for a paged cache).

Parity status (tests/test_prefix_index_pins.py): pinned on the pages' worked
examples (the "firm" insertion, the today/tomorrow requests, the 2,000-token
request with 1,900 cached, the 1,000-request chatbot with one system prompt),
on brute-force longest-prefix matching over the live sequences, and on
invariants (reference counts, conservation of blocks, salt isolation).
"""
from __future__ import annotations

from collections import OrderedDict, deque
from typing import Dict, List, Optional, Sequence, Tuple

__all__ = ["OutOfBlocks", "ChainHashPrefixCache", "RadixTree"]


class OutOfBlocks(RuntimeError):
    """Not enough free or evictable blocks for a request."""


# --------------------------------------------------------------------------
# chain-hash prefix cache over a paged block pool (page A §02, §05, §06)
# --------------------------------------------------------------------------
class ChainHashPrefixCache:
    """Block-granular prefix cache: identity of block i of a request =
    (identity of block i-1, token IDs of block i, extra), with the first
    block's parent being the tenant's salt."""

    def __init__(self, num_blocks: int, block_size: int):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.B = block_size
        self.num_blocks = num_blocks
        self.free: deque = deque(range(num_blocks))       # FIFO free list
        self.ref = [0] * num_blocks                       # requests using each block
        self.cached: Dict[tuple, int] = {}                # published identity -> block
        self.ident: Dict[int, tuple] = {}                 # block -> published identity
        self.evictable: "OrderedDict[int, None]" = OrderedDict()  # ref 0 and published, LRU first
        self.requests: Dict[int, dict] = {}
        self._next_rid = 0

    # identity of every full block of a token list (page A §05 chaining)
    def _chain(self, tokens: Sequence[int], salt: int, extra) -> List[tuple]:
        out, parent = [], ("salt", salt)
        for i in range(len(tokens) // self.B):
            parent = (parent, tuple(tokens[i * self.B:(i + 1) * self.B]), extra)
            out.append(parent)
        return out

    def _take(self) -> int:
        if self.free:
            return self.free.popleft()
        blk, _ = self.evictable.popitem(last=False)  # least recently released
        del self.cached[self.ident.pop(blk)]
        return blk

    def admit(self, tokens: Sequence[int], salt: int = 0, extra=None
              ) -> Tuple[int, List[int], int, List[int]]:
        """A new request: returns (request id, block table, prefix length,
        slot of every token from the prefix length on)."""
        tokens = [int(t) for t in tokens]
        n = len(tokens)
        if n == 0:
            raise ValueError("a request has at least one token")
        chain = self._chain(tokens, salt, extra)
        hits = 0
        while hits < len(chain) and chain[hits] in self.cached:
            hits += 1
        if hits * self.B == n:  # everything cached: still compute the last block
            hits -= 1
        need = -(-n // self.B) - hits
        hit_blocks = [self.cached[chain[i]] for i in range(hits)]
        reclaimable = sum(1 for b in self.evictable if b not in hit_blocks)
        if need > len(self.free) + reclaimable:
            raise OutOfBlocks(f"need {need} blocks, {len(self.free)} free + {reclaimable} evictable")
        for b in hit_blocks:
            if self.ref[b] == 0:
                del self.evictable[b]
            self.ref[b] += 1
        new_blocks = []
        for _ in range(need):
            b = self._take()
            self.ref[b] = 1
            new_blocks.append(b)
        table = hit_blocks + new_blocks
        prefix = hits * self.B
        slots = [table[t // self.B] * self.B + t % self.B for t in range(prefix, n)]
        rid = self._next_rid
        self._next_rid += 1
        self.requests[rid] = {"blocks": table, "tokens": tokens, "salt": salt, "extra": extra,
                              "published": hits}
        return rid, list(table), prefix, slots

    def append(self, rid: int, token: int) -> int:
        """One generated token joins the request (page C §3 decode): returns its
        slot, allocating a block when the last one is full."""
        r = self.requests[rid]
        t = len(r["tokens"])
        if t // self.B == len(r["blocks"]):
            if not self.free and not self.evictable:
                raise OutOfBlocks("no block for the new token")
            b = self._take()
            self.ref[b] = 1
            r["blocks"].append(b)
        r["tokens"].append(int(token))
        return r["blocks"][t // self.B] * self.B + t % self.B

    def commit(self, rid: int) -> int:
        """The request's KV is written: its full blocks become matchable (page A
        §04, new KV is inserted after a request). Returns how many blocks were
        published; a block whose identity is already cached stays private."""
        r = self.requests[rid]
        chain = self._chain(r["tokens"], r["salt"], r["extra"])
        published = 0
        for i in range(r["published"], len(chain)):
            b = r["blocks"][i]
            if chain[i] not in self.cached and b not in self.ident:
                self.cached[chain[i]] = b
                self.ident[b] = chain[i]
                published += 1
        r["published"] = len(chain)
        return published

    def release(self, rid: int) -> None:
        """The request is finished: its blocks lose a reference, tail first.
        Published blocks nobody uses stay cached (evictable), the rest are free."""
        r = self.requests.pop(rid)
        for b in reversed(r["blocks"]):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                if b in self.ident:
                    self.evictable[b] = None
                else:
                    self.free.append(b)

    def stats(self) -> Tuple[int, int, int]:
        """(free blocks, evictable cached blocks, cached blocks)."""
        return len(self.free), len(self.evictable), len(self.cached)


# --------------------------------------------------------------------------
# radix tree (page A §03, §04; page B "RadixAttention")
# --------------------------------------------------------------------------
class _Node:
    __slots__ = ("key", "values", "children", "parent", "lock", "access", "nid")

    def __init__(self, key: tuple, values: list, parent: Optional["_Node"], nid: int):
        self.key = key            # the tokens on the edge from the parent
        self.values = values      # one value per token of the edge (e.g. its KV slot)
        self.children: Dict[tuple, "_Node"] = {}
        self.parent = parent
        self.lock = 0             # requests holding the path through this node
        self.access = 0           # logical time of the last use
        self.nid = nid            # creation order, breaks LRU ties


class RadixTree:
    """Compressed trie of token sequences with one value per stored token.
    Children are keyed by their first page of tokens; matching proceeds in
    whole pages."""

    def __init__(self, page: int = 1):
        if page <= 0:
            raise ValueError("page must be positive")
        self.page = page
        self._nid = 0
        self.root = self._new((), [], None)
        self.clock = 0

    def _new(self, key, values, parent) -> _Node:
        n = _Node(tuple(key), list(values), parent, self._nid)
        self._nid += 1
        return n

    def _tick(self) -> int:
        self.clock += 1
        return self.clock

    def _common_pages(self, a: Sequence[int], b: Sequence[int]) -> int:
        """Length (a multiple of the page) of the common page-aligned prefix."""
        n, p = 0, self.page
        while n + p <= len(a) and n + p <= len(b) and tuple(a[n:n + p]) == tuple(b[n:n + p]):
            n += p
        return n

    def _split(self, node: _Node, at: int) -> _Node:
        """Cut node's edge after `at` tokens; returns the new upper node."""
        upper = self._new(node.key[:at], node.values[:at], node.parent)
        upper.lock, upper.access = node.lock, node.access
        node.parent.children[node.key[:self.page]] = upper
        node.key, node.values = node.key[at:], node.values[at:]
        node.parent = upper
        upper.children[node.key[:self.page]] = node
        return upper

    def _walk(self, tokens: Sequence[int]) -> Tuple[_Node, int]:
        """Deepest node whose path is a prefix of tokens, splitting an edge
        matched part-way so that the match ends on a node; and the matched
        length."""
        node, pos = self.root, 0
        tokens = list(tokens)
        while pos + self.page <= len(tokens):
            child = node.children.get(tuple(tokens[pos:pos + self.page]))
            if child is None:
                break
            c = self._common_pages(child.key, tokens[pos:])
            if c < len(child.key):
                return self._split(child, c), pos + c
            node, pos = child, pos + c
        return node, pos

    def match_prefix(self, tokens: Sequence[int]) -> Tuple[int, list]:
        """Longest cached prefix (in whole pages): its length and values. The
        nodes on the path count as used now (LRU)."""
        t = self._tick()
        node, pos = self.root, 0
        values: list = []
        tokens = list(tokens)
        while pos + self.page <= len(tokens):
            child = node.children.get(tuple(tokens[pos:pos + self.page]))
            if child is None:
                break
            c = self._common_pages(child.key, tokens[pos:])
            child.access = t
            values += child.values[:c]
            pos += c
            if c < len(child.key):
                break
            node = child
        return pos, values

    def insert(self, tokens: Sequence[int], values: Sequence) -> int:
        """Store a finished request's tokens (whole pages only) with their
        values; returns how many leading tokens were already stored (their
        old values are kept)."""
        tokens = list(tokens)
        n = len(tokens) - len(tokens) % self.page
        if len(values) < n:
            raise ValueError("one value per token")
        t = self._tick()
        node, pos = self._walk(tokens[:n])
        existing = pos
        x = node
        while x is not None:
            x.access = t
            x = x.parent
        if pos < n:
            leaf = self._new(tokens[pos:n], values[pos:n], node)
            leaf.access = t
            node.children[leaf.key[:self.page]] = leaf
        return existing

    def _path_nodes(self, tokens: Sequence[int], length: int) -> List[_Node]:
        if length % self.page:
            raise ValueError("lock lengths are whole pages")
        node, pos = self._walk(list(tokens)[:length])
        if pos != length:
            raise KeyError("the prefix to lock is not stored")
        out = []
        while node is not self.root:
            out.append(node)
            node = node.parent
        return out

    def lock(self, tokens: Sequence[int], length: int) -> None:
        """A running request uses the first `length` stored tokens: none of
        their nodes may be evicted until unlock."""
        for x in self._path_nodes(tokens, length):
            x.lock += 1

    def unlock(self, tokens: Sequence[int], length: int) -> None:
        path = self._path_nodes(tokens, length)
        if any(x.lock <= 0 for x in path):
            raise ValueError("unlock without lock")
        for x in path:
            x.lock -= 1

    def _nodes(self) -> List[_Node]:
        out, stack = [], [self.root]
        while stack:
            x = stack.pop()
            out.append(x)
            stack.extend(x.children.values())
        return out

    def evict(self, num_tokens: int) -> list:
        """Remove unlocked leaves, least recently used first (ties: oldest
        node first), until at least num_tokens tokens are gone or nothing can
        go. A node with children is never removed; once its children are gone
        it is a leaf like any other. Returns the values removed, in order."""
        freed: list = []
        while len(freed) < num_tokens:
            leaves = [x for x in self._nodes()
                      if x is not self.root and not x.children and x.lock == 0]
            if not leaves:
                break
            victim = min(leaves, key=lambda x: (x.access, x.nid))
            freed += victim.values
            del victim.parent.children[victim.key[:self.page]]
        return freed

    def total_tokens(self) -> int:
        return sum(len(x.key) for x in self._nodes())

    def paths(self) -> List[tuple]:
        """Every stored node as (path tokens from the root, lock), sorted; for
        tests that check the tree's shape."""
        out = []
        for x in self._nodes():
            if x is self.root:
                continue
            key, y = [], x
            while y is not self.root:
                key = list(y.key) + key
                y = y.parent
            out.append((tuple(key), x.lock))
        return sorted(out)
