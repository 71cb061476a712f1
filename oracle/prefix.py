"""Reference prefix cache (test infrastructure; see ``oracle/__init__``).

Written from [manager] "Build a paged KV cache manager from scratch":
* "Architecture Overview" / "Step 4: The Prefix Tree (Radix Trie)": a trie
  whose edges are the token ids of one full block and whose nodes carry the
  block holding those tokens; a request's prompt is matched block by block
  from the root and reuses the blocks found; the request's blocks are then
  inserted ("published");
* "Step 2: The Block Pool": a block whose refcount drops to zero is kept for
  reuse and reclaimed least recently used first.

Readings (shared with the native manager): only full blocks are published
and matched, and a match leaves at least one prompt token to compute; a
zero-refcount block that is not in the trie is freed at once (as in
``RefPool``), one that is in the trie is cached; an allocation that finds the
free stack empty evicts the least recently released cached block with its
subtree, listed breadth first and handled deepest first: cached nodes go back
on the free stack, nodes still in use only leave the trie; publishing stops at
a path that already leads to another block, at a block already in the trie
elsewhere, or at a released block.
"""
from __future__ import annotations

from collections import OrderedDict

from .paging import Exhausted, blocks_for


class _Node:
    def __init__(self, block, parent, key):
        self.block = block
        self.parent = parent          # _Node or None (root)
        self.key = key                # token tuple of the edge from the parent
        self.children = {}            # token tuple -> _Node (insertion order kept)


class RefPrefixPool:
    """``RefPool``'s interface (stack, refs, pop, retain, release) plus the trie."""

    def __init__(self, num_blocks: int, first_pops=None):
        order = range(num_blocks) if first_pops is None else [int(b) for b in first_pops]
        assert sorted(order) == list(range(num_blocks))
        self.num_blocks = num_blocks
        self.stack = list(reversed(list(order)))
        self.refs: dict = {}
        self.root = _Node(None, None, None)
        self.node_of: dict = {}       # block -> _Node, for blocks in the trie
        self.cached = OrderedDict()   # zero-refcount blocks in the trie, least recently released first

    @property
    def num_free(self) -> int:
        return len(self.stack)

    @property
    def num_cached(self) -> int:
        return len(self.cached)

    def _evict(self, block) -> None:
        top = self.node_of[block]
        del top.parent.children[top.key]
        order = [top]
        i = 0
        while i < len(order):
            order += list(order[i].children.values())
            i += 1
        for node in reversed(order):
            b = node.block
            del self.node_of[b]
            node.children = {}
            if b not in self.refs:        # cached: back on the free stack
                del self.cached[b]
                self.stack.append(b)

    def pop(self) -> int:
        if not self.stack:
            if not self.cached:
                raise Exhausted("no free block")
            self._evict(next(iter(self.cached)))
        b = self.stack.pop()
        self.refs[b] = 1
        return b

    def pop_for(self, num_tokens: int, block_size: int) -> list:
        n = blocks_for(num_tokens, block_size)
        if n > len(self.stack) + len(self.cached):
            raise Exhausted(f"need {n} blocks")
        return [self.pop() for _ in range(n)]

    def retain(self, b: int) -> None:
        if b not in self.refs:
            raise ValueError(f"block {b} is not allocated")
        self.refs[b] += 1

    def release(self, b: int) -> None:
        if b not in self.refs:
            raise ValueError(f"block {b} is not allocated")
        self.refs[b] -= 1
        if self.refs[b] == 0:
            del self.refs[b]
            if b in self.node_of:
                self.cached[b] = True
            else:
                self.stack.append(b)

    def match(self, tokens, block_size: int) -> list:
        """Blocks of the longest published chain matching the prompt's full
        blocks, leaving at least one token; each is retained (revived when cached)."""
        node, found = self.root, []
        for j in range((len(tokens) - 1) // block_size):
            key = tuple(int(t) for t in tokens[j * block_size:(j + 1) * block_size])
            if key not in node.children:
                break
            node = node.children[key]
            found.append(node.block)
        for b in found:
            if b in self.refs:
                self.refs[b] += 1
            else:
                del self.cached[b]
                self.refs[b] = 1
        return found

    def publish(self, table, length: int, tokens, block_size: int) -> None:
        node = self.root
        for j in range(min(len(tokens), length) // block_size):
            b = table[j]
            if b < 0:
                break
            key = tuple(int(t) for t in tokens[j * block_size:(j + 1) * block_size])
            if key in node.children:
                if node.children[key].block != b:
                    break
                node = node.children[key]
                continue
            if b in self.node_of:
                break
            child = _Node(b, node, key)
            node.children[key] = child
            self.node_of[b] = child
            node = child
