"""Prefix-hash index of cached sender states (test infrastructure only).

MapFlow article, storage-and-execution section (second component): the sparse
blocks kept for different layers and positions differ in number; the shared
prefix cache indexes them by a prefix hash that carries the information of the
preceding context, and a receiver finds the cached blocks it can use through it;
one sender state can serve several downstream models.

Readings (the page names the idea, not a hash or a policy):
* a cached unit is one block-row (64 query positions) of one layer, all sender
  heads; block-row b of a causal map depends on tokens 0 .. 64 b + 63 only, so
  its key is a chain hash over the 64-token blocks up to and including b;
* the chain hash is 64-bit FNV-1a (Fowler-Noll-Vo, variant 1a: start from the
  offset basis, for each byte xor it in and multiply by the FNV prime modulo
  2^64) over the previous block's hash (8 bytes, little-endian; a caller seed for
  block 0) followed by the block's 64 token ids (4 bytes each, little-endian,
  two's complement); only whole blocks are hashed;
* a lookup reuses the longest run of leading hits; entries are evicted least
  recently used first (a lookup hit or a re-insert makes an entry the most
  recent); capacity is a count of entries.
"""
from collections import OrderedDict

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
MASK = (1 << 64) - 1


def fnv1a64(data: bytes, h: int = FNV_OFFSET) -> int:
    """FNV-1a, 64 bits, of a byte string (optionally continuing from ``h``)."""
    for b in data:
        h ^= b
        h = (h * FNV_PRIME) & MASK
    return h


def prefix_hashes(tokens, seed: int):
    """Chain hashes of the whole 64-token blocks of ``tokens``."""
    out, prev = [], seed & MASK
    for b in range(len(tokens) // 64):
        data = prev.to_bytes(8, "little") + b"".join(
            (int(t) & 0xFFFFFFFF).to_bytes(4, "little") for t in tokens[64 * b: 64 * b + 64])
        prev = fnv1a64(data)
        out.append(prev)
    return out


class PrefixIndexModel:
    """The index's behaviour as a plain ordered dictionary (most recent last)."""

    def __init__(self, capacity):
        self.capacity = capacity
        self.d = OrderedDict()

    def insert(self, layer, h, value):
        key = (layer, h)
        if key in self.d:
            self.d[key] = value
            self.d.move_to_end(key)
            return True
        if len(self.d) >= self.capacity:
            return False
        self.d[key] = value
        return True

    def lookup(self, layer, hashes):
        found = []
        for h in hashes:
            key = (layer, h)
            if key not in self.d:
                break
            self.d.move_to_end(key)
            found.append(self.d[key])
        return found

    def erase(self, layer, h):
        return self.d.pop((layer, h), None) is not None

    def evict_lru(self):
        if not self.d:
            return None
        key, value = self.d.popitem(last=False)
        return key, value
