"""Reference model of the host block manager with a prefix cache.

Test infrastructure only (see the package docstring).  Plain Python lists and
dicts, written from the pages:

* a pool of equal blocks, a free list, "KV cache block pool exhausted" when
  it runs short, a new block only when the tail block is full --
  [nano-vllm blog §2.2], [CANN notes §2.3];
* a prefix cache over full blocks only (100 tokens -> at most 96 cached);
  a block is identified by the whole token prefix up to its end plus an
  extra key (what the chained hash H(prev, tokens, extra) stands for); a new
  prompt reuses cached blocks from the start up to the first miss --
  [vLLM notes, 链式哈希 / 查找与复用 / 边界条件], [nano-vllm blog §3.2, §4.3];
* reference counts; blocks at count 0 keep their cache entry in a free queue
  and are evicted least-recently-used first when blocks are needed --
  [vLLM notes, 引用计数与 LRU];
* fork shares every block; writing into a shared tail block first moves the
  writer to a copy (copy-on-write) -- [nano-vllm blog §2.2, §4.3].

Readings where the pages are silent (listed with the others in the design
notes): a sequence's blocks are released tail first; the initial free order
is given; a full block whose prefix is already cached under another block is
not cached a second time; a fully cached prompt reports every token cached.

Identity by exact prefix here, and by a verified hash in the library, make
the same decisions; the hash function itself is not modelled.
"""
from __future__ import annotations


class ModelPoolExhausted(RuntimeError):
    pass


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int, extra_key: int = 0, initial_order=None):
        self.num_blocks, self.block_size, self.extra = num_blocks, block_size, extra_key
        self.free = list(initial_order) if initial_order is not None else list(range(num_blocks))
        self.ref = [0] * num_blocks
        self.key_of = {}        # block -> its cache key (prefix tuple, extra)
        self.cache = {}         # cache key -> block
        self.seqs = {}          # seq id -> {"tokens": [...], "table": [...]}
        self.copies = []
        self.lookups = self.hits = self.evictions = 0

    def _key(self, tokens, nblocks):
        return (tuple(tokens[: nblocks * self.block_size]), self.extra)

    def _allocate(self):
        b = self.free.pop(0)                       # least recently used
        if b in self.key_of:
            del self.cache[self.key_of.pop(b)]
            self.evictions += 1
        self.ref[b] = 1
        return b

    def _release(self, b):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)                    # most recently used

    def _register(self, b, key):
        if key not in self.cache:
            self.cache[key] = b
            self.key_of[b] = key

    def add_sequence(self, seq_id, tokens):
        tokens = list(tokens)
        if seq_id in self.seqs:
            raise ValueError("sequence present")
        bs = self.block_size
        full, total = len(tokens) // bs, -(-len(tokens) // bs)
        hits = []
        for i in range(full):
            b = self.cache.get(self._key(tokens, i + 1))
            if b is None:
                break
            hits.append(b)
        revived = sum(1 for b in hits if self.ref[b] == 0)
        if len(self.free) - revived < total - len(hits):
            raise ModelPoolExhausted("KV cache block pool exhausted")
        table = []
        for b in hits:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
            table.append(b)
        for i in range(len(hits), total):
            b = self._allocate()
            table.append(b)
            if i < full:
                self._register(b, self._key(tokens, i + 1))
        self.lookups += len(hits) + 1 if len(hits) < full else full
        self.hits += len(hits)
        self.seqs[seq_id] = {"tokens": tokens, "table": table}
        return len(hits) * bs

    def append_token(self, seq_id, token):
        seq = self.seqs[seq_id]
        bs = self.block_size
        n = len(seq["tokens"])
        if n % bs == 0:
            if not self.free:
                raise ModelPoolExhausted("KV cache block pool exhausted")
            seq["table"].append(self._allocate())
        else:
            tail = seq["table"][-1]
            if self.ref[tail] > 1:
                if not self.free:
                    raise ModelPoolExhausted("KV cache block pool exhausted")
                b = self._allocate()
                self.copies.append((tail, b))
                self._release(tail)
                seq["table"][-1] = b
        seq["tokens"].append(token)
        if (n + 1) % bs == 0:
            self._register(seq["table"][-1], self._key(seq["tokens"], (n + 1) // bs))

    def fork(self, parent_id, child_id):
        if child_id in self.seqs:
            raise ValueError("sequence present")
        p = self.seqs[parent_id]
        for b in p["table"]:
            self.ref[b] += 1
        self.seqs[child_id] = {"tokens": list(p["tokens"]), "table": list(p["table"])}

    def free_sequence(self, seq_id):
        for b in reversed(self.seqs.pop(seq_id)["table"]):
            self._release(b)

    def take_copies(self):
        out, self.copies = self.copies, []
        return out
