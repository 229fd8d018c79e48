"""Reference block manager (oracle; test infrastructure): plain Python lists and dicts,
no index structures, written from the policy the library documents for its host block
manager (koas-w "errors and solutions", "KV Cache management": a global pool of fixed
blocks handed out and recycled per request, a block_table per request; PocketLLM
"cpp_engine Batching Implementation (Phase 3.1)", risk 3: cross-request prefix sharing).

Policy: a new block is the lowest-numbered free block without a cached prefix, else the
cached free block released longest ago (ties: lowest number); a block that becomes full
is indexed under its chained content key unless that key is indexed already; a new
sequence reuses indexed blocks for its leading full blocks while they match, never for
the block of its last token; appending to a shared partial block copies it first;
released blocks go back last block first.

Content keys here are the full token-id tuples of the prefix up to and including the
block (the library hashes them and compares the ids on a hit), so this model has no
hash at all. Pinned by the invariants tested on it (ownership, refcounts, free count,
slots against tables, cached blocks holding the tokens they are indexed under) and by a
hand-worked scenario.
"""


class BlockManagerRef:
    def __init__(self, num_blocks, block_size=16, prefix_caching=True):
        self.n, self.bs, self.pc = num_blocks, block_size, prefix_caching
        self.ref = [0] * num_blocks
        self.key = [None] * num_blocks         # prefix tuple a cached block is indexed by
        self.released = [0] * num_blocks
        self.seqs = {}                         # id -> {"blocks": [...], "tokens": [...]}
        self.clock = 0

    # -- helpers
    def free_blocks(self):
        return [b for b in range(self.n) if self.ref[b] == 0]

    def num_free(self):
        return len(self.free_blocks())

    def _indexed(self, key):
        for b in range(self.n):
            if self.key[b] == key:
                return b
        return None

    def _take(self):
        plain = [b for b in self.free_blocks() if self.key[b] is None]
        if plain:
            b = min(plain)
        else:
            cached = [b for b in self.free_blocks() if self.key[b] is not None]
            b = min(cached, key=lambda x: (self.released[x], x))
            self.key[b] = None
        self.ref[b] = 1
        return b

    def _release(self, b):
        self.ref[b] -= 1
        if self.ref[b] == 0 and self.key[b] is not None:
            self.released[b] = self.clock
            self.clock += 1

    def _publish(self, b, prefix):
        if self.pc and self.key[b] is None and self._indexed(prefix) is None:
            self.key[b] = prefix

    # -- operations (return values mirror the library's)
    def add_sequence(self, sid, tokens):
        assert sid not in self.seqs
        tokens = list(tokens)
        n, bs = len(tokens), self.bs
        nblocks = -(-n // bs)
        reusable = (n - 1) // bs if n > 0 else 0
        hit = []
        for i in range(reusable):
            b = self._indexed(tuple(tokens[:(i + 1) * bs])) if self.pc else None
            if b is None:
                break
            hit.append(b)
        from_free = sum(1 for b in hit if self.ref[b] == 0)
        if nblocks - len(hit) > self.num_free() - from_free:
            return None                                     # out of blocks, no change
        for b in hit:
            self.ref[b] += 1
        blocks = list(hit)
        for i in range(len(hit), nblocks):
            b = self._take()
            blocks.append(b)
            if (i + 1) * bs <= n:
                self._publish(b, tuple(tokens[:(i + 1) * bs]))
        self.seqs[sid] = {"blocks": blocks, "tokens": tokens}
        return len(hit) * bs

    def append(self, sid, token):
        s = self.seqs[sid]
        pos, bs = len(s["tokens"]), self.bs
        cs = cd = -1
        if pos % bs == 0:
            if self.num_free() < 1:
                return None
            s["blocks"].append(self._take())
        elif self.ref[s["blocks"][-1]] > 1:
            if self.num_free() < 1:
                return None
            old = s["blocks"][-1]
            b = self._take()
            self._release(old)
            s["blocks"][-1] = b
            cs, cd = old, b
        s["tokens"].append(token)
        if (pos + 1) % bs == 0:
            self._publish(s["blocks"][-1], tuple(s["tokens"][:pos + 1]))
        return s["blocks"][-1] * bs + pos % bs, cs, cd

    def fork(self, parent, child):
        assert child not in self.seqs
        p = self.seqs[parent]
        for b in p["blocks"]:
            self.ref[b] += 1
        self.seqs[child] = {"blocks": list(p["blocks"]), "tokens": list(p["tokens"])}

    def free(self, sid):
        for b in reversed(self.seqs.pop(sid)["blocks"]):
            self._release(b)

    def table(self, sid):
        return list(self.seqs[sid]["blocks"]), len(self.seqs[sid]["tokens"])

    def slots(self, sid, first, count):
        bl = self.seqs[sid]["blocks"]
        return [bl[p // self.bs] * self.bs + p % self.bs for p in range(first, first + count)]
