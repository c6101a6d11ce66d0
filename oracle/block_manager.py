"""Reference model of the paged block manager -- TEST INFRASTRUCTURE ONLY.

Only ``tests/`` may import this module; the product library never uses it.  It is a plain
restatement, in Python lists and dicts, of what the pages say the block manager keeps
("vllm-project-vllm -- L2", section 9 "Memory Management"; section 8 on the block-table
invariant; section 11 steps 2 and 5):
  * a sequence's KV lives in fixed-size blocks that are allocated one at a time as tokens
    arrive, so a sequence wastes at most block_size - 1 slots;
  * blocks are shared copy-on-write: a fork only adds references, and a sequence that writes
    into a shared block first moves to a private copy;
  * every physical block is free, uniquely owned, or shared with a positive reference count;
  * blocks of a preempted sequence can be swapped to CPU memory and back.
Choices the pages leave open follow the C ABI's stated policy: the lowest-numbered free block
is taken first, status codes are those of include/pagedkv.h.
"""
from __future__ import annotations

OK, SHAPE, STATE, NOT_FOUND, NO_SPACE = 0, -2, -8, -9, -10


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int, num_host_blocks: int = 0):
        self.bs = block_size
        self.nb = num_blocks
        self.nhb = num_host_blocks
        self.ref = [0] * num_blocks
        self.free = set(range(num_blocks))
        self.host_used = [False] * num_host_blocks
        self.seqs = {}                     # id -> {"blocks": [...], "n": tokens, "swapped": bool}

    # -- helpers
    def _take(self):
        b = min(self.free)
        self.free.remove(b)
        return b

    def _take_host(self):
        h = self.host_used.index(False)
        self.host_used[h] = True
        return h

    def _unref(self, b):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.add(b)

    def blocks_needed(self, n):
        return -(-n // self.bs)

    # -- operations (same meaning and status codes as the C ABI)
    def add(self, sid, n):
        if n < 0:
            return SHAPE
        if sid in self.seqs:
            return STATE
        need = self.blocks_needed(n)
        if need > len(self.free):
            return NO_SPACE
        blocks = []
        for _ in range(need):
            b = self._take()
            self.ref[b] = 1
            blocks.append(b)
        self.seqs[sid] = {"blocks": blocks, "n": n, "swapped": False}
        return OK

    def append(self, sid):
        """-> (status, slot, copy_src, copy_dst)"""
        s = self.seqs.get(sid)
        if s is None:
            return NOT_FOUND, None, -1, -1
        if s["swapped"]:
            return STATE, None, -1, -1
        pos = s["n"]
        src = dst = -1
        if pos % self.bs == 0:                       # the last block is full: a new block
            if not self.free:
                return NO_SPACE, None, -1, -1
            b = self._take()
            self.ref[b] = 1
            s["blocks"].append(b)
        else:
            last = s["blocks"][-1]
            if self.ref[last] > 1:                   # shared: write into a private copy
                if not self.free:
                    return NO_SPACE, None, -1, -1
                b = self._take()
                self.ref[b] = 1
                self.ref[last] -= 1
                s["blocks"][-1] = b
                src, dst = last, b
        s["n"] = pos + 1
        return OK, s["blocks"][-1] * self.bs + pos % self.bs, src, dst

    def fork(self, parent, child, n=-1):
        p = self.seqs.get(parent)
        if p is None:
            return NOT_FOUND
        if p["swapped"] or child in self.seqs:
            return STATE
        n = p["n"] if n < 0 else n
        if n > p["n"]:
            return SHAPE
        blocks = p["blocks"][: self.blocks_needed(n)]
        for b in blocks:
            self.ref[b] += 1
        self.seqs[child] = {"blocks": list(blocks), "n": n, "swapped": False}
        return OK

    def release(self, sid):
        s = self.seqs.pop(sid, None)
        if s is None:
            return NOT_FOUND
        for b in s["blocks"]:
            if s["swapped"]:
                self.host_used[b] = False
            else:
                self._unref(b)
        return OK

    def swap_out(self, sid):
        """-> (status, [(device block, host block), ...])"""
        s = self.seqs.get(sid)
        if s is None:
            return NOT_FOUND, []
        if s["swapped"]:
            return STATE, []
        if len(s["blocks"]) > self.host_used.count(False):
            return NO_SPACE, []
        pairs = []
        for i, d in enumerate(s["blocks"]):
            h = self._take_host()
            pairs.append((d, h))
            s["blocks"][i] = h
            self._unref(d)
        s["swapped"] = True
        return OK, pairs

    def swap_in(self, sid):
        """-> (status, [(host block, device block), ...])"""
        s = self.seqs.get(sid)
        if s is None:
            return NOT_FOUND, []
        if not s["swapped"]:
            return STATE, []
        if len(s["blocks"]) > len(self.free):
            return NO_SPACE, []
        pairs = []
        for i, h in enumerate(s["blocks"]):
            d = self._take()
            self.ref[d] = 1
            pairs.append((h, d))
            s["blocks"][i] = d
            self.host_used[h] = False
        s["swapped"] = False
        return OK, pairs

    def table(self, sids, max_blocks):
        rows, lens = [], []
        for sid in sids:
            s = self.seqs.get(sid)
            if s is None:
                return NOT_FOUND, None, None
            if s["swapped"]:
                return STATE, None, None
            if len(s["blocks"]) > max_blocks:
                return SHAPE, None, None
            rows.append(s["blocks"] + [0] * (max_blocks - len(s["blocks"])))
            lens.append(s["n"])
        return OK, rows, lens

    def invariant_holds(self) -> bool:
        """Every block free with no reference, or referenced exactly ref[b] times; every
        sequence holds exactly ceil(n / block_size) blocks; host blocks used at most once."""
        count = [0] * self.nb
        hcount = [0] * self.nhb
        for s in self.seqs.values():
            if len(s["blocks"]) != self.blocks_needed(s["n"]):
                return False
            for b in s["blocks"]:
                if s["swapped"]:
                    hcount[b] += 1
                else:
                    count[b] += 1
        if any(c != r for c, r in zip(count, self.ref)):
            return False
        if any((b in self.free) != (count[b] == 0) for b in range(self.nb)):
            return False
        return all(hc == int(u) for hc, u in zip(hcount, self.host_used))
