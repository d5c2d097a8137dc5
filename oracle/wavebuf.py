"""Wave buffer (GPU block cache over a host tier), oracle side.

TEST INFRASTRUCTURE ONLY (see the package docstring). The RetroInfer pages
(framerc blog section 2.2, the wave buffer) keep hot 2 KB KV blocks in GPU
memory with a block mapping table and LRU replacement, updated off the
critical path; they state no finer rule. Readings, shared with the library:

- after a decode step that retrieved the clusters R, the needed blocks are
  every block of every cluster of R (ceil(n_c / T) blocks from
  block_off[c]), in ascending block order;
- a needed block that is cached is a hit: its slot is marked used at this
  step;
- the misses, ascending, take the slots not used at this step, least
  recently used first (by last-use step, then slot id; never-used slots have
  step 0), as many as there are; each evicts its slot's old block.

One WaveBufferSim per unit; plain Python lists and sorted(), no batching.
"""


def needed_blocks(R, sizes, block_off, T):
    """Blocks of the clusters R, ascending."""
    out = []
    for c in sorted(int(x) for x in R):
        n = int(sizes[c])
        first = int(block_off[c])
        out.extend(range(first, first + (n + T - 1) // T))
    return sorted(out)


class WaveBufferSim:
    def __init__(self, n_slots, n_blocks):
        self.n_slots = n_slots
        self.block_slot = [-1] * n_blocks
        self.slot_block = [-1] * n_slots
        self.slot_last = [0] * n_slots

    def step(self, t, blocks):
        """Apply one step's needed blocks (ascending); returns (hits, misses,
        admitted (block, slot) pairs)."""
        hits = 0
        misses = []
        for b in blocks:
            s = self.block_slot[b]
            if s >= 0:
                hits += 1
                self.slot_last[s] = t
            else:
                misses.append(b)
        free = sorted((self.slot_last[s], s) for s in range(self.n_slots)
                      if self.slot_last[s] != t)
        admitted = []
        for b, (_, s) in zip(misses, free):
            old = self.slot_block[s]
            if old >= 0:
                self.block_slot[old] = -1
            self.block_slot[b] = s
            self.slot_block[s] = b
            self.slot_last[s] = t
            admitted.append((b, s))
        return hits, len(misses), admitted
