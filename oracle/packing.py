"""CPU oracle for the multi-adapter microbatch packer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/`` may import this module; the library's packer (host C++ in
``lora_fine_tuning_amd/csrc/packer.cpp``) shares no code with it.

What is computed, and where the pages say so:

* Greedy packing (papers.chlience.com notes on LoRAFusion, section 4
  "Multi-LoRA scheduler"; juhe.plus blog, section 4.2 step 2): the samples of
  a global batch go into microbatches of at most ``capacity`` tokens; the
  pages' packer solves a two-stage MILP and falls back to a greedy packing.
  The greedy rule is not spelled out; the reading taken here is first-fit
  decreasing: samples by length, longest first (ties: lower sample index
  first), each into the lowest-numbered open microbatch with room, else a
  new one.  Written as the plain linear scan over the open microbatches.
* Segment table of a microbatch (juhe.plus blog, section 4.1: every tile
  carries an adapter id and the kernel looks the adapter up): the
  microbatch's samples grouped by adapter -- adapters in increasing id,
  samples of one adapter in increasing sample index -- one segment per
  adapter present.
* Bubble lemma (papers.chlience.com notes, section 4; juhe.plus blog,
  section 4.2 step 1): with S pipeline stages, if a sample of adapter a's
  global batch j sits in microbatch k, no sample of the adapter's next batch
  may sit in a microbatch before k + S - 1.  Checked here over every pair of
  samples; "next batch" is the adapter's next batch index that has samples.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple


def pack_ffd(lengths: Sequence[int], capacity: int) -> List[int]:
    """Microbatch index of every sample (first-fit decreasing)."""
    if capacity <= 0:
        raise ValueError("capacity must be positive")
    for ln in lengths:
        if ln < 1 or ln > capacity:
            raise ValueError(f"sample length {ln} outside [1, {capacity}]")
    order = sorted(range(len(lengths)), key=lambda i: (-lengths[i], i))
    room: List[int] = []          # free tokens of each open microbatch
    mb = [-1] * len(lengths)
    for i in order:
        for b in range(len(room)):
            if room[b] >= lengths[i]:
                room[b] -= lengths[i]
                mb[i] = b
                break
        else:
            room.append(capacity - lengths[i])
            mb[i] = len(room) - 1
    return mb


def microbatch_segments(lengths: Sequence[int], adapter: Sequence[int], mb_of_sample: Sequence[int],
                        mb: int) -> Tuple[List[int], List[int], List[int]]:
    """(sample order, seg_off, seg_adapter) of microbatch ``mb``."""
    members = [i for i in range(len(lengths)) if mb_of_sample[i] == mb]
    members.sort(key=lambda i: (adapter[i], i))
    seg_off, seg_ad = [0], []
    rows = 0
    for i in members:
        if not seg_ad or seg_ad[-1] != adapter[i]:
            if seg_ad:
                seg_off.append(rows)
            seg_ad.append(adapter[i])
        rows += lengths[i]
    if seg_ad:
        seg_off.append(rows)
    return members, seg_off, seg_ad


def bubble_violations(mb_of_sample: Sequence[int], adapter: Sequence[int], batch: Sequence[int],
                      stages: int) -> List[Tuple[int, int]]:
    """(adapter, batch) pairs whose next batch starts too early, sorted."""
    if stages < 1:
        raise ValueError("stages must be >= 1")
    n = len(mb_of_sample)
    batches_of = {}
    for i in range(n):
        batches_of.setdefault(adapter[i], set()).add(batch[i])
    bad = set()
    for i in range(n):
        later = sorted(b for b in batches_of[adapter[i]] if b > batch[i])
        if not later:
            continue
        nxt = later[0]
        for j in range(n):
            if adapter[j] == adapter[i] and batch[j] == nxt and mb_of_sample[j] < mb_of_sample[i] + stages - 1:
                bad.add((adapter[i], batch[i]))
    return sorted(bad)
