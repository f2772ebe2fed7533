"""Plain CPU oracle of KVCMAS anchor-pool updates.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this module; only
the tests do.  It shares no code with the HIP library.

Source: "KVCMAS: Efficient KV cache Correction for Shared Context in Multi-Agent Systems"
(arXiv 2609.34060), App. A.3:
  * "Anchor Pool Management": each shared-context slot keeps a pool of up to V anchors, each
    with a low-rank source representation and corrections for its consumers.
  * "Cache Materialization and Pool Updates": an unreliable match triggers dense prefill;
    then Delta = C_j - Align(C_i) (Eq. 12) and the source are factorised and inserted as a
    new anchor; accepted corrections are not reinserted; when the pool is full the least
    frequently used anchor among the five oldest entries is evicted.
  * "Variable Segment Lengths": a correction uses the anchors covering the segment, else the
    longest covered prefix (the correction set).

Readings where the pages are silent (listed in the repository's design notes):
  * an anchor stores the correction of the consumer whose fallback created it (every
    fallback inserts a new anchor); a consumer's view is the anchors holding its correction;
  * "used" = in the correction set of an accepted hop of that consumer; a flagged hop uses
    nothing;
  * a free slot is filled first, the lowest index; ties in use count go to the oldest.

Eq. 12 itself and the factorisation are in kvc_oracle (observed_delta, rope,
truncated_svd).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

EVICT_WINDOW = 5   # App. A.3: "among the five oldest entries"


@dataclass
class Anchor:
    stamp: int        # insertion order (1, 2, ...)
    length: int       # stored rows
    consumer: int     # consumer whose correction the anchor holds
    uses: int = 0     # accepted hops whose correction set contained it


@dataclass
class PoolPolicy:
    capacity: int
    slots: List[Optional[Anchor]] = field(default_factory=list)
    clock: int = 0

    def __post_init__(self):
        assert 1 <= self.capacity
        self.slots = [None] * self.capacity

    def anchors_of(self, consumer: int) -> List[int]:
        """The consumer's view: slots holding an anchor with its correction."""
        return [i for i, a in enumerate(self.slots) if a is not None and a.consumer == consumer]

    def correction_set(self, consumer: int, seg_len: int) -> List[int]:
        """App. A.3 "Variable Segment Lengths": anchors covering min(S, longest) rows."""
        mine = self.anchors_of(consumer)
        if not mine:
            return []
        s_cov = min(seg_len, max(self.slots[i].length for i in mine))
        return [i for i in mine if self.slots[i].length >= s_cov]

    def victim(self) -> int:
        """The slot a new anchor takes: an empty one (lowest index) if any; else, among the
        EVICT_WINDOW oldest anchors, the least frequently used, the oldest on a tie."""
        for i, a in enumerate(self.slots):
            if a is None:
                return i
        oldest = sorted(range(self.capacity), key=lambda i: self.slots[i].stamp)[:EVICT_WINDOW]
        return min(oldest, key=lambda i: (self.slots[i].uses, self.slots[i].stamp))

    def record_hop(self, consumer: int, seg_len: int, flagged: bool) -> Tuple[int, int]:
        """One hop into `consumer` after its gate decision.  Returns (slot, evicted): (-1, -1)
        for an accepted correction (nothing reinserted, its correction set gains a use); for a
        dense fallback the slot the new anchor takes and the slot evicted (or -1)."""
        if not flagged:
            for i in self.correction_set(consumer, seg_len):
                self.slots[i].uses += 1
            return -1, -1
        slot = self.victim()
        evicted = slot if self.slots[slot] is not None else -1
        self.clock += 1
        self.slots[slot] = Anchor(stamp=self.clock, length=seg_len, consumer=consumer)
        return slot, evicted

    def view(self, consumer: int) -> Tuple[List[int], List[int]]:
        """(anchor_len, live) over all slots for `consumer`'s match / correct calls."""
        lens, live = [], []
        for a in self.slots:
            mine = a is not None and a.consumer == consumer
            lens.append(a.length if mine else 0)
            live.append(1 if mine else 0)
        return lens, live
