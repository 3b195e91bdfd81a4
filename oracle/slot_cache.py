"""Plain-Python oracle of the adapter slot cache.

TEST INFRASTRUCTURE (see the package docstring).  It follows the managers of
the pages step by step, in their own terms:

* [vLLM] "vLLM LoRA 实现深度解析" §5.3 activate_adapter: an id that is
  already active is skipped; otherwise the first slot whose entry in
  lora_index_to_id is None is taken, and with none free the base manager
  raises "No free lora slots".
* [vLLM] §7 LRU 缓存策略: the LRU manager first removes the oldest active
  adapter when the active set is full, then activates as above, then
  touches the adapter (most recently used); pinned adapters are not removed.
* [MAX-V3] "LoRAManagerV3" activate_adapter / unload_adapter /
  is_active_lora: activation assigns an LRU slot, evicting the least
  recently used adapter when full; unloading frees the slot.

Recency is an explicit list of active ids, oldest first (not a counter).  A
batch first touches its adapters that are already active, then activates
the others in first-appearance order, never removing an adapter of the
batch.  Errors are raised as SlotCacheError with the library's status codes
(7 no free slot, 8 not active, 1 bad argument).
"""

from __future__ import annotations

import copy
from typing import List, Optional, Tuple

LRU, NO_EVICT = 0, 1
NO_FREE_SLOT, NOT_ACTIVE, INVALID_ARGUMENT = 7, 8, 1


class SlotCacheError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"slot cache error {code}")
        self.code = code


class OracleSlotCache:
    def __init__(self, num_slots: int, policy: int = LRU):
        if num_slots <= 0 or policy not in (LRU, NO_EVICT):
            raise SlotCacheError(INVALID_ARGUMENT)
        self.policy = policy
        self.lora_index_to_id: List[Optional[int]] = [None] * num_slots
        self.order: List[int] = []  # active ids, least recently used first
        self.pinned: set = set()

    def _touch(self, adapter_id: int) -> None:
        self.order.remove(adapter_id)
        self.order.append(adapter_id)

    def _activate(self, adapter_id: int, keep=()) -> Tuple[int, bool, int]:
        if adapter_id < 0:
            raise SlotCacheError(INVALID_ARGUMENT)
        if adapter_id in self.lora_index_to_id:           # §5.3: already active
            self._touch(adapter_id)                        # §7: touch
            return self.lora_index_to_id.index(adapter_id), False, -1
        evicted = -1
        if None not in self.lora_index_to_id:
            if self.policy == NO_EVICT:                    # §5.3: "No free lora slots"
                raise SlotCacheError(NO_FREE_SLOT)
            victims = [a for a in self.order if a not in self.pinned and a not in keep]
            if not victims:
                raise SlotCacheError(NO_FREE_SLOT)
            evicted = victims[0]                           # §7: remove_oldest
            self.lora_index_to_id[self.lora_index_to_id.index(evicted)] = None
            self.order.remove(evicted)
        slot = self.lora_index_to_id.index(None)          # §5.3: first free slot
        self.lora_index_to_id[slot] = adapter_id
        self.order.append(adapter_id)                      # most recently used
        return slot, True, evicted

    def activate(self, adapter_id: int) -> Tuple[int, bool, int]:
        return self._activate(adapter_id)

    def activate_batch(self, adapter_ids) -> Tuple[List[int], List[int], List[int]]:
        if any(a < -1 for a in adapter_ids):
            raise SlotCacheError(INVALID_ARGUMENT)
        saved = copy.deepcopy((self.lora_index_to_id, self.order, self.pinned))
        request_slot, load_slots, load_ids, done = [], [], [], []
        try:
            # the batch's active adapters are touched first, in first-appearance
            # order, so that loading the others never removes them
            for a in adapter_ids:
                if a != -1 and a not in done and a in self.lora_index_to_id:
                    self._touch(a)
                    done.append(a)
            for a in adapter_ids:
                if a == -1:
                    request_slot.append(-1)
                    continue
                if a in done:
                    request_slot.append(self.lora_index_to_id.index(a))
                    continue
                slot, load, _ = self._activate(a, keep=done)
                done.append(a)
                request_slot.append(slot)
                if load:
                    load_slots.append(slot)
                    load_ids.append(a)
        except SlotCacheError:
            self.lora_index_to_id, self.order, self.pinned = saved
            raise
        return request_slot, load_slots, load_ids

    def unload(self, adapter_id: int) -> int:
        if adapter_id < 0:
            raise SlotCacheError(INVALID_ARGUMENT)
        if adapter_id not in self.lora_index_to_id:
            raise SlotCacheError(NOT_ACTIVE)
        slot = self.lora_index_to_id.index(adapter_id)
        self.lora_index_to_id[slot] = None
        self.order.remove(adapter_id)
        self.pinned.discard(adapter_id)
        return slot

    def pin(self, adapter_id: int, pinned: bool = True) -> Tuple[int, bool, int]:
        if adapter_id < 0:
            raise SlotCacheError(INVALID_ARGUMENT)
        if not pinned:
            if adapter_id not in self.lora_index_to_id:
                raise SlotCacheError(NOT_ACTIVE)
            self.pinned.discard(adapter_id)
            return self.lora_index_to_id.index(adapter_id), False, -1
        result = self._activate(adapter_id)
        self.pinned.add(adapter_id)
        return result

    def lookup(self, adapter_id: int) -> int:
        return self.lora_index_to_id.index(adapter_id) if adapter_id in self.lora_index_to_id else -1

    def slot_table(self) -> Tuple[List[int], List[int]]:
        ids = [-1 if a is None else a for a in self.lora_index_to_id]
        return ids, [1 if a is not None and a in self.pinned else 0 for a in self.lora_index_to_id]
