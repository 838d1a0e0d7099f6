// slot.hpp — the address rule of the paged pool, shared by the host entry point
// (pkv_physical_slot) and the device write path (slot mapping, append).
//
// "03 | PagedAttention and the KV-cache memory system", §3: position pos of a
// sequence lies in logical block pos / B at offset pos mod B, and the sequence's
// block-table row names the physical block that holds each logical block, so the
// token's slot (its row across the whole pool) is row[pos / B] * B + pos mod B.
// "KV Cache: capacity, layout, lifecycle", "Page-table addressing", ranks the
// lookups that fail: a block size below 1 or a negative position is a bad
// argument, a logical block past the row is unmapped, and a negative physical
// id names no block (a bad argument as well).
#pragma once

#include <stdint.h>

namespace pkv {

enum : int { kSlotOk = 0, kSlotBadArgument = 1, kSlotUnmapped = 2 };

struct SlotLookup {
  int fault;       // kSlotOk or the first failing class above
  long long slot;  // valid when fault == kSlotOk
};

// constexpr, so that host code and kernels call the same function
constexpr SlotLookup lookup_slot(const int32_t* row, long long row_len, long long block_size,
                                 long long pos) {
  if (block_size < 1 || pos < 0) return SlotLookup{kSlotBadArgument, -1};
  const long long logical = pos / block_size;
  if (logical >= row_len) return SlotLookup{kSlotUnmapped, -1};
  const long long phys = row[logical];
  if (phys < 0) return SlotLookup{kSlotBadArgument, -1};
  return SlotLookup{kSlotOk, phys * block_size + (pos - logical * block_size)};
}

}  // namespace pkv
