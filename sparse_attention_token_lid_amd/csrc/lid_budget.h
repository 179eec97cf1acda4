// lid_budget.h -- candidate-buffer accounting of the prefill kernel's
// streaming top-k: how many slots a wavefront's LDS buffer has and when it
// must be cut back.  Shared by the kernel, the host's plan (lid_api.hip) and
// a host emulation test that checks every reachable buffer count; the
// functions are constexpr, so host and device code use the same ones.
//
// The kernel hands its scores to the top-k in units of 64 keys, one per lane
// (two units per 128-key tile).  All 64 lanes store: a passing key at
// count + (its rank among the n passing lanes), every other lane at
// count + n + lane, past the new count, where the entry is dead.  So a unit
// with 0 < n < 64 passing keys touches slots up to count + n + 63, and the
// buffer must have 128 free slots before every unit.  Compaction points are
// the tile barriers: a wavefront that could not take another tile's two
// units raises a flag before the barrier, and after it every wavefront
// holding more than K + kTrimSlack keys is trimmed to between K and
// K + kTrimSlack keys (all keys that can still reach its top K stay).
#pragma once

namespace lid {

constexpr int kUnitKeys = 64;     // keys handed to a wavefront's top-k at once
constexpr int kUnitsPerTile = 2;  // hand-offs between two compaction points
constexpr int kTrimSlack = 128;   // an in-stream trim keeps at most this many keys beyond K

// Candidate slots per wavefront.  After a compaction point a buffer holds
// at most max(cap - 3 * 64 (not flagged), K + kTrimSlack (trimmed or too
// short to trim)) keys, and two units must then fit, each with 128 free
// slots in front of it: so cap >= K + kTrimSlack + 3 * 64.  Above that, 2 K
// + 184 slots leave room for longer runs between trims at large K (184: with
// K = 512, eight such buffers fit in LDS beside the key tiles and the linear
// terms of the prefill kernel).
constexpr int prefill_cap(int K) {
  return 2 * K + 184 > K + kTrimSlack + (kUnitsPerTile + 1) * kUnitKeys ? 2 * K + 184
                                                                        : K + kTrimSlack + (kUnitsPerTile + 1) * kUnitKeys;
}

// End of a tile: raise the flag when the buffer could not take another
// tile's units.
constexpr bool prefill_flag(int count, int cap) { return count > cap - (kUnitsPerTile + 1) * kUnitKeys; }

// After the barrier of a flagged tile: a wavefront is trimmed when it holds
// more than K + kTrimSlack keys.
constexpr bool prefill_trim(int count, int K) { return count > K + kTrimSlack; }

// Before the last unit, after the stream: room for one unit.
constexpr bool prefill_room(int count, int cap) { return count > cap - 2 * kUnitKeys; }

}  // namespace lid
