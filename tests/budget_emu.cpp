// Host emulation of the prefill kernel's candidate-buffer accounting
// (lid_budget.h, the same constexpr rules the kernel uses): for each k_top
// given on the command line it walks every buffer count a wavefront can
// reach at a compaction point, under any sequence of hand-offs (0..64
// passing keys each, two per tile), flags and trims (a trim leaves its
// worst case, K + kTrimSlack keys), and checks that no hand-off writes past
// the buffer's capacity, neither inside the stream nor in the last unit
// after it.  Prints "ok K cap states" per k_top, or the first violation and
// exits 1.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "lid_budget.h"

using namespace lid;

// A hand-off of n passing keys at count c: the passing lanes store at
// c .. c + n - 1, every other lane at c + n + lane (lane < 64); with no
// passing key no lane stores.
static int last_slot(int c, int n) { return n == 0 ? c - 1 : (n == kUnitKeys ? c + n - 1 : c + n + kUnitKeys - 1); }
static bool unit_fits(int c, int n, int cap) { return last_slot(c, n) < cap; }

int main(int argc, char** argv) {
  for (int a = 1; a < argc; ++a) {
    const int K = std::atoi(argv[a]);
    const int cap = prefill_cap(K);
    std::vector<char> reach(cap + 1, 0), seen(cap + 1, 0);
    reach[0] = 1;  // an empty buffer before the first tile
    bool changed = true;
    int states = 0;
    while (changed) {
      changed = false;
      for (int c0 = 0; c0 <= cap; ++c0) {
        if (!reach[c0] || seen[c0]) continue;
        seen[c0] = 1;
        ++states;
        // the last unit after the stream, behind the room check
        {
          const int c = (prefill_room(c0, cap) && prefill_trim(c0, K)) ? K + kTrimSlack : c0;
          for (int n = 0; n <= kUnitKeys; ++n)
            if (!unit_fits(c, n, cap)) {
              std::printf("violation K=%d cap=%d: last unit at count %d with %d passing\n", K, cap, c, n);
              return 1;
            }
        }
        // one tile: two units, then the flag, the barrier and the trims
        for (int n1 = 0; n1 <= kUnitKeys; ++n1) {
          if (!unit_fits(c0, n1, cap)) {
            std::printf("violation K=%d cap=%d: first unit at count %d with %d passing\n", K, cap, c0, n1);
            return 1;
          }
          const int c1 = c0 + n1;
          for (int n2 = 0; n2 <= kUnitKeys; ++n2) {
            if (!unit_fits(c1, n2, cap)) {
              std::printf("violation K=%d cap=%d: second unit at count %d with %d passing\n", K, cap, c1, n2);
              return 1;
            }
            const int c2 = c1 + n2;
            if (c2 > cap) {
              std::printf("violation K=%d cap=%d: count %d past capacity\n", K, cap, c2);
              return 1;
            }
            // after the barrier: if any wavefront flagged, this one is trimmed
            // when it holds too many; if it flagged itself, someone did
            const int trimmed = prefill_trim(c2, K) ? K + kTrimSlack : c2;
            int outs[2] = {trimmed, c2};
            const int nouts = prefill_flag(c2, cap) ? 1 : 2;  // not flagged: nobody may have
            for (int o = 0; o < nouts; ++o) {
              if (outs[o] > cap) {
                std::printf("violation K=%d cap=%d: count %d after the barrier\n", K, cap, outs[o]);
                return 1;
              }
              if (!reach[outs[o]]) {
                reach[outs[o]] = 1;
                changed = true;
              }
            }
          }
        }
      }
    }
    std::printf("ok K=%d cap=%d states=%d\n", K, cap, states);
  }
  return 0;
}
