// Tile records for the streaming decode passes (layout: kRecInts in
// internal.h): everything a pass needs about a routed tile, in one row that
// a wave reads with one load per lane.
#pragma once

#include "device.h"
#include "internal.h"

namespace moe {

// Records of tiles [0, *p.n_tiles) from the tile table, the sorted order and
// the slots' routing weights, by threads tid, tid + nthreads, ...; thread 0
// of the writer also resets the passes' unit counters. The tile table and
// sorted arrays must be visible to the calling threads.
__device__ inline void write_tile_records(const Perm& p, const float* slot_w, int i0, int stride) {
  const int n = *p.n_tiles * kRecInts;
  for (int i = i0; i < n; i += stride) {
    const int t = i / kRecInts, f = i - t * kRecInts;
    const int4 ti = p.tile_info[t];
    int v = 0;
    if (f == 0) {
      v = ti.x;
    } else if (f == 1) {
      v = ti.y;
    } else if (f == 2) {
      v = ti.z;
    } else if (f >= 4) {
      const int c = (f - 4) & 15, kind = (f - 4) >> 4;
      const int pos = ti.y + min(c, ti.z - 1);
      if (kind == 0) {
        v = p.sorted_tok[pos];
      } else {
        const int slot = p.sorted_slots[pos];
        v = kind == 1 ? slot : __float_as_int(slot_w[slot]);
      }
    }
    p.tile_rec[i] = v;
  }
  if (i0 == 0) {
    p.queues[0] = 0;
    p.queues[1] = 0;
  }
}

}  // namespace moe
