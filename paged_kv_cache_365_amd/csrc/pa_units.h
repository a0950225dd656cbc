// Work-unit numbering of the decode launches (one-dimensional grids).
//
// Plain integer arithmetic with no HIP dependency: the decode kernel calls it
// on the device, and tests/unit_of_check.cpp compiles this header for the host
// (defining PA_UNITS_FN) to check that the numbering is a permutation.
#pragma once

#ifndef PA_UNITS_FN
#define PA_UNITS_FN __host__ __device__ __forceinline__
#endif

namespace pa {

// Work unit of a workgroup.  The grid is one-dimensional; units are numbered
// sibling-fastest, then partition, KV head, sequence: n = ((s * H_kv + g) *
// parts + p) * wgs + w, where the wgs siblings w split the rows of one
// (s, g, p) and read the same K/V tiles.  Workgroups are handed to the 8 XCDs
// round-robin (workgroup i to XCD i mod 8), and each XCD has its own L2, so
// when there are siblings the ids are permuted to put all siblings of a unit
// on one XCD, dispatched back to back: the tiles the first one brings into
// that L2 serve the others.  Without siblings the numbering is the identity.
struct Unit {
  int sibling, part, kv_head, seq;
};

PA_UNITS_FN Unit unit_of(int id, int total, int wgs, int parts, int kv_heads) {
  constexpr int kXcds = 8;
  int n = id;
  if (wgs > 1) {
    const int span = kXcds * wgs;
    const int whole = total / span * span;  // the tail past whole multiples keeps its ids
    if (id < whole) {
      const int xcd = id % kXcds;
      const int slot = id / kXcds;  // position in this XCD's dispatch order
      n = ((slot / wgs) * kXcds + xcd) * wgs + slot % wgs;
    }
  }
  Unit u;
  u.sibling = n % wgs;
  n /= wgs;
  u.part = n % parts;
  n /= parts;
  u.kv_head = n % kv_heads;
  u.seq = n / kv_heads;
  return u;
}

}  // namespace pa
