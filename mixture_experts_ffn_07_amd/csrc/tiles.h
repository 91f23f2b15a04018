// Work-item order shared by the grouped GEMMs of the batched path.
#pragma once

namespace moe {

constexpr int kXcds = 8;   // workgroups are dispatched to the 8 XCDs round-robin by linear id

// Item L of a 1-D grid (dispatched to XCD L % 8) takes the (L % 8)-th eighth
// of the item space, so consecutive items - the N-blocks of one M-tile - share
// an XCD and its L2.  n_items must be a multiple of 8.
__device__ __forceinline__ int xcd_item(int L, int n_items) {
  return (L % kXcds) * (n_items / kXcds) + L / kXcds;
}

// The grid is sized for the most M-tiles any routing can produce; the real
// count is known on the device only.  Workgroups past the real items exit,
// and the XCD remap runs over the real item space so every XCD gets an equal
// share.  Returns -1 for a workgroup with nothing to do.
__device__ __forceinline__ int real_item(int L, int nblk, int n_tiles) {
  const int n_real = (nblk * n_tiles + kXcds - 1) / kXcds * kXcds;
  if (L >= n_real) return -1;
  const int item = xcd_item(L, n_real);
  return item / nblk < n_tiles ? item : -1;
}

}  // namespace moe
