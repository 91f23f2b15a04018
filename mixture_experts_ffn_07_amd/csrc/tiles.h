// Work-item order shared by the grouped GEMMs of the batched path.
#pragma once

#include <stdint.h>

namespace moe {

// Test permutation of a kernel's work items (MOE_DEBUG_PERMUTE_ORDER): with
// key 0 item i stays i; otherwise item i of n becomes (a*i + key) mod n, where
// a is one of four primes above 2^29 picked by the key, so a is coprime to any
// n below 2^29 and the map is a bijection.  The kernels apply it on top of
// their own workgroup -> item order, so a different workgroup computes each
// item; a result that depended on which workgroup (or in which order) items
// run would change.
__device__ __forceinline__ int permute_item(int i, int n, uint32_t key) {
  if (key == 0 || n <= 1) return i;
  const uint32_t a = (key & 6) == 0 ? 2147483647u : (key & 6) == 2 ? 1000000007u
                   : (key & 6) == 4 ? 998244353u : 1000000009u;
  return static_cast<int>((static_cast<uint64_t>(a) * static_cast<uint32_t>(i) + key) %
                          static_cast<uint32_t>(n));
}

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
