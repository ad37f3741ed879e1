// prefill_sched.hpp -- work items and the K tile row order shared by the causal prefill
// kernels (gfx950).
//
// A work item is 128 query rows (BR) of one (b, h). A persistent workgroup takes the items at
// positions j, 2W - 1 - j, 2W + j, ... of its class's list (the snake order), which lists the
// query blocks longest first, so that every workgroup gets about the same number of tiles.
// With B*H a multiple of 8 the classes are the heads with bh % 8 == x % 8 for workgroup x
// (dispatched to XCD x % 8), so each head's K and V are read through one XCD's L2.
#pragma once

#include "plx_device.hpp"

namespace plx {
namespace prefill {

constexpr int BR = 128;  // query rows per work item

// K row of key k of a tile: inside each 32-key group, key 8 q + 4 b + i goes to row
// 16 b + 4 q + i (bits 2 and 3 of the index swapped), so that the score accumulators of each
// lane hold the 8 consecutive keys that the value product's operand wants.
__device__ __forceinline__ int krow(int k) {
    return (k & ~31) | (((k >> 2) & 1) << 4) | (((k >> 3) & 3) << 2) | (k & 3);
}

// Key stored at K row r (the inverse of krow).
__device__ __forceinline__ int krow_inv(int r) {
    return (r & ~31) | (((r >> 2) & 3) << 3) | (((r >> 4) & 1) << 2) | (r & 3);
}

__device__ __forceinline__ int item_position(int kk, int j, int Wc) {
    return kk * Wc + ((kk & 1) ? Wc - 1 - j : j);
}

struct Item {
    int bh, q0, ntiles, nfull;  // ntiles key tiles of BC keys; the first nfull need no mask
};

template <int BC>
__device__ __forceinline__ Item item_at(int pos, int cls, int ncls, int nbh_c, int nqb, int T) {
    Item it;
    const int qb = nqb - 1 - pos / nbh_c;
    it.bh = cls + ncls * (pos % nbh_c);
    it.q0 = qb * BR;
    const int kend = min(it.q0 + BR, T);
    it.ntiles = (kend + BC - 1) / BC;
    it.nfull = min(it.ntiles, it.q0 / BC);
    return it;
}

}  // namespace prefill
}  // namespace plx
