// Tile-level mask tests of the backward kernels, shared by the device code
// and a host check that brute-forces them over tile offsets.
//
// A backward kernel forms a tile's probabilities with the causal and tail
// mask only where the tile's queries and keys meet the causal diagonal or a
// sequence end; everywhere else it runs a copy of the weight loop without
// the per-element compare.  These wave-uniform tests decide which copy runs:
// they may say "masked" for a tile that needs no mask (that only costs time),
// never "unmasked" for a tile holding a score the row may not see.
#pragma once

#include <hip/hip_runtime.h>

namespace iaea {

// dQ kernel: the 32 keys k0 .. k0 + 31 against the wave's 32 query rows
// wq0 .. wq0 + 31 of a sequence of seq_len tokens.  Only rows inside the
// sequence are stored; every stored row sees at least the keys up to
// min(wq0, seq_len - 1) (causal) or seq_len - 1.
__host__ __device__ constexpr bool dq_half_tile_unmasked(bool causal, int wq0, int k0, int seq_len) {
  return (causal ? (wq0 < seq_len - 1 ? wq0 : seq_len - 1) : seq_len - 1) >= k0 + 31;
}

// dK/dV kernels: the 32 queries qb0 .. qb0 + 31 against the wave's 32 keys
// wk0 .. wk0 + 31.  Every one of these queries feeds the keys' gradient sums,
// so all of them must lie inside the sequence, as must the keys, and under
// the causal mask the first query must come no earlier than the last key.
__host__ __device__ constexpr bool dkdv_half_tile_unmasked(bool causal, int qb0, int wk0, int seq_len) {
  return (!causal || qb0 >= wk0 + 31) && qb0 + 32 <= seq_len && wk0 + 32 <= seq_len;
}

}  // namespace iaea
