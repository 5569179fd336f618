// Host check of the backward kernels' tile mask tests (attn_mask.h, the
// header the kernels include): by brute force over sequence lengths and tile
// offsets, whenever a test picks the unmasked weight loop, every score that
// loop keeps must be visible - query and key inside the sequence and, when
// causal, the key no later than the query.  dK/dV: all 32 queries of the half
// tile feed the sums; dQ: only the stored rows (inside the sequence) count.
// Prints how often each test took the unmasked path; exits 1 on a violation.
#include <cstdio>

#include "attn_mask.h"

static bool visible(bool causal, int q, int k, int n) { return q < n && k < n && (!causal || k <= q); }

int main() {
  const int lens[] = {1, 31, 32, 33, 63, 64, 65, 96, 127, 128, 129, 200, 256, 300, 1000};
  long taken_dkdv = 0, taken_dq = 0, bad = 0;
  for (int causal = 0; causal < 2; ++causal)
    for (int n : lens) {
      const int tiles = (n + 63) / 64;
      // dK/dV: 64-query tile j, its 32-query half, the wave's 32 keys at wk0
      for (int j = 0; j < tiles; ++j)
        for (int half = 0; half < 2; ++half)
          for (int wk0 = 0; wk0 < n; wk0 += 32) {
            const int qb0 = j * 64 + half * 32;
            if (!iaea::dkdv_half_tile_unmasked(causal, qb0, wk0, n)) continue;
            ++taken_dkdv;
            for (int q = qb0; q < qb0 + 32; ++q)
              for (int k = wk0; k < wk0 + 32; ++k)
                if (!visible(causal, q, k, n)) {
                  if (bad++ < 10) std::printf("dkdv: n %d causal %d q0 %d k0 %d: q %d k %d\n", n, causal, qb0, wk0, q, k);
                }
          }
      // dQ: the wave's 32 queries at wq0, 64-key tile j, its 32-key half
      for (int wq0 = 0; wq0 < n; wq0 += 32)
        for (int j = 0; j < tiles; ++j)
          for (int kb = 0; kb < 2; ++kb) {
            const int k0 = j * 64 + kb * 32;
            if (!iaea::dq_half_tile_unmasked(causal, wq0, k0, n)) continue;
            ++taken_dq;
            for (int q = wq0; q < wq0 + 32 && q < n; ++q)
              for (int k = k0; k < k0 + 32; ++k)
                if (!visible(causal, q, k, n)) {
                  if (bad++ < 10) std::printf("dq: n %d causal %d q0 %d k0 %d: q %d k %d\n", n, causal, wq0, k0, q, k);
                }
          }
    }
  // not vacuous: interior tiles of a long causal sequence skip the mask,
  // diagonal ones do not
  const bool interior = iaea::dkdv_half_tile_unmasked(true, 1024, 256, 16384) &&
                        iaea::dq_half_tile_unmasked(true, 1024, 256 + 32, 16384) &&
                        !iaea::dkdv_half_tile_unmasked(true, 256, 256, 16384) &&
                        !iaea::dq_half_tile_unmasked(true, 256, 256, 16384);
  std::printf("unmasked dkdv %ld dq %ld violations %ld interior %d\n", taken_dkdv, taken_dq, bad, (int)interior);
  return (bad == 0 && interior && taken_dkdv > 0 && taken_dq > 0) ? 0 : 1;
}
