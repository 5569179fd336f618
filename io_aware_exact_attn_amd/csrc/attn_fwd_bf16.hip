// bf16 exact attention forward for gfx950 (MI355X).
//
// One workgroup owns BM = 256 query rows (8 waves of 32) of one (sequence,
// head) and streams that head's keys and values through LDS in tiles of 64
// rows: query blocks are the outer (parallel) loop, key/value blocks the
// inner loop, the order of the FlashAttention-2 part of "FlashAttention,
// pelatihan multi-GPU, dan kuantisasi bobot" (section 1).  Per query row the
// kernel keeps the running maximum m, the normaliser l and the weighted value
// sum u of the section "Softmax qua nhiều khối cần thống kê chạy" of "Flash
// Attention và IO"; when m moves to m_new the old l and u are scaled by
// exp(m - m_new).  The division u / l happens once, after the last tile (the
// deferred rescale of the FlashAttention-2 part).  Scores and probabilities
// live only in registers.
//
// MI355X mapping
//  * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16: with keys and
//    d on the MFMA rows, every lane owns one query column, so the softmax
//    needs no cross-lane reduction except an exchange between lanes l and
//    l ^ 32 for the rare rescale and at the end.
//  * Two wave groups ping-pong on each SIMD (waves w and w + 4 share one):
//    every wave alternates a matrix phase (MFMAs and LDS reads) with a
//    softmax phase (VALU only), one group a phase behind the other, so one
//    wave of each SIMD drives the matrix cores while the other drives the
//    VALU.  A workgroup barrier ends every phase.
//  * Q stays in VGPRs for the whole loop.  K and V tiles go from HBM straight
//    to double-buffered LDS with buffer_load_dwordx4 ... lds (1 KB per
//    instruction); the buffer size stops at the end of the sequence, so rows
//    past it read as zeros.  V^T fragments come from ds_read_b64_tr_b16.
//  * LDS rows are XOR-swizzled in 16-byte granules so both the K fragment
//    reads and the transposed V reads are free of bank conflicts.
//  * Causal: tiles above the diagonal are never loaded or computed, and
//    workgroups are issued longest first across all heads (the dispatcher
//    then balances the CUs like a longest-first list schedule), with each
//    head kept on one XCD (L2).
#include "attn_common.h"
#include "attn_kernels.h"


namespace iaea {

template <int P> using Parity = std::integral_constant<int, P>;

// Compile-time shape of a kernel instance: head dimension D and how many
// MFMA steps ahead of its use an LDS operand fragment is read.
template <int D_, int PF_ = 3>
struct BfCfg {
  static constexpr int D = D_, PF = PF_;
  static constexpr int NW = 8;       // waves per workgroup: two groups of one wave per SIMD
};

// A lane whose weights of a tile sum to at most kLazyMax has no weight above
// it, so the reference maximum only moves when some lane's sum exceeds it (or
// a weight overflows to inf).  u / l does not depend on the reference, so this
// is exact up to rounding; bf16 and fp32 keep the same relative precision at
// any magnitude.  The bound only limits range: with weights <= 2^64 the fp32
// sums l and u stay finite while N * max|v| stays below 2^68.
constexpr float kLazyMax = 0x1p64;

template <class Cfg, bool CAUSAL, bool PACKED, bool OUT_F32>
__global__ void __launch_bounds__(Cfg::NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
attn_fwd_bf16_kernel(FwdArgs a) {
  constexpr int D = Cfg::D, NW = Cfg::NW, PF = Cfg::PF;
  constexpr int BN = 64;                 // keys per tile
  constexpr int BM = 32 * NW;            // query rows per workgroup
  constexpr int ROWB = D * 2;            // bytes of one K/V row
  constexpr int TILE = BN * ROWB;        // bytes of one K or V tile
  constexpr int LW = NW / 2;             // waves that issue the tile loads (the second group)
  constexpr int CPW = TILE / 1024 / LW;  // 1 KB load chunks per loading wave per tile
  constexpr int DC = D / 16;             // k-steps of the QK^T MFMA
  constexpr int DB = D / 32;             // 32-wide blocks of d in O
  constexpr int NQK = 2 * DC;            // QK^T MFMAs per tile and wave
  constexpr int NPV = 4 * DB;            // P.V MFMAs per tile and wave
  constexpr int NS = NQK + NPV;          // MFMA steps of a tile
  static_assert(CPW * LW * 1024 == TILE, "tile must split into whole 1 KB chunks per wave");
  static_assert(PF >= 1 && PF < NS, "fragment prefetch distance");

  // K(j) lives in buffer j % 2, V(j) in buffer 2 + j % 2
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];

  int h, b, seq_start, seq_len, qblk;
  if (!decode_work<BM, CAUSAL, PACKED>(a, blockIdx.x, h, b,
                                       seq_start, seq_len, qblk))
    return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool lag = wave >= NW / 2;       // the second group, one phase behind
  const int hl = lane >> 5;              // which half of the wave
  const int l32 = lane & 31;
  const int q0 = qblk * BM;
  const int wq0 = q0 + wave * 32;        // first query row of this wave
  const int kv_end = CAUSAL ? min(seq_len, q0 + BM) : seq_len;
  const int n_iter = (kv_end + BN - 1) / BN;
  const int wave_kv_end = CAUSAL ? min(seq_len, wq0 + 32) : seq_len;
  const int wave_iters = (wq0 < seq_len) ? (wave_kv_end + BN - 1) / BN : 0;

  const int64_t rs = (int64_t)a.H * D;   // elements between consecutive tokens
  const int64_t head_off = (int64_t)h * D;
  const uint16_t* __restrict__ qg = (const uint16_t*)a.q;
  const uint16_t* __restrict__ kg = (const uint16_t*)a.k;
  const uint16_t* __restrict__ vg = (const uint16_t*)a.v;
  const float c = a.c;

  // ---- Q fragments (MFMA B operand of S^T = K Q^T), kept for the whole loop
  bf16x8 qf[DC];
  {
    const int t = wq0 + l32;
    const bool ok = t < seq_len;
    const uint16_t* p = qg + (int64_t)(seq_start + (ok ? t : 0)) * rs + head_off + 8 * hl;
    // rows past the end read row 0 and are zeroed: the loads stay
    // unconditional, so they issue together with the tile loads below
    const uint32_t keep = ok ? 0xffffffffu : 0u;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      u32x4 raw = *(const u32x4*)(p + dc * 16);
      raw &= keep;
      raw ^= a.qsign;
      qf[dc] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // ---- K/V tiles: HBM -> LDS directly (buffer_load_dwordx4 ... lds).  Lane
  // i of a wave writes LDS bytes [chunk + 16 i, chunk + 16 i + 16); it fetches
  // the logical granule that the swizzle places there.  The per-lane byte
  // offset inside a tile is loop-invariant; the tile base is wave-uniform.  The
  // buffer's size ends at the end of the sequence, so rows past it read as
  // zeros (those keys are masked and their weights are 0).
  const int lw = wave % LW;              // this wave's share of a tile
  uint32_t lane_off[CPW];
#pragma unroll
  for (int cc = 0; cc < CPW; ++cc) {
    const int byte = (lw * CPW + cc) * 1024 + lane * 16;
    const int row = byte / ROWB;
    const int g = ((byte % ROWB) >> 4) ^ swz<D>(row);
    lane_off[cc] = (uint32_t)(((int64_t)row * rs + head_off + g * 8) * 2);
  }
  // bytes of one token row of all heads; the host keeps BN rows under 2^32 bytes
  [[maybe_unused]] const uint32_t row_bytes = (uint32_t)rs * 2u;
  auto issue_tile = [&](const uint16_t* __restrict__ src, int buf, int j) __attribute__((always_inline)) {
#if __HIP_DEVICE_COMPILE__   // the 16-byte LDS DMA form exists only for the device target
    const int kv0 = j * BN;
    const uint32_t nrec = (uint32_t)min(seq_len - kv0, BN) * row_bytes;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const char*)src + (uint64_t)(uint32_t)(seq_start + kv0) * row_bytes), (short)0, (int)nrec,
        kBufferFlags);
    // one LDS base (M0) for all chunks: chunk cc's 1 KB step rides in the
    // instruction offset, which applies to the LDS and the memory address
    // alike, so the memory offset gives it back (lane_off[cc] >= cc * 1 KB,
    // since a token row in memory is at least as long as one in the tile)
    static_for<CPW>([&](auto ci) __attribute__((always_inline)) {
      constexpr int cc = decltype(ci)::value;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (IAEA_LDS void*)(smem + buf * TILE + lw * CPW * 1024),
                                               16, lane_off[cc] - cc * 1024, 0, cc * 1024, 0);
    });
#endif
  };

  // ---- loop-invariant LDS read offsets; buffer bases and the steps over key
  // blocks are compile-time immediates.  K fragment (A operand of S^T): row
  // kb * 32 + l32, granule 2 * dc + hl.  V^T fragment (ds_read_b64_tr_b16): in
  // each 16-lane group, source lane s points at key row 4 * half + s / 4 (and
  // + 8 for the upper four keys) and d offset 4 * (s % 4) of the group's 16 d
  // columns; lane i then holds d column i of four consecutive keys.  The
  // swizzle repeats every 16 rows, so whole 16-row steps stay immediates.
  uint32_t koff[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) koff[dc] = l32 * ROWB + (((2 * dc + hl) ^ swz<D>(l32)) << 4);
  uint32_t voff[2][DB];
  {
    const int g16 = lane >> 4;
    const int v_row = 4 * (g16 >> 1) + ((lane & 15) >> 2);
    const int v_dcol = 16 * (g16 & 1) + 4 * (lane & 3);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int row = v_row + 8 * hi;
        const int d = db * 32 + v_dcol;
        voff[hi][db] = row * ROWB + (((d >> 3) ^ swz<D>(row)) << 4) + (d & 7) * 2;
      }
  }

  // The MFMA steps of the matrix phase of tile j, in issue order.  Steps
  // [0, NQK) compute S^T(j + 1) = K(j + 1) Q^T, alternating between the two
  // 32-key halves so consecutive MFMAs are independent; steps [NQK, NS) add
  // V(j)^T P(j)^T to O^T, 16 keys (chunk kc) at a time.  frag<P, s>() reads
  // step s's LDS operand for a tile of parity P (K(j + 1) in buffer P ^ 1,
  // V(j) in buffer 2 + P).
  auto frag = [&](auto par, auto step) __attribute__((always_inline)) -> bf16x8 {
    constexpr int P = decltype(par)::value, s = decltype(step)::value;
    if constexpr (s < NQK) {
      constexpr int kb = s & 1, dc = s >> 1;
      return *(const bf16x8*)(smem + (P ^ 1) * TILE + kb * 32 * ROWB + koff[dc]);
    } else {
      constexpr int kc = (s - NQK) / DB, db = (s - NQK) % DB;
      const char* vt = smem + (2 + P) * TILE + kc * 16 * ROWB;
      const bf16x4 lo = ds_read_tr16(vt + voff[0][db]);
      const bf16x4 hi = ds_read_tr16(vt + voff[1][db]);
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };

  // ---- running state
  // m_run: reference maximum of the row (raw score units); lx_run: this lane's
  // sum of the weights (half of the row's keys); oacc: u^T; lacc: l, the sum of
  // the bf16-rounded weights that enter P.V (see the row-sum MFMA below).
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = (f32x16){};
  float m_run = -INFINITY, lx_run = 0.f;
  f32x4 lacc = {0.f, 0.f, 0.f, 0.f};
  f32x16 negm;                           // -m_run in every register: the score MFMA's start value
  f32x16 sc[2];                          // S^T of the current tile (two 32-key halves)
  bf16x8 pf[4];                          // P^T of the current tile, four 16-key chunks

  // The row sums come from v_mfma_f32_16x16x32_bf16 with a 0/1 selector as
  // the A operand: in a P fragment lanes n and n + 32 hold query n and lanes
  // n + 16 and n + 48 query n + 16, so rows 0-7 of the selector pick k-groups
  // 0 and 2 and rows 8-15 k-groups 1 and 3.  Result lane i then holds query i
  // (i < 16), i - 16 (16 <= i < 48) or i - 32 (i >= 48).
  bf16x8 lsel;
  {
    const __bf16 one = ((lane & 15) < 8) == (((lane >> 4) & 1) == 0) ? (__bf16)1.0f : (__bf16)0.0f;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) lsel[jj] = one;
  }
  const bool lacc_swapped = lane >= 16 && lane < 48;
  const float inv_c = 1.f / c;

  // ---- prologue: K(0), K(1) (first group) and V(0) (second group)
  // resident, S(0) computed from 0 (every wave)
  if (n_iter > 0) {
    if (!lag) {
      issue_tile(kg, 0, 0);
      if (n_iter > 1) issue_tile(kg, 1, 1);
    } else {
      issue_tile(vg, 2, 0);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (wave_iters > 0) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const bf16x8 kf = *(const bf16x8*)(smem + kb * 32 * ROWB + koff[dc]);
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[dc], dc == 0 ? (f32x16){} : sc[kb], 0, 0, 0);
      }
  }
  __syncthreads();   // every wave has read K(0) before K(2) replaces it

  // Weights exp2(s' c - shift_c) of the tile into pf, where s' = s - m_run
  // (the score MFMAs start from -m_run); returns this lane's sum of them.
  auto weights = [&](float shift_c, bool fused) __attribute__((always_inline)) -> float {
    float x0 = 0.f, x1 = 0.f;
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      // registers 8 c2 .. 8 c2 + 7 of the kb half: keys of chunk ch
      const int kb = ch / 2, c2 = ch % 2;
      u32x4 w;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float s0 = sc[kb][8 * c2 + 2 * jj], s1 = sc[kb][8 * c2 + 2 * jj + 1];
        const float e0 = fast_exp2(fused ? __builtin_fmaf(s0, c, -shift_c) : s0 * c);
        const float e1 = fast_exp2(fused ? __builtin_fmaf(s1, c, -shift_c) : s1 * c);
        w[jj] = pack_bf16x2(e0, e1);
        if (jj & 1) x1 += e0 + e1;
        else        x0 += e0 + e1;
      }
      pf[ch] = __builtin_bit_cast(bf16x8, w);
    }
    return x0 + x1;
  };

  // Softmax phase Y(j).  The score MFMAs start from -m, so tile j arrives as
  // s - m and its weight is exp2((s - m) c) with one multiply; the tile's row
  // maximum is not needed to form the weights.  Only when some lane's weights
  // sum to more than kLazyMax (and on a row's first tile, whose scores were
  // computed from 0) does the wave take the maximum, move the reference to it,
  // scale the running state by exp(m - m_new) and form the weights again -
  // before P(j) enters P.V in X(j).  The second group issues the loads of
  // K(j + 2) and V(j + 1) here, where they share issue slots with VALU work.
  auto phase_y = [&](auto par, int j) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    if (lag) {
      if (j + 2 < n_iter) issue_tile(kg, P, j + 2);          // into the buffer of K(j)
      if (j + 1 < n_iter) issue_tile(vg, 2 + (P ^ 1), j + 1);  // into the buffer of V(j - 1)
    }
    if (j < wave_iters) {
      const int kv0 = j * BN;
      // keys past the end of the sequence and, when causal, future keys get
      // -inf; the key of register r is kv0 + kb*32 + (r/4)*8 + half*4 + r%4
      if ((kv0 + BN > seq_len) || (CAUSAL && kv0 + BN - 1 > wq0)) {
        const int lim = (CAUSAL ? min(wq0 + l32, seq_len - 1) : seq_len - 1) - (kv0 + hl * 4);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kb * 32 + (r >> 2) * 8 + (r & 3) > lim) sc[kb][r] = -INFINITY;
      }
      // a row's first tile (the same tile for every lane of the wave) goes
      // straight to the maximum; later tiles form their weights first
      const bool first = m_run == -INFINITY;
      float lx = 0.f;
      if (!first) lx = weights(0.f, false);
      if (__ballot(first || lx > kLazyMax) != 0) {
        float m = fmaxf(sc[0][0], sc[1][0]);
#pragma unroll
        for (int r = 1; r < 16; ++r) m = fmaxf(m, fmaxf(sc[0][r], sc[1][r]));
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
        const float mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        if (first) {
          // S(0) was computed from 0: the reference becomes the row maximum
          m_run = mx;
          lx = weights(mx * c, true);
        } else {
          // scores are relative to m_run; this lane's reference moves up by
          // mc = max(mx, 0) c exp2 units
          const float mc = fmaxf(mx, 0.f) * c;
          float alpha;
          if (__ballot(mc > 119.f) != 0) {
            // a large move, whose weights may have overflowed: shift by
            // exactly mc and form them again
            alpha = fast_exp2(-mc);
            m_run += fmaxf(mx, 0.f);
            lx = weights(mc, true);
          } else {
            // a small move by a whole number k of exp2 units: the running
            // state scales by exactly 2^-k, and so do this tile's bf16
            // weights, k coming off their exponent fields (a weight that
            // would drop below the smallest normal bf16 becomes 0)
            const float kf = ceilf(mc);
            alpha = __builtin_amdgcn_ldexpf(1.f, -(int)kf);
            m_run = __builtin_fmaf(kf, inv_c, m_run);
            const unsigned short dk = (unsigned short)((int)kf << 7);
            const u16x8 dk8 = {dk, dk, dk, dk, dk, dk, dk, dk};
#pragma unroll
            for (int ch = 0; ch < 4; ++ch)
              pf[ch] = __builtin_bit_cast(bf16x8, __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x8, pf[ch]), dk8));
            lx *= alpha;
          }
          lx_run *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
          // lacc lane i holds the query of lane i ^ 16 for 16 <= i < 48 (its
          // own otherwise); the 16-lane swap hands every lane the alpha of
          // lane i ^ 16 as one of its two results, the one that is not its own
          const auto a16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(alpha), __float_as_uint(alpha),
                                                            false, false);
          const float partner = __uint_as_float(a16[0] == __float_as_uint(alpha) ? a16[1] : a16[0]);
          lacc *= lacc_swapped ? partner : alpha;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) negm[r] = -m_run;
      }
      lx_run += lx;
    }
    // a bare s_barrier: __syncthreads() would also wait here for the tile
    // loads just issued, which are waited for at the end of X(j) instead.
    // The memory clobber keeps LDS accesses on their side of it.
    asm volatile("s_barrier" ::: "memory");
  };

  // Matrix phase X(j): S(j + 1) into sc, O^T += V(j)^T P(j)^T, l += row sums
  // of P(j).  MFMAs and LDS reads only; operand fragments are read PF steps
  // ahead of their MFMA.  The second group waits here for the tile loads it
  // issued in Y(j).
  auto phase_x = [&](auto par, int j) __attribute__((always_inline)) {
    if (j < wave_iters) {
      bf16x8 fr[PF + 1];
      static_for<PF>([&](auto step) __attribute__((always_inline)) {
        fr[decltype(step)::value] = frag(par, step);
      });
      static_for<NS>([&](auto step) __attribute__((always_inline)) {
        constexpr int s = decltype(step)::value;
        if constexpr (s + PF < NS) fr[(s + PF) % (PF + 1)] = frag(par, std::integral_constant<int, s + PF>{});
        if constexpr (s < NQK) {
          constexpr int kb = s & 1, dc = s >> 1;
          sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[s % (PF + 1)], qf[dc],
                                                           dc == 0 ? negm : sc[kb], 0, 0, 0);
        } else {
          constexpr int kc = (s - NQK) / DB, db = (s - NQK) % DB;
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[s % (PF + 1)], pf[kc], oacc[db], 0, 0, 0);
          if constexpr (db == DB - 1)
            lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lsel, pf[kc], lacc, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    if (lag) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  // Phase schedule.  The first group runs Y(0) X(0) Y(1) X(1) ...; the second
  // group runs the same one phase later.  In the phase where the first group
  // runs X(j) the second runs Y(j) and issues K(j + 2) and V(j + 1); their
  // buffers held K(j) and V(j - 1), last read in the phase before (X(j - 1)
  // of the second group).  They are waited for at the end of the second
  // group's X(j), one phase before the first group's X(j + 1) reads them.
  if (lag) __syncthreads();
  for (int j = 0; j < n_iter; j += 2) {
    phase_y(Parity<0>{}, j);
    phase_x(Parity<0>{}, j);
    if (j + 1 < n_iter) {
      phase_y(Parity<1>{}, j + 1);
      phase_x(Parity<1>{}, j + 1);
    }
  }
  if (!lag) __syncthreads();

  // ---- epilogue: O = u / l, LSE = ln2 * (m * c + log2 lx)
  // l of this lane's query i % 32 sits in lacc of lane i + 16 (16 <= i < 32),
  // i - 32 (32 <= i < 48) or i itself
  const int lsrc = (lane >= 16 && lane < 32) ? lane + 16 : (lane >= 32 && lane < 48) ? lane - 32 : lane;
  const float l_tot = __shfl(lacc[0], lsrc);
  const auto swx = __builtin_amdgcn_permlane32_swap(__float_as_uint(lx_run), __float_as_uint(lx_run), false, false);
  const float lx_tot = __uint_as_float(swx[0]) + __uint_as_float(swx[1]);
  const int64_t lse_base = PACKED ? ((int64_t)h * a.N + seq_start) : ((int64_t)(b * a.H + h) * a.N);
  const int t = wq0 + l32;
  const bool any = l_tot > 0.f;
  const float inv = any ? 1.f / l_tot : 0.f;
  if (t < seq_len && hl == 0) a.lse[lse_base + t] = any ? kLn2 * (m_run * c + __log2f(lx_tot)) : -INFINITY;
  if constexpr (OUT_F32) {
    if (t < seq_len) {
      const int64_t orow = (int64_t)(seq_start + t) * rs + head_off;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = db * 32 + g * 8 + hl * 4;
          *(f32x4*)((float*)a.o + orow + d) = (f32x4){oacc[db][g * 4 + 0] * inv, oacc[db][g * 4 + 1] * inv,
                                                      oacc[db][g * 4 + 2] * inv, oacc[db][g * 4 + 3] * inv};
        }
    }
  } else {
    // bf16 O goes out through LDS (free after the last barrier): each wave
    // writes its 32 rows into its own slice, then reads them back in row
    // order, so every global store covers whole 16-byte pieces of
    // consecutive rows.  A row's 16-byte granules are XOR-swizzled by the row
    // and its two 8-byte halves swapped on odd multiples of NG rows, so the
    // 8-byte writes of the 32 rows spread over all banks.
    constexpr int NG = ROWB / 16;              // 16-byte granules per row
    char* slice = smem + wave * 32 * ROWB;
    const int wflip = (l32 / NG) & 1;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int G = db * 4 + g;
        *(u32x2*)(slice + l32 * ROWB + ((G ^ (l32 & (NG - 1))) << 4) + ((hl ^ wflip) << 3)) =
            (u32x2){pack_bf16x2(oacc[db][g * 4 + 0] * inv, oacc[db][g * 4 + 1] * inv),
                    pack_bf16x2(oacc[db][g * 4 + 2] * inv, oacc[db][g * 4 + 3] * inv)};
      }
#pragma unroll
    for (int k = 0; k < 32 * NG / 64; ++k) {
      const int cidx = k * 64 + lane;
      const int row = cidx / NG, G = cidx % NG;
      const u32x4 x = *(const u32x4*)(slice + row * ROWB + ((G ^ (row & (NG - 1))) << 4));
      const bool flip = (row / NG) & 1;
      const u32x4 y = flip ? (u32x4){x[2], x[3], x[0], x[1]} : x;
      if (wq0 + row < seq_len)
        *(u32x4*)((uint16_t*)a.o + (int64_t)(seq_start + wq0 + row) * rs + head_off + G * 8) = y;
    }
  }
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------

template <class Cfg, bool CAUSAL, bool PACKED, bool OUT_F32>
static hipError_t launch_one(FwdArgs a, hipStream_t st) {
  constexpr int NW = Cfg::NW;
  constexpr int BM = 32 * NW;
  if (PACKED) {
    a.slots = (a.N + BM - 1) / BM + a.B;
    a.n_work = a.H * a.slots;
  } else {
    a.slots = (a.N + BM - 1) / BM;
    a.n_work = a.B * a.H * a.slots;
  }
  const int grid = (a.n_work + kXcds - 1) / kXcds * kXcds;
  a.per_xcd = grid / kXcds;
  void* args[] = {&a};
  // the launch's own status (hipGetLastError could report an earlier, unrelated call)
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_bf16_kernel<Cfg, CAUSAL, PACKED, OUT_F32>),
                         dim3(grid), dim3(NW * 64), args, 0, st);
}

// Kernel instance per head dimension.
template <int D> struct BfTile { using Cfg = BfCfg<D, 3>; };

template <int D, bool CAUSAL, bool PACKED>
static hipError_t launch_d(const FwdArgs& a, bool out_f32, hipStream_t st) {
  using Cfg = typename BfTile<D>::Cfg;
  return out_f32 ? launch_one<Cfg, CAUSAL, PACKED, true>(a, st)
                 : launch_one<Cfg, CAUSAL, PACKED, false>(a, st);
}

hipError_t launch_attn_fwd_bf16(const FwdArgs& a, int d, bool causal, bool packed, bool out_f32,
                                hipStream_t st) {
  if (d == 128) {
    if (causal) return packed ? launch_d<128, true, true>(a, out_f32, st) : launch_d<128, true, false>(a, out_f32, st);
    return packed ? launch_d<128, false, true>(a, out_f32, st) : launch_d<128, false, false>(a, out_f32, st);
  }
  if (causal) return packed ? launch_d<64, true, true>(a, out_f32, st) : launch_d<64, true, false>(a, out_f32, st);
  return packed ? launch_d<64, false, true>(a, out_f32, st) : launch_d<64, false, false>(a, out_f32, st);
}

int bf16_rows_per_workgroup(int d) {
  return d == 128 ? 32 * BfTile<128>::Cfg::NW : 32 * BfTile<64>::Cfg::NW;
}

}  // namespace iaea
