// bf16 exact attention forward for gfx950 (MI355X).
//
// One workgroup owns BM = NW * 32 * QB query rows of one (sequence, head) and
// streams that head's keys and values through LDS in tiles of 64 rows: query
// blocks are the outer (parallel) loop, key/value blocks the inner loop, the
// order of the FlashAttention-2 part of "FlashAttention, pelatihan multi-GPU,
// dan kuantisasi bobot" (section 1).  Per query row the kernel keeps the
// running maximum m, the normaliser l and the weighted value sum u of the
// section "Softmax qua nhiều khối cần thống kê chạy" of "Flash Attention và
// IO"; a new tile with maximum m_b moves m to max(m, m_b), scales the old l
// and u by exp(m - m_new) and adds exp(s - m_new) and exp(s - m_new) * v.  The
// division u / l happens once, after the last tile (the deferred rescale of
// the FlashAttention-2 part).  Scores and probabilities live only in
// registers.
//
// MI355X mapping
//  * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16: with keys and
//    d on the MFMA rows, every lane owns one query column, so the row max,
//    the row sum, the rescale and the final 1/l are per-lane scalars, and the
//    only cross-lane step is one exchange between lanes l and l ^ 32.
//  * Q stays in VGPRs for the whole loop; K and V tiles are loaded with
//    128-bit coalesced global loads into double-buffered LDS (one barrier per
//    tile); V^T fragments come from ds_read_b64_tr_b16 transposed LDS reads.
//  * LDS rows are XOR-swizzled in 16-byte granules so both the K fragment
//    reads and the transposed V reads are free of bank conflicts.
//  * Causal: tiles above the diagonal are never loaded or computed, and
//    workgroups are issued heaviest first; the block -> tile mapping keeps
//    the workgroups of one head on one XCD (L2) at a time.
#include "attn_common.h"
#include "attn_kernels.h"

namespace iaea {

// 16-byte-granule XOR swizzle of an LDS row (see the file comment).
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

template <int D>
__device__ __forceinline__ int lds_off(int row, int granule) {
  return row * (D * 2) + ((granule ^ swz<D>(row)) << 4);
}

__device__ __forceinline__ bf16x4 ds_read_tr16(const char* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((IAEA_LDS s16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

// Compile-time shape of a kernel instance: head dimension D, query blocks of
// 32 rows per wave QB, waves per workgroup NW, the occupancy the register
// budget is sized for (waves per SIMD), and the instruction interleave.
// The running state is rescaled only when the running maximum grows by more
// than 2^kLazyLog2: u / l does not depend on the reference maximum, so this
// is exact up to rounding and only lets P reach 2^kLazyLog2.
template <int D_, int QB_, int NW_, int WPE_, bool SCHED_ = false, int VPM_ = 6>
struct BfCfg {
  static constexpr int D = D_, QB = QB_, NW = NW_, WPE = WPE_;
  static constexpr bool SCHED = SCHED_;   // hand interleaving of QK^T MFMAs and softmax VALU
  static constexpr int VPM = VPM_;        // VALU instructions per MFMA in that interleave
};

constexpr float kLazyLog2 = 8.f;

template <int P> struct Parity { static constexpr int value = P; };

template <class Cfg, bool CAUSAL, bool PACKED, bool OUT_F32>
__global__ void __launch_bounds__(Cfg::NW * 64) __attribute__((amdgpu_waves_per_eu(Cfg::WPE)))
attn_fwd_bf16_kernel(FwdArgs a) {
  constexpr int D = Cfg::D, QB = Cfg::QB, NW = Cfg::NW;
  constexpr int BN = 64;                 // keys per tile
  constexpr int QW = 32 * QB;            // query rows per wave
  constexpr int BM = QW * NW;            // query rows per workgroup
  constexpr int ROWB = D * 2;            // bytes of one K/V row
  constexpr int TILE = BN * ROWB;        // bytes of one K or V tile
  constexpr int CPW = TILE / 1024 / NW;  // 1 KB direct-load chunks per wave per tile
  constexpr int DC = D / 16;             // k-steps of the QK^T MFMA
  constexpr int DB = D / 32;             // 32-wide blocks of d in O
  static_assert(CPW * NW * 1024 == TILE, "tile must split into whole 1 KB chunks per wave");

  // K(j) lives in buffer j % 2, V(j) in buffer 2 + j % 2
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];

  int h, b, seq_start, seq_len, qblk;
  if (!decode_work<BM, CAUSAL, PACKED>(a, logical_block(blockIdx.x, a.per_xcd), h, b,
                                       seq_start, seq_len, qblk))
    return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5;              // which half of the wave
  const int l32 = lane & 31;
  const int q0 = qblk * BM;
  const int wq0 = q0 + wave * QW;        // first query row of this wave
  const int kv_end = CAUSAL ? min(seq_len, q0 + BM) : seq_len;
  const int n_iter = (kv_end + BN - 1) / BN;
  const int wave_kv_end = CAUSAL ? min(seq_len, wq0 + QW) : seq_len;
  const int wave_iters = (wq0 < seq_len) ? (wave_kv_end + BN - 1) / BN : 0;

  const int64_t rs = (int64_t)a.H * D;   // elements between consecutive tokens
  const int64_t head_off = (int64_t)h * D;
  const uint16_t* __restrict__ qg = (const uint16_t*)a.q;
  const uint16_t* __restrict__ kg = (const uint16_t*)a.k;
  const uint16_t* __restrict__ vg = (const uint16_t*)a.v;
  const float c = a.c;

  // ---- Q fragments (MFMA B operand of S^T = K Q^T), kept for the whole loop
  bf16x8 qf[QB][DC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int t = wq0 + qb * 32 + l32;
    const bool ok = t < seq_len;
    const uint16_t* p = qg + (int64_t)(seq_start + (ok ? t : 0)) * rs + head_off + 8 * hl;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      u32x4 raw = ok ? *(const u32x4*)(p + dc * 16) : (u32x4){0u, 0u, 0u, 0u};
      raw ^= a.qsign;
      qf[qb][dc] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // ---- K/V tiles: global -> LDS directly (global_load_lds_dwordx4).  Lane i of
  // a wave writes LDS bytes [chunk + 16 i, chunk + 16 i + 16); it fetches the
  // logical granule that the swizzle places there.  The per-lane byte offset
  // inside a tile is loop-invariant; the tile base is wave-uniform.  Rows past
  // the end of the sequence re-read its last row: those keys are masked and
  // their weights are 0.
  uint32_t lane_off[CPW];
  int lane_row[CPW];
#pragma unroll
  for (int cc = 0; cc < CPW; ++cc) {
    const int byte = (wave * CPW + cc) * 1024 + lane * 16;
    const int row = byte / ROWB;
    const int g = ((byte % ROWB) >> 4) ^ swz<D>(row);
    lane_row[cc] = row;
    lane_off[cc] = (uint32_t)(((int64_t)row * rs + head_off + g * 8) * 2);
  }
  auto issue_tile = [&](const uint16_t* __restrict__ src, int buf, int j) {
    const int kv0 = j * BN;
    const char* base = (const char*)(src + (int64_t)(seq_start + kv0) * rs);
    char* dst = smem + buf * TILE + wave * CPW * 1024;
    if (kv0 + BN <= seq_len) {
#pragma unroll
      for (int cc = 0; cc < CPW; ++cc)
        __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(base + lane_off[cc]),
                                         (IAEA_LDS void*)(dst + cc * 1024), 16, 0, 0);
    } else {
#pragma unroll
      for (int cc = 0; cc < CPW; ++cc) {
        const int over = max(0, kv0 + lane_row[cc] - (seq_len - 1));
        const uint32_t off = lane_off[cc] - (uint32_t)((int64_t)over * rs * 2);
        __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(base + off),
                                         (IAEA_LDS void*)(dst + cc * 1024), 16, 0, 0);
      }
    }
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

  auto qk = [&](auto kbuf_tag, f32x16 (&s)[QB][2]) {
    constexpr int KB = decltype(kbuf_tag)::value;
    const char* kt = smem + KB * TILE;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const bf16x8 kf = *(const bf16x8*)(kt + kb * 32 * ROWB + koff[dc]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              kf, qf[qb][dc], dc == 0 ? (f32x16){} : s[qb][kb], 0, 0, 0);
      }
    }
  };

  f32x16 oacc[QB][DB];
  float m_run[QB], l_run[QB], lx_run[QB];   // reference max, rounded and exact sums
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
    lx_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[qb][db] = (f32x16){};
  }

  // P = exp2(s * c - ms) for one 32-query block, rounded to bf16 and packed as
  // the four 16-key B operands of O^T += V^T P^T.  Also returns this lane's
  // sums of the weights: lr of the bf16-rounded ones (those enter P.V, so
  // u / lr is an exact weighted average of them: a dominant key returns its
  // value) and lx of the unrounded ones (for the LSE).
  auto weights = [&](const f32x16 (&sq)[2], float ms, bf16x8 (&pq)[4], float& lr, float& lx) {
    float r0 = 0.f, r1 = 0.f, x0 = 0.f, x1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = fast_exp2(__builtin_fmaf(sq[kb][8 * c2 + 2 * j], c, -ms));
          const float p1 = fast_exp2(__builtin_fmaf(sq[kb][8 * c2 + 2 * j + 1], c, -ms));
          const uint32_t pk = pack_bf16x2(p0, p1);
          if (j & 1) { r1 = sum2_bf16(pk, r1); x1 += p0 + p1; }
          else       { r0 = sum2_bf16(pk, r0); x0 += p0 + p1; }
          w[j] = pk;
        }
        pq[kb * 2 + c2] = __builtin_bit_cast(bf16x8, w);
      }
    lr = r0 + r1;
    lx = x0 + x1;
  };

  // one pipeline step for tile `it` (parity P): S(it) is in s_cur; S(it + 1)
  // goes to s_nxt on the matrix cores while S(it)'s softmax runs on the VALU
  auto step = [&](auto par, int it, f32x16 (&s_cur)[QB][2], f32x16 (&s_nxt)[QB][2]) {
    constexpr int P = decltype(par)::value;
    // prefetch K two tiles ahead into the buffer K(it) used, V one tile ahead
    if (it + 2 < n_iter) issue_tile(kg, P, it + 2);
    if (it + 1 < n_iter) issue_tile(vg, 2 + (P ^ 1), it + 1);

    if (it < wave_iters) {
      const int kv0 = it * BN;
      // mask keys past the end of the sequence and, when causal, future keys:
      // the key of register r is kv0 + kb*32 + (r/4)*8 + half*4 + r%4
      const bool edge = (kv0 + BN > seq_len) || (CAUSAL && kv0 + BN - 1 > wq0);
      if (edge) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int lim = (CAUSAL ? min(wq0 + qb * 32 + l32, seq_len - 1) : seq_len - 1) - (kv0 + hl * 4);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (kb * 32 + (r >> 2) * 8 + (r & 3) > lim) s_cur[qb][kb][r] = -INFINITY;
        }
      }

      // unconditional, so the matrix work shares a basic block with the
      // softmax below and the two can be interleaved; past the wave's last
      // tile the result is never used
      qk(Parity<P ^ 1>{}, s_nxt);

      // running-statistics softmax update of this tile.  The weights are first
      // formed against the current reference maximum m (no dependence on this
      // tile's maximum, so they overlap the MFMAs above).  The reference moves
      // to m_new = max(m, m_b) - and the old l and u are scaled by
      // exp(m - m_new) - only when some row of the wave grew by more than
      // 2^kLazyLog2 (always on a row's first tile, where m = -inf); then the
      // weights are formed again.  u / l does not depend on the reference.
      bf16x8 pf[QB][4];
      float mx[QB], lr[QB], lx[QB];
      bool move = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float ms = (m_run[qb] == -INFINITY) ? 0.f : m_run[qb] * c;
        weights(s_cur[qb], ms, pf[qb], lr[qb], lx[qb]);
        float m = fmaxf(s_cur[qb][0][0], s_cur[qb][1][0]);
#pragma unroll
        for (int r = 1; r < 16; ++r) m = fmaxf(m, fmaxf(s_cur[qb][0][r], s_cur[qb][1][r]));
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m),
                                                         false, false);
        mx[qb] = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        move |= (mx[qb] - m_run[qb]) * c > kLazyLog2 || m_run[qb] == -INFINITY;
      }
      if constexpr (Cfg::SCHED) {
        // interleave: one K-fragment read, one MFMA of S(it + 1), then a slice
        // of this tile's softmax, so the VALU runs under the matrix cores
#pragma unroll
        for (int i = 0; i < 2 * DC * QB; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, Cfg::VPM, 0);   // VALU
        }
      }
      if (__ballot(move) != 0) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float m_new = fmaxf(m_run[qb], mx[qb]);
          const float alpha = (m_run[qb] == -INFINITY) ? 0.f : fast_exp2((m_run[qb] - m_new) * c);
          m_run[qb] = m_new;
          l_run[qb] *= alpha;
          lx_run[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[qb][db] *= alpha;
          const float ms = (m_new == -INFINITY) ? 0.f : m_new * c;
          weights(s_cur[qb], ms, pf[qb], lr[qb], lx[qb]);
        }
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        l_run[qb] += lr[qb];
        lx_run[qb] += lx[qb];
      }

      // O^T += V^T P^T over four 16-key chunks
      const char* vt = smem + (2 + P) * TILE;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x4 lo = ds_read_tr16(vt + kc * 16 * ROWB + voff[0][db]);
          const bf16x4 hi = ds_read_tr16(vt + kc * 16 * ROWB + voff[1][db]);
          const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][kc], oacc[qb][db], 0, 0, 0);
        }
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  // prologue: K(0), K(1), V(0) resident, S(0) computed
  if (n_iter > 0) {
    issue_tile(kg, 0, 0);
    issue_tile(vg, 2, 0);
    if (n_iter > 1) issue_tile(kg, 1, 1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  f32x16 sa[QB][2], sb[QB][2];
  if (wave_iters > 0) qk(Parity<0>{}, sa);
  __syncthreads();   // every wave has read K(0) before K(2) replaces it

  for (int it = 0; it < n_iter; it += 2) {
    step(Parity<0>{}, it, sa, sb);
    if (it + 1 < n_iter) step(Parity<1>{}, it + 1, sb, sa);
  }

  // ---- epilogue: O = u / l, LSE = ln2 * (m * c + log2 l)
  const int64_t lse_base = PACKED ? ((int64_t)h * a.N + seq_start) : ((int64_t)(b * a.H + h) * a.N);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run[qb]),
                                                     __float_as_uint(l_run[qb]), false, false);
    const float l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const auto swx = __builtin_amdgcn_permlane32_swap(__float_as_uint(lx_run[qb]),
                                                      __float_as_uint(lx_run[qb]), false, false);
    const float lx_tot = __uint_as_float(swx[0]) + __uint_as_float(swx[1]);
    const int t = wq0 + qb * 32 + l32;
    if (t >= seq_len) continue;
    const bool any = l_tot > 0.f;
    const float inv = any ? 1.f / l_tot : 0.f;
    if (hl == 0) a.lse[lse_base + t] = any ? kLn2 * (m_run[qb] * c + __log2f(lx_tot)) : -INFINITY;
    const int64_t orow = (int64_t)(seq_start + t) * rs + head_off;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + g * 8 + hl * 4;
        const float o0 = oacc[qb][db][g * 4 + 0] * inv, o1 = oacc[qb][db][g * 4 + 1] * inv;
        const float o2 = oacc[qb][db][g * 4 + 2] * inv, o3 = oacc[qb][db][g * 4 + 3] * inv;
        if constexpr (OUT_F32) {
          *(f32x4*)((float*)a.o + orow + d) = (f32x4){o0, o1, o2, o3};
        } else {
          *(u32x2*)((uint16_t*)a.o + orow + d) = (u32x2){pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
        }
      }
  }
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------

template <class Cfg, bool CAUSAL, bool PACKED, bool OUT_F32>
static hipError_t launch_one(FwdArgs a, hipStream_t st) {
  constexpr int NW = Cfg::NW;
  constexpr int BM = 32 * Cfg::QB * NW;
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
template <int D> struct BfTile;
template <> struct BfTile<128> { using Cfg = BfCfg<128, 1, 4, 2, false>; };
template <> struct BfTile<64>  { using Cfg = BfCfg<64, 1, 4, 2, false>; };

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
  using C128 = BfTile<128>::Cfg;
  using C64 = BfTile<64>::Cfg;
  return d == 128 ? 32 * C128::QB * C128::NW : 32 * C64::QB * C64::NW;
}

}  // namespace iaea
