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

// Locate (head, sequence start, length, q block) of this workgroup.  Returns
// false when the workgroup has no work (grid padding, or packed slots past the
// last document).
template <int BM, bool CAUSAL, bool PACKED>
__device__ __forceinline__ bool decode_work(const FwdArgs& a, int lb, int& h, int& b,
                                            int& seq_start, int& seq_len, int& qblk) {
  if (lb >= a.n_work) return false;
  if constexpr (!PACKED) {
    const int bh = lb / a.slots;
    const int r = lb - bh * a.slots;
    qblk = CAUSAL ? (a.slots - 1 - r) : r;
    b = bh / a.H;
    h = bh - b * a.H;
    seq_start = b * a.N;
    seq_len = a.N;
    return true;
  } else {
    h = lb / a.slots;
    const int s = lb - h * a.slots;
    b = 0;
    const int lane = threadIdx.x & 63;
    int base = 0;
    for (int e0 = 0; e0 < a.B; e0 += 64) {
      const int e = e0 + lane;
      int nb = 0;
      if (e < a.B) {
        const int len = a.cu_seqlens[e + 1] - a.cu_seqlens[e];
        nb = len > 0 ? (len + BM - 1) / BM : 0;
      }
      int incl = nb;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
      }
      const int excl = incl - nb;
      const bool mine = (e < a.B) && (s >= base + excl) && (s < base + incl);
      const unsigned long long m = __ballot(mine);
      if (m) {
        const int src = __ffsll((long long)m) - 1;
        const int doc = e0 + src;
        const int first = base + __shfl(excl, src);
        const int nbd = __shfl(nb, src);
        seq_start = a.cu_seqlens[doc];
        seq_len = a.cu_seqlens[doc + 1] - seq_start;
        const int r = s - first;
        qblk = CAUSAL ? (nbd - 1 - r) : r;
        b = doc;
        return true;
      }
      base += __shfl(incl, 63);
    }
    return false;
  }
}

template <int D, int QB, int NW, bool CAUSAL, bool PACKED, bool OUT_F32>
__global__ void __launch_bounds__(NW * 64)
attn_fwd_bf16_kernel(FwdArgs a) {
  constexpr int BN = 64;                 // keys per tile
  constexpr int QW = 32 * QB;            // query rows per wave
  constexpr int BM = QW * NW;            // query rows per workgroup
  constexpr int G = D / 8;               // 16-byte granules per row
  constexpr int NT = NW * 64;
  constexpr int TILE = BN * D * 2;       // bytes of one K or V tile
  constexpr int LOADS = BN * G / NT;     // granules per thread per tile
  constexpr int DC = D / 16;             // k-steps of the QK^T MFMA
  constexpr int DB = D / 32;             // 32-wide blocks of d in O
  static_assert(LOADS * NT == BN * G, "tile must split evenly over the threads");

  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * TILE];

  int h, b, seq_start, seq_len, qblk;
  if (!decode_work<BM, CAUSAL, PACKED>(a, logical_block(blockIdx.x, a.per_xcd), h, b,
                                       seq_start, seq_len, qblk))
    return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
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

  // ---- K/V tile staging: global -> registers -> swizzled LDS
  u32x4 kreg[LOADS], vreg[LOADS];
  auto gload = [&](int it) {
    const int kv0 = it * BN;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int idx = threadIdx.x + i * NT;
      const int row = idx / G, g = idx % G;
      const int t = kv0 + row;
      const bool ok = t < seq_len;
      const int64_t off = (int64_t)(seq_start + (ok ? t : 0)) * rs + head_off + g * 8;
      kreg[i] = ok ? *(const u32x4*)(kg + off) : (u32x4){0u, 0u, 0u, 0u};
      vreg[i] = ok ? *(const u32x4*)(vg + off) : (u32x4){0u, 0u, 0u, 0u};
    }
  };
  auto lstore = [&](int stage) {
    char* kt = smem + stage * 2 * TILE;
    char* vt = kt + TILE;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int idx = threadIdx.x + i * NT;
      const int row = idx / G, g = idx % G;
      *(u32x4*)(kt + lds_off<D>(row, g)) = kreg[i];
      *(u32x4*)(vt + lds_off<D>(row, g)) = vreg[i];
    }
  };

  f32x16 oacc[QB][DB];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[qb][db] = (f32x16){};
  }

  // lane-constant parts of the transposed V read (ds_read_b64_tr_b16): in each
  // 16-lane group, source lane s points at key row 4*half + s/4 and d offset
  // 4*(s%4) of the group's 16 d columns; lane i then holds d column i of four
  // consecutive keys.
  const int g16 = lane >> 4;
  const int v_row = 4 * (g16 >> 1) + ((lane & 15) >> 2);
  const int v_dcol = 16 * (g16 & 1) + 4 * (lane & 3);

  if (n_iter > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int it = 0; it < n_iter; ++it) {
    if (it + 1 < n_iter) gload(it + 1);
    if (it < wave_iters) {
      const char* kt = smem + (it & 1) * 2 * TILE;
      const char* vt = kt + TILE;
      const int kv0 = it * BN;

      // S^T[key][query] for two 32-key halves of the tile
      f32x16 s[QB][2];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb][0] = s[qb][1] = (f32x16){};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          const bf16x8 kf = *(const bf16x8*)(kt + lds_off<D>(kb * 32 + l32, dc * 2 + hl));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][dc], s[qb][kb], 0, 0, 0);
        }
      }

      // mask keys past the end of the sequence and, when causal, future keys
      const bool edge = (kv0 + BN > seq_len) || (CAUSAL && kv0 + BN - 1 > wq0);
      if (edge) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int qi = wq0 + qb * 32 + l32;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int kj = kv0 + kb * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
              if (kj >= seq_len || (CAUSAL && kj > qi)) s[qb][kb][r] = -INFINITY;
            }
        }
      }

      // running-statistics softmax update
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = s[qb][0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
        mx = wave_max_half_swap(mx);
        const float m_new = fmaxf(m_run[qb], mx);
        const float ms_new = (m_new == -INFINITY) ? 0.f : m_new * c;
        const float alpha = (m_run[qb] == -INFINITY) ? 0.f : fast_exp2(m_run[qb] * c - ms_new);
        m_run[qb] = m_new;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[qb][db] *= alpha;
        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(__builtin_fmaf(s[qb][kb][r], c, -ms_new));
            s[qb][kb][r] = p;
            lsum += p;
          }
        l_run[qb] += lsum;
      }

      // O^T += V^T P^T over four 16-key chunks
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          bf16x8 pf[QB];
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            u32x4 w;
#pragma unroll
            for (int j = 0; j < 4; ++j)
              w[j] = pack_bf16x2(s[qb][kb][8 * c2 + 2 * j], s[qb][kb][8 * c2 + 2 * j + 1]);
            pf[qb] = __builtin_bit_cast(bf16x8, w);
          }
          const int row = kb * 32 + 16 * c2 + v_row;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int d = db * 32 + v_dcol;
            const bf16x4 lo = ds_read_tr16(vt + lds_off<D>(row, d >> 3) + (d & 7) * 2);
            const bf16x4 hi = ds_read_tr16(vt + lds_off<D>(row + 8, d >> 3) + (d & 7) * 2);
            const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb], oacc[qb][db], 0, 0, 0);
          }
        }
      }
    }
    if (it + 1 < n_iter) lstore((it + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O = u / l, LSE = ln2 * (m * c + log2 l)
  const int64_t lse_base = PACKED ? ((int64_t)h * a.N + seq_start) : ((int64_t)(b * a.H + h) * a.N);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);
    const int t = wq0 + qb * 32 + l32;
    if (t >= seq_len) continue;
    const bool any = l_tot > 0.f;
    const float inv = any ? 1.f / l_tot : 0.f;
    if (hl == 0) a.lse[lse_base + t] = any ? kLn2 * (m_run[qb] * c + __log2f(l_tot)) : -INFINITY;
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

template <int D, int QB, int NW, bool CAUSAL, bool PACKED, bool OUT_F32>
static hipError_t launch_one(FwdArgs a, hipStream_t st) {
  constexpr int BM = 32 * QB * NW;
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
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_bf16_kernel<D, QB, NW, CAUSAL, PACKED, OUT_F32>),
                         dim3(grid), dim3(NW * 64), args, 0, st);
}

// Tile shape per head dimension: queries per wave (32 * QB) and waves per
// workgroup.
template <int D> struct BfTile;
template <> struct BfTile<128> { static constexpr int QB = 1, NW = 4; };
template <> struct BfTile<64>  { static constexpr int QB = 1, NW = 4; };

template <int D, bool CAUSAL, bool PACKED>
static hipError_t launch_d(const FwdArgs& a, bool out_f32, hipStream_t st) {
  constexpr int QB = BfTile<D>::QB, NW = BfTile<D>::NW;
  return out_f32 ? launch_one<D, QB, NW, CAUSAL, PACKED, true>(a, st)
                 : launch_one<D, QB, NW, CAUSAL, PACKED, false>(a, st);
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
  return d == 128 ? 32 * BfTile<128>::QB * BfTile<128>::NW : 32 * BfTile<64>::QB * BfTile<64>::NW;
}

}  // namespace iaea
