// bf16 exact attention backward for gfx950 (MI355X): dQ, dK, dV.
//
// "Flash Attention và IO" asks for the backward pass to be timed beside the
// forward when the goal is training (section "Kernel đúng còn phải hợp với
// tải") and its gradients to be compared with another implementation's
// (section "Bài tập kiểm tính đúng trước khi đo tốc độ").  The pages print no
// backward algorithm; what is computed is the derivative of the forward, per
// (sequence, head), with the forward's log-sum-exp L saved instead of the N x N
// probabilities (the recomputation that keeps the forward IO-aware):
//     P_ij = exp(scale q_i . k_j - L_i)  (0 for a masked key)
//     D_i  = dO_i . O_i                   = sum_j P_ij (dO_i . v_j)
//     dV_j = sum_i P_ij dO_i
//     dS_ij = P_ij (dO_i . v_j - D_i)
//     dQ_i = scale sum_j dS_ij k_j,       dK_j = scale sum_i dS_ij q_i.
// Two kernels, both tile by tile through LDS, nothing N x N in memory:
//   * dQ: one workgroup per 128 query rows first forms D of its rows from
//     their dO and O (and writes it for the other kernel), then walks the
//     key/value tiles, as the forward does, with S^T = K Q^T and
//     dP^T = V dO^T and dQ^T += K^T dS^T;
//   * dK/dV: one workgroup per 128 keys walks the query tiles, with
//     S = Q K^T and dP = dO V^T, dV^T += dO^T P and dK^T += Q^T dS (at
//     d = 128 two waves share 32 keys, each forming S and dP for half of a
//     query tile and accumulating half of the coordinates).
// Splitting dQ from dK/dV recomputes S and dP once more but needs no atomics
// and no fp32 accumulation buffer for dQ.
//
// MI355X mapping: v_mfma_f32_32x32x16_bf16 throughout.  In each kernel the
// operand that stays (Q and dO, or K and V) lives in VGPRs as the B operand,
// so every lane owns one row (query or key) of every accumulator; the
// streamed tiles go from HBM straight to double-buffered, swizzled LDS
// (buffer_load_dwordx4 ... lds); P and dS are rounded to bf16 and reused as
// the B operand of the next product in the accumulator's own register order,
// with the A operand read in the matching order by ds_read_b64_tr_b16.
#include <atomic>
#include <mutex>
#include <type_traits>

#include "attn_common.h"
#include "attn_kernels.h"
#include "attn_mask.h"

namespace iaea {

namespace bwd {
constexpr int NW = 4;            // waves per workgroup, 32 rows each
constexpr int BM = 32 * NW;      // rows (queries or keys) per workgroup
constexpr int BN = 64;           // rows of a streamed tile
}  // namespace bwd

// ---------------------------------------------------------------------------
// shared pieces of the two gradient kernels
// ---------------------------------------------------------------------------

// The lane's 8 bf16 of d-chunk dc (B operand, k = d) of row `row` of a [.][H][D]
// tensor; zero when the row is outside the sequence.
template <int D>
__device__ __forceinline__ void load_row_frags(const uint16_t* __restrict__ base, int64_t rs, bool ok,
                                               int hl, bf16x8 (&f)[D / 16]) {
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) {
    const u32x4 raw = ok ? *(const u32x4*)(base + dc * 16 + 8 * hl) : (u32x4){0u, 0u, 0u, 0u};
    f[dc] = __builtin_bit_cast(bf16x8, raw);
    (void)rs;
  }
}

// Stores an accumulator X^T (rows = d, one column per lane: the lane's own row
// of X) times `mul` as bf16 into row `row` of a [.][H][D] tensor.
template <int D>
__device__ __forceinline__ void store_row(uint16_t* __restrict__ dst, const f32x16 (&acc)[D / 32], float mul,
                                          int hl) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = db * 32 + g * 8 + hl * 4;
      *(u32x2*)(dst + d) = (u32x2){pack_bf16x2(acc[db][g * 4 + 0] * mul, acc[db][g * 4 + 1] * mul),
                                   pack_bf16x2(acc[db][g * 4 + 2] * mul, acc[db][g * 4 + 3] * mul)};
    }
}

// ---------------------------------------------------------------------------
// dQ: query blocks outer, key/value tiles inner
// ---------------------------------------------------------------------------

template <int D, bool CAUSAL, bool PACKED>
__global__ void __launch_bounds__(bwd::NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dq_kernel(BwdArgs a) {
  using namespace bwd;
  constexpr int ROWB = D * 2, TILE = BN * ROWB;
  constexpr int CPW = TILE / 1024 / NW;        // 1 KB load chunks per wave per tile
  constexpr int DC = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];   // K0 K1 V0 V1

  int h, b, seq_start, seq_len, qblk;
  if (!decode_work<BM, CAUSAL, PACKED>(a, blockIdx.x, h, b, seq_start, seq_len, qblk)) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5, l32 = lane & 31;
  const int q0 = qblk * BM, wq0 = q0 + wave * 32;
  const int kv_end = CAUSAL ? min(seq_len, q0 + BM) : seq_len;
  const int n_iter = (kv_end + BN - 1) / BN;
  const int wave_kv_end = CAUSAL ? min(seq_len, wq0 + 32) : seq_len;
  const int wave_iters = (wq0 < seq_len) ? (wave_kv_end + BN - 1) / BN : 0;
  const int64_t rs = (int64_t)a.H * D;
  const int64_t head_off = (int64_t)h * D;
  const int64_t lrow = PACKED ? (int64_t)h * a.N + seq_start : (int64_t)(b * a.H + h) * a.N;

  // this lane's query row: Q and dO fragments, L log2(e) and D
  const int t = wq0 + l32;
  const bool tok = t < seq_len;
  const int64_t trow = (int64_t)(seq_start + (tok ? t : 0)) * rs + head_off;
  bf16x8 qf[DC], df[DC], of[DC];
  load_row_frags<D>((const uint16_t*)a.q + trow, rs, tok, hl, qf);
  load_row_frags<D>((const uint16_t*)a.dout + trow, rs, tok, hl, df);
  load_row_frags<D>((const uint16_t*)a.o + trow, rs, tok, hl, of);
  const float lse2 = tok ? a.lse[lrow + t] * kLog2e : 0.f;
  // D = dO . O of the row, from the fragments: the two halves of the wave
  // hold the two halves of the row's coordinates and exchange their sums.
  // D goes to the caller's buffer for the dK/dV kernel, enqueued after this
  // one.
  float dlt;
  {
    float part = 0.f;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int e = 0; e < 8; ++e) part = __builtin_fmaf((float)df[dc][e], (float)of[dc][e], part);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
    dlt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if (tok && hl == 0) a.delta[lrow + t] = dlt;
  }
  // dO negated (exactly, by its sign bits) and every dP^T sum started at D:
  // the products leave D - dP, so dS comes out negated and dQ is negated at
  // the store
#pragma unroll
  for (int dc = 0; dc < DC; ++dc)
    df[dc] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, df[dc]) ^ 0x80008000u);
  f32x16 d0;
#pragma unroll
  for (int r = 0; r < 16; ++r) d0[r] = dlt;

  // tile loads
  uint32_t lane_off[CPW];
#pragma unroll
  for (int cc = 0; cc < CPW; ++cc) {
    const int byte = (wave * CPW + cc) * 1024 + lane * 16;
    const int row = byte / ROWB;
    const int gr = ((byte % ROWB) >> 4) ^ swz<D>(row);
    lane_off[cc] = (uint32_t)(((int64_t)row * rs + head_off + gr * 8) * 2);
  }
  [[maybe_unused]] const uint32_t row_bytes = (uint32_t)rs * 2u;
  auto issue_tile = [&](const void* src, int buf, int j) __attribute__((always_inline)) {
#if __HIP_DEVICE_COMPILE__
    const int kv0 = j * BN;
    const uint32_t nrec = (uint32_t)min(seq_len - kv0, BN) * row_bytes;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const char*)src + (uint64_t)(uint32_t)(seq_start + kv0) * row_bytes), (short)0, (int)nrec,
        kBufferFlags);
    static_for<CPW>([&](auto ci) __attribute__((always_inline)) {
      constexpr int cc = decltype(ci)::value;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (IAEA_LDS void*)(smem + buf * TILE + wave * CPW * 1024),
                                               16, lane_off[cc] - cc * 1024, 0, cc * 1024, 0);
    });
#endif
  };

  // LDS read offsets: plain fragments (A operand, rows = keys, k = d) and
  // transposed ones (A operand, rows = d, k = 16 keys in the register order of
  // the packed chunks)
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

  f32x16 dqacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqacc[db] = (f32x16){};

  // one key/value tile; the buffer parity is a template constant, so that
  // every LDS address is a per-lane offset plus an immediate
  auto tile = [&](auto par, int j) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();                           // tile j landed; tile j - 1 no longer read
    if (j + 1 < n_iter) {
      issue_tile(a.k, P ^ 1, j + 1);
      issue_tile(a.v, 2 + (P ^ 1), j + 1);
    }
    if (j >= wave_iters) return;
    const char* kt = smem + P * TILE;
    const char* vt = smem + (2 + P) * TILE;
    const int kv0 = j * BN;
    // the tile in two halves of 32 keys: S^T and dP^T of a half, then its
    // product into dQ^T
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // 2 DC MFMA steps, S^T and dP^T alternating, each operand fragment read
      // PF steps ahead of its MFMA (a scheduling barrier between steps)
      constexpr int PF = 3;
      f32x16 s, dp;
      auto sfrag = [&](auto step) __attribute__((always_inline)) -> bf16x8 {
        constexpr int st = decltype(step)::value;
        return *(const bf16x8*)(((st & 1) ? vt : kt) + kb * 32 * ROWB + koff[st >> 1]);
      };
      bf16x8 fa[PF + 1];
      static_for<PF>([&](auto step) __attribute__((always_inline)) {
        fa[decltype(step)::value] = sfrag(step);
      });
      static_for<2 * DC>([&](auto step) __attribute__((always_inline)) {
        constexpr int st = decltype(step)::value, dc = st >> 1;
        if constexpr (st + PF < 2 * DC) fa[(st + PF) % (PF + 1)] = sfrag(std::integral_constant<int, st + PF>{});
        if constexpr (st & 1)
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[st % (PF + 1)], df[dc], dc == 0 ? d0 : dp, 0, 0, 0);
        else
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[st % (PF + 1)], qf[dc], dc == 0 ? (f32x16){} : s, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      });
      // P^T and dS^T in place; key of register r: kv0 + kb*32 + (r/4)*8 + hl*4 + r%4.
      // The mask is applied only where some key of the half lies past the
      // wave's first query (causal) or the sequence end.
      const int lim = (CAUSAL ? min(t, seq_len - 1) : seq_len - 1) - (kv0 + kb * 32 + hl * 4);
      auto weights = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(__builtin_fmaf(s[r], a.c, -lse2));
          if constexpr (decltype(masked)::value)
            if ((r >> 2) * 8 + (r & 3) > lim) p = 0.f;
          s[r] = p * dp[r];                    // -dS^T
        }
      };
      if (dq_half_tile_unmasked(CAUSAL, wq0, kv0 + kb * 32, seq_len)) weights(std::false_type{});
      else weights(std::true_type{});
      // dQ^T += K^T dS^T, 16 keys at a time: 2 DB MFMA steps (chunk t / DB,
      // d block t % DB), each transposed K fragment read PF2 steps ahead
      bf16x8 dsf[2];
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        u32x4 w;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) w[jj] = pack_bf16x2(s[8 * c2 + 2 * jj], s[8 * c2 + 2 * jj + 1]);
        dsf[c2] = __builtin_bit_cast(bf16x8, w);
      }
      constexpr int PF2 = 2;
      auto tfrag = [&](auto step) __attribute__((always_inline)) -> bf16x8 {
        constexpr int t = decltype(step)::value, c2 = t / DB, db = t % DB;
        const char* kk = kt + (kb * 2 + c2) * 16 * ROWB;
        const bf16x4 lo = ds_read_tr16(kk + voff[0][db]);
        const bf16x4 hi = ds_read_tr16(kk + voff[1][db]);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      bf16x8 ft[PF2 + 1];
      static_for<PF2>([&](auto step) __attribute__((always_inline)) {
        ft[decltype(step)::value] = tfrag(step);
      });
      static_for<2 * DB>([&](auto step) __attribute__((always_inline)) {
        constexpr int t = decltype(step)::value, c2 = t / DB, db = t % DB;
        if constexpr (t + PF2 < 2 * DB) ft[(t + PF2) % (PF2 + 1)] = tfrag(std::integral_constant<int, t + PF2>{});
        dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ft[t % (PF2 + 1)], dsf[c2], dqacc[db], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      });
    }
  };
  if (n_iter > 0) {
    issue_tile(a.k, 0, 0);
    issue_tile(a.v, 2, 0);
  }
  for (int j = 0; j < n_iter; j += 2) {
    tile(std::integral_constant<int, 0>{}, j);
    if (j + 1 < n_iter) tile(std::integral_constant<int, 1>{}, j + 1);
  }
  if (tok) store_row<D>((uint16_t*)a.dq + trow, dqacc, -a.scale, hl);
}

// ---------------------------------------------------------------------------
// dK, dV: key blocks outer, query tiles inner
// ---------------------------------------------------------------------------

// d = 64: K, V and both accumulators fit two waves per SIMD in one wave per
// 32 keys.  (At d = 128 they keep about 192 VGPRs live; the wave-pair kernel
// below splits the coordinates instead.)
template <int D, bool CAUSAL, bool PACKED>
__global__ void __launch_bounds__(bwd::NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dkdv_kernel(BwdArgs a) {
  static_assert(D == 64, "d = 128 uses bwd_dkdv_pair_kernel");
  using namespace bwd;
  constexpr int ROWB = D * 2, TILE = BN * ROWB;
  constexpr int CPW = TILE / 1024 / NW;
  constexpr int DC = D / 16, DB = D / 32;
  // Q0 Q1 dO0 dO1, then L log2(e) and D of both tiles (BN floats each)
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE + 4 * BN * 4];
  float* lse_t = (float*)(smem + 4 * TILE);    // [2][BN]
  float* dlt_t = lse_t + 2 * BN;               // [2][BN]

  int h, b, seq_start, seq_len, kblk;
  // key blocks in natural order: under the causal mask the first blocks see
  // the most query tiles, so this is longest first
  if (!decode_work<BM, false, PACKED>(a, blockIdx.x, h, b, seq_start, seq_len, kblk)) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5, l32 = lane & 31;
  const int k0 = kblk * BM, wk0 = k0 + wave * 32;
  const int j_begin = CAUSAL ? k0 / BN : 0;
  const int j_end = (seq_len + BN - 1) / BN;
  const int wave_begin = CAUSAL ? wk0 / BN : 0;      // earlier tiles are all masked for this wave
  const bool wave_live = wk0 < seq_len;
  const int64_t rs = (int64_t)a.H * D;
  const int64_t head_off = (int64_t)h * D;
  [[maybe_unused]] const int64_t lrow = PACKED ? (int64_t)h * a.N + seq_start : (int64_t)(b * a.H + h) * a.N;

  // this lane's key row: K and V fragments
  const int key = wk0 + l32;
  const bool kok = key < seq_len;
  const int64_t krow = (int64_t)(seq_start + (kok ? key : 0)) * rs + head_off;
  bf16x8 kf[DC], vf[DC];
  load_row_frags<D>((const uint16_t*)a.k + krow, rs, kok, hl, kf);
  load_row_frags<D>((const uint16_t*)a.v + krow, rs, kok, hl, vf);
  // V negated (exactly, by its sign bits): the dP sums start at D and end at
  // D - dP, so dS comes out negated and dK is negated at the store
#pragma unroll
  for (int dc = 0; dc < DC; ++dc)
    vf[dc] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, vf[dc]) ^ 0x80008000u);

  uint32_t lane_off[CPW];
#pragma unroll
  for (int cc = 0; cc < CPW; ++cc) {
    const int byte = (wave * CPW + cc) * 1024 + lane * 16;
    const int row = byte / ROWB;
    const int gr = ((byte % ROWB) >> 4) ^ swz<D>(row);
    lane_off[cc] = (uint32_t)(((int64_t)row * rs + head_off + gr * 8) * 2);
  }
  [[maybe_unused]] const uint32_t row_bytes = (uint32_t)rs * 2u;
  auto issue_tile = [&](int buf, int j) __attribute__((always_inline)) {
#if __HIP_DEVICE_COMPILE__
    const int q0 = j * BN;
    const int nrows = min(seq_len - q0, BN);
    const uint32_t nrec = (uint32_t)nrows * row_bytes;
    const uint64_t off = (uint64_t)(uint32_t)(seq_start + q0) * row_bytes;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const char*)a.q + off), (short)0, (int)nrec, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const char*)a.dout + off), (short)0, (int)nrec, kBufferFlags);
    static_for<CPW>([&](auto ci) __attribute__((always_inline)) {
      constexpr int cc = decltype(ci)::value;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (IAEA_LDS void*)(smem + buf * TILE + wave * CPW * 1024),
                                               16, lane_off[cc] - cc * 1024, 0, cc * 1024, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (IAEA_LDS void*)(smem + (2 + buf) * TILE + wave * CPW * 1024),
                                               16, lane_off[cc] - cc * 1024, 0, cc * 1024, 0);
    });
    // the tile's L and D: one dword per lane (rows past the end read as 0)
    if (wave < 2) {
      const float* src = wave == 0 ? a.lse : a.delta;
      const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(src + lrow + q0), (short)0, nrows * 4, kBufferFlags);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (IAEA_LDS void*)((wave == 0 ? lse_t : dlt_t) + buf * BN),
                                               4, lane * 4, 0, 0, 0);
    }
#endif
  };

  uint32_t qoff[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) qoff[dc] = l32 * ROWB + (((2 * dc + hl) ^ swz<D>(l32)) << 4);
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

  f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dkacc[db] = dvacc[db] = (f32x16){};

  // one query tile; the buffer parity is a template constant, so that every
  // LDS address is a per-lane offset plus an immediate
  auto tile = [&](auto par, int j) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 1 < j_end) issue_tile(P ^ 1, j + 1);
    if (!wave_live || j < wave_begin) return;
    const char* qt = smem + P * TILE;
    const char* dt = smem + (2 + P) * TILE;
    const int q0 = j * BN;
    // visible queries of this lane's key, as offsets in the tile: [lo, hi]
    const int lo = CAUSAL ? key - q0 : 0;
    const int hi = kok ? seq_len - 1 - q0 : -1;
    // the tile in two halves of 32 queries: S and dP of a half, then its
    // products into dV and dK, so only one half's scores are live at a time
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      __builtin_amdgcn_sched_barrier(0);       // one half's loads at a time: fewer live registers
      // query of register r: q0 + qb*32 + (r/4)*8 + hl*4 + r%4; its L and D
      // come from the tile's LDS rows, four at a time: D starts the dP sums,
      // -L log2(e) is formed beside the MFMAs
      f32x16 s, dp, d0, nl;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 l4 = *(const f32x4*)(lse_t + P * BN + qb * 32 + g * 8 + hl * 4);
        const f32x4 d4 = *(const f32x4*)(dlt_t + P * BN + qb * 32 + g * 8 + hl * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          d0[g * 4 + i] = d4[i];
          nl[g * 4 + i] = -l4[i] * kLog2e;
        }
      }
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const bf16x8 qfr = *(const bf16x8*)(qt + qb * 32 * ROWB + qoff[dc]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qfr, kf[dc], dc == 0 ? (f32x16){} : s, 0, 0, 0);
        const bf16x8 dfr = *(const bf16x8*)(dt + qb * 32 * ROWB + qoff[dc]);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dfr, vf[dc], dc == 0 ? d0 : dp, 0, 0, 0);
      }
      // P goes to s, -dS to dp
      auto weights = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int qi = qb * 32 + g * 8 + hl * 4;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = g * 4 + i;
            float p = fast_exp2(__builtin_fmaf(s[r], a.c, nl[r]));
            if constexpr (decltype(masked)::value)
              if (qi + i < lo || qi + i > hi) p = 0.f;
            s[r] = p;
            dp[r] = p * dp[r];
          }
        }
      };
      // the mask only where the half's queries meet the diagonal or a tail
      if (dkdv_half_tile_unmasked(CAUSAL, q0 + qb * 32, wk0, seq_len))
        weights(std::false_type{});
      else
        weights(std::true_type{});
      // dV^T += dO^T P and dK^T += Q^T dS, 16 queries at a time
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        u32x4 pw, dw;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          pw[jj] = pack_bf16x2(s[8 * c2 + 2 * jj], s[8 * c2 + 2 * jj + 1]);
          dw[jj] = pack_bf16x2(dp[8 * c2 + 2 * jj], dp[8 * c2 + 2 * jj + 1]);
        }
        const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
        const bf16x8 dsf = __builtin_bit_cast(bf16x8, dw);
        const int kc = qb * 2 + c2;
        const char* dd = dt + kc * 16 * ROWB;
        const char* qq = qt + kc * 16 * ROWB;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x4 dlo = ds_read_tr16(dd + voff[0][db]);
          const bf16x4 dhi = ds_read_tr16(dd + voff[1][db]);
          dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_shufflevector(dlo, dhi, 0, 1, 2, 3, 4, 5, 6, 7), pf, dvacc[db], 0, 0, 0);
          const bf16x4 qlo = ds_read_tr16(qq + voff[0][db]);
          const bf16x4 qhi = ds_read_tr16(qq + voff[1][db]);
          dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7), dsf, dkacc[db], 0, 0, 0);
        }
      }
    }
  };
  if (j_begin < j_end) issue_tile(0, j_begin);
  for (int j = j_begin; j < j_end; j += 2) {
    tile(std::integral_constant<int, 0>{}, j);
    if (j + 1 < j_end) tile(std::integral_constant<int, 1>{}, j + 1);
  }
  if (kok) {
    store_row<D>((uint16_t*)a.dk + krow, dkacc, -a.scale, hl);
    store_row<D>((uint16_t*)a.dv + krow, dvacc, 1.f, hl);
  }
}

// ---------------------------------------------------------------------------
// dK, dV with wave pairs (d = 128): no recomputation at two waves per SIMD
// ---------------------------------------------------------------------------

// Eight waves per 128 keys, two per group of 32 keys.  Both waves of a pair
// hold the group's K and V rows (all d) and split each 64-query tile: wave
// half h forms S = Q K^T, dP = dO V^T, P and dS for queries 32 h .. 32 h + 31
// and leaves its two 16-query chunks of P and dS, packed as the next
// product's B operand, in LDS; after a barrier each wave takes its partner's
// chunks and accumulates dV^T += dO^T P and dK^T += Q^T dS for all 64 queries
// but only its own 64 of the 128 coordinates.  The dP accumulator starts at
// D and V is held negated, so the products leave D - dP: dS comes out
// negated at one multiply per score, and dK is negated where it is stored.
template <int D, bool CAUSAL, bool PACKED>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dkdv_pair_kernel(BwdArgs a) {
  using namespace bwd;
  static_assert(D == 128, "wave pairs split d = 128 in two");
  constexpr int NWP = 8;                       // waves per workgroup
  constexpr int ROWB = D * 2, TILE = BN * ROWB;
  constexpr int CPW = TILE / 1024 / NWP;       // 1 KB load chunks per wave per tile
  constexpr int DC = D / 16, DBH = D / 64;     // k-steps of S; 32-wide d blocks per wave
  // Q0 Q1 dO0 dO1 | L, D of both tiles | P, dS chunks [4 pairs][2 kinds][4 chunks][64 lanes][16 B]
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE + 4 * BN * 4 + 4 * 2 * 4 * 64 * 16];
  float* lse_t = (float*)(smem + 4 * TILE);    // [2][BN]
  float* dlt_t = lse_t + 2 * BN;               // [2][BN]
  char* xch = smem + 4 * TILE + 4 * BN * 4;

  int h, b, seq_start, seq_len, kblk;
  if (!decode_work<BM, false, PACKED>(a, blockIdx.x, h, b, seq_start, seq_len, kblk)) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pair = wave >> 1, half = wave & 1;
  const int hl = lane >> 5, l32 = lane & 31;
  const int k0 = kblk * BM, wk0 = k0 + pair * 32;
  const int j_begin = CAUSAL ? k0 / BN : 0;
  const int j_end = (seq_len + BN - 1) / BN;
  const int pair_begin = CAUSAL ? wk0 / BN : 0;
  const bool pair_live = wk0 < seq_len;
  const int64_t rs = (int64_t)a.H * D;
  const int64_t head_off = (int64_t)h * D;
  [[maybe_unused]] const int64_t lrow = PACKED ? (int64_t)h * a.N + seq_start : (int64_t)(b * a.H + h) * a.N;

  const int key = wk0 + l32;
  const bool kok = key < seq_len;
  const int64_t krow = (int64_t)(seq_start + (kok ? key : 0)) * rs + head_off;
  bf16x8 kf[DC], vf[DC];
  load_row_frags<D>((const uint16_t*)a.k + krow, rs, kok, hl, kf);
  load_row_frags<D>((const uint16_t*)a.v + krow, rs, kok, hl, vf);
  // V negated (exactly, by its sign bits): the dP accumulator starts at D and
  // ends at D - dP, so dS comes out negated and dK is negated at the store
#pragma unroll
  for (int dc = 0; dc < DC; ++dc)
    vf[dc] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, vf[dc]) ^ 0x80008000u);

  uint32_t lane_off[CPW];
#pragma unroll
  for (int cc = 0; cc < CPW; ++cc) {
    const int byte = (wave * CPW + cc) * 1024 + lane * 16;
    const int row = byte / ROWB;
    const int gr = ((byte % ROWB) >> 4) ^ swz<D>(row);
    lane_off[cc] = (uint32_t)(((int64_t)row * rs + head_off + gr * 8) * 2);
  }
  [[maybe_unused]] const uint32_t row_bytes = (uint32_t)rs * 2u;
  auto issue_tile = [&](int buf, int j) __attribute__((always_inline)) {
#if __HIP_DEVICE_COMPILE__
    const int q0 = j * BN;
    const int nrows = min(seq_len - q0, BN);
    const uint32_t nrec = (uint32_t)nrows * row_bytes;
    const uint64_t off = (uint64_t)(uint32_t)(seq_start + q0) * row_bytes;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const char*)a.q + off), (short)0, (int)nrec, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const char*)a.dout + off), (short)0, (int)nrec, kBufferFlags);
    static_for<CPW>([&](auto ci) __attribute__((always_inline)) {
      constexpr int cc = decltype(ci)::value;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (IAEA_LDS void*)(smem + buf * TILE + wave * CPW * 1024),
                                               16, lane_off[cc] - cc * 1024, 0, cc * 1024, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (IAEA_LDS void*)(smem + (2 + buf) * TILE + wave * CPW * 1024),
                                               16, lane_off[cc] - cc * 1024, 0, cc * 1024, 0);
    });
    if (wave < 2) {
      const float* src = wave == 0 ? a.lse : a.delta;
      const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(src + lrow + q0), (short)0, nrows * 4, kBufferFlags);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (IAEA_LDS void*)((wave == 0 ? lse_t : dlt_t) + buf * BN),
                                               4, lane * 4, 0, 0, 0);
    }
#endif
  };

  uint32_t qoff[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) qoff[dc] = (half * 32 + l32) * ROWB + (((2 * dc + hl) ^ swz<D>(l32)) << 4);
  uint32_t voff[2][DBH];
  {
    const int g16 = lane >> 4;
    const int v_row = 4 * (g16 >> 1) + ((lane & 15) >> 2);
    const int v_dcol = 16 * (g16 & 1) + 4 * (lane & 3);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
      for (int dbl = 0; dbl < DBH; ++dbl) {
        const int row = v_row + 8 * hi;
        const int d = (half * DBH + dbl) * 32 + v_dcol;
        voff[hi][dbl] = row * ROWB + (((d >> 3) ^ swz<D>(row)) << 4) + (d & 7) * 2;
      }
  }
  // this pair's exchange slots: kind 0 = P, 1 = dS; chunk kc of the tile
  char* const pxch = xch + pair * (2 * 4 * 64 * 16);
  auto slot = [&](int kind, int kc) __attribute__((always_inline)) -> char* {
    return pxch + ((kind * 4 + kc) * 64 + lane) * 16;
  };

  f32x16 dkacc[DBH], dvacc[DBH];
#pragma unroll
  for (int dbl = 0; dbl < DBH; ++dbl) dkacc[dbl] = dvacc[dbl] = (f32x16){};

  // one query tile; the buffer parity is a template constant, so that every
  // LDS address is a per-lane offset plus an immediate
  auto tile = [&](auto par, int j) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();                           // tile j landed; last tile's chunks all read
    if (j + 1 < j_end) issue_tile(P ^ 1, j + 1);
    const bool live = pair_live && j >= pair_begin;
    const char* qt = smem + P * TILE;
    const char* dt = smem + (2 + P) * TILE;
    const int q0 = j * BN;
    bf16x8 own_p[2], own_ds[2];
    if (live) {
      // S and dP of this wave's 32 queries (rows 32 half .. of the tile): 16
      // MFMA steps, S and dP alternating, each operand fragment read PF steps
      // ahead of its MFMA so the LDS latency hides behind earlier MFMAs
      f32x16 s, dp;
      f32x16 nl;                               // -L log2(e) of the 16 query rows, formed
                                               // among the MFMAs rather than in the weight loop
      {
        f32x16 d0;                             // D of each of the 16 query rows
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 d4 = *(const f32x4*)(dlt_t + P * BN + half * 32 + g * 8 + hl * 4);
          const f32x4 l4 = *(const f32x4*)(lse_t + P * BN + half * 32 + g * 8 + hl * 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            d0[g * 4 + i] = d4[i];
            nl[g * 4 + i] = -l4[i] * kLog2e;
          }
        }
        constexpr int PF = 3;
        auto afrag = [&](auto step) __attribute__((always_inline)) -> bf16x8 {
          constexpr int st = decltype(step)::value;
          return *(const bf16x8*)(((st & 1) ? dt : qt) + qoff[st >> 1]);
        };
        bf16x8 fa[PF + 1];
        static_for<PF>([&](auto step) __attribute__((always_inline)) {
          fa[decltype(step)::value] = afrag(step);
        });
        static_for<2 * DC>([&](auto step) __attribute__((always_inline)) {
          constexpr int st = decltype(step)::value, dc = st >> 1;
          if constexpr (st + PF < 2 * DC) fa[(st + PF) % (PF + 1)] = afrag(std::integral_constant<int, st + PF>{});
          if constexpr (st & 1)
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[st % (PF + 1)], vf[dc], dc == 0 ? d0 : dp, 0, 0, 0);
          else
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[st % (PF + 1)], kf[dc], dc == 0 ? (f32x16){} : s, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      const int lo = CAUSAL ? key - q0 : 0;
      const int hi = kok ? seq_len - 1 - q0 : -1;
      auto weights = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int qi = half * 32 + g * 8 + hl * 4;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = g * 4 + i;
            float p = fast_exp2(__builtin_fmaf(s[r], a.c, nl[r]));
            if constexpr (decltype(masked)::value)
              if (qi + i < lo || qi + i > hi) p = 0.f;
            s[r] = p;
            dp[r] = p * dp[r];                 // -dS
          }
        }
      };
      // the mask only where this wave's queries meet the diagonal or a tail
      if (dkdv_half_tile_unmasked(CAUSAL, q0 + half * 32, wk0, seq_len))
        weights(std::false_type{});
      else
        weights(std::true_type{});
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        u32x4 pw, dw;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          pw[jj] = pack_bf16x2(s[8 * c2 + 2 * jj], s[8 * c2 + 2 * jj + 1]);
          dw[jj] = pack_bf16x2(dp[8 * c2 + 2 * jj], dp[8 * c2 + 2 * jj + 1]);
        }
        own_p[c2] = __builtin_bit_cast(bf16x8, pw);
        own_ds[c2] = __builtin_bit_cast(bf16x8, dw);
        *(u32x4*)slot(0, half * 2 + c2) = pw;
        *(u32x4*)slot(1, half * 2 + c2) = dw;
      }
    }
    __syncthreads();                           // both halves' chunks in LDS
    if (!live) return;
    // dV^T += dO^T P and dK^T += Q^T dS over the tile's four 16-query chunks,
    // this wave's 64 coordinates: 16 MFMA steps, the wave's own two chunks
    // first (chunk kl ^ 2 half for local chunk kl), then the partner's, whose
    // P and dS are read from LDS at the start; each transposed fragment is
    // read PF steps ahead of its MFMA
    {
      constexpr int PF = 3;
      bf16x8 xp[2], xds[2];                    // the partner's chunks
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        xp[c2] = *(const bf16x8*)slot(0, (half ^ 1) * 2 + c2);
        xds[c2] = *(const bf16x8*)slot(1, (half ^ 1) * 2 + c2);
      }
      // step t: local chunk t / 4, d block (t / 2) % 2, dV (even) or dK (odd)
      auto cfrag = [&](auto step) __attribute__((always_inline)) -> bf16x8 {
        constexpr int t = decltype(step)::value, kl = t >> 2, dbl = (t >> 1) & 1;
        const int kc = kl ^ (2 * half);
        const char* base = ((t & 1) ? qt : dt) + kc * 16 * ROWB;
        const bf16x4 lo = ds_read_tr16(base + voff[0][dbl]);
        const bf16x4 hi = ds_read_tr16(base + voff[1][dbl]);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      bf16x8 fc[PF + 1];
      static_for<PF>([&](auto step) __attribute__((always_inline)) {
        fc[decltype(step)::value] = cfrag(step);
      });
      static_for<16>([&](auto step) __attribute__((always_inline)) {
        constexpr int t = decltype(step)::value, kl = t >> 2, dbl = (t >> 1) & 1;
        if constexpr (t + PF < 16) fc[(t + PF) % (PF + 1)] = cfrag(std::integral_constant<int, t + PF>{});
        bf16x8 pb;
        if constexpr (kl < 2) pb = (t & 1) ? own_ds[kl] : own_p[kl];
        else pb = (t & 1) ? xds[kl - 2] : xp[kl - 2];
        if constexpr (t & 1)
          dkacc[dbl] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fc[t % (PF + 1)], pb, dkacc[dbl], 0, 0, 0);
        else
          dvacc[dbl] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fc[t % (PF + 1)], pb, dvacc[dbl], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      });
    }
  };
  if (j_begin < j_end) issue_tile(0, j_begin);
  for (int j = j_begin; j < j_end; j += 2) {
    tile(std::integral_constant<int, 0>{}, j);
    if (j + 1 < j_end) tile(std::integral_constant<int, 1>{}, j + 1);
  }
  if (kok) {
    // this wave's 64 coordinates of the key's dK and dV rows
#pragma unroll
    for (int dbl = 0; dbl < DBH; ++dbl)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = (half * DBH + dbl) * 32 + g * 8 + hl * 4;
        *(u32x2*)((uint16_t*)a.dk + krow + d) =
            (u32x2){pack_bf16x2(dkacc[dbl][g * 4 + 0] * -a.scale, dkacc[dbl][g * 4 + 1] * -a.scale),
                    pack_bf16x2(dkacc[dbl][g * 4 + 2] * -a.scale, dkacc[dbl][g * 4 + 3] * -a.scale)};
        *(u32x2*)((uint16_t*)a.dv + krow + d) =
            (u32x2){pack_bf16x2(dvacc[dbl][g * 4 + 0], dvacc[dbl][g * 4 + 1]),
                    pack_bf16x2(dvacc[dbl][g * 4 + 2], dvacc[dbl][g * 4 + 3])};
      }
  }
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------

template <int D, bool CAUSAL, bool PACKED>
static hipError_t launch_bwd_t(BwdArgs a, hipStream_t st) {
  constexpr int BM = bwd::BM;
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
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dq_kernel<D, CAUSAL, PACKED>), dim3(grid),
                                 dim3(bwd::NW * 64), args, 0, st);
  if (e != hipSuccess) return e;
  if constexpr (D == 64)
    return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dkdv_kernel<D, CAUSAL, PACKED>), dim3(grid),
                           dim3(bwd::NW * 64), args, 0, st);
  else
    return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dkdv_pair_kernel<D, CAUSAL, PACKED>), dim3(grid),
                           dim3(512), args, 0, st);
}

template <int D>
static hipError_t launch_bwd_d(const BwdArgs& a, bool causal, bool packed, hipStream_t st) {
  if (packed) return causal ? launch_bwd_t<D, true, true>(a, st) : launch_bwd_t<D, false, true>(a, st);
  return causal ? launch_bwd_t<D, true, false>(a, st) : launch_bwd_t<D, false, false>(a, st);
}

hipError_t launch_attn_bwd(const BwdArgs& a, int d, bool causal, bool packed, hipStream_t st) {
  return d == 128 ? launch_bwd_d<128>(a, causal, packed, st) : launch_bwd_d<64>(a, causal, packed, st);
}

int bwd_rows_per_workgroup() { return bwd::BM; }

// ---------------------------------------------------------------------------
// fixed scratch of the no-allocation entry point
// ---------------------------------------------------------------------------

// D per row for callers that cannot allocate: a file-scope device array, one
// copy per GPU, alive until the process ends.  In host code the name is only a
// stand-in for the symbol; kernels get the device address that
// hipGetSymbolAddress returns, looked up once per device.
static __device__ __align__(256) float scratch[kBwdScratchRows];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t bwd_scratch_address(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      p = static_cast<float*>(addr);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace iaea
