// Block-scaled fp8 (OCP e4m3) exact attention forward for gfx950, d = 128.
//
// Same method as the bf16 kernel - query blocks outer, key/value tiles
// inner, running maximum m, normaliser l and weighted sum u per query row,
// u / l once at the end ("Flash Attention và IO", section "Softmax qua nhiều
// khối cần thống kê chạy"; FlashAttention-2 part of "FlashAttention,
// pelatihan multi-GPU, dan kuantisasi bobot", section 1) - with the FP8
// operands and per-tile scales of that section's FlashAttention-3 part.
//
// Scales.  Token t of (b, h) holds e4m3(byte) * scale[b][h][t / 128]; for
// packed documents the blocks restart at each document's first token and
// token t of document b uses slot cu[b] / 128 + b + t / 128 of the head's row
// scale[h][.] (t counted from the document start).  A
// wave's 32 query rows and a 64-key tile each lie inside one 128-token block,
// so each contraction sees one scale per operand and the dequantisation
// factors out of the MFMA: S = scale * sq * sk * (Q^ K^T), and a tile's
// P.V contribution carries one sv.  No scale is shared across blocks of 128
// tokens, so a token never influences the scale of an earlier block (the
// causal-leakage concern of "FLAMIA: Blackwell Üzerinde Hızlı ve Nedensel
// Olarak Güvenli Eğitim İçin Flash Mikro-Ölçeklemeli Dikkat Mekanizması",
// section "Uzun Bağlamlarda Dikkat (Attention) Maliyeti ve Blackwell
// Mimarisi").
//
// P for the P.V contraction.  The reference maximum m is lazy, as in the
// bf16 kernel: a tile's weights are formed against the current m, which moves
// only when some lane's weights sum to more than 2^64 (and on a row's first
// tile).  P enters P.V as two e4m3 terms with a power-of-two scale per query
// (both lanes that hold its two 32-key halves use it): with the query's 64
// weights in the tile summing to less than 2^E, hi = e4m3(P 2^(8-E)) and
// lo = e4m3((P - hi 2^(E-8)) 2^(13-E)), and the MFMA's E8M0 operand scales
// apply 2^(E-8) and 2^(E-13) back.  P 2^(8-E) < 256, where e4m3 steps by at
// most 16, so the remainder is at most 2^(E-5) and lo at most 256 (< 448).  The
// tile's V scale joins them: its power-of-two part in the same E8M0 scale,
// the rest f = sv / 2^e in [1, 2) in the exponent of the weights (P' = P f).
// The accumulator therefore stays in real units, with no per-tile rescale,
// and the scale of a tile's P depends on that tile only.  l sums the
// unquantised fp32 P.
// MI355X mapping: S^T = K Q^T on v_mfma_f32_32x32x16_bf16 from e4m3 operands
// converted exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8; MX block scales
// applied in the same conversion), O^T = V^T P^T on
// v_mfma_scale_f32_32x32x64_f8f6f4 (every lane owns one query column, as in
// the bf16 kernel); direct global->LDS loads of fp8 K/V tiles into
// double-buffered, swizzled LDS; V^T fragments from ds_read_b64_tr_b8.
// Why the scores are not on the fp8 instruction: it sums its 64 products in
// groups of eight consecutive ones and keeps, in each group, only the bits
// down to 2^-13 of the group's largest product exponent (the sum of the two
// operands' exponents), truncating the rest.  With the +-20 outliers of
// block-scaled inputs a group can hold one 448 x 448 product beside ordinary
// ones, whose low bits are then lost: scores move by up to ~1e-2, and O, where
// two keys of weight ~1/2 carry +-20 values, by several times 5e-2.  In P.V the
// weights' power-of-two scale keeps every product of a group within the
// dynamic range where this costs ~2^-13 relative.
#include "attn_common.h"
#include "attn_kernels.h"

namespace iaea {

namespace fp8 {

constexpr int D = 128;
constexpr int BN = 64;          // keys per tile
constexpr int NW = 4;           // waves per workgroup, 32 query rows each
constexpr int BM = 32 * NW;     // = 128: one scale block of queries
constexpr int ROWB = D;         // bytes per K/V row
constexpr int TILE = BN * ROWB; // 8 KB
constexpr int CPW = TILE / 1024 / NW;
constexpr uint32_t kScaleOne = 0x7f7f7f7fu;     // E8M0 2^0 in every byte
constexpr float kLazyMax = 0x1p64;              // as in the bf16 kernel

// 16-byte-granule swizzle of a 128-byte row (a permutation of row bits 1..3):
// conflict-free for the K fragment reads (16 consecutive rows, one granule)
// and for the transposed V reads (8 rows x 2 granules per half-wave).
__device__ __forceinline__ int swz(int row) {
  return (((row >> 1) & 1) << 1) | ((row >> 2) & 1) | (((row >> 3) & 1) << 2);
}
__device__ __forceinline__ int lds_off(int row, int granule) {
  return row * ROWB + ((granule ^ swz(row)) << 4);
}

// The restrict-qualified pointer gives the read alias-scope metadata, so the
// compiler does not wait for the next tile's in-flight LDS DMA before it.
__device__ __forceinline__ i32x2 ds_read_tr8(const char* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((IAEA_LDS i32x2*)(p));
}

// Eight e4m3 values (two dwords, byte order) to bf16, times the power of two
// `sc` (an E8M0 scale as a float, or 1): exact, since every e4m3 value times a
// power of two in bf16's normal range is a bf16 value.
__device__ __forceinline__ bf16x8 cvt8(uint32_t w0, uint32_t w1, float sc) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, true);
  return (bf16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
// E8M0 byte -> the float 2^(byte - 127) (bytes 1 .. 254)
__device__ __forceinline__ float e8m0_float(uint32_t byte) { return __uint_as_float(byte << 23); }

__device__ __forceinline__ f32x16 mfma(const i32x8& a, const i32x8& b, const f32x16& c, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, kScaleOne, 0, sb);
}
// both operand scales, byte OA of sa and byte OB of sb.  Scale block 0 of the
// 64-long contraction is bytes 0..15 of every lane's operand and takes its
// scale from the lane in the lower half-wave; block 1 is bytes 16..31, scaled
// from the upper half-wave's lane.
template <int OA, int OB>
__device__ __forceinline__ f32x16 mfma2(const i32x8& a, const i32x8& b, const f32x16& c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OA, sa, OB, sb);
}

}  // namespace fp8

template <int P> struct F8Parity { static constexpr int value = P; };

// MX: MXFP8 operands instead (E8M0 byte scales per 32 elements: along d for
// Q and K, per token; along 32-token blocks for V, per coordinate), applied by
// the matrix instruction itself; P's power of two then goes per 32-key block.
template <bool CAUSAL, bool PACKED, bool MX>
__global__ void __launch_bounds__(fp8::NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
attn_fwd_fp8_kernel(FwdArgs a) {
  using namespace fp8;
  // K0 K1 V0 V1, then (MX) the K and V scale bytes of both buffers
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE + (MX ? 4 * 256 : 0)];
  [[maybe_unused]] char* const kscl = smem + 4 * TILE;         // [2][64 keys][4 groups]
  [[maybe_unused]] char* const vscl = smem + 4 * TILE + 512;   // [2][2 blocks][128 coordinates]

  int h, b, seq_start, seq_len, qblk;
  if (!decode_work<BM, CAUSAL, PACKED>(a, blockIdx.x, h, b,
                                      seq_start, seq_len, qblk))
    return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5;
  const int l32 = lane & 31;
  const int q0 = qblk * BM;
  const int wq0 = q0 + wave * 32;
  const int kv_end = CAUSAL ? min(seq_len, q0 + BM) : seq_len;
  const int n_iter = (kv_end + BN - 1) / BN;
  const int wave_kv_end = CAUSAL ? min(seq_len, wq0 + 32) : seq_len;
  const int wave_iters = (wq0 < seq_len) ? (wave_kv_end + BN - 1) / BN : 0;

  const int64_t rs = (int64_t)a.H * D;   // bytes between consecutive tokens
  const int64_t head_off = (int64_t)h * D;
  const uint8_t* __restrict__ qg = (const uint8_t*)a.q;
  const uint8_t* __restrict__ kg = (const uint8_t*)a.k;
  const uint8_t* __restrict__ vg = (const uint8_t*)a.v;
  // this (sequence, head)'s scales; packed documents keep block k of
  // document b in slot seq_start / 128 + b + k of the head's row
  const int64_t sbase = PACKED ? (int64_t)h * a.nsb + seq_start / 128 + b : (int64_t)(b * a.H + h) * a.nsb;
  const float* __restrict__ ks = a.k_scale + sbase;
  const float* __restrict__ vs = a.v_scale + sbase;
  const float sq = (!MX && wq0 < seq_len) ? a.q_scale[sbase + wq0 / 128] : 1.f;
  const float cq = a.c * sq;
  // MX: the base of this head's K scale bytes and of this (sequence, head)'s
  // rows of V scale blocks
  [[maybe_unused]] const uint8_t* const ksb = (const uint8_t*)a.k_scale + (int64_t)h * 4;
  [[maybe_unused]] const uint8_t* const vsb =
      (const uint8_t*)a.v_scale +
      (PACKED ? (int64_t)h * a.nsb + seq_start / 32 + b : (int64_t)(b * a.H + h) * a.nsb) * D;

  // ---- Q as bf16 fragments, the B operand of S^T = K Q^T on
  // v_mfma_f32_32x32x16_bf16.  The fp8 matrix instruction is not used for the
  // scores: it sums its products in groups of eight, dropping the bits below
  // 2^-13 of the largest operand-exponent pair of each group, and with outliers
  // that moves scores by up to ~1e-2.  e4m3 values convert to bf16 exactly,
  // and the bf16 instruction accumulates to fp32 accuracy.  Step st of the 128
  // coordinates covers d = 32 (st / 2) + 16 half + 8 (st % 2) + 0..7, so one
  // 16-byte granule (2 (st / 2) + half) of a row serves steps 2g and 2g + 1; K
  // fragments follow the same order.  MX: the 32-coordinate block of steps 2g,
  // 2g + 1 is g, and its E8M0 scale is applied in the conversion.
  bf16x8 qb[8];
  {
    const int t = wq0 + l32;
    const bool ok = t < seq_len;
    const uint8_t* p = qg + (int64_t)(seq_start + (ok ? t : 0)) * rs + head_off + 16 * hl;
    [[maybe_unused]] uint32_t qsw = 0x7f7f7f7fu;
    if constexpr (MX) {
      if (ok) qsw = *(const uint32_t*)((const uint8_t*)a.q_scale + ((int64_t)(seq_start + t) * a.H + h) * 4);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x4 raw = ok ? *(const u32x4*)(p + 32 * g) : (u32x4){0u, 0u, 0u, 0u};
      raw ^= a.qsign;
      const float sc = MX ? e8m0_float((qsw >> (8 * g)) & 0xffu) : 1.f;
      qb[2 * g] = cvt8(raw[0], raw[1], sc);
      qb[2 * g + 1] = cvt8(raw[2], raw[3], sc);
    }
  }

  // ---- K/V tiles: HBM -> LDS (buffer_load_dwordx4 ... lds, as in the bf16
  // kernel); the buffer size ends at the end of the sequence, so rows past it
  // read as zeros
  uint32_t lane_off[CPW];
#pragma unroll
  for (int cc = 0; cc < CPW; ++cc) {
    const int byte = (wave * CPW + cc) * 1024 + lane * 16;
    const int row = byte / ROWB;
    const int g = ((byte % ROWB) >> 4) ^ swz(row);
    lane_off[cc] = (uint32_t)((int64_t)row * rs + head_off + g * 16);
  }
  [[maybe_unused]] const uint32_t row_bytes = (uint32_t)rs;
  auto issue_tile = [&](const uint8_t* __restrict__ src, int buf, int j) __attribute__((always_inline)) {
#if __HIP_DEVICE_COMPILE__   // the 16-byte LDS DMA form exists only for the device target
    const int kv0 = j * BN;
    const uint32_t nrec = (uint32_t)min(seq_len - kv0, BN) * row_bytes;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const char*)src + (uint64_t)(uint32_t)(seq_start + kv0) * row_bytes), (short)0, (int)nrec,
        kBufferFlags);
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (IAEA_LDS void*)(smem + buf * TILE + (wave * CPW + cc) * 1024),
                                               16, lane_off[cc], 0, 0, 0);
#endif
  };
  // MX: the tile's scale bytes, one dword per lane (rows past the end read 0,
  // a finite scale on zero data): wave 0 the 64 keys' four groups, wave 1 the
  // two 32-token V blocks' 128 coordinates
  auto issue_scales = [&](int buf, int j) __attribute__((always_inline)) {
#if __HIP_DEVICE_COMPILE__
    if constexpr (MX) {
      const int kv0 = j * BN;
      if (wave == 0) {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(ksb + (int64_t)(seq_start + kv0) * a.H * 4), (short)0,
            (int)((uint32_t)min(seq_len - kv0, BN) * (uint32_t)a.H * 4u), kBufferFlags);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (IAEA_LDS void*)(kscl + buf * 256), 4, lane * a.H * 4, 0, 0, 0);
      } else if (wave == 1) {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(vsb + (int64_t)(kv0 / 32) * D), (short)0, min((seq_len - kv0 + 31) / 32, 2) * D, kBufferFlags);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (IAEA_LDS void*)(vscl + buf * 256), 4, lane * 4, 0, 0, 0);
      }
    }
#else
    (void)buf; (void)j;
#endif
  };

  // ---- loop-invariant LDS read offsets.  K fragment: row kb*32 + l32, bytes
  // dc*64 + 32*half + 0..31 (granules 4dc + 2half, +1).  V^T fragment
  // (ds_read_b64_tr_b8): in each 16-lane group, source lane s points at key
  // row K(s/2) and d offset 8*(s%2) of the group's 16 d columns; lane i then
  // holds d column i of the eight keys K(0..7).  Read t covers the keys of
  // bytes 8t..8t+7 of the P^T operand.
  uint32_t koff[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) koff[g] = lds_off(l32, 2 * g + hl);
  uint32_t voff[4][4];
  {
    const int g16 = lane >> 4;
    const int s = lane & 15;
    const int r = s >> 1;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int row = (t >> 1) * 32 + 16 * (t & 1) + 4 * hl + (r >> 2) * 8 + (r & 3);
        const int d = db * 32 + 16 * (g16 & 1) + 8 * (s & 1);
        voff[t][db] = lds_off(row, d >> 4) + (d & 15);
      }
  }

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = (f32x16){};
  float m_run = -INFINITY;   // lazy reference maximum, in the exp2 domain (scales folded in)
  float l_run = 0.f;         // this lane's sum of the fp32 weights P (half of the row's keys)

  auto step = [&](auto par, int it) {
    constexpr int P = decltype(par)::value;
    if (it + 1 < n_iter) {
      issue_tile(kg, P ^ 1, it + 1);
      issue_tile(vg, 2 + (P ^ 1), it + 1);
      issue_scales(P ^ 1, it + 1);
    }
    if (it < wave_iters) {
      const int kv0 = it * BN;
      const char* kt = smem + P * TILE;
      const char* vt = smem + (2 + P) * TILE;
      const float sk = MX ? 1.f : ks[kv0 / 128];
      const float sv = MX ? 1.f : vs[kv0 / 128];
      const float ct = cq * sk;
      // sv = f 2^esv with f in [1, 2)
      const float f = MX ? 1.f : 2.f * __builtin_amdgcn_frexp_mantf(sv);
      const int esv = MX ? 0 : __builtin_amdgcn_frexp_expf(sv) - 1;
      const float lf = MX ? 0.f : __log2f(f);
      // MX: the scale bytes of this lane's key rows (K, one per 32-coordinate
      // block) and of its V block
      [[maybe_unused]] uint32_t ksw[2] = {0x7f7f7f7fu, 0x7f7f7f7fu};
      [[maybe_unused]] uint32_t vsc = kScaleOne;
      if constexpr (MX) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) ksw[kb] = *(const uint32_t*)(kscl + P * 256 + (kb * 32 + l32) * 4);
        const uint8_t* vp = (const uint8_t*)vscl + P * 256 + hl * 128 + l32;
        vsc = (uint32_t)vp[0] | ((uint32_t)vp[32] << 8) | ((uint32_t)vp[64] << 16) | ((uint32_t)vp[96] << 24);
      }

      // S^T for the two 32-key halves of the tile on the bf16 instruction (K
      // rows converted from e4m3 exactly, MX block scales applied), masked
      f32x16 s[2];
      auto scores = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const u32x4 x = *(const u32x4*)(kt + kb * 32 * ROWB + koff[g]);
            const float sc = MX ? e8m0_float((ksw[kb] >> (8 * g)) & 0xffu) : 1.f;
            const bf16x8 k0 = cvt8(x[0], x[1], sc), k1 = cvt8(x[2], x[3], sc);
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qb[2 * g], g == 0 ? (f32x16){} : s[kb], 0, 0, 0);
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qb[2 * g + 1], s[kb], 0, 0, 0);
          }
        if ((kv0 + BN > seq_len) || (CAUSAL && kv0 + BN - 1 > wq0)) {
          const int lim = (CAUSAL ? min(wq0 + l32, seq_len - 1) : seq_len - 1) - (kv0 + hl * 4);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (kb * 32 + (r >> 2) * 8 + (r & 3) > lim) s[kb][r] = -INFINITY;
        }
      };
      // P' = exp2(s ct - m + log2 f) = P f in place of the scores; returns the
      // lane's sum of P' (and, in xb, its sum over each 32-key half)
      float xb[2];
      auto weights = [&]() __attribute__((always_inline)) -> float {
        const float shift = m_run - lf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          float x0 = 0.f, x1 = 0.f;
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            s[kb][r] = fast_exp2(__builtin_fmaf(s[kb][r], ct, -shift));
            s[kb][r + 1] = fast_exp2(__builtin_fmaf(s[kb][r + 1], ct, -shift));
            if (r & 2) x1 += s[kb][r] + s[kb][r + 1];
            else       x0 += s[kb][r] + s[kb][r + 1];
          }
          xb[kb] = x0 + x1;
        }
        return xb[0] + xb[1];
      };
      scores();
      // a row's first tile (the same tile for every lane of the wave) takes
      // its maximum before the weights; later tiles form their weights first
      const bool first = m_run == -INFINITY;
      float lx = 0.f;
      if (!first) lx = weights();
      if (__ballot(first || lx > kLazyMax) != 0) {
        // the reference moves to the tile maximum (rare after the first tile;
        // then the scores are formed again, their registers hold weights)
        if (!first) scores();
        float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s[0][r], s[1][r]));
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        const float mxs = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * ct;
        const float m_new = first ? mxs : m_run + fmaxf(mxs - m_run, 0.f);
        const float alpha = first ? 1.f : fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
        lx = weights();
      }
      l_run = __builtin_fmaf(lx, 1.f / f, l_run);

      // P' as two e4m3 terms with the query's power-of-two scale 2^E above the
      // sum of its 64 weights in this tile: hi = e4m3(P' 2^(8-E)),
      // lo = e4m3((P' - hi 2^(E-8)) 2^(13-E)).  The conversions apply the
      // power-of-two part of their scale operand.  The matrix instruction takes
      // one B scale per column, so both lanes holding a query's 32-key halves
      // (l and l ^ 32) must quantise against the same E.
      // (MX: the instruction scales each 32-key block from its own lane, so E
      // is per block: block kb's 32 keys are 16 in each of lanes l and l ^ 32.)
      int Eb[2];
      if constexpr (MX) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const auto bsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(xb[kb]), __float_as_uint(xb[kb]), false, false);
          const float bq = __uint_as_float(bsw[0]) + __uint_as_float(bsw[1]);
          Eb[kb] = bq > 0.f ? __builtin_amdgcn_frexp_expf(bq) : 0;
        }
      } else {
        const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lx), __float_as_uint(lx), false, false);
        const float lq = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
        Eb[0] = Eb[1] = lq > 0.f ? __builtin_amdgcn_frexp_expf(lq) : 0;
      }
      const int E = hl ? Eb[1] : Eb[0];         // the block this lane's operand scale covers
      i32x8 phi, plo;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        // p index j -> S register j / 16, j % 16: bytes 0..3 of word w are p[4w .. 4w + 3]
        const int j = 4 * w, kb = j >> 4, r = j & 15;
        const float sh = __builtin_amdgcn_ldexpf(1.f, Eb[kb] - 8), sl = __builtin_amdgcn_ldexpf(1.f, Eb[kb] - 13);
        s16x2 h2 = {0, 0}, l2 = {0, 0};
        h2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h2, s[kb][r], s[kb][r + 1], sh, false);
        h2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h2, s[kb][r + 2], s[kb][r + 3], sh, true);
        const uint32_t hw = __builtin_bit_cast(uint32_t, h2);
        const auto b01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw, sh, false);
        const auto b23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw, sh, true);
        l2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l2, s[kb][r] - b01[0], s[kb][r + 1] - b01[1], sl, false);
        l2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l2, s[kb][r + 2] - b23[0], s[kb][r + 3] - b23[1], sl, true);
        phi[w] = (int)hw;
        plo[w] = (int)__builtin_bit_cast(uint32_t, l2);
      }
      // E8M0 scales of the P^T operand: 2^(E-8) and 2^(E-13) times the
      // power-of-two part 2^esv of the V scale (clamped to the format's range;
      // a clamp only touches tiles whose weights are ~2^-100 of the row's)
      // (the byte is repeated in all four operand bytes, as the fixed scales are)
      const uint32_t ehi = (uint32_t)min(max(127 + E - 8 + esv, 0), 254) * 0x01010101u;
      const uint32_t elo = (uint32_t)min(max(127 + E - 13 + esv, 0), 254) * 0x01010101u;

      // O^T += V^T P'^T (hi and lo terms), 64 keys per MFMA
      static_for<4>([&](auto dbi) __attribute__((always_inline)) {
        constexpr int db = decltype(dbi)::value;
        i32x8 vf;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const i32x2 x = ds_read_tr8(vt + voff[t][db]);
          vf[2 * t] = x[0];
          vf[2 * t + 1] = x[1];
        }
        if constexpr (MX) {
          oacc[db] = mfma2<db, 0>(vf, phi, oacc[db], vsc, ehi);
          oacc[db] = mfma2<db, 0>(vf, plo, oacc[db], vsc, elo);
        } else {
          oacc[db] = mfma(vf, phi, oacc[db], ehi);
          oacc[db] = mfma(vf, plo, oacc[db], elo);
        }
      });
    }
    __syncthreads();
  };

  if (n_iter > 0) {
    issue_tile(kg, 0, 0);
    issue_tile(vg, 2, 0);
    issue_scales(0, 0);
  }
  __syncthreads();
  for (int it = 0; it < n_iter; it += 2) {
    step(F8Parity<0>{}, it);
    if (it + 1 < n_iter) step(F8Parity<1>{}, it + 1);
  }

  // ---- epilogue: O = u / l, LSE = ln2 * (m + log2 l)
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
  const float l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  const int t = wq0 + l32;
  if (t < seq_len) {
    const bool any = l_tot > 0.f;
    const float mul = any ? 1.f / l_tot : 0.f;
    if (hl == 0)
      a.lse[(PACKED ? (int64_t)h * a.N + seq_start : (int64_t)(b * a.H + h) * a.N) + t] =
          any ? kLn2 * (m_run + __log2f(l_tot)) : -INFINITY;
    const int64_t orow = (int64_t)(seq_start + t) * rs + head_off;   // element index (D per token-head)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + g * 8 + hl * 4;
        *(u32x2*)((uint16_t*)a.o + orow + d) =
            (u32x2){pack_bf16x2(oacc[db][g * 4 + 0] * mul, oacc[db][g * 4 + 1] * mul),
                    pack_bf16x2(oacc[db][g * 4 + 2] * mul, oacc[db][g * 4 + 3] * mul)};
      }
  }
}

template <bool CAUSAL, bool PACKED, bool MX>
static hipError_t launch_fp8(FwdArgs a, hipStream_t st) {
  if (PACKED) {
    a.slots = (a.N + fp8::BM - 1) / fp8::BM + a.B;
    a.n_work = a.H * a.slots;
  } else {
    a.slots = (a.N + fp8::BM - 1) / fp8::BM;
    a.n_work = a.B * a.H * a.slots;
  }
  const int grid = (a.n_work + kXcds - 1) / kXcds * kXcds;
  a.per_xcd = grid / kXcds;
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_fp8_kernel<CAUSAL, PACKED, MX>), dim3(grid),
                         dim3(fp8::NW * 64), args, 0, st);
}

hipError_t launch_attn_fwd_fp8(const FwdArgs& a, bool causal, bool packed, hipStream_t st) {
  if (packed) return causal ? launch_fp8<true, true, false>(a, st) : launch_fp8<false, true, false>(a, st);
  return causal ? launch_fp8<true, false, false>(a, st) : launch_fp8<false, false, false>(a, st);
}

hipError_t launch_attn_fwd_mxfp8(const FwdArgs& a, bool causal, bool packed, hipStream_t st) {
  if (packed) return causal ? launch_fp8<true, true, true>(a, st) : launch_fp8<false, true, true>(a, st);
  return causal ? launch_fp8<true, false, true>(a, st) : launch_fp8<false, false, true>(a, st);
}

}  // namespace iaea
