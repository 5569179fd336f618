// Block-scaled e4m3 quantisation of bf16 tensors for gfx950 (MI355X).
//
// The FP8 path of "FlashAttention, pelatihan multi-GPU, dan kuantisasi bobot"
// (section 1, its FlashAttention-3 part) feeds the attention kernels operands
// that carry one scale per tile; FLAMIA ("FLAMIA: Blackwell Üzerinde Hızlı ve
// Nedensel Olarak Güvenli Eğitim İçin Flash Mikro-Ölçeklemeli Dikkat
// Mekanizması", sections "Uzun Bağlamlarda Dikkat (Attention) Maliyeti ve
// Blackwell Mimarisi" and "FLAMIA Mimarisi ve Temel Tasarım İlkeleri") counts
// the quantisation step in its timings and keeps every scale on one side of
// the causal boundary, for packed documents too.  This kernel is that step:
// for every block of 128 consecutive tokens of one (sequence or document,
// head), over all d,
//     s = amax / 448 in fp32 (1 for an all-zero block),
//     byte = e4m3(x / s), the quotient rounded once to fp32 and then to the
//            nearest e4m3 value (ties to even, 448 the largest),
// with document-local blocks for packed input (a document's first block
// starts at its first token; block k of document d keeps its scale in slot
// cu[d] / 128 + d + k of the head's row of scales).
//
// MI355X mapping: the work is a stream through HBM (2 bytes read and 1 written
// per element), so the kernel is built for bandwidth: one 256-thread
// workgroup per block (two or four blocks per workgroup, with the later
// blocks' loads issued first, measured slower), 16-byte loads that cover whole 256-byte token rows, the
// block maximum taken on the bf16 bit patterns (the magnitude order of
// non-negative floats is the integer order of their bits; v_pk_max_u16 takes
// two at a time), one wave reduction plus one LDS exchange for the block
// maximum, and v_cvt_pk_fp8_f32 for the rounding to e4m3.  The quotient x / s
// needs to be the correctly rounded one; s is the same for the whole block, so
// one division gives r = RN(1 / s) and each element then takes q0 = RN(x r)
// and two correction steps q <- RN(q + (x - q s) r), the remainder x - q s
// exact by fma.  The last step is Markstein's: it returns RN(x / s) when r is
// within half an ulp of 1 / s and q within one ulp of x / s.  q0 can be 1.5
// ulp off; after the first step q is within half an ulp plus 2^-24 of one,
// which the second step needs; the sign is copied from x, so -0 stays -0.
// Quotients below the fp32 normal range end as e4m3 zero either way.
#include "attn_common.h"
#include "attn_kernels.h"

namespace iaea {

namespace qz {
constexpr int BLK = 128;   // tokens per scale block
constexpr int NT = 256;    // threads per workgroup
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
}  // namespace qz

// One work item: block `slot` of head h of sequence b (packed: of the
// document that owns the slot).  Returns false for a slot no block maps to.
struct QItem {
  int64_t base;   // element offset of the block's first token, this head
  int64_t sidx;   // index of its scale
  int nt;         // tokens in the block
};

template <bool PACKED>
__device__ __forceinline__ bool q_item(const QuantArgs& a, int item, int D, QItem& it) {
  const int slot = item % a.nsb;
  const int rest = item / a.nsb;
  const int h = rest % a.H;
  const int b = rest / a.H;
  int seq_start, seq_len, blk;
  if constexpr (!PACKED) {
    blk = slot;
    seq_start = b * a.N;
    seq_len = a.N;
    it.sidx = ((int64_t)b * a.H + h) * a.nsb + slot;
  } else {
    // the document of this slot: the largest doc with cu[doc] / 128 + doc <=
    // slot (that function of doc is strictly increasing)
    int lo = 0, hi = a.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.cu_seqlens[mid] / qz::BLK + mid <= slot) lo = mid;
      else hi = mid - 1;
    }
    seq_start = a.cu_seqlens[lo];
    seq_len = a.cu_seqlens[lo + 1] - seq_start;
    blk = slot - (seq_start / qz::BLK + lo);
    if (blk * qz::BLK >= seq_len) return false;
    it.sidx = (int64_t)h * a.nsb + slot;
  }
  const int t0 = blk * qz::BLK;
  it.nt = min(qz::BLK, seq_len - t0);
  it.base = (int64_t)(seq_start + t0) * a.H * D + (int64_t)h * D;
  return true;
}

// One workgroup per block: load it, take its maximum, quantise and store.
template <int D, bool PACKED>
__global__ void __launch_bounds__(qz::NT) quantize_fp8_kernel(QuantArgs a) {
  constexpr int GPR = D / 8;                  // 16-byte bf16 granules per token row
  constexpr int NG = qz::BLK * GPR / qz::NT;  // granules per thread
  static_assert(NG * qz::NT == qz::BLK * GPR, "block must split evenly over the threads");
  const int tid = threadIdx.x;
  const int64_t rs = (int64_t)a.H * D;        // elements (and output bytes) between tokens
  QItem it;
  if (!q_item<PACKED>(a, blockIdx.x, D, it)) return;   // no block maps to this slot
  const uint16_t* __restrict__ x = (const uint16_t*)a.x + it.base;
  uint8_t* __restrict__ y = (uint8_t*)a.y + it.base;

  // ---- load the block (a wave covers 64 / GPR whole token rows per step)
  u32x4 v[NG];
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int g = i * qz::NT + tid;
    const int row = g / GPR, col = g % GPR;
    v[i] = row < it.nt ? *(const u32x4*)(x + row * rs + col * 8) : (u32x4){0u, 0u, 0u, 0u};
  }

  // ---- block maximum of |x| on the bit patterns: wave, then workgroup
  qz::u16x2 m2 = {0, 0};
#pragma unroll
  for (int i = 0; i < NG; ++i)
#pragma unroll
    for (int w = 0; w < 4; ++w)
      m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(qz::u16x2, v[i][w] & 0x7fff7fffu));
  uint32_t mb = m2[0] > m2[1] ? m2[0] : m2[1];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mb = max(mb, (uint32_t)__shfl_xor((int)mb, off));
  __shared__ uint32_t wmax[qz::NT / 64];
  if ((tid & 63) == 0) wmax[tid >> 6] = mb;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < qz::NT / 64; ++w) mb = max(mb, wmax[w]);
  const float amax = __uint_as_float(mb << 16);
  const float s = amax == 0.f ? 1.f : __fdiv_rn(amax, 448.f);
  const float rcp = __fdiv_rn(1.f, s);
  if (tid == 0) a.scales[it.sidx] = s;
  auto quot = [&](float xv) __attribute__((always_inline)) {
    const float q0 = xv * rcp;
    const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, s, xv), rcp, q0);
    // x = -0 would come out +0 (the corrections add +0 to -0)
    return __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q1, s, xv), rcp, q1), xv);
  };

  // ---- quantise: x / s rounded to fp32, then to e4m3
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int g = i * qz::NT + tid;
    const int row = g / GPR, col = g % GPR;
    uint32_t w2[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const uint32_t p = v[i][2 * half], r = v[i][2 * half + 1];
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(quot(__uint_as_float(p << 16)),
                                                 quot(__uint_as_float(p & 0xffff0000u)), 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(quot(__uint_as_float(r << 16)),
                                             quot(__uint_as_float(r & 0xffff0000u)), word, true);
      w2[half] = (uint32_t)word;
    }
    if (row < it.nt) *(u32x2*)(y + row * rs + col * 8) = (u32x2){w2[0], w2[1]};
  }
}

// ---------------------------------------------------------------------------
// Incoherent processing ("FlashAttention, pelatihan multi-GPU, dan kuantisasi
// bobot", section 1, its FlashAttention-3 part: Q and K multiplied by a random
// orthogonal matrix before quantisation, to soften outliers).  The matrix is
// M = diag(s) H_d, random signs on the input coordinates and then the
// Sylvester Hadamard matrix (entry (i, j) = (-1)^popcount(i & j)), left
// unnormalised (M M^T = d I: the attention on rotated Q and K takes scale / d).
// Each rotated value is a signed sum of d bf16 values; the sum is taken in
// fp64, exact whenever the row's nonzero exponents span at most 38 binades
// (a bf16 value is an 8-bit integer times a power of two), and rounded once
// to fp32 (a sum that is exactly zero as +0); the block quantisation above
// then runs on those fp32 values.
//
// MI355X mapping: one workgroup per 128-token block as above; a token row is
// spread over D / 32 lanes of one quad, 32 coordinates each (four 16-byte
// loads), and the transform is the in-place fast Walsh-Hadamard butterfly:
// five stages inside the lane's registers, then log2(D / 32) stages across
// the row's lanes by DPP quad permutations (no LDS traffic).  The block
// maximum is taken on the fp32 bit patterns.
// ---------------------------------------------------------------------------
// v from the lane whose index differs in the bit(s) of the quad permutation
// CTRL (DPP, within each group of four lanes), for a double as two dwords
template <int CTRL>
__device__ __forceinline__ double dpp_swap(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xf, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xf, 0xf, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

template <int D, bool PACKED>
__global__ void __launch_bounds__(qz::NT) quantize_fp8_rot_kernel(QuantArgs a) {
  constexpr int EPL = 32;                     // coordinates per lane
  constexpr int LPR = D / EPL;                // lanes per token row: 4 (d = 128) or 2 (d = 64)
  constexpr int RPP = qz::NT / LPR;           // token rows per pass
  constexpr int NP = qz::BLK / RPP;           // passes per block
  const int tid = threadIdx.x;
  const int li = tid % LPR;                   // this lane's coordinates: li * 32 ...
  const int64_t rs = (int64_t)a.H * D;
  QItem it;
  if (!q_item<PACKED>(a, blockIdx.x, D, it)) return;
  const uint16_t* __restrict__ x = (const uint16_t*)a.x + it.base;
  uint8_t* __restrict__ y = (uint8_t*)a.y + it.base;

  u32x4 raw[NP][4];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int row = p * RPP + tid / LPR;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      raw[p][c] = row < it.nt ? *(const u32x4*)(x + row * rs + li * EPL + c * 8) : (u32x4){0u, 0u, 0u, 0u};
  }
  // sign flips as xor masks on the bf16 pairs: word w of chunk c holds
  // coordinates 8c + 2w (low half) and 8c + 2w + 1 (high half)
  const u32x4 sg0 = *(const u32x4*)(a.signs + li * EPL);
  const u32x4 sg1 = *(const u32x4*)(a.signs + li * EPL + 16);
  uint32_t flip[4][4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int e0 = 8 * c + 2 * w, e1 = e0 + 1;
      const uint32_t s0 = (e0 < 16 ? sg0 : sg1)[(e0 & 15) >> 2], s1 = (e1 < 16 ? sg0 : sg1)[(e1 & 15) >> 2];
      const uint32_t b0 = (s0 >> ((e0 & 3) * 8 + 7)) & 1u;
      const uint32_t b1 = (s1 >> ((e1 & 3) * 8 + 7)) & 1u;
      flip[c][w] = (b0 << 15) | (b1 << 31);
    }

  float r[NP][EPL];
  uint32_t mb = 0;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    double v[EPL];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t u = raw[p][c][w] ^ flip[c][w];
        v[8 * c + 2 * w] = (double)__uint_as_float(u << 16);
        v[8 * c + 2 * w + 1] = (double)__uint_as_float(u & 0xffff0000u);
      }
#pragma unroll
    for (int hb = 1; hb < EPL; hb <<= 1)
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        if (!(e & hb)) {
          const double s0 = v[e], s1 = v[e + hb];
          v[e] = s0 + s1;
          v[e + hb] = s0 - s1;
        }
    // the row's other lanes: xor 1 (quad permutation 1 0 3 2), then xor 2
    // (2 3 0 1) for d = 128
    {
      const bool upper = (li & 1) != 0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const double o = dpp_swap<0xB1>(v[e]);
        v[e] = upper ? o - v[e] : v[e] + o;
      }
    }
    if constexpr (LPR == 4) {
      const bool upper = (li & 2) != 0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const double o = dpp_swap<0x4E>(v[e]);
        v[e] = upper ? o - v[e] : v[e] + o;
      }
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      r[p][e] = (float)(v[e] + 0.0);          // + 0.0: an exact zero sum becomes +0
      mb = max(mb, __float_as_uint(r[p][e]) & 0x7fffffffu);
    }
  }

  // block maximum: wave, then workgroup
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mb = max(mb, (uint32_t)__shfl_xor((int)mb, off));
  __shared__ uint32_t wmax[qz::NT / 64];
  if ((tid & 63) == 0) wmax[tid >> 6] = mb;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < qz::NT / 64; ++w) mb = max(mb, wmax[w]);
  const float amax = __uint_as_float(mb);
  const float s = amax == 0.f ? 1.f : __fdiv_rn(amax, 448.f);
  const float rcp = __fdiv_rn(1.f, s);
  if (tid == 0) a.scales[it.sidx] = s;
  auto quot = [&](float xv) __attribute__((always_inline)) {
    const float q0 = xv * rcp;
    const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, s, xv), rcp, q0);
    return __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q1, s, xv), rcp, q1), xv);
  };
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int row = p * RPP + tid / LPR;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4 out;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int e = 16 * c + 4 * w;
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(quot(r[p][e]), quot(r[p][e + 1]), 0, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(quot(r[p][e + 2]), quot(r[p][e + 3]), word, true);
        out[w] = (uint32_t)word;
      }
      if (row < it.nt) *(u32x4*)(y + row * rs + li * EPL + 16 * c) = out;
    }
  }
}

template <int D, bool PACKED>
static hipError_t launch_qr(const QuantArgs& a, hipStream_t st) {
  const int64_t grid = (int64_t)a.nsb * a.H * (PACKED ? 1 : a.B);
  void* args[] = {const_cast<QuantArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&quantize_fp8_rot_kernel<D, PACKED>), dim3((unsigned)grid),
                         dim3(qz::NT), args, 0, st);
}

hipError_t launch_quantize_fp8_rotated(const QuantArgs& a, int d, bool packed, hipStream_t st) {
  if (d == 128) return packed ? launch_qr<128, true>(a, st) : launch_qr<128, false>(a, st);
  return packed ? launch_qr<64, true>(a, st) : launch_qr<64, false>(a, st);
}

template <int D, bool PACKED>
static hipError_t launch_q(const QuantArgs& a, hipStream_t st) {
  const int64_t grid = (int64_t)a.nsb * a.H * (PACKED ? 1 : a.B);
  void* args[] = {const_cast<QuantArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&quantize_fp8_kernel<D, PACKED>), dim3((unsigned)grid),
                         dim3(qz::NT), args, 0, st);
}

hipError_t launch_quantize_fp8(const QuantArgs& a, int d, bool packed, hipStream_t st) {
  if (d == 128) return packed ? launch_q<128, true>(a, st) : launch_q<128, false>(a, st);
  return packed ? launch_q<64, true>(a, st) : launch_q<64, false>(a, st);
}

int64_t quantize_fp8_grid(int B, int H, int N, bool packed) {
  const int64_t nb = (N + qz::BLK - 1) / qz::BLK;
  return packed ? (nb + B) * H : nb * H * B;
}

}  // namespace iaea
