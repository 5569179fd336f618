// MXFP8 quantisation of bf16 tensors for gfx950 (MI355X): e4m3 elements with
// one power-of-two scale (E8M0 byte, exponent + 127) per block of 32.
//
// FLAMIA ("FLAMIA: Blackwell Üzerinde Hızlı ve Nedensel Olarak Güvenli Eğitim
// İçin Flash Mikro-Ölçeklemeli Dikkat Mekanizması", section "FLAMIA Mimarisi ve
// Temel Tasarım İlkeleri") runs attention on MXFP8 operands, and its closing
// section warns that micro-scales must not carry information from future
// tokens.  For a block with maximum magnitude amax:
//     e = floor(log2 amax) - 8 (8: the exponent of e4m3's top binade), clamped
//         to [-127, 127]; e = 0 for an all-zero block;
//     byte = e4m3(x / 2^e), rounded to nearest (ties to even), clamped to 448.
// Blocks run along the contraction each operand enters:
//   * along d for Q and K (32 coordinates of one token and head): a scale then
//     depends on its own token only;
//   * along tokens for V (32 consecutive tokens of one head and coordinate),
//     restarting at each packed document's first token; block k of document j
//     keeps its scales in slot cu[j] / 32 + j + k of the head's rows.
//
// MI355X mapping: both are streams through HBM (2 bytes read, 1 + 1/32
// written per element).  Along d: one thread per block, four 16-byte loads,
// the exponent read off the bf16 bits of the maximum.  Along tokens: one wave
// per (sequence, head, 32-token block), each lane two adjacent coordinates, so
// each token row is one coalesced 256-byte load for the wave.  The division by
// 2^e is exact (v_ldexp_f32) and v_cvt_pk_fp8_f32 rounds to e4m3.
#include "attn_common.h"
#include "attn_kernels.h"

namespace iaea {

namespace mxq {
constexpr int BLK = 32;
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// floor(log2 |x|) - 8 from the bf16 bits of |x| (nonzero), clamped
__device__ __forceinline__ int block_exp(uint32_t m) {
  if (m == 0) return 0;
  const int ef = (int)(m >> 7);
  const int fl = ef > 0 ? ef - 127 : -133 + (31 - __builtin_clz(m));   // subnormal: 2^-133 * mantissa
  return min(max(fl - 8, -127), 127);
}

// e4m3 bytes of x0 .. x3 divided by 2^e (exact) and clamped to +-448
__device__ __forceinline__ uint32_t enc4(float x0, float x1, float x2, float x3, int e) {
  auto f = [e](float x) __attribute__((always_inline)) {
    return __builtin_fminf(__builtin_fmaxf(__builtin_amdgcn_ldexpf(x, -e), -448.f), 448.f);
  };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(f(x0), f(x1), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(f(x2), f(x3), w, true);
  return (uint32_t)w;
}
}  // namespace mxq

// Q/K: one thread per 32-element block along d.  `rows` token-head rows of D.
template <int D>
__global__ void __launch_bounds__(256) mx_quant_d_kernel(QuantArgs a, int64_t rows) {
  constexpr int GPR = D / mxq::BLK;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= rows * GPR) return;
  const uint16_t* x = (const uint16_t*)a.x + g * mxq::BLK;
  uint8_t* y = (uint8_t*)a.y + g * mxq::BLK;
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = *(const u32x4*)(x + 8 * i);
  mxq::u16x2 m2 = {0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int w = 0; w < 4; ++w) m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(mxq::u16x2, v[i][w] & 0x7fff7fffu));
  const int e = mxq::block_exp(m2[0] > m2[1] ? m2[0] : m2[1]);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4& s = v[2 * i + j / 2];
      const uint32_t p = s[2 * (j & 1)], q = s[2 * (j & 1) + 1];
      o[j] = mxq::enc4(__uint_as_float(p << 16), __uint_as_float(p & 0xffff0000u), __uint_as_float(q << 16),
                       __uint_as_float(q & 0xffff0000u), e);
    }
    *(u32x4*)(y + 16 * i) = o;
  }
  ((uint8_t*)a.scales)[g] = (uint8_t)(e + 127);
}

// V: one wave per 32-token block of one (sequence or document, head); lane
// owns coordinates 2 lane, 2 lane + 1 (lanes >= D / 2 idle).
template <int D, bool PACKED>
__global__ void __launch_bounds__(256) mx_quant_tok_kernel(QuantArgs a) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int slot = item % a.nsb;
  const int rest = item / a.nsb;
  if (rest >= a.H * (PACKED ? 1 : a.B)) return;
  const int h = rest % a.H;
  const int b = rest / a.H;
  int seq_start, seq_len, blk;
  int64_t sidx;
  if constexpr (!PACKED) {
    blk = slot;
    seq_start = b * a.N;
    seq_len = a.N;
    sidx = ((int64_t)b * a.H + h) * a.nsb + slot;
  } else {
    int lo = 0, hi = a.B - 1;       // the document of this slot (as the 128-token quantiser)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.cu_seqlens[mid] / mxq::BLK + mid <= slot) lo = mid;
      else hi = mid - 1;
    }
    seq_start = a.cu_seqlens[lo];
    seq_len = a.cu_seqlens[lo + 1] - seq_start;
    blk = slot - (seq_start / mxq::BLK + lo);
    if (blk * mxq::BLK >= seq_len) return;
    sidx = (int64_t)h * a.nsb + slot;
  }
  if (2 * lane >= D) return;
  const int t0 = blk * mxq::BLK;
  const int nt = min(mxq::BLK, seq_len - t0);
  const int64_t rs = (int64_t)a.H * D;
  const uint16_t* x = (const uint16_t*)a.x + (int64_t)(seq_start + t0) * rs + (int64_t)h * D + 2 * lane;
  uint8_t* y = (uint8_t*)a.y + (int64_t)(seq_start + t0) * rs + (int64_t)h * D + 2 * lane;
  uint32_t v[mxq::BLK];
  uint32_t m0 = 0, m1 = 0;
#pragma unroll
  for (int t = 0; t < mxq::BLK; ++t) {
    v[t] = t < nt ? *(const uint32_t*)(x + t * rs) : 0u;
    m0 = max(m0, v[t] & 0x7fffu);
    m1 = max(m1, (v[t] >> 16) & 0x7fffu);
  }
  const int e0 = mxq::block_exp(m0), e1 = mxq::block_exp(m1);
#pragma unroll
  for (int t = 0; t < mxq::BLK; ++t) {
    if (t < nt) {
      const float c0 = __builtin_fminf(__builtin_fmaxf(__builtin_amdgcn_ldexpf(__uint_as_float(v[t] << 16), -e0), -448.f), 448.f);
      const float c1 = __builtin_fminf(
          __builtin_fmaxf(__builtin_amdgcn_ldexpf(__uint_as_float(v[t] & 0xffff0000u), -e1), -448.f), 448.f);
      *(uint16_t*)(y + t * rs) = (uint16_t)__builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
    }
  }
  *(uint16_t*)((uint8_t*)a.scales + sidx * D + 2 * lane) = (uint16_t)((e0 + 127) | ((e1 + 127) << 8));
}

template <int D>
static hipError_t launch_mx_t(const QuantArgs& a, bool packed, bool tokens, hipStream_t st) {
  void* args2[2];
  if (!tokens) {
    QuantArgs aa = a;
    int64_t rows = (int64_t)(packed ? a.N : (int64_t)a.B * a.N) * a.H;
    args2[0] = &aa;
    args2[1] = &rows;
    const int64_t grid = (rows * (D / mxq::BLK) + 255) / 256;
    return hipLaunchKernel(reinterpret_cast<const void*>(&mx_quant_d_kernel<D>), dim3((unsigned)grid), dim3(256),
                           args2, 0, st);
  }
  QuantArgs aa = a;
  void* args[] = {&aa};
  const int64_t items = (int64_t)a.nsb * a.H * (packed ? 1 : a.B);
  const int64_t grid = (items + 3) / 4;
  if (packed)
    return hipLaunchKernel(reinterpret_cast<const void*>(&mx_quant_tok_kernel<D, true>), dim3((unsigned)grid),
                           dim3(256), args, 0, st);
  return hipLaunchKernel(reinterpret_cast<const void*>(&mx_quant_tok_kernel<D, false>), dim3((unsigned)grid),
                         dim3(256), args, 0, st);
}

hipError_t launch_quantize_mxfp8(const QuantArgs& a, int d, bool packed, bool tokens, hipStream_t st) {
  return d == 128 ? launch_mx_t<128>(a, packed, tokens, st) : launch_mx_t<64>(a, packed, tokens, st);
}

}  // namespace iaea
