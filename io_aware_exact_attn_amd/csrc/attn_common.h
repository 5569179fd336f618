// Shared device helpers for the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace iaea {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

#define IAEA_LDS __attribute__((address_space(3)))

constexpr int kWave = 64;
constexpr int kXcds = 8;          // MI355X: workgroups go round-robin to 8 XCDs
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Word 3 of a raw (stride 0) buffer resource on CDNA: 32-bit data format,
// out-of-range dwords read as zero.
constexpr int kBufferFlags = 0x00020000;

// Kernel arguments shared by the bf16 and fp8 paths.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* q_scale;      // fp8: fp32 [B][H][nsb]; MXFP8: E8M0 bytes read through
  const float* k_scale;      //   the same pointers (q, k [tokens][H][d / 32],
  const float* v_scale;      //   v [rows of 32-token blocks][d]), cast back in the kernel
  void* o;
  float* lse;
  const int32_t* cu_seqlens; // packed documents, device, B + 1 entries
  int B, H, N;               // N: tokens per sequence, or total tokens when packed
  int nsb;                   // fp8: scale blocks per sequence = ceil(N / 128) (packed + B);
                             // MXFP8: V's 32-token blocks, ceil(N / 32) (packed + B)
  int slots;                 // workgroup slots per head (packed) or q blocks per sequence
  int n_work;                // number of real work items
  int per_xcd;               // grid / 8
  float c;                   // |scale| * log2(e), clamped to [FLT_MIN, FLT_MAX]
  uint32_t qsign;            // 0x80008000 when scale < 0 (bf16 sign flip of q), else 0
  float lse_mul;             // ln 2: LSE = ln2 * (m_scaled + log2 l)
};

// Arguments of the backward kernels.
struct BwdArgs {
  const void* q;             // bf16 [B][N][H][d] (packed [N][H][d]), as the forward
  const void* k;
  const void* v;
  const void* o;             // the forward's output
  const void* dout;          // upstream gradient dO, layout of o
  const float* lse;          // the forward's LSE, [B][H][N] (packed [H][N])
  float* delta;              // D = rowsum(dO * O), layout of lse (written, then read)
  void* dq;                  // bf16 outputs, layout of q
  void* dk;
  void* dv;
  const int32_t* cu_seqlens; // packed documents, device, B + 1 entries
  int B, H, N;
  int slots;                 // workgroup slots per head (packed) or blocks per sequence
  int n_work;                // number of real work items
  int per_xcd;               // grid / 8
  float scale;               // the forward's scale (any sign)
  float c;                   // scale * log2(e)
};

// Arguments of the e4m3 block quantiser.
struct QuantArgs {
  const void* x;             // bf16 input, [B][N][H][d] or packed [N][H][d]
  void* y;                   // e4m3 output, same layout
  float* scales;             // [B][H][nsb] or packed [H][nsb]; the MXFP8 quantiser writes
                             // E8M0 bytes through it (its own layouts)
  const int32_t* cu_seqlens; // packed documents, device, B + 1 entries
  const int8_t* signs;       // rotating quantiser: d random signs (+1 / -1), device
  int B, H, N;
  int nsb;                   // scale slots per (sequence, head): ceil(N / 128), packed + B
};

// 16-byte-granule XOR swizzle of a bf16 LDS row of D elements: conflict-free
// for the MFMA fragment reads along rows (16 consecutive rows, one granule)
// and for the transposed reads (ds_read_b64_tr_b16) of the bf16 kernels.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// The restrict-qualified pointer gives the read alias-scope metadata; without
// it the compiler cannot tell it from the in-flight LDS DMA of other buffers
// and waits for every outstanding tile load before it.
__device__ __forceinline__ bf16x4 ds_read_tr16(const char* __restrict__ p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((IAEA_LDS s16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

// Calls f(integral_constant<int, I>) for I = 0 .. N - 1, fully unrolled, so
// register arrays are indexed by compile-time constants.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Undo the round-robin XCD dispatch: consecutive logical indices land on one
// XCD, so workgroups that run together on an XCD share its L2 (packed
// documents: a head's documents stay together).
__device__ __forceinline__ int logical_block(int bid, int per_xcd) {
  return (bid % kXcds) * per_xcd + bid / kXcds;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  // one v_cvt_pk_bf16_f32 (round to nearest even)
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Locate (head, sequence start, length, q block) of workgroup bid.  Returns
// false when the workgroup has no work (grid padding, or packed slots past the
// last document).
//
// Fixed-length sequences: the workgroups go out in rank order of their cost
// (rank r covers q block slots - 1 - r of every (sequence, head) when causal),
// so the dispatcher, which hands the next workgroup to the first free CU,
// schedules longest first and the last ones to start are the shortest.  The
// (sequence, head) index is the minor one: the round-robin over the 8 XCDs
// then keeps each (sequence, head) on one XCD when B H is a multiple of 8.
template <int BM, bool CAUSAL, bool PACKED, class Args>
__device__ __forceinline__ bool decode_work(const Args& a, int bid, int& h, int& b,
                                            int& seq_start, int& seq_len, int& qblk) {
  if constexpr (!PACKED) {
    const int lb = bid;
    if (lb >= a.n_work) return false;
    const int nbh = a.B * a.H;
    const int r = lb / nbh;
    const int bh = lb - r * nbh;
    qblk = CAUSAL ? (a.slots - 1 - r) : r;
    b = bh / a.H;
    h = bh - b * a.H;
    seq_start = b * a.N;
    seq_len = a.N;
    return true;
  } else {
    const int lane = threadIdx.x & 63;
    if (a.B <= 64) {
      // Up to 64 documents, one per lane: documents go out longest first,
      // each with its q blocks longest first, and the head as the minor
      // index (so a document's blocks run together on an XCD for locality).
      // The last workgroups to start are those of the shortest documents.
      const int t = bid / a.H;
      h = bid - t * a.H;
      // lane f holds document f's start and length: one load of each bound,
      // and the start comes back from its lane instead of a second load
      // (lanes past the last document read the last bound twice: length 0;
      // the loads and the loop below are branch-free)
      const int c0 = a.cu_seqlens[min(lane, a.B)];
      const int len = a.cu_seqlens[min(lane + 1, a.B)] - c0;
      const int nb = len > 0 ? (len + BM - 1) / BM : 0;
      // items before this document's first: the work of every document that
      // comes before it in the order (longer, or as long and earlier)
      int first = 0;
      for (int f = 0; f < a.B; ++f) {
        const int lf = __builtin_amdgcn_readlane(len, f);
        const int nf = __builtin_amdgcn_readlane(nb, f);
        const int before = (int)(lf > len) | ((int)(lf == len) & (int)(f < lane));
        first += nf & -before;
      }
      const unsigned long long m = __ballot(lane < a.B && t >= first && t < first + nb);
      if (m == 0) return false;
      const int doc = __ffsll((long long)m) - 1;
      const int r = t - __builtin_amdgcn_readlane(first, doc);
      const int nbd = __builtin_amdgcn_readlane(nb, doc);
      seq_start = __builtin_amdgcn_readlane(c0, doc);
      seq_len = __builtin_amdgcn_readlane(len, doc);
      qblk = CAUSAL ? (nbd - 1 - r) : r;
      b = doc;
      return true;
    }
    // more documents: each head's slots in document order, per-XCD contiguous
    const int lb = logical_block(bid, a.per_xcd);
    if (lb >= a.n_work) return false;
    h = lb / a.slots;
    const int s = lb - h * a.slots;
    b = 0;
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

}  // namespace iaea
