// C ABI of the attention library: argument validation (host only, before any
// HIP call), kernel selection and launch.  No allocation; the only global
// state is the per-device address of attn_bwd_noalloc's fixed scratch.
#include <cfloat>
#include <cmath>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "../../include/attn.h"
#include "attn_kernels.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Common checks of both entry points; fills the size/scale fields of `a`.
int check_common(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 int B, int H, int N, float scale, int causal, iaea::FwdArgs& a) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  if (B < 1 || H < 1 || N < 1) return ATTN_ERR_SHAPE;
  // every tensor index (token * H + h) * d and the LSE index h * N + t stay
  // below 2^31 rows of d elements; the grid stays below 2^31 workgroups
  if ((int64_t)B * N * H >= (int64_t)1 << 31) return ATTN_ERR_SHAPE;
  if (causal != 0 && causal != 1) return ATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return ATTN_ERR_ALIGN;
  // exp2 of (s - m) * c with c = |scale| * log2(e); the sign of scale is folded
  // into q (an exact bf16 sign flip).  c = 0 would make masked entries
  // (-inf * 0) undefined, so a zero scale runs with the smallest normal
  // float: every score then contributes exp2(~0) = 1, the zero-scale result.
  double c = std::fabs((double)scale) * 1.4426950408889634;
  if (c < FLT_MIN) c = FLT_MIN;
  if (c > FLT_MAX) c = FLT_MAX;
  a = iaea::FwdArgs{};
  a.q = q; a.k = k; a.v = v; a.o = const_cast<void*>(o); a.lse = const_cast<float*>(lse);
  a.B = B; a.H = H; a.N = N;
  a.c = (float)c;
  a.qsign = std::signbit(scale) ? 0x80008000u : 0u;
  a.lse_mul = 0.6931471805599453f;
  return ATTN_OK;
}

// Checks shared by the two backward entry points (everything but the D
// workspace); fills `a` except a.delta.
int check_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
              const void* dq, const void* dk, const void* dv, int B, int H, int N, int d, float scale, int causal,
              const int32_t* cu_seqlens, iaea::BwdArgs& a) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return ATTN_ERR_NULL;
  if (B < 1 || H < 1 || N < 1) return ATTN_ERR_SHAPE;
  if ((int64_t)B * N * H >= (int64_t)1 << 31) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return ATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
  if ((int64_t)H * d > ((int64_t)1 << 24)) return ATTN_ERR_SHAPE;
  for (const void* p : {q, k, v, o, dout, (const void*)lse, dq, dk, dv})
    if (!aligned16(p)) return ATTN_ERR_ALIGN;
  if (cu_seqlens && !aligned16(cu_seqlens)) return ATTN_ERR_ALIGN;
  const int64_t bm = iaea::bwd_rows_per_workgroup();
  if (cu_seqlens && (int64_t)H * ((N + bm - 1) / bm + B) + 8 >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
  a = iaea::BwdArgs{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
  a.dq = const_cast<void*>(dq); a.dk = const_cast<void*>(dk); a.dv = const_cast<void*>(dv);
  a.cu_seqlens = cu_seqlens;
  a.B = B; a.H = H; a.N = N;
  a.scale = scale;
  a.c = (float)((double)scale * 1.4426950408889634);
  return ATTN_OK;
}

}  // namespace

extern "C" {

ATTN_API int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int N, int d, float scale, int causal,
                      const int32_t* cu_seqlens, int dtype, void* stream) {
  iaea::FwdArgs a;
  const int st = check_common(q, k, v, o, lse, B, H, N, scale, causal, a);
  if (st != ATTN_OK) return st;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (dtype != ATTN_BF16 && dtype != ATTN_BF16_OUT_F32) return ATTN_ERR_UNSUPPORTED;
  // a 64-row K/V tile of all heads (64 * H * d * 2 bytes) is addressed with 32-bit offsets
  if ((int64_t)H * d > ((int64_t)1 << 24)) return ATTN_ERR_SHAPE;
  if (cu_seqlens && !aligned16(cu_seqlens)) return ATTN_ERR_ALIGN;
  if (cu_seqlens) {
    // packed: B documents over N tokens; the grid has ceil(N / BM) + B slots per head
    const int64_t bm = iaea::bf16_rows_per_workgroup(d);
    if ((int64_t)H * ((N + bm - 1) / bm + B) + 8 >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
  }
  a.cu_seqlens = cu_seqlens;
  const hipError_t e = iaea::launch_attn_fwd_bf16(a, d, causal == 1, cu_seqlens != nullptr,
                                                  dtype == ATTN_BF16_OUT_F32,
                                                  reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

ATTN_API int attn_fwd_fp8(const void* q, const void* k, const void* v,
                          const float* q_scale, const float* k_scale, const float* v_scale,
                          void* o, float* lse, int B, int H, int N, int d, float scale,
                          int causal, const int32_t* cu_seqlens, void* stream) {
  iaea::FwdArgs a;
  const int st = check_common(q, k, v, o, lse, B, H, N, scale, causal, a);
  if (st != ATTN_OK) return st;
  if (!q_scale || !k_scale || !v_scale) return ATTN_ERR_NULL;
  if (d != 128) return ATTN_ERR_UNSUPPORTED;
  // a 64-row K/V tile of all heads (64 * H * d bytes) is addressed with 32-bit offsets
  if ((int64_t)H * d > ((int64_t)1 << 24)) return ATTN_ERR_SHAPE;
  if (!aligned16(q_scale) || !aligned16(k_scale) || !aligned16(v_scale)) return ATTN_ERR_ALIGN;
  if (cu_seqlens && !aligned16(cu_seqlens)) return ATTN_ERR_ALIGN;
  // packed: ceil(N / 128) + B workgroup slots and scale slots per head
  if (cu_seqlens && (int64_t)H * ((N + 127) / 128 + B) + 8 >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
  a.q_scale = q_scale; a.k_scale = k_scale; a.v_scale = v_scale;
  a.cu_seqlens = cu_seqlens;
  a.nsb = (N + 127) / 128 + (cu_seqlens ? B : 0);
  a.qsign = std::signbit(scale) ? 0x80808080u : 0u;   // e4m3 sign bits
  const hipError_t e = iaea::launch_attn_fwd_fp8(a, causal == 1, cu_seqlens != nullptr,
                                                 reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

ATTN_API int attn_fwd_mxfp8(const void* q, const void* k, const void* v, const uint8_t* q_scale,
                            const uint8_t* k_scale, const uint8_t* v_scale, void* o, float* lse, int B, int H,
                            int N, int d, float scale, int causal, const int32_t* cu_seqlens, void* stream) {
  iaea::FwdArgs a;
  const int st = check_common(q, k, v, o, lse, B, H, N, scale, causal, a);
  if (st != ATTN_OK) return st;
  if (!q_scale || !k_scale || !v_scale) return ATTN_ERR_NULL;
  if (d != 128) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)H * d > ((int64_t)1 << 24)) return ATTN_ERR_SHAPE;
  if (!aligned16(q_scale) || !aligned16(k_scale) || !aligned16(v_scale)) return ATTN_ERR_ALIGN;
  if (cu_seqlens && !aligned16(cu_seqlens)) return ATTN_ERR_ALIGN;
  if (cu_seqlens && (int64_t)H * ((N + 127) / 128 + B) + 8 >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
  // V scale slots per head row (ceil(N / 32), packed + B) are int; a tile's K
  // scale bytes (64 tokens x H x 4) are addressed with 32-bit offsets
  if ((int64_t)H * ((N + 31) / 32 + (cu_seqlens ? B : 0)) >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
  if ((int64_t)64 * H * 4 >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
  a.q_scale = reinterpret_cast<const float*>(q_scale);
  a.k_scale = reinterpret_cast<const float*>(k_scale);
  a.v_scale = reinterpret_cast<const float*>(v_scale);
  a.cu_seqlens = cu_seqlens;
  a.nsb = (N + 31) / 32 + (cu_seqlens ? B : 0);
  a.qsign = std::signbit(scale) ? 0x80808080u : 0u;
  const hipError_t e = iaea::launch_attn_fwd_mxfp8(a, causal == 1, cu_seqlens != nullptr,
                                                   reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

ATTN_API int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, float* delta, void* dq, void* dk, void* dv,
                      int B, int H, int N, int d, float scale, int causal,
                      const int32_t* cu_seqlens, void* stream) {
  if (!delta) return ATTN_ERR_NULL;
  iaea::BwdArgs a;
  const int st = check_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, cu_seqlens, a);
  if (st != ATTN_OK) return st;
  if (!aligned16(delta)) return ATTN_ERR_ALIGN;
  a.delta = delta;
  const hipError_t e = iaea::launch_attn_bwd(a, d, causal == 1, cu_seqlens != nullptr,
                                             reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

ATTN_API int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv,
                              int B, int H, int N, int d, float scale, int causal,
                              const int32_t* cu_seqlens, void* stream) {
  iaea::BwdArgs a;
  const int st = check_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, cu_seqlens, a);
  if (st != ATTN_OK) return st;
  const int64_t rows = (int64_t)(cu_seqlens ? 1 : B) * N * H;
  if (rows > iaea::kBwdScratchRows) return ATTN_ERR_SCRATCH;
  float* scratch = nullptr;
  if (iaea::bwd_scratch_address(&scratch) != hipSuccess) return ATTN_ERR_HIP;
  a.delta = scratch;
  const hipError_t e = iaea::launch_attn_bwd(a, d, causal == 1, cu_seqlens != nullptr,
                                             reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

ATTN_API int attn_quantize_fp8(const void* x, void* y, float* scales, int B, int H, int N, int d,
                               const int32_t* cu_seqlens, void* stream) {
  if (!x || !y || !scales) return ATTN_ERR_NULL;
  if (B < 1 || H < 1 || N < 1) return ATTN_ERR_SHAPE;
  if ((int64_t)B * N * H >= (int64_t)1 << 31) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(y) || !aligned16(scales)) return ATTN_ERR_ALIGN;
  if (cu_seqlens && !aligned16(cu_seqlens)) return ATTN_ERR_ALIGN;
  if (iaea::quantize_fp8_grid(B, H, N, cu_seqlens != nullptr) >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
  iaea::QuantArgs a{};
  a.x = x; a.y = y; a.scales = scales; a.cu_seqlens = cu_seqlens;
  a.B = B; a.H = H; a.N = N;
  a.nsb = (N + 127) / 128 + (cu_seqlens ? B : 0);
  const hipError_t e = iaea::launch_quantize_fp8(a, d, cu_seqlens != nullptr,
                                                 reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

ATTN_API int attn_quantize_fp8_rotated(const void* x, void* y, float* scales, const int8_t* signs, int B, int H,
                                       int N, int d, const int32_t* cu_seqlens, void* stream) {
  if (!x || !y || !scales || !signs) return ATTN_ERR_NULL;
  if (B < 1 || H < 1 || N < 1) return ATTN_ERR_SHAPE;
  if ((int64_t)B * N * H >= (int64_t)1 << 31) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(y) || !aligned16(scales) || !aligned16(signs)) return ATTN_ERR_ALIGN;
  if (cu_seqlens && !aligned16(cu_seqlens)) return ATTN_ERR_ALIGN;
  if (iaea::quantize_fp8_grid(B, H, N, cu_seqlens != nullptr) >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
  iaea::QuantArgs a{};
  a.x = x; a.y = y; a.scales = scales; a.cu_seqlens = cu_seqlens; a.signs = signs;
  a.B = B; a.H = H; a.N = N;
  a.nsb = (N + 127) / 128 + (cu_seqlens ? B : 0);
  const hipError_t e = iaea::launch_quantize_fp8_rotated(a, d, cu_seqlens != nullptr,
                                                         reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

ATTN_API int attn_quantize_mxfp8(const void* x, void* y, uint8_t* scales, int B, int H, int N, int d,
                                 const int32_t* cu_seqlens, int along_tokens, void* stream) {
  if (!x || !y || !scales) return ATTN_ERR_NULL;
  if (B < 1 || H < 1 || N < 1) return ATTN_ERR_SHAPE;
  if ((int64_t)B * N * H >= (int64_t)1 << 31) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (along_tokens != 0 && along_tokens != 1) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(y) || !aligned16(scales)) return ATTN_ERR_ALIGN;
  if (cu_seqlens && !aligned16(cu_seqlens)) return ATTN_ERR_ALIGN;
  const bool packed = cu_seqlens != nullptr;
  iaea::QuantArgs a{};
  a.x = x; a.y = y; a.scales = reinterpret_cast<float*>(scales); a.cu_seqlens = cu_seqlens;
  a.B = B; a.H = H; a.N = N;
  a.nsb = (N + 31) / 32 + (packed ? B : 0);
  if (along_tokens && ((int64_t)a.nsb * H * (packed ? 1 : B) + 3) / 4 >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
  const hipError_t e = iaea::launch_quantize_mxfp8(a, d, packed, along_tokens == 1,
                                                   reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

ATTN_API const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "B, H or N out of range";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head dimension, dtype, causal flag or layout";
    case ATTN_ERR_SCALE: return "scale is not finite";
    case ATTN_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case ATTN_ERR_HIP: return "kernel launch failed";
    case ATTN_ERR_SCRATCH: return "more rows than the fixed scratch of attn_bwd_noalloc holds (2^21)";
    default: return "unknown status";
  }
}

ATTN_API const char* attn_kernel_name(int d, int causal, int packed, int dtype, int fp8) {
  if (causal != 0 && causal != 1) return "";
  if (fp8 == 2) {
    if (d != 128) return "";
    static const char* mx[2][2] = {{"attn_fwd_fp8_kernel<full,fixed,mx>", "attn_fwd_fp8_kernel<full,packed,mx>"},
                                   {"attn_fwd_fp8_kernel<causal,fixed,mx>", "attn_fwd_fp8_kernel<causal,packed,mx>"}};
    return mx[causal][packed ? 1 : 0];
  }
  if (fp8) {
    if (d != 128) return "";
    static const char* f8[2][2] = {{"attn_fwd_fp8_kernel<full,fixed>", "attn_fwd_fp8_kernel<full,packed>"},
                                   {"attn_fwd_fp8_kernel<causal,fixed>", "attn_fwd_fp8_kernel<causal,packed>"}};
    return f8[causal][packed ? 1 : 0];
  }
  if ((d != 64 && d != 128) || (dtype != ATTN_BF16 && dtype != ATTN_BF16_OUT_F32)) return "";
  static const char* names[2][2][2][2] = {
      {{{"attn_fwd_bf16_kernel<d64,full,fixed,bf16>", "attn_fwd_bf16_kernel<d64,full,fixed,f32>"},
        {"attn_fwd_bf16_kernel<d64,full,packed,bf16>", "attn_fwd_bf16_kernel<d64,full,packed,f32>"}},
       {{"attn_fwd_bf16_kernel<d64,causal,fixed,bf16>", "attn_fwd_bf16_kernel<d64,causal,fixed,f32>"},
        {"attn_fwd_bf16_kernel<d64,causal,packed,bf16>", "attn_fwd_bf16_kernel<d64,causal,packed,f32>"}}},
      {{{"attn_fwd_bf16_kernel<d128,full,fixed,bf16>", "attn_fwd_bf16_kernel<d128,full,fixed,f32>"},
        {"attn_fwd_bf16_kernel<d128,full,packed,bf16>", "attn_fwd_bf16_kernel<d128,full,packed,f32>"}},
       {{"attn_fwd_bf16_kernel<d128,causal,fixed,bf16>", "attn_fwd_bf16_kernel<d128,causal,fixed,f32>"},
        {"attn_fwd_bf16_kernel<d128,causal,packed,bf16>", "attn_fwd_bf16_kernel<d128,causal,packed,f32>"}}}};
  return names[d == 128][causal][packed ? 1 : 0][dtype == ATTN_BF16_OUT_F32];
}

}  // extern "C"
