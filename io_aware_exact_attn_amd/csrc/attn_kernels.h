// Internal launchers of the gfx950 attention kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include "attn_common.h"

namespace iaea {

// bf16 q/k/v; d in {64, 128}; o bf16 or fp32.  Arguments already validated.
hipError_t launch_attn_fwd_bf16(const FwdArgs& a, int d, bool causal, bool packed, bool out_f32,
                                hipStream_t st);
int bf16_rows_per_workgroup(int d);

// e4m3 q/k/v with per-128-token scales; d = 128; o bf16; fixed length or
// packed documents (document-local scale blocks).
hipError_t launch_attn_fwd_fp8(const FwdArgs& a, bool causal, bool packed, hipStream_t st);
hipError_t launch_attn_fwd_mxfp8(const FwdArgs& a, bool causal, bool packed, hipStream_t st);

// bf16 backward: D = rowsum(dO * O) into a.delta, then dQ, then dK and dV;
// d in {64, 128}.  Arguments already validated.
hipError_t launch_attn_bwd(const BwdArgs& a, int d, bool causal, bool packed, hipStream_t st);
int bwd_rows_per_workgroup();

// Rows of D (B * H * N, or H * N packed) that the fixed scratch of the
// no-allocation backward holds: 2^21 floats, 8 MiB per GPU.
constexpr int64_t kBwdScratchRows = (int64_t)1 << 21;
// Device address of that scratch on the current device (looked up once per
// device, then cached).
hipError_t bwd_scratch_address(float** out);

// bf16 -> e4m3 with per-128-token block scales; d in {64, 128}.
hipError_t launch_quantize_fp8(const QuantArgs& a, int d, bool packed, hipStream_t st);
hipError_t launch_quantize_fp8_rotated(const QuantArgs& a, int d, bool packed, hipStream_t st);
hipError_t launch_quantize_mxfp8(const QuantArgs& a, int d, bool packed, bool tokens, hipStream_t st);
int64_t quantize_fp8_grid(int B, int H, int N, bool packed);

}  // namespace iaea
