"""fp64 CPU oracle for the exact attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code with the HIP library.

Parity status of each function (what pins it, in ``tests/test_oracle_pins.py``):

  attention / attention_rows   pinned: worked two-score example of the page,
                               closed forms (two keys, uniform scores, causal
                               row 0, hard attention), scipy softmax and
                               logsumexp, mpmath brute force, LSE merge,
                               permutation equivariance, varlen = per-document
  online_softmax_states        pinned: the page's worked example states, in
                               both orders, and agreement with attention()
  e4m3_decode                  pinned: OCP e4m3fn closed-form values and torch's
                               float8_e4m3fn decode of all 256 bytes
  bf16_decode                  pinned: torch's bfloat16 decode of all 65536
                               bit patterns
  dequantize_e4m3_blocks       pinned: exact round trip with scale 1 blocks and
                               hand-built blocks
  quantize.e4m3_encode         pinned (tests/test_quantize_oracle.py): every
                               finite byte round-trips, hand-computed midpoints
                               and saturation, torch's float8_e4m3fn cast
  quantize.quantize_blocks     pinned: hand-built blocks, block maximum -> 448,
                               all-zero blocks, packed = per-document, distinct
                               scale slots, dequantisation error bound; planted
                               mistakes each trip a pin
  quantize.dequantize_blocks   pinned: the dequantisation error bound above
  backward.attention_grads     pinned (tests/test_backward_oracle.py): central
                               finite differences (fixed, causal, packed),
                               torch autograd in float64, closed forms (equal
                               scores, one key), key-shift invariance; planted
                               mistakes each trip a pin
  backward.row_dot             pinned: rowsum(dO * O) = rowsum(P * dP)
  rotation.hadamard            pinned (tests/test_rotation_oracle.py): scipy's
                               hadamard, the closed form of the entries
  rotation.rotate              pinned: orthogonality, one-hot rows, inner
                               products times d, sums beyond float64 (an fp32
                               tie broken at 2^-80), plain-loop sums of bf16
                               rows, attention invariance with scale / d
  rotation.rotate_quantize_blocks  pinned: a rotated one-hot block; planted
                               mistakes each trip a pin
  mx.quantize_mx_d / _tokens   pinned (tests/test_mx_oracle.py): hand-computed
                               blocks (power-of-two maximum, floor of the
                               exponent, saturation, all-zero, small elements),
                               the format's error bound, block orientation,
                               document-local restart, causality of scales;
                               planted mistakes each trip a pin
  mx.dequantize_mx_*           pinned: exact on e4m3-grid values, error bound
"""
from .exact import (attention, attention_rows, online_softmax_states,
                        e4m3_decode, bf16_decode, dequantize_e4m3_blocks)
from . import backward, mx, quantize, rotation

__all__ = ["attention", "attention_rows", "online_softmax_states",
           "e4m3_decode", "bf16_decode", "dequantize_e4m3_blocks",
           "backward", "mx", "quantize", "rotation"]
