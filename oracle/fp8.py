"""FP8 canvas attention (oracle side; test infrastructure only: nothing outside
tests/, the smoke check and the CPU baseline imports it).

What the pages fix: the pages' timings are taken on an H100 with FP8 precision
(explainer "DiffusionGemma: Google's open diffusion LLM", section "Throughput
flips at about 32 concurrent users", quoting the caption of the report's
Figure 12).  They do not say which tensors are FP8, nor the FP8 format.

Readings taken (each also listed in the design notes, F1-F3):
  F1  the format is OCP 8-bit floating point E4M3 ("E4M3FN"): 1 sign bit, 4
      exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
      subnormals m/8 * 2^-6; S.1111.111 is NaN; there are no infinities, and
      the largest finite magnitude is 448.
  F2  Q, the prefix and canvas K and V arrive as E4M3 bytes with one float32
      scale per tensor kind: the real values are q_scale * q, k_scale * k,
      v_scale * v (one k_scale for prefix and canvas keys, one v_scale for the
      values).
  F3  the attention is then exactly the bf16/fp32 definition of
      oracle.attention on those real values (no further rounding is part of
      the definition).

Pins (tests/test_oracle_fp8.py): all 256 codes against torch.float8_e4m3fn
(an independent implementation); closed-form codes (0x38 = 1, 0x7E = 448,
0x01 = 2^-9, 0x08 = 2^-6, 0x7F and 0xFF NaN, 0x80 = -0); the decoded grid is
exactly the set of values with 3 mantissa bits in range; moving a factor
between q_scale and k_scale leaves the output unchanged, and v_scale scales it.
"""
import numpy as np

from .attention import canvas_attention


def e4m3_to_float(codes):
    """Decode E4M3 bytes (uint8 array) to float64 per reading F1."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 15
    m = b & 7
    normal = sign * (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = sign * (m / 8.0) * 2.0 ** -6
    out = np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, out)


def canvas_attention_fp8(q, k_prefix, v_prefix, k_canvas, v_canvas, q_scale=1.0, k_scale=1.0, v_scale=1.0,
                         scale=None, causal=False):
    """Attention on E4M3 byte tensors with per-tensor scales (F2, F3): O [N,Hq,D] float64."""
    dq = lambda x, s: None if x is None else e4m3_to_float(x) * float(np.float32(s))
    d = np.asarray(q).shape[2]
    sc = 1.0 / np.sqrt(d) if scale is None else scale
    return canvas_attention(dq(q, q_scale), dq(k_prefix, k_scale), dq(v_prefix, v_scale), dq(k_canvas, k_scale),
                            dq(v_canvas, v_scale), scale=sc, causal=causal)
