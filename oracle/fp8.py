"""FP8 (E4M3) KV cache: the encoding, the scaled append, and what the decode reads (oracle; test infrastructure).

The Tiny-vLLM summary lists an FP8 datatype only as a future direction ("[Hacker
News 요약] C++와 CUDA로 vLLM의 경량 고성능 LLM 추론 엔진 'Tiny-vLLM' 직접
구축하기", section "향후 전망"); the pages fix nothing else.  Readings taken here:

* format: the 8-bit E4M3 layout (1 sign bit, 4 exponent bits with bias 7, 3
  mantissa bits; exponent 0 holds subnormals m * 2^-9; no infinities; S.1111.111
  is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448);
* one fp32 scale per pool (K and V separately): a stored code c stands for
  decode(c) * scale;
* the append rounds fp32(x) * fp32(1 / scale) to the nearest code, ties to the
  even mantissa, magnitudes beyond 448 (and infinities) saturate to +-448, and
  NaN becomes 0x7F;
* the decode attends over the dequantised K and V (the same softmax(scale q K^T) V
  as oracle.attention, on decode(code) * scale).

Encoding and decoding are written from the bit layout, not from a library.
"""
import math

import numpy as np

MAX_E4M3 = 448.0
NAN_CODE = 0x7F


def decode_code(c: int) -> float:
    """The value of one E4M3 code (float; NaN for S.1111.111)."""
    c = int(c) & 0xFF
    s = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# all 256 codes, as float64
DECODE_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)


def encode_value(x: float) -> int:
    """Nearest E4M3 code to x (ties to even mantissa), saturating at +-448; NaN -> 0x7F."""
    if math.isnan(x):
        return NAN_CODE
    sign = 0x80 if (x < 0 or (x == 0 and math.copysign(1.0, x) < 0)) else 0
    a = abs(x)
    if a >= MAX_E4M3:
        return sign | 0x7E
    # candidates: the finite non-negative codes 0x00 .. 0x7E are increasing in value
    mags = DECODE_TABLE[:0x7F]
    hi = int(np.searchsorted(mags, a, side="left"))     # first code with value >= a
    if hi < len(mags) and mags[hi] == a:
        return sign | hi
    lo = hi - 1
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    if d_lo < d_hi:
        c = lo
    elif d_hi < d_lo:
        c = hi
    else:
        c = lo if (lo & 1) == 0 else hi                  # tie: even mantissa (the code's last bit)
    return sign | c


def encode(x) -> np.ndarray:
    """encode_value over an array (uint8 codes): the same nearest-code search, ties to the
    even code, saturation and NaN rule, taken for all elements at once."""
    x = np.asarray(x, dtype=np.float64)
    mags = DECODE_TABLE[:0x7F]                       # finite non-negative codes, increasing
    a = np.abs(x)
    hi = np.minimum(np.searchsorted(mags, a, side="left"), 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    c = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where((lo & 1) == 0, lo, hi)))
    c = np.where(mags[hi] == a, hi, c)               # exactly representable
    c = np.where(a >= MAX_E4M3, 0x7E, c)             # saturate (infinities too)
    code = np.where(np.signbit(x), 0x80, 0) | c
    return np.where(np.isnan(x), NAN_CODE, code).astype(np.uint8)


def quantize_for_append(x_f32: np.ndarray, scale: float) -> np.ndarray:
    """The codes the append stores for fp32 inputs x: encode(fp32(x * fp32(1/scale)))."""
    inv = np.float32(1.0) / np.float32(scale)
    prod = np.asarray(x_f32, dtype=np.float32) * inv    # one fp32 multiply, rounded to nearest even
    return encode(prod.astype(np.float64))


def dequantize(codes: np.ndarray, scale: float) -> np.ndarray:
    """float64 values the decode attends over: decode(code) * scale."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)] * float(np.float32(scale))


def decode(q, k_codes, v_codes, k_scale, v_scale, block_tables, context_lens, scale, *, q_dtype, num_blocks,
           num_kv_heads, block_size):
    """Paged decode attention over FP8 pools, float64.

    q: uint16 bits [B, Hq, D] (q_dtype "bf16" / "fp16"); k_codes, v_codes: uint8 pools
    [N, Hkv, bs, D] (token-major like the 16-bit pools); returns float64 [B, Hq, D]."""
    from .attention import attend, gather_context, kv_head_of
    from .numerics import bits_to_f64, scale_as_passed

    q = np.asarray(q)
    B, Hq, D = q.shape
    G = Hq // num_kv_heads
    k_log = np.asarray(k_codes, dtype=np.uint8).reshape(num_blocks, num_kv_heads, block_size, D)
    v_log = np.asarray(v_codes, dtype=np.uint8).reshape(num_blocks, num_kv_heads, block_size, D)
    scale64 = scale_as_passed(scale)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for i in range(B):
        L = int(context_lens[i])
        if L == 0:
            continue
        kc, vc = gather_context(k_log, v_log, block_tables[i], L, block_size, num_blocks)
        kf = dequantize(kc, k_scale)
        vf = dequantize(vc, v_scale)
        qi = bits_to_f64(q[i], q_dtype)
        for g in range(num_kv_heads):
            heads = [h for h in range(Hq) if kv_head_of(h, G) == g]
            out[i, heads] = attend(qi[heads], kf[:, g, :], vf[:, g, :], scale64)
    return out


def append(k_bits, v_bits, src_dtype, slot_mapping, k_pool, v_pool, k_scale, v_scale, *, num_blocks, block_size):
    """The FP8 append: every token t with slot s >= 0 stores quantize_for_append of its
    K and V rows (16-bit inputs, exact in fp32) at slot s; pools are uint8 arrays
    [N, Hkv, bs, D], changed in place (token-major like the 16-bit pools)."""
    from .numerics import bits_to_f64

    k_pool = np.asarray(k_pool)
    v_pool = np.asarray(v_pool)
    k_bits = np.asarray(k_bits)
    v_bits = np.asarray(v_bits)
    for t, s in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if s < 0:
            continue
        assert s < num_blocks * block_size, "slot outside the pool"
        n, off = divmod(int(s), block_size)
        k_pool[n, :, off, :] = quantize_for_append(bits_to_f64(k_bits[t], src_dtype).astype(np.float32), k_scale)
        v_pool[n, :, off, :] = quantize_for_append(bits_to_f64(v_bits[t], src_dtype).astype(np.float32), v_scale)
    return k_pool, v_pool
