"""Exact conversion of 16-bit storage values to float64 (oracle; test infrastructure).

bfloat16 keeps the sign and 8-bit exponent of fp32 and the top 7 mantissa bits
("[Hacker News 요약] ... 'Tiny-vLLM' 직접 구축하기", section "모델 로딩 및 데이터
형식 심층 이해"), so a bf16 bit pattern b is the fp32 pattern b << 16, which is
exact in float64.  fp16 goes through numpy's exact half -> double conversion.
"""
import numpy as np


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def scale_as_passed(scale: float) -> float:
    """The softmax scale as the kernel receives it: rounded to fp32 first."""
    return float(np.float32(scale))
