"""CPU oracle for paged decode attention and the KV append -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The GPU library never calls it and shares no code with it.

It is plain and slow on purpose: numpy float64, one sequence at a time, the
softmax written out from its definition.  Each function cites the passage it
follows.  The pages cited are:

* "vLLM — PagedAttention으로 LLM 추론 성능을 2~4배 끌어올린 서빙 엔진" (dev.to),
  sections "PagedAttention — OS 가상 메모리에서 영감" (fixed-size blocks, logical
  blocks mapped to non-contiguous physical blocks, blocks handed out as tokens
  arrive, free blocks usable by other requests), "프로젝트 구조"
  (block_manager.py keeps the physical/logical block mapping), "KV Cache가 왜
  병목인가" (K and V of every past token kept per layer and head; the KV-size
  product) and "Prefill vs Decode" (decode makes one token per step and mostly
  reads the KV cache).
* "[Hacker News 요약] C++와 CUDA로 vLLM의 경량 고성능 LLM 추론 엔진 'Tiny-vLLM'
  직접 구축하기", section "고성능 추론을 위한 고급 최적화 기법" (attention over
  Q/K/V projections as in "Attention is all you need", GQA where several query
  heads share one key/value head, softmax and a causal mask), and section
  "모델 로딩 및 데이터 형식 심층 이해" (bfloat16 storage).
* "Nano-vLLM로 배우는 vLLM 추론 엔진 작동 원리 한눈에 정리", section "KV 캐시와
  Block Manager" (fixed-size blocks, block metadata on the CPU and KV tensors on
  the GPU, shared prompt prefixes reused block by block).

Readings where the pages are silent (cache layout inside a block, GQA grouping
order, whether the context length counts the appended token, what a padding
entry or a tail slot holds) are stated in the module that takes them.

Modules: numerics (bf16/fp16 bits to float64), layout (where an element lives
inside the physical cache), attention (the decode definition), prefill (causal
attention of many new tokens per sequence), append (the slot scatter), brute
(scalar loops for tiny cases), alloc_check (validity of block tables and
slots), kv_bytes (KV-size accounting), fp8 (the E4M3 KV cache), loop (replay
of a continuous-batching plan).
"""
from . import numerics, layout, attention, append, brute, alloc_check, kv_bytes, prefill  # noqa: F401
from .attention import decode  # noqa: F401
from .append import kv_append  # noqa: F401
