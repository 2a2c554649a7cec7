"""The five workloads (shapes, formats, cache sizes, routing statistics).

Shapes follow the model shapes named on the pages: the 35B-A3B expert shape
(Edge0 summary, "무엇인가": 40 layers x 256 experts, 1.77 MB per expert), the
DeepSeek-V4-Flash shape (FreeToken deep dive §1 and FreeToken blog §二: 43 layers x
256 experts, top-6) and the Qwen3.8-Flash-Next shape (NVMe streaming page,
"왜 이 모델인가": 48 layers x 512 experts, top-10, 2560 x 640 matrices).
"""
from dataclasses import dataclass, field
from typing import Tuple

from . import FMT_INT4, FMT_NVFP4


@dataclass(frozen=True)
class Workload:
    name: str
    L: int
    E: int
    K: int
    H: int
    I: int
    fmt: int
    S: int
    f_q16: int
    seed: int
    zipf_s: float = 0.0          # 0 -> routing from route() on seeded x and router weights
    batches: Tuple[int, ...] = (1,)
    warmup_tokens: int = 0
    measure_tokens: int = 0
    spec_keep: float = -1.0      # >= 0 -> speculative next-layer requests
    prefill_T: int = 0
    f_sweep: Tuple[int, ...] = field(default_factory=tuple)


def seed_of(c: int) -> int:
    return 20261202 + c


TINY = Workload("tiny-moe-decode", L=2, E=8, K=2, H=64, I=128, fmt=FMT_INT4, S=4, f_q16=65536,
                seed=seed_of(1), batches=(1,), measure_tokens=64,
                f_sweep=(0, 1, 16384, 32768, 49152, 65535, 65536))

A3B = Workload("35b-a3b-decode", L=40, E=256, K=8, H=2048, I=512, fmt=FMT_INT4, S=5120, f_q16=26214,
               seed=seed_of(2), zipf_s=1.1, batches=(1,), warmup_tokens=1024, measure_tokens=256)

DSV4_DECODE = Workload("dsv4-flash-decode", L=43, E=256, K=6, H=4096, I=2048, fmt=FMT_NVFP4, S=2201,
                       f_q16=45875, seed=seed_of(3), zipf_s=1.0, batches=(1, 4), warmup_tokens=256,
                       measure_tokens=64)

DSV4_PREFILL = Workload("dsv4-flash-prefill", L=43, E=256, K=6, H=4096, I=2048, fmt=FMT_NVFP4, S=2201,
                        f_q16=45875, seed=seed_of(4), prefill_T=2048)

QWEN_NEXT = Workload("qwen3.8-flash-next-decode", L=48, E=512, K=10, H=2560, I=640, fmt=FMT_NVFP4,
                     S=2457, f_q16=65535, seed=seed_of(5), zipf_s=1.2, batches=(1, 8, 16),
                     warmup_tokens=512, measure_tokens=128, spec_keep=0.65)

ALL = (TINY, A3B, DSV4_DECODE, DSV4_PREFILL, QWEN_NEXT)
