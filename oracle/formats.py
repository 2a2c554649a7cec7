"""Number formats and the record decoder (oracle side).

The pages name the formats only: int4 with a group step ([Edge0] "무엇인가" and
"어떻게 쓰나"), NVFP4 with e4m3 block scales ([NVMe-8GB] "왜 이 모델인가",
"엔진" item 4), and the per-expert record gate|up|down|gate_scale|up_scale|
down_scale ([NVMe-8GB] "엔진" item 1).  The bit-level definitions used here:

* int4-g32-bf16: nibble u in [0, 15], value (u - 8) * s, s one bf16 per 32
  consecutive inputs of a row.
* NVFP4: e2m1 code c (bit 3 sign, bits 2..1 exponent with bias 1, bit 0
  mantissa; exponent 0 is subnormal), times one e4m3 scale per 16 inputs of a
  row, times one fp32 scale per matrix.
* e4m3: OCP E4M3FN, bias 7, subnormals, S.1111.111 = NaN, no infinities.

Record byte layout (the layout the library is written against; restated here
independently of the writer): a matrix of N output rows by Kd inputs is cut
into tiles of 16 rows x 32 inputs, tile index (n // 16) * (Kd // 32) + k // 32
(row slices outer, inputs inner).  A tile's 256 payload bytes hold element
(n, k) at byte (q*16 + r)*4 + i//2 with r = n%16, q = (k%32)//8, i = k%8, even
i in the low nibble.  Each tile has 32 scale bytes at the same index in the
scale area: int4 keeps the bf16 of (n, k//32) at byte r*2; NVFP4 keeps the
e4m3 of (n, k//16) at byte ((k%32)//16)*16 + r.  Record = gate[I,H] | up[I,H] |
down[H,I] payloads, then their scales in the same order.
"""
from __future__ import annotations

import numpy as np

INT4 = 0
NVFP4 = 1

MATRICES = ("gate", "up", "down")


# ----------------------------------------------------------------------------- scalars

def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round to bf16, nearest-even (via fp32; inputs here are far from ties at fp32 precision)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def e2m1_value(code) -> np.ndarray:
    """Value of an e2m1 code (0..15): (-1)^s * 2^(e-1) * (1 + m/2), or m/2 when e = 0."""
    c = np.asarray(code, dtype=np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(s == 1, -mag, mag)


def e4m3_value(code) -> np.ndarray:
    """Value of an OCP E4M3FN code (0..255); NaN for S.1111.111."""
    c = np.asarray(code, dtype=np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def int4_value(u) -> np.ndarray:
    return np.asarray(u, dtype=np.int64) - 8


# ----------------------------------------------------------------------------- record layout

def record_bytes(H: int, I: int) -> int:
    """gate, up, down payloads (H*I/2 bytes each) + scales (H*I/16 bytes each, both formats)."""
    return 3 * (H * I // 2) + 3 * (H * I // 16)


def matrix_shape(m: int, H: int, I: int):
    return (H, I) if m == 2 else (I, H)


def tile_index(Kd: int, n: np.ndarray, k: np.ndarray) -> np.ndarray:
    return (n // 16) * (Kd // 32) + k // 32


def payload_index(Kd: int, n: np.ndarray, k: np.ndarray):
    """(byte offset within the matrix payload, nibble shift 0|4) of elements (n, k)."""
    r, q, i = n % 16, (k % 32) // 8, k % 8
    return tile_index(Kd, n, k) * 256 + (q * 16 + r) * 4 + i // 2, (i % 2) * 4


def scale_index(fmt: int, Kd: int, n: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Byte offset within the matrix scale area of the scale that covers (n, k)."""
    base = tile_index(Kd, n, k) * 32
    if fmt == INT4:
        return base + (n % 16) * 2
    return base + ((k % 32) // 16) * 16 + n % 16


def dequant_matrix(rec: np.ndarray, fmt: int, H: int, I: int, m: int, ts: float = 1.0) -> np.ndarray:
    """Dequantized matrix m (0 gate [I,H], 1 up [I,H], 2 down [H,I]) of one record, float64."""
    rec = np.asarray(rec, dtype=np.uint8)
    assert rec.size == record_bytes(H, I)
    N, Kd = matrix_shape(m, H, I)
    pay = rec[m * (H * I // 2):(m + 1) * (H * I // 2)]
    sca = rec[3 * (H * I // 2) + m * (H * I // 16): 3 * (H * I // 2) + (m + 1) * (H * I // 16)]
    n, k = np.meshgrid(np.arange(N, dtype=np.int64), np.arange(Kd, dtype=np.int64), indexing="ij")
    off, sh = payload_index(Kd, n, k)
    code = (pay[off].astype(np.int64) >> sh) & 15
    so = scale_index(fmt, Kd, n, k)
    if fmt == INT4:
        sbits = sca[so].astype(np.uint16) | (sca[so + 1].astype(np.uint16) << 8)
        return int4_value(code).astype(np.float64) * bf16_bits_to_f64(sbits)
    return e2m1_value(code) * e4m3_value(sca[so]) * float(ts)


def dequant_record(rec: np.ndarray, fmt: int, H: int, I: int, ts=(1.0, 1.0, 1.0)):
    """(W_gate [I,H], W_up [I,H], W_down [H,I]) in float64."""
    return tuple(dequant_matrix(rec, fmt, H, I, m, float(ts[m])) for m in range(3))
