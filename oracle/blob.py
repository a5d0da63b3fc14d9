"""Expert blob layout and fp64 dequantisation (test infrastructure).

The pages split one expert "row" into four tensors -- the fused gate/up weight
("w13"), the down weight ("w2") and one block-scale tensor for each -- and give
their sizes (page "GLM 5.3 Testing: HBM Expert Allocation", section "What the
slot cache is": 18.874 MB of weights plus 2.359 MB of scales; page "GB300 GLM 5.3
Testing", section "E1 v2": four row-copy launches per cached layer).  The order
of the parts, the nibble order and the scale-block direction are this project's
reading (the pages are silent):

  [w13 codes  : 2I rows x H/2 bytes]   rows 0..I-1 gate, rows I..2I-1 up
  [w13 scales : 2I rows x H/16 bytes]  one E4M3 per 16 consecutive K elements
  [w2 codes   : H rows x I/2 bytes]
  [w2 scales  : H rows x I/16 bytes]

Byte j of a code row holds element 2j in its low nibble and 2j+1 in its high
nibble.  Element value = e2m1(code) * e4m3(block scale) * global scale, with one
fp32 global scale per (expert, matrix).
"""
import numpy as np

from .formats import decode_e2m1, decode_e4m3


def part_layout(H: int, I: int):
    """{part: (offset, nbytes)} for one blob."""
    sizes = [
        ("w13_codes", 2 * I * (H // 2)),
        ("w13_scales", 2 * I * (H // 16)),
        ("w2_codes", H * (I // 2)),
        ("w2_scales", H * (I // 16)),
    ]
    out, off = {}, 0
    for name, n in sizes:
        out[name] = (off, n)
        off += n
    return out


def blob_size(H: int, I: int) -> int:
    lay = part_layout(H, I)
    return sum(n for _, n in lay.values())


def _dequant_matrix(codes: np.ndarray, scales: np.ndarray, rows: int, K: int, gs: float) -> np.ndarray:
    codes = codes.reshape(rows, K // 2)
    w = np.empty((rows, K), dtype=np.float64)
    w[:, 0::2] = decode_e2m1(codes & 0x0F)
    w[:, 1::2] = decode_e2m1(codes >> 4)
    sc = decode_e4m3(scales.reshape(rows, K // 16))
    w *= np.repeat(sc, 16, axis=1)
    w *= float(np.float32(gs))
    return w


def dequant_expert(blob, H: int, I: int, gs13: float, gs2: float):
    """Return (G [I,H], U [I,H], D [H,I]) in float64 for one expert blob."""
    blob = np.asarray(blob, dtype=np.uint8).reshape(-1)
    lay = part_layout(H, I)
    if blob.size != blob_size(H, I):
        raise ValueError("blob has %d bytes, layout needs %d" % (blob.size, blob_size(H, I)))
    o, n = lay["w13_codes"]
    so, sn = lay["w13_scales"]
    w13 = _dequant_matrix(blob[o:o + n], blob[so:so + sn], 2 * I, H, gs13)
    o, n = lay["w2_codes"]
    so, sn = lay["w2_scales"]
    w2 = _dequant_matrix(blob[o:o + n], blob[so:so + sn], H, I, gs2)
    return w13[:I], w13[I:], w2
