"""The matrix-core decode computes floor(x / L) of packed field values with
one fp16 FMA: a field value x enters as the fp16 value 1536 + x (exact in
[1024, 2048), where the fp16 spacing is 1) and RNE((1536 + x) m + k) must
equal 1536 + floor(x / L).  This checks the kernel's constants m and k for
every field value of each level count, in exact rational arithmetic (the
FMA rounds once), and that they are fp16 values."""
import os
import re
from fractions import Fraction

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "..", "kv_cache_mixed_top_amd", "csrc", "decode_mfma_kernel.h")


def _constants():
    text = open(SRC).read()
    m = re.search(r"constexpr float floor_m\(\) \{\s*return (.*?);\s*\}", text, re.S).group(1)
    k = re.search(r"constexpr float floor_k\(\) \{\s*return (.*?);\s*\}", text, re.S).group(1)

    def table(expr):
        # "L == 6 ? a : L == 5 ? b : c" -> {6: a, 5: b, None: c}
        out = {}
        for L, v in re.findall(r"L == (\d+) \? ([0-9.]+)f", expr):
            out[int(L)] = float(v)
        out[None] = float(re.findall(r": ([0-9.]+)f\s*$", expr.strip())[0])
        return out
    return table(m), table(k)


def _rne_int(v: Fraction) -> int:
    fl = v.numerator // v.denominator
    fr = v - fl
    if fr != Fraction(1, 2):
        return fl + (1 if fr > Fraction(1, 2) else 0)
    return fl if fl % 2 == 0 else fl + 1


@pytest.mark.parametrize("L,xmax", [(6, 216), (5, 125), (3, 243), (8, 64)])
def test_floor_by_fma(L, xmax):
    mt, kt = _constants()
    m = mt.get(L, mt[None])
    k = kt.get(L, kt[None])
    assert float(np.float16(m)) == m and float(np.float16(k)) == k     # fp16 operands
    fm, fk = Fraction(m), Fraction(k)
    for x in range(xmax):
        v = (1536 + x) * fm + fk
        assert 1024 <= v < 2048, (L, x)           # stays where the fp16 spacing is 1
        assert _rne_int(v) == 1536 + x // L, (L, x)
