"""The constant SiLU tables the build generates for the fused quant kernels,
checked on the CPU against the oracle: every bf16 entry inside the table's
window is the oracle's silu of its gate, the entries outside it have the
closed forms of the kernel's lookup, and every fp16 entry (the gates with
2^-10 <= |g| < 2^7) is the oracle's silu.  The GPU tests check the full
lookups, the gates outside the tables included, exhaustively."""
import os
import re

import numpy as np
import pytest

from conftest import ROOT
from oracle import quant as oq

INC = os.path.join(ROOT, "_build", "silu_tables.inc")
pytestmark = pytest.mark.skipif(not os.path.exists(INC), reason="library not built")


def _table(name):
    body = open(INC).read().split(name)[1].split("};")[0].split("=", 1)[1]
    out = []
    for v in re.findall(r"-?0x[0-9a-fA-Fp.+-]+|-?__builtin_huge_val\(\)", body):
        out.append(float("-inf" if v.startswith("-") else "inf") if "huge" in v
                   else float.fromhex(v))
    return np.array(out, dtype=np.float64)


def test_bf16_table_is_the_oracle_silu():
    t = _table("kSiluBf16Table").reshape(2, 35, 128, 2)
    s = np.arange(2)[:, None, None]
    e = np.arange(100, 135)[None, :, None]
    m = np.arange(128)[None, None, :]
    g = ((s.astype(np.uint32) << 31) | (e.astype(np.uint32) << 23)
         | (m.astype(np.uint32) << 16)).view(np.float32)
    a, b = t[..., 0], t[..., 1]
    inside = g[:, 1:34].reshape(-1)
    want = oq.silu_f32(inside).view(np.uint32)
    assert np.array_equal(b[:, 1:34].reshape(-1).astype(np.float32).view(np.uint32), want)
    assert np.all(a[:, 1:34] == 0)
    # |g| < 2^-26: g / 2; g >= 2^7: g; g <= -2^7: -0 -- each with a -0 addend
    assert np.all(a[:, 0] == 0.5) and np.all(a[0, 34] == 1.0) and np.all(a[1, 34] == 0.0)
    assert np.all(np.signbit(b[:, 0])) and np.all(b[:, 0] == 0)
    assert np.all(np.signbit(b[:, 34])) and np.all(b[:, 34] == 0)


def test_fp16_table_is_the_oracle_silu():
    # every fp16 gate with exponent field 5..21 (2^-10 <= |g| < 2^7), per sign
    t = _table("kSiluF16Table")
    span = 17 << 10
    assert t.size == 2 * span
    mag = (5 << 10) + np.arange(span, dtype=np.uint32)
    bits = np.concatenate([mag, mag | 0x8000]).astype(np.uint16)
    g = bits.view(np.float16).astype(np.float32)
    assert np.all(np.abs(g[:span]) >= 2.0 ** -10) and np.all(np.abs(g[:span]) < 2.0 ** 7)
    want = oq.silu_f32(g).view(np.uint32)
    assert np.array_equal(t.astype(np.float32).view(np.uint32), want)
