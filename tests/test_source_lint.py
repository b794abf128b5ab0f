"""Source patterns the device compiler is known to mishandle.

__builtin_bit_cast to a scalar type applied directly to an element of an
ext_vector value (``__builtin_bit_cast(float, v[1])``) is lowered as a load from
the vector's first element, silently: the cast reads v[0] whatever the index.
Casting an rvalue (``(unsigned)v[1]``, ``v[i] << 16``) or a whole vector is
fine. No kernel source may use a scalar bit cast of a subscripted operand.
"""

import glob
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SCALARS = r"(?:float|double|int|unsigned|unsigned int|uint32_t|int32_t|uint16_t|short|_Float16|__bf16)"
PATTERN = re.compile(r"__builtin_bit_cast\(\s*" + SCALARS + r"\s*,\s*[A-Za-z_][A-Za-z0-9_.]*\s*\[[^]]*\]\s*\)")


def test_no_scalar_bit_cast_of_a_vector_element():
    bad = []
    for f in sorted(glob.glob(os.path.join(ROOT, "mla_latent_kv_amd", "csrc", "*"))):
        for n, line in enumerate(open(f), 1):
            if PATTERN.search(line):
                bad.append(f"{os.path.basename(f)}:{n}: {line.strip()}")
    assert not bad, "\n".join(bad)


def test_lint_pattern_matches_the_known_bad_form():
    assert PATTERN.search("x1 += __builtin_bit_cast(float, v[1]);")
    assert not PATTERN.search("return Pair32{__builtin_bit_cast(float, (unsigned)r[0])};")
    assert not PATTERN.search("const float lo = __builtin_bit_cast(float, v[i] << 16);")
    assert not PATTERN.search("qa[ks] = __builtin_bit_cast(f16x8, src[ks * 64 + lane]);")
