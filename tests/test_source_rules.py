"""Host-side checks of the HIP sources for forms that compile to wrong code on this
toolchain.

`__builtin_bit_cast(T, v[i])`, with v an ext_vector_type value and the element
taken inside the cast, has been compiled to a read of element 0 whatever i is
(seen twice in these kernels, each time as a silent wrong result).  The sources
copy the element into a scalar first; this test keeps it that way."""
import glob
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = sorted(glob.glob(os.path.join(ROOT, "gated_delta_rule_29_amd", "csrc", "*.hip")) +
                 glob.glob(os.path.join(ROOT, "gated_delta_rule_29_amd", "csrc", "*.hpp")))
BITCAST_OF_ELEMENT = re.compile(r"__builtin_bit_cast\(\s*[\w:]+\s*,\s*[\w.]+(\[[^\]]+\])+\s*\)")


def test_sources_found():
    assert len(SOURCES) >= 4


def test_no_bit_cast_of_a_subscripted_element():
    bad = []
    for path in SOURCES:
        for n, line in enumerate(open(path), 1):
            if BITCAST_OF_ELEMENT.search(line):
                bad.append(f"{os.path.basename(path)}:{n}: {line.strip()}")
    assert not bad, "\n".join(bad)


def test_the_pattern_catches_the_known_form():
    assert BITCAST_OF_ELEMENT.search("m = __builtin_bit_cast(uint32_t, u[i]) & 1;")
    assert BITCAST_OF_ELEMENT.search("__builtin_bit_cast(float, X[rt][ct][m])")
    assert not BITCAST_OF_ELEMENT.search("__builtin_bit_cast(uint32_t, val)")
