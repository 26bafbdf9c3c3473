"""The pages' one worked numeric example (tests/golden/worked_example_fp4.json)."""
import json
import os

import numpy as np

import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def load():
    with open(os.path.join(HERE, "golden", "worked_example_fp4.json"), encoding="utf-8") as f:
        return json.load(f)


def block_of(values):
    x = np.zeros(32, dtype=np.float32)
    x[:len(values)] = values
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)       # the values are exact in BF16
    assert np.array_equal(O.widen(bits, "bf16")[:len(values)], np.array(values))
    return bits


def test_shared_scale_is_2_pow_minus_4_under_both_rules():
    g = load()
    bits = block_of(g["inputs_bf16"])
    for mode in (O.FLOOR, O.ROUNDUP):
        out = O.quantize(bits.reshape(1, 32), "bf16", O.E2M1, mode, O.ROW)
        assert int(out["row_scales"][0, 0, 0]) == g["pinned"]["scale_code"]
        assert int(out["row_scales"][0, 0, 0]) - 127 == g["pinned"]["scale_exponent"]


def test_scaled_values_printed_on_the_page():
    g = load()
    bits = block_of(g["inputs_bf16"])
    out = O.quantize(bits.reshape(1, 32), "bf16", O.E2M1, O.FLOOR, O.ROW)
    codes = O.unpack_e2m1(out["row_codes"][0, 0])[:4]
    vals = O.value_table(O.E2M1)[codes]
    for i in g["pinned"]["agreeing_scaled_positions"]:
        assert vals[i] == g["printed_scaled_fp4"][i]
    assert codes.tolist() == g["pinned"]["scaled_codes_rne"]
    assert vals.tolist() == g["pinned"]["scaled_values_rne"]


def test_direct_cast_printed_on_the_page():
    g = load()
    x = np.array(g["inputs_bf16"])
    codes = O.encode_elements(x, O.E2M1)               # scale 2^0: no block scaling
    vals = O.value_table(O.E2M1)[codes]
    for i in g["pinned"]["agreeing_direct_positions"]:
        assert vals[i] == g["printed_direct_fp4"][i]
    assert codes.tolist() == g["pinned"]["direct_codes_rne"]
    assert vals.tolist() == g["pinned"]["direct_values_rne"]
