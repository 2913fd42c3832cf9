"""Pins of the oracle's MXFP4 decode ("Phase 19: MoE - gpt-oss-20b", section 3
and the tensor-layout listing: 32-element blocks along the input dim, 16 bytes
per block, low nibble = even index, one E8M0 scale per block, value =
lut[code] * 2^(e8m0 - 127)) against the E2M1 table of the OCP MX v1.0 spec."""
import json
import os

import numpy as np

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))
TABLE = json.load(open(os.path.join(HERE, "golden", "e2m1_values.json")))["values"]


def test_decode_exhaustive_against_spec_table():
    for code in range(16):
        for e in range(0, 255):
            v = oracle.mxfp4_value(code, e)
            ref = TABLE[code] * 2.0 ** (e - 127)
            assert v == ref or (v == 0.0 and ref == 0.0), (code, e)


def _table_dequant(codes, scales, cols):
    """Independent table-driven decoder: codes [rows][cols/32][16] u8."""
    rows = codes.shape[0]
    b = codes.reshape(rows, cols // 2)
    lo, hi = b & 15, b >> 4
    q = np.empty((rows, cols), np.uint8)
    q[:, 0::2], q[:, 1::2] = lo, hi
    vals = np.array(TABLE, np.float64)[q]
    return vals * np.exp2(np.repeat(scales.reshape(rows, cols // 32).astype(np.float64) - 127.0, 32, axis=1))


def test_nibble_order_and_block_scale_index():
    codes = np.zeros((1, 2, 16), np.uint8)
    codes[0, 0, 0] = 0x21      # element 0 <- code 1 (0.5), element 1 <- code 2 (1.0)
    codes[0, 1, 15] = 0xF7     # element 62 <- code 7 (6.0), element 63 <- code 15 (-6.0)
    scales = np.array([[127, 130]], np.uint8)
    m = oracle.RefMat(oracle.REF_MXFP4, codes.ctypes.data, scales.ctypes.data)
    el = lambda col: oracle.lib().ref_elem(m, 0, col, 64)
    assert el(0) == 0.5 and el(1) == 1.0 and el(2) == 0.0
    assert el(62) == 6.0 * 8 and el(63) == -6.0 * 8
    full = _table_dequant(codes, scales, 64)
    assert all(el(j) == full[0, j] for j in range(64))


def test_dequantised_values_exact_in_bf16():
    # every E2M1 value times 2^(e-127), e in [118, 130], has <= 2 significant bits
    for code in range(16):
        for e in range(118, 131):
            v = np.float32(oracle.mxfp4_value(code, e))
            assert synth.bf16_to_f32(synth.bf16_bits(np.array([v])))[0] == v


def test_mxfp4_layer_equals_bf16_layer_with_table_dequantised_weights():
    c = synth.make_case("gptoss20b_mxfp4", T=2, E=4, H=64, F=64, k=2)
    L4 = oracle.Layer(c)
    out4, i4, w4, _ = L4.forward()
    cb = synth.make_case("gptoss20b_mxfp4", T=2, E=4, H=64, F=64, k=2)
    E, H, F = cb.E, cb.H, cb.F
    gu = _table_dequant(cb.t.pop("gate_up_codes").reshape(E * 2 * F, H // 32, 16),
                        cb.t.pop("gate_up_scales"), H).reshape(E, 2 * F, H)
    dn = _table_dequant(cb.t.pop("down_codes").reshape(E * H, F // 32, 16),
                        cb.t.pop("down_scales"), F).reshape(E, H, F)
    cb.t["gate_up_w"] = synth.bf16_bits(gu.astype(np.float32))
    cb.t["down_w"] = synth.bf16_bits(dn.astype(np.float32))
    assert np.array_equal(synth.bf16_to_f32(cb.t["gate_up_w"]), gu.astype(np.float32))
    cb.w_dtype = "bf16"
    outb, ib, wb, _ = oracle.Layer(cb).forward()
    assert np.array_equal(i4, ib) and np.array_equal(w4, wb)
    assert np.array_equal(out4, outb)
