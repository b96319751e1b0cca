"""Writes the oracle regression fixtures in this folder.

It calls only ``oracle/`` (and the seeded input generators); nothing here
comes from the HIP library.  Run from the repository root:

    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

from oracle import fp4, int4  # noqa: E402
from weight_only_bit_group_amd import synth  # noqa: E402


def main():
    case = synth.single_linear(0)
    packed, s, z = int4.quantize_pack(case["W"], case["group"])
    y = int4.forward(synth.bf16_bits_to_f32(case["X"]), packed, s, z, case["group"])
    with open(os.path.join(HERE, "int4_small.json"), "w") as f:
        json.dump({"source": "oracle.int4 on the 256x256 fp32 single-linear case, seed 0, g=128",
                   "packed_hex": packed.tobytes().hex(),
                   "scales_bits": s.view(np.uint32).tolist(),
                   "zeros": z.tolist(),
                   "y_row0_first8": y[0, :8].tolist()}, f)
    w = synth.fp4_weight_f32(5, 8, 64)
    codes, b, ts = fp4.encode(w)
    with open(os.path.join(HERE, "fp4_small.json"), "w") as f:
        json.dump({"source": "oracle.fp4.encode on an 8x64 N(0,0.02) matrix, seed 5",
                   "codes_hex": codes.tobytes().hex(), "block_scales": b.tolist(),
                   "ts_bits": int(np.float32(ts).view(np.uint32))}, f)


if __name__ == "__main__":
    main()
