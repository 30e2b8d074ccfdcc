"""Write the golden fixtures under tests/golden/.

Only the seeded input generators (datagen) and the oracle are called here.

rpbh_d3072.json  -- the OrbitQuant page's rotation draw for d = 3072 (seed
                    0x0EB17 + d; randperm then Rademacher signs from the same
                    generator, "orbit_quant.py", rpbh_params): head values and
                    sha256 of the little-endian arrays.
tq3_signs.json   -- the TQ3 page's sign vector (seed 42, _generate_sign_flips)
                    as a 128-bit mask, bit j set when sign j is -1.
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import datagen  # noqa: E402


def main():
    perm, signs = datagen.rpbh_params(3072)
    rp = {
        "source": "orbit_quant.py page, rpbh_params(d=3072); torch CPU generator",
        "seed": 0x0EB17 + 3072,
        "perm_head": perm[:8].tolist(),
        "signs_head": signs[:16].tolist(),
        "perm_int64_sha256": hashlib.sha256(perm.numpy().astype("<i8").tobytes()).hexdigest(),
        "signs_int8_sha256": hashlib.sha256(signs.numpy().astype("i1").tobytes()).hexdigest(),
    }
    with open(os.path.join(HERE, "rpbh_d3072.json"), "w") as f:
        json.dump(rp, f, indent=1)
    s = datagen.tq3_signs()
    mask = int.from_bytes(datagen.sign_mask_bytes(s), "little")
    ts = {
        "source": "tq3_core.py page, _generate_sign_flips(128, seed=42)",
        "mask_hex": hex(mask),
        "plus_count": int((s > 0).sum()),
    }
    with open(os.path.join(HERE, "tq3_signs.json"), "w") as f:
        json.dump(ts, f, indent=1)


if __name__ == "__main__":
    main()
