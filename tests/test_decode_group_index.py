"""CPU check of how the m <= 32 weight stream and the INT8 tile find the
quantization group of a fold unit without integer division: group =
floor((u + 1/2) * r) in float32, with u the unit index (32 or 64 K values
per unit) and r = 1/upg rounded to float32, upg = units per group. Checked
exhaustively against integer division for every group the pages allow with
k < 2^16 (k up to 65535, the Constraints section's limit), for every unit
index up to one past the last (the INT8 tile also asks for the group of the
next unit)."""
import numpy as np


def test_float_group_index_is_exact():
    for unit_k in (32, 64):
        for G in range(unit_k, 65536, unit_k):
            if unit_k == 64 and G % 128 == 0:
                continue                 # the weight stream folds those every 128 K values
            upg = G // unit_k
            units = np.arange(65536 // unit_k + 1, dtype=np.int64)
            r = np.float32(1.0) / np.float32(upg)
            got = ((units.astype(np.float32) + np.float32(0.5)) * r).astype(np.int64)
            assert np.array_equal(got, units // upg), G
