"""The storage-type dispatch of the GPU parity checks without torch or a GPU:
the same rules and floor factors as gpu_util.check_values, for CPU tests of
the checker itself."""

import numpy as np

from tolerance import FLOOR_FACTOR, check_bf16, check_f16, check_f32


def check_values_cpu(got, ref64, dtype, scale=None):
    check = {"bf16": check_bf16, "f16": check_f16}.get(dtype, check_f32)
    sc = None if scale is None else np.asarray(scale, dtype=np.float64) * FLOOR_FACTOR[dtype]
    return check("cpu", got, ref64, scale=sc)
