"""Source checks on the HIP kernels that need no GPU."""
import glob
import os

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "weight_recurrent_sequence_amd", "csrc")


def test_mfma_builtins_only_in_the_fragment_helpers():
    # every matrix product goes through the helpers of falcon_device.h, whose
    # K = 16 bf16 product runs on the K = 32 instruction unless a kernel asks
    # for the 16x16x16 one by name (the assembly checks cover those kernels)
    paths = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h")))
    assert paths
    for path in paths:
        if os.path.basename(path) == "falcon_device.h":
            continue
        assert "__builtin_amdgcn_mfma" not in open(path).read(), path
