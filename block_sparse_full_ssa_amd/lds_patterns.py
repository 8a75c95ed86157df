"""The LDS read patterns of the attention kernels, one probe launch each.

Run under ``rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE
SQ_INSTS_LDS GRBM_GUI_ACTIVE``: every mode of ``ssa_probe_lds`` is launched
exactly once, in order 0 .. 9, so the n-th dispatch of the probe kernel is
mode n (the modes are listed with the probe's declaration).  The counters
then give the LDS cycles per read instruction and the share of those cycles
lost to bank conflicts for each pattern.
"""
from __future__ import annotations

import torch

MODES = 10


def main() -> None:
    import block_sparse_full_ssa_amd as ssa
    blocks = 2048
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    for mode in range(MODES):
        ssa.ssa_probe_lds(sink, blocks, 64, mode)
    torch.cuda.synchronize()
    print(f"ran LDS probe modes 0 .. {MODES - 1}", flush=True)


if __name__ == "__main__":
    main()
