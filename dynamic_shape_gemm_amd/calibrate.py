"""Offline stage: measure the micro-kernel performance table on this GPU.

    python -m dynamic_shape_gemm_amd.calibrate [out_path]

Runs mkp_calibrate (every library kernel at full occupancy for t = 1..256 K
steps, 20 warm-up launches per point; the MikPoly page's offline
micro-kernel performance model, section 3) and writes the table, by default
to calib/gfx950.tbl next to the library, where mkp loads it at start-up.
"""
import os
import sys

import dynamic_shape_gemm_amd as mkp


def main():
    out = sys.argv[1] if len(sys.argv) > 1 else os.path.join(os.path.dirname(mkp.LIB_PATH), "calib", "gfx950.tbl")
    os.makedirs(os.path.dirname(out) or ".", exist_ok=True)
    mkp.mkp_calibrate(out)
    print(open(out).read())


if __name__ == "__main__":
    main()
