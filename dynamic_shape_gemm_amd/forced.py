"""Run one micro-kernel, forced, on one GEMM shape: for profiling a single
kernel under rocprofv3.

    python -m dynamic_shape_gemm_amd.forced m256n256k64 4096 4096 4096 [--splits S] [--calls N] [--copies C]

B is K x N (`_nk` kernels: N x K); operands are uniform bf16 bit patterns
drawn on the device; the calls go through the C ABI on the current stream.
With --copies C > 1 the calls take B from C copies in turn, so that a B
smaller than the 256 MB last-level cache still streams from HBM.
"""
from __future__ import annotations

import argparse


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("kernel")
    ap.add_argument("M", type=int)
    ap.add_argument("N", type=int)
    ap.add_argument("K", type=int)
    ap.add_argument("--splits", type=int, default=1)
    ap.add_argument("--calls", type=int, default=8)
    ap.add_argument("--copies", type=int, default=1)
    a = ap.parse_args()
    import torch
    import dynamic_shape_gemm_amd as mkp

    if not torch.cuda.is_available():
        raise SystemExit("needs a GPU")
    torch.cuda.set_device(0)
    st = torch.cuda.current_stream().cuda_stream
    bt = a.kernel.endswith("_nk")
    mkp.mkp_set_option("transpose_b", 0)
    mkp.mkp_set_option("force_kernel", a.kernel)
    mkp.mkp_set_option("force_splitk", a.splits)
    A = torch.randint(-16000, 16000, (a.M, a.K), dtype=torch.int16, device="cuda")
    Bs = [torch.randint(-16000, 16000, (a.N, a.K) if bt else (a.K, a.N), dtype=torch.int16, device="cuda")
          for _ in range(max(1, a.copies))]
    C = torch.empty((a.M, a.N), dtype=torch.float32, device="cuda")
    fn = mkp.mkp_gemm_bt if bt else mkp.mkp_gemm
    for i in range(a.calls):
        fn(a.M, a.N, a.K, A, a.K, Bs[i % len(Bs)], a.K if bt else a.N, C, a.N, st)
    torch.cuda.synchronize()
    print(f"{a.kernel} s={a.splits} {a.M}x{a.N}x{a.K}: {a.calls} calls", flush=True)


if __name__ == "__main__":
    main()
