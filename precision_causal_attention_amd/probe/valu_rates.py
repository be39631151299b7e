"""Issue costs of the softmax's vector instructions on the GPU (probe library).

python3 -m precision_causal_attention_amd.probe.valu_rates

Runs every probe of libflamia_probe.so's flamia_probe_valu_rate (8 workgroups
per CU, i.e. 8 waves per SIMD, each thread 8 independent chains) and prints,
per instruction (or pair of instructions), the median launch time of 5, the
cycles per wave-instruction per SIMD at 2.4 GHz and the cost relative to
v_fma_f32.
"""
from __future__ import annotations

import ctypes
import os
import sys

PKG = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CUS = 256
SIMDS = 4 * CUS
CLOCK_HZ = 2.4e9
CHAINS = 8


def main() -> int:
    import torch

    path = os.path.join(PKG, "libflamia_probe.so")
    if not os.path.exists(path):
        print(f"{path} is missing: build it with precision_causal_attention_amd.build.build()", file=sys.stderr)
        return 2
    lib = ctypes.CDLL(path)
    lib.flamia_probe_valu_count.restype = ctypes.c_int
    lib.flamia_probe_valu_name.restype = ctypes.c_char_p
    lib.flamia_probe_valu_name.argtypes = [ctypes.c_int]
    lib.flamia_probe_valu_rate.restype = ctypes.c_int
    lib.flamia_probe_valu_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    wg, iters = 8 * CUS, 2048
    sink = torch.zeros(wg * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    # wave-instructions each SIMD issues per launch (pairs count once)
    per_simd = wg * 4 / SIMDS * iters * CHAINS
    rows = []
    for op in range(lib.flamia_probe_valu_count()):
        times = []
        for rep in range(6):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            rc = lib.flamia_probe_valu_rate(op, wg, iters, ctypes.c_void_p(sink.data_ptr()),
                                            ctypes.c_void_p(stream.cuda_stream))
            b.record(stream)
            if rc != 0:
                raise RuntimeError(f"flamia_probe_valu_rate({op}) failed: {rc}")
            torch.cuda.synchronize()
            if rep:
                times.append(a.elapsed_time(b))
        times.sort()
        ms = times[len(times) // 2]
        rows.append((lib.flamia_probe_valu_name(op).decode(), ms))
    base = rows[0][1]
    print("| instruction | ms per launch | cycles per wave-instruction (2.4 GHz) | relative to v_fma_f32 |")
    print("|---|---|---|---|")
    for name, ms in rows:
        print(f"| {name} | {ms:.3f} | {ms * 1e-3 * CLOCK_HZ / per_simd:.2f} | {ms / base:.2f} |")
    return 0


if __name__ == "__main__":
    sys.exit(main())
