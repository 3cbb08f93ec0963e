"""Measured ceilings of the device (measurement infrastructure, run on the GPU):

    python tests/hw/ceilings.py

  * the scaled fp8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) in a register-only loop on every CU
    (tests/hw/libmfmaprobe.so, mfma_peak): TFLOP/s at the sustained clock;
  * HBM bandwidth of a plain device-to-device copy of 4 GiB (torch's copy kernel): GB/s counted
    as bytes read + bytes written.
Prints one JSON line."""
import ctypes
import json
import os

import torch

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmfmaprobe.so")


def main():
    lib = ctypes.CDLL(LIB)
    lib.mfma_peak.restype = ctypes.c_float
    lib.mfma_peak.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    blocks, iters = cus * 8, 4000
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    ms = lib.mfma_peak(iters, blocks, ctypes.c_void_p(out.data_ptr()))
    flop = blocks * 4 * iters * 4 * (2.0 * 32 * 32 * 64)   # waves x chains x iterations x FLOP per MFMA
    src = torch.empty(1 << 30, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_ms = e0.elapsed_time(e1) / 5
    print(json.dumps({"device": props.name, "cus": cus,
                      "mfma_scale_f8_tflops": round(flop / (ms * 1e-3) / 1e12, 1), "mfma_ms": round(ms, 4),
                      "copy_gbs": round(2 * src.numel() * 4 / (copy_ms * 1e-3) / 1e9, 1), "copy_ms": round(copy_ms, 4)}),
          flush=True)


if __name__ == "__main__":
    main()
