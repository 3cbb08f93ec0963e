"""LDS read-pattern costs on the device (measurement infrastructure, run on the GPU):

    python tests/hw/lds_banks.py

Times one read instruction kind (16-byte, 8-byte, 8-byte transpose) at the per-lane offsets of the
kernels' LDS operand reads (tests/hw/libldsprobe.so, lds_probe) and prints, per pattern, the time per
wave read instruction per CU and its ratio to the linear pattern of the same kind.  Lane l is
(n, g) = (l % 32, l // 32) for row reads (lane n reads row n, lane half g its block or chunk g), and
(G, i16) = (l // 16, l % 16), row 16 (G // 2) + i16 // 2, for the transpose reads."""
import ctypes
import json
import os

import torch

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libldsprobe.so")
B128, B64, TR8 = 0, 1, 2
SIZE = {B128: 16, B64: 8, TR8: 8}


def qrow(n):
    """Query row that lane n feeds the backward's E4M3 S and dP products (rows of a 32-row block)."""
    return (((n >> 2) & 1) << 4) | (((n >> 3) & 3) << 2) | (n & 3)


def kslot(r):
    """16-byte slot of row r in the backward's paired-row E4M3 K tile."""
    return 8 * r + 2 * (r >> 1) + ((r >> 3) & 1)


def qslot(r):
    """16-byte slot of row r in the backward's paired-row E4M3 Q and dO tiles."""
    return 8 * r + 2 * (r >> 1) + ((r >> 4) & 1)


def row_pattern(f):
    return [f(l % 32, l // 32) for l in range(64)]


def tr_pattern(f):
    out = []
    for l in range(64):
        G, i16 = l // 16, l % 16
        out.append(f(16 * (G // 2) + i16 // 2, G, i16))
    return out


PATTERNS = [
    (B128, "linear 16 B per lane", [16 * l for l in range(64)]),
    (B128, "rows 144 B (backward E4M3 V), chunk g", row_pattern(lambda n, g: 144 * n + 16 * g)),
    (B128, "rows 144 B, permuted query rows qrow(n)", row_pattern(lambda n, g: 144 * qrow(n) + 16 * g)),
    (B128, "paired rows kslot(n) (backward E4M3 K)", row_pattern(lambda n, g: 16 * kslot(n) + 16 * g)),
    (B128, "paired rows qslot(qrow(n)) (backward E4M3 Q, dO)", row_pattern(lambda n, g: 16 * qslot(qrow(n)) + 16 * g)),
    (B128, "rows 128 B, chunk g in slot g ^ (n & 7)", row_pattern(lambda n, g: 128 * n + 16 * (g ^ (n & 7)))),
    (B128, "rows 128 B, chunk g in slot g ^ ((n >> 1) & 7) (forward E4M3 K)",
     row_pattern(lambda n, g: 128 * n + 16 * (g ^ ((n >> 1) & 7)))),
    (B128, "rows 64 B, chunk g (backward E2M1 Q, K)", row_pattern(lambda n, g: 64 * n + 16 * g)),
    (B128, "rows 64 B, chunk g in slot g ^ (n & 3)", row_pattern(lambda n, g: 64 * n + 16 * (g ^ (n & 3)))),
    (B128, "rows 64 B, chunk g in slot g ^ ((n >> 2) & 3) (forward E2M1 K, GEMM E4M3)",
     row_pattern(lambda n, g: 64 * n + 16 * (g ^ ((n >> 2) & 3)))),
    (B128, "rows 80 B, chunk g", row_pattern(lambda n, g: 80 * n + 16 * g)),
    (B128, "rows 32 B, chunk g in slot g ^ ((n >> 3) & 1) (GEMM E2M1)",
     row_pattern(lambda n, g: 32 * n + 16 * (g ^ ((n >> 3) & 1)))),
    (B64, "linear 8 B per lane", [8 * l for l in range(64)]),
    (B64, "rows 96 B, block g at 24 g (backward E2M3 Q)", row_pattern(lambda n, g: 96 * n + 24 * g)),
    (B64, "rows 104 B, block g at 24 g (backward E2M3 K)", row_pattern(lambda n, g: 104 * n + 24 * g)),
    (B64, "rows 112 B, block g at 24 g (forward E2M3 K)", row_pattern(lambda n, g: 112 * n + 24 * g)),
    (B64, "rows 80 B, block g at 24 g (GEMM E2M3)", row_pattern(lambda n, g: 80 * n + 24 * g)),
    (B64, "column blocks 24 B apart (backward E2M3 column-packed Q, K)",
     row_pattern(lambda n, g: 24 * (n + 32 * g))),
    (TR8, "rows 128 B unswizzled", tr_pattern(lambda r, G, i: 128 * r + 16 * (G & 1) + 8 * (i & 1))),
    (TR8, "rows 144 B", tr_pattern(lambda r, G, i: 144 * r + 16 * (G & 1) + 8 * (i & 1))),
    (TR8, "paired rows kslot(r) (backward E4M3 K)", tr_pattern(lambda r, G, i: 16 * kslot(r) + 16 * (G & 1) + 8 * (i & 1))),
    (TR8, "paired rows qslot(r) (backward E4M3 Q, dO)", tr_pattern(lambda r, G, i: 16 * qslot(r) + 16 * (G & 1) + 8 * (i & 1))),
    (TR8, "rows 80 B", tr_pattern(lambda r, G, i: 80 * r + 16 * (G & 1) + 8 * (i & 1))),
    (TR8, "rows 64 B, 32 spare bytes after every fourth (backward E4M3 dS)",
     tr_pattern(lambda r, G, i: 64 * r + 32 * (r >> 2) + 16 * (G & 1) + 8 * (i & 1))),
    (TR8, "rows 128 B, slot ^ (r & 7) (forward V)",
     tr_pattern(lambda r, G, i: 128 * r + 16 * ((G & 1) ^ (r & 7)) + 8 * (i & 1))),
    (TR8, "rows 128 B, slot ^ ((r >> 1) & 7)",
     tr_pattern(lambda r, G, i: 128 * r + 16 * ((G & 1) ^ ((r >> 1) & 7)) + 8 * (i & 1))),
    (B128, "rows 128 B, chunk g in slot g ^ ((n & 6) | ((n >> 3) & 1))",
     row_pattern(lambda n, g: 128 * n + 16 * (g ^ ((n & 6) | ((n >> 3) & 1))))),
    (TR8, "rows 128 B, slot ^ ((r & 6) | ((r >> 3) & 1))",
     tr_pattern(lambda r, G, i: 128 * r + 16 * ((G & 1) ^ ((r & 6) | ((r >> 3) & 1))) + 8 * (i & 1))),
    (TR8, "rows 128 B, slot ^ ((r & 6) | ((r >> 3) & 1)), rows r + 8",
     tr_pattern(lambda r, G, i: 128 * (r + 8) + 16 * ((G & 1) ^ (((r + 8) & 6) | (((r + 8) >> 3) & 1))) + 8 * (i & 1))),
    (TR8, "rows 64 B, slot ^ (2 ((r >> 2) & 1))",
     tr_pattern(lambda r, G, i: 64 * r + 16 * ((G & 1) ^ (2 * ((r >> 2) & 1))) + 8 * (i & 1))),
    (TR8, "rows 64 B, slot ^ (r & 3) (backward small-format dS)",
     tr_pattern(lambda r, G, i: 64 * r + 16 * ((G & 1) ^ (r & 3)) + 8 * (i & 1))),
]


def main():
    lib = ctypes.CDLL(LIB)
    lib.lds_probe.restype = ctypes.c_float
    lib.lds_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = cus * 8, 512
    out = torch.empty(blocks * 512, dtype=torch.int32, device="cuda")
    base = {}
    rows = []
    for kind, name, offs in PATTERNS:
        assert len(offs) == 64 and all(0 <= o and o + SIZE[kind] + 7 * 4096 <= 65536 for o in offs), name
        assert all(o % SIZE[kind] == 0 for o in offs), name
        pat = torch.tensor(offs, dtype=torch.int32, device="cuda")
        ms = min(lib.lds_probe(kind, ctypes.c_void_p(pat.data_ptr()), ctypes.c_void_p(out.data_ptr()), blocks, iters)
                 for _ in range(3))
        if ms <= 0:
            raise RuntimeError("lds_probe failed")
        ns = ms * 1e6 / (blocks * 8 * iters * 8 / cus)   # per wave read instruction per CU
        base.setdefault(kind, ns)
        rows.append({"read": ["b128", "b64", "tr8_b64"][kind], "pattern": name, "ns_per_read_per_cu": round(ns, 3),
                     "vs_linear": round(ns / base[kind], 2)})
        print(f"{rows[-1]['read']:8s} {name:78s} {ns:6.2f} ns  x{ns / base[kind]:.2f}", flush=True)
    print(json.dumps({"cus": cus, "patterns": rows}))


if __name__ == "__main__":
    main()
