"""Writes tests/golden/requant_nvfp4_full.txt: for each of the 256 NVFP4 expert tensors
[2048, 6144] of the load-time re-quantizer workload, the SHA-256 of the canonical codes and of
the UE8M0 scale bytes that the exact oracle (oracle.requant, integer arithmetic) produces.

The GPU test compares the library's output with these digests byte for byte over the whole
workload, so the oracle's 0.9 GB of output need not be stored. Inputs come from
workloads.nvfp4_tensor (seeded); nothing here calls the library.

Run from the repository root:  python tests/golden/make_requant_digests.py   (a few CPU-minutes)
"""
import hashlib
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import requant  # noqa: E402
import workloads  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "requant_nvfp4_full.txt")


def main():
    c = workloads.REQUANT
    lines = ["# nvfp4_to_w2 over the NVFP4 re-quantizer workload: n=256 tensors of [2048, 6144],",
             "# inputs workloads.nvfp4_tensor(i); codes [2048, 1536] and scale bytes [2048, 192] per tensor",
             "# from the exact oracle (oracle.requant.requant_rows). Written by make_requant_digests.py.",
             "# tensor sha256(codes) sha256(scales)"]
    t0 = time.time()
    for i in range(c["n"]):
        a, b, s = workloads.nvfp4_tensor(i)
        codes, scales = requant.requant_rows(a, b, s)
        lines.append(f"{i} {hashlib.sha256(codes.tobytes()).hexdigest()} {hashlib.sha256(scales.tobytes()).hexdigest()}")
        if i % 32 == 31:
            print(f"{i + 1} tensors, {time.time() - t0:.0f} s", flush=True)
    with open(OUT, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("wrote", OUT)


if __name__ == "__main__":
    main()
