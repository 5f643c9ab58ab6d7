"""Device copies of known size, for calibrating rocprofv3's HBM byte counters.

Measurement only: for 256 MiB, 1 GiB and 2 GiB per side, three blit copies
(torch's copy_) and three elementwise kernels (torch.add), each reading and
writing that many bytes, so that a --pmc pass of FETCH_SIZE or WRITE_SIZE
over this script shows what the counter reads for a known byte count.

    rocprofv3 --pmc FETCH_SIZE -f csv -d OUT -o fetch -- python3 -m dropless_moe_expert_amd.counter_calibration
"""
import torch


def main() -> None:
    dev = torch.device("cuda")
    for mib in (256, 1024, 2048):
        n = mib << 19   # int16 elements: mib MiB per side
        src = torch.ones(n, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        for _ in range(3):
            torch.add(src, 1, out=dst)
        torch.cuda.synchronize()
        print("copied", mib, "MiB per side", flush=True)
        del src, dst


if __name__ == "__main__":
    main()
