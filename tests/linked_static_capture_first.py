"""Child process of tests/test_zz_no_alloc.py: the first
pc_twoshot_linked_static call of a fresh process is made inside a HIP graph
capture (so the static workspace's address is looked up during capture).
Every replay must equal the oracle, report no abandoned wait, and advance
the library's call counters (checked through the results staying exact
over replays).  Prints OK on success."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import oracle  # noqa: E402
from collective_datapath_amd import binding as B  # noqa: E402
from collective_datapath_amd import synth  # noqa: E402


def main():
    n, k = 8, 8 * 65536
    xs = [synth.normal_bf16(2400, 0, r, k) for r in range(n)]
    ins = [torch.from_numpy(x.view(np.int16)).to("cuda:0") for x in xs]
    outs = [torch.empty(k, dtype=torch.int16, device="cuda:0") for _ in range(n)]
    gave_up = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            B.pc_twoshot_linked_static(ins, outs, k, gave_up)
    torch.cuda.synchronize()
    want = oracle.reduce(xs)
    for rep in range(3):
        for o in outs:
            o.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o in outs:
            assert np.array_equal(o.cpu().numpy().view(np.uint16), want), rep
        assert int(gave_up.item()) == 0, rep
    print("OK", flush=True)


if __name__ == "__main__":
    main()
