"""Child process of tests/test_parity_gpu.py: the first pc_twoshot_linked
call of a fresh process is made inside a HIP graph capture (so the launch
set-up runs during capture).  Every replay must equal the oracle and
advance the device-side call counter by one.  Prints OK on success."""
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
    xs = [synth.normal_bf16(1800, 0, r, k) for r in range(n)]
    ins = [torch.from_numpy(x.view(np.int16)).to("cuda:0") for x in xs]
    outs = [torch.empty(k, dtype=torch.int16, device="cuda:0") for _ in range(n)]
    ws = torch.zeros(B.pc_twoshot_linked_workspace_bytes(n, k) // 8, dtype=torch.int64, device="cuda:0")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            B.pc_twoshot_linked(ins, outs, k, ws)
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
        w = ws.cpu().numpy().view(np.uint64)
        assert np.all(w[:B.PC_LINKED_GROUPS] == rep + 1) and w[B.PC_LINKED_STATUS_WORD] == 0, rep
    print("OK", flush=True)


if __name__ == "__main__":
    main()
