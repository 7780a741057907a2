"""Small workloads for hardware-counter runs under rocprofv3.

  python3 profile_drv.py attn [workload] [reps]
      forward + backward of a synthetic workload through the C ABI, `reps` times
  python3 profile_drv.py mul [workload] [layout] [reps]
      triangle multiplication core, both directions, forward + backward, `reps` times
  python3 profile_drv.py copy [mib] [reps]
      a plain device-to-device copy of `mib` MiB (torch's copy kernel), used to
      calibrate FETCH_SIZE / WRITE_SIZE against a known byte count
"""
from __future__ import annotations

import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _attn(name: str, reps: int):
    import numpy as np
    import torch

    import triangle_attention_amd as ta
    from tri_synth import WORKLOADS, workload_inputs

    w = WORKLOADS[name]
    inp = workload_inputs(w)

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v, bias, dO = (dev(inp[n]) for n in ("q", "k", "v", "bias", "dO"))
    m = None if inp["key_mask"] is None else torch.from_numpy(inp["key_mask"]).cuda()
    for _ in range(reps):
        o, lse, res = ta.forward(q, k, v, bias, m)
        ta.backward(q, k, v, bias, m, o, lse, res, dO)
    torch.cuda.synchronize()
    print(f"attn {name} x{reps} done", flush=True)


def _mul(name: str, layout: str, reps: int):
    import numpy as np
    import torch

    import triangle_attention_amd as ta
    from tri_synth import TRIMUL_WORKLOADS, make_pair_inputs

    w = TRIMUL_WORKLOADS[name]
    B, N, C = w["B"], w["N"], w["C"]
    inp = make_pair_inputs(B, N, C, seed=w["seed"])

    def dev(bits):
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
        return t.permute(0, 3, 1, 2).contiguous() if layout == "channels_first" else t

    a, b, dx = dev(inp["a"]), dev(inp["b"]), dev(inp["dx"])
    x, da, db = torch.empty_like(a), torch.empty_like(a), torch.empty_like(a)
    lay = ta.TRI_MUL_LAYOUTS[layout]
    nws = ta.tri_mul_workspace_bytes(lay, B, N, C)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
    for _ in range(reps):
        for d in (0, 1):
            assert ta.tri_mul_fwd(d, lay, B, N, C, a, b, x, ws, nws) == 0
            assert ta.tri_mul_bwd(d, lay, B, N, C, a, b, dx, da, db, ws, nws) == 0
    torch.cuda.synchronize()
    print(f"mul {name} {layout} x{reps} done", flush=True)


def _copy(mib: int, reps: int):
    import torch

    a = torch.zeros(mib << 18, dtype=torch.float32, device="cuda")  # mib MiB
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"copy {mib} MiB x{reps} done", flush=True)


def main(argv):
    what = argv[1] if len(argv) > 1 else "attn"
    if what == "copy":
        _copy(int(argv[2]) if len(argv) > 2 else 256, int(argv[3]) if len(argv) > 3 else 3)
    elif what == "mul":
        _mul(argv[2] if len(argv) > 2 else "trimul_n768_c128", argv[3] if len(argv) > 3 else "channels_first",
             int(argv[4]) if len(argv) > 4 else 2)
    else:
        _attn(argv[2] if len(argv) > 2 else "n768_h4_d32", int(argv[3]) if len(argv) > 3 else 3)


if __name__ == "__main__":
    main(sys.argv)
