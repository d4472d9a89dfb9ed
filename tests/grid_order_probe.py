"""Run paged decodes of several kernel shapes in the order given on the command line, in
one fresh process, and print each shape's balanced-split grid as JSON.

Used by tests/test_gpu_grid.py: the grid of a kernel must not depend on which kernel the
process launched first. Each shape is launched for real (a small seeded workload) before
its grid is read back with pkv_decode_split_workgroups.

    python -m tests.grid_order_probe f32-d128-g8 bf16-d64-g1
"""

from __future__ import annotations

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# name -> (dtype, n_heads, n_kv_heads, d_head)
SHAPES = {
    "f32-d128-g8": ("f32", 64, 8, 128),
    "bf16-d64-g1": ("bf16", 8, 8, 64),
    "bf16-d128-g4": ("bf16", 32, 8, 128),
    "f16-d128-g1": ("f16", 32, 32, 128),
}


def main(order):
    import torch

    from paged_kv_cache_26_amd import pkv
    from paged_kv_cache_26_amd import workload as wlm

    pkv.load_library()
    grids = {}
    for name in order:
        dtype, H, Hkv, d = SHAPES[name]
        spec = wlm.Spec(f"grid-{name}", dtype, 3, H, Hkv, d, "gqa", lengths=(700, 1300, 90))
        wl = wlm.make_workload(spec, seed=5)
        t = wlm.to_torch(wl, "cuda:0")
        out = torch.empty_like(t["q"])
        print(f"decode {name}", file=sys.stderr, flush=True)
        pkv.pkv_paged_decode_attention(out, t["q"], t["k_pool"], t["v_pool"], t["block_tables"],
                                       t["context_lens"], wl.max_context_len, wl.scale)
        torch.cuda.synchronize()
        grids[name] = pkv.pkv_decode_split_workgroups(H, Hkv, d, 1, wlm.DTYPE_CODE[dtype])
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    print(json.dumps({"order": list(order), "grids": grids, "compute_units": cus}), flush=True)


if __name__ == "__main__":
    main(sys.argv[1:])
