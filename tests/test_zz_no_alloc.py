"""The allocation-free SwiGLU entry point (GPU): same result as the workspace entry point.

fuse_swiglu_auto_noalloc keeps the split-K partials in the library's fixed per-device array.  It
is called through the C ABI twice in a row -- a shape whose plan takes 24 MiB of the 64 MiB array,
then a smaller one that reuses it -- and each result is compared with fuse_swiglu_auto (caller
workspace) on the same inputs, under the bf16 rule and bit for bit (same plan, same kernels,
same summation order).  A shape that needs no split, a plan too large for the array (refused,
output untouched) and a stream other than the current one are covered too.
"""
import numpy as np
import pytest
import torch

import oracle
from memory_bound_amd import api, synth
from oracle.tolerance import assert_close

pytestmark = pytest.mark.gpu

SCRATCH = 64 << 20


def _case(M, N, K, seed):
    d = synth.swiglu_inputs(M, N, K, "bf16", seed=seed)
    return d, d["a"].cuda(), d["b1"].cuda(), d["b2"].cuda()


def test_noalloc_matches_workspace_entry_point_two_calls():
    for M, N, K, seed in ((1024, 1024, 1536, 31), (256, 512, 1536, 32)):
        splits = api.fuse_auto_splits(api.FUSE_OP_SWIGLU, M, N, K)
        need = api.load().fuse_auto_workspace_bytes(api.FUSE_OP_SWIGLU, M, N, K, api.FUSE_BF16)
        print(f"\n[gpu-case] swiglu noalloc {M}x{N}x{K}: {splits} splits, {need} bytes of partials", flush=True)
        assert splits > 1 and 0 < need <= SCRATCH
        d, a, b1, b2 = _case(M, N, K, seed)
        want = api.fuse_swiglu_auto(a, b1, b2)
        got = api.fuse_swiglu_auto_noalloc(a, b1, b2)
        torch.cuda.synchronize()
        assert_close(got, want.cpu().double().numpy(), "bf16", f"noalloc vs workspace {M}x{N}x{K}")
        assert torch.equal(got, want)
        rows = torch.arange(0, M, 37)
        assert_close(got[rows.cuda()], oracle.swiglu(d["a"][rows], d["b1"], d["b2"]), "bf16",
                     f"noalloc vs oracle {M}x{N}x{K}")


def test_noalloc_without_split_side_stream_and_refusal(monkeypatch):
    print("\n[gpu-case] swiglu noalloc: single-kernel plan, side stream, oversized plan", flush=True)
    d, a, b1, b2 = _case(2048, 1024, 64, 33)  # 64 tiles: the plan does not split
    assert api.fuse_auto_splits(api.FUSE_OP_SWIGLU, 2048, 1024, 64) == 1
    assert torch.equal(api.fuse_swiglu_auto_noalloc(a, b1, b2), api.fuse_swiglu_auto(a, b1, b2))
    d, a, b1, b2 = _case(256, 512, 1536, 34)
    want = api.fuse_swiglu_auto(a, b1, b2)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out = torch.empty_like(want)
    api.fuse_swiglu_auto_noalloc(a, b1, b2, out=out, stream=side)
    side.synchronize()
    assert torch.equal(out, want)
    # 48 splits of a 1024 x 1024 output would need 384 MiB of partials: refused, nothing launched
    monkeypatch.setenv("FUSE_SPLITK", "48")
    d, a, b1, b2 = _case(1024, 1024, 1536, 35)
    out = torch.full((1024, 1024), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(api.FuseError) as e:
        api.fuse_swiglu_auto_noalloc(a, b1, b2, out=out)
    assert e.value.status == 7
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
