"""emu_scaled_mm_noalloc, the entry point for callers that cannot allocate:
bit for bit the same outputs as emu_scaled_mm (which uses a caller-given
workspace), on plans that use the scratch (split partials, stored slow-mode
chunk results, infinity lists) and on a plan whose chunk results do not fit
it, two calls in a row with the second smaller than the first (the scratch
keeps the first call's contents); and the host-side refusal of split
partials beyond the scratch."""
import ctypes

import numpy as np
import pytest
import torch

from bit_exact_fp8_amd import api
from bit_exact_fp8_amd.inputs import FP8_DTYPES, OUT_DTYPES, Workload, make_operands


def test_partials_beyond_the_scratch_are_refused():
    """split_S * M * N * 4 bytes above the scratch: EMU_ERR_WORKSPACE on the
    host, before any device call (fake, never dereferenced addresses)."""
    lib = api._lib()
    M, N, K, S = 2048, 2048, 1024, 8
    assert S * M * N * 4 > api.NOALLOC_SCRATCH_BYTES
    st = lib.emu_scaled_mm_noalloc(16, 0, K, 16, 0, K, M, N, K, 16, 16, None, 16, 0, N, 1, S, 0, None, None)
    assert st == api.EMU_ERR_WORKSPACE
    assert b"scratch" in lib.emu_last_error_message()
    # just inside: 4 splits of 2048 x 2048 are exactly 64 MiB
    assert 4 * M * N * 4 == api.NOALLOC_SCRATCH_BYTES
    st = lib.emu_scaled_mm_noalloc(16, 0, K, 16, 0, K, M, N, K, 16, 16, None, 16, 0, N, 1, 4, 0, None,
                                   ctypes.pointer(api.PlanOptions(len(api.TILE_CONFIGS), -1)))
    assert st == api.EMU_ERR_INVALID_ARG      # refused for the plan options, not the size


def _bits(t):
    t = t.cpu()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    if t.element_size() == 1:
        return t.view(torch.uint8).numpy()
    return t.view(torch.int16).numpy()


def _pair(dev, wl, seed, profile="hopper", defer=None, infinities=False):
    """(noalloc output, workspace output) of one problem, on one stream."""
    x, w = make_operands(wl, seed)
    if infinities:
        gen = torch.Generator().manual_seed(seed + 2000)
        hit = torch.rand(w.shape, generator=gen) < 2e-3
        w[hit] = 0x7C | (torch.randint(0, 2, w.shape, generator=gen, dtype=torch.uint8) << 7)[hit]
        w[1, :] = 0x7C
    xd = x.to(dev).view(FP8_DTYPES[wl.xfmt])
    wd = w.to(dev).view(FP8_DTYPES[wl.wfmt])
    sx = torch.tensor([wl.scale_x], dtype=torch.float32, device=dev)
    sw = torch.tensor([wl.scale_w], dtype=torch.float32, device=dev)
    out = torch.full((wl.M, wl.N), float("nan"), dtype=OUT_DTYPES[wl.out], device=dev)
    print(f"[gpu] noalloc {wl.name} {wl.M}x{wl.N}x{wl.K} S={wl.split_S} fast={wl.fast} {profile} "
          f"defer={defer}", flush=True)
    api.scaled_mm_noalloc(xd, wd.t(), sx, sw, out, use_fast_accum=wl.fast, split_S=wl.split_S, profile=profile,
                          defer=defer)
    ref = api.scaled_mm(xd, wd.t(), sx, sw, out_dtype=OUT_DTYPES[wl.out], use_fast_accum=wl.fast,
                        split_S=wl.split_S, profile=profile, defer=defer)
    torch.cuda.synchronize(dev)
    return _bits(out), _bits(ref)


CASES = [
    # split partials in the scratch (8 and 3 splits)
    (Workload("splitk", 16, 256, 65536, x_sigma=8.0, w_sigma=8.0, split_S=8),
     Workload("splitk_small", 16, 128, 8192, x_sigma=8.0, w_sigma=8.0, split_S=3), "hopper", None, False),
    # stored slow-mode chunk results (small output grids), ada pairwise in splits
    (Workload("slow", 64, 512, 4096, fast=False, out="fp32", zero_frac=0.05, subnormal_frac=0.05),
     Workload("slow_small", 32, 256, 1024, fast=False, out="fp32", split_S=3), "ada-pairwise", None, False),
    # chunk results of 128 MiB do not fit: planned without them, same bits
    (Workload("slow_big", 256, 4096, 4096, fast=False, out="fp32", zero_frac=0.05, subnormal_frac=0.05),
     Workload("slow_mid", 64, 1024, 2048, fast=False, out="fp32"), "hopper", None, False),
    # infinity lists in the scratch (deferred plan forced), e5m2 w
    (Workload("inf", 256, 512, 1024, wfmt="e5m2", w_sigma=1000.0),
     Workload("inf_small", 64, 256, 512, wfmt="e5m2", w_sigma=1000.0), "hopper", "on", True),
]


@pytest.mark.gpu
@pytest.mark.parametrize("first,second,profile,defer,infinities", CASES)
def test_noalloc_matches_the_workspace_entry_point(first, second, profile, defer, infinities):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    for i, wl in enumerate((first, second)):
        got, want = _pair(dev, wl, 11 + i, profile, defer, infinities)
        bad = np.argwhere(got != want)
        assert len(bad) == 0, (wl.name, len(bad), bad[:3].tolist())
