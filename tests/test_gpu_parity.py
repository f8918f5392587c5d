"""GPU parity: the HIP library, called through its C ABI, against the CPU
oracle, bit for bit (tolerance 0 ULP), on seeded inputs.

Covers the five workloads (the 8192^3 one at full size on sampled outputs),
every FP8 code pair, an edge-case sweep (ragged M, K not a multiple of 32 or
128, K = 0, more splits than k-tiles, NaN / Inf / zero / subnormal codes,
non-power-of-two scales, every output type, accumulator output), and the
invariants the pages state (out= buffer ignored, determinism across streams,
padding rows independent)."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from bit_exact_fp8_amd import api
from bit_exact_fp8_amd.inputs import (FP8_DTYPES, OUT_DTYPES, WORKLOADS, Workload, inject,
                                      make_operands, random_codes, scale_bits)

pytestmark = pytest.mark.gpu
THREADS = min(16, os.cpu_count() or 1)


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def bits_of(t: torch.Tensor) -> np.ndarray:
    t = t.cpu()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    if t.element_size() == 1:
        return t.view(torch.uint8).numpy().astype(np.uint32)
    return t.view(torch.int16).numpy().view(np.uint16).astype(np.uint32)


def gpu_run(dev, x, xfmt, w, wfmt, sx, sw, out="bf16", fast=True, S=1, stream=None, prefill=None,
            profile="hopper", sr=None, tile=None, defer=None):
    xd = x.to(dev).view(FP8_DTYPES[xfmt])
    wd = w.to(dev).view(FP8_DTYPES[wfmt])
    sxd = torch.tensor([sx], dtype=torch.float32, device=dev)
    swd = torch.tensor([sw], dtype=torch.float32, device=dev)
    srd = None if sr is None else torch.tensor([sr], dtype=torch.float32, device=dev)
    o = None
    if prefill is not None:
        o = torch.empty((x.shape[0], w.shape[0]), dtype=OUT_DTYPES[out], device=dev)
        o.view(torch.uint8).fill_(prefill)
    with torch.cuda.stream(stream or torch.cuda.current_stream(dev)):
        y = api.scaled_mm(xd, wd.t(), sxd, swd, out_dtype=OUT_DTYPES[out], use_fast_accum=fast,
                          split_S=S, profile=profile, out=o, scale_result=srd, tile=tile, defer=defer)
        acc = api.accumulate(xd, wd, use_fast_accum=fast, split_S=S, profile=profile, tile=tile, defer=defer)
    torch.cuda.synchronize(dev)
    return bits_of(y), bits_of(acc)


def oracle_run(orc, x, xfmt, w, wfmt, sx, sw, out="bf16", fast=True, S=1, profile="hopper", sr=None):
    return orc.scaled_mm(x.numpy(), xfmt, w.numpy(), wfmt, scale_bits(sx), scale_bits(sw), out, fast, S,
                         profile=profile, threads=THREADS,
                         sr_bits=oracle.ONE if sr is None else scale_bits(sr))


def assert_same(got, want, what):
    bad = got != want
    if bad.any():
        idx = np.argwhere(bad)
        i = tuple(idx[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} differ; first at {i}: "
                             f"gpu {int(got[i]):#x} oracle {int(want[i]):#x}")


def check(dev, orc, x, xfmt, w, wfmt, sx, sw, out, fast, S, what, profile="hopper", sr=None, tile=None,
          defer=None):
    note(f"[gpu] {what}: M={x.shape[0]} N={w.shape[0]} K={x.shape[1]} {xfmt}x{wfmt} "
         f"fast={fast} S={S} out={out} profile={profile} scale_result={sr} tile={tile} defer={defer}")
    y, acc = gpu_run(dev, x, xfmt, w, wfmt, sx, sw, out, fast, S, profile=profile, sr=sr, tile=tile, defer=defer)
    acc_o, y_o = oracle_run(orc, x, xfmt, w, wfmt, sx, sw, out, fast, S, profile=profile, sr=sr)
    assert_same(acc, acc_o, what + " accumulator")
    assert_same(y, y_o, what + " output")


# ---- the workloads -------------------------------------------------------------
@pytest.mark.parametrize("name,seed", [
    ("tiny", 0), ("tiny", 1), ("tiny", 2),
    ("proj_64x5760x1920", 0), ("proj_64x5760x1920", 1), ("proj_64x5760x1920", 2),
    ("slow_256x4096x4096", 0), ("slow_256x4096x4096", 1), ("slow_256x4096x4096", 2),
    ("splitk_16x256x65536_s8", 0), ("splitk_16x256x65536_s8", 1), ("splitk_16x256x65536_s8", 2),
    ("proj_2048x5760x1920", 0),
])
def test_workload_full(dev, orc, name, seed):
    wl = WORKLOADS[name]
    x, w = make_operands(wl, seed)
    check(dev, orc, x, wl.xfmt, w, wl.wfmt, wl.scale_x, wl.scale_w, wl.out, wl.fast, wl.split_S,
          f"{name} seed {seed}")


def test_mixed_8192_sampled(dev, orc):
    """Full-size 8192^3 e4m3 x e5m2 run, compared on sampled outputs that the
    oracle computes one by one: random points plus the corners and tile
    boundaries."""
    wl = WORKLOADS["mixed_8192"]
    x, w = make_operands(wl, 0)
    note("[gpu] mixed_8192 seed 0: full-size run")
    y, acc = gpu_run(dev, x, wl.xfmt, w, wl.wfmt, wl.scale_x, wl.scale_w, wl.out, wl.fast, wl.split_S)
    rng = np.random.default_rng(0)
    ms = list(rng.integers(0, wl.M, 3000)) + [0, 0, wl.M - 1, wl.M - 1, 63, 64, 127, 128, 4095, 4096]
    ns = list(rng.integers(0, wl.N, 3000)) + [0, wl.N - 1, 0, wl.N - 1, 127, 128, 63, 64, 4096, 4095]
    ms, ns = np.array(ms, dtype=np.int64), np.array(ns, dtype=np.int64)
    acc_o, y_o = orc.points(x.numpy(), wl.xfmt, w.numpy(), wl.wfmt, ms, ns, scale_bits(wl.scale_x),
                            scale_bits(wl.scale_w), wl.out, wl.fast, wl.split_S)
    assert_same(acc[ms, ns], acc_o, "mixed_8192 accumulator")
    assert_same(y[ms, ns], y_o, "mixed_8192 output")
    # a 1024 x 1024 window of whole output rows and columns: rows 512..1535
    # cross the boundary of two groups of 8 tile-rows (512) and of two XCDs'
    # shares of the tile order (1024); columns 3584..4607 cross the middle
    m0, n0, side = 512, 3584, 1024
    note("[gpu] mixed_8192 seed 0: 1024 x 1024 window against the oracle")
    acc_w, y_w = orc.scaled_mm(x.numpy()[m0:m0 + side], wl.xfmt, w.numpy()[n0:n0 + side], wl.wfmt,
                               scale_bits(wl.scale_x), scale_bits(wl.scale_w), wl.out, wl.fast, wl.split_S,
                               threads=THREADS)
    assert_same(acc[m0:m0 + side, n0:n0 + side], acc_w, "mixed_8192 window accumulator")
    assert_same(y[m0:m0 + side, n0:n0 + side], y_w, "mixed_8192 window output")


# ---- every code pair ------------------------------------------------------------
# tiles: automatic; the matrix-core maxima of 4-row thread tiles (6: 64x64,
# 7: 64x128, 9: 16x64) and of 2-row ones with binary16 values (11: 32x32,
# 12: 32x16); binary16 values with 4 lanes per output (8: 16x8)
CODE_PAIR_TILES = [None, 6, 7, 9, 8, 11, 12]


@pytest.mark.parametrize("tile", CODE_PAIR_TILES)
@pytest.mark.parametrize("xfmt,wfmt", [("e4m3fn", "e4m3fn"), ("e4m3fn", "e5m2"), ("e5m2", "e4m3fn")])
def test_every_code_pair(dev, orc, xfmt, wfmt, tile):
    """All 65,536 code pairs, one nonzero product per output (validation
    page, claims table: every pair of FP8 codes through the epilogue), with
    the automatic tile (one lane per output, packed-maximum exponents), the
    tiles whose block maxima come from the matrix cores, and the tiles that
    keep binary16 values (truncating with the mixed-precision FMA)."""
    K = 16
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    x = torch.zeros((256, K), dtype=torch.uint8)
    w = torch.zeros((256, K), dtype=torch.uint8)
    x[:, 3] = codes
    w[:, 3] = codes
    for out in ("bf16", "fp16", "fp32"):
        check(dev, orc, x, xfmt, w, wfmt, 1 / 3, 0.1, out, True, 1, f"code pairs {xfmt}x{wfmt}", tile=tile)
    for out, sr in (("e4m3fn", None), ("e4m3fn", 9.6), ("e5m2", -0.37)):
        if out == "e5m2" and xfmt == wfmt == "e4m3fn":
            continue  # rejected combination
        check(dev, orc, x, xfmt, w, wfmt, 1 / 3, 0.1, out, True, 1, f"code pairs {xfmt}x{wfmt}", sr=sr,
              tile=tile)


# ---- adversarial blocks for the matrix-core exponent maximum ------------------------------
# Quarter-block (8-code) patterns of one operand row: the largest finite
# codes (field exponent 8 for e4m3fn, 15 for e5m2), subnormal codes (field
# exponent at emin), a single subnormal among zeros, zeros, and random
# finite codes; each with random signs.
QUARTER_KINDS = ("max", "subnormal", "lone_subnormal", "zero", "random")


def _adversarial_rows(rows, K, fmt, rng):
    top = 0x7E if fmt == "e4m3fn" else 0x7B
    nsub = 7 if fmt == "e4m3fn" else 3
    out = np.zeros((rows, K), dtype=np.uint8)
    for r in range(rows):
        for q0 in range(0, K, 8):
            kind = QUARTER_KINDS[rng.integers(0, len(QUARTER_KINDS))]
            sign = (rng.integers(0, 2, 8) << 7).astype(np.uint8)
            if kind == "max":
                q = np.full(8, top, dtype=np.uint8)
            elif kind == "subnormal":
                q = rng.integers(1, nsub + 1, 8).astype(np.uint8)
            elif kind == "lone_subnormal":
                q = np.zeros(8, dtype=np.uint8)
                q[rng.integers(0, 8)] = rng.integers(1, nsub + 1)
            elif kind == "zero":
                q = np.zeros(8, dtype=np.uint8)
            else:
                q = rng.integers(0, 256, 8).astype(np.uint8)
                special = (q & 0x7F) == 0x7F if fmt == "e4m3fn" else (q & 0x7C) == 0x7C
                q[special] &= 0x70
            out[r, q0:q0 + 8] = q | sign
        # a few whole blocks of zeros: their E comes from the incoming c alone
        for b in rng.choice(K // 32, max(1, K // 128), replace=False):
            out[r, 32 * b:32 * b + 32] &= 0x80
    return torch.from_numpy(out)


@pytest.mark.parametrize("tile", [None, 6, 7, 9, 11, 12])
@pytest.mark.parametrize("xfmt,wfmt", [("e4m3fn", "e5m2"), ("e5m2", "e4m3fn"), ("e4m3fn", "e4m3fn")])
def test_matrix_core_maximum_adversarial(dev, orc, xfmt, wfmt, tile):
    """Blocks built to hit the edges of the matrix-core block maximum: eight
    equal products at the largest field-exponent sum in a quarter (g = 23
    for e4m3fn x e5m2: the sum of the quarter's powers reaches its upper
    bound), eight subnormal x subnormal products (g = -20, the smallest), a
    lone smallest product among zeros, all-zero quarters, and whole blocks
    of zero products after nonzero ones, whose exponent comes from the
    incoming accumulator alone; also mixed with random codes.  Fast and
    slow, unsplit and split, 32- and 16-product blocks, every output row
    and column against the oracle."""
    fmt_id = {"e4m3fn": 1, "e5m2": 2}
    rng = np.random.default_rng(10 * fmt_id[xfmt] + fmt_id[wfmt] + 100 * (tile or 0))
    M, N, K = 130, 144, 1024
    x = _adversarial_rows(M, K, xfmt, rng)
    w = _adversarial_rows(N, K, wfmt, rng)
    for fast, S, profile in ((True, 1, "hopper"), (False, 1, "hopper"), (True, 3, "ada-pairwise"),
                             (False, 2, "ada-serial")):
        check(dev, orc, x, xfmt, w, wfmt, 0.1, 1 / 3, "fp32", fast, S,
              f"adversarial maxima {xfmt}x{wfmt} tile {tile}", profile=profile, tile=tile)


def test_matrix_core_maximum_extreme_blocks(dev, orc):
    """Whole 32-product blocks of the two extremes on every matrix-core tile:
    32 products at g = 23 (all four quarters at the upper bound of the power
    sum), 32 subnormal products at g = -20, and alternating blocks of the
    two, so that a block of the smallest products follows an accumulator
    2^43 times larger (swamped to nothing) and vice versa."""
    M, N, K = 64, 128, 512
    rng = np.random.default_rng(9)
    x = np.zeros((M, K), dtype=np.uint8)
    w = np.zeros((N, K), dtype=np.uint8)
    for b in range(K // 32):
        big = (b % 2 == 0) if b < 8 else (b % 3 == 0)
        x[:, 32 * b:32 * b + 32] = 0x7E if big else rng.integers(1, 8, (M, 32))
        w[:, 32 * b:32 * b + 32] = 0x7B if big else rng.integers(1, 4, (N, 32))
    x |= (rng.integers(0, 2, (M, K)) << 7).astype(np.uint8)
    w |= (rng.integers(0, 2, (N, K)) << 7).astype(np.uint8)
    x, w = torch.from_numpy(x), torch.from_numpy(w)
    for tile in (None, 6, 7, 9, 11, 12):
        for fast in (True, False):
            check(dev, orc, x, "e4m3fn", w, "e5m2", 1.0, 1.0, "fp32", fast, 1,
                  f"extreme blocks tile {tile} fast={fast}", tile=tile)


# ---- edge-case sweep --------------------------------------------------------------
def _edge_case(seed):
    rng = np.random.default_rng(seed)
    gen = torch.Generator().manual_seed(seed)
    xfmt, wfmt = [("e4m3fn", "e4m3fn"), ("e4m3fn", "e5m2"), ("e5m2", "e4m3fn")][seed % 3]
    M = int(rng.choice([1, 3, 16, 17, 33, 64, 70, 129]))
    N = int(rng.choice([16, 32, 48, 80, 144, 272]))
    K = int(rng.choice([0, 16, 32, 48, 112, 128, 144, 400, 1040, 2064]))
    fast = bool(rng.integers(0, 2))
    S = int(rng.choice([1, 1, 2, 3, 5, 17]))
    out = str(rng.choice(["bf16", "fp16", "fp32"]))
    x = random_codes((M, K), xfmt, gen, finite=True)
    w = random_codes((N, K), wfmt, gen, finite=True)
    x = inject(x, xfmt, 0.2, 0.1, gen)
    w = inject(w, wfmt, 0.2, 0.1, gen)
    if seed % 4 == 0 and K:  # a few NaN / Inf codes
        for _ in range(3):
            if xfmt == "e5m2":
                x[rng.integers(0, M), rng.integers(0, K)] = int(rng.choice([0x7C, 0xFC, 0x7E]))
            else:
                x[rng.integers(0, M), rng.integers(0, K)] = int(rng.choice([0x7F, 0xFF]))
            if wfmt == "e5m2":
                w[rng.integers(0, N), rng.integers(0, K)] = int(rng.choice([0x7C, 0xFC, 0x7D]))
            else:
                w[rng.integers(0, N), rng.integers(0, K)] = 0x7F
    sx = float(rng.choice([1 / 64, 0.1, -1 / 3, 3.0e-30, 2.0 ** -140, 65504.0]))
    sw = float(rng.choice([1 / 32, 1 / 3, 7.0, -0.3]))
    return x, xfmt, w, wfmt, sx, sw, out, fast, S


@pytest.mark.parametrize("seed", range(40))
def test_edge_cases(dev, orc, seed):
    x, xfmt, w, wfmt, sx, sw, out, fast, S = _edge_case(seed)
    check(dev, orc, x, xfmt, w, wfmt, sx, sw, out, fast, S, f"edge case {seed}")


@pytest.mark.parametrize("fast,S", [(True, 1), (False, 1), (True, 4), (False, 3)])
def test_large_tiles(dev, orc, fast, S):
    """Sizes that select the 64x128 and 32x64 workgroup tiles, with ragged edges."""
    wl = Workload("t", 1040, 4112, 160, zero_frac=0.05, subnormal_frac=0.05)
    x, w = make_operands(wl, 3)
    check(dev, orc, x, "e4m3fn", w, "e4m3fn", 0.1, 1 / 3, "bf16", fast, S, f"large tiles fast={fast} S={S}")


@pytest.mark.parametrize("profile", ["hopper", "ada-pairwise"])
@pytest.mark.parametrize("cfg", range(len(api.TILE_CONFIGS)))
@pytest.mark.parametrize("shape", [(1, 16, 48), (37, 80, 400), (70, 144, 1040)])
def test_every_tile_config(dev, orc, cfg, shape, profile):
    """Every tile configuration (including 2 and 4 lanes per output) gives the
    oracle's bits, fast and slow, unsplit and split, on ragged shapes, with
    32-product blocks (hopper) and 16-product blocks over round-robin splits
    (ada)."""
    M, N, K = shape
    gen = torch.Generator().manual_seed(100 + cfg)
    x = inject(random_codes((M, K), "e4m3fn", gen), "e4m3fn", 0.1, 0.05, gen)
    w = inject(random_codes((N, K), "e5m2", gen), "e5m2", 0.1, 0.05, gen)
    for fast, S in ((True, 1), (False, 1), (True, 3), (False, 2)):
        check(dev, orc, x, "e4m3fn", w, "e5m2", 0.1, 1 / 3, "bf16", fast, S,
              f"tile {api.TILE_CONFIGS[cfg]} {shape}", profile=profile, tile=cfg)


@pytest.mark.parametrize("shape,forced", [
    ((64, 8192, 288), -1),   # 2 x 256 = 512 workgroups of the 32x32 tile: its 4-stage form
    ((96, 5472, 224), -1),   # 3 x 171 = 513 workgroups: its 2-stage form
    ((96, 5472, 224), 10),   # the 4-stage form forced on that grid
    ((80, 4000, 400), -1),   # ragged rows, columns and K (4-stage form, 375 workgroups)
])
def test_stage_forms_of_the_32x32_tile(dev, orc, shape, forced):
    """The host's choice between the 32x32 tile's 2- and 4-stage forms (at
    most 512 workgroups take the 4-stage one) gives the oracle's bits on both
    sides of the boundary, fast and slow, unsplit and split."""
    M, N, K = shape
    gen = torch.Generator().manual_seed(M + N + K)
    x = inject(random_codes((M, K), "e4m3fn", gen), "e4m3fn", 0.05, 0.05, gen)
    w = inject(random_codes((N, K), "e4m3fn", gen), "e4m3fn", 0.05, 0.05, gen)
    for fast, S in ((True, 1), (False, 1)):
        check(dev, orc, x, "e4m3fn", w, "e4m3fn", 0.1, 1 / 3, "bf16", fast, S,
              f"32x32 stage forms {shape} tile {forced}", tile=forced)


@pytest.mark.parametrize("profile", ["hopper", "ada-pairwise"])
def test_16x8_tile_long_klists(dev, orc, profile):
    """The 16x8 tile with 4 lanes per output stages 32 K-blocks per barrier
    on long k-lists of 32-product blocks, 16 on those of 16-product blocks
    and on shorter ones, and 8 on short ones: a ragged K whose last round is
    partial (2960 = 92.5 stages of 32; 32 per round unsplit and over 3
    splits, 16 over 2), fast and slow, unsplit and split into k-lists of
    different lengths, NaN / Inf codes in one row, and chains from incoming
    accumulators (at most 16 per round), against the oracle."""
    M, N, K = 17, 48, 2960
    gen = torch.Generator().manual_seed(2960)
    x = inject(random_codes((M, K), "e4m3fn", gen), "e4m3fn", 0.1, 0.05, gen)
    w = inject(random_codes((N, K), "e5m2", gen), "e5m2", 0.1, 0.05, gen)
    w[5, 1999] = 0x7C  # an infinity in one column
    for fast, S in ((True, 1), (False, 1), (True, 3), (False, 2), (True, 2)):
        check(dev, orc, x, "e4m3fn", w, "e5m2", 0.1, 1 / 3, "bf16", fast, S,
              f"16x8 tile, long k-list, {profile}", profile=profile, tile=8)
    c = _c_patterns(M, N, np.random.default_rng(7))
    got = gpu_accumulate_c(dev, x, "e4m3fn", w, "e5m2", c, profile, tile=8)
    want = orc.accumulate_c(x.numpy(), "e4m3fn", w.numpy(), "e5m2", c, profile=profile)
    assert_same(got, want, f"16x8 tile, long k-list, incoming accumulators, {profile}")


@pytest.mark.parametrize("seed", [101, 102])
def test_randomized_cases(dev, orc, seed):
    """200 seeded random problems per seed: ragged shapes (K = 0 included),
    every format pair, 1 to 9 splits, fast and slow, every profile, every
    output type (FP8 with scale_result), the automatic or a forced tile
    configuration, zeros, subnormals and (in a fifth of them) NaN / Inf
    codes; each compared bit for bit with the oracle."""
    import random
    rnd = random.Random(seed)
    for c in range(200):
        M = rnd.choice([1, 2, 15, 16, 17, 33, 64, 65, 100, 128, 200])
        N = 16 * rnd.randint(1, 48)
        K = 16 * rnd.choice([0, 1, 2, 3, 7, 8, 9, 16, 17, 33, 64, 65, 96])
        xf, wf = rnd.choice([("e4m3fn", "e4m3fn"), ("e4m3fn", "e5m2"), ("e5m2", "e4m3fn")])
        S = rnd.choice([1, 1, 1, 2, 3, 5, 8, 9])
        fast = rnd.random() < 0.5
        profile = rnd.choice(["hopper", "hopper", "ada-serial", "ada-pairwise"])
        outs = ["bf16", "fp16", "fp32", "e4m3fn"] + ([] if (xf, wf) == ("e4m3fn", "e4m3fn") else ["e5m2"])
        out = rnd.choice(outs)
        sr = rnd.choice([0.5, 3.0, 1 / 3]) if out in ("e4m3fn", "e5m2") else None
        tile = rnd.choice([-1, -1, -1] + list(range(len(api.TILE_CONFIGS))))
        sx = rnd.choice([1 / 64, 0.1, 1 / 3, -2.5, 7.0])
        sw = rnd.choice([1 / 32, 0.3, 1 / 3, 4.0])
        gen = torch.Generator().manual_seed(seed * 100000 + c)
        finite = rnd.random() < 0.8
        x = inject(random_codes((M, K), xf, gen, finite=finite), xf, 0.05, 0.05, gen)
        w = inject(random_codes((N, K), wf, gen, finite=finite), wf, 0.05, 0.05, gen)
        check(dev, orc, x, xf, w, wf, sx, sw, out, fast, S,
              f"random case {seed}/{c} tile {tile} finite={finite}", profile=profile, sr=sr, tile=tile)


# ---- dense specials ---------------------------------------------------------------
@pytest.mark.parametrize("profile,S,fast", [("hopper", 1, True), ("hopper", 3, True), ("ada-pairwise", 5, True),
                                            ("hopper", 1, False), ("ada-serial", 2, False)])
def test_dense_specials(dev, orc, profile, S, fast):
    """Many NaN rows (x) and E5M2 infinities with zeros (w), so that NaN rows,
    Inf rows, Inf x 0 pairs and mixed-sign infinite products all occur, in
    several splits: the NaN rows take the flag shortcut, the Inf rows the
    per-output walk; in slow mode on this small grid the chunk results are
    stored and the chunks holding special codes rescanned."""
    gen = torch.Generator().manual_seed(77 + S)
    rng = np.random.default_rng(77 + S)
    M, N, K = 70, 96, 1040
    x = inject(random_codes((M, K), "e4m3fn", gen), "e4m3fn", 0.05, 0.02, gen)
    w = inject(random_codes((N, K), "e5m2", gen), "e5m2", 0.3, 0.02, gen)
    for m in rng.choice(M, 30, replace=False):
        x[m, rng.integers(0, K)] = int(rng.choice([0x7F, 0xFF]))
    for n in rng.choice(N, 40, replace=False):
        for _ in range(int(rng.integers(1, 3))):
            w[n, rng.integers(0, K)] = int(rng.choice([0x7C, 0xFC]))
    for n in rng.choice(N, 5, replace=False):
        w[n, rng.integers(0, K)] = 0x7E  # e5m2 NaN
    assert fast or api.workspace_bytes(M, N, K, S, fast, profile) > (S > 1) * S * M * N * 4  # chunked
    for out in ("bf16", "fp32", "e4m3fn"):
        check(dev, orc, x, "e4m3fn", w, "e5m2", 0.1, 1 / 3, out, fast, S, f"dense specials {profile}",
              profile=profile)


def _inf_rows_and_columns(e5_rows: int, other_rows: int, K: int, seed: int):
    """Codes with whole rows of infinities, rows with exactly SPL = 8 and 9
    16-code chunks holding infinities (the per-row chunk list's capacity and
    its overflow), single infinities next to zeros, NaN codes, and partner
    rows that are zero-free and of one sign (so that +Inf and -Inf results
    occur as well as NaN)."""
    gen = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    e5 = inject(random_codes((e5_rows, K), "e5m2", gen), "e5m2", 0.05, 0.02, gen)
    ot = inject(random_codes((other_rows, K), "e4m3fn", gen), "e4m3fn", 0.05, 0.02, gen)
    e5[1, :] = 0x7C                                                  # +Inf row
    e5[2, :] = torch.from_numpy(rng.choice([0x7C, 0xFC], K).astype(np.uint8))  # Inf row, both signs
    for r, nchunks, codes in ((3, 8, [0x7C]), (4, 9, [0xFC]), (5, 8, [0x7C, 0xFC]), (6, 1, [0x7C])):
        for c in rng.choice(K // 16, nchunks, replace=False):
            e5[r, 16 * c + rng.integers(0, 16)] = int(rng.choice(codes))
    e5[7, rng.integers(0, K)] = 0x7D                                 # e5m2 NaN
    e5[8, 0], e5[8, K - 1] = 0xFC, 0xFC                              # first and last k
    pos = ot[0, :] & 0x7F
    pos[pos == 0] = 0x01
    pos[pos == 0x7F] = 0x7E
    ot[0, :] = pos                                                   # zero-free, positive
    ot[1, :] = ot[0, :] | 0x80                                       # zero-free, negative
    ot[2, :] = ot[0, :]
    ot[2, 16 * 5 + 3] = 0x00                                         # one zero
    ot[3, rng.integers(0, K)] = 0xFF                                 # e4m3fn NaN
    return e5, ot


@pytest.mark.parametrize("cfg", [-1, 1, 5, 6])
@pytest.mark.parametrize("profile,S,fast", [("hopper", 1, True), ("hopper", 3, True), ("ada-pairwise", 5, True),
                                            ("hopper", 1, False), ("ada-serial", 2, False)])
def test_inf_rows_and_columns(dev, orc, profile, S, fast, cfg):
    """Rows and columns of infinities (validation page, claims table: NaN
    and Inf rows and columns through the GEMM epilogue), on both operands,
    with the automatic tile and forced ones (one lane per output, four
    lanes per output, matrix-core exponents)."""
    K = 1040
    for e5_is_x in (True, False):
        e5, ot = _inf_rows_and_columns(40 if e5_is_x else 48, 48 if e5_is_x else 40, K, 5 + S)
        if e5_is_x:
            x, xfmt, w, wfmt = e5, "e5m2", ot, "e4m3fn"
        else:
            x, xfmt, w, wfmt = ot, "e4m3fn", e5, "e5m2"
        check(dev, orc, x, xfmt, w, wfmt, 0.1, 1 / 3, "bf16", fast, S,
              f"inf rows {xfmt}x{wfmt} {profile} tile {cfg}", profile=profile, tile=cfg)


# ---- infinities resolved after the main kernel --------------------------------------------
def _listed_infinities(e5, rng):
    """Rows with 63, 64 and 65 infinities around the per-row list's capacity
    of 64 (row 9: 64 of both signs, row 10: 65 negative ones, past the
    capacity, rows 11 and 12: 63 and 64 positive ones)."""
    K = e5.shape[1]
    for r, count, codes in ((9, 64, [0x7C, 0xFC]), (10, 65, [0xFC]), (11, 63, [0x7C]), (12, 64, [0x7C])):
        row = e5[r, :] & 0x7F
        row[row == 0x7C] = 0x3C                                      # no infinities but the listed ones
        row[row > 0x7C] = 0x3C
        ks = rng.choice(K, count, replace=False)
        row[ks] = torch.from_numpy(rng.choice(codes, count).astype(np.uint8))
        e5[r, :] = row


def _deferred_operands(e5_is_x, e5_rows, other_rows, K, seed):
    e5, ot = _inf_rows_and_columns(e5_rows, other_rows, K, seed)
    _listed_infinities(e5, np.random.default_rng(seed + 1))
    if e5_is_x:
        return e5, "e5m2", ot, "e4m3fn"
    return ot, "e4m3fn", e5, "e5m2"


@pytest.mark.parametrize("profile,S,fast,K", [("hopper", 1, True, 1040), ("hopper", 3, True, 1040),
                                              ("ada-pairwise", 5, True, 1040), ("ada-serial", 2, False, 1040),
                                              ("hopper", 1, True, 64496), ("ada-serial", 1, True, 64496)])
def test_deferred_infinities(dev, orc, profile, S, fast, K):
    """The deferred-infinity plan forced on small shapes: the row pass lists
    each e5m2 row's infinities and the fix-up kernel resolves the outputs
    those rows make non-finite (whole rows of infinities and rows past the
    list's capacity through the row walk; NaN rows in either operand left to
    the main kernel; a partial last block of staged rows), on both operands,
    against the oracle; with negative and zero scales (the epilogue's sign
    and Inf * 0), every output kind, and K = 64,496, the largest K whose
    rows fit the fix-up's LDS.  Small slow-mode grids store chunk results and
    keep the main kernel's own handling."""
    for e5_is_x in (True, False):
        x, xfmt, w, wfmt = _deferred_operands(e5_is_x, 44 if e5_is_x else 48, 48 if e5_is_x else 44, K,
                                              21 + S + K)
        if K > 2048:
            check(dev, orc, x, xfmt, w, wfmt, 0.1, 1 / 3, "bf16", fast, S,
                  f"deferred infinities {xfmt}x{wfmt} K={K}", profile=profile, defer="on")
            continue
        for out, sx in (("bf16", 0.1), ("fp32", -0.1), ("e5m2", 0.0), ("fp16", 2.0), ("e4m3fn", 0.1)):
            check(dev, orc, x, xfmt, w, wfmt, sx, 1 / 3, out, fast, S,
                  f"deferred infinities {xfmt}x{wfmt} out={out} sx={sx}", profile=profile, defer="on")


@pytest.mark.parametrize("cfg", range(len(api.TILE_CONFIGS)))
def test_deferred_infinities_every_tile(dev, orc, cfg):
    """The deferred plan with every tile configuration of the main kernel
    (each skips its own infinity scan for the fix-up to resolve), fast
    accumulation in one and in three splits, the e5m2 operand on either
    side."""
    K = 528
    for e5_is_x in (True, False):
        x, xfmt, w, wfmt = _deferred_operands(e5_is_x, 36 if e5_is_x else 48, 48 if e5_is_x else 36, K,
                                              51 + cfg)
        for S in (1, 3):
            check(dev, orc, x, xfmt, w, wfmt, 0.1, 1 / 3, "bf16", True, S,
                  f"deferred infinities tile {api.TILE_CONFIGS[cfg]} {xfmt}x{wfmt} S={S}", tile=cfg, defer="on")


def test_deferred_infinities_strided(dev, orc):
    """The deferred plan on operands whose rows are longer than K (ldx, ldw
    > K) and an output whose rows are longer than N (ldo > N), with the e5m2
    operand on either side; the padding of the output rows stays untouched."""
    K, pad = 1040, 64
    for e5_is_x in (True, False):
        x, xfmt, w, wfmt = _deferred_operands(e5_is_x, 44 if e5_is_x else 48, 48 if e5_is_x else 44, K, 41)
        M, N = x.shape[0], w.shape[0]
        xw = torch.zeros((M, K + pad), dtype=torch.uint8)
        ww = torch.zeros((N, K + pad), dtype=torch.uint8)
        xw[:, :K], ww[:, :K] = x, w
        xw[:, K:], ww[:, K:] = 0x7C if e5_is_x else 0x7F, 0x7F if e5_is_x else 0x7C  # specials past K
        xd = xw.to(dev)[:, :K].view(FP8_DTYPES[xfmt])
        wd = ww.to(dev)[:, :K].view(FP8_DTYPES[wfmt])
        ob = torch.full((M, N + 16), -7.0, dtype=torch.bfloat16, device=dev)
        o = ob[:, :N]
        sx = torch.tensor([0.1], device=dev)
        sw = torch.tensor([1 / 3], device=dev)
        note(f"[gpu] deferred infinities strided {xfmt}x{wfmt}")
        api.scaled_mm(xd, wd.t(), sx, sw, out_dtype=torch.bfloat16, use_fast_accum=True, out=o, defer="on")
        torch.cuda.synchronize(dev)
        _, y_o = oracle_run(orc, x, xfmt, w, wfmt, 0.1, 1 / 3, "bf16", True, 1)
        assert_same(bits_of(o.contiguous()), y_o, f"deferred infinities strided {xfmt}x{wfmt}")
        assert bool((ob[:, N:] == -7.0).all()), "output padding written"


@pytest.mark.parametrize("MN,S,profile", [(2304, 1, "hopper"), (1440, 2, "ada-serial")])
def test_deferred_infinities_slow_grid(dev, orc, MN, S, profile):
    """Slow accumulation on a grid large enough that no chunk results are
    stored (2304 x 2304 x 1040, or 1440 x 1440 x 1040 in two splits), so the
    deferred plan applies (with two groups of 2,048 e5m2 rows in the fix-up
    grid at 2304, after the combine kernel at S = 2); every output against
    the oracle."""
    x, xfmt, w, wfmt = _deferred_operands(False, MN, MN, 1040, 31 + S)
    part = S * MN * MN * 4 if S > 1 else 0
    assert api.workspace_bytes(MN, MN, 1040, S, False, profile, defer="on") == part + MN * 65 * 4  # no chunks
    check(dev, orc, x, xfmt, w, wfmt, 0.1, 1 / 3, "bf16", False, S, f"deferred infinities, slow grid S={S}",
          profile=profile, defer="on")


@pytest.mark.parametrize("profile,S", [("hopper", 1), ("ada-pairwise", 3)])
def test_deferred_infinities_workload(dev, orc, profile, S):
    """The 8192^3 e4m3fn x e5m2 workload with one w code in 1,000 an
    infinity (random signs), some w rows with 64, 65 or K infinities and a
    few NaN rows in both operands: the automatic plan defers the infinities
    (2^39 multiply-adds); every output must equal the main kernel's own
    handling (deferral forced off), and sampled outputs, a third of them in
    NaN or infinity rows, the oracle's.  Also with the ada profile in three
    splits (the fix-up after the pairwise combination)."""
    wl = WORKLOADS["mixed_8192"]
    x, w = make_operands(wl, 0)
    gen = torch.Generator().manual_seed(2000)
    hit = torch.rand(w.shape, generator=gen) < 1e-3
    signs = torch.randint(0, 2, w.shape, generator=gen, dtype=torch.uint8) << 7
    w[hit] = signs[hit] | 0x7C
    rng = np.random.default_rng(5)
    w[100, :] = 0x7C
    _listed_infinities(w[200:213], rng)
    w[300, 4000] = 0x7E                                              # e5m2 NaN
    x[400, 17] = 0xFF                                                # e4m3fn NaN
    part = S * wl.M * wl.N * 4 if S > 1 else 0
    assert api.workspace_bytes(wl.M, wl.N, wl.K, S, True, profile) == part + wl.N * 65 * 4
    note(f"[gpu] mixed_8192 with infinities {profile} S={S}: deferred (automatic)")
    y, acc = gpu_run(dev, x, wl.xfmt, w, wl.wfmt, wl.scale_x, wl.scale_w, wl.out, wl.fast, S, profile=profile)
    note(f"[gpu] mixed_8192 with infinities {profile} S={S}: in the main kernel")
    y0, acc0 = gpu_run(dev, x, wl.xfmt, w, wl.wfmt, wl.scale_x, wl.scale_w, wl.out, wl.fast, S,
                       profile=profile, defer="off")
    assert_same(acc, acc0, "deferred vs in-kernel infinities, accumulator")
    assert_same(y, y0, "deferred vs in-kernel infinities, output")
    ms = list(rng.integers(0, wl.M, 1500)) + [400] * 20 + list(rng.integers(0, wl.M, 60))
    ns = list(rng.integers(0, wl.N, 1500)) + list(rng.integers(0, wl.N, 20)) + \
        [100] * 10 + [300] * 10 + list(range(200, 213)) * 3 + [209]
    ms, ns = np.array(ms, dtype=np.int64), np.array(ns, dtype=np.int64)
    acc_o, y_o = orc.points(x.numpy(), wl.xfmt, w.numpy(), wl.wfmt, ms, ns, scale_bits(wl.scale_x),
                            scale_bits(wl.scale_w), wl.out, wl.fast, S, profile=profile)
    assert_same(acc[ms, ns], acc_o, "mixed_8192 with infinities, accumulator")
    assert_same(y[ms, ns], y_o, "mixed_8192 with infinities, output")
    nonfinite = int(((acc_o & 0x7F800000) == 0x7F800000).sum())
    assert nonfinite > 500, nonfinite


# ---- the largest shapes the grid limits allow --------------------------------------------
@pytest.mark.parametrize("S", [1, 2])
def test_rows_beyond_one_launch(dev, orc, S):
    """M above 65535 workgroup rows of the 16-row tile: the host splits the
    launch into row slices (and, for S = 2, the partials keep one layout);
    every output against the oracle.  Also the incoming-accumulator entry
    point over the same rows."""
    M, N, K = 65535 * 16 + 37, 16, 32
    gen = torch.Generator().manual_seed(71 + S)
    x = inject(random_codes((M, K), "e4m3fn", gen), "e4m3fn", 0.1, 0.05, gen)
    w = inject(random_codes((N, K), "e5m2", gen), "e5m2", 0.1, 0.05, gen)
    tile = 8  # 16x8 tiles, 4 lanes per output
    check(dev, orc, x, "e4m3fn", w, "e5m2", 0.5, 0.25, "bf16", True, S, f"rows beyond one launch S={S}", tile=tile)
    if S == 1:
        c = _c_patterns(M, N, np.random.default_rng(3))
        got = gpu_accumulate_c(dev, x, "e4m3fn", w, "e5m2", c, tile=tile)
        want = orc.accumulate_c(x.numpy(), "e4m3fn", w.numpy(), "e5m2", c)
        assert_same(got, want, "incoming accumulators, rows beyond one launch")


@pytest.mark.parametrize("profile", ["hopper", "ada-serial", "ada-pairwise"])
@pytest.mark.parametrize("fast", [True, False])
def test_largest_split_count(dev, orc, profile, fast):
    """split_S = 65535 (the largest grid z) on a K of three k-tiles: every
    split after the third is empty and adds +0 (partials are never -0), in
    the serial combination and in the pairwise tree (whose strides of 2 and
    1 then add p2 to p0 and p1 to that, as for S = 3; beyond 16 splits the
    tree runs in place in the workspace), so the result must equal the S = 3
    one, which the oracle checks."""
    tile = 128 if profile == "hopper" else 64
    M, N, K = 20, 32, 3 * tile
    gen = torch.Generator().manual_seed(73)
    x = inject(random_codes((M, K), "e4m3fn", gen), "e4m3fn", 0.1, 0.05, gen)
    w = inject(random_codes((N, K), "e4m3fn", gen), "e4m3fn", 0.1, 0.05, gen)
    check(dev, orc, x, "e4m3fn", w, "e4m3fn", 0.5, 0.25, "fp32", fast, 3, f"three splits {profile}",
          profile=profile)
    y3, acc3 = gpu_run(dev, x, "e4m3fn", w, "e4m3fn", 0.5, 0.25, "fp32", fast, 3, profile=profile)
    note(f"[gpu] split_S = 65535 {profile} fast={fast}")
    y, acc = gpu_run(dev, x, "e4m3fn", w, "e4m3fn", 0.5, 0.25, "fp32", fast, 65535, profile=profile)
    assert_same(acc, acc3, f"split_S = 65535 accumulator {profile}")
    assert_same(y, y3, f"split_S = 65535 output {profile}")


# ---- incoming accumulators -------------------------------------------------------------
C_CRAFTED = [0, 0x80000000, 1, 0x80000001, 0x3FF, 0x400, 0x7FFFFF, 0x807FFFFF, 0x800000, 0x00FFFFFF,
             0x3F7FFFFF, 0xBF7FFFFF, 0x3F800001, 0x7F7FFFFF, 0xFF7FFFFF, 0x7F800000, 0xFF800000,
             0x7FC00001, 0xFFFFFFFF, 0x2F7FFFFF, 0x0B000000, 0x45FFFFFF, 0xC5800001]


def _c_patterns(M, N, rng):
    c = rng.integers(0, 2**32, (M, N), dtype=np.uint64).astype(np.uint32)
    c = np.where((c & 0x7F800000) == 0x7F800000, c & 0xBFFFFFFF, c)  # mostly finite
    c.flat[:min(len(C_CRAFTED), c.size)] = C_CRAFTED[:c.size]
    if M > 2:
        c[1] &= np.uint32(0x80FFFFFF)  # tiny normals and subnormals
        c[2] = (c[2] & np.uint32(0x807FFFFF)) | np.uint32(0x47000000)  # about the chains' own size
    return c


def gpu_accumulate_c(dev, x, xfmt, w, wfmt, c_bits, profile="hopper", tile=None):
    xd = x.to(dev).view(FP8_DTYPES[xfmt])
    wd = w.to(dev).view(FP8_DTYPES[wfmt])
    cd = torch.from_numpy(c_bits.view(np.float32).copy()).to(dev)
    acc = api.accumulate(xd, wd, use_fast_accum=True, profile=profile, c=cd, tile=tile)
    torch.cuda.synchronize(dev)
    return bits_of(acc)


@pytest.mark.parametrize("tile", [-1] + list(range(len(api.TILE_CONFIGS))))
@pytest.mark.parametrize("profile", ["hopper", "ada-serial"])
def test_incoming_accumulators(dev, orc, profile, tile):
    """Fast chains from incoming accumulators (normal, tiny, subnormal,
    signed zero, infinite, NaN and chain-sized c), on ragged shapes, K = 0,
    rows of zero codes (the accumulator-only path), NaN / Inf codes, every
    format pair and every tile configuration, against the oracle."""
    rng = np.random.default_rng(41 + tile)
    for idx, (M, N, K) in enumerate([(5, 16, 0), (37, 80, 1040), (4, 48, 96), (70, 144, 272), (16, 256, 512)]):
        xfmt, wfmt = [("e4m3fn", "e5m2"), ("e5m2", "e4m3fn"), ("e4m3fn", "e4m3fn")][idx % 3]
        gen = torch.Generator().manual_seed(idx + 100 * tile)
        x = inject(random_codes((M, K), xfmt, gen), xfmt, 0.1, 0.05, gen)
        w = inject(random_codes((N, K), wfmt, gen), wfmt, 0.1, 0.05, gen)
        if K:
            x[0] = x[0] & 0x80  # a row of zero codes: c alone through every block
            w[3, K // 2] = 0x7C if wfmt == "e5m2" else 0x7F  # a special code in one column
            if xfmt == "e5m2":
                x[M - 1, 0] = 0xFC
        c = _c_patterns(M, N, rng)
        note(f"[gpu] incoming accumulators {profile} tile {tile}: M={M} N={N} K={K} {xfmt}x{wfmt}")
        got = gpu_accumulate_c(dev, x, xfmt, w, wfmt, c, profile, tile=tile)
        want = orc.accumulate_c(x.numpy(), xfmt, w.numpy(), wfmt, c, profile=profile)
        assert_same(got, want, f"incoming accumulators {profile} tile {tile} #{idx}")


@pytest.mark.parametrize("profile", ["hopper", "ada-pairwise"])
def test_incoming_accumulators_compose_chains(dev, orc, profile):
    """The GPU's accumulator of the first K1 columns, fed back as the incoming
    accumulator of the rest, gives the GPU's accumulator of all columns (K1 a
    multiple of the block width), on the 64 x 5760 x 1920 projection shape."""
    wl = WORKLOADS["proj_64x5760x1920"]
    x, w = make_operands(wl, 9)
    K1 = 640
    xd = x.to(dev).view(FP8_DTYPES[wl.xfmt])
    wd = w.to(dev).view(FP8_DTYPES[wl.wfmt])
    whole = api.accumulate(xd, wd, use_fast_accum=True, profile=profile)
    first = api.accumulate(xd[:, :K1].contiguous(), wd[:, :K1].contiguous(), use_fast_accum=True, profile=profile)
    rest = api.accumulate(xd[:, K1:].contiguous(), wd[:, K1:].contiguous(), use_fast_accum=True, profile=profile,
                          c=first)
    torch.cuda.synchronize(dev)
    assert_same(bits_of(rest), bits_of(whole), f"composed chains {profile}")
    ms = np.arange(0, wl.M, 7)
    ns = np.arange(0, wl.N, 331)
    mm, nn = np.meshgrid(ms, ns, indexing="ij")
    acc_o, _ = orc.points(x.numpy(), wl.xfmt, w.numpy(), wl.wfmt, mm.ravel(), nn.ravel(), scale_bits(1.0),
                          scale_bits(1.0), "fp32", True, 1, profile=profile)
    assert_same(bits_of(whole)[mm, nn].ravel(), acc_o, f"composed chains {profile}: sampled oracle")


def test_incoming_accumulators_in_place(dev, orc):
    """acc may be c_in itself (through the C ABI)."""
    M, N, K = 33, 64, 256
    gen = torch.Generator().manual_seed(5)
    x = inject(random_codes((M, K), "e4m3fn", gen), "e4m3fn", 0.1, 0.05, gen)
    w = inject(random_codes((N, K), "e5m2", gen), "e5m2", 0.1, 0.05, gen)
    c = _c_patterns(M, N, np.random.default_rng(5))
    want = orc.accumulate_c(x.numpy(), "e4m3fn", w.numpy(), "e5m2", c)
    xd, wd = x.to(dev), w.to(dev)
    buf = torch.from_numpy(c.view(np.float32).copy()).to(dev)
    lib = api._lib()
    st = lib.emu_accumulate_c(xd.data_ptr(), 0, K, wd.data_ptr(), 1, K, M, N, K, buf.data_ptr(), N, buf.data_ptr(),
                              N, 0, torch.cuda.current_stream(dev).cuda_stream, None)
    assert st == api.EMU_OK
    torch.cuda.synchronize(dev)
    assert_same(bits_of(buf), want, "incoming accumulators in place")


# ---- FP8 outputs ------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(16))
def test_fp8_outputs(dev, orc, seed):
    """FP8 outputs (scale_result, saturation, subnormals, NaN) over the edge
    cases: ragged sizes, splits (the combine kernel's store), both profiles,
    scale_result absent, fractional, negative, tiny or huge."""
    x, xfmt, w, wfmt, sx, sw, _, fast, S = _edge_case(2000 + seed)
    out = "e4m3fn" if (seed % 2 == 0 or xfmt == wfmt) else "e5m2"
    sr = [None, 0.3, -7.5, 2.0 ** -10, 3.0e5, 1.0][seed % 6]
    profile = ("hopper", "ada-pairwise")[seed % 2]
    check(dev, orc, x, xfmt, w, wfmt, sx, sw, out, fast, S, f"fp8 output {seed}", profile=profile, sr=sr)


def test_fp8_output_workload(dev, orc):
    """The user guide's example shape with an e4m3fn output (torch's default
    out_dtype for e4m3fn inputs) and a scale_result that saturates part of it."""
    wl = WORKLOADS["proj_64x5760x1920"]
    x, w = make_operands(wl, 0)
    check(dev, orc, x, wl.xfmt, w, wl.wfmt, wl.scale_x, wl.scale_w, "e4m3fn", wl.fast, 1,
          "proj e4m3fn output", sr=0.75)


def test_fp8_rejections(dev):
    """e4m3fn x e4m3fn -> e5m2 is rejected; scale_result needs an FP8 output."""
    x, w = make_operands(WORKLOADS["tiny"], 0)
    xd = x.to(dev).view(torch.float8_e4m3fn)
    wd = w.to(dev).view(torch.float8_e4m3fn)
    one = torch.ones(1, device=dev)
    with pytest.raises(api.EmuError) as e:
        api.scaled_mm(xd, wd.t(), one, one, out_dtype=torch.float8_e5m2)
    assert e.value.status == api.EMU_ERR_REJECTED
    with pytest.raises(api.EmuError) as e:
        api.scaled_mm(xd, wd.t(), one, one, out_dtype=torch.bfloat16, scale_result=one)
    assert e.value.status == api.EMU_ERR_UNSUPPORTED
    y = api.scaled_mm(xd, wd.t(), one, one)  # out_dtype defaults to the input dtype
    assert y.dtype == torch.float8_e4m3fn


# ---- the RTX 4060 (ada) profiles ------------------------------------------------
@pytest.mark.parametrize("name,seed,profile", [
    ("tiny", 0, "ada-serial"), ("tiny", 1, "ada-pairwise"),
    ("proj_64x5760x1920", 0, "ada-serial"),
    ("slow_256x4096x4096", 0, "ada-pairwise"),
    ("splitk_16x256x65536_s8", 0, "ada-serial"), ("splitk_16x256x65536_s8", 1, "ada-pairwise"),
    ("proj_2048x5760x1920", 0, "ada-serial"),
])
def test_ada_workload_full(dev, orc, name, seed, profile):
    """The workloads under the RTX 4060 profiles: 16-product blocks, 64-wide
    k-tiles dealt round-robin to the splits, serial or pairwise combination."""
    wl = WORKLOADS[name]
    x, w = make_operands(wl, seed)
    check(dev, orc, x, wl.xfmt, w, wl.wfmt, wl.scale_x, wl.scale_w, wl.out, wl.fast, wl.split_S,
          f"{name} seed {seed}", profile=profile)


@pytest.mark.parametrize("seed", range(24))
def test_ada_edge_cases(dev, orc, seed):
    """The edge-case sweep (ragged sizes, K = 0, empty splits, specials, every
    output type) under the ada profiles, with split counts from 1 to 17 so
    that the pairwise tree has absent leaves and the round-robin layout has
    splits of unequal length and a short last tile."""
    x, xfmt, w, wfmt, sx, sw, out, fast, S = _edge_case(1000 + seed)
    S = [1, 2, 3, 4, 5, 7, 8, 9, 16, 17][seed % 10]
    profile = ("ada-serial", "ada-pairwise")[seed % 2]
    check(dev, orc, x, xfmt, w, wfmt, sx, sw, out, fast, S, f"ada edge case {seed}", profile=profile)


def test_ada_large_sampled(dev, orc):
    """A 2048 x 2048 x 8192 e4m3 x e5m2 problem (the matrix-core exponent
    path at size) under ada-pairwise with S = 3, on sampled outputs."""
    wl = Workload("ada_large", 2048, 2048, 8192, "e4m3fn", "e5m2", 40.0, 1000.0, 0.01, 0.01,
                  1 / 256, 1 / 256, True, 3, "bf16")
    x, w = make_operands(wl, 0)
    note("[gpu] ada_large: full-size run")
    y, acc = gpu_run(dev, x, wl.xfmt, w, wl.wfmt, wl.scale_x, wl.scale_w, wl.out, wl.fast, wl.split_S,
                     profile="ada-pairwise")
    rng = np.random.default_rng(1)
    ms = np.array(list(rng.integers(0, wl.M, 600)) + [0, wl.M - 1, 63, 64], dtype=np.int64)
    ns = np.array(list(rng.integers(0, wl.N, 600)) + [wl.N - 1, 0, 64, 63], dtype=np.int64)
    acc_o, y_o = orc.points(x.numpy(), wl.xfmt, w.numpy(), wl.wfmt, ms, ns, scale_bits(wl.scale_x),
                            scale_bits(wl.scale_w), wl.out, wl.fast, wl.split_S, profile="ada-pairwise")
    assert_same(acc[ms, ns], acc_o, "ada_large accumulator")
    assert_same(y[ms, ns], y_o, "ada_large output")


# ---- invariants -------------------------------------------------------------------
def test_out_buffer_is_ignored(dev):
    """The result does not depend on what the output buffer held (validation
    page, scope table row 'Epilogue')."""
    x, w = make_operands(WORKLOADS["tiny"], 5)
    ys = [gpu_run(dev, x, "e4m3fn", w, "e4m3fn", 0.1, 0.3, "bf16", True, 1, prefill=p)[0]
          for p in (0x00, 0xFF, 0x7F)]
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])


def test_deterministic_across_streams(dev):
    """The same call twice, on two different streams, gives the same bits
    (validation page, claims table: the bits do not change when the scheduling is perturbed)."""
    wl = WORKLOADS["splitk_16x256x65536_s8"]
    x, w = make_operands(wl, 4)
    s1, s2 = torch.cuda.Stream(dev), torch.cuda.Stream(dev)
    a = gpu_run(dev, x, "e4m3fn", w, "e4m3fn", wl.scale_x, wl.scale_w, "bf16", True, 8, stream=s1)
    b = gpu_run(dev, x, "e4m3fn", w, "e4m3fn", wl.scale_x, wl.scale_w, "bf16", True, 8, stream=s2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_padding_rows_do_not_change_other_rows(dev):
    """Padding M changes no other row (user guide section 7)."""
    x, w = make_operands(WORKLOADS["proj_64x5760x1920"], 6, N=256)
    gen = torch.Generator().manual_seed(6)
    pad = random_codes((37, x.shape[1]), "e4m3fn", gen)
    y0, a0 = gpu_run(dev, x, "e4m3fn", w, "e4m3fn", 1 / 64, 1 / 32)
    y1, a1 = gpu_run(dev, torch.cat([x, pad]), "e4m3fn", w, "e4m3fn", 1 / 64, 1 / 32)
    assert np.array_equal(y0, y1[:x.shape[0]]) and np.array_equal(a0, a1[:x.shape[0]])


def test_strided_rows(dev, orc):
    """Operands whose rows are longer than K (ldx, ldw > K)."""
    x, w = make_operands(WORKLOADS["tiny"], 7, K=512)
    K = 208
    xs = x.to(dev)[:, :K].view(torch.float8_e4m3fn)
    ws = w.to(dev)[:, :K].view(torch.float8_e4m3fn)
    sx = torch.tensor([0.1], device=dev)
    sw = torch.tensor([0.2], device=dev)
    y = api.scaled_mm(xs, ws.t(), sx, sw, out_dtype=torch.float16, use_fast_accum=False)
    torch.cuda.synchronize(dev)
    acc_o, y_o = oracle_run(orc, x[:, :K].contiguous(), "e4m3fn", w[:, :K].contiguous(), "e4m3fn", 0.1, 0.2,
                            "fp16", False, 1)
    assert_same(bits_of(y), y_o, "strided rows")
