"""Census of the blocks an exact int8 matrix-core path could take.

    python bench.py --f4-census

Measurement on the host only (no GPU, no kernel): for each workload, a
16 x 16 sample of outputs over the first 4,096 positions of split 0's k-list
(hopper profile: 32-product blocks, slow workloads restart every 128), it
counts the blocks whose block sum is an exact integer dot product of int8
mantissa planes, i.e. where the block step would cut nothing:

  A  no term is cut: every nonzero product's field exponent sum g is within
     7 of the block exponent E (its term P * 2^(g - E + 7) is an integer);
  B  the incoming accumulator is exact at the quantum 2^(E - 13): it is +0
     or its exponent is E (a conservative test);
  C  the planes fit int8 and one scale serves the whole dot product: in the
     output's x row and w column, the block's nonzero codes span at most 3
     binades each (significand times 2^spread <= 127 with 4-bit
     significands), and the two rows' smallest exponents add up to at least
     E - 7.

The accumulator the tests need is approximated by the exact (float64) running
sum of the products, which is all a census needs: truncation changes it by a
few units of its 14th bit.  The census decides whether the int8 path is
built: a workload would have to pass A, B and C on at least BUILD_THRESHOLD of
its blocks for the path to repay the per-block test it adds to every block
(about as many instructions as the block maximum itself).
"""
from __future__ import annotations

import json

import numpy as np

from .inputs import WORKLOAD_ORDER, WORKLOADS, make_operands

BUILD_THRESHOLD = 0.25
SAMPLE = 16
K_SAMPLE = 4096
BLOCK = 32
CHUNK = 128
SPLIT_TILE = 128


def decode(codes: np.ndarray, fmt: str):
    """(sign, field exponent at emin for subnormals, significand with 3
    fraction bits, nonzero) per code; NaN / Inf codes do not occur in the
    workloads."""
    c = codes.astype(np.int64)
    s = c >> 7
    if fmt == "e4m3fn":
        ef, mf = (c >> 3) & 15, c & 7
        e = np.maximum(ef, 1) - 7
        M = np.where(ef > 0, 8 + mf, mf)
    else:
        ef, mf = (c >> 2) & 31, c & 3
        e = np.maximum(ef, 1) - 15
        M = 2 * np.where(ef > 0, 4 + mf, mf)
    return s, e, M, M > 0


def census_workload(name: str, seed: int = 0) -> dict:
    wl = WORKLOADS[name]
    x, w = make_operands(wl, seed)
    nt = -(-wl.K // SPLIT_TILE)
    tps = -(-nt // wl.split_S)
    klen = min(wl.K, tps * SPLIT_TILE, K_SAMPLE)   # split 0's k-list starts at k = 0
    klen -= klen % BLOCK
    res = census_codes(x.numpy()[:SAMPLE, :klen], wl.xfmt, w.numpy()[:SAMPLE, :klen], wl.wfmt, wl.fast)
    return {"workload": name, **res}


def census_codes(xs: np.ndarray, xfmt: str, ws: np.ndarray, wfmt: str, fast: bool) -> dict:
    """The census over all outputs of x [m, k] and w [n, k] (k a multiple of
    the block width), chained from +0 (fast) or restarted every 128."""
    rows_m, rows_n, klen = xs.shape[0], ws.shape[0], xs.shape[1]
    sa, ea, Ma, nza = decode(xs, xfmt)
    sb, eb, Mb, nzb = decode(ws, wfmt)
    nb = klen // BLOCK
    # [m, n, k] products
    P = Ma[:, None, :] * Mb[None, :, :]
    nz = P > 0
    g = ea[:, None, :] + eb[None, :, :]
    val = np.where((sa[:, None, :] ^ sb[None, :, :]) == 1, -1.0, 1.0) * P * np.exp2(g - 6.0)
    Pb, gb, nzb3, valb = (a.reshape(rows_m, rows_n, nb, BLOCK) for a in (P, g, nz, val))
    # per-row / per-column exponent spans of the block's nonzero codes
    ea_b, eb_b = ea.reshape(rows_m, nb, BLOCK), eb.reshape(rows_n, nb, BLOCK)
    nza_b, nzb_b = nza.reshape(rows_m, nb, BLOCK), nzb.reshape(rows_n, nb, BLOCK)
    big, small = 10**6, -10**6
    a_max = np.where(nza_b, ea_b, small).max(-1)
    a_min = np.where(nza_b, ea_b, big).min(-1)
    b_max = np.where(nzb_b, eb_b, small).max(-1)
    b_min = np.where(nzb_b, eb_b, big).min(-1)
    fit_a = (a_max - a_min) <= 3
    fit_b = (b_max - b_min) <= 3
    counts = {"blocks": 0, "empty": 0, "A": 0, "AB": 0, "ABC": 0}
    c = np.zeros((rows_m, rows_n))
    for blk in range(nb):
        if not fast and (blk * BLOCK) % CHUNK == 0:
            c[:] = 0.0
        nzk = nzb3[:, :, blk, :]
        any_nz = nzk.any(-1)
        gmax = np.where(nzk, gb[:, :, blk, :], small).max(-1)
        ec = np.where(c != 0, np.floor(np.log2(np.abs(np.where(c != 0, c, 1.0)))), small)
        E = np.maximum(gmax, ec)
        A = np.where(nzk, E[..., None] - gb[:, :, blk, :] <= 7, True).all(-1)
        B = (c == 0) | (ec == E)
        C = fit_a[:, None, blk] & fit_b[None, :, blk] & \
            (a_min[:, None, blk] + b_min[None, :, blk] >= E - 7)
        live = any_nz | (c != 0)
        counts["blocks"] += int(live.sum())
        counts["empty"] += int((~live).sum())
        counts["A"] += int((A & live).sum())
        counts["AB"] += int((A & B & live).sum())
        counts["ABC"] += int((A & B & C & live).sum())
        c = c + valb[:, :, blk, :].sum(-1)
    n = max(counts["blocks"], 1)
    return {"outputs": rows_m * rows_n, "k_positions": klen, **counts,
            "frac_exact_terms": counts["A"] / n, "frac_exact_block": counts["AB"] / n,
            "frac_int8_path": counts["ABC"] / n}


def main():
    rows = [census_workload(name) for name in WORKLOAD_ORDER]
    best = max(r["frac_int8_path"] for r in rows)
    for r in rows:
        print(json.dumps({"f4_census": r}), flush=True)
    print(json.dumps({"f4_decision": {"threshold": BUILD_THRESHOLD, "best_workload_fraction": best,
                                      "build_int8_path": best >= BUILD_THRESHOLD}}), flush=True)


if __name__ == "__main__":
    main()
