"""The host I/O model that picks the bf16 forward's tiling (no GPU needed).

It enumerates the tilings that fit a gfx950 CU, prices them per (query, key)
pair and ranks them; the forward runs the best-ranked compiled one.  Checked
here: every enumerated tiling really fits (LDS, registers, waves), the ranking
puts the tallest resident query tile first among the near-cheapest (the I/O
criterion), attn_query_tiling reports the pick, and the pick is the tiling
measured fastest on MI355X for every bf16 workload (the committed sweep under
profiles/, made by `bench.py --mode tilings`).
"""

import json
import os
import re

import pytest

from exact_long_sequence_amd import attnio

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SWEEP = os.path.join(ROOT, "profiles", "attn_fwd_bf16_tilings_sweep_all_workloads.md")
LDS = 160 * 1024


@pytest.mark.parametrize("d", [64, 128])
def test_every_enumerated_tiling_fits_a_cu(d):
    ev = attnio.attn_tiling_enumerate(d)
    assert len(ev) > 10
    for e in ev:
        t = e["tiling"]
        assert t["d"] == d and t["BM"] == 32 * t["waves"] * t["qb"]
        assert t["wg_per_cu"] * t["lds_bytes"] <= LDS
        ring = t["stages"] * 2 * t["BN"] * d * 2
        assert t["lds_bytes"] >= ring and t["lds_bytes"] >= t["BM"] * d * 2
        waves_per_simd = t["waves"] // 4 * t["wg_per_cu"]
        assert waves_per_simd <= 8 and t["waves"] * 64 <= 1024
        assert e["vgpr_budget"] == min(256, 512 // waves_per_simd)
        assert e["vgpr_estimate"] <= e["vgpr_budget"]
        # the predicted cost is the costliest of the four levels
        assert e["cycles_per_pair"] >= e["issue_cycles_per_pair"]
        assert e["l2_to_lds_bytes_per_pair"] == pytest.approx(4 * d / t["BM"])
        assert e["beyond_l2_bytes_per_pair"] == pytest.approx(4 * d / (32 * t["wg_per_cu"] * t["BM"]))
        assert e["lds_read_bytes_per_pair"] == pytest.approx(4 * d / (32 * t["qb"]))


@pytest.mark.parametrize("d", [64, 128])
def test_every_compiled_tiling_is_feasible_and_ranked(d):
    ev = attnio.attn_tiling_enumerate(d)
    ranked = {e["compiled"] for e in ev if e["compiled"] >= 0}
    built = {i for i in range(attnio.attn_tiling_count()) if attnio.attn_tiling_get(i)["d"] == d}
    assert built == ranked


@pytest.mark.parametrize("d", [64, 128])
def test_ranking_puts_the_tallest_query_tile_first(d):
    """Among the tilings predicted within 15% of the cheapest, the first has the
    fewest bytes into LDS per pair (the tallest BM), and the cheapest
    prediction among those."""
    ev = attnio.attn_tiling_enumerate(d)
    best = min(e["cycles_per_pair"] for e in ev)
    band = [e for e in ev if e["cycles_per_pair"] <= 1.15 * best]
    first = ev[0]
    assert first in band
    assert first["tiling"]["BM"] == max(e["tiling"]["BM"] for e in band)
    tallest = [e for e in band if e["tiling"]["BM"] == first["tiling"]["BM"]]
    assert first["beyond_l2_bytes_per_pair"] == min(e["beyond_l2_bytes_per_pair"] for e in tallest)
    # the whole order is: band first, then the rest by predicted cost
    outside = [e["cycles_per_pair"] for e in ev[len(band):]]
    assert outside == sorted(outside)


def test_no_larger_query_tile_fits():
    """Brute force over the parameters: no tiling with a taller resident query
    tile than the pick's fits the registers of its residency."""
    for d in (64, 128):
        pick = attnio.attn_tiling_enumerate(d)[0]["tiling"]
        for waves in (4, 8, 16):
            for qb in (1, 2):
                bm = 32 * waves * qb
                if bm <= pick["BM"]:
                    continue
                # the smallest register need: 32-key tiles, VALU row sum
                need = qb * (d // 2 + d // 4 + 16 + 8) + 4 * ((4 if qb == 1 else 2) + 1) + 2 * qb + 9
                budget = min(256, 512 // (waves // 4))
                assert need > budget, (d, waves, qb, need, budget)


def test_query_tiling_reports_the_pick():
    for d in (64, 128):
        first = attnio.attn_tiling_enumerate(d)[0]
        assert first["compiled"] >= 0
        t = attnio.attn_tiling_get(first["compiled"])
        for causal in (False, True):
            assert attnio.attn_query_tiling(d, causal) == {"BM": t["BM"], "BN": t["BN"], "stages": t["stages"]}


def test_pick_is_the_measured_fastest_tiling():
    """The committed same-box sweep of every compiled tiling on the four bf16
    workloads: the model's pick must be the fastest, or within 1% of it."""
    text = open(SWEEP).read()
    lines = [json.loads(l) for l in re.findall(r'^\{"mode": "tilings".*\}$', text, flags=re.M)]
    assert {l["workload"] for l in lines} == {"bf16_h16_n8k_d128", "bf16_causal_h32_n32k_d128",
                                              "bf16_causal_h8_n128k_d64", "bf16_padded_b4_h32_n16k_d128_q8"}
    for l in lines:
        d = 64 if l["workload"].endswith("d64") else 128
        pick = attnio.attn_tiling_enumerate(d)[0]["compiled"]
        ms = {r["tiling"]: r["ms_median"] for r in l["results"]}
        assert pick in ms
        assert ms[pick] <= 1.01 * min(ms.values()), (l["workload"], pick, ms)
