"""Pins of the oracle's traffic and work counts against the lesson page's 28 rows (CPU only)."""
import json
from pathlib import Path

import pytest

from oracle import traffic as TR

GOLD = Path(__file__).resolve().parent / "golden"
ROWS = json.loads((GOLD / "lesson_traffic_rows.json").read_text())["rows"]


@pytest.mark.parametrize("row", ROWS, ids=lambda r: f"{r['kind']}-N{r['N']}-d{r['d']}")
def test_walker_reproduces_page_row(row):
    N, d, B = row["N"], row["d"], row["B"]
    if row["kind"] == "fused":
        w = TR.walk_fused(N, d, B)
        keys = ["globalReads", "globalWrites", "fma", "exps", "barriers", "sharedReads", "sharedWrites",
                "globalBytes", "extraMemoryBytes", "sharedPerWorkgroupBytes"]
    else:
        w = TR.walk_unfused(N, d, B)
        keys = ["globalReads", "globalWrites", "fma", "exps", "globalBytes", "extraMemoryBytes"]
    for k in keys:
        assert w[k] == row[k], k
    elems = w["globalReads"] + w["globalWrites"]
    assert TR.over_theta(row["kind"], N, d, B, elems) == pytest.approx(row["overTheta"], abs=5e-5)
    if row["kind"] == "unfused":
        assert TR.score_share(N, d, B) == pytest.approx(row["scoreShare"], abs=5e-5)
        fused = TR.walk_fused(N, d, B)
        assert w["globalBytes"] / fused["globalBytes"] == pytest.approx(row["overFused"], abs=5e-5)


@pytest.mark.parametrize("N,d,B", [(100, 8, 32), (64, 64, 32), (300, 16, 128), (17, 4, 5)])
def test_closed_forms_equal_walkers(N, d, B):
    w, c = TR.walk_fused(N, d, B), TR.closed_fused(N, d, B)
    for k in c:
        assert w[k] == c[k], k
    w, c = TR.walk_unfused(N, d, B), TR.closed_unfused(N, d, B)
    for k in c:
        assert w[k] == c[k], k


def test_unfused_minus_fused_is_four_score_tables():
    for N, d, B in [(64, 16, 128), (1024, 64, 32), (4096, 16, 128)]:
        u, f = TR.closed_unfused(N, d, B), TR.closed_fused(N, d, B)
        assert (u["globalReads"] + u["globalWrites"]) - (f["globalReads"] + f["globalWrites"]) == 4 * N * N
