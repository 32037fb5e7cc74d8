"""Write the page-printed values used as oracle pins into tests/golden/*.json.

Reads the text of the "Lesson K23 fused attention" facts page (a single JSON
record: blocks traffic.rows, controls.vector, controls.checker, probe.heads and
correctness.rows) from a local text copy of the page named on the command
line, and keeps only numbers and field names.  Run once:

    python tests/golden/extract_page_fixtures.py PAGE_TEXT_FILE

The outputs are committed; no test reads the page text at run time.
"""
import json
import sys
from pathlib import Path

OUT = Path(__file__).resolve().parent
PAGE = "Lesson K23 'fused attention' facts page"


def page_record(src: Path) -> dict:
    for line in src.read_text().splitlines():
        line = line.strip()
        if line.startswith("{") and '"traffic"' in line:
            return json.loads(line)
    sys.exit("facts record not found")


def main() -> None:
    if len(sys.argv) != 2:
        sys.exit("usage: extract_page_fixtures.py PAGE_TEXT_FILE")
    rec = page_record(Path(sys.argv[1]))
    keep = ["N", "d", "B", "kind", "globalReads", "globalWrites", "fma", "exps", "barriers", "sharedReads",
            "sharedWrites", "globalBytes", "extraMemoryBytes", "sharedPerWorkgroupBytes", "overTheta", "scoreShare",
            "overFused"]
    rows = [{k: r[k] for k in keep} for r in rec["traffic"]["rows"]]
    (OUT / "lesson_traffic_rows.json").write_text(json.dumps(
        {"source": f"{PAGE}, block traffic.rows (one head, float32, no mask)", "rows": rows}, indent=1) + "\n")

    vec = rec["controls"]["vector"]
    (OUT / "online_vector.json").write_text(json.dumps(
        {"source": f"{PAGE}, block controls.vector (values printed to 4 decimals)",
         **{k: vec[k] for k in ["values", "maxWeightDiff", "maxRises", "sum", "brokenSum", "trace", "brokenTrace"]}},
        indent=1) + "\n")

    heads = [{k: h[k] for k in ["layer", "head", "row", "rowMax", "argmax", "trace"]} for h in rec["probe"]["heads"]]
    (OUT / "probe_traces.json").write_text(json.dumps(
        {"source": f"{PAGE}, block probe.heads (scaled scores of query 10, tiles of 4 keys, 4 decimals)",
         "heads": heads}, indent=1) + "\n")

    (OUT / "lesson_checker.json").write_text(json.dumps(
        {"source": f"{PAGE}, blocks correctness.rows and controls.checker",
         "checker": rec["controls"]["checker"],
         "rows": [{k: r[k] for k in ["N", "d", "B", "kind", "ok", "outputs"]} for r in rec["correctness"]["rows"]]},
        indent=1) + "\n")


if __name__ == "__main__":
    main()
