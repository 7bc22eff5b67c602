"""Recipe that wrote page_layout_bytes.json from the benchmark pages' text.

It reads the pages as mounted at /root/reference/PAPER.md (three JSON documents,
one per page) and keeps, for every "chunked" record of kernel_ssd_cpu.json, the
argument and output byte counts.  It is not run by the tests.
"""
import json
import re
import sys

src = sys.argv[1] if len(sys.argv) > 1 else "/root/reference/PAPER.md"
out = sys.argv[2] if len(sys.argv) > 2 else "page_layout_bytes.json"
txt = open(src).read()
parts = re.split(r"=-=-= page \d of 3: (\S+) =-=-=", txt)
rows = []
for i in range(1, len(parts), 2):
    url, body = parts[i], parts[i + 1]
    if not url.endswith("kernel_ssd_cpu.json"):
        continue
    doc = json.loads(body)
    for r in doc["results"]:
        if r.get("impl") != "chunked":
            continue
        rows.append({
            "page": "kernel_ssd_cpu.json",
            "record": f"chunked·{r['mode']}·{r['config']}·T{r['seq']}",
            "mode": r["mode"], "config": r["config"],
            "B": r["batch"], "G": r["groups"], "H": r["heads"], "T": r["seq"],
            "dk": r["dk"], "dv": r["dv"],
            "xla_arg_mb": r["xla_arg_mb"], "xla_out_mb": r["xla_out_mb"],
        })
json.dump({"source": "benchmark page kernel_ssd_cpu.json, results records of impl chunked; "
                     "fields xla_arg_mb and xla_out_mb (MiB)",
           "rows": rows}, open(out, "w"), indent=1)
print(len(rows), "rows")
