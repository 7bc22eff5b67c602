"""Recipe that wrote page_layout_bytes.json from the text of the benchmark
pages.

Source: kernel_ssd_cpu.json, results records of impl "chunked", fields
xla_arg_mb and xla_out_mb (MiB).  The recipe takes the extracted text of the
pages as its input (the three JSON documents, each introduced by a line that
names the page's address) and keeps, for every chunked record of that page,
the shape and the two byte counts.  It is not run by the tests.

    python extract_page_bytes.py PAGES_TEXT OUT_JSON
"""
import json
import re
import sys

if len(sys.argv) != 3:
    sys.exit("usage: extract_page_bytes.py PAGES_TEXT OUT_JSON")
src, out = sys.argv[1], sys.argv[2]
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
