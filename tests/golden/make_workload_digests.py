"""Write tests/golden/workload_digests.json: the SHA-256 digests (first 16 hex
digits, as bench.py reports them under inputs_sha256) of every input tensor of
the five named workloads, drawn by the seeded generator.

    python tests/golden/make_workload_digests.py

Calls only decode_attention_03_amd.workloads (generate, digest): no attention
arithmetic, no HIP library.  tests/test_workloads.py compares fresh draws
against this file, so a change of the generator, of torch's random streams or
of the rounding into the storage types shows up as a failing CPU test instead
of a silently different benchmark.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from decode_attention_03_amd import workloads  # noqa: E402

OUT = os.path.join(HERE, "workload_digests.json")


def digests() -> dict:
    out = {}
    for c, w in sorted(workloads.WORKLOADS.items()):
        inp = workloads.generate(w)
        out[w.name] = {"config": c, "max_kv_len": inp["max_kv_len"], **workloads.digest(inp)}
        del inp
    return out


def main() -> None:
    rec = {"generator": "decode_attention_03_amd/workloads.py",
           "digest": "first 16 hex digits of SHA-256 over each tensor's storage bytes",
           "workloads": digests()}
    with open(OUT, "w", encoding="utf-8") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
