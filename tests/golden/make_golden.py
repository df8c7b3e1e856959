"""Writes oracle_cfg1.json from oracle/ only (never from the HIP path)."""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402


def main():
    w = workloads.make_config(1, with_qkv=False)
    kb_off, ext = oracle.extrema(w.cu_seqlens, w.startend, w.n_vec, w.causal, 4)
    cls = oracle.classify(w.cu_seqlens, kb_off, ext, w.causal, 4, 4)
    doc = {
        "written_by": "tests/golden/make_golden.py (oracle only)",
        "config": 1, "block_q": 4, "block_k": 4,
        "kb_off": kb_off.tolist(), "extrema": ext.tolist(),
        "classes": cls[0].tolist(),
        "class_counts": oracle.class_counts(cls).tolist(),
        "unmasked_pairs": oracle.unmasked_pairs(w.cu_seqlens, w.startend, w.n_vec, w.causal),
    }
    with open(os.path.join(HERE, "oracle_cfg1.json"), "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
