"""Host checks of bench.py's bookkeeping (no GPU): the counter records are keyed on the code of
the kernel sources, so a comment edit keeps a record valid and a code edit voids it, and every
record in profiles/ names a kernel bench.py knows."""
import glob
import os
import re

import bench as B


def test_comments_do_not_change_the_code_key():
    code = "int f(int x) {\n  return x + 1;  // one more\n}\n/* block\n comment */\n"
    assert B.source_code_only(code) == B.source_code_only(code.replace("one more", "another comment"))
    assert B.source_code_only(code) == B.source_code_only(code.replace("block\n comment", "other"))
    assert B.source_code_only(code) != B.source_code_only(code.replace("x + 1", "x + 2"))
    assert "//" not in B.source_code_only(code) and "/*" not in B.source_code_only(code)


def test_counter_records_name_known_kernels_and_workloads():
    recs = glob.glob(os.path.join(B.PROFILES, "counters_*.md"))
    assert recs
    for p in recs:
        text = open(p).read()
        m = re.search(r"^- kernel: (\S+)$", text, flags=re.M)
        if m is None:  # summaries of several kernels carry no record
            continue
        assert m.group(1) in B.KERNEL_SOURCES, p
        assert re.search(r"^- source_sha256: `[0-9a-f]{64}`$", text, flags=re.M), p
        assert re.search(r"^- traffic_bytes_per_launch: \d+$", text, flags=re.M), p
