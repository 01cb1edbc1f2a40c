"""Host-side logic of bench.py (no GPU needed).

The HBM-traffic figure that bench.py reports for the k = 4 batch-1 launch was
measured with rocprofv3 counters on particular kernel sources; bench.py reports
it only while the code of those sources is unchanged.  The digest it compares
covers the code with comments removed, so a comment edit keeps the figure and
any code edit drops it.
"""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_host_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


SRC = """// header comment
#include "x.h"
/* block
   comment */
int f(int a) {   // trailing comment
    return a + 1;  /* inline */ }
"""


def test_comments_and_blank_lines_do_not_count():
    b = _bench()
    code = b.source_code_text(SRC)
    assert "comment" not in code and "inline" not in code
    assert code == '#include "x.h"\nint f(int a) {\n    return a + 1;    }\n'
    edited = SRC.replace("// header comment", "// another header\n\n// and one more line")
    assert b.source_code_text(edited) == code


def test_code_edits_count():
    b = _bench()
    code = b.source_code_text(SRC)
    assert b.source_code_text(SRC.replace("a + 1", "a + 2")) != code
    assert b.source_code_text(SRC.replace("int f", "long f")) != code


def test_traffic_reported_only_for_the_measured_sources():
    b = _bench()
    digest = b.headline_source_digest()
    assert len(digest) == 64
    expected = b.TRAFFIC_K4_BYTES if digest.startswith(b.TRAFFIC_K4_SOURCE_SHA256_PREFIX) else None
    assert b.measured_traffic() == expected
    b.TRAFFIC_K4_SOURCE_SHA256_PREFIX = "not-a-digest"
    assert b.measured_traffic() is None
