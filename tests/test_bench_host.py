"""Host-side helpers of bench.py (no GPU): the source digest that keys the recorded HBM
traffic to the kernels it was measured on."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_code_only_drops_comments_and_blank_space_but_keeps_literals():
    src = ('int a = 1;   // trailing\n'
           '/* block\n   comment */\n'
           '\n'
           'const char* s = "x // y /* z */";  char q = \'"\';\n'
           '  return   a;\n')
    assert bench.code_only(src) == 'int a = 1;\nconst char* s = "x // y /* z */"; char q = \'"\';\nreturn a;'


def test_digest_ignores_comments_but_not_code(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    monkeypatch.setitem(bench.OP_SOURCES, "probe", ["k.hip"])
    f = tmp_path / "k.hip"
    f.write_text("x = y * 2;  // twice\n")
    d0 = bench.source_digest("probe")
    f.write_text("// a comment added above\nx = y * 2;  // two times\n")
    assert bench.source_digest("probe") == d0
    f.write_text("x = y * 3;\n")
    assert bench.source_digest("probe") != d0
