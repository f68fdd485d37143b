"""The kernel-source hash that bench.py checks before it reports the HBM
traffic recorded in profiles/: comments and layout do not change it, code
does (host only, no GPU)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_comments_and_layout_are_ignored():
    a = "int f(int x) {\n  return x + 1;  // one more\n}\n"
    b = "/* header\n   comment */\nint f(int x)\n{ return x + 1; }\n"
    assert bench.strip_comments(a).replace(" ", "") == bench.strip_comments(b).replace(" ", "")


def test_code_changes_are_seen():
    assert bench.strip_comments("return x + 1;") != bench.strip_comments("return x + 2;")


def test_comment_markers_inside_literals_are_code():
    src = 'const char* s = "// not a comment /* either */"; char c = \'/\'; // tail'
    out = bench.strip_comments(src)
    assert '"// not a comment /* either */"' in out
    assert "'/'" in out
    assert "tail" not in out


def test_hash_is_stable_and_short():
    h = bench.kernel_source_hash()
    assert h == bench.kernel_source_hash()
    assert len(h) == 16 and all(ch in "0123456789abcdef" for ch in h)
