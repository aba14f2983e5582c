"""Host-side parts of bench.py (no GPU): the key that ties a stored counter
summary to the kernel code it was taken on."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_tokens_ignores_comments_and_layout():
    a = "int f(int x) {\n    return x + 1;  // one more\n}\n"
    b = "/* header */\nint f(int x) { return x + 1; }\n"
    assert bench.code_tokens(a) == bench.code_tokens(b)


def test_code_tokens_sees_code_changes():
    a = "int f(int x) { return x + 1; }"
    for b in ("int f(int x) { return x + 2; }", "int f(int x) { return x - 1; }", "int f(int y) { return y + 1; }"):
        assert bench.code_tokens(a) != bench.code_tokens(b)


def test_code_tokens_keeps_literals_whole():
    # comment markers inside string and character literals are code
    src = 'const char* s = "a // b /* c */"; char q = \'"\'; int x; // gone'
    assert bench.code_tokens(src) == 'const char* s = "a // b /* c */"; char q = \'"\'; int x;'

