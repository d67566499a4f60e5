"""Host-side pieces of bench.py: the source hash that dates the profiles in profiles/ ignores
comments and layout (so a comment edit does not orphan a counter run) and changes with the code."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_code_text_drops_comments_and_layout_only():
    b = load_bench()
    a = b.code_text('int a = 1;  // one\n/* block\n comment */ float x  =  2.0f;\n')
    assert a == b.code_text("int a = 1; float x = 2.0f;")
    # string and character literals keep comment-like text
    s = 'const char* p = "// not a comment"; char c = \'/\'; /* gone */ int d;'
    assert b.code_text(s) == 'const char* p = "// not a comment"; char c = \'/\'; int d;'
    assert b.code_text('char q = \'"\'; int e; // x') == "char q = '\"'; int e;"
    # a change to the code itself shows
    assert b.code_text("int a = 1;") != b.code_text("int a = 2;")
