"""Host-side checks of bench.py's bookkeeping (no GPU)."""
import bench


def test_strip_comments_keeps_code_and_strings():
    src = 'int a = 1; // note\n/* block\n comment */ const char *s = "x // y /* z */";\nchar q = \'/\';  int  b;\n'
    assert bench.strip_comments(src) == 'int a = 1; const char *s = "x // y /* z */"; char q = \'/\'; int b;'


def test_strip_comments_escaped_quote_in_string():
    assert bench.strip_comments('"a\\"//b" // c') == '"a\\"//b"'


def test_comment_edit_leaves_code_unchanged_but_code_edit_does_not():
    base = "asm volatile(\"v_mov_b32 v0, 0\\n\"); // the move\n"
    assert bench.strip_comments(base) == bench.strip_comments(base.replace("the move", "clear v0"))
    assert bench.strip_comments(base) != bench.strip_comments(base.replace("v0, 0", "v0, 1"))
