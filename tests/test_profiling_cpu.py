"""The profile summaries' source digest: comments do not count, code does."""

from quantized_expert_gemv_amd.profiling import _code_only


def test_comment_edits_leave_the_code_text_unchanged():
    a = "int f(int x) {  // doubles\n  return 2 * x;\n}\n"
    b = "/* a block\n   comment */\nint f(int x) {\n\n  return 2 * x;  // twice\n}\n"
    assert _code_only(a) == _code_only(b)


def test_code_edits_change_the_code_text():
    a = "int f(int x) {\n  return 2 * x;\n}\n"
    b = "int f(int x) {\n  return 3 * x;\n}\n"
    assert _code_only(a) != _code_only(b)
