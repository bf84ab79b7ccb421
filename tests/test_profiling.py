"""The kernel-source hash that ties committed counter figures to the code they were taken on:
comments and layout do not change it, code does. CPU only."""
from moe_grouped_gemm_e4m3_amd.profiling import _code_only, source_hash


def test_comments_and_layout_are_ignored():
    a = 'int f(int x) {  // add one\n  return x + 1; /* the\n value */ }\n'
    b = 'int f(int x) {\n  /* different words */ return   x + 1;\n}'
    assert _code_only(a) == _code_only(b)
    assert source_hash([a, "x"]) == source_hash([b, "x"])


def test_literals_are_kept_and_code_counts():
    src = 'const char* s = "a // b /* c */"; char q = \'"\'; int y = 2;'
    assert _code_only(src) == src
    assert source_hash([src, ""]) != source_hash([src.replace("2", "3"), ""])


def test_current_sources_hash():
    h = source_hash()
    assert len(h) == 16 and int(h, 16) >= 0
