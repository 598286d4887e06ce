"""Profile bookkeeping (CPU): the kernel-source digest that ties a committed
profile to the code it measured ignores comments and layout, and nothing
else."""
from differentiable_adaptive_ode_amd.profiling import _code_only


def test_comments_and_layout_are_ignored():
    a = "int a = 1;  // one\n/* block\n comment */ float b = a / 2;\n"
    b = "int a = 1;\nfloat   b = a / 2; // half\n"
    assert _code_only(a) == _code_only(b) == "int a = 1; float b = a / 2;"


def test_literals_and_operators_are_kept():
    src = 'const char* s = "x // y /* z */"; char c = \'/\'; d = e / f; g = "\\"//";'
    assert _code_only(src) == src


def test_a_code_change_is_seen():
    assert _code_only("r = fma(a, b, c);") != _code_only("r = fma(a, c, b);")
