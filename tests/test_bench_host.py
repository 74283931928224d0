"""CPU checks of bench.py's host logic: the hash that ties the committed counter records to
the kernel sources ignores comments and blank space but nothing else."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_code_only_drops_comments_and_blank_space():
    import bench

    src = 'int a = 1; // note\n/* block\n comment */ int  b =\t2;\n'
    assert bench._code_only(src) == "int a = 1; int b = 2;"


def test_code_only_keeps_literals():
    import bench

    src = 'const char* s = "// kept /* too */"; char c = \'"\'; char d = \'\\\'\'; // gone'
    assert bench._code_only(src) == 'const char* s = "// kept /* too */"; char c = \'"\'; char d = \'\\\'\';'


def test_code_changes_change_the_hash():
    import bench

    a = bench._code_only("int f() { return 1; } // one")
    b = bench._code_only("int f() { return 1; }   /* two */")
    c = bench._code_only("int f() { return 2; }")
    assert a == b and a != c
