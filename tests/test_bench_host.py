"""Host logic of bench.py that needs no GPU: the kernel-source hash that ties
committed counter figures to the code they were taken on."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _hash_of(tmp_path, text):
    p = tmp_path / "k.hip"
    p.write_text(text)
    return bench.kernel_source_hash([str(p)])


def test_comment_and_whitespace_edits_keep_the_hash(tmp_path):
    base = 'int f(int x) {  // old note\n  return x + 1; /* block */\n}\nconst char* s = "a // b";\n'
    edited = '/* header */\nint f(int x) {   // new note\n\n  return x + 1;\n}\nconst char* s = "a // b";\n'
    assert _hash_of(tmp_path, base) == _hash_of(tmp_path, edited)


def test_code_edits_change_the_hash(tmp_path):
    base = 'int f(int x) { return x + 1; }\nconst char* s = "a // b";\n'
    assert _hash_of(tmp_path, base) != _hash_of(tmp_path, base.replace("x + 1", "x + 2"))
    # text inside a string literal (inline assembly, for one) is code
    assert _hash_of(tmp_path, base) != _hash_of(tmp_path, base.replace("a // b", "a // c"))

