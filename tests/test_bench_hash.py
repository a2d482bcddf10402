"""The kernel-source hash that ties recorded profiles to the code: comments
and spacing do not change it, code does (CPU only)."""
import bench


def test_code_only_drops_comments_and_keeps_literals():
    text = 'int a = 1; // note\n/* block\n note */ const char* s = "// not a comment"; char q = \'"\';\n'
    assert bench._code_only(text) == 'int a = 1; const char* s = "// not a comment"; char q = \'"\';'


def test_comment_edit_keeps_code_and_code_edit_changes_it():
    base = "__global__ void k(int* x) {\n  x[0] = 1;  // store\n}\n"
    reworded = "// a kernel\n__global__ void k(int* x) {\n  x[0] = 1;  /* the store */\n}\n"
    changed = "__global__ void k(int* x) {\n  x[0] = 2;  // store\n}\n"
    assert bench._code_only(base) == bench._code_only(reworded)
    assert bench._code_only(base) != bench._code_only(changed)


def test_hash_is_stable():
    assert bench.kernel_source_hash() == bench.kernel_source_hash()
    assert len(bench.kernel_source_hash()) == 16
