"""Host logic of bench.py: the kernel source hash ignores comments and layout, not code."""
import bench


def test_code_only_strips_comments_keeps_strings():
    src = 'int a = 1; // note\n/* block\n comment */ const char* s = "x // y /* z */";\n  int   b;'
    assert bench._code_only(src) == 'int a = 1; const char* s = "x // y /* z */"; int b;'


def test_code_only_handles_escapes_and_chars():
    assert bench._code_only("char c = '\\''; // q\nchar d = '/';") == "char c = '\\''; char d = '/';"
    assert bench._code_only('s = "a\\"//b"; // c') == 's = "a\\"//b";'


def test_code_changes_change_the_hash_comments_do_not(tmp_path, monkeypatch):
    csrc = tmp_path / "exact_attention_forward_amd" / "csrc"
    csrc.mkdir(parents=True)
    f = csrc / "k.hip"
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    f.write_text("int f() { return 1; }\n")
    h0 = bench.kernel_source_hash()
    f.write_text("// explained\nint f() {\n  return 1;  /* one */\n}\n")
    assert bench.kernel_source_hash() == h0
    f.write_text("int f() { return 2; }\n")
    assert bench.kernel_source_hash() != h0
