"""Host logic of bench.py: the kernel source hash ignores comments and layout, not code; the HBM summary."""
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


def test_hbm_summary_divides_recorded_bytes_by_time(monkeypatch):
    rec = {"fwd": 8e8, "dq": 1.2e9, "dkv": 1.0e9}
    monkeypatch.setattr(bench, "measured_traffic", lambda s: rec[s])
    per = {"fwd": 0.2, "dq": 0.4, "dkv": 0.5}
    h = bench.hbm_summary(per, 1.0)
    assert h["bytes_per_step"] == 3.0e9
    assert h["achieved"] == 3000.0 and h["unit"] == "GB/s" and h["peak"] == 8000.0
    assert h["frac"] == 0.375
    assert h["kernels"]["fwd64_kernel"] == {"bytes": 8e8, "achieved": 4000.0}
    assert h["kernels"]["dkv64_kernel"]["achieved"] == 2000.0


def test_hbm_summary_withheld_without_a_matching_record(monkeypatch):
    monkeypatch.setattr(bench, "measured_traffic", lambda s: None if s == "dq" else 1.0)
    assert bench.hbm_summary({"fwd": 1.0, "dq": 1.0, "dkv": 1.0}, 3.0) is None
