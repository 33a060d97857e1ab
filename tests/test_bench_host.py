"""Host logic of bench.py (no GPU): the key that ties the measured HBM
traffic constants to the kernel sources ignores comments and layout but not
code (a changed kernel reports its traffic as null until the counters are
taken again)."""
import bench


def _digest(tmp_path, text):
    f = tmp_path / "k.hip"
    f.write_text(text)
    return bench.sources_sha256([str(f)])


def test_source_key_ignores_comments_and_layout(tmp_path):
    base = _digest(tmp_path, "int f(int x) {\n    return x + 1;  // one more\n}\n")
    assert base == _digest(tmp_path, "/* header */\nint f(int x) {\n  return x + 1;  // another note\n}\n")
    assert base == _digest(tmp_path, "int f(int x) { return x + 1; }")
    assert base != _digest(tmp_path, "int f(int x) {\n    return x + 2;  // one more\n}\n")

