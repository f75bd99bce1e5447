"""bench.py reports HBM traffic from profiles/ only while the HIP code is the
code that was measured: the source hash ignores comments and whitespace and
changes with any code token."""

import os
import shutil

import bench


def _tree(tmp_path):
    root = tmp_path / "repo"
    shutil.copytree(os.path.join(bench.ROOT, "block_sparse_long_scores_amd", "csrc"),
                    root / "block_sparse_long_scores_amd" / "csrc")
    return root


def _hash(monkeypatch, root):
    monkeypatch.setattr(bench, "ROOT", str(root))
    return bench.kernel_source_hash()


def test_hash_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    root = _tree(tmp_path)
    h0 = _hash(monkeypatch, root)
    f = root / "block_sparse_long_scores_amd" / "csrc" / "pool_select.hip"
    text = f.read_text()
    f.write_text("// a new first line\n/* and a\n   block comment */\n" + text.replace("\n", "\n\n", 5))
    assert _hash(monkeypatch, root) == h0


def test_hash_changes_with_code(tmp_path, monkeypatch):
    root = _tree(tmp_path)
    h0 = _hash(monkeypatch, root)
    f = root / "block_sparse_long_scores_amd" / "csrc" / "pool_select.hip"
    text = f.read_text()
    assert "constexpr int kSelThreads = 256;" in text
    f.write_text(text.replace("constexpr int kSelThreads = 256;", "constexpr int kSelThreads = 128;"))
    assert _hash(monkeypatch, root) != h0
