import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (full-size workloads)")


@pytest.fixture(scope="session")
def gpu():
    """The loaded HIP library on cuda:0; fails loudly when it is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a GPU")
    import block_sparse_long_scores_amd as fp2
    fp2.load()
    return fp2


def pytest_terminal_summary(terminalreporter):
    """Per-block parity figures of the full-size checks (every label that
    names a benchmark workload): the worst (query block, KV head) pair and
    the last query block's rel-L2, next to the tolerance each pair is held to."""
    from tests.helpers import PARITY_LOG
    rows = [r for r in PARITY_LOG if r["label"].startswith(("llama8b", "paged_batch6"))]
    if not rows:
        return
    terminalreporter.section("per-block parity (full-size workloads)")
    for r in rows:
        lse = f", worst lse {r['worst_lse']:.2e}" if r["worst_lse"] is not None else ""
        terminalreporter.write_line(
            f"{r['label']}: {r['pairs']} pairs, worst rel_l2 {r['worst_rel_l2']:.2e} (block {r['worst_block']} "
            f"head {r['worst_head']}), worst max_abs {r['worst_max_abs']:.2e}, last block {r['last_block']} "
            f"rel_l2 {r['last_rel_l2']:.2e}{lse}; tol {r['tol']:.0e}{'' if r['fp8'] else ' / 2e-02 abs'}")
