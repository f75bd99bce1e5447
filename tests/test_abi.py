"""C-ABI contract checks that need no GPU: the library loads, exports every
function include/fp2.h declares, and host-side validation rejects bad
arguments with the documented status before anything is enqueued."""

import ctypes
import math
import os
import re

import pytest

import block_sparse_long_scores_amd as fp2

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fp2.h")

FAKE = 0x1000  # non-NULL pointer that is never dereferenced by validation


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fp2_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = fp2.load()
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
        assert n in fp2.EXPORTED, n
    assert fp2.fp2_version().startswith("fp2")


def params(**kw):
    d = dict(num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=128, tau=1.0)
    d.update(kw)
    return fp2.make_params(d["num_q_heads"], d["num_kv_heads"], d["head_dim"], d["block_size"], tau=d["tau"])


def select(p, batch=1, sq=1024, sk=1024, ws=1 << 30, q=FAKE, wsp=FAKE):
    return fp2.fp2_select_blocks(p, batch, sq, sk, q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, wsp, ws, None)


def test_block_counts():
    assert fp2.fp2_num_q_blocks(1024, 1024, 128) == 8
    assert fp2.fp2_num_q_blocks(100, 1000, 128) == 1      # positions 900..999
    assert fp2.fp2_num_q_blocks(200, 1000, 128) == 2      # 800..999 spans blocks 6, 7
    assert fp2.fp2_num_k_blocks(1000, 128) == 8
    assert fp2.fp2_num_q_blocks(10, 5, 128) == 0


def test_workspace_sizes():
    p = params()
    assert fp2.fp2_select_workspace_size(p, 1, 1024, 1024) == 2 * 8 * 128 * 4
    assert fp2.fp2_select_workspace_size(params(head_dim=96), 1, 1024, 1024) == 0
    mq, mk = fp2.fp2_paged_mask_dims(p, 16384, 131072)
    assert (mq, mk) == (129, 1024)
    assert fp2.fp2_paged_workspace_size(p, 6, 32768, 131072) > 0
    # per-query-head selection pools every query head: G = 4 times the pooled queries
    for mode in (1, 2):
        u = params()
        u.select_mode = mode
        assert fp2.fp2_select_workspace_size(u, 1, 1024, 1024) == 4 * 2 * 8 * 128 * 4
        assert fp2.fp2_paged_workspace_size(u, 6, 32768, 131072) > fp2.fp2_paged_workspace_size(p, 6, 32768, 131072)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_one_workspace_size_covers_both_paths(mode):
    """fp2_workspace_size(p, batch, max_sq, max_sk) is at least the select
    workspace of every smaller call and the paged workspace of every smaller
    batch; it is 0 for invalid parameters."""
    p = params()
    p.select_mode = mode
    for B, msq, msk in [(1, 131072, 131072), (6, 32768, 131072), (3, 1000, 5000), (2, 1, 129)]:
        w = fp2.fp2_workspace_size(p, B, msq, msk)
        assert w > 0 and w % 256 == 0
        for b in range(1, B + 1):
            assert w >= fp2.fp2_paged_workspace_size(p, b, msq, msk)
        for sk in sorted({msk, max(msq, msk - 1), max(msq, msk - 127), msq}):
            for sq in sorted({msq, max(1, msq - 1), max(1, msq // 2), 1, 129, 128}):
                if sq <= min(msq, sk):
                    assert w >= fp2.fp2_select_workspace_size(p, B, sq, sk), (B, sq, sk)
    assert fp2.fp2_workspace_size(params(head_dim=96), 1, 1024, 1024) == 0
    assert fp2.fp2_workspace_size(p, 0, 1024, 1024) == 0
    assert fp2.fp2_workspace_size(p, 1, 2048, 1024) == 0


def test_validation_errors():
    lib = fp2.load()
    assert lib.fp2_select_blocks(None, 1, 8, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == fp2.FP2_EINVAL
    assert "params" in fp2.last_error()
    assert select(params(num_q_heads=6, num_kv_heads=4)) == fp2.FP2_EINVAL
    assert select(params(head_dim=96)) == fp2.FP2_EUNSUPPORTED
    assert select(params(block_size=32)) == fp2.FP2_EUNSUPPORTED
    assert select(params(tau=float("nan"))) == fp2.FP2_EINVAL
    assert select(params(), batch=0) == fp2.FP2_EINVAL
    assert select(params(), sq=2048, sk=1024) == fp2.FP2_EINVAL
    assert select(params(), q=None) == fp2.FP2_EINVAL
    assert select(params(), ws=16) == fp2.FP2_EWORKSPACE
    assert select(params(), wsp=None) == fp2.FP2_EWORKSPACE
    assert "workspace" in fp2.last_error()
    p = params()
    p.in_dtype = fp2.FP2_FP8_E4M3
    assert select(p) == fp2.FP2_EINVAL                      # fp8 without scales
    # head counts beyond the pooling kernel's row capacity are rejected up front
    assert select(params(num_q_heads=128, num_kv_heads=8)) == fp2.FP2_EUNSUPPORTED
    assert "heads" in fp2.last_error()
    assert select(params(num_q_heads=64, num_kv_heads=64)) == fp2.FP2_EUNSUPPORTED
    assert fp2.fp2_max_seqlen_k(params(num_q_heads=128, num_kv_heads=8)) == 0
    assert fp2.fp2_max_seqlen_k(params(num_q_heads=64, num_kv_heads=8)) > 0
    for mode in (3, -1):
        p = params()
        p.select_mode = mode
        assert select(p) == fp2.FP2_EINVAL
        assert "select_mode" in fp2.last_error()
    p = params()
    p.out_dtype = 7
    assert fp2.fp2_dense_prefill(p, 1, 8, 8, FAKE, FAKE, FAKE, FAKE, None, None) == fp2.FP2_EUNSUPPORTED
    p = params()
    p.out_dtype = fp2.FP2_FP8_E4M3                          # e4m3 output without its scale
    assert fp2.fp2_dense_prefill(p, 1, 8, 8, FAKE, FAKE, FAKE, FAKE, None, None) == fp2.FP2_EINVAL
    assert "o_scale" in fp2.last_error()
    p = params()
    p.mean_correction = 1
    assert fp2.fp2_sparse_prefill(p, 1, 8, 8, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None,
                                  None) == fp2.FP2_EINVAL   # correction needs pooled blocks


def test_longest_sequence_limit():
    """fp2_max_seqlen_k is the exact edge: one key block more is rejected
    (before anything is launched) by the attention entry points."""
    p = params(num_q_heads=32, num_kv_heads=8)
    m = fp2.fp2_max_seqlen_k(p)
    assert m > 1 << 21 and m % 128 == 0
    assert fp2.fp2_max_seqlen_k(params(head_dim=96)) == 0
    over = m + 128
    assert fp2.fp2_sparse_prefill(p, 1, 1, over, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                  None) == fp2.FP2_EUNSUPPORTED
    assert "too long" in fp2.last_error()
    assert fp2.fp2_dense_prefill(p, 1, 1, over, FAKE, FAKE, FAKE, FAKE, None, None) == fp2.FP2_EUNSUPPORTED
    npg = over // 64 + 1
    assert fp2.fp2_sparse_prefill_paged(p, 1, FAKE, FAKE, FAKE, 1, over, FAKE, FAKE, npg, 64, FAKE, npg, FAKE, None,
                                        None, None, FAKE, 1 << 40, None) == fp2.FP2_EUNSUPPORTED


def test_paged_validation_errors():
    p = params()
    args = dict(q=FAKE, cu=FAKE, sk=FAKE, mq=1024, mk=4096, kc=FAKE, vc=FAKE, npages=64, page=64, table=FAKE,
                mpp=64, out=FAKE, lse=None, idx=None, cnt=None, ws=FAKE, wsb=1 << 30)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return fp2.fp2_sparse_prefill_paged(p, 2, a["q"], a["cu"], a["sk"], a["mq"], a["mk"], a["kc"], a["vc"],
                                            a["npages"], a["page"], a["table"], a["mpp"], a["out"], a["lse"],
                                            a["idx"], a["cnt"], a["ws"], a["wsb"], None)
    assert call(page=48) == fp2.FP2_EUNSUPPORTED
    assert call(page=256) == fp2.FP2_EUNSUPPORTED           # must divide the block size
    assert call(page=1) == fp2.FP2_EUNSUPPORTED             # a block spans at most 64 pages
    assert call(table=None) == fp2.FP2_EINVAL
    assert call(idx=FAKE) == fp2.FP2_EINVAL                 # idx without cnt
    assert call(mpp=8) == fp2.FP2_EINVAL                    # table too short for max_seqlen_k
    assert call(wsb=1024) == fp2.FP2_EWORKSPACE
    assert call(npages=0) == fp2.FP2_EINVAL

    def pooled(bsk=FAKE, bsv=FAKE, cached=FAKE, **kw):
        a = dict(args)
        a.update(kw)
        return fp2.fp2_sparse_prefill_paged_pooled(p, 2, a["q"], a["cu"], a["sk"], a["mq"], a["mk"], a["kc"], a["vc"],
                                                   a["npages"], a["page"], a["table"], a["mpp"], a["out"], a["lse"],
                                                   a["idx"], a["cnt"], a["ws"], a["wsb"], bsk, bsv, cached, None)
    assert pooled(bsk=None) == fp2.FP2_EINVAL
    assert pooled(cached=None) == fp2.FP2_EINVAL
    assert pooled(bsv=None) == fp2.FP2_EINVAL               # mean correction needs the V sums
    assert pooled(page=48) == fp2.FP2_EUNSUPPORTED          # the paged checks apply as well


def test_status_strings():
    assert fp2.status_string(fp2.FP2_OK) == "FP2_OK"
    assert fp2.status_string(fp2.FP2_EWORKSPACE) == "FP2_EWORKSPACE"
    assert fp2.status_string(-99) == "FP2_UNKNOWN"


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU; --gpus N > 1 exits with a message before
    touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_header_is_plain_c(tmp_path):
    """include/fp2.h compiles as C99 and a C program links against the
    library and gets the documented host-side answers (no device calls)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    lib = fp2.LIB_PATH
    src = tmp_path / "abi.c"
    src.write_text(r'''
#include <math.h>
#include <stdio.h>
#include "fp2.h"
int main(void) {
  fp2_params p = {0};
  p.num_q_heads = 32; p.num_kv_heads = 8; p.head_dim = 128; p.block_size = 128;
  p.tau = 1.0f; p.mean_correction = 1; p.in_dtype = FP2_BF16; p.out_dtype = FP2_BF16;
  if (fp2_num_q_blocks(1024, 1024, 128) != 8) return 1;
  if (fp2_max_seqlen_k(&p) <= 0) return 2;
  if (fp2_select_blocks(NULL, 1, 8, 8, 0, 0, 0, 0, 0, 0, 0, 0, 0, NULL) != FP2_EINVAL) return 3;
  p.tau = NAN;
  if (fp2_dense_prefill(&p, 1, 8, 8, 0, 0, 0, 0, 0, NULL) != FP2_EINVAL) return 4;
  printf("%s | %s\n", fp2_version(), fp2_last_error());
  return 0;
}
''')
    exe = tmp_path / "abi"
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(root, "include"), str(src), lib,
                        "-lm", f"-Wl,-rpath,{os.path.dirname(lib)}", "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "NaN" in r.stdout
