"""The C-ABI library loads on the CPU and exports every function that
include/dsa.h declares (no compute: that needs a GPU)."""
import ctypes
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "dsa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", src)))


def _lib_path():
    from sparse_attention_scores_amd import build
    if not os.path.exists(build.LIB):
        build.build()
    return build.LIB


def test_header_declares_the_path_entry_points():
    names = _declared()
    for n in ("dsa_index_scores", "dsa_topk", "dsa_sparse_attend", "dsa_pool_select",
              "dsa_pool_keys", "dsa_visibility_ranges", "dsa_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib_path())
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_knows_every_export():
    from sparse_attention_scores_amd import binding
    assert sorted(binding.EXPORTS) == _declared()


def test_host_side_validation_without_gpu():
    """Argument errors are reported before anything touches the GPU."""
    from sparse_attention_scores_amd import binding
    lib = binding.load()
    assert lib.dsa_topk(None, 1, 10, 10, None, None, 0, None, None, 0, None) == -1
    assert b"top_k" in lib.dsa_last_error()
    assert lib.dsa_topk(None, 1, 10, 10, None, None, 4096, None, None, 0, None) == -2
    assert lib.dsa_index_scores(None, None, 0, None, 0, None, None, None, None, None, None) == -1
    assert lib.dsa_topk_workspace_size(8, 131072, 2048) > 0
    assert lib.dsa_topk_workspace_size(8, 8192, 2048) == 0
