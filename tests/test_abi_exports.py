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
    # torch first: libdsa then binds to torch's HIP runtime instead of mapping
    # a second one (the binding refuses a process with two)
    import torch  # noqa: F401

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
    assert lib.dsa_topk(None, 1, 10, 10, None, None, 0, 0, None, None, 0, None) == -1
    assert b"top_k" in lib.dsa_last_error()
    assert lib.dsa_topk(None, 1, 10, 10, None, None, 4096, 0, None, None, 0, None) == -2
    assert lib.dsa_index_scores(None, None, 0, None, 0, None, None, None, None, None, None) == -1
    assert lib.dsa_topk_workspace_size(8, 131072, 2048) > 0
    assert lib.dsa_topk_workspace_size(8, 8192, 2048) == 0


def test_workspace_errors_without_gpu():
    """A missing or short workspace is DSA_ERR_WORKSPACE, found on the host
    before any launch (the pointers below are never dereferenced: every call
    here fails validation)."""
    from sparse_attention_scores_amd import binding
    lib = binding.load()
    fake = ctypes.c_void_p(0x1000)
    # long rows: the threshold top-k keeps its pairs and candidates in the
    # workspace (a 64-byte header, 5 blocks x 24 pairs of 8 + 4 bytes, then
    # 16384 candidates of 8 bytes on a 256-byte boundary)
    need = lib.dsa_topk_workspace_size(1, 20000, 2048)
    assert need == 1536 + 16384 * 8
    assert lib.dsa_topk(fake, 1, 20000, 20000, fake, fake, 2048, 0, fake, None, 0, None) == -4
    assert b"workspace" in lib.dsa_last_error()
    assert lib.dsa_topk(fake, 1, 20000, 20000, fake, fake, 2048, 0, fake, fake, need - 1,
                        None) == -4
    # few decode rows: the gather kernel's split-K partials
    dims = binding._AttnDims(2, 1, 8192, 64, 576, 512, 1, 2048, 576 ** -0.5)
    need = lib.dsa_sparse_attend_workspace_size(ctypes.byref(dims))
    assert need > 0
    for ws, nb in ((None, 0), (fake, need - 1)):
        rc = lib.dsa_sparse_attend(ctypes.byref(dims), 1, fake, fake, 576, fake, 576, fake,
                                   None, None, fake, None, ws, nb, None)
        assert rc == -4, rc
    # the per-head kernel's tile-major selection bitmap (300 queries padded
    # to 512, 10 words of keys) and its fp16 copy of V
    dims = binding._AttnDims(1, 300, 300, 8, 192, 256, 8, 40, 192 ** -0.5)
    need = lib.dsa_sparse_attend_workspace_size(ctypes.byref(dims))
    assert need >= 512 * 10 * 4 + 300 * 8 * 256 * 2
    rc = lib.dsa_sparse_attend(ctypes.byref(dims), 1, fake, fake, 8 * 192, fake, 8 * 256, fake,
                               None, None, fake, None, fake, need - 4, None)
    assert rc == -4, rc


def test_binding_rejects_short_or_mistyped_tensors():
    """The binding checks shapes and dtypes before the ABI call, so a short
    range tensor or a bf16 score tensor is an error, not a device fault
    (CPU tensors reach the checks after the device check only, so these use
    a stand-in that passes it)."""
    import pytest
    import torch

    from sparse_attention_scores_amd import binding

    class Dev(torch.Tensor):
        @property
        def is_cuda(self):
            return True

    def dev(t):
        return t.as_subclass(Dev)

    S = dev(torch.zeros(2, 10, dtype=torch.bfloat16))
    lo = dev(torch.zeros(2, dtype=torch.int32))
    with pytest.raises(TypeError):
        binding.topk(S, lo, lo, 4)
    S = dev(torch.zeros(2, 10))
    short = dev(torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError):
        binding.topk(S, short, lo, 4)
    with pytest.raises(TypeError):
        binding.pool_select(dev(torch.zeros(1, 4, 2, dtype=torch.bfloat16)), lo, lo, 4, 1, 8)
    with pytest.raises(ValueError):
        binding.pool_select(dev(torch.zeros(2, 4, 2)), lo, short, 4, 1, 8)


def test_noalloc_topk_limit_without_gpu():
    """The allocation-free top-k refuses rows whose chunk winners would not
    fit its fixed scratch, before anything else (pointers never used)."""
    from sparse_attention_scores_amd import binding
    lib = binding.load()
    fake = ctypes.c_void_p(0x1000)
    # 2000 rows of 20000 keys at k 2048 need 2000 * 2 * 2048 * 8 bytes > 16 MiB
    assert lib.dsa_topk_workspace_size(2000, 20000, 2048) > (16 << 20)
    rc = lib.dsa_topk_noalloc(fake, 2000, 20000, 20000, fake, fake, 2048, 0, fake, None)
    assert rc == -2
    assert b"scratch" in lib.dsa_last_error()
    assert lib.dsa_topk_noalloc(fake, 1, 10, 10, fake, fake, 0, 0, fake, None) == -1


def test_index_share_rule_without_gpu():
    """dsa_index_share_source (host function) against the oracle's rule and
    the pages' 21 full layers of 78."""
    import oracle
    from sparse_attention_scores_amd import binding
    for il in range(-3, 400):
        assert binding.index_share_source(il) == oracle.index_share_source(il), il
    full = [il for il in range(78) if binding.index_share_source(il) == il]
    assert full == [0, 1, 2] + list(range(6, 75, 4))
