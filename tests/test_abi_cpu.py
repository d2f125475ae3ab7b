"""The C-ABI library without a GPU: it loads, binds to the HIP runtime torch
already loaded, exports every entry point include/kvoff.h declares, and its
argument checks and no-device path return the documented statuses."""
import os
import re

import pytest

import sparse_kv_cache_mean_amd as kv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "kvoff.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const char\*|int64_t|size_t|int|void)\s+(kvoff_\w+)\(",
                                 text, re.M)))


def test_header_declarations_are_exported():
    L = kv.lib()
    names = _declared()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
    assert sorted(kv.EXPORTS) == names


def test_single_hip_runtime_in_process():
    kv.lib()
    with open("/proc/self/maps") as f:
        paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    assert len(paths) == 1, paths


def test_strerror_covers_statuses():
    for st in (kv.KVOFF_OK, kv.KVOFF_EINVAL, kv.KVOFF_ENOMEM, kv.KVOFF_ENODEV, kv.KVOFF_EHIP,
               kv.KVOFF_ERANGE, kv.KVOFF_ESTATE):
        assert kv.kvoff_strerror(st) != "unknown status"
    assert kv.kvoff_strerror(-99) == "unknown status"


GOOD = dict(num_layers=1, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
            dtype=kv.KVOFF_F16, max_requests=1, host_capacity_blocks=16)


@pytest.mark.parametrize("bad", [
    dict(num_layers=0), dict(num_q_heads=6), dict(num_q_heads=96, num_kv_heads=2),
    dict(head_dim=64), dict(block_size=8), dict(dtype=3), dict(max_requests=0),
    dict(host_capacity_blocks=0), dict(host_mem_kind=5),
])
def test_create_rejects_bad_config(bad):
    with pytest.raises(kv.KvoffError) as e:
        kv.kvoff_create(**{**GOOD, **bad})
    assert e.value.status == kv.KVOFF_EINVAL


def test_create_without_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    with pytest.raises(kv.KvoffError) as e:
        kv.kvoff_create(**GOOD)
    assert e.value.status == kv.KVOFF_ENODEV


def test_null_context_is_rejected():
    assert kv.lib().kvoff_destroy(None) == kv.KVOFF_OK
    assert kv.lib().kvoff_register_request(None, 10, None) == kv.KVOFF_EINVAL
    assert kv.lib().kvoff_step(None, None) == kv.KVOFF_EINVAL
    assert kv.kvoff_workspace_size(None, kv.KVOFF_CALL_SPARSE_DECODE, 1, 1, 0) == 0
    assert kv.lib().kvoff_set_kernel_timing(None, 1) == kv.KVOFF_EINVAL
    assert kv.lib().kvoff_get_kernel_times(None, None) == kv.KVOFF_EINVAL


def test_c_program_compiles_and_links_against_the_abi(tmp_path):
    """include/kvoff.h is valid C and a C program links libkvoff.so alone."""
    from tests import cabi
    exe = cabi.build(str(tmp_path))
    assert os.path.exists(exe)
