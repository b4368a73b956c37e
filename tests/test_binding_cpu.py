"""The Python binding has no CPU path: every entry point refuses host tensors with an error
instead of computing anything (CPU only; the library loads without a GPU)."""
import pytest
import torch

import fp8_mla_split_amd as mla


def _cpu(*shape, dtype=torch.float32):
    return torch.zeros(shape, dtype=dtype)


def test_every_entry_point_refuses_host_tensors():
    q8 = _cpu(1, 1, 16, 576, dtype=torch.uint8)
    pool = _cpu(1, 64, 576, dtype=torch.uint8)
    table = _cpu(1, 1, dtype=torch.int32)
    lens = _cpu(1, dtype=torch.int32)
    po = _cpu(1, 4, 16, 512, dtype=torch.float16)
    pl = _cpu(1, 4, 16)
    calls = [
        lambda: mla.quantize_fp8_sat(_cpu(64), 1.0),
        lambda: mla.quantize_fp8_sat_dynamic(_cpu(64)),
        lambda: mla.quantize_fp8_sat_dynamic(_cpu(64, dtype=torch.bfloat16)),
        lambda: mla.kv_append_fp8_sat(_cpu(1, 1, 576), pool, table, lens, 1.0),
        lambda: mla.decode_splitkv(q8, pool, table, lens, 1.0, 1.0, 0.07, 64, 4, 0),
        lambda: mla.splitkv_combine(po, pl, 1, 16, 1.0),
        lambda: mla.splitkv_combine_partial(po, pl, 1, 16, _cpu(1, 16, 512,
                                                                dtype=torch.float16),
                                            _cpu(1, 16)),
    ]
    for call in calls:
        with pytest.raises(ValueError):
            call()


def test_status_codes_are_named():
    assert mla.status_string(0) == "MLA_OK"
    assert mla.status_string(3) == "MLA_ERR_WORKSPACE"
    err = mla.MLAError(2, "where")
    assert "MLA_ERR_UNSUPPORTED" in str(err) and err.code == 2
