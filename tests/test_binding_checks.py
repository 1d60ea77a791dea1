"""The Python binding checks every caller-supplied output buffer before it
hands a raw pointer to the library (the kernels write through it, so a buffer
of the wrong size, type, device or stride would be written out of bounds).
These tests run the binding's checks on CPU tensors: no library call and no
launch is reached."""
import pytest
import torch

vsa = pytest.importorskip("block_sparse_attention_19_amd")

CPU = torch.device("cpu")


def test_out_accepts_exact_buffer_and_none():
    t = torch.empty((2, 3, 4), dtype=torch.bfloat16)
    assert vsa._out(t, (2, 3, 4), torch.bfloat16, CPU, "out") is t
    assert vsa._out(None, (2, 3, 4), torch.bfloat16, CPU, "out") is None


@pytest.mark.parametrize("make, msg", [
    (lambda: torch.empty((2, 3, 5), dtype=torch.bfloat16), "shape"),
    (lambda: torch.empty((2, 3), dtype=torch.bfloat16), "shape"),
    (lambda: torch.empty((2, 3, 4), dtype=torch.float32), "bfloat16"),
    (lambda: torch.empty((2, 4, 3), dtype=torch.bfloat16).transpose(1, 2), "contiguous"),
    (lambda: torch.empty((2, 3, 4), dtype=torch.bfloat16, device="meta"), "meta"),
    (lambda: [0.0] * 24, "tensor"),
])
def test_out_rejects(make, msg):
    with pytest.raises(ValueError, match=msg):
        vsa._out(make(), (2, 3, 4), torch.bfloat16, CPU, "out")


def test_attn_outputs_checks_out_and_lse():
    o_shape, l_shape = (1, 2, 128, 64), (1, 2, 128)
    out, lse = vsa._attn_outputs(None, None, True, o_shape, l_shape, CPU)
    assert out.shape == o_shape and out.dtype == torch.bfloat16
    assert lse.shape == l_shape and lse.dtype == torch.float32
    out, lse = vsa._attn_outputs(None, None, False, o_shape, l_shape, CPU)
    assert lse is None
    with pytest.raises(ValueError, match="lse_out"):
        vsa._attn_outputs(None, torch.empty((1, 2, 127), dtype=torch.float32), True,
                          o_shape, l_shape, CPU)
    with pytest.raises(ValueError, match="lse_out"):
        vsa._attn_outputs(None, torch.empty(l_shape, dtype=torch.float16), True,
                          o_shape, l_shape, CPU)
    with pytest.raises(ValueError, match="out"):
        vsa._attn_outputs(torch.empty((1, 2, 128, 128), dtype=torch.bfloat16), None, True,
                          o_shape, l_shape, CPU)


def test_workspace_checks():
    ws = torch.empty(1024, dtype=torch.uint8)
    assert vsa._workspace(ws, 512, CPU) is ws
    assert vsa._workspace(None, 512, CPU).numel() == 512
    assert vsa._workspace(torch.empty(16, dtype=torch.uint8), 512, CPU).numel() == 512
    with pytest.raises(ValueError, match="workspace"):
        vsa._workspace(torch.empty(1024, dtype=torch.int32), 512, CPU)
    with pytest.raises(ValueError, match="workspace"):
        vsa._workspace(torch.empty(2048, dtype=torch.uint8)[::2], 512, CPU)


def test_overlap():
    a = torch.empty(100, dtype=torch.bfloat16)
    assert vsa._overlap(a, a)
    assert vsa._overlap(a[10:20], a[15:30])
    assert not vsa._overlap(a[:50], a[50:])


def test_inputs_must_be_device_tensors():
    s = vsa.shape(1, 2, 64, 8, 16, 16)
    x = torch.empty((1, 2048, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        vsa.tile_permute(x, s)
