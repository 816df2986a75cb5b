"""The streaming-read probe (a measurement aid beside the decode path): it
reads the buffer, writes nothing for ordinary data, and rejects bad
arguments before any launch."""

import pytest

pytestmark = pytest.mark.gpu


def test_read_probe_runs_and_writes_nothing_for_ordinary_data():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from split_kv_flash_amd import SplitKVError, binding

    buf = torch.ones(1 << 24, dtype=torch.float32, device="cuda")  # 64 MiB
    scratch = torch.full((1024,), 7.0, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    binding.attn_decode_read_probe(buf, buf.numel() * 4, 1024, scratch, s)
    torch.cuda.synchronize()
    assert torch.all(scratch == 7.0)
    with pytest.raises(SplitKVError):
        binding.attn_decode_read_probe(buf, 16, 1024, scratch, s)
