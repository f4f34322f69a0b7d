"""The GPU fill kernels give the same bits as the numpy generator (the two
sides of every parity test start from identical inputs)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind,dt,npdt", [
    (synth.KIND_BF16_NORMAL12, torch.int16, np.uint16),
    (synth.KIND_BF16_NORMAL6, torch.int16, np.uint16),
    (synth.KIND_BF16_WIDE, torch.int16, np.uint16),
    (synth.KIND_F32_UNIT, torch.float32, np.uint32),
    (synth.KIND_I8_NORMAL, torch.int8, np.int8),
    (synth.KIND_F32_SCALE, torch.float32, np.uint32),
])
@pytest.mark.parametrize("offset", [0, 3, (1 << 33) + 5])
def test_fill_matches_numpy(kind, dt, npdt, offset):
    n = 100_003
    t = torch.empty(n, dtype=dt, device="cuda:0")
    synth.fill_gpu(kind, 0x1234_5678_9ABC_DEF0, 9, t, offset=offset)
    torch.cuda.synchronize()
    got = t.cpu().numpy().view(npdt)
    want = synth.tensor(kind, 0x1234_5678_9ABC_DEF0, 9, n, offset=offset).view(npdt)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("kind", [synth.KIND_MXFP4, synth.KIND_MXFP4_WIDE])
@pytest.mark.parametrize("d,offset", [(128, 0), (2560, 3), (2560, 1360 * 7 + 5)])
def test_mxfp4_fill_matches_numpy(kind, d, offset):
    rb = synth.mxfp4_row_bytes(d)
    nrows = 37
    t = torch.empty(nrows * rb, dtype=torch.uint8, device="cuda:0")
    synth.fill_gpu_mxfp4(kind, 0xABCDEF, 3, t, d, offset=offset)
    torch.cuda.synchronize()
    e = np.arange(offset, offset + nrows * rb, dtype=np.uint64)
    want = synth.mxfp4_bytes(kind, synth.words(0xABCDEF, 3, e), e % np.uint64(rb), d)
    assert np.array_equal(t.cpu().numpy(), want)
