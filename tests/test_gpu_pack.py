"""The packed weight layout of the projections (include/mla_decode.h,
mla_pack_weight), bit for bit against its definition written with numpy
reshapes, and the argument checks of the entry point.

The layout: the 1 KB block of column tile ct and k-step ks sits at byte
(ks * n/32 + ct) * 1024, and its 16-byte lane piece l holds
W[32 ct + l % 32][16 ks + 8 (l / 32) .. + 7].
"""

import numpy as np
import pytest

from tests.parity import say

pytestmark = pytest.mark.gpu


def packed_reference(w):
    """[n, k] -> flat packed order: [ks][ct][h][n % 32][8] with lane = n % 32 + 32 h."""
    n, k = w.shape
    t = w.reshape(n // 32, 32, k // 16, 2, 8)          # [ct][row][ks][h][e]
    return np.ascontiguousarray(t.transpose(2, 0, 3, 1, 4)).reshape(-1)


def test_reference_layout_by_hand():
    """The numpy definition against the stated formula, element by element."""
    n, k = 64, 48
    w = np.arange(n * k, dtype=np.int64).reshape(n, k)
    p = packed_reference(w)
    for ks in range(k // 16):
        for ct in range(n // 32):
            for lane in range(64):
                base = ((ks * (n // 32) + ct) * 64 + lane) * 8
                row, col = 32 * ct + lane % 32, 16 * ks + 8 * (lane // 32)
                assert list(p[base:base + 8]) == list(w[row, col:col + 8])


@pytest.mark.parametrize("n,k", [(32, 16), (64, 48), (576, 7168), (1536, 7168), (24576, 1536),
                                 (7168, 16384)])
def test_pack_weight_bit_exact(n, k):
    import torch
    from mla_latent_kv_amd import binding
    say(f"case pack {n}x{k}")
    g = torch.Generator(device="cpu").manual_seed(n + k)
    w = torch.randint(-32768, 32768, (n, k), generator=g, dtype=torch.int32).to(torch.int16)
    dec = binding.MLADecoder(0, max_q_tokens=2)
    p = dec.pack(w.cuda())
    torch.cuda.synchronize()
    got = p.cpu().numpy()
    dec.close()
    np.testing.assert_array_equal(got, packed_reference(w.numpy()))


def test_pack_weight_rejects_bad_shapes_and_overlap():
    import ctypes
    import torch
    from mla_latent_kv_amd import binding
    lib = binding.load_library()
    dec = binding.MLADecoder(0, max_q_tokens=2)
    w = torch.zeros(64 * 64, dtype=torch.int16, device="cuda")
    out = torch.zeros(64 * 64, dtype=torch.int16, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for n, k in ((33, 64), (64, 24), (0, 64), (64, 0)):
        assert lib.mla_pack_weight(dec.ctx, w.data_ptr(), out.data_ptr(), n, k, s) == -1, (n, k)
    assert lib.mla_pack_weight(dec.ctx, w.data_ptr(), w.data_ptr(), 64, 64, s) == -1
    assert lib.mla_pack_weight(dec.ctx, w.data_ptr(), w.data_ptr() + 1024, 32, 32, s) == -1
    assert lib.mla_pack_weight(dec.ctx, w.data_ptr() + 2, out.data_ptr(), 32, 32, s) == -3
    assert lib.mla_pack_weight(dec.ctx, w.data_ptr(), out.data_ptr(), 64, 64, s) == 0
    torch.cuda.synchronize()
    dec.close()
