"""mok_schedule_noalloc (the router with its scratch in the library's static per-device array)
against mok_schedule (the same kernels with a caller workspace), through the C ABI: two calls
in a row, the second on a smaller shape, each bit-identical in every output; and the host-side
rejection of a shape whose scratch exceeds the array."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import datagen

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import combine_router_top_schedule_amd as mok


def _outputs(d, logits, noalloc):
    s = mok.query_sizes(d)
    N, K = d.num_segments * d.tokens_per_segment, d.top_k
    idx = torch.full((N * K,), -7, dtype=torch.int32, device="cuda")
    p = torch.full((N * K,), -7.0, dtype=torch.float32, device="cuda")
    saved = torch.zeros(int(s.saved_bytes), dtype=torch.uint8, device="cuda")
    if noalloc:
        mok.mok_schedule_noalloc(d, logits, idx, p, saved)
    else:
        ws = torch.zeros(int(s.ws_bytes), dtype=torch.uint8, device="cuda")
        mok.mok_schedule(d, logits, idx, p, saved, ws)
    torch.cuda.synchronize()
    return idx, p, saved


@pytest.mark.parametrize("order", ["big_then_small"])
def test_schedule_noalloc_equals_schedule(order):
    cfgs = [datagen.CONFIGS["dsv3"], datagen.CONFIGS["tiny"].replace(S=3, T=100, e0=2, E_loc=3)]
    for cfg in cfgs:
        d = mok.desc_from_config(cfg)
        logits = torch.from_numpy(datagen.logits(cfg)).cuda()
        ref = _outputs(d, logits, noalloc=False)
        got = _outputs(d, logits, noalloc=True)
        for a, b in zip(ref, got):
            assert torch.equal(a, b), cfg.name
        hdr = got[2][:1024].view(torch.int32).cpu().numpy()
        assert hdr[4] == 0                      # the router's device-side status
        assert hdr[0] > 0 and hdr[2] > 0        # pairs and touched tokens were counted
        print(f"  {cfg.name}: N={cfg.N} P={hdr[0]} U={hdr[2]} identical")


def test_schedule_noalloc_rejects_shapes_beyond_its_scratch():
    # 4,194,304 tokens with 64 local experts need 16384 * 66 * 4 bytes of scan state: more than
    # the 1 MiB array. The call is rejected on the host before anything is launched, so the
    # small placeholder buffers are never touched.
    d = mok.desc(128, 256, 2, 128, 2048, 2048, 0, 64)
    buf = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    f = torch.zeros(256, dtype=torch.float32, device="cuda")
    i = torch.zeros(256, dtype=torch.int32, device="cuda")
    rc = mok.lib().mok_schedule_noalloc(ctypes.byref(d), f.data_ptr(), i.data_ptr(), f.data_ptr(),
                                       buf.data_ptr(), None)
    assert rc == 10 and mok.lib().mok_status_str(rc)
