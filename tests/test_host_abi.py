"""Host-side checks of libmok that need no GPU: the library loads, exports every function the
header declares, validates descriptors, sizes buffers from host-known bounds, and reproduces
the pages' two-wave minibatch floor."""
import ctypes
import os
import re

import pytest

import combine_router_top_schedule_amd as mok

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mok.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mok_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert "mok_layer_fwd" in names and "mok_layer_bwd" in names and len(names) >= 13
    lib = ctypes.CDLL(mok.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    # and the binding knows every one of them
    assert set(names) <= set(mok._SIGS)


def test_abi_version_and_status_strings():
    assert mok.abi_version() == 5
    for code in range(11):
        assert mok.lib().mok_status_str(code)


def _d(**kw):
    base = dict(H=7168, E=256, K=8, I=2048, S=64, T=2048, e0=0, E_loc=4, M=2368,
                ring_bytes=256 << 20)
    base.update(kw)
    return mok.desc(**base)


@pytest.mark.parametrize("bad", [dict(H=7100), dict(I=100), dict(K=0), dict(K=17),
                                 dict(E=4, K=8), dict(e0=254, E_loc=4), dict(E_loc=0),
                                 dict(E_loc=65, E=256), dict(M=-1), dict(M=100, dtype="mxfp8"), dict(S=0), dict(E=2000),
                                 dict(S=100000, T=2048)])
def test_descriptor_validation(bad):
    with pytest.raises(mok.MokError) as ei:
        mok.query_sizes(_d(**bad))
    assert ei.value.code == 2


def test_dtype_validation():
    d = _d()
    d.dtype = 7
    with pytest.raises(mok.MokError) as ei:
        mok.query_sizes(d)
    assert ei.value.code == 3


def test_sizes_follow_host_bounds():
    s = mok.query_sizes(_d())
    N = 64 * 2048
    assert s.rows_max == N * 4                                # N * min(K, E_loc)
    assert s.slots_bytes >= N * 8 * 7168 * 2                  # Z: [N*K][H] BF16
    assert s.xd_bytes >= s.rows_max * 7168 * 2
    # the ring is split into 8 per-XCD shares; each holds 3 gather slots (X of 256 rows), 3 h
    # slots (h of 256 rows) and then as many activation slots (g|u of 256 rows) as fit: at the
    # DeepSeek-V3 shape 9 per XCD, more than the ~69 row tiles of the layer
    share = (256 << 20) // 8
    assert s.x_slot_bytes == 256 * 7168 * 2
    assert s.h_slot_bytes == 256 * 2048 * 2
    assert s.slot_bytes == 256 * 2 * 2048 * 2
    assert s.ring_slots == 8 * ((share - 3 * s.x_slot_bytes - 3 * s.h_slot_bytes)
                                // s.slot_bytes) == 72
    assert s.ring_min_bytes == 8 * (3 * s.x_slot_bytes + 3 * s.h_slot_bytes + 2 * s.slot_bytes)
    sm = mok.query_sizes(_d(dtype="mxfp8"))
    assert sm.rows_max == N * 4 + 4 * 31                      # per-expert padding to 32 rows
    assert sm.x_slot_bytes == 256 * (7168 + 7168 // 32)       # E4M3 codes + UE8M0 scales
    assert sm.h_slot_bytes == 256 * (2048 + 2048 // 32)
    assert sm.slot_bytes == 256 * 2 * 2048 * 2                # g|u stays BF16
    assert sm.ring_slots == 8 * ((share - 3 * sm.x_slot_bytes - 3 * sm.h_slot_bytes)
                                 // sm.slot_bytes)
    # packed weights: gate/up (2 E_loc I H), Wd, Wd^T, [Wg^T | Wu^T] (2 E_loc H I) values (BF16)
    # or codes and scales (MXFP8); the workspace has room to pack them per call
    m = 4 * 7168 * 2048
    assert s.packed_bytes == 6 * m * 2
    assert sm.packed_bytes == 6 * m + 6 * m // 32
    assert s.ws_bytes >= s.packed_bytes and s.bwd_ws_bytes >= s.ws_bytes
    assert sm.ws_bytes >= sm.packed_bytes
    # null arguments are rejected before anything runs
    assert mok.lib().mok_schedule(ctypes.byref(_d()), None, None, None, None, None, None) == 1
    w = mok.MokWeights()
    assert mok.lib().mok_pack_weights(ctypes.byref(_d()), ctypes.byref(w), None, None) == 1
    # MXFP8 needs the quantised codes and scales
    assert mok.lib().mok_pack_weights(ctypes.byref(_d(dtype="mxfp8")), ctypes.byref(w), 256,
                                      None) == 3


def test_two_wave_floor_matches_pages_figure():
    # The pages' 2,368-token floor for Kimi-2.5 shapes (intermediate 2048) is two waves of
    # 128 x 256 tiles over 148 compute units; the formula reproduces it exactly.
    assert mok.two_wave_floor(148, 128, 256, 2048) == 2368
    # MI355X, 256 CUs: 256 x 256 tiles -> 8192 tokens; 128 x 128 -> 2048.
    assert mok.two_wave_floor(256, 256, 256, 2048) == 8192
    assert mok.two_wave_floor(256, 128, 128, 2048) == 2048


def test_measurement_hook_kernel_ids():
    # fused forward, the two backward GEMM launches, the dispatch gather and the merge;
    # null events switch the hook off
    for k in range(6):
        mok.mok_trace_kernel(k)
    with pytest.raises(mok.MokError):
        mok.mok_trace_kernel(6)
