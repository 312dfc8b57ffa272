"""moeq_expert_ffn_noalloc (working memory in the library's fixed device
array) against moeq_expert_ffn with a caller workspace, through the C ABI:
two calls in a row, the second with fewer tokens, each bit for bit equal
to the workspace call; and a call that needs more than the array holds is
rejected before anything is enqueued."""

import ctypes

import numpy as np
import pytest

from synth import configs, gen
from tests import layers

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _noalloc(lib, dev, x, rt, n_comp, opts):
    from bit_quantized_moe_token_amd import _lib
    y = torch.empty((rt.T, dev.H), dtype=torch.float32, device="cuda")
    st = lib.moeq_expert_ffn_noalloc(dev.handle, ctypes.c_void_p(x.data_ptr()), rt.T, rt.k, ctypes.byref(rt.c),
                                     n_comp, ctypes.c_void_p(y.data_ptr()), _lib.F32, ctypes.byref(opts),
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, y


def test_noalloc_matches_workspace_call():
    from bit_quantized_moe_token_amd import _lib, moeq
    lib = _lib.lib()
    cfg = configs.reduced(configs.get("decode"), H=512, I=1792, T=40)
    orc = layers.oracle_layer(cfg, 0, cache_blocks=3 * cfg["E"])
    dev = layers.device_layer(cfg, 0, orc)
    x = gen.gen_x(cfg, 0)
    logits = gen.gen_logits(cfg, 0)
    opts = _lib.FfnOptions(0, 0)
    for T in (40, 9):                      # the second call is smaller
        xd = torch.from_numpy(x[:T].copy()).cuda()
        rt = moeq.route(torch.from_numpy(logits[:T].copy()).cuda(), cfg["k"])
        ref = moeq.expert_ffn(dev, xd, rt, cfg["n_comp"], out_dtype=torch.float32)
        st, y = _noalloc(lib, dev, xd, rt, cfg["n_comp"], opts)
        assert st == _lib.OK, lib.moeq_last_error()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"T={T}: no-allocation result differs from the workspace call"
        sub = dict(cfg, T=T)
        layers.check_y(y.cpu().numpy(), layers.oracle_y(orc, sub, x[:T], logits[:T], cfg["n_comp"]),
                       f"noalloc T={T}")


def test_noalloc_rejects_oversized_call():
    from bit_quantized_moe_token_amd import _lib, moeq
    lib = _lib.lib()
    cap = ctypes.c_size_t(0)
    assert lib.moeq_ffn_noalloc_max_bytes(ctypes.byref(cap)) == _lib.OK
    cfg = configs.reduced(configs.get("decode"), H=512, I=1792, T=16)
    orc = layers.oracle_layer(cfg, 0, cache_blocks=3 * cfg["E"])
    dev = layers.device_layer(cfg, 0, orc)
    # a batch whose workspace exceeds the fixed array (sized by the library)
    opts = _lib.FfnOptions(0, 0)
    T = 16
    while True:
        need = ctypes.c_size_t(0)
        assert lib.moeq_ffn_workspace_size(dev.handle, T, cfg["k"], ctypes.byref(opts), ctypes.byref(need)) == _lib.OK
        if need.value > cap.value:
            break
        T *= 2
    logits = torch.from_numpy(np.zeros((T, cfg["E"]), dtype=np.float32)).cuda()
    rt = moeq.route(logits, cfg["k"])
    xd = torch.zeros((T, cfg["H"]), dtype=torch.float16, device="cuda")
    st, _ = _noalloc(lib, dev, xd, rt, cfg["n_comp"], opts)
    assert st == _lib.ERR_WORKSPACE
    assert b"fixed device array" in lib.moeq_last_error()
