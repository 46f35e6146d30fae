"""cad_span_forward_noalloc against cad_span_forward: the same kernels, with the workspace taken
from the library's static device array instead of a caller buffer, so every output must be
bit-identical.  Two calls in a row, the second with a smaller input (the array keeps the first
call's contents), then a forward too large for the array, which must be refused."""
import ctypes

import numpy as np
import pytest
import torch

from spec_verify_cad_amd import cad, synth
from spec_verify_cad_amd.configs import QWEN15, SMALL

from gpu_util import log, prefill

pytestmark = pytest.mark.gpu


def _noalloc(layer, cache, tokens, Nq, mode=cad.MASK_CAUSAL, W=1, D=1, flags=0, argmax_out=None, hidden_out=None,
             logits_out=None, top2_gap=None):
    """The C-ABI call itself (ctypes), returning its status."""
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    return cad.lib().cad_span_forward_noalloc(ctypes.byref(layer.desc), ctypes.byref(cache.desc), p(tokens), cache.B,
                                              Nq, mode, W, D, flags, p(argmax_out), p(hidden_out), p(logits_out),
                                              p(top2_gap), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _outputs(shape, R, M):
    return (torch.full((R,), -7, dtype=torch.int32, device="cuda"),
            torch.zeros((M, shape.hidden), dtype=torch.int16, device="cuda"),
            torch.zeros((R, shape.vocab), dtype=torch.float32, device="cuda"),
            torch.zeros((R,), dtype=torch.float32, device="cuda"))


def _pair(layer, caches, L0, toks, mode=cad.MASK_CAUSAL, W=1, D=1, flags=cad.COMMIT_ALL):
    """The same forward through both entry points from identical caches; every output, the cache
    rows and the lengths must agree bit for bit."""
    B, Nq = toks.shape
    s = layer.shape
    R = B if flags & cad.LOGITS_LAST else B * Nq
    t = torch.from_numpy(np.ascontiguousarray(toks, dtype=np.int32)).cuda()
    outs = []
    for i, c in enumerate(caches):
        c.len.fill_(L0)
        a, h, lg, gp = _outputs(s, R, B * Nq)
        if i == 0:
            cad.span_forward(layer, c, t, Nq, mode, W, D, flags, a, h, lg, top2_gap=gp)
        else:
            assert _noalloc(layer, c, t, Nq, mode, W, D, flags, a, h, lg, gp) == cad.CAD_OK
        outs.append((a, h, lg, gp))
    torch.cuda.synchronize()
    for x, y in zip(*outs):
        assert torch.equal(x, y)
    assert torch.equal(caches[0].len, caches[1].len)
    assert torch.equal(caches[0].k, caches[1].k) and torch.equal(caches[0].v, caches[1].v)


@pytest.mark.parametrize("shape", [SMALL, QWEN15], ids=["small", "1.5b"])
def test_noalloc_forward_equals_the_workspace_forward(shape):
    log(f"no-alloc forward, {shape.hidden} hidden")
    w = synth.layer_weights(shape, 61)
    layer = cad.DeviceLayer(shape, w)
    B, L0 = 2, 300
    cap = L0 + 80
    ctx = np.stack([synth.uniform_tokens(62 + b, L0, shape.vocab) for b in range(B)])
    caches = [cad.DeviceCache(shape, B, cap) for _ in range(2)]
    for c in caches:
        prefill(layer, c, ctx, chunk=128)
    big = np.stack([synth.uniform_tokens(70 + b, 32, shape.vocab) for b in range(B)])
    small = big[:, :5]
    _pair(layer, caches, L0, big)                                   # first call: 64 rows
    _pair(layer, caches, L0, small)                                 # second call, smaller: 10 rows
    _pair(layer, caches, L0, big[:, :24], mode=cad.MASK_BLOCK, W=3, D=8, flags=0)
    _pair(layer, caches, L0, big[:, :13], flags=cad.COMMIT_ALL | cad.LOGITS_LAST)
    # a forward whose workspace exceeds the array is refused and enqueues nothing
    t = torch.from_numpy(np.ascontiguousarray(np.tile(big, (1, 2)), dtype=np.int32)).cuda()
    need = cad.span_forward_workspace(layer, B, 64, cad.MASK_CAUSAL, 1, 1, cap, cad.COMMIT_ALL)
    caches[1].len.fill_(L0)
    a, h, lg, gp = _outputs(shape, B * 64, B * 64)
    st = _noalloc(layer, caches[1], t, 64, flags=cad.COMMIT_ALL, argmax_out=a)
    torch.cuda.synchronize()
    if need > cad.NOALLOC_SCRATCH_BYTES:
        assert st == cad.CAD_EWORKSPACE and int(caches[1].len[0]) == L0
    else:
        assert st == cad.CAD_OK
