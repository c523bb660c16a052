"""path_decode_step_noalloc: the decode step with its split partials in the library's fixed scratch array.

Host checks (no GPU): the entry point is exported, reports its scratch size, and rejects a problem whose
partials do not fit with PATH_ERR_SCRATCH before touching the device.  GPU checks: through the C ABI, two
calls in a row (the second smaller, so it runs over what the first left in the scratch array) give
bit-identical outputs, log-sum-exps and updated caches to path_decode_step on copies of the same caches.
"""
import ctypes

import numpy as np
import pytest
import torch

from dependent_positional_attention_amd import native, synth
from tests.gpu_util import dev, dev_f32

FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: validation fails first


def test_noalloc_scratch_size_and_limit():
    L = native.lib()
    assert native.path_decode_noalloc_scratch_bytes() == 32 << 20
    # batch 32, 24 heads, d = 128, a 1M-slot cache: 1024 splits of partials need 409 MB > 32 MiB
    cap = 1 << 20
    st = L.path_decode_step_noalloc(FAKE, FAKE, None, cap, cap - 1, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                    None, 32, 24, 128, 0.1, 1, 0, None)
    assert st == native.PATH_ERR_SCRATCH
    assert b"scratch" in L.path_status_string(st)
    # the same call at a size that fits would go on to the device; a bad argument is still caught first
    assert L.path_decode_step_noalloc(FAKE, FAKE, None, 100, 100, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                      None, 1, 1, 64, 0.1, 1, 0, None) == native.PATH_ERR_INVALID_ARG
    assert L.path_decode_step_noalloc(FAKE, FAKE, None, 100, 5, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                      None, 1, 1, 48, 0.1, 1, 0, None) == native.PATH_ERR_UNSUPPORTED


def _case(B, H, T0, d, fox, seed):
    ck, cv = synth.make_decode_cache(B, H, T0, d, dtype="bf16", seed=seed)
    st = synth.make_decode_steps(1, B, H, d, dtype="bf16", seed=seed)
    cap = T0 + 4
    kc = torch.zeros((B, H, cap, d), device="cuda", dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    kc[:, :, :T0] = dev(ck, "bf16")
    vc[:, :, :T0] = dev(cv, "bf16")
    fc = f_t = None
    if fox:
        rng = np.random.default_rng(seed)
        fc = torch.from_numpy(rng.normal(-1.0, 0.5, (B, H, cap)).astype(np.float32)).cuda()
        f_t = torch.from_numpy(rng.normal(-0.05, 0.02, (B, H)).astype(np.float32)).cuda()
    args = [dev(st.q[0], "bf16"), dev(st.k[0], "bf16"), dev(st.v[0], "bf16"), dev(st.w[0], "bf16"),
            dev_f32(st.beta[0])]
    return kc, vc, fc, f_t, args, st.scale


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point_twice():
    cases = [(2, 3, 3000, 64, True, 5), (1, 2, 500, 64, False, 6)]  # the second call is smaller
    for B, H, T0, d, fox, seed in cases:
        print(f"[case] noalloc decode B={B} H={H} T0={T0} d={d} fox={fox}", flush=True)
        kc, vc, fc, f_t, args, scale = _case(B, H, T0, d, fox, seed)
        kc2, vc2 = kc.clone(), vc.clone()
        fc2 = None if fc is None else fc.clone()
        o1, l1 = native.path_decode_step(kc, vc, T0, *args, f_t, fcache=fc, scale=scale)
        o2 = torch.empty_like(o1)
        l2 = torch.empty_like(l1)
        native.path_decode_step_noalloc(kc2, vc2, T0, *args, f_t, fcache=fc2, scale=scale, out=o2, lse=l2)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "out differs"
        assert torch.equal(l1, l2), "lse differs"
        assert torch.equal(kc.view(torch.int16), kc2.view(torch.int16)), "key cache differs"
        assert torch.equal(vc.view(torch.int16), vc2.view(torch.int16)), "value cache differs"
        if fc is not None:
            assert torch.equal(fc, fc2), "FoX slot biases differ"
        assert torch.isfinite(o2.float()).all()
