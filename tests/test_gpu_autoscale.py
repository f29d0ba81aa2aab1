"""GPU parity of pa_cache_write_autoscale: codes and scales bit-exact against
oracle.cache_write_autoscale_ref over a prefill of whole and partial blocks
followed by decode appends, some of which grow a block's scale."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import log

pytestmark = pytest.mark.gpu
pa = pytest.importorskip("paged_kv_cache_272_amd")


def _src(rng, shape, kind, mult):
    x = (rng.standard_normal(shape) * mult).astype(np.float32)
    if kind == "bf16":
        bits = (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        return bits, torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return x, torch.from_numpy(x).cuda()


@pytest.mark.parametrize("kv,src,hkv", [("fp8", "bf16", 8), ("fp8", "f32", 2), ("int4", "bf16", 8),
                                        ("int4", "f32", 4)])
def test_autoscale_matches_oracle(kv, src, hkv):
    rng = np.random.default_rng(171)
    d, nb = 128, 24
    width = d if kv == "fp8" else d // 2
    k_host = np.zeros((nb, hkv, 16, width), np.uint8)
    v_host = np.zeros_like(k_host)
    ks_host = np.ones((nb, hkv), np.float32)
    vs_host = np.ones((nb, hkv), np.float32)
    dev = [torch.from_numpy(a.copy()).cuda() for a in (k_host, v_host, ks_host, vs_host)]
    # three sequences: prompts of 37, 16 and 5 tokens in scattered blocks, then 20 decode steps
    tables = [[3, 17, 9, 4], [11, 2, 14], [20, 6]]
    lens = [37, 16, 5]

    def slot(b, pos):
        return tables[b][pos // 16] * 16 + pos % 16

    steps = [[slot(b, p) for b in range(3) for p in range(lens[b])]]
    for it in range(20):
        steps.append([slot(b, lens[b] + it) for b in range(3)])
    for n, slots in enumerate(steps):
        mult = 1.0 if n == 0 else float(rng.choice([0.3, 1.0, 6.0]))
        kx, kt = _src(rng, (len(slots), hkv, d), src, mult)
        vx, vt = _src(rng, (len(slots), hkv, d), src, mult)
        sm = np.array(slots, np.int64)
        k_host, v_host, ks_host, vs_host = oracle.cache_write_autoscale_ref(k_host, v_host, ks_host, vs_host, kx,
                                                                            vx, sm, src, kv)
        pa.pa_cache_write_autoscale(kt, vt, dev[0], dev[1], dev[2], dev[3], torch.from_numpy(sm).cuda())
        torch.cuda.synchronize()
        for got, want in zip(dev, (k_host, v_host, ks_host, vs_host)):
            assert np.array_equal(got.cpu().numpy().view(np.uint8), want.view(np.uint8)), f"step {n}"
    log(f"autoscale {kv} from {src}: {len(steps)} calls bit-exact")
