"""GPU parity of attn_decode_paged_noalloc (the entry point that allocates
nothing: its split partials live in the library's static per-device array)
against attn_decode_paged with a caller workspace, through the C ABI: two calls
in a row, the second with a smaller input, each bit for bit equal to the
workspace entry point on the same inputs and within the oracle's tolerance.
"""
import sys

import numpy as np
import pytest

import oracle
from synth import gen
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _run_pair(ea, p):
    t = gu.torch()
    q = gu.dev(p.q, "bf16")
    kc, vc = gu.dev(p.k_cache, "bf16"), gu.dev(p.v_cache, "bf16")
    bt, sl = gu.dev(p.block_table, "i32"), gu.dev(p.seq_lens, "i32")
    o1, o2 = gu.empty_out(q.shape, "bf16"), gu.empty_out(q.shape, "bf16")
    l1 = t.empty((p.B, p.A), dtype=t.float32, device="cuda")
    l2 = t.empty_like(l1)
    for x in (o1, o2, l1, l2):
        x.fill_(float("nan"))
    nb = ea.attn_decode_paged_workspace_bytes(p.B, p.A, p.A_kv, p.d, p.page_size, p.seq_lens)
    assert 0 < nb <= ea.DECODE_NOALLOC_MAX_BYTES
    ws = t.empty(nb, dtype=t.uint8, device="cuda")
    ea.attn_decode_paged(q, kc, vc, bt, sl, p.seq_lens, o1, l1, ws, scale=p.scale)
    ea.attn_decode_paged_noalloc(q, kc, vc, bt, sl, p.seq_lens, o2, l2, scale=p.scale)
    t.cuda.synchronize()
    return (gu.host_f64(o1), l1.cpu().numpy().astype(np.float64), gu.host_f64(o2),
            l2.cpu().numpy().astype(np.float64), (o1, o2, l1, l2))


def test_noalloc_decode_matches_workspace_entry_point():
    import exact_attention_108_amd as ea
    t = gu.torch()
    orc = oracle.default()
    cases = [
        # lens, A, A_kv, d, page_size: the second call is smaller
        ([3000, 17, 900, 5000, 1, 2048, 700, 64, 0, 4100, 333, 1024], 32, 8, 128, 16),
        ([130, 5, 600], 8, 2, 64, 32),
    ]
    for n, (lens, A, A_kv, d, ps) in enumerate(cases):
        _say("noalloc decode", n, lens, A, A_kv, d, ps)
        p = gen.make_paged(lens, A, A_kv, d, ps, dtype="bf16", seed=1500 + n, extra_pages=2)
        o1, l1, o2, l2, tens = _run_pair(ea, p)
        assert t.equal(tens[0].view(t.int16), tens[1].view(t.int16)) and t.equal(tens[2], tens[3]), n
        o_ref, l_ref = orc.decode_paged(p.q, p.k_cache, p.v_cache, p.block_table, p.seq_lens, dtype="bf16",
                                        scale=p.scale)
        _say(gu.check(o2, l2, o_ref, l_ref, "bf16", f"noalloc decode {n}"))
