"""The allocation-free draft step (mtp_draft_step_noalloc, the library's static
scratch) against mtp_draft_step with a caller's workspace: the same kernels on
the same inputs, so ids, hidden rows, logits and the appended cache rows must
agree bit for bit.  Two calls in a row share the one static array; the second
is smaller (one row, a shorter cache) and runs on what the first left there.
"""
import sys

import numpy as np
import pytest

from mtp_speculative_draft_amd import synth

torch = pytest.importorskip("torch")
import mtp_speculative_draft_amd as mtp  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _bits(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy().view(np.uint32)


def _both(dl, S, e, tokens, table, h, cache_len, m):
    """One call of each entry point on its own copy of the caches; returns the
    outputs of both (noalloc first, so it runs on the scratch as the previous
    call left it)."""
    V, H = S.layer.vocab, S.layer.hidden
    out = []
    for noalloc in (True, False):
        kc, vc = _t(S.k_cache), _t(S.v_cache)
        ids = torch.full((m,), -7, dtype=torch.int32, device=DEV)
        hid = torch.full((m, H), float("nan"), dtype=torch.float32, device=DEV)
        lg = torch.full((m, V), float("nan"), dtype=torch.float32, device=DEV)
        if noalloc:
            mtp.mtp_draft_step_noalloc(dl, e, tokens, table, h, kc, vc, cache_len, ids, hid, lg)
        else:
            mtp.mtp_draft_step(dl, e, tokens, table, h, kc, vc, cache_len, ids_out=ids, hidden_out=hid, logits_out=lg)
        rows = slice(cache_len, cache_len + m)
        out.append((_bits(ids), _bits(hid), _bits(lg), _bits(kc[:, rows]), _bits(vc[:, rows])))
        del kc, vc
    return out


def _same(a, b, what):
    for name, x, y in zip(("ids", "hidden", "logits", "k rows", "v rows"), a, b):
        assert x.shape == y.shape, (what, name)
        assert np.array_equal(x, y), f"{what}: {name} differ at {int(np.count_nonzero(x != y))} places"


def test_noalloc_draft_step_equals_the_workspace_call_twice_in_a_row():
    S = synth.config4_step()
    L = S.layer
    dl = mtp.DeviceLayer(L)
    table = _t(S.table)
    H = L.hidden
    # first call: the verify shape at full size (4 rows, cache 4096)
    m1, c1 = 4, S.cache_len
    need1 = mtp.mtp_draft_step_workspace_size(dl, c1, m1)
    _say(f"noalloc call 1: m={m1} cache_len={c1} hidden={H} vocab={L.vocab} workspace {need1} B")
    assert 0 < need1 <= mtp.MTP_NOALLOC_SCRATCH_BYTES
    g = synth.rng(4242)
    toks = torch.from_numpy(g.integers(0, L.vocab, size=m1).astype(np.int32)).to(DEV)
    h4 = _t(synth.normal(g, (m1, H)))
    e4 = _t(np.repeat(S.e0, m1, axis=0))
    a, b = _both(dl, S, e4, toks, table, h4, c1, m1)
    _same(a, b, "call 1")
    _say(f"  call 1 ids {a[0].view(np.int32).tolist()}")
    # second call, smaller: one row over a shorter cache, no token (e row)
    m2, c2 = 1, 1000
    need2 = mtp.mtp_draft_step_workspace_size(dl, c2, m2)
    _say(f"noalloc call 2: m={m2} cache_len={c2} workspace {need2} B")
    assert need2 < need1
    h1 = _t(synth.normal(g, (m2, H)))
    e1 = _t(synth.normal(g, (m2, H)))
    a, b = _both(dl, S, e1, None, table, h1, c2, m2)
    _same(a, b, "call 2")
    _say(f"  call 2 ids {a[0].view(np.int32).tolist()}")
    assert (a[0].view(np.int32) >= 0).all() and (a[0].view(np.int32) < L.vocab).all()
