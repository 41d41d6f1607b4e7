"""Failure reporting and concurrency of the projection kernels whose
workgroups wait for each other (calls of more than 2,048 tokens at d = 5120,
every call at widths outside that family).

* A call whose bounded wait gives up must end normally and be reported by
  hc_workspace_status (forced from the host with hc_debug_force_timeout,
  which makes every exchange record look stale and bounds the waits to zero
  time); the workspace must serve the next call bit for bit as before.
* Calls issued on two streams at once, each with its own workspace (or the
  binding's per-stream default one), must give bitwise the results of the
  same calls run one after another.
Everything is called through the C-ABI (thin binding)."""
import pytest
import torch

import hyper_connection_residual_02_amd as hcl
from hyper_connection_residual_02_amd import inputs as hin

pytestmark = pytest.mark.gpu
DEV = "cuda"
TIMEOUT = -10


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hcl.load()
    yield
    hcl.debug_force_timeout(0)
    torch.cuda.synchronize()


def _inputs(d, n, seed):
    w = hin.Workload("robust", 1, n, 4, d, 0.007, 0.5, 2.0, 1.0)
    return hin.make_inputs(w, DEV, seed=seed)


def _fused(t, ws):
    return hcl.hc_fused_mix_pre(t["R"], t["W"], t["scale"], t["base"], want_pre=True, want_mixes=True,
                                workspace=ws)


def _same(a, b):
    for u, v in zip(a, b):
        iv = torch.int16 if u.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(u.view(iv), v.view(iv))


@pytest.mark.parametrize("d,n", [(5120, 5000), (64, 900)])
def test_forced_give_up_is_reported_and_the_workspace_recovers(d, n):
    t = _inputs(d, n, seed=21)
    ws = hcl.Workspace()
    ref = _fused(t, ws)
    torch.cuda.synchronize()
    assert ws.status() == 0
    hcl.debug_force_timeout(1)
    _fused(t, ws)
    torch.cuda.synchronize()              # every kernel of the failed call has ended
    assert ws.status(clear=False) == TIMEOUT
    assert ws.status() == TIMEOUT         # reported until cleared
    assert ws.status() == 0
    again = _fused(t, ws)
    torch.cuda.synchronize()
    assert ws.status() == 0
    _same(again, ref)
    with pytest.raises(hcl.HCError):
        hcl.debug_force_timeout(1)
        _fused(t, ws)
        torch.cuda.synchronize()
        hcl.check_workspace(ws)


def test_forced_give_up_of_the_no_alloc_call():
    t = _inputs(5120, 3000, seed=22)
    f = dict(dtype=torch.float32, device=DEV)
    out = dict(h=torch.empty(1, 3000, 5120, dtype=torch.bfloat16, device=DEV), post=torch.empty(1, 3000, 4, **f),
               comb=torch.empty(1, 3000, 4, 4, **f))
    hcl.noalloc_status()
    hcl.debug_force_timeout(1)
    hcl.hc_fused_mix_pre_noalloc(t["R"], t["W"], t["scale"], t["base"], out=out)
    torch.cuda.synchronize()
    assert hcl.noalloc_status() == TIMEOUT
    hcl.hc_fused_mix_pre_noalloc(t["R"], t["W"], t["scale"], t["base"], out=out)
    torch.cuda.synchronize()
    assert hcl.noalloc_status() == 0
    ref = _fused(t, hcl.Workspace())
    torch.cuda.synchronize()
    _same((out["h"], out["post"], out["comb"]), (ref[0], ref[2], ref[3]))


def test_short_calls_never_wait_so_never_give_up():
    # calls of at most 2,048 tokens at d = 5120 have no waits between
    # workgroups: a pending forced give-up is not consumed by them
    t = _inputs(5120, 100, seed=23)
    ws = hcl.Workspace()
    ref = _fused(t, ws)
    hcl.debug_force_timeout(1)
    got = _fused(t, ws)
    hcl.debug_force_timeout(0)
    torch.cuda.synchronize()
    assert ws.status() == 0
    _same(got, ref)


@pytest.mark.parametrize("explicit", [True, False])
def test_concurrent_calls_on_two_streams_match_sequential(explicit):
    # two persistent-kernel calls (d = 5120 and the cooperative kernel at
    # d = 64) issued back to back on two streams, three times over
    ta, tb = _inputs(5120, 6000, seed=24), _inputs(64, 3000, seed=25)
    refa, refb = _fused(ta, hcl.Workspace()), _fused(tb, hcl.Workspace())
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    wa, wb = (hcl.Workspace(), hcl.Workspace()) if explicit else (None, None)
    got = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            ga = _fused(ta, wa)
        with torch.cuda.stream(s2):
            gb = _fused(tb, wb)
        got.append((ga, gb))
    torch.cuda.synchronize()
    for ga, gb in got:
        _same(ga, refa)
        _same(gb, refb)
    if explicit:
        assert wa.status() == 0 and wb.status() == 0
    else:
        assert hcl.workspace_status() == 0
