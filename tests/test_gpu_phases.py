"""Phase log on the GPU: the kernels' records are consistent and logging leaves every result
bit-identical (the log is a diagnostic written beside the product, never into it)."""
import numpy as np
import pytest

import dense_matrix_unit_tiled_amd as dmu
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CAP = 4096

TILE_DIMS = {"256x256": (256, 256), "256x128": (256, 128), "128x128": (128, 128), "64x128": (64, 128)}


def logged(run):
    """Run `run()` with a fresh phase log; returns (its result, records as uint64, kind)."""
    torch = gu._torch()
    log = torch.zeros(CAP * 8, dtype=torch.int64, device="cuda:0")
    dmu.dmu_phase_log(log, CAP)
    try:
        out = run()
        n, kind = dmu.dmu_phase_log_last()
    finally:
        dmu.dmu_phase_log(None, 0)
    torch.cuda.synchronize()
    return out, log.view(-1, 8)[:n].cpu().numpy().view(np.uint64), kind


def check_records(r, n, ktiles=None):
    assert r.shape == (n, 8)
    start, loop, fix, end, c0, c1 = (r[:, i].astype(np.int64) for i in range(6))
    assert np.all(start > 0)
    assert np.all(start <= loop) and np.all(loop <= fix) and np.all(fix <= end)
    assert np.all(c1 > c0)
    xcc = (r[:, 6] >> np.uint64(32)) & np.uint64(0xF)
    assert np.all(xcc < 8)
    if ktiles is not None:
        assert np.all((r[:, 7] >> np.uint64(32)) == np.uint64(ktiles))
    # the records of one launch span microseconds, not seconds (100 MHz clock)
    assert end.max() - start.min() < 100_000_000


@pytest.mark.parametrize("force", [None, "256x128", "128x128", "64x128"])
def test_one_per_tile_records_and_same_bits(force):
    p = workloads.make("c3", "random", 31, M=700, N=500, K=1030)
    plain = gu.run_dmu(p, force=force)
    (got, name), r, kind = logged(lambda: gu.run_dmu(p, force=force, return_name=True))
    gu.assert_bits_equal(got, plain)
    bm, bn = TILE_DIMS[name.split("_")[1]]
    tiles = -(-700 // bm) * -(-500 // bn)
    assert kind == 1
    check_records(r, tiles, ktiles=-(-1030 * 2 // 128))
    wg = (r[:, 7] & np.uint64(0xFFFFFFFF)).astype(np.int64)
    assert sorted(wg) == list(range(tiles))


def test_persistent_records(monkeypatch):
    monkeypatch.setenv("DMU_PERSIST", "always")
    p = workloads.make("c4s", "random", 32, batch=3, M=512, N=512, K=128)
    # (forced: a problem this small would take the 64-row tile, which has no persistent form)
    plain = gu.run_dmu(p, force="128x128")
    (got, name), r, kind = logged(lambda: gu.run_dmu(p, force="128x128", return_name=True))
    gu.assert_bits_equal(got, plain)
    assert kind == 2
    bm, bn = TILE_DIMS[name.split("_")[1]]
    # one record per tile (index = tile number), written by the worker that ran the tile
    check_records(r, p.batch * -(-512 // bm) * -(-512 // bn), ktiles=2)


def test_streamk_records_and_same_bits():
    p = workloads.make("c2", "structured", 33, M=512, N=384, K=2048)
    plain, _, _ = gu.run_streamk(p)
    (got, name, ws), r, kind = logged(lambda: gu.run_streamk(p))
    gu.assert_bits_equal(got, plain)
    assert kind == 3 and r.shape[0] > 0
    check_records(r, r.shape[0])
    # the workers' K-tiles add up to every tile's K loop
    kt = (r[:, 7] >> np.uint64(32)).astype(np.int64)
    tiles = -(-512 // 128) * -(-384 // 128)
    assert kt.sum() == tiles * (2048 * 2 // 128)


def test_fallback_writes_no_records():
    p = workloads.make("c3", "random", 34, M=130, N=70, K=33)  # odd K: 2-byte rows, the fallback
    got, r, kind = logged(lambda: gu.run_dmu(p, return_name=True))
    assert "generic" in got[1]
    assert kind == 0 and r.shape[0] == 0


def test_attention_records_and_same_bits():
    """The attention kernel writes one record per workgroup (kind 4), and its output does not
    change with the log."""
    torch = gu._torch()
    rng = np.random.default_rng(35)
    batch, sq, sk, hd = 2, 300, 200, 128
    Q, K, V = (workloads.to_bits(rng.uniform(-1, 1, batch * n * hd), "f16") for n in (sq, sk, sk))
    dQ, dK, dV = gu.to_dev(Q), gu.to_dev(K), gu.to_dev(V)

    def run():
        dO = torch.zeros(batch * sq * hd, dtype=torch.float32, device="cuda:0")
        a = dmu.attention_args(batch, sq, sk, hd, dQ, hd, dK, hd, dV, hd, dO, hd, in_type="f16",
                               out_type="f32", scale=0.1, stride_q=sq * hd, stride_k=sk * hd,
                               stride_v=sk * hd, stride_o=sq * hd)
        dmu.dmu_attention(a)
        torch.cuda.synchronize()
        return dO.cpu().numpy()

    plain = run()
    got, r, kind = logged(run)
    assert np.array_equal(got.view(np.uint32), plain.view(np.uint32))
    assert kind == 4
    check_records(r, batch * -(-sq // 256), ktiles=-(-sk // 64))
