"""oscar_read_records (the read-bandwidth probe of the INT2 record stream): the per-lane XOR it
writes equals the same fold computed on the host over the records it is asked to read (each
record once), for runs that end on an odd record, workers without records, a multi-workgroup
grid, and record ids outside the pool (read as the pool's last record)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def expected(pool: np.ndarray, ids: np.ndarray, workers: int) -> np.ndarray:
    """Per worker: the XOR of every 32-bit word of each record of its run, each record once,
    folded to 64 lanes (lane l holds bytes 16 l .. 16 l + 15 of the first 1024 bytes and, for
    l < 32, of the last 512)."""
    n = len(ids)
    C = ((n + workers - 1) // workers + 1) & ~1
    rec = pool.reshape(-1, 1536)
    last = rec.shape[0] - 1
    out = np.zeros((workers, 64), dtype=np.uint32)
    for w in range(workers):
        acc = np.zeros((64, 4), dtype=np.uint32)
        for i in range(w * C, min(n, w * C + C)):
            rid = int(ids[i])
            words = rec[rid if 0 <= rid <= last else last].view(np.uint32)
            acc ^= words[:256].reshape(64, 4)
            acc[:32] ^= words[256:].reshape(32, 4)
        out[w] = acc[:, 0] ^ acc[:, 1] ^ acc[:, 2] ^ acc[:, 3]
    return out.reshape(-1)


@pytest.mark.parametrize("n,workers,bad_ids", [(1, 1, False), (7, 2, False), (300, 16, False),
                                               (1001, 64, False), (301, 16, True)])
def test_read_records_fold(n, workers, bad_ids):
    from int2_rotated_kv_rotate_amd import ops
    rng = np.random.default_rng(n * 31 + workers)
    num_records = 96
    pool = rng.integers(0, 256, size=num_records * 1536, dtype=np.uint8)
    ids = rng.integers(0, num_records, size=n).astype(np.int32)
    if bad_ids:   # ids past the pool and negative ids read the last record
        ids[::7] = num_records + 5
        ids[3::11] = -2
    d_pool = torch.from_numpy(pool).cuda()
    d_ids = torch.from_numpy(ids).cuda()
    out = torch.full((64 * workers,), -1, dtype=torch.int32, device="cuda")
    ops.read_records(d_pool, d_ids, workers, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, expected(pool, ids, workers))
