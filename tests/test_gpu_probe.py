"""oscar_read_records (the read-bandwidth probe of the INT2 record stream): the per-lane XOR it
writes equals the same fold computed on the host over the records it is asked to read, for
runs that end on an odd record, workers without records and a multi-workgroup grid."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def expected(pool: np.ndarray, ids: np.ndarray, workers: int) -> np.ndarray:
    n = len(ids)
    C = ((n + workers - 1) // workers + 1) & ~1
    rec = pool.reshape(-1, 1536)
    out = np.zeros((workers, 64), dtype=np.uint32)
    for w in range(workers):
        r0, r1 = w * C, min(n, w * C + C)
        acc = np.zeros((64, 4), dtype=np.uint32)
        for i in range(r0, r1, 2):
            ib = min(i + 1, r1 - 1)
            for rid in (ids[i], ids[ib]):
                words = rec[rid].view(np.uint32)
                acc ^= words[:256].reshape(64, 4)
                acc[:32] ^= words[256:].reshape(32, 4)
        out[w] = acc[:, 0] ^ acc[:, 1] ^ acc[:, 2] ^ acc[:, 3]
    return out.reshape(-1)


@pytest.mark.parametrize("n,workers", [(1, 1), (7, 2), (300, 16), (1001, 64)])
def test_read_records_fold(n, workers):
    from int2_rotated_kv_rotate_amd import ops
    rng = np.random.default_rng(n * 31 + workers)
    num_records = 96
    pool = rng.integers(0, 256, size=num_records * 1536, dtype=np.uint8)
    ids = rng.integers(0, num_records, size=n).astype(np.int32)
    d_pool = torch.from_numpy(pool).cuda()
    d_ids = torch.from_numpy(ids).cuda()
    out = torch.full((64 * workers,), -1, dtype=torch.int32, device="cuda")
    ops.read_records(d_pool, d_ids, workers, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, expected(pool, ids, workers))
