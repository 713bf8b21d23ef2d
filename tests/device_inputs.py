"""Device-side helpers of the tests and the benchmark (not part of the library): output
buffers pre-filled with NaN / sentinel values, so that an entry a kernel failed to write
is visible, and paged copies of per-batch K/V rows for the block-table tests."""
import numpy as np
import torch


def empty_outputs(W, dtype, device="cuda"):
    B, Hq, nq, dv, k = W["B"], W["Hq"], W["n_q"], W["d_v"], W["k"]
    O = torch.full((B, Hq, nq, dv), float("nan"), dtype=dtype, device=device)
    lse = torch.full((B, Hq, nq), float("nan"), dtype=torch.float32, device=device)
    idx = torch.full((B, nq, k), -7, dtype=torch.int32, device=device)
    return O, lse, idx


def device_pool(X, block_table, page_size, pool_rows, fill=3.0e4, check_rows=256, seed=0):
    """Paged copy of per-batch device rows X [B, H, n_kv, d]: a pool [1, H, pool_rows, d] in
    which logical row j of batch b is row block_table[b, j // page_size] * page_size +
    j % page_size; rows no batch uses hold `fill`.  Pages are copied as slices (no indexed
    scatter over the whole pool), then `check_rows` random rows and each batch's last row
    are compared with their sources."""
    B, H, n_kv, d = X.shape
    bt = np.asarray(block_table, np.int64)
    npg = -(-n_kv // page_size)
    if bt.min(initial=0) < 0 or (bt[:, :npg].max(initial=0) + 1) * page_size > pool_rows:
        raise ValueError("device_pool: the block table names rows outside the pool")
    pool = torch.full((1, H, pool_rows, d), fill, dtype=X.dtype, device=X.device)
    for b in range(B):
        for pg in range(npg):
            lo, dst = pg * page_size, int(bt[b, pg]) * page_size
            hi = min(lo + page_size, n_kv)
            pool[0, :, dst:dst + hi - lo].copy_(X[b, :, lo:hi])
    rng = np.random.default_rng(seed)
    bs = np.concatenate([rng.integers(0, B, check_rows), np.arange(B)])
    js = np.concatenate([rng.integers(0, n_kv, check_rows), np.full(B, n_kv - 1)])
    for b, j in zip(bs.tolist(), js.tolist()):
        r = int(bt[b, j // page_size]) * page_size + j % page_size
        if not torch.equal(pool[0, :, r].view(torch.uint8), X[b, :, j].view(torch.uint8)):  # bytes: NaN rows too
            raise RuntimeError("device_pool: pool row %d does not hold batch %d position %d" % (r, b, j))
    return pool
