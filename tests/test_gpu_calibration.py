"""The access-pattern probe (lsa_calibrate_access) moves exactly the rows it
is asked to, in every mode, and skips row numbers outside the tables."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from content_routed_block_amd import lsa as m
    return m


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
def test_calibrate_access_copies_rows(lsa, mode):
    rows, n = 1000, 777
    g = torch.Generator().manual_seed(mode)
    src = torch.randint(-2**31, 2**31 - 1, (rows, 32), dtype=torch.int32, generator=g).cuda()
    dst = torch.full((rows, 32), 7, dtype=torch.int32, device="cuda")
    ridx = torch.randperm(rows, generator=g)[:n].to(torch.int32)
    widx = torch.randperm(rows, generator=g)[:n].to(torch.int32)
    if mode == 3:
        ridx[5], widx[6] = rows, rows + 123     # out of the tables: skipped
    lsa.calibrate_access(src, dst, n, mode, ridx.cuda(), widx.cuda())
    torch.cuda.synchronize()
    want = torch.full((rows, 32), 7, dtype=torch.int32)
    s, d = src.cpu(), dst.cpu()
    r = ridx.long() if mode & 1 else torch.arange(n)
    w = widx.long() if mode & 2 else torch.arange(n)
    keep = (r < rows) & (w < rows)
    want[w[keep]] = s[r[keep]]
    assert torch.equal(d, want)
