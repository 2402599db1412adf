"""The allocation-free split-K entry point (pgemm_f16_splitk_noalloc),
called through the C ABI, against pgemm_f16_splitk with a caller workspace:
bit-identical results on two calls in a row, the second smaller, on the same
static buffer."""
import sys

import numpy as np
import pytest

import software_pipelined_tiled_pgemm_amd as pg
from software_pipelined_tiled_pgemm_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# (M, N, K, splits): the long-K configuration at the default split count,
# whose partials fill the static buffer exactly, then a ragged smaller shape.
CALLS = [(2048, 2048, 32768, 4), (520, 776, 4104, 3)]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_noalloc_matches_workspace_entry_point_on_consecutive_calls():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    L = pg.lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev).cuda_stream
    for (M, N, K, splits) in CALLS:
        say("splitk noalloc M=%d N=%d K=%d splits=%d" % (M, N, K, splits))
        need = pg.pgemm_f16_splitk_workspace_bytes(M, N, K, splits)
        assert 0 < need <= pg.STATIC_SCRATCH_BYTES
        A, B = inputs.gemm_inputs(M, N, K)
        tA, tB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
        C = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
        rc = L.pgemm_f16_splitk_noalloc(tA.data_ptr(), tB.data_ptr(), C.data_ptr(), M, N, K,
                                        splits, stream)
        assert rc == pg.PGEMM_OK, pg.status_string(rc)
        ws = torch.empty(need // 4, dtype=torch.float32, device=dev)
        R = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
        rc = L.pgemm_f16_splitk(tA.data_ptr(), tB.data_ptr(), R.data_ptr(), M, N, K, splits,
                                ws.data_ptr(), need, stream)
        assert rc == pg.PGEMM_OK, pg.status_string(rc)
        torch.cuda.synchronize()
        got, ref = C.cpu().numpy(), R.cpu().numpy()
        assert not np.isnan(ref).any()
        assert np.array_equal(got.view(np.uint16), ref.view(np.uint16)), \
            "%d of %d outputs differ" % ((got.view(np.uint16) != ref.view(np.uint16)).sum(), got.size)


def test_noalloc_rejects_requests_beyond_the_buffer():
    L = pg.lib()
    # 5 partials of 2048^2 fp32 = 80 MiB > 64 MiB: rejected before any launch
    M = N = 2048
    K, splits = 40960, 5
    assert pg.pgemm_f16_splitk_workspace_bytes(M, N, K, splits) > pg.STATIC_SCRATCH_BYTES
    A = torch.empty((M, K), dtype=torch.float16, device="cuda:0")
    B = torch.empty((K, N), dtype=torch.float16, device="cuda:0")
    C = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    rc = L.pgemm_f16_splitk_noalloc(A.data_ptr(), B.data_ptr(), C.data_ptr(), M, N, K, splits, None)
    assert rc == pg.PGEMM_ESCRATCH
