"""The streaming-read reference kernel (coli_probe_read) through the C ABI:
it reads every byte it is given -- the XOR of all 32-bit words it returns
equals numpy's over the same buffer, for sizes that leave ragged tails of
its per-workgroup stride, and for a buffer larger than its grid covers in
one pass -- and a zero size launches nothing."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from int4_routed_expert_layer_amd import binding as B  # noqa: E402


@pytest.mark.parametrize("n_words", [4, 4 * 1021, 4 * 262147, 4 * (1 << 22) + 12])
def test_probe_read_xors_every_word(n_words):
    rng = np.random.default_rng(n_words)
    host = rng.integers(-2**31, 2**31, size=n_words, dtype=np.int64).astype(np.int32)
    buf = torch.from_numpy(host).to("cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    B.probe_read(buf, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.view(np.uint32))
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(want)


def test_probe_read_of_nothing_leaves_the_sink():
    buf = torch.ones(4, dtype=torch.int32, device="cuda:0")
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda:0")
    assert B.lib.coli_probe_read(B.C.c_void_p(buf.data_ptr()), 0, B.C.c_void_p(sink.data_ptr()),
                                 B.C.c_void_p(torch.cuda.current_stream().cuda_stream)) == B.OK
    torch.cuda.synchronize()
    assert int(sink.cpu()[0]) == 7
