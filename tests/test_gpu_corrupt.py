"""The GPU decoder on the seeded corrupt streams of stream_mutations (the oracle's base streams,
mutated): the same verdict as the oracle's decoder (OK or CORRUPT), the same decoded values when
both accept, and no write outside the output (sentinel guards on both sides of it).  Every
decoder read stays inside the stream by construction: the header is read only when 128 bytes are
there, the index and planes only once the header's sizes check against the stream's, a segment only
inside its index bounds, and a chunk's records only once its terminator count checks."""
import numpy as np
import pytest

from stream_mutations import cases

torch = pytest.importorskip("torch")
hq = pytest.importorskip("kv_quantization_tile_amd")

pytestmark = pytest.mark.gpu

GUARD = 256                  # binary32 values of sentinel on each side of the output (16-byte aligned)
SENTINEL = 0x7FBADBAD        # a NaN pattern no decode produces


def test_gpu_decoder_on_corrupt_streams(orc):
    print("case: corrupt-stream sweep on the GPU decoder", flush=True)
    ws = hq.workspace(0)
    n_ok = n_bad = 0
    for name, s, n in cases(orc):
        rc_orc = orc.decode_status(s, n)
        sd = torch.from_numpy(s).cuda() if s.size else torch.empty(0, dtype=torch.uint8, device="cuda")
        buf = torch.full((n + 2 * GUARD,), SENTINEL, dtype=torch.int32, device="cuda")
        out = buf[GUARD:GUARD + n].view(torch.float32)
        if sd.numel() == 0:
            sd = torch.zeros(16, dtype=torch.uint8, device="cuda")[:0]
        hq.hq_decode(sd, n, out=out, ws=ws, check=False)
        rc = hq.hq_status(ws)
        host = buf.cpu().numpy()
        assert (host[:GUARD] == SENTINEL).all() and (host[GUARD + n:] == SENTINEL).all(), name
        assert rc == rc_orc, (name, rc, rc_orc)
        if rc == hq.HQ_OK:
            y = orc.decode(s, n)
            assert np.array_equal(host[GUARD:GUARD + n].view(np.uint32), y.view(np.uint32)), name
            n_ok += 1
        else:
            n_bad += 1
    assert n_ok > 50 and n_bad > 100, (n_ok, n_bad)
