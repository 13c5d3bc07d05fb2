"""The GPU one-lane encoder (k_encode, more than 16384 streams, staged
symbols) on streams forced to carry through long runs of 0xFF bytes, so that
carries reach dwords a lane has already written out of its pending bytes:
stream lengths, slab offsets and payload bit for bit against the oracle, with
the pair-offset staging (A = 32, a power of two) and the clamped staging
(A = 40).  The straddling streams are built as in the oracle's own forced-carry
pin; a big-integer model of the coder confirms that the runs are long."""
import numpy as np
import pytest

import entropy_coding_02_amd as kvc
import oracle
from coder_model import exact_encode
from gpu_util import say
from test_oracle_coder import _straddling_sequence, cdf_from_counts

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("A", [32, 40])
def test_forced_carries_one_lane_encoder(A):
    import torch
    L, C, T, Tc = 1, 64, 8448, 256  # 16896 streams, C % 16 == 0
    NC = T // Tc
    rng = np.random.default_rng(300 + A)
    tab = np.empty((NC, L, 2, C, A), np.uint16)
    for j in range(NC):
        for kv in range(2):
            tab[j, 0, kv] = np.array(
                [cdf_from_counts((rng.integers(0, 4, A) * rng.integers(1, 30000, A) + 1).tolist()) for _ in range(C)],
                dtype=np.uint16)
    sym = rng.integers(0, A, (L, 2, T, C)).astype(np.uint8)
    longest = 0
    for t in range(0, T, 16):  # every 16th token row of K and V straddles a byte boundary
        for kv in range(2):
            rows = tab[t // Tc, 0, kv]
            q = _straddling_sequence(rows, rng, int(rng.integers(16, C)), resolve_up=bool((t // 16 + kv) % 2))
            sym[0, kv, t] = q
            if t % 512 == 0:
                longest = max(longest, exact_encode(q.tolist(), rows.tolist())[1]["max_ff_run"])
    assert longest >= 6, longest  # runs longer than the 2-3 pending bytes

    say(f"[gpu] forced carries, one-lane encoder, A={A}")
    d = kvc.Desc(L, C, T, [[A, A]], Tc)
    assert d.alphabet == A and d.n_streams > 16384
    buf = kvc.alloc(d)
    st = torch.from_numpy(sym).cuda()
    cdf = torch.from_numpy(tab.reshape(-1).view(np.int16)).cuda()
    kvc.kvc_encode(d, st, cdf, buf.scratch, buf.stream_len, buf.slab_off, buf.payload, buf.dev_status)
    torch.cuda.synchronize()
    assert int(buf.dev_status.item()) == 0
    want_len, want_off, want_pay = oracle.encode(sym, tab, Tc, A)
    got_len = buf.stream_len[: d.n_streams].cpu().numpy().view(np.uint16)
    got_off = buf.slab_off[: d.n_slabs + 1].cpu().numpy().view(np.uint64)
    assert np.array_equal(got_len, want_len)
    assert np.array_equal(got_off, want_off)
    n = int(want_off[-1])
    assert np.array_equal(buf.payload[:n].cpu().numpy(), want_pay[:n])
