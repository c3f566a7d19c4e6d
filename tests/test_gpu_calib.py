"""The calibration probes behind the bench's measured peaks, on the GPU:
the copy and read probes touch every byte of their buffers exactly once
(ragged sizes and empty chunks included), and the MFMA probe's per-wave sums
equal the closed form of its operands: the sum of all entries of A B is
sum_k (sum_i A[i][k]) (sum_j B[k][j])."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
import expert_load_balance_amd as moe  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (bytes, workgroups): one vector; several rounds per thread; a ragged tail;
# chunks left empty (more workgroups than vectors)
_SIZES = [(16, 1), (1 << 20, 7), (5 * (1 << 20) + 48, 64), (32, 4), (3 * 65536 + 16, 3)]


def _bytes(n, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g).to(DEV)


@pytest.mark.parametrize("nbytes,wg", _SIZES)
def test_copy_probe_is_exact(nbytes, wg):
    src = _bytes(nbytes, nbytes)
    dst = torch.zeros_like(src)
    moe.moe_probe_copy(src, dst, wg)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


@pytest.mark.parametrize("nbytes,wg", _SIZES)
def test_read_probe_reads_every_vector_once(nbytes, wg):
    src = _bytes(nbytes, nbytes + 1)
    sink = torch.full((wg * 256,), -1, dtype=torch.int32, device=DEV)
    moe.moe_probe_read(src, wg, sink)
    torch.cuda.synchronize()
    words = src.cpu().numpy().view(np.uint32).reshape(-1, 4)
    fold = words[:, 0] ^ words[:, 1] ^ words[:, 2] ^ words[:, 3]
    n16 = fold.size
    chunk = -(-n16 // wg)
    want = np.zeros(wg * 256, dtype=np.uint32)
    for b in range(wg):
        seg = fold[b * chunk:min((b + 1) * chunk, n16)]
        np.bitwise_xor.at(want, b * 256 + np.arange(seg.size) % 256, seg)
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want)


def _operand(seed):
    """The probe's eight bf16 operand values for one lane, as float64: sign and
    mantissa bits from a 32-bit multiplicative hash, exponent 2^-7."""
    out = np.empty(8)
    for i in range(8):
        h = ((seed * 8 + i + 1) * 2654435761) & 0xFFFFFFFF
        h ^= h >> 13
        h = (h * 0x85EBCA6B) & 0xFFFFFFFF
        h ^= h >> 16
        sign = -1.0 if (h >> 8) & 0x8000 else 1.0
        out[i] = sign * 2.0 ** -7 * (1 + (h & 0x7F) / 128)
    return out


def test_mfma_probe_matches_closed_form():
    wg, iters, chains = 2, 3, 4
    sink = torch.full((wg * 256,), float("nan"), dtype=torch.float32, device=DEV)
    moe.moe_probe_mfma(wg, iters, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().astype(np.float64).reshape(-1, 64).sum(axis=1)  # per wave
    for wave in range(wg * 4):
        ids = wave * 64 + np.arange(64)
        total = scale = 0.0
        for c in range(chains):
            a = np.stack([_operand(int(i) * 2 * chains + 2 * c) for i in ids])      # [lane][8]
            b = np.stack([_operand(int(i) * 2 * chains + 2 * c + 1) for i in ids])
            # lanes 32 h .. 32 h + 31 carry K-half h of all 32 rows (A) or
            # columns (B); element e is k = 8 h + e of the 16-deep product
            for h in range(2):
                ca = a[32 * h:32 * h + 32].sum(axis=0)
                cb = b[32 * h:32 * h + 32].sum(axis=0)
                total += float((ca * cb).sum())
                scale += float((np.abs(a[32 * h:32 * h + 32]).sum(axis=0)
                                * np.abs(b[32 * h:32 * h + 32]).sum(axis=0)).sum())
        assert abs(got[wave] - iters * total) <= 1e-4 * iters * scale, (wave, got[wave], iters * total)
