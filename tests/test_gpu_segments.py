"""kvs_compress_block_seg against kvs_compress_block on the same cache.

The two-segment call must give the one-buffer call's results bit for bit:
scores, kept positions and compacted rows.  Rows of the segment buffers that
lie outside the cache are filled with NaN, so any read outside the segments
would show up in the scores.  Covers bf16 (d = 128 and 64, MFMA path) and fp32
(vector path), one chunk over the cache and several chunks, and head lengths
of 0, 8, a multiple of 8 inside the cache, and N.
"""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import kv_cache_compression_kvs_amd as pkg
    return pkg


def nan_like(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


CASES = [
    # (dtype, d, L, Hq, Hkv, N, S, chunk, nq, keep, head_rows)
    (torch.bfloat16, 128, 2, 6, 2, 1520, 4, 1516, 96, 1000, 1000),
    (torch.bfloat16, 128, 2, 6, 2, 1520, 4, 1516, 96, 1000, 0),
    (torch.bfloat16, 128, 2, 6, 2, 1520, 4, 1516, 96, 1000, 8),
    (torch.bfloat16, 128, 2, 6, 2, 1520, 4, 1516, 96, 1000, 1520),
    (torch.bfloat16, 128, 2, 8, 2, 4300, 4, 1024, 41, 860, 2048),
    (torch.bfloat16, 64, 1, 4, 2, 2053, 4, 700, 37, 300, 1536),
    (torch.float32, 64, 1, 4, 2, 777, 4, 300, 20, 150, 512),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{str(c[0])[6:]}-d{c[1]}-N{c[5]}-h{c[10]}")
def test_segments_match_one_buffer(K, case):
    dtype, d, L, Hq, Hkv, N, S, chunk, nq, keep, h = case
    g = torch.Generator().manual_seed(N * 31 + h)
    R = -(-(N - S) // chunk)
    q = torch.randn(L, Hq, R * nq, d, generator=g).to(dtype).cuda()
    k = torch.randn(L, Hkv, N, d, generator=g).to(dtype).cuda()
    v = torch.randn(L, Hkv, N, d, generator=g).to(dtype).cuda()
    k[..., 3] += 4.0  # an outlier channel, as in the synthetic workloads
    p = K.make_problem(L, Hq, Hkv, d, N, S, chunk, nq, dtype)
    ws = K.workspace(p)
    rows = Hkv * keep * L

    def outputs():
        return (torch.empty(L * Hkv * N, device="cuda"),
                torch.empty(rows, dtype=torch.int32, device="cuda"),
                torch.empty(rows, d, dtype=dtype, device="cuda"),
                torch.empty(rows, d, dtype=dtype, device="cuda"))

    s1, kept1, ko1, vo1 = outputs()
    got1 = K.kvs_compress_block(p, q, k, v, keep * L, None, 0.0, s1, kept1, ko1, vo1, 0, ws=ws)

    # head segment: rows [0, h) in a buffer with a larger slab stride; tail
    # segment: rows [h, N) starting at row 5 of another one; NaN elsewhere
    hs, t0 = h + 24, 5
    ts = t0 + (N - h) + 11
    kh, vh = nan_like((L, Hkv, hs, d), dtype), nan_like((L, Hkv, hs, d), dtype)
    kt, vt = nan_like((L, Hkv, ts, d), dtype), nan_like((L, Hkv, ts, d), dtype)
    kh[:, :, :h], vh[:, :, :h] = k[:, :, :h], v[:, :, :h]
    kt[:, :, t0:t0 + N - h], vt[:, :, t0:t0 + N - h] = k[:, :, h:], v[:, :, h:]
    p2 = K.make_problem(L, Hq, Hkv, d, N, S, chunk, nq, dtype, kv_row_stride=0)
    s2, kept2, ko2, vo2 = outputs()
    got2 = K.kvs_compress_block_seg(p2, q, kh, vh, h, hs, kt, vt, t0, ts, keep * L, None, 0.0,
                                    s2, kept2, ko2, vo2, 0, ws=ws)
    torch.cuda.synchronize()
    assert list(got1) == list(got2)
    assert torch.equal(s1, s2), "scores differ"
    assert torch.equal(kept1, kept2), "kept positions differ"
    assert torch.equal(ko1, ko2) and torch.equal(vo1, vo2), "compacted rows differ"
