"""Pins the oracle's key compression and store to things other than itself.

The step (page "Qwen3.8-Flash-Next Day-0 in SGLang", section on Qwen sparse
attention): every 4 raw index keys are averaged in FP32, normalised and
rotated with the MRoPE position of the block's first token into one bf16
compressed key, stored at full_slot/4; the unfinished block's raw keys wait in
a 4-slot ring per request.

Pins: closed forms for the average and the normalisation (hand-picked keys
with rational unit vectors), the FP32 averaging the page fixes, the rotation
against transformers' Qwen2-VL MRoPE routine, the relative-position property
of a rotary embedding, chunking invariance of the ring, the slots written, and
the rejected arguments.  The bf16 rounding is pinned to closed-form ties and
to torch's FP32 -> bf16 cast.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth

DIM = 128


def _bf16(x: float) -> int:
    import torch
    return int(torch.tensor([x], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF


def _ci(k_raw, starts, counts, *, pages=None, mrope=None, ring=None, ring_pos=None, rot=0,
        sections=(0, 0, 0), theta=1.0e6, page_table=None, num_pages=None):
    """A hand-built compression call.  k_raw float values (rounded to bf16)."""
    B = len(starts)
    k_raw = synth.f32_to_bf16_bits(np.asarray(k_raw, dtype=np.float32).reshape(-1, DIM))
    ptr = np.zeros(B + 1, dtype=np.int32)
    ptr[1:] = np.cumsum(counts)
    if page_table is None:
        pages = pages or [(s + n + 63) // 64 for s, n in zip(starts, counts)]
        pt = np.full((B, max(pages)), -1, dtype=np.int32)
        off = 0
        for b, n in enumerate(pages):
            pt[b, :n] = np.arange(off, off + n)
            off += n
        num_pages = off
    else:
        pt = np.asarray(page_table, dtype=np.int32)
    kc = np.zeros((num_pages * 16, DIM), dtype=np.uint16)
    rg = np.zeros((B, 4, DIM), dtype=np.uint16) if ring is None else synth.f32_to_bf16_bits(
        np.asarray(ring, dtype=np.float32)).reshape(B, 4, DIM)
    rp = np.zeros((B, 3), dtype=np.int32) if ring_pos is None else np.asarray(ring_pos, dtype=np.int32)
    return synth.CompressInputs(name="pin", k_raw=k_raw, req_tok_ptr=ptr,
                                tok_start=np.asarray(starts, dtype=np.int32),
                                mrope_pos=None if mrope is None else np.asarray(mrope, dtype=np.int32),
                                ring=rg, ring_pos=rp, page_table=pt, kcache=kc, num_pages=int(num_pages),
                                rotary_dim=rot, sections=tuple(sections), theta=theta, seed=0)


# ---------------------------------------------------------------------------
# double -> bf16
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),                   # tie -> even mantissa (down)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),               # tie -> even mantissa (up)
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),      # just above the tie: one rounding, not two
    (-2.5, 0xC020),
    (-0.0, 0x8000),
    (2.0 ** -126, 0x0080),                       # smallest normal
    (2.0 ** -133, 0x0001),                       # smallest subnormal
    (2.0 ** -134, 0x0000),                       # half of it: tie -> even (zero)
    (1.5 * 2.0 ** -133, 0x0002),                 # tie between 1 and 2 quanta -> 2
    ((2.0 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),    # largest finite
    ((2.0 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),    # tie above it rounds to even -> infinity
    (float("inf"), 0x7F80),
    (float("-inf"), 0xFF80),
])
def test_f64_to_bf16_closed_forms(x, bits):
    assert int(oracle.f64_to_bf16_bits([x])[0]) == bits


def test_f64_to_bf16_nan_and_torch_cast():
    nan = int(oracle.f64_to_bf16_bits([float("nan")])[0])
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-40, 38, 3000),
                        rng.standard_normal(500) * 1e-41]).astype(np.float32)
    import torch
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f64_to_bf16_bits(v.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


# ---------------------------------------------------------------------------
# average and normalisation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("slot", [0, 1, 2, 3])
def test_one_key_at_each_slot(slot):
    """Keys (0.., v, ..0): the mean is v/4 and its direction v/|v|; with
    v = 3 e_7 + 4 e_100 the key is 0.6 e_7 + 0.8 e_100."""
    k = np.zeros((4, DIM))
    k[slot, 7], k[slot, 100] = 3.0, 4.0
    o = oracle.compress_store(_ci(k, [0], [4]))
    want = np.zeros(DIM, dtype=np.uint16)
    want[7], want[100] = _bf16(0.6), _bf16(0.8)
    np.testing.assert_array_equal(o["kcache"][0], want)
    assert abs(o["exact"][0, 7] - 0.6) < 1e-15 and abs(o["exact"][0, 100] - 0.8) < 1e-15
    assert np.all(np.isnan(o["exact"][1:]))


def test_cancelling_keys():
    """(v, -v, w, 0) averages to w/4: the key is w/|w| = (5/13, 12/13)."""
    k = np.zeros((4, DIM))
    k[0, :] = np.linspace(-2, 2, DIM)
    k[1, :] = -k[0, :]
    k[2, 3], k[2, 90] = 5.0, 12.0
    ci = _ci(k, [0], [4])
    ci.k_raw[1] = ci.k_raw[0] ^ 0x8000           # exact negation of the bf16 pattern
    o = oracle.compress_store(ci)
    e = o["exact"][0]
    assert abs(e[3] - 5 / 13) < 1e-15 and abs(e[90] - 12 / 13) < 1e-15
    assert np.count_nonzero(e) == 2


def test_zero_mean_stays_zero():
    k = np.zeros((8, DIM))
    k[4] = np.linspace(-1, 1, DIM)
    k[5] = -k[4]
    k[6] = k[4]
    k[7] = -k[4]
    o = oracle.compress_store(_ci(k, [0], [8]))
    assert np.all(o["kcache"][:2] == 0) and np.all(o["exact"][:2] == 0)


def test_average_is_taken_in_fp32():
    """Dim a holds (1, 2^-24, 2^-24, 0) and dim b (1, 0, 0, 0).  In FP32 each
    1 + 2^-24 rounds back to 1 (tie to even), so both means are 0.25 and the
    normalised values equal 1/sqrt(2) exactly; a wider average would make a
    larger."""
    k = np.zeros((4, DIM))
    k[0, 5], k[1, 5], k[2, 5] = 1.0, 2.0 ** -24, 2.0 ** -24
    k[0, 9] = 1.0
    o = oracle.compress_store(_ci(k, [0], [4]))
    assert o["exact"][0, 5] == o["exact"][0, 9]
    assert abs(o["exact"][0, 5] - 2 ** -0.5) < 1e-15


def test_unit_norm_and_scale_invariance():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((64, DIM))
    base = _ci(k, [0], [64], rot=DIM, sections=(16, 24, 24))
    o = oracle.compress_store(base)
    nrm = np.sqrt(np.sum(o["exact"][:16] ** 2, axis=1))
    np.testing.assert_allclose(nrm, 1.0, atol=1e-14)
    o2 = oracle.compress_store(_ci(k * 2.0 ** 20, [0], [64], rot=DIM, sections=(16, 24, 24)))
    np.testing.assert_array_equal(o2["kcache"], o["kcache"])


# ---------------------------------------------------------------------------
# rotation
# ---------------------------------------------------------------------------

def _hf_mrope(y: np.ndarray, pos3: np.ndarray, rot: int, sections, theta: float) -> np.ndarray:
    """transformers' Qwen2-VL multimodal rotary embedding applied to the first
    ``rot`` dims of each row of y (float64); ``pos3`` [n][3]."""
    import torch
    from transformers.models.qwen2_vl import modeling_qwen2_vl as m
    from transformers.models.qwen2_vl.configuration_qwen2_vl import Qwen2VLTextConfig
    cfg = Qwen2VLTextConfig(hidden_size=rot, num_attention_heads=1, num_key_value_heads=1,
                            rope_parameters={"rope_type": "default", "rope_theta": theta,
                                             "mrope_section": list(sections)})
    emb = m.Qwen2VLRotaryEmbedding(cfg)
    pid = torch.from_numpy(np.ascontiguousarray(pos3.T[:, None, :], dtype=np.int64))   # [3][1][n]
    x = torch.from_numpy(np.ascontiguousarray(y[None, None, :, :rot]))                 # [1][1][n][rot]
    cos, sin = emb(x, pid)
    out, _ = m.apply_multimodal_rotary_pos_emb(x, x, cos, sin, list(sections))
    res = y.copy()
    res[:, :rot] = out[0, 0].numpy()
    return res


@pytest.mark.parametrize("rot,sections,theta", [(128, (16, 24, 24), 1.0e6), (64, (8, 12, 12), 1.0e4),
                                                (128, (40, 0, 24), 5.0e5)])
def test_rotation_matches_transformers_qwen2_vl_mrope(rot, sections, theta):
    """The rotated key equals transformers' MRoPE of the unrotated key at the
    MRoPE position of the block's first token.  Positions stay below 400 so
    that the library's FP32 angles are good to ~1e-5."""
    rng = np.random.default_rng(11)
    n = 96
    k = rng.standard_normal((n, DIM))
    mpos = synth.mrope_positions(np.arange(n), [(10, 5), (50, 4)])
    mpos[:, 0] += 200                                  # distinct t, h, w components
    mpos[:, 2] += 100
    plain = oracle.compress_store(_ci(k, [0], [n], mrope=mpos))
    rotd = oracle.compress_store(_ci(k, [0], [n], mrope=mpos, rot=rot, sections=sections, theta=theta))
    y = plain["exact"][: n // 4]
    want = _hf_mrope(y, mpos[0::4], rot, sections, theta)
    np.testing.assert_allclose(rotd["exact"][: n // 4], want, atol=5e-5, rtol=0)
    # the last token's position would give a different key
    wrong = _hf_mrope(y, mpos[3::4], rot, sections, theta)
    assert np.max(np.abs(rotd["exact"][: n // 4] - wrong)) > 1e-2


def test_text_positions_make_the_section_layout_moot():
    rng = np.random.default_rng(12)
    n = 64
    k = rng.standard_normal((n, DIM))
    start = 1000
    text = np.repeat(np.arange(start, start + n)[:, None], 3, axis=1)
    outs = [oracle.compress_store(_ci(k, [start], [n], mrope=text, rot=DIM, sections=sec))["kcache"]
            for sec in [(64, 0, 0), (16, 24, 24), (0, 0, 64)]]
    outs.append(oracle.compress_store(_ci(k, [start], [n], rot=DIM, sections=(16, 24, 24)))["kcache"])
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])


def test_relative_position_property():
    """<R(p) a, R(q) b> depends on p - q only."""
    rng = np.random.default_rng(13)
    k = rng.standard_normal((8, DIM))

    def keys(p0, p1):
        mpos = np.zeros((8, 3), dtype=np.int32)
        mpos[0:4] = p0
        mpos[4:8] = p1
        return oracle.compress_store(_ci(k, [0], [8], mrope=mpos, rot=DIM, sections=(16, 24, 24)))["exact"]

    base = keys([5, 7, 9], [40, 3, 17])
    d0 = base[0] @ base[1]
    for shift in [1, 123, 4096, 70000]:
        e = keys([5 + shift, 7 + shift, 9 + shift], [40 + shift, 3 + shift, 17 + shift])
        assert abs(e[0] @ e[1] - d0) < 1e-9
    e = keys([6, 7, 9], [40, 3, 17])
    assert abs(e[0] @ e[1] - d0) > 1e-6


# ---------------------------------------------------------------------------
# ring and store
# ---------------------------------------------------------------------------

def _multi(seed=5):
    return synth.build_compress_batch("pin", seed, starts=[130, 4093, 0, 77, 255], counts=[37, 3, 9, 1, 70],
                                      ctx_tokens=[200, 4100, 64, 90, 400],
                                      images=[[(100, 6)], [], [], [(20, 3)], [(250, 5)]])


def test_chunked_calls_equal_one_call():
    ci = _multi()
    whole = oracle.compress_store(ci)
    # the same tokens in three calls, the ring carrying the state across
    rng = np.random.default_rng(1)
    counts = np.diff(ci.req_tok_ptr)
    cuts = [np.sort(rng.integers(0, n + 1, size=2)) for n in counts]
    kc, rg, rp = ci.kcache, ci.ring, ci.ring_pos
    for part in range(3):
        lo = [0 if part == 0 else int(c[part - 1]) for c in cuts]
        hi = [int(c[part]) if part < 2 else int(n) for c, n in zip(cuts, counts)]
        idx = np.concatenate([np.arange(ci.req_tok_ptr[b] + lo[b], ci.req_tok_ptr[b] + hi[b])
                              for b in range(ci.num_req)]).astype(np.int64)
        ptr = np.zeros(ci.num_req + 1, dtype=np.int32)
        ptr[1:] = np.cumsum([h - l for l, h in zip(lo, hi)])
        part_ci = synth.CompressInputs(**{**ci.__dict__, "k_raw": ci.k_raw[idx], "req_tok_ptr": ptr,
                                          "tok_start": (ci.tok_start + np.array(lo)).astype(np.int32),
                                          "mrope_pos": ci.mrope_pos[idx]})
        o = oracle.compress_store(part_ci, kcache=kc, ring=rg, ring_pos=rp)
        kc, rg, rp = o["kcache"], o["ring"], o["ring_pos"]
    np.testing.assert_array_equal(kc, whole["kcache"])
    np.testing.assert_array_equal(rg, whole["ring"])
    np.testing.assert_array_equal(rp, whole["ring_pos"])


def test_ring_holds_the_latest_token_of_each_slot():
    ci = _multi()
    o = oracle.compress_store(ci)
    for b in range(ci.num_req):
        s, n = int(ci.tok_start[b]), int(ci.req_tok_ptr[b + 1] - ci.req_tok_ptr[b])
        e = s + n - 1
        for u in range(4):
            p = e - ((e - u) % 4)                       # latest position <= e in slot u
            want = ci.k_raw[ci.req_tok_ptr[b] + p - s] if p >= s else ci.ring[b, u]
            np.testing.assert_array_equal(o["ring"][b, u], want)
        p0 = e - e % 4
        want = ci.mrope_pos[ci.req_tok_ptr[b] + p0 - s] if p0 >= s else ci.ring_pos[b]
        np.testing.assert_array_equal(o["ring_pos"][b], want)


def test_writes_exactly_the_completed_blocks():
    ci = _multi()
    o = oracle.compress_store(ci)
    expect = set()
    for b in range(ci.num_req):
        s, n = int(ci.tok_start[b]), int(ci.req_tok_ptr[b + 1] - ci.req_tok_ptr[b])
        for p in range(s, s + n):
            if p % 4 == 3:
                j = p // 4
                expect.add(int(ci.page_table[b, 4 * j // 64]) * 16 + j % 16)
    written = set(np.nonzero(~np.isnan(o["exact"][:, 0]))[0].tolist())
    changed = set(np.nonzero(np.any(o["kcache"] != ci.kcache, axis=1))[0].tolist())
    assert written == expect and changed <= expect
    assert len(expect) == sum(1 for b in range(ci.num_req)
                              for p in range(ci.tok_start[b], ci.tok_start[b] + ci.req_tok_ptr[b + 1]
                                             - ci.req_tok_ptr[b]) if p % 4 == 3)


def test_block_straddling_the_call_reads_the_ring():
    """Tokens 4m .. 4m+1 arrive in an earlier call (they sit in the ring);
    tokens 4m+2, 4m+3 arrive now: the block averages all four."""
    k = np.zeros((4, DIM))
    k[0, 1], k[1, 1] = 8.0, 8.0                         # earlier tokens (ring slots 0, 1)
    k[2, 2], k[3, 2] = 6.0, 6.0                         # new tokens
    ring = np.zeros((1, 4, DIM))
    ring[0, :2] = k[:2]
    ci = _ci(k[2:], [4 * 5 + 2], [2], ring=ring)
    o = oracle.compress_store(ci)
    e = o["exact"][5]
    assert abs(e[1] - 0.8) < 1e-15 and abs(e[2] - 0.6) < 1e-15


# ---------------------------------------------------------------------------
# rejected arguments and data
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kw", [dict(rot=3, sections=(1, 0, 0)), dict(rot=130, sections=(65, 0, 0)),
                                dict(rot=-2, sections=(0, 0, 0)), dict(rot=64, sections=(16, 8, 7)),
                                dict(rot=64, sections=(-1, 17, 16)), dict(rot=64, sections=(16, 8, 8), theta=0.0),
                                dict(rot=64, sections=(16, 8, 8), theta=float("inf"))])
def test_rejects_bad_arguments(kw):
    ci = _ci(np.ones((4, DIM)), [0], [4], **kw)
    with pytest.raises(oracle.OracleError):
        oracle.compress_store(ci)


def test_rejects_bad_data():
    with pytest.raises(oracle.OracleError):
        oracle.compress_store(_ci(np.ones((4, DIM)), [-4], [4], pages=[1]))
    ci = _ci(np.ones((4, DIM)), [60], [4], pages=[1])    # block 15 fits page 0
    oracle.compress_store(ci)
    ci = _ci(np.ones((8, DIM)), [60], [8], pages=[1])    # block 16 needs a second page
    with pytest.raises(oracle.OracleError):
        oracle.compress_store(ci)
