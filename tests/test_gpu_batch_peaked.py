"""GPU parity on the launch shapes the benchmark uses and on peaked attention.

* Appends over a whole batch in single launches (one launch per step for all
  sequences, as a decode step does, and one bulk launch of many tokens per
  sequence), on ragged lengths that cross every region boundary and on
  scattered pages: codes and metadata codes bit-exact with the oracle for
  every sequence, then the decode within tolerance.
* Peaked attention: queries scaled x8 and x32 (the fixed-point query step
  grows with the query norm); one dominant key in the sink, in the first, a
  middle and the last history page and in the recent window; logits that
  rise page by page so the scan's running reference moves many times.

Each case prints its error against the 2e-3 tolerance.
"""
import numpy as np
import pytest

from bit_rotated_kv_int2_amd import oscar as O
from bit_rotated_kv_int2_amd import synth
from oracle import oscar_ref as R
from pool_helpers import (append_sequence, decode_check, gather_history, oracle_calibration,
                          rotation_tensors)

pytestmark = pytest.mark.gpu
D = 128
TOL = 2e-3


def _f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def _to_bits(x):
    """float array -> bf16 bit patterns (uint16), round to nearest even."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _decode(params, rot, pool, q_bits, variant=0):
    import torch
    ws = O.alloc_workspace(O.decode_workspace_size(params, pool.batch, pool.max_pages, variant))
    q = torch.from_numpy(np.ascontiguousarray(q_bits).view(np.int16)).cuda()
    out = torch.zeros((pool.batch, params.num_q_heads, D), dtype=torch.float32, device="cuda")
    O.decode_attention(params, rot, pool, q, out, ws, variant=variant)
    torch.cuda.synchronize()
    return out.cpu().numpy()


# ---------------------------------------------------------------------------
# batch appends in single launches
# ---------------------------------------------------------------------------

def test_batch_appends_single_launches():
    """Four sequences (two KV heads, G = 4) starting at 0, 100, 300 and 2017
    tokens, pages scattered: 40 decode-step appends of one token per sequence
    (one launch each, over the whole batch), then one bulk launch of 150
    tokens per sequence.  The sequences cross the sink, window and
    demotion boundaries at different steps."""
    import torch
    wl = synth.Workload(120, "test-batch-append", 4, 2, 8, 128, 0, 2400, n_cal=512, outliers="pairs10",
                        scattered_pages=True)
    cals = oracle_calibration(wl, n_cal=512)
    rot = rotation_tensors(cals)
    params = O.make_params(wl.n_kv, wl.n_q)
    lens0 = np.array([0, 100, 300, 2017], np.int32)
    n_single, n_bulk = 40, 150
    final = lens0 + n_single + n_bulk
    bt, total = synth.block_table(wl, final)
    pool = O.KVPool(params, wl.batch, total, bt)
    toks = [synth.kv_tokens(wl, 0, b, 0, int(final[b])) for b in range(wl.batch)]
    for b in range(wl.batch):
        if lens0[b]:
            append_sequence(params, rot, pool, b, toks[b][0][:lens0[b]], toks[b][1][:lens0[b]])

    def batch_tokens(start, n):
        k = np.stack([toks[b][0][start[b]:start[b] + n] for b in range(wl.batch)])
        v = np.stack([toks[b][1][start[b]:start[b] + n] for b in range(wl.batch)])
        return (torch.from_numpy(k.view(np.int16)).cuda().contiguous(),
                torch.from_numpy(v.view(np.int16)).cuda().contiguous())

    pos = lens0.copy()
    for _ in range(n_single):
        k, v = batch_tokens(pos, 1)
        O.quantize_append(params, rot, pool, k, v)
        pos += 1
    torch.cuda.synchronize()
    assert np.array_equal(pool.seq_lens.cpu().numpy(), pos)
    k, v = batch_tokens(pos, n_bulk)
    O.quantize_append(params, rot, pool, k, v)
    pos += n_bulk
    torch.cuda.synchronize()
    assert np.array_equal(pool.seq_lens.cpu().numpy(), final)
    assert int(pool.error_flags.cpu()[0]) == 0

    pages = pool.pages.cpu().numpy()
    btc = pool.block_table.cpu().numpy()
    refs = []
    for b in range(wl.batch):
        L = int(final[b])
        kb, vb = toks[b]
        pools = [R.build_head_pool(_f64(kb[:, h]), _f64(vb[:, h]), cals[h]) for h in range(wl.n_kv)]
        n_hist = max(0, L - 320)
        for h in range(wl.n_kv):
            (kc, ks, kz), (vc, vs, vz) = gather_history(pages, btc[b], h, n_hist)
            ref = pools[h]
            assert np.array_equal(kc, ref.hist_k.codes), (b, h)
            assert np.array_equal(ks, ref.hist_k.s8) and np.array_equal(kz, ref.hist_k.z8), (b, h)
            assert np.array_equal(vc, ref.hist_v.codes), (b, h)
            assert np.array_equal(vs, ref.hist_v.s8) and np.array_equal(vz, ref.hist_v.z8), (b, h)
        refs.append(pools)
    # BF16 windows hold the raw tokens of the last 256 positions
    ring = pool.recent_k.cpu().numpy().view(np.uint16)
    for b in range(wl.batch):
        L = int(final[b])
        for p in range(max(64, L - 256), L):
            assert np.array_equal(ring[b, :, p % 256], toks[b][0][p]), (b, p)
    q = synth.decode_queries(wl, 0)
    for variant in (0, 1):
        out = _decode(params, rot, pool, q, variant)
        for b in range(wl.batch):
            want = R.decode_sequence(_f64(q[b]), refs[b], cals, 1 / np.sqrt(D))
            err = decode_check(out[b], want)
            print(f"batch append seq {b} (L {final[b]}) variant {variant}: err/||o|| = {err:.3e}", flush=True)
            assert err <= TOL


# ---------------------------------------------------------------------------
# peaked attention
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def tiny():
    wl = synth.WORKLOADS["tiny-4k"]
    cals = oracle_calibration(wl, n_cal=2048)
    rot = rotation_tensors(cals)
    params = O.make_params(wl.n_kv, wl.n_q)
    kb, vb = synth.kv_tokens(wl, 0, 0, 0, 4096)
    q = synth.decode_queries(wl, 0)
    return wl, cals, rot, params, kb, vb, q


def _run_case(tiny, kb, vb, q_bits, label):
    wl, cals, rot, params = tiny[:4]
    L = kb.shape[0]
    n_pages = (max(0, L - 320) + 63) // 64
    pool = O.KVPool(params, 1, max(n_pages, 1), np.arange(max(n_pages, 1), dtype=np.int32)[None])
    append_sequence(params, rot, pool, 0, kb, vb)
    ref_pool = R.build_head_pool(_f64(kb[:, 0]), _f64(vb[:, 0]), cals[0])
    want = R.decode_sequence(_f64(q_bits[0]), [ref_pool], cals, 1 / np.sqrt(D))
    for variant in (0, 1):
        out = _decode(params, rot, pool, q_bits, variant)
        err = decode_check(out[0], want)
        print(f"{label} variant {variant}: err/||o|| = {err:.3e} (tolerance {TOL})", flush=True)
        assert err <= TOL, (label, variant, err)


@pytest.mark.parametrize("scale", [8.0, 32.0])
def test_scaled_queries(tiny, scale):
    """Query norms x8 and x32: attention concentrates on the best-aligned keys
    and the query's fixed-point step grows with its norm."""
    _, _, _, _, kb, vb, q = tiny
    qs = _to_bits(_f64(q) * scale)
    _run_case(tiny, kb, vb, qs, f"query x{scale:g}")


@pytest.mark.parametrize("where", ["sink", "first_page", "middle_page", "last_page", "recent"])
@pytest.mark.parametrize("scale", [1.0, 8.0])
def test_dominant_key(tiny, where, scale):
    """One key aligned with query head 0 (and with a strongly shifted value),
    placed in each region of the pool; the other heads see diffuse
    attention."""
    _, _, _, _, kb, vb, q = tiny
    L = 4096
    pos = {"sink": 10, "first_page": 64 + 5, "middle_page": 64 + 29 * 64 + 40,
           "last_page": L - 256 - 3, "recent": L - 100}[where]
    qd = _f64(q)[0] * scale
    kb, vb = kb.copy(), vb.copy()
    d0 = qd[0] / np.linalg.norm(qd[0])
    kb[pos, 0] = _to_bits(d0 * 40.0)
    vb[pos, 0] = _to_bits(_f64(vb[pos, 0]) + 4.0)
    _run_case(tiny, kb, vb, _to_bits(qd[None]), f"dominant key in {where}, query x{scale:g}")


def test_logits_rise_page_by_page(tiny):
    """Every history page holds keys a little better aligned with the query
    than the page before (over 59 pages the aligned part grows from 0 to 6
    units per channel direction), so the running maximum of the scan moves
    past its headroom again and again."""
    _, _, _, _, kb, vb, q = tiny
    qd = _f64(q)[0]
    kb = kb.copy()
    kf = _f64(kb[:, 0])
    n_hist = 4096 - 320
    for t in range(n_hist):
        pg = t // 64
        h = pg % 4                                  # each page favours one query head in turn
        d = qd[h] / np.linalg.norm(qd[h])
        kf[64 + t] += d * (6.0 * pg / 58.0) * np.sqrt(D) / 4.0
    kb[:, 0] = _to_bits(kf)
    _run_case(tiny, kb, vb, q, "logits rising page by page")
