"""GPU parity of the shared-prefix decode (decode option prefix_pages).

Every sequence of a batch starts with the same sink tokens and the same P
history pages (one shared sink slot, equal block-table entries), followed by
a private suffix.  With prefix_pages = P the P pages are scanned once per KV
head for up to eight sequences at a time and merged into each sequence's
own scan.  The oracle knows nothing of the sharing: it decodes each
sequence from its full token stream.  Bar: max |o_gpu - o_ref| <= 2e-3
||o_ref|| per (sequence, head), as for the plain decode, and agreement with
the plain decode of the same pool within float32 summation order.
"""
import numpy as np
import pytest

from bit_rotated_kv_int2_amd import oscar as O
from bit_rotated_kv_int2_amd import synth
from oracle import oscar_ref as R
from pool_helpers import append_sequence, decode_check, oracle_calibration, rotation_tensors

pytestmark = pytest.mark.gpu
D = 128
TOL = 2e-3


def _f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def _build(n_kv, n_q, batch, P, suffixes, seed, scatter=True, codebook=False):
    """Pool of `batch` sequences sharing sink + P pages; suffix b has suffixes[b] tokens."""
    wl = synth.Workload(seed, f"test-prefix-{seed}", batch, n_kv, n_q, D, 1, 1, n_cal=512, outliers="pairs10")
    cals = oracle_calibration(wl, n_cal=512)
    if codebook:
        _, k, v = synth.calibration_set(wl, 0, n_cal=512)
        f = synth.bf16_bits_to_f32
        cals = [R.calibrate_codebook(c, f(k)[h], f(v)[h]) for h, c in enumerate(cals)]
    rot = rotation_tensors(cals)
    params = O.make_params(n_kv, n_q)
    prefix = 64 + 64 * P
    lens = [prefix + s for s in suffixes]
    pages = [(L - 320 + 63) // 64 for L in lens]
    max_pages = max(pages)
    n_phys = P + sum(p - P for p in pages)
    perm = np.random.default_rng(seed).permutation(n_phys).astype(np.int32) if scatter else np.arange(n_phys, dtype=np.int32)
    bt = np.full((batch, max_pages), -1, np.int32)
    nxt = P
    for b in range(batch):
        bt[b, :P] = perm[:P]
        for j in range(P, pages[b]):
            bt[b, j] = perm[nxt]
            nxt += 1
    pool = O.KVPool(params, batch, n_phys, bt, sink_slot=np.zeros(batch, np.int32), n_sink_slots=1)
    pk, pv = synth.kv_tokens(wl, 0, 0, 0, prefix)
    toks = []
    for b in range(batch):
        sk, sv = synth.kv_tokens(wl, 0, 100 + b, 0, suffixes[b])
        kb, vb = np.concatenate([pk, sk]), np.concatenate([pv, sv])
        toks.append((kb, vb))
        append_sequence(params, rot, pool, b, kb, vb, chunks=[prefix, suffixes[b]])
    q = synth.decode_queries(wl, 0)
    return wl, cals, rot, params, pool, toks, q


def _decode(params, rot, pool, q_bits, prefix_pages=0, blocks=0, noalloc=False):
    import torch
    q = torch.from_numpy(q_bits.view(np.int16)).cuda().contiguous()
    out = torch.zeros((pool.batch, params.num_q_heads, D), dtype=torch.float32, device="cuda")
    if noalloc:
        O.decode_attention_noalloc(params, rot, pool, q, out, blocks=blocks, prefix_pages=prefix_pages)
    else:
        ws = O.alloc_workspace(O.decode_workspace_size(params, pool.batch, pool.max_pages, 0, blocks, prefix_pages))
        O.decode_attention(params, rot, pool, q, out, ws, blocks=blocks, prefix_pages=prefix_pages)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _oracle(wl, cals, kb, vb, q_b):
    pools = [R.build_head_pool(_f64(kb[:, h]), _f64(vb[:, h]), cals[h]) for h in range(wl.n_kv)]
    return R.decode_sequence(_f64(q_b), pools, cals, 1 / np.sqrt(D))


@pytest.mark.parametrize("n_q,batch,P", [(24, 10, 11), (16, 3, 6), (32, 9, 5), (8, 10, 9), (4, 3, 4)])
def test_prefix_decode_matches_oracle(n_q, batch, P):
    """G = 12, 8, 16, 4 and 2; batches of 10 and 9 leave a second group of
    sequences with idle waves; ragged suffixes, some without private history
    pages and some ending in a partial page; scattered physical pages.
    Default grid (several prefix chunks) and blocks = 8 (one chunk, and one
    split per sequence and KV head, whose partial then goes to the merge
    instead of the output)."""
    base = [256, 257, 300, 320, 383, 384, 448, 700, 1000, 1500]
    suffixes = [base[(3 * b + P) % len(base)] for b in range(batch)]
    wl, cals, rot, params, pool, toks, q = _build(2, n_q, batch, P, suffixes, seed=200 + n_q + P)
    plain = _decode(params, rot, pool, q)
    worst = 0.0
    for blocks in (0, 8):
        out = _decode(params, rot, pool, q, prefix_pages=P, blocks=blocks)
        assert int(pool.error_flags.cpu()[0]) == 0
        for b in range(batch):
            ref = _oracle(wl, cals, toks[b][0], toks[b][1], q[b])
            e = decode_check(out[b], ref)
            worst = max(worst, e)
            assert e <= TOL, (b, blocks, e)
        # same pool, plain decode: the same sums in another order
        assert decode_check(out, plain) <= 1e-4, blocks
    print(f"G={n_q // 2} batch={batch} P={P}: worst error vs oracle {worst:.3e}")


def test_prefix_decode_noalloc_and_codebook():
    """The no-allocation entry point takes the prefix option too; with a
    codebook the prefix pages go through the level lookup like the rest."""
    suffixes = [300, 700, 1000]
    wl, cals, rot, params, pool, toks, q = _build(2, 24, 3, 7, suffixes, seed=311, codebook=True)
    assert any(not np.array_equal(c.levels_K, R.UNIFORM_LEVELS) for c in cals)
    out_ws = _decode(params, rot, pool, q, prefix_pages=7)
    out_na = _decode(params, rot, pool, q, prefix_pages=7, noalloc=True)
    assert np.array_equal(out_ws, out_na)
    assert int(pool.error_flags.cpu()[0]) == 0
    for b in range(3):
        assert decode_check(out_ws[b], _oracle(wl, cals, toks[b][0], toks[b][1], q[b])) <= TOL, b
    plain = _decode(params, rot, pool, q)
    assert decode_check(out_ws, plain) <= 1e-4


def test_prefix_decode_flags_bad_input():
    """A sequence whose prefix entries differ from sequence 0's sets the page
    flag; one shorter than the prefix sets the length flag; an out-of-range
    entry in the shared pages sets the page flag (the page is skipped).
    Every case stays in bounds: the prefix pages are sequence 0's."""
    import torch
    suffixes = [300, 400, 500]
    wl, cals, rot, params, pool, toks, q = _build(2, 24, 3, 6, suffixes, seed=377)
    bt_ok = pool.block_table.clone()

    def run(P):
        pool.error_flags.zero_()
        _decode(params, rot, pool, q, prefix_pages=P)
        return int(pool.error_flags.cpu()[0])

    assert run(6) == 0
    bt = bt_ok.clone()
    bt[2, 3] = bt_ok[2, 8]                    # sequence 2 points elsewhere in the prefix
    pool.block_table.copy_(bt)
    assert run(6) & O.DEVERR_PAGE
    pool.block_table.copy_(bt_ok)
    # a prefix longer than sequence 0's history (7 pages of 6 + 300 - 256 tokens)
    assert run(int(pool.max_pages)) & O.DEVERR_LENGTH
    bt = bt_ok.clone()
    bt[:, 2] = pool.n_pages + 5                # out of range for every sequence
    pool.block_table.copy_(bt)
    assert run(6) & O.DEVERR_PAGE
    pool.block_table.copy_(bt_ok)
    torch.cuda.synchronize()
    assert run(6) == 0


@pytest.mark.parametrize("n_q,batch", [(8, 3), (24, 3), (24, 1)])
def test_prefix_is_whole_history(n_q, batch):
    """Every sequence's history is exactly the shared prefix (prefix_pages =
    max_pages): the per-sequence scans have no pages of their own and only
    their BF16 windows and the prefix partials reach the merge."""
    P = 5
    wl, cals, rot, params, pool, toks, q = _build(2, n_q, batch, P, [256] * batch, seed=400 + n_q + batch)
    assert pool.max_pages == P
    out = _decode(params, rot, pool, q, prefix_pages=P)
    assert int(pool.error_flags.cpu()[0]) == 0
    for b in range(batch):
        e = decode_check(out[b], _oracle(wl, cals, toks[b][0], toks[b][1], q[b]))
        assert e <= TOL, (b, e)
    assert decode_check(out, _decode(params, rot, pool, q)) <= 1e-4
