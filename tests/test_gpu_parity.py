"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

Write path: codes and metadata codes (s8, z8) bit-exact with the oracle; bulk appends
bit-identical to sequential appends.  Decode: for every (sequence, query
head), max |o_gpu - o_ref| <= 2e-3 * ||o_ref||_2 (float32 accumulation on the
GPU, float64 oracle).  Inputs are seeded synthetic data from ``synth``; the
rotation artifact fed to both sides comes from the oracle's calibration.
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


def _torch():
    import torch
    return torch


def _tokens(wl, seq, L, layer=0):
    kb, vb = synth.kv_tokens(wl, layer, seq, 0, L)
    return kb, vb


def _f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def _decode_gpu(params, rot, pool, q_bits, variant, blocks=0):
    torch = _torch()
    ws = O.alloc_workspace(O.decode_workspace_size(params, pool.batch, pool.max_pages, variant, blocks))
    q = torch.from_numpy(q_bits.view(np.int16)).cuda().contiguous()
    out = torch.zeros((pool.batch, params.num_q_heads, D), dtype=torch.float32, device="cuda")
    O.decode_attention(params, rot, pool, q, out, ws, variant=variant, blocks=blocks)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _oracle_decode(wl, cals, kb, vb, q_bits_b):
    """Oracle output [Hq, d] for one sequence with tokens kb/vb [L, Hkv, d]."""
    pools = [R.build_head_pool(_f64(kb[:, h]), _f64(vb[:, h]), cals[h]) for h in range(wl.n_kv)]
    return R.decode_sequence(_f64(q_bits_b), pools, cals, 1 / np.sqrt(D)), pools


@pytest.fixture(scope="module")
def tiny():
    wl = synth.WORKLOADS["tiny-4k"]
    cals = oracle_calibration(wl, n_cal=2048)
    rot = rotation_tensors(cals)
    params = O.make_params(wl.n_kv, wl.n_q)
    kb, vb = _tokens(wl, 0, 4096)
    q = synth.decode_queries(wl, 0)
    return wl, cals, rot, params, kb, vb, q


def _fresh_pool(params, n_pages, batch=1):
    bt = np.arange(batch * n_pages, dtype=np.int32).reshape(batch, n_pages)
    return O.KVPool(params, batch, batch * n_pages, bt)


def test_write_bitexact_tiny(tiny):
    wl, cals, rot, params, kb, vb, _ = tiny
    L = 4096
    n_hist = L - 64 - 256
    pool = _fresh_pool(params, 59)
    append_sequence(params, rot, pool, 0, kb, vb)
    pages = pool.pages.cpu().numpy()
    (kc, ks, kz), (vc, vs, vz) = gather_history(pages, pool.block_table.cpu().numpy()[0], 0, n_hist)
    ref = R.build_head_pool(_f64(kb[:, 0]), _f64(vb[:, 0]), cals[0])
    assert np.array_equal(kc, ref.hist_k.codes)
    assert np.array_equal(ks, ref.hist_k.s8)
    assert np.array_equal(kz, ref.hist_k.z8)
    assert np.array_equal(vc, ref.hist_v.codes)
    assert np.array_equal(vs, ref.hist_v.s8)
    assert np.array_equal(vz, ref.hist_v.z8)
    # BF16 windows hold the raw tokens
    sink = pool.sink_k.cpu().numpy().view(np.uint16)[0, 0]
    assert np.array_equal(sink, kb[:64, 0])
    ring = pool.recent_v.cpu().numpy().view(np.uint16)[0, 0]
    for pos in range(L - 256, L):
        assert np.array_equal(ring[pos % 256], vb[pos, 0])
    assert int(pool.seq_lens.cpu()[0]) == L
    assert int(pool.error_flags.cpu()[0]) == 0


def test_sequential_appends_equal_bulk(tiny):
    wl, cals, rot, params, kb, vb, _ = tiny
    L = 2500
    a = _fresh_pool(params, 59)
    append_sequence(params, rot, a, 0, kb[:L], vb[:L])
    b = _fresh_pool(params, 59)
    chunks = [1, 63, 1, 255, 1, 17, 300, 1, 1, 1, 64, 129, 700]
    chunks.append(L - sum(chunks))
    append_sequence(params, rot, b, 0, kb[:L], vb[:L], chunks=chunks)
    assert np.array_equal(a.pages.cpu().numpy(), b.pages.cpu().numpy())
    assert np.array_equal(a.recent_k.cpu().numpy(), b.recent_k.cpu().numpy())
    assert np.array_equal(a.recent_v.cpu().numpy(), b.recent_v.cpu().numpy())
    assert np.array_equal(a.sink_k.cpu().numpy(), b.sink_k.cpu().numpy())


def test_single_token_appends(tiny):
    """Decode-time appends one token at a time past the window (demotion path)."""
    wl, cals, rot, params, kb, vb, _ = tiny
    L0, L1 = 330, 400
    a = _fresh_pool(params, 59)
    append_sequence(params, rot, a, 0, kb[:L1], vb[:L1], chunks=[L0] + [1] * (L1 - L0))
    pages = a.pages.cpu().numpy()
    n_hist = L1 - 320
    (kc, ks, kz), (vc, vs, vz) = gather_history(pages, a.block_table.cpu().numpy()[0], 0, n_hist)
    ref = R.build_head_pool(_f64(kb[:L1, 0]), _f64(vb[:L1, 0]), cals[0])
    assert np.array_equal(kc, ref.hist_k.codes) and np.array_equal(vc, ref.hist_v.codes)
    assert np.array_equal(vs, ref.hist_v.s8)


@pytest.mark.parametrize("variant", [0, 1])
def test_decode_tiny(tiny, variant):
    wl, cals, rot, params, kb, vb, q = tiny
    pool = _fresh_pool(params, 59)
    append_sequence(params, rot, pool, 0, kb, vb)
    out = _decode_gpu(params, rot, pool, q, variant)
    ref, _ = _oracle_decode(wl, cals, kb, vb, q[0])
    r = decode_check(out[0], ref)
    print(f"variant {variant}: max err / norm = {r:.3e}")
    assert r <= TOL


@pytest.mark.parametrize("L", [1, 63, 64, 65, 300, 320, 321, 383, 384, 385, 1000, 4095])
def test_decode_edge_lengths(tiny, L):
    wl, cals, rot, params, kb, vb, q = tiny
    pool = _fresh_pool(params, 59)
    append_sequence(params, rot, pool, 0, kb[:L], vb[:L])
    ref, _ = _oracle_decode(wl, cals, kb[:L], vb[:L], q[0])
    for variant in (0, 1):
        out = _decode_gpu(params, rot, pool, q, variant)
        assert decode_check(out[0], ref) <= TOL, (L, variant)


def test_decode_empty_sequence(tiny):
    wl, cals, rot, params, kb, vb, q = tiny
    pool = _fresh_pool(params, 59)
    out = _decode_gpu(params, rot, pool, q, 0)
    assert np.all(out == 0)


def test_batch_scattered_ragged():
    """Several sequences, two KV heads (G = 4), pages scattered by a seeded
    permutation, ragged lengths with partial last pages."""
    wl = synth.Workload(90, "test-scattered", 3, 2, 8, 128, 700, 2222, n_cal=512, outliers="pairs10",
                        scattered_pages=True)
    cals = oracle_calibration(wl, n_cal=512)
    rot = rotation_tensors(cals)
    params = O.make_params(wl.n_kv, wl.n_q)
    lens = np.array([700, 1500, 2222], np.int32)
    bt, total = synth.block_table(wl, lens)
    pool = O.KVPool(params, wl.batch, total, bt)
    toks = []
    for b in range(wl.batch):
        kb, vb = synth.kv_tokens(wl, 0, b, 0, int(lens[b]))
        toks.append((kb, vb))
        append_sequence(params, rot, pool, b, kb, vb, chunks=[int(lens[b]) - 3, 1, 1, 1])
    q = synth.decode_queries(wl, 0)
    for variant in (0, 1):
        out = _decode_gpu(params, rot, pool, q, variant)
        for b in range(wl.batch):
            ref, _ = _oracle_decode(wl, cals, toks[b][0], toks[b][1], q[b])
            assert decode_check(out[b], ref) <= TOL, (b, variant)
    assert int(pool.error_flags.cpu()[0]) == 0


def test_ragged_batch_mixed_page_orders():
    """One launch whose workgroups take different page orders: four
    sequences of ragged length (3000 to 41000 tokens, two KV heads, pages
    scattered) on two splits of ceil(636 / 2) pages, so that some
    workgroups keep the static order (under 48 pages), some hand pages out
    dynamically after four early tiles (48 to 191) and some are long scans
    (192 and more, every tile after the pages)."""
    wl = synth.Workload(95, "test-mixed-order", 4, 2, 8, 128, 3000, 41000, n_cal=512, outliers="pairs10",
                        scattered_pages=True)
    cals = oracle_calibration(wl, n_cal=512)
    rot = rotation_tensors(cals)
    params = O.make_params(wl.n_kv, wl.n_q)
    lens = np.array([3000, 9000, 23000, 41000], np.int32)
    n_pg = (lens - 320 + 63) // 64
    pps = (int(n_pg.max()) + 1) // 2                # pages per split
    per_wg = np.concatenate([np.minimum(n_pg, pps), np.maximum(n_pg - pps, 0)])
    assert (per_wg[per_wg > 0] < 48).any() and ((per_wg >= 48) & (per_wg < 192)).any() and (per_wg >= 192).any()
    bt, total = synth.block_table(wl, lens)
    pool = O.KVPool(params, wl.batch, total, bt)
    toks = []
    for b in range(wl.batch):
        kb, vb = synth.kv_tokens(wl, 0, b, 0, int(lens[b]))
        toks.append((kb, vb))
        append_sequence(params, rot, pool, b, kb, vb)
    q = synth.decode_queries(wl, 0)
    out = _decode_gpu(params, rot, pool, q, 0, blocks=2 * wl.batch * wl.n_kv)   # two splits per (sequence, KV head)
    for b in range(wl.batch):
        ref, _ = _oracle_decode(wl, cals, toks[b][0], toks[b][1], q[b])
        assert decode_check(out[b], ref) <= TOL, b
    assert int(pool.error_flags.cpu()[0]) == 0


@pytest.mark.parametrize("G", [1, 2, 3, 5, 8, 16])
def test_decode_group_sizes(G):
    """Query heads per KV head from 1 to 16: one, two and four M-tiles of
    four heads, partly filled tiles (G = 1, 2, 3, 5), two KV heads, two
    sequences of ragged length (partial last page); every decode variant."""
    wl = synth.Workload(100 + G, f"test-g{G}", 2, 2, 2 * G, 128, 900, 1700, n_cal=256, outliers="pairs10",
                        scattered_pages=True)
    cals = oracle_calibration(wl, n_cal=256)
    rot = rotation_tensors(cals)
    params = O.make_params(wl.n_kv, wl.n_q)
    lens = np.array([1700, 931], np.int32)
    bt, total = synth.block_table(wl, lens)
    pool = O.KVPool(params, wl.batch, total, bt)
    toks = []
    for b in range(wl.batch):
        kb, vb = synth.kv_tokens(wl, 0, b, 0, int(lens[b]))
        toks.append((kb, vb))
        append_sequence(params, rot, pool, b, kb, vb, chunks=[int(lens[b]) - 1, 1])
    q = synth.decode_queries(wl, 0)
    refs = [_oracle_decode(wl, cals, toks[b][0], toks[b][1], q[b])[0] for b in range(wl.batch)]
    for variant in (0, 1):
        out = _decode_gpu(params, rot, pool, q, variant)
        for b in range(wl.batch):
            err = decode_check(out[b], refs[b])
            print(f"G {G} variant {variant} seq {b}: max err / norm = {err:.3e}", flush=True)
            assert err <= TOL, (G, b, variant, err)
    assert int(pool.error_flags.cpu()[0]) == 0


def test_ragged_batch_empty_and_short_sequences():
    """Sixteen sequences x eight KV heads (G = 4) of very different lengths
    (empty, windows only, one partial page, up to 41 pages), pages scattered,
    two splits per (sequence, KV head): some splits have no pages, some only
    BF16 tiles.  Every decode variant must match the oracle; empty sequences
    give zeros."""
    wl = synth.Workload(91, "test-balanced", 16, 8, 32, 128, 0, 2950, n_cal=512, outliers="pairs10",
                        scattered_pages=True)
    cals = oracle_calibration(wl, n_cal=512)
    rot = rotation_tensors(cals)
    params = O.make_params(wl.n_kv, wl.n_q)
    lens = np.array([0, 1, 70, 320, 321, 385, 900, 1800, 2950, 2222, 64, 2000, 1234, 333, 2949, 1500], np.int32)
    bt, total = synth.block_table(wl, lens)
    pool = O.KVPool(params, wl.batch, total, bt)
    toks = []
    for b in range(wl.batch):
        kb, vb = synth.kv_tokens(wl, 0, b, 0, int(lens[b]))
        toks.append((kb, vb))
        if lens[b]:
            append_sequence(params, rot, pool, b, kb, vb)
    q = synth.decode_queries(wl, 0)
    for variant in (0, 1):
        out = _decode_gpu(params, rot, pool, q, variant)
        for b in range(wl.batch):
            if lens[b] == 0:
                assert np.all(out[b] == 0), (b, variant)
                continue
            ref, _ = _oracle_decode(wl, cals, toks[b][0], toks[b][1], q[b])
            assert decode_check(out[b], ref) <= TOL, (b, variant)
    assert int(pool.error_flags.cpu()[0]) == 0


def test_shared_prefix_gqa12():
    """G = 12 query heads per KV head; two sequences share the sink slot and
    the prefix pages (same physical page ids), private suffixes."""
    wl = synth.Workload(91, "test-prefix", 2, 1, 12, 128, 1600, 1600, n_cal=512, outliers="pairs10")
    cals = oracle_calibration(wl, n_cal=512)
    rot = rotation_tensors(cals)
    params = O.make_params(wl.n_kv, wl.n_q)
    prefix = 64 + 8 * 64            # sink + 8 whole pages
    L = 1600
    n_pages = (L - 320 + 63) // 64
    bt = np.zeros((2, n_pages), np.int32)
    bt[0] = np.arange(n_pages)
    bt[1, :8] = np.arange(8)
    bt[1, 8:] = np.arange(n_pages, 2 * n_pages - 8)
    pool = O.KVPool(params, 2, 2 * n_pages - 8, bt, sink_slot=[0, 0], n_sink_slots=1)
    pk, pv = synth.kv_tokens(wl, 0, 0, 0, prefix)
    toks = []
    for b in range(2):
        sk, sv = synth.kv_tokens(wl, 0, 10 + b, 0, L - prefix)
        kb = np.concatenate([pk, sk])
        vb = np.concatenate([pv, sv])
        toks.append((kb, vb))
        append_sequence(params, rot, pool, b, kb, vb, chunks=[prefix, L - prefix])
    q = synth.decode_queries(wl, 0)
    for variant in (0, 1):
        out = _decode_gpu(params, rot, pool, q, variant)
        for b in range(2):
            ref, _ = _oracle_decode(wl, cals, toks[b][0], toks[b][1], q[b])
            assert decode_check(out[b], ref) <= TOL, (b, variant)


def test_single_workgroup_long_history(tiny):
    """One scan workgroup over a 150K-token history on scattered pages: each of
    its waves takes more than 192 pages, so the block-table entries it holds
    in registers run out and are reloaded in the middle of the scan."""
    wl, cals, rot, params, _, _, q = tiny
    L = 150_000
    kb, vb = _tokens(wl, 1, L)
    n_pages = (L - 64 - 256 + 63) // 64
    assert n_pages // 12 > 192
    perm = np.random.default_rng(7).permutation(n_pages).astype(np.int32)
    pool = O.KVPool(params, 1, n_pages, perm[None])
    append_sequence(params, rot, pool, 0, kb, vb)
    out = _decode_gpu(params, rot, pool, q, 0, blocks=1)
    ref, _ = _oracle_decode(wl, cals, kb, vb, q[0])
    err = decode_check(out[0], ref)
    print(f"150K tokens, one workgroup: err/||o|| = {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("blocks", [1, 2, 3, 8])
def test_dynamic_page_order(tiny, blocks):
    """Workgroups of 48 and more pages hand their pages (and the BF16 tiles
    not taken before the pages) out to the waves dynamically: one to eight
    workgroups over a 40037-token history (621 pages, the last one partly
    filled), so that the workgroups of the later splits also take tiles
    u = split + S k and the last split owns the partial page.  With 8
    workgroups (78 pages each) waves 0..3 take four tiles first."""
    wl, cals, rot, params, _, _, q = tiny
    L = 40037
    kb, vb = _tokens(wl, 2, L)
    n_pages = (L - 64 - 256 + 63) // 64
    assert n_pages // blocks >= 2 * 12 * 2 and (L - 320) % 64
    perm = np.random.default_rng(11).permutation(n_pages).astype(np.int32)
    pool = O.KVPool(params, 1, n_pages, perm[None])
    append_sequence(params, rot, pool, 0, kb, vb)
    out = _decode_gpu(params, rot, pool, q, 0, blocks=blocks)
    ref, _ = _oracle_decode(wl, cals, kb, vb, q[0])
    err = decode_check(out[0], ref)
    print(f"40037 tokens, {blocks} workgroup(s): err/||o|| = {err:.3e}")
    assert err <= TOL


def test_dynamic_page_order_bad_entries_flagged(tiny):
    """Out-of-range block-table entries on the dynamic page order (one
    workgroup over 621 pages): a prologue page, a page handed out by the
    counter and the partly filled last page are skipped and flagged, and the
    output stays finite."""
    wl, cals, rot, params, _, _, q = tiny
    L = 40037
    kb, vb = _tokens(wl, 2, L)
    n_pages = (L - 64 - 256 + 63) // 64
    pool = O.KVPool(params, 1, n_pages, np.arange(n_pages, dtype=np.int32)[None])
    append_sequence(params, rot, pool, 0, kb, vb)
    bt = pool.block_table.clone()
    for i in (5, 300, n_pages - 1):
        pool.block_table[0, i] = 1 << 20
    try:
        out = _decode_gpu(params, rot, pool, q, 0, blocks=1)
    finally:
        pool.block_table.copy_(bt)
    assert np.all(np.isfinite(out))
    assert int(pool.error_flags.cpu()[0]) & O.DEVERR_PAGE


def test_bad_block_table_entry_flagged(tiny):
    wl, cals, rot, params, kb, vb, q = tiny
    pool = _fresh_pool(params, 59)
    append_sequence(params, rot, pool, 0, kb, vb)
    torch = _torch()
    bt = pool.block_table.clone()
    pool.block_table[0, 5] = 1 << 20          # outside [0, n_pages): skipped, flagged
    out = _decode_gpu(params, rot, pool, q, 0)
    assert np.all(np.isfinite(out))
    assert int(pool.error_flags.cpu()[0]) & O.DEVERR_PAGE
    pool.block_table.copy_(bt)


def test_bf16_baseline_decode(tiny):
    """In-house BF16 decode on the raw bf16 tokens equals exact attention."""
    torch = _torch()
    wl, cals, rot, params, kb, vb, q = tiny
    L = 4000
    n_pages = (L + 63) // 64
    cache = O.Bf16Cache(params, 1, n_pages, np.arange(n_pages, dtype=np.int32)[None])
    kt = np.zeros((n_pages * 64, 1, D), np.uint16)
    vt = np.zeros_like(kt)
    kt[:L], vt[:L] = kb[:L], vb[:L]
    cache.k_pages.copy_(torch.from_numpy(kt.reshape(n_pages, 64, 1, D).transpose(0, 2, 1, 3).copy().view(np.int16)))
    cache.v_pages.copy_(torch.from_numpy(vt.reshape(n_pages, 64, 1, D).transpose(0, 2, 1, 3).copy().view(np.int16)))
    cache.seq_lens.fill_(L)
    ws = O.alloc_workspace(O.bf16_workspace_size(params, 1, n_pages))
    qt = torch.from_numpy(q.view(np.int16)).cuda()
    out = torch.zeros((1, wl.n_q, D), dtype=torch.float32, device="cuda")
    O.bf16_decode_attention(params, cache, qt, out, ws)
    torch.cuda.synchronize()
    ref = R.attention_dense(_f64(q[0]), _f64(kb[:L, 0]), _f64(vb[:L, 0]), 1 / np.sqrt(D))
    assert decode_check(out.cpu().numpy()[0], ref) <= TOL


def test_decode_repeat_same_workspace(tiny):
    """Consecutive decodes sharing one workspace all match the oracle and one
    another (the completion counters return to zero after every call; a
    counter left behind would skip or misplace a later call's merge).  The
    BF16 tiles go to the waves of a workgroup in the order they finish their
    pages, so repeats may differ in summation order only."""
    torch = _torch()
    wl, cals, rot, params, kb, vb, q = tiny
    pool = _fresh_pool(params, 59)
    append_sequence(params, rot, pool, 0, kb, vb)
    ws = O.alloc_workspace(O.decode_workspace_size(params, 1, pool.max_pages))
    qt = torch.from_numpy(q.view(np.int16)).cuda()
    outs = []
    for _ in range(3):
        out = torch.zeros((1, wl.n_q, D), dtype=torch.float32, device="cuda")
        O.decode_attention(params, rot, pool, qt, out, ws)
        outs.append(out)
    torch.cuda.synchronize()
    ref, _ = _oracle_decode(wl, cals, kb, vb, q[0])
    first = outs[0].cpu().numpy()[0]
    for o in outs:
        o = o.cpu().numpy()[0]
        assert decode_check(o, ref) <= TOL
        assert decode_check(o, first) <= 1e-5



@pytest.mark.parametrize("kind", ["naive", "clip", "hadamard"])
def test_quantiser_variants_parity(tiny, kind):
    """The quantiser variants of the diagnostics (naive INT2, clip only,
    Hadamard only) differ from OSCAR only in U and tau, so the library runs
    them unchanged: codes and metadata bit-exact, decode within tolerance."""
    from oracle import variants as V
    torch = _torch()
    wl, cals, _, params, kb, vb, q = tiny
    _, kc, vc = synth.calibration_set(wl, 0, n_cal=2048)
    vcal = [V.variant_calibration(kind, cals[0], _f64(kc[0]), _f64(vc[0]))]
    vrot = rotation_tensors(vcal)
    pool = _fresh_pool(params, 59)
    append_sequence(params, vrot, pool, 0, kb, vb)
    torch.cuda.synchronize()
    (kc_, ks, kz), (vc_, vs, vz) = gather_history(pool.pages.cpu().numpy(), pool.block_table.cpu().numpy()[0], 0,
                                                  4096 - 320)
    ref = R.build_head_pool(_f64(kb[:, 0]), _f64(vb[:, 0]), vcal[0])
    assert np.array_equal(kc_, ref.hist_k.codes) and np.array_equal(vc_, ref.hist_v.codes)
    assert np.array_equal(ks, ref.hist_k.s8) and np.array_equal(kz, ref.hist_k.z8)
    assert np.array_equal(vs, ref.hist_v.s8) and np.array_equal(vz, ref.hist_v.z8)
    out = _decode_gpu(params, vrot, pool, q, 0)
    want = R.decode_sequence(_f64(q[0]), [ref], vcal, 1 / np.sqrt(D))
    err = decode_check(out[0], want)
    print(f"variant {kind}: max err / norm = {err:.3e}")
    assert err <= TOL
    assert int(pool.error_flags.cpu()[0]) == 0


def test_stream_read_probe_reads_every_word():
    """The benchmark's streaming-read probe (its own helper library) covers the
    whole buffer: the xor of its per-thread checksums is the xor of every
    32-bit word (16 MiB = two full grid strides of 256 x 512 threads x 4
    words of 16 bytes)."""
    import ctypes
    from bit_rotated_kv_int2_amd import build as B
    torch = _torch()
    probe = ctypes.CDLL(B.PROBE_LIB_PATH)
    probe.bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_void_p]
    probe.bench_stream_read.restype = ctypes.c_int
    g = torch.Generator().manual_seed(3)
    host = torch.randint(-2**31, 2**31 - 1, (4 << 20,), dtype=torch.int64, generator=g).to(torch.int32)
    buf = host.cuda()
    sink = torch.empty(256 * 512, dtype=torch.int32, device="cuda")
    assert probe.bench_stream_read(buf.data_ptr(), buf.numel() * 4, sink.data_ptr(), 256,
                                   torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want
