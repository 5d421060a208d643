"""GPU parity of the Lloyd-Max codebook path (the 2-bit codes standing for
four per-head reconstruction levels): codes and metadata codes bit-exact with
the oracle through bulk and single-token appends, and decode within the
2e-3 tolerance on the MFMA scan (codebook lookup before the products) and on
the VALU scan, for one and several M-tiles of query heads.  The codebook
given to both sides is the oracle's calibration."""
import numpy as np
import pytest

from bit_rotated_kv_int2_amd import oscar as O
from bit_rotated_kv_int2_amd import synth
from oracle import oscar_ref as R
from pool_helpers import append_sequence, decode_check, gather_history, oracle_calibration, rotation_tensors

pytestmark = pytest.mark.gpu
D = 128
TOL = 2e-3


def _f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def _codebook_cals(wl, n_cal=512):
    cals = oracle_calibration(wl, n_cal=n_cal)
    _, k, v = synth.calibration_set(wl, 0, n_cal=n_cal)
    f = synth.bf16_bits_to_f32
    return [R.calibrate_codebook(c, f(k)[h], f(v)[h]) for h, c in enumerate(cals)]


def _decode(params, rot, pool, q_bits, variant):
    import torch
    ws = O.alloc_workspace(O.decode_workspace_size(params, pool.batch, pool.max_pages, variant))
    q = torch.from_numpy(np.ascontiguousarray(q_bits).view(np.int16)).cuda()
    out = torch.zeros((pool.batch, params.num_q_heads, D), dtype=torch.float32, device="cuda")
    O.decode_attention(params, rot, pool, q, out, ws, variant=variant)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("G", [4, 12])
def test_codebook_write_and_decode(G):
    """Three sequences of ragged length on scattered pages, two KV heads,
    G query heads per KV head; bulk appends then single-token appends."""
    wl = synth.Workload(140 + G, f"test-codebook-g{G}", 3, 2, 2 * G, 128, 500, 3333, n_cal=512,
                        outliers="pairs10", scattered_pages=True)
    cals = _codebook_cals(wl)
    assert any(not np.array_equal(c.levels_K, R.UNIFORM_LEVELS) for c in cals)
    rot = rotation_tensors(cals)
    params = O.make_params(wl.n_kv, wl.n_q)
    lens = np.array([3333, 500, 2049], np.int32)
    bt, total = synth.block_table(wl, lens)
    pool = O.KVPool(params, wl.batch, total, bt)
    toks = []
    for b in range(wl.batch):
        kb, vb = synth.kv_tokens(wl, 0, b, 0, int(lens[b]))
        toks.append((kb, vb))
        append_sequence(params, rot, pool, b, kb, vb, chunks=[int(lens[b]) - 5] + [1] * 5)
    assert int(pool.error_flags.cpu()[0]) == 0
    pages = pool.pages.cpu().numpy()
    btc = pool.block_table.cpu().numpy()
    refs = []
    for b in range(wl.batch):
        kb, vb = toks[b]
        pools = [R.build_head_pool(_f64(kb[:, h]), _f64(vb[:, h]), cals[h]) for h in range(wl.n_kv)]
        n_hist = max(0, int(lens[b]) - 320)
        for h in range(wl.n_kv):
            (kc, ks, kz), (vc, vs, vz) = gather_history(pages, btc[b], h, n_hist)
            assert np.array_equal(kc, pools[h].hist_k.codes), (b, h)
            assert np.array_equal(vc, pools[h].hist_v.codes), (b, h)
            assert np.array_equal(ks, pools[h].hist_k.s8) and np.array_equal(kz, pools[h].hist_k.z8)
            assert np.array_equal(vs, pools[h].hist_v.s8) and np.array_equal(vz, pools[h].hist_v.z8)
        refs.append(pools)
    q = synth.decode_queries(wl, 0)
    for variant in (0, 1):
        out = _decode(params, rot, pool, q, variant)
        for b in range(wl.batch):
            want = R.decode_sequence(_f64(q[b]), refs[b], cals, 1 / np.sqrt(D))
            err = decode_check(out[b], want)
            print(f"codebook G {G} seq {b} variant {variant}: err/||o|| = {err:.3e}", flush=True)
            assert err <= TOL


def test_uniform_words_match_the_default_grid():
    """Codebook words equal to the uniform grid give the same codes as no
    codebook (bit for bit) and a decode within summation-order differences
    of the default scan."""
    import torch
    wl = synth.WORKLOADS["tiny-4k"]
    cals = oracle_calibration(wl, n_cal=512)
    params = O.make_params(wl.n_kv, wl.n_q)
    plain = rotation_tensors(cals)
    words = torch.full((1,), O.UNIFORM_LEVELS, dtype=torch.int64).to(torch.int32).cuda()
    uni = O.RotationTensors(plain.U_K, plain.U_V, plain.tau_K, plain.tau_V, words, words.clone())
    kb, vb = synth.kv_tokens(wl, 0, 0, 0, 3000)
    pools = []
    for rot in (plain, uni):
        pool = O.KVPool(params, 1, 59, np.arange(59, dtype=np.int32)[None])
        append_sequence(params, rot, pool, 0, kb, vb, chunks=[2990] + [1] * 10)
        pools.append(pool)
    assert np.array_equal(pools[0].pages.cpu().numpy(), pools[1].pages.cpu().numpy())
    q = synth.decode_queries(wl, 0)
    a = _decode(params, plain, pools[0], q, 0)
    b = _decode(params, uni, pools[1], q, 0)
    assert decode_check(b[0], a[0]) <= 1e-5
