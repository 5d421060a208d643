"""A decode step captured in a HIP graph: single-token appends over a batch
and the decode (workspace entry point and the entry point that allocates
nothing), replayed several times with the program's own eager work and
synchronisations between the replays.  After every replay the graph's pool
must equal, bit for bit, a second pool driven by the same calls eagerly,
and its output must equal the eager output up to summation order; the
final state is also checked against the oracle."""
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


def test_graph_replays_match_eager():
    import torch
    wl = synth.Workload(160, "test-graph", 3, 2, 8, 128, 0, 1600, n_cal=512, outliers="pairs10",
                        scattered_pages=True)
    cals = oracle_calibration(wl, n_cal=512)
    rot = rotation_tensors(cals)
    params = O.make_params(wl.n_kv, wl.n_q)
    lens0 = np.array([300, 1000, 1500], np.int32)
    n_rep = 4
    final = lens0 + 1 + n_rep
    bt, total = synth.block_table(wl, final)
    toks = [synth.kv_tokens(wl, 0, b, 0, int(final[b])) for b in range(wl.batch)]
    pools = []
    for _ in range(2):
        pool = O.KVPool(params, wl.batch, total, bt)
        for b in range(wl.batch):
            append_sequence(params, rot, pool, b, toks[b][0][:lens0[b]], toks[b][1][:lens0[b]])
        pools.append(pool)
    pg, pe = pools   # graph pool, eager pool
    # one new token per sequence and one query per step (the same in every step)
    k1 = torch.from_numpy(np.stack([toks[b][0][lens0[b]:lens0[b] + 1] for b in range(wl.batch)]).view(np.int16)).cuda()
    v1 = torch.from_numpy(np.stack([toks[b][1][lens0[b]:lens0[b] + 1] for b in range(wl.batch)]).view(np.int16)).cuda()
    q = torch.from_numpy(synth.decode_queries(wl, 0).view(np.int16)).cuda()
    wsg = O.alloc_workspace(O.decode_workspace_size(params, wl.batch, pg.max_pages))
    wse = O.alloc_workspace(O.decode_workspace_size(params, wl.batch, pe.max_pages))
    outg = torch.zeros((wl.batch, wl.n_q, D), dtype=torch.float32, device="cuda")
    outg_na = torch.zeros_like(outg)
    oute = torch.zeros_like(outg)
    oute_na = torch.zeros_like(outg)

    def step(pool, ws, out, out_na):
        O.quantize_append(params, rot, pool, k1, v1)
        O.decode_attention(params, rot, pool, q, out, ws)
        O.decode_attention_noalloc(params, rot, pool, q, out_na)

    # the first step eagerly on both pools (it also sets up the no-allocation buffer)
    step(pg, wsg, outg, outg_na)
    step(pe, wse, oute, oute_na)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(pg, wsg, outg, outg_na)
    for rep in range(n_rep):
        outg.zero_()
        outg_na.zero_()
        g.replay()
        torch.cuda.synchronize()
        step(pe, wse, oute, oute_na)
        torch.cuda.synchronize()
        # eager work of the program between replays
        junk = torch.randn(1 << 20, device="cuda").square().sum()
        assert torch.isfinite(junk)
        assert np.array_equal(pg.seq_lens.cpu().numpy(), lens0 + 2 + rep)
        assert np.array_equal(pg.seq_lens.cpu().numpy(), pe.seq_lens.cpu().numpy())
        assert torch.equal(pg.pages, pe.pages) and torch.equal(pg.recent_k, pe.recent_k)
        assert torch.equal(pg.recent_v, pe.recent_v)
        og, oe = outg.cpu().numpy(), oute.cpu().numpy()
        ogn, oen = outg_na.cpu().numpy(), oute_na.cpu().numpy()
        for b in range(wl.batch):
            e1, e2 = decode_check(og[b], oe[b]), decode_check(ogn[b], oen[b])
            print(f"replay {rep} seq {b}: graph vs eager {e1:.2e}, no-alloc graph vs eager {e2:.2e}", flush=True)
            assert e1 <= 1e-5 and e2 <= 1e-5, (rep, b, e1, e2)
    assert int(pg.error_flags.cpu()[0]) == 0
    # the final graph state against the oracle: the pool holds lens0 + 1 + n_rep
    # tokens per sequence, the last n_rep + 1 of them the repeated new token
    pages = pg.pages.cpu().numpy()
    btc = pg.block_table.cpu().numpy()
    og = outg.cpu().numpy()
    for b in range(wl.batch):
        L0 = int(lens0[b])
        kb = np.concatenate([toks[b][0][:L0]] + [toks[b][0][L0:L0 + 1]] * (1 + n_rep))
        vb = np.concatenate([toks[b][1][:L0]] + [toks[b][1][L0:L0 + 1]] * (1 + n_rep))
        ref_pools = [R.build_head_pool(_f64(kb[:, h]), _f64(vb[:, h]), cals[h]) for h in range(wl.n_kv)]
        n_hist = max(0, len(kb) - 320)
        for h in range(wl.n_kv):
            (kc, ks, kz), (vc, vs, vz) = gather_history(pages, btc[b], h, n_hist)
            assert np.array_equal(kc, ref_pools[h].hist_k.codes) and np.array_equal(vc, ref_pools[h].hist_v.codes)
            assert np.array_equal(ks, ref_pools[h].hist_k.s8) and np.array_equal(vz, ref_pools[h].hist_v.z8)
        want = R.decode_sequence(_f64(synth.decode_queries(wl, 0)[b]), ref_pools, cals, 1 / np.sqrt(D))
        err = decode_check(og[b], want)
        print(f"graph final seq {b}: err/||o|| = {err:.3e}", flush=True)
        assert err <= TOL


@pytest.mark.parametrize("n_q", [8, 24])
def test_graph_replays_prefix_decode(n_q):
    """The shared-prefix decode (prefix_pages; query-operand, prefix-scan and
    scan launches) captured in a graph, workspace and no-allocation entry
    points: every replay, with eager work in between, equals the eager call
    up to summation order, and the oracle within tolerance."""
    import torch
    from test_gpu_prefix import _build, _oracle
    P = 6
    suffixes = [300, 500, 256, 700, 1000]
    wl, cals, rot, params, pool, toks, qb = _build(2, n_q, 5, P, suffixes, seed=501 + n_q)
    q = torch.from_numpy(qb.view(np.int16)).cuda().contiguous()
    ws = O.alloc_workspace(O.decode_workspace_size(params, pool.batch, pool.max_pages, prefix_pages=P))
    outg = torch.zeros((pool.batch, params.num_q_heads, D), dtype=torch.float32, device="cuda")
    outg_na, oute = torch.zeros_like(outg), torch.zeros_like(outg)

    def dec(out, out_na):
        O.decode_attention(params, rot, pool, q, out, ws, prefix_pages=P)
        if out_na is not None:
            O.decode_attention_noalloc(params, rot, pool, q, out_na, prefix_pages=P)

    dec(oute, outg_na)   # eager, and sets up the no-allocation buffer
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dec(outg, outg_na)
    for rep in range(3):
        outg.zero_()
        outg_na.zero_()
        g.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").square().sum()
        assert torch.isfinite(junk)
        dec(oute, None)
        torch.cuda.synchronize()
        og, ogn, oe = outg.cpu().numpy(), outg_na.cpu().numpy(), oute.cpu().numpy()
        e1, e2 = decode_check(og, oe), decode_check(ogn, oe)
        print(f"G={n_q // 2} replay {rep}: graph vs eager {e1:.2e}, no-alloc graph vs eager {e2:.2e}", flush=True)
        assert e1 <= 1e-5 and e2 <= 1e-5, (rep, e1, e2)
    assert int(pool.error_flags.cpu()[0]) == 0
    og = outg.cpu().numpy()
    for b in range(pool.batch):
        assert decode_check(og[b], _oracle(wl, cals, toks[b][0], toks[b][1], qb[b])) <= TOL, b
