"""The oracle's worker pool (no GPU): its jobs return what direct oracle calls
return, and summing the backward's per-run key gradients over a partition of
the rows gives the full gradients. The full-size GPU parity tests rely on it."""
import numpy as np

import oracle.pool as opool
import oracle.rswa as orc
import workloads as wl


def test_decode_sequence_job_matches_direct_calls():
    w = wl.DecodeWorkload("pool-decode", batch=2, heads=3, head_dim=64, ref_len=20, window=4, steps=9,
                          dtype="bf16", sigma_q=1.0, sigma_kv=1.0, base_seed=515)
    checks = [1, 4, 5, 9]
    with opool.SharedArrays() as arrays:
        kref, vref = wl.ref_kv_all(w)
        arrays.put("kref", kref)
        arrays.put("vref", vref)
        q, k, v = wl.steps_qkv(w, 1, w.steps)
        for name, a in (("q", q), ("k", k), ("v", v)):
            arrays.put(name, a)
        tasks = [(w.dtype, w.ref_len, w.window, w.scale, b, [0, 2], checks) for b in range(w.batch)]
        res = opool.pool_map(opool.decode_sequence_job, tasks, arrays, processes=2)
    f = lambda a: wl.to_f64(a, "bf16")
    for b in range(w.batch):
        for T in checks:
            first = max(1, T - w.window + 1)
            for i, h in enumerate([0, 2]):
                ref = orc.decode_output(f(q[T - 1, b, h]), f(kref[b, h]), f(vref[b, h]),
                                        f(k[first - 1:T, b, h]), f(v[first - 1:T, b, h]), first,
                                        w.ref_len, w.window, T, w.scale)
                np.testing.assert_array_equal(res[b][T][i], ref)


def test_masked_jobs_match_direct_calls():
    N, L_m, n, H = 90, 30, 8, 3
    mw = wl.MaskedWorkload("pool-masked", seq_len=N, heads=H, head_dim=64, ref_len=L_m, window=n,
                           dtype="bf16", sigma=1.0, base_seed=516)
    Q, K, V = (wl.bf16_bits_to_f32(a) for a in wl.packed_qkv(mw))
    G = wl.bf16_bits_to_f32(wl.packed_dout(mw))
    keys, hs = [0, 5, 29, 31, 60, 89], [0, 2]
    for mode in (orc.PREFIX_CAUSAL, orc.PREFIX_FULL):
        with opool.SharedArrays() as arrays:
            for name, a in (("Q", Q), ("K", K), ("V", V), ("dO", G)):
                arrays.put(name, a)
            rows = list(range(N))
            chunks = [rows[i::4] for i in range(4)]
            fw = opool.pool_map(opool.masked_rows_job, [(c, L_m, n, mw.scale, mode) for c in chunks],
                                arrays, processes=2)
            bw = opool.pool_map(opool.masked_bwd_keys_job,
                                [(c, keys, hs, L_m, n, mw.scale, mode) for c in chunks], arrays,
                                processes=2)
        Q64, K64, V64, G64 = (a.astype(np.float64) for a in (Q, K, V, G))
        for c, part in zip(chunks, fw):
            np.testing.assert_array_equal(part, orc.masked_attention_rows(Q64, K64, V64, c, L_m, n,
                                                                          mw.scale, mode))
        _, dK, dV = orc.masked_attention_backward(Q64[:, hs], K64[:, hs], V64[:, hs], G64[:, hs],
                                                  L_m, n, mw.scale, mode)
        np.testing.assert_allclose(sum(p[0] for p in bw), dK[keys], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(sum(p[1] for p in bw), dV[keys], rtol=1e-12, atol=1e-13)
