"""Every kind of launch the library makes, captured in one HIP graph and
replayed several times with eager work and synchronisations in between; each
replay must reproduce the eager results bit for bit (the library records no
memset nodes and allocates nothing, so capture is plain kernel nodes)."""
import numpy as np
import pytest
import torch

import oracle
from unstructured_sparse_linear_csr_amd import binding as sp
from unstructured_sparse_linear_csr_amd import inputs

from gpu_util import check_close, dev, host, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sp.lib()
    yield
    torch.cuda.synchronize()


def test_graph_of_long_row_and_sliced_launches():
    """The row-split SpMM (few, long rows) and the streaming SpMM over column
    slices of B held in LDS, captured and replayed the same way."""
    m1, k1, n1 = 96, 4096, 128
    lengths = np.random.default_rng(1300).integers(300, 3000, m1).astype(np.int32)
    rl1 = inputs.random_row_lists(1301, m1, k1, lengths)
    m2, k2, n2 = 16384, 8192, 8
    rl2 = inputs.random_row_lists(1302, m2, k2,
                                  np.random.default_rng(1303).integers(250, 360, m2).astype(np.int32))
    args = []
    for (m, k, n, rl, seed) in ((m1, k1, n1, rl1, 1304), (m2, k2, n2, rl2, 1305)):
        ro = dev(oracle.csr_offsets_from_lengths(rl.lengths))
        args.append((m, k, n, rl.nnz, ro, dev(rl.cols), dev(rl.values),
                     dev(inputs.random_dense(seed, k, n)), torch.empty(m, n, device="cuda")))

    def work():
        for (m, k, n, nnz, ro, ci, v, b, c) in args:
            sp.sp_spmm(m, k, n, nnz, None, v, ro, ci, b, c)

    note("graph of split and sliced launches: eager reference")
    work()
    torch.cuda.synchronize()
    want = [host(a[-1]).copy() for a in args]
    ref, s = oracle.spmm(m1, k1, n1, oracle.csr_offsets_from_lengths(rl1.lengths), rl1.cols,
                         rl1.values, host(args[0][7]))
    check_close(want[0], ref, s, "split rows in the graph test")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        work()
    for rep in range(3):
        note(f"split/sliced graph replay {rep}")
        for a in args:
            a[-1].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, w in zip(args, want):
            assert np.array_equal(host(a[-1]).view(np.int32), w.view(np.int32)), rep


def test_graph_of_every_launch_kind():
    w = inputs.transformer_ffn()
    a = w["a"]
    m, k, n, d, nnz = w["m"], w["k"], w["n"], w["d"], a.nnz
    lengths, cols, vals = dev(a.lengths), dev(a.cols), dev(a.values)
    b, x, y = dev(w["b"]), dev(w["x"]), dev(w["y"])
    prior = dev(inputs.random_dense(950, nnz))
    ro = torch.empty(m + 1, dtype=torch.int32, device="cuda")
    ri = torch.empty(m, dtype=torch.int32, device="cuda")
    ws = torch.empty(sp.sp_csr_transpose_workspace(m, k, nnz), dtype=torch.uint8, device="cuda")
    t_ro = torch.empty(k + 1, dtype=torch.int32, device="cuda")
    t_ci = torch.empty(nnz, dtype=torch.int32, device="cuda")
    t_v = torch.empty(nnz, device="cuda")
    t_p = torch.empty(nnz, dtype=torch.int32, device="cuda")
    t_ri = torch.empty(k, dtype=torch.int32, device="cuda")
    outs = {name: torch.empty(shape, device="cuda") for name, shape in {
        "c": (m, n), "c_bal": (m, n), "c_bf16": (m, n), "dx": (k, n), "s": (nnz,), "s_bal": (nnz,),
        "s_gen": (nnz,), "s_dk": (nnz,), "s_dkw": (nnz,), "p": (nnz,), "att": (m, d), "c_pair": (m, n),
        "s_pair": (nnz,)}.items()}
    b16, v16 = b.to(torch.bfloat16), vals.to(torch.bfloat16)
    y_dk = y.t().contiguous()
    y_ws = torch.empty(sp.sp_sddmm_general_workspace(k, d), dtype=torch.uint8, device="cuda")
    dy = dev(inputs.random_dense(951, m, n))

    def work():
        sp.sp_csr_build_from_lengths(m, lengths, ro, ri)
        sp.sp_spmm(m, k, n, nnz, ri, vals, ro, cols, b, outs["c"])
        sp.sp_spmm_balanced(m, k, n, nnz, ri, vals, ro, cols, b, outs["c_bal"])
        sp.sp_spmm_ex(m, k, n, nnz, ri, v16, ro, cols, b16, outs["c_bf16"])
        sp.sp_sddmm(m, k, d, nnz, ri, ro, cols, x, y, outs["s"])
        sp.sp_sddmm_balanced(m, k, d, nnz, ri, ro, cols, x, y, outs["s_bal"])
        outs["s_gen"].copy_(prior)
        sp.sp_sddmm_general(m, k, d, nnz, ri, ro, cols, vals, x, y, sp.SP_Y_KD, 0.5, 2.0,
                            outs["s_gen"])
        sp.sp_sddmm_general(m, k, d, nnz, ri, ro, cols, None, x, y_dk, sp.SP_Y_DK, 1.0, 0.0,
                            outs["s_dk"])
        sp.sp_sddmm_general(m, k, d, nnz, ri, ro, cols, vals, x, y_dk, sp.SP_Y_DK, 1.0, 0.0,
                            outs["s_dkw"], workspace=y_ws)
        sp.sp_sddmm_softmax(m, k, d, nnz, ri, ro, cols, x, y, 0.0625, outs["p"])
        sp.sp_csr_row_softmax(m, nnz, ri, ro, outs["s"], outs["s"])
        sp.sp_sparse_attention(m, m, d, nnz, ri, ro, cols, x, x, x, 0.0625, outs["att"])
        sp.sp_spmm_sddmm(m, k, n, nnz, ri, vals, ro, cols, b, outs["c_pair"], m, k, d, nnz, ri,
                         ro, cols, x, y, 1.0, outs["s_pair"])
        sp.sp_csr_transpose(m, k, nnz, ro, cols, vals, t_ro, t_ci, t_v, t_p, ws)
        sp.sp_csr_transpose_values(nnz, t_p, vals, t_v)
        sp.sp_row_swizzle(k, t_ro, t_ri)
        sp.sp_spmm(k, m, n, nnz, t_ri, t_v, t_ro, t_ci, dy, outs["dx"])

    note("graph of every launch kind: eager reference")
    work()
    torch.cuda.synchronize()
    want = {name: host(t).copy() for name, t in outs.items()}
    want["t_ro"], want["t_ci"] = host(t_ro).copy(), host(t_ci).copy()
    # the structure the graph computes must also be the oracle's
    assert np.array_equal(want["t_ro"], oracle.csr_transpose(m, k, oracle.csr_offsets_from_lengths(a.lengths), a.cols)[0])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    scratch = torch.empty(1 << 20, device="cuda")
    for rep in range(3):
        note(f"graph replay {rep}")
        for t in outs.values():
            t.fill_(float("nan"))
        t_ro.fill_(-1)
        t_ci.fill_(-1)
        scratch.normal_()  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t in outs.items():
            assert np.array_equal(host(t).view(np.int32), want[name].view(np.int32)), (rep, name)
        assert np.array_equal(host(t_ro), want["t_ro"]) and np.array_equal(host(t_ci), want["t_ci"])


def test_graph_of_panel_union_launches():
    """The panel-union kernels (batched scores, scores + softmax, P V and
    one-pass attention on a band mask, 4 heads) and the multi-row SDDMM (one
    batch entry of short rows), captured and replayed like the rest."""
    m, d, heads = 512, 64, 4
    lists = []
    for i in range(m):
        cols = set(range(max(0, i - 47), i + 1)) | set(range(0, max(0, i - 47), 64))
        lists.append(sorted(cols))
    lengths = np.array([len(c) for c in lists], np.int32)
    ro_np = oracle.csr_offsets_from_lengths(lengths)
    ci_np = np.concatenate([np.asarray(c, np.int32) for c in lists])
    nnz = int(ro_np[-1])
    ro, ci = dev(ro_np), dev(ci_np)
    q = dev(inputs.random_dense(960, heads, m, d))
    kk = dev(inputs.random_dense(961, heads, m, d))
    v = dev(inputs.random_dense(962, heads, m, d))
    pv = dev(np.abs(inputs.random_dense(963, heads, nnz)) / 48.0)
    short = inputs.random_row_lists(964, 300, 400, np.full(300, 5, np.int32))
    s_ro, s_ci = dev(oracle.csr_offsets_from_lengths(short.lengths)), dev(short.cols)
    sx, sy = dev(inputs.random_dense(965, 300, d)), dev(inputs.random_dense(966, 400, d))
    outs = {name: torch.empty(shape, device="cuda") for name, shape in {
        "s": (heads, nnz), "p": (heads, nnz), "o": (heads, m, d), "att": (heads, m, d),
        "short": (short.nnz,)}.items()}
    st = m * d
    assert sp.sp_sddmm_kernel_name(m, m, d, nnz, q, kk, heads, st, st, nnz) == "panel_union"
    assert sp.sp_spmm_kernel_name(m, m, d, nnz, pv, ci, v, outs["o"], heads, nnz, st,
                                  st) == "panel_union"
    assert sp.sp_sddmm_kernel_name(300, 400, d, short.nnz, sx, sy) == "multirow"

    def work():
        sp.sp_sddmm_batched(m, m, d, nnz, None, ro, ci, q, kk, 0.125, outs["s"], heads, st, st,
                            nnz)
        sp.sp_sddmm_softmax(m, m, d, nnz, None, ro, ci, q, kk, 0.125, outs["p"], heads, st, st,
                            nnz)
        sp.sp_spmm_batched(m, m, d, nnz, None, pv, ro, ci, v, outs["o"], heads, nnz, st, st)
        sp.sp_sparse_attention(m, m, d, nnz, None, ro, ci, q, kk, v, 0.125, outs["att"], heads,
                               st, st, st, st)
        sp.sp_sddmm(300, 400, d, short.nnz, None, s_ro, s_ci, sx, sy, outs["short"])

    note("graph of panel-union launches: eager reference")
    work()
    torch.cuda.synchronize()
    want = {name: host(t).copy() for name, t in outs.items()}
    s_ref, s_abs = oracle.sddmm(m, m, d, ro_np, ci_np, host(q)[0], host(kk)[0])
    check_close(want["s"][0], 0.125 * s_ref, 0.125 * s_abs, "union scores in the graph test")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(3):
        note(f"panel-union graph replay {rep}")
        for t in outs.values():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t in outs.items():
            assert np.array_equal(host(t).view(np.int32), want[name].view(np.int32)), (rep, name)
