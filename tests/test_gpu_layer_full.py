"""GPU parity of the grouped expert layer at full size, in the launch
configuration bench.py times, on sampled outputs.

Workloads: the Qwen3-30B-A3B-shaped layer (E=128, H=2048, I=768, top-8) as
nvfp4 W4A4 over 16384 tokens with Zipf(1.1) load, w8a8 with uniform routing,
and w4afp8 and fp8 over 32768 tokens with Zipf(1.1) load.

The routing permutation is compared whole, bit for bit. The other outputs are
compared on three experts: the most loaded, the least loaded non-empty one and
the median. For each of them:

  * the fake-quant weights and all routed rows of X^ must be bit-exact;
  * H^ must be bit-exact except for a counted, bounded number of elements one
    grid step apart (the kernel's SiLU is within a few float32 ulps of the
    oracle's correctly rounded one);
  * the GEMM outputs on sampled rows must be within 1e-2;
  * the weight- and activation-scale gradients, reduced over every row of the
    expert, must be within 2e-3.

Each stage's oracle takes the device's own inputs to that stage, so a value that
lands on a rounding midpoint after a GEMM is the same on both sides. Also checked
bit-exact on sampled tokens: the combine, dX and dY_r. d topk_w is checked
within 2e-3."""
import numpy as np
import pytest

import synth
from oracle import codec, layer as OL, routing
from tests.fq_testutil import (assert_array_equal, assert_bits_equal, assert_fake_quant_near_bits,
                               check_gemm, check_scale_grad, torch)
from tests.layer_run import DeviceLayer, spec_for

pytestmark = pytest.mark.gpu

WORKLOADS = [("qwen3", "nvfp4"), ("qwen3u", "w8a8"), ("qwen3l", "w4afp8"), ("qwen3l", "fp8")]


def _rows(dl, name, idx, width, dtype=None):
    """Rows `idx` of a saved/workspace [R, width] buffer, gathered on the device."""
    T_ = torch()
    t = dl.buf(name, dtype or T_.bfloat16, (dl.L.R, width))
    return t[T_.as_tensor(np.asarray(idx, np.int64), device="cuda")].float().cpu().numpy()


def _guard(q, x, g, terms):
    B, R, C = np.shape(x)
    return codec._reduce_to_scale(q, np.abs(np.asarray(g) * terms["c"] * terms["dfac"]), B, R, C)


def _sample(lo, hi, rng, n=48):
    """Row indices of [lo, hi): the first and last rows of the expert (its first
    and ragged last tile) and n random rows."""
    m = hi - lo
    pick = set(range(lo, min(hi, lo + n))) | set(range(max(lo, hi - n), hi))
    if m > 2 * n:
        pick |= set((lo + rng.choice(m, size=n, replace=False)).tolist())
    return np.array(sorted(pick), np.int64)


@pytest.mark.parametrize("case_name,fmt", WORKLOADS, ids=[f"{c}-{f}" for c, f in WORKLOADS])
def test_full_size_layer_sampled(case_name, fmt):
    T_ = torch()
    case = synth.CASES[case_name]
    data = synth.make_layer(case)
    P = synth.layer_params(data, fmt)
    L = spec_for(fmt, case.E, case.H, case.I, case.T, case.k)
    k, H, I = L.k, L.H, L.I
    dl = DeviceLayer(L, data, P)
    dl.forward()
    dl.backward()
    T_.cuda.synchronize()
    print(f"[full] {case_name} {fmt}: device fwd+bwd done", flush=True)

    # F1: the whole permutation, bit-exact
    counts, offsets, src_of, row_of = routing.route(data["ids"], L.E)
    for n, ref in (("counts", counts), ("offsets", offsets), ("src_of", src_of), ("row_of", row_of)):
        assert_array_equal(dl.read(n), ref, n)

    nz = np.nonzero(counts)[0]
    order = nz[np.argsort(counts[nz], kind="stable")]
    experts = sorted({int(order[-1]), int(order[0]), int(order[len(order) // 2])})
    rng = np.random.default_rng(7)
    sa1, sa2 = P.get("s_a1"), P.get("s_a2")
    T_w1hat = dl.buf("w1hat", T_.bfloat16, (L.E, 2 * I, H)) if L.w1.enabled else None
    T_w2hat = dl.buf("w2hat", T_.bfloat16, (L.E, H, I)) if L.w2.enabled else None
    for e in experts:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        allr = np.arange(lo, hi)
        rows = _sample(lo, hi, rng)
        # F3 for this expert's matrices
        w1t = codec.fake_quant(L.w1, data["W1"][e:e + 1], None if P["s_w1"] is None else P["s_w1"][e:e + 1],
                               None if P["t_w1"] is None else P["t_w1"][e:e + 1])
        w2t = codec.fake_quant(L.w2, data["W2"][e:e + 1], None if P["s_w2"] is None else P["s_w2"][e:e + 1],
                               None if P["t_w2"] is None else P["t_w2"][e:e + 1])
        W1h, W2h = w1t["y"][0], w2t["y"][0]
        assert_bits_equal(T_w1hat[e].float().cpu().numpy(), W1h, f"W1^ expert {e}")
        assert_bits_equal(T_w2hat[e].float().cpu().numpy(), W2h, f"W2^ expert {e}")
        # F2: every routed row of the expert, bit-exact
        Xh = _rows(dl, "xhat", allr, H)
        tok = src_of[allr] // k
        a1 = OL.stage_act_quant(L.a1, data["X"][tok], sa1, e)
        assert_bits_equal(Xh, a1["y"][0], f"X^ expert {e}")
        # F4, F5, F6 on sampled rows
        s = rows - lo
        Z1 = _rows(dl, "z1", allr, 2 * I)
        check_gemm(Z1[s], OL.gemm_nt(Xh[s], W1h), f"Z1 expert {e}")
        h = OL.stage_swiglu(Z1, I)
        a2 = OL.stage_act_quant(L.a2, h, sa2, e)
        Hh = _rows(dl, "hhat", allr, I)
        assert_fake_quant_near_bits(Hh, a2, L.a2, f"H^ expert {e}")
        check_gemm(_rows(dl, "yr", rows, H), OL.gemm_nt(Hh[s], W2h), f"Y_r expert {e}")
        # B1 on sampled rows
        dYr = _rows(dl, "dyr", allr, H)
        assert_bits_equal(dYr[s], OL.stage_permute_dy(data["dY"], data["w"], src_of[rows], k), f"dY_r expert {e}")
        # B2
        dHh = _rows(dl, "dhhat", allr, I)
        check_gemm(dHh[s], OL.gemm_nn(dYr[s], W2h), f"dH^ expert {e}")
        # B4 (A2 STE + SwiGLU backward) and ds_a2 over all rows of the expert
        if L.a2.enabled:
            scale, tscale = OL._act_params(L.a2, sa2, e)
            dh, ds = codec.backward(L.a2, h[None], dHh[None].astype(np.float64), scale, tscale, terms=a2)
            dh = dh[0]
            if ds is not None:
                check_scale_grad(dl.g["ds_a2"][e:e + 1].cpu().numpy(), ds[:1],
                                 _guard(L.a2, h[None], dHh[None], a2).ravel()[:1], f"ds_a2 expert {e}")
        else:
            dh = dHh.astype(np.float64)
        dZ1 = _rows(dl, "dz1", allr, 2 * I)
        check_gemm(dZ1[s], OL.stage_swiglu_backward(Z1[s], dh[s], I), f"dZ1 expert {e}")
        # B5 on sampled rows; ds_a1 over all rows
        dXh = _rows(dl, "dxhat", allr, H)
        check_gemm(dXh[s], OL.gemm_nn(dZ1[s], W1h), f"dX^ expert {e}")
        if L.a1.has_param():
            scale, tscale = OL._act_params(L.a1, sa1, e)
            _, ds = codec.backward(L.a1, a1["x0"], dXh[None].astype(np.float64), scale, tscale, terms=a1)
            check_scale_grad(dl.g["ds_a1"][e:e + 1].cpu().numpy(), ds[:1],
                             _guard(L.a1, a1["x0"], dXh[None], a1).ravel()[:1], f"ds_a1 expert {e}")
        # B3, B6 + B8: weight-scale gradients of the expert from the device's operands.
        # The oracle's dW is exact (float64) while the device accumulates it in fp32
        # over the expert's rows, so the cancellation guard takes |g| <= |A|^T |B|.
        for n, q, W, t, A, B in (("ds_w1", L.w1, data["W1"][e:e + 1], w1t, dZ1, Xh),
                                 ("ds_w2", L.w2, data["W2"][e:e + 1], w2t, dYr, Hh)):
            if dl.g[n] is None:
                continue
            sc = P["s_" + n[3:]][e:e + 1]
            ts = None if P["t_" + n[3:]] is None else P["t_" + n[3:]][e:e + 1]
            _, ref = codec.backward(q, W, OL.gemm_tn(A, B)[None], sc, ts, terms=t)
            got = dl.g[n][e:e + 1].cpu().numpy()
            check_scale_grad(got, ref, _guard(q, W, OL.gemm_tn(np.abs(A), np.abs(B))[None], t),
                             f"{n} expert {e}")
        print(f"[full] expert {e} ({hi - lo} rows) ok", flush=True)

    # Every expert's weight-scale gradients, as a property: the weight-gradient
    # kernel deals the experts' tiles out to the XCDs, so an expert it never
    # reached would leave its gradients untouched.  Finite everywhere, and
    # nonzero for each expert with routed rows (the gradient of a random
    # layer vanishes nowhere in a whole expert's blocks).
    for n in ("ds_w1", "ds_w2"):
        if dl.g[n] is None:
            continue
        g_all = dl.g[n].float().cpu().numpy().reshape(L.E, -1)
        assert np.all(np.isfinite(g_all)), f"{n}: non-finite values"
        missing = [e for e in range(L.E) if counts[e] > 0 and not np.any(g_all[e] != 0)]
        assert not missing, f"{n}: experts with rows but no gradient: {missing[:10]}"

    # F7, B7 and d topk_w on sampled tokens, from the device's own Y_r and dX^
    toks = np.unique(np.concatenate([[0, L.T - 1], rng.choice(L.T, size=64, replace=False)]))
    rsel = row_of.reshape(L.T, k)[toks]
    nt = len(toks)
    loc = np.arange(nt * k)                      # local rows: token-major, slot j ascending
    Yr_t = _rows(dl, "yr", rsel.ravel(), H)
    w_t = data["w"][toks]
    got_y = dl.y[T_.as_tensor(toks, device="cuda")].float().cpu().numpy()
    assert_bits_equal(got_y, OL.stage_combine(Yr_t, loc, w_t, k), "y (sampled tokens)")
    dXh_t = _rows(dl, "dxhat", rsel.ravel(), H)
    dxt = dXh_t.astype(np.float64)
    if L.a1.enabled:
        ids_t = data["ids"][toks].ravel()
        for i in range(nt * k):
            e = int(ids_t[i])
            x_row = data["X"][toks[i // k]][None]
            a1 = OL.stage_act_quant(L.a1, x_row, sa1, e)
            scale, tscale = OL._act_params(L.a1, sa1, e)
            dxt[i] = codec.backward(L.a1, a1["x0"], dXh_t[i][None, None].astype(np.float64), scale, tscale,
                                    terms=a1)[0][0, 0]
    got_dx = dl.dx[T_.as_tensor(toks, device="cuda")].float().cpu().numpy()
    assert_bits_equal(got_dx, OL.stage_unpermute_sum(dxt, loc, nt, k), "dX (sampled tokens)")
    dy_t = data["dY"][toks]
    dw_ref = OL.stage_topk_weight_grad(dy_t, Yr_t, loc, nt, k)
    dw_abs = OL.stage_topk_weight_grad(np.abs(dy_t), np.abs(Yr_t), loc, nt, k)
    got_dw = dl.dw[T_.as_tensor(toks, device="cuda")].cpu().numpy()
    check_scale_grad(got_dw, dw_ref, dw_abs, "d topk_w (sampled tokens)")
