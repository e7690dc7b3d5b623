"""Kernel-level GPU checks through the C ABI: flatten edge cases (every source
misalignment, per-bucket calls in any order, nonfinite values at edges),
the standalone parameter cast over a sweep of fp32 patterns, overflow skips
leaving state bit-identical, resume, the R-rank simulation, the device
input generator, and the timing entry points."""
import numpy as np
import pytest

import oracle
import synth
import zero_partitioned_mixed_plan_amd as z
from harness import Case, DeviceRun, OracleRun, log, to_device_grad, torch_dtype

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _bits(t):
    import torch
    if t.dtype == torch.float32:
        return t.view(torch.int32).cpu().numpy().view(np.uint32)
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _to_dev_half(bits, dt):
    """Gradient bits (uint16, or uint32 for "f32") as a device tensor."""
    return to_device_grad(np.ascontiguousarray(bits), dt, DEV)


def test_device_generator_matches_host_bit_for_bit():
    import torch
    for (k, i0, n, sig, sc, p, mult) in [(synth.key(0, 1, 1), 0, 1 << 20, 1e-3, 1.0, 0.0, 1.0),
                                         (synth.key(7, 1, 3), 12345678901, 300001, 1e-3, 65536.0,
                                          0.0, 1.0),
                                         (synth.key(0, 1, 2), 3 << 30, 200000, 1e-3, 1.0, 0.01,
                                          100.0)]:
        d = torch.empty(n, dtype=torch.float32, device=DEV)
        synth.dev_fill_f32(d, k, i0, sig, sc, synth.outlier_thresh(p), mult)
        h = synth.host_values(k, i0, n, sig, sc, synth.outlier_thresh(p), mult)
        assert np.array_equal(d.cpu().numpy().view(np.uint32), h.view(np.uint32))
        for dt in ("f16", "bf16"):
            dh = torch.empty(n, dtype=torch_dtype(dt), device=DEV)
            synth.dev_fill_half(dh, k, i0, sig, sc, synth.outlier_thresh(p), mult, chunk=65536)
            assert np.array_equal(_bits(dh), synth.half_bits(h, dt))


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_flatten_every_source_misalignment(dt):
    """Tensors are views at element offsets 0..7 of one buffer, so their
    sources sit at every 2-byte misalignment of a 16-byte block (every
    4-byte one for fp32 gradients)."""
    import torch
    rng = np.random.default_rng(3)
    numels = [5000, 4099, 2048, 3, 70000, 1, 2047, 9000, 4097, 12345, 600, 8191]
    R, A = 3, 8
    for r in range(R):
        op = oracle.plan(numels, R, r, A, bucket_elems=9000)
        plan = z.zero_partition_plan(numels, R, r, A, 9000)
        big = torch.empty(sum(numels) + 16 * len(numels) + 64, dtype=torch_dtype(dt), device=DEV)
        host, views, off = [], [], 0
        for i, n in enumerate(numels):
            mis = i % 8
            off += mis
            bits = synth.grad_bits(rng.normal(0, 1e-2, n).astype(np.float32), dt)
            v = big[off:off + n]
            v.copy_(_to_dev_half(bits, dt))
            host.append(bits)
            views.append(v)
            off += n + (8 - (off + n) % 8)
        expect = oracle.flatten(op, host)
        bound = z.GradList(plan, views)
        for mode in ("all", "buckets", "reverse", "bound", "bound buckets"):
            flat = torch.full((max(op.S, 8),), float("nan"), dtype=torch_dtype(dt), device=DEV)
            if mode == "all":
                z.zero_flatten_grads(plan, -1, views, flat)
            elif mode == "bound":
                z.zero_flatten_grads(plan, -1, bound, flat)
            elif mode == "bound buckets":  # one bound list serves every bucket
                for b in range(plan.n_buckets):
                    z.zero_flatten_grads(plan, b, bound, flat)
            else:
                tb = plan.tensor_buckets()
                order = range(plan.n_buckets) if mode == "buckets" else \
                    reversed(range(plan.n_buckets))
                for b in order:
                    z.zero_flatten_grads(plan, b, [v if tb[i] == b else None
                                                   for i, v in enumerate(views)], flat)
            got = _bits(flat)[:op.S]
            assert np.array_equal(got, expect), (r, mode)


# The flatten copies tiles of 2048 16-bit words and, within each launch,
# hands every XCD runs of 256 consecutive tiles over the largest whole
# multiple of 2048 tiles; the remaining tiles keep dispatch order.  These
# sizes put a launch just below, at and past such multiples, with ragged
# last tiles and misaligned sources.
_TILE_WORDS = 2048
_RUN_TILES = 2048


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_flatten_tile_runs_at_launch_size_edges(dt):
    import torch
    wpe = 2 if dt == "f32" else 1  # 16-bit words per element
    rng = np.random.default_rng(17)
    for n_tiles, last in [(2047, 2048), (2048, 1000), (2048, 2048), (2049, 3), (5001, 77)]:
        words = (n_tiles - 1) * _TILE_WORDS + last
        E = words // wpe
        cuts = np.sort(rng.choice(np.arange(1, E), 6, replace=False))
        numels = np.diff(np.concatenate([[0], cuts, [E]])).tolist()
        op = oracle.plan(numels, 1, 0, 8, bucket_elems=E // 3)
        plan = z.zero_partition_plan(numels, 1, 0, 8, E // 3)
        assert -(-(op.real * wpe) // _TILE_WORDS) == n_tiles
        big = torch.empty(E + 16 * len(numels) + 64, dtype=torch_dtype(dt), device=DEV)
        host, views, off = [], [], 0
        for i, n in enumerate(numels):
            off += (2 * i + 1) % 8  # every source misaligned
            bits = synth.grad_bits(rng.normal(0, 1e-2, n).astype(np.float32), dt)
            big[off:off + n].copy_(_to_dev_half(bits, dt))
            host.append(bits)
            views.append(big[off:off + n])
            off += n
        expect = oracle.flatten(op, host)
        for mode in ("all", "buckets"):
            flat = torch.full((op.S,), float("nan"), dtype=torch_dtype(dt), device=DEV)
            if mode == "all":
                z.zero_flatten_grads(plan, -1, views, flat)
            else:
                for b in range(plan.n_buckets):
                    z.zero_flatten_grads(plan, b, views, flat)
            assert np.array_equal(_bits(flat), expect), (n_tiles, last, mode)
        log(f"[kernels] tile runs {dt}: {n_tiles} tiles, last {last} words: flat bit-equal")


@pytest.mark.parametrize("dt", ["f16", "f32"])
def test_overflow_inside_and_after_the_tile_runs(dt):
    # one tensor of 2048 + 3 tiles: an inf in the remapped region (first,
    # middle and last tile of the runs) and in the tail tile is each found
    wpe = 2 if dt == "f32" else 1
    n = (_RUN_TILES * _TILE_WORDS + 3 * _TILE_WORDS - 100) // wpe
    bad = 0x7F800000 if dt == "f32" else 0x7C00
    run_end = _RUN_TILES * _TILE_WORDS // wpe
    for pos in (0, run_end // 2 + 12345, run_end - 1, run_end, n - 1):
        flag, same, expect, _ = _gate_case(dt, [pos], bad, numels=(n,), R=1, r=0)
        assert expect and flag == 1 and same, pos
    flag, same, expect, _ = _gate_case(dt, [], bad, numels=(n,), R=1, r=0)
    assert not expect and flag == 0


def _gate_case(dt, bad_pos, bad_bits, numels=(3000, 4099, 65, 70001, 2048), R=2, r=1):
    """One step whose flat shard carries bad_bits at shard positions bad_pos;
    returns (flag, state unchanged?)."""
    import torch
    numels = list(numels)
    op = oracle.plan(numels, R, r, 8)
    plan = z.zero_partition_plan(numels, R, r, 8)
    rng = np.random.default_rng(11)
    host = [synth.grad_bits(rng.normal(0, 1e-2, n).astype(np.float32), dt) for n in numels]
    for pos in bad_pos:
        s = int(np.searchsorted(op.seg_shard_off, pos, side="right") - 1)
        host[int(op.seg_tensor[s])][int(op.seg_tensor_off[s] + pos - op.seg_shard_off[s])] = \
            bad_bits
    grads = [_to_dev_half(h, dt) for h in host]
    flat = torch.empty(op.S, dtype=torch_dtype(dt), device=DEV)
    master = torch.randn(op.S, device=DEV) * 0.02
    m = torch.randn(op.S, device=DEV) * 1e-4
    v = torch.rand(op.S, device=DEV) * 1e-6
    param = torch.zeros(op.P, dtype=torch_dtype("bf16" if dt == "f32" else dt), device=DEV)
    keep = [x.clone() for x in (master, m, v, param)]
    z.zero_flatten_grads(plan, -1, grads, flat)
    flag = z.zero_adam_step(plan, z.AdamHParams(), 3, 1024.0, flat, master, m, v, param, 0)
    same = all(torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else
                           a.view(torch.int16), b.view(torch.int32) if b.dtype == torch.float32
                           else b.view(torch.int16)) for a, b in zip((master, m, v, param), keep))
    expect = oracle.nonfinite(oracle.flatten(op, host), dt)
    return flag, same, expect, op


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_overflow_positions_and_skip_leaves_state_bit_identical(dt):
    inf = {"f16": [0x7C00, 0xFC00, 0x7E00, 0x7C01], "bf16": [0x7F80, 0xFF80, 0x7FC0, 0x7F81],
           "f32": [0x7F800000, 0xFF800000, 0x7FC00000, 0x7F800001]}[dt]
    op = oracle.plan([3000, 4099, 65, 70001, 2048], 2, 1, 8)
    edges = [0, op.real - 1] + op.seg_shard_off.tolist()[1:] + \
        [s - 1 for s in op.seg_shard_off.tolist()[1:]] + [2047, 2048, 4095, 12345]
    for bits in inf:
        for pos in edges:
            flag, same, expect, _ = _gate_case(dt, [pos], bits)
            assert expect == 1
            assert flag == 1 and same, (hex(bits), pos)
    # largest finite values, subnormals and -0 never trip
    fin = {"f16": [0x7BFF, 0xFBFF, 0x0001, 0x8000], "bf16": [0x7F7F, 0xFF7F, 0x0001, 0x8000],
           "f32": [0x7F7FFFFF, 0xFF7FFFFF, 0x00000001, 0x80000000]}[dt]
    for bits in fin:
        flag, same, expect, _ = _gate_case(dt, [0, 17, op.real - 1], bits)
        assert expect == 0 and flag == 0 and not same


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_write_param_cast_sweep(dt):
    import torch
    lows = []
    for b in range(8):
        for lo in (0x0000, 0x0001, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x0ABC, 0x1555):
            lows.append((b << 13) | lo)
    lows = np.array(sorted(set(lows)), dtype=np.uint32)
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    pats = (hi[:, None] | lows[None, :]).ravel()
    x = pats.view(np.float32)
    n = x.size
    plan = z.zero_partition_plan([n], 1, 0, 1)
    master = torch.from_numpy(x.copy()).to(DEV)
    param = torch.zeros(n, dtype=torch_dtype(dt), device=DEV)
    z.zero_write_param_shard(plan, master, param, 0)
    got = _bits(param)
    exp = oracle.float_to_half(x, dt)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], exp[~nan])
    exp_mask = 0x7C00 if dt == "f16" else 0x7F80
    frac = 0x03FF if dt == "f16" else 0x007F
    assert np.all((got[nan] & exp_mask) == exp_mask) and np.all((got[nan] & frac) != 0)
    # rank 1 of 2, written through a buffer whose element 0 sits 6 bytes past
    # a 16-byte boundary; elements outside the shard stay untouched
    plan = z.zero_partition_plan([7, n - 7], 2, 1, 1)
    big = torch.zeros(n + 3, dtype=torch_dtype(dt), device=DEV)
    dst = big[3:]
    z.zero_write_param_shard(plan, master[plan.begin:], dst, 0)
    b, e = plan.begin, plan.begin + plan.real
    got = _bits(dst)
    nn = np.isnan(x[b:e])
    assert np.array_equal(got[b:e][~nn], oracle.float_to_half(x[b:e], dt)[~nn])
    assert not got[:b].any() and not _bits(big)[:3].any()


def test_resume_is_bit_identical():
    """k steps, save (master, m, v, t, scale, good_steps), restore into fresh
    buffers and plan, continue: identical to the uninterrupted run."""
    case = Case(numels=[3000, 1, 100003, 65, 4099], world_size=2, rank=0, grad_dtype="f16",
                param_dtype="f16", steps=8, dynamic=True, init_scale=512.0, window=3,
                inject={3: 77})
    orc = OracleRun(case)
    straight = DeviceRun(case)
    grads_per_it = {}
    for it in range(1, 9):
        _, grads, _ = orc.step(it)
        grads_per_it[it] = grads
        straight.step(it, grads)
    a = DeviceRun(case)
    for it in range(1, 5):
        a.step(it, grads_per_it[it])
    saved = dict(master=a.master.clone(), m=a.m.clone(), v=a.v.clone(),
                 param=a.param_full.clone(), t=a.t, scale=a.scaler.scale,
                 good=a.scaler.good_steps)
    del a
    b = DeviceRun(case)
    b.master.copy_(saved["master"])
    b.m.copy_(saved["m"])
    b.v.copy_(saved["v"])
    b.param_full.copy_(saved["param"])
    b.t = saved["t"]
    b.scaler.c.scale = saved["scale"]
    b.scaler.c.good_steps = saved["good"]
    for it in range(5, 9):
        b.step(it, grads_per_it[it])
    for x, y in zip(straight.state_host()[:4], b.state_host()[:4]):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))
    assert (b.t, b.scaler.scale) == (straight.t, straight.scaler.scale)


@pytest.mark.parametrize("R", [2, 4])
def test_rank_simulation_equals_unpartitioned_step(R):
    """Every rank of R updates its shard into one full parameter buffer; the
    result equals the single-rank (unpartitioned) oracle step over the whole
    model."""
    import torch
    numels = [3000, 1, 7, 100003, 65, 2048, 511, 30000, 13]
    P = sum(numels)
    rng = np.random.default_rng(2)
    steps = 3
    grads = [[synth.half_bits(rng.normal(0, 1e-2, n).astype(np.float32), "bf16") for n in numels]
             for _ in range(steps)]
    full_master0 = rng.normal(0, 0.02, P).astype(np.float32)
    # unpartitioned oracle
    op1 = oracle.plan(numels, 1, 0, 1)
    om = np.zeros(op1.S, np.float32)
    om[:P] = full_master0
    omo, ov = np.zeros_like(om), np.zeros_like(om)
    for t in range(1, steps + 1):
        oracle.adam_step(t, 1.0, oracle.flatten(op1, grads[t - 1]), "bf16", om, omo, ov)
    oparam = np.zeros(P, np.uint16)
    oracle.write_param(om, P, 0, 0, oparam, "bf16")
    # R ranks on the GPU into one buffer
    param = torch.zeros(P, dtype=torch.bfloat16, device=DEV)
    masters = []
    for r in range(R):
        plan = z.zero_partition_plan(numels, R, r, 64)
        m0 = np.zeros(plan.S, np.float32)
        m0[:plan.real] = full_master0[plan.begin:plan.begin + plan.real]
        master = torch.from_numpy(m0).to(DEV)
        mo = torch.zeros(plan.S, device=DEV)
        va = torch.zeros(plan.S, device=DEV)
        flat = torch.empty(plan.S, dtype=torch.bfloat16, device=DEV)
        for t in range(1, steps + 1):
            z.zero_flatten_grads(plan, -1, [_to_dev_half(g, "bf16") for g in grads[t - 1]], flat)
            assert z.zero_adam_step(plan, z.AdamHParams(), t, 1.0, flat, master, mo, va, param,
                                    0) == 0
        masters.append(master.cpu().numpy()[:plan.real])
    assert np.array_equal(_bits(param), oparam)
    assert np.array_equal(np.concatenate(masters).view(np.uint32), om[:P].view(np.uint32))


def test_timing_entry_points():
    import torch
    case = Case(numels=[1 << 20, 12345], world_size=2, rank=0, grad_dtype="bf16",
                param_dtype="bf16", steps=1)
    g = DeviceRun(case)
    with pytest.raises(z.ZeroError):
        g.plan.kernel_ms(2)
    g.plan.set_timing(True)
    orc = OracleRun(case)
    _, grads, _ = orc.step(1)
    g.step(1, grads)
    assert g.plan.kernel_ms(0) > 0 and g.plan.kernel_ms(2) > 0
    with pytest.raises(z.ZeroError):
        g.plan.kernel_ms(3)
    z.zero_write_param_shard(g.plan, g.master, g.param_full, 0)
    torch.cuda.synchronize()
    assert g.plan.kernel_ms(3) > 0


def test_wrong_device_and_bad_buffers_raise():
    import torch
    plan = z.zero_partition_plan([1000], 1, 0, 8)
    flat = torch.empty(1000, dtype=torch.bfloat16, device=DEV)
    master = torch.empty(1000, device=DEV)
    with pytest.raises(ValueError):          # too small for the shard
        z.zero_adam_step(plan, z.AdamHParams(), 1, 1.0, flat[:10], master, master, master)
    with pytest.raises(TypeError):           # fp32 gradient buffer
        z.zero_flatten_grads(plan, -1, [master], flat)
    with pytest.raises(z.ZeroError):         # window misses the shard
        z.zero_write_param_shard(plan, master, flat[:10], 0)


@pytest.mark.parametrize("pdt", ["f16", "bf16"])
def test_write_param_ragged_sizes_and_windows(pdt):
    """The standalone cast on shards whose real length leaves a partial
    2048-element block or a partial 4-element vector (and tiny ones),
    written through parameter windows at several bases; everything outside
    the shard's range stays untouched.  A 16-byte aligned master with an
    8-byte aligned destination takes the vector kernel, any other alignment
    (a window 2 or 6 bytes off, a master 4 bytes off) the element kernel."""
    import torch
    rng = np.random.default_rng(23)
    for numels, R, r, A in [([1], 1, 0, 1), ([5], 1, 0, 1), ([7], 1, 0, 1), ([2049], 1, 0, 1),
                            ([4095, 3], 2, 1, 1), ([2048 * 7 + 1, 2047], 3, 2, 8),
                            ([100003, 65, 2048], 2, 0, 64), ([100003, 65, 2048], 2, 1, 64),
                            ([4096 * 3 + 6], 1, 0, 1), ([2048 * 9 + 3, 1], 2, 1, 2)]:
        plan = z.zero_partition_plan(numels, R, r, A)
        P, S, real, begin = sum(numels), plan.S, plan.real, plan.begin
        master = rng.normal(0, 0.5, S).astype(np.float32)
        for moff in (0, 1):
            mbuf = torch.zeros(S + 4, device=DEV)
            mbuf[moff:moff + S] = torch.from_numpy(master).to(DEV)
            for base in (0, begin, max(begin - 3, 0)):
                numel = P - base
                buf = torch.full((numel + 5,), 7.0, dtype=torch_dtype(pdt), device=DEV)
                win = buf[:numel]
                z.zero_write_param_shard(plan, mbuf[moff:moff + S], win, base)
                got = _bits(buf)
                want = _bits(torch.full((numel + 5,), 7.0, dtype=torch_dtype(pdt)))
                oracle.write_param(master, real, begin, base, want, pdt)
                assert np.array_equal(got, want), (numels, R, r, base, moff)


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_partial_flatten_makes_the_step_scan(dt):
    """Only some buckets are flattened; the rest of the flat shard is filled
    another way (as a reduce-scatter would).  The step must test the whole
    shard: an inf planted in the unflattened part skips it, a finite one
    applies it exactly as the oracle does."""
    import torch
    numels = [3000, 1, 7, 100003, 65, 2048, 511, 30000, 13, 4099]
    op = oracle.plan(numels, 2, 0, 8, bucket_elems=20000)
    plan = z.zero_partition_plan(numels, 2, 0, 8, 20000)
    assert plan.n_buckets >= 3
    rng = np.random.default_rng(5)
    host = [synth.grad_bits(rng.normal(0, 1e-2, n).astype(np.float32), dt) for n in numels]
    expect_flat = oracle.flatten(op, host)
    tb = plan.tensor_buckets()
    segs = plan.segments()
    skip_b = tb[int(op.seg_tensor[0])]            # the bucket holding the first segment
    lo = min(s.shard_off for s in segs if s.bucket == skip_b)
    hi = max(s.shard_off + s.numel for s in segs if s.bucket == skip_b)
    for plant in (False, True):
        grads = [_to_dev_half(h, dt) for h in host]
        flat = torch.empty(op.S, dtype=torch_dtype(dt), device=DEV)
        for b in range(plan.n_buckets):
            if b != skip_b:
                z.zero_flatten_grads(plan, b, [g if tb[i] == b else None
                                               for i, g in enumerate(grads)], flat)
        part = expect_flat[lo:hi].copy()
        if plant:
            part[(hi - lo) // 2] = {"f16": 0x7C00, "bf16": 0x7F80, "f32": 0x7F800000}[dt]
        flat[lo:hi].copy_(_to_dev_half(part, dt))
        m0 = rng.normal(0, 0.02, op.S).astype(np.float32)
        master = torch.from_numpy(m0.copy()).to(DEV)
        mo = torch.zeros(op.S, device=DEV)
        va = torch.zeros(op.S, device=DEV)
        flag = z.zero_adam_step(plan, z.AdamHParams(), 1, 1.0, flat, master, mo, va)
        om, omo, ov = m0.copy(), np.zeros(op.S, np.float32), np.zeros(op.S, np.float32)
        oflat = expect_flat.copy()
        oflat[lo:hi] = part
        oflag = oracle.adam_step(1, 1.0, oflat, dt, om, omo, ov)
        assert flag == oflag == (1 if plant else 0)
        assert np.array_equal(master.cpu().numpy().view(np.uint32), om.view(np.uint32))
        assert np.array_equal(va.cpu().numpy().view(np.uint32), ov.view(np.uint32))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_flatten_independent_of_bucket_size_and_order(dt):
    """The flat shard does not depend on the bucket size (from one element --
    every tensor its own bucket -- to one bucket for the whole model) or on
    the order buckets are flattened in."""
    import torch
    numels = [5000, 4099, 2048, 3, 70000, 1, 2047, 9000, 4097, 12345, 600, 8191, 0, 77]
    rng = np.random.default_rng(21)
    host = [synth.grad_bits(rng.normal(0, 1e-2, n).astype(np.float32), dt) for n in numels]
    grads = [_to_dev_half(h, dt) for h in host]
    for r in range(3):
        expect = None
        for B in (1, 1000, 1 << 20, 1 << 25, sum(numels)):
            op = oracle.plan(numels, 3, r, 8, bucket_elems=B)
            plan = z.zero_partition_plan(numels, 3, r, 8, B)
            want = oracle.flatten(op, host)
            if expect is None:
                expect = want
            assert np.array_equal(want, expect), (r, B)   # the oracle's own invariance
            tb = plan.tensor_buckets()
            for order in (range(plan.n_buckets), reversed(range(plan.n_buckets))):
                flat = torch.full((op.S,), float("nan"), dtype=torch_dtype(dt), device=DEV)
                for b in order:
                    z.zero_flatten_grads(plan, b, [g if tb[i] == b else None
                                                   for i, g in enumerate(grads)], flat)
                assert np.array_equal(_bits(flat), expect), (dt, r, B)


def test_two_runs_are_bit_identical():
    """The same case run twice from scratch gives the same bits (no atomics or
    reductions whose order could change a value)."""
    case = Case(numels=[3000, 1, 7, 100003, 65, 2048, 511, 300000, 13, 0, 4099, 77777],
                world_size=3, rank=1, grad_dtype="f16", param_dtype="f16", steps=4,
                grad_sigma=1e-2, dynamic=True, init_scale=1024.0, window=2, inject={3: 4321},
                flatten_mode="buckets_shuffled", bucket_elems=50000)
    states = []
    for _ in range(2):
        orc, gpu = OracleRun(case), DeviceRun(case)
        for it in range(1, case.steps + 1):
            gpu.step(it, orc.step(it)[1])
        states.append(gpu.state_host())
    for a, b in zip(*states):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_write_param_cast_all_2_32_patterns(dt):
    """The GPU's fp32 -> half cast (write_param; the fused update uses the same
    conversion) over all 2^32 fp32 bit patterns, in 2^28-pattern chunks,
    against the oracle computed beside it on the host's cores: every non-NaN
    input bit for bit, NaN to a NaN."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    import torch
    chunk = 1 << 28
    plan = z.zero_partition_plan([chunk], 1, 0, 1)
    master = torch.empty(chunk, dtype=torch.float32, device=DEV)
    param = torch.empty(chunk, dtype=torch_dtype(dt), device=DEV)
    emask, frac = (0x7C00, 0x03FF) if dt == "f16" else (0x7F80, 0x007F)
    workers = max(1, min(16, os.cpu_count() or 1))
    sub = chunk // workers
    with ThreadPoolExecutor(workers) as ex:
        for c in range((1 << 32) // chunk):
            u = np.arange(c * chunk, (c + 1) * chunk, dtype=np.uint32)
            x = u.view(np.float32)
            master.copy_(torch.from_numpy(x))
            z.zero_write_param_shard(plan, master, param, 0)
            got = _bits(param)
            exp = np.concatenate(list(ex.map(
                lambda i: oracle.float_to_half(x[i * sub:(i + 1) * sub], dt), range(workers))))
            nan = np.isnan(x)
            bad = np.flatnonzero((got != exp) & ~nan)
            assert bad.size == 0, (dt, [hex(int(u[i])) for i in bad[:4]])
            gn = got[nan]
            assert np.all((gn & emask) == emask) and np.all((gn & frac) != 0), (dt, c)
    log(f"[cast] {dt}: all 2^32 fp32 patterns match the oracle")
