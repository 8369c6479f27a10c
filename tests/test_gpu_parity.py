"""GPU parity: the HIP kernels against the CPU oracle, element by element,
bit-exact, through the C ABI (via the Python binding).

Covers the five named workloads at their full sizes (the oracle runs over
row chunks in threads), an edge suite over row lengths that span several
tiles with ragged tails and the long-row path, the hand-worked golden
blocks, ragged group ranges, the standalone dequantizer, determinism and
argument errors.  Every output is written inside 256 guard bytes on both
sides (gpuutil.Guards), which must be left untouched."""
import numpy as np
import pytest
import torch

import fp4_block_quantization_amd as fq
import oracle
import workloads
from goldens import load
from gpuutil import (Guards, assert_same, bits_of, host, oracle_mx, oracle_mx_dense,
                     oracle_nvfp4, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fq.lib()


def f32_to_bf16_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def check_nvfp4(x_bits, fos, dequant=True, label=""):
    x = to_dev(x_bits)
    gu = Guards()
    codes, scales, ts, dq = fq.nvfp4_quantize(x, four_over_six=fos, dequant=dequant,
                                              out=gu.nvfp4(*x_bits.shape, dequant))
    gu.check(label)
    want = oracle_nvfp4(x_bits, fos, dequant=dequant)
    assert_same(host(codes), want[0], label + " codes")
    assert_same(host(scales), want[1], label + " block_scales")
    assert_same(host(ts)[:, None], want[2][:, None], label + " token_scales")
    if dequant:
        assert_same(bits_of(dq), want[3], label + " dequant")
    return codes, scales, ts, dq


def check_mx(x_bits, label="", dense_and_reconstruct=True):
    x = to_dev(x_bits)
    R, H = x_bits.shape
    gu = Guards()
    got = fq.mxfp4_resq_quantize(x, out=gu.mx(R, H))
    gu.check(label)
    want = oracle_mx(x_bits)
    for g, w, n in zip(got, want, ("codes", "scales", "res_codes", "res_meta", "res_scales")):
        assert_same(host(g), w, label + " " + n)
    if not dense_and_reconstruct:
        return
    # Rollout-ResQ-Dense
    gd = fq.mxfp4_resq_dense_quantize(x, out=gu.mx_dense(R, H))
    gu.check(label + " dense")
    wd = oracle_mx_dense(x_bits)
    for g, w, n in zip(gd, wd, ("codes", "scales", "res_codes", "res_scales")):
        assert_same(host(g), w, label + " dense " + n)
    # reconstruction, each side from its own quantize outputs
    c, s, rc, rm, rs = got
    for mode, args, wargs in ((0, (None, None, None), (None, None, None)),
                              (1, (rc, rm, rs), (want[2], want[3], want[4])),
                              (2, (gd[2], None, gd[3]), (wd[2], None, wd[3]))):
        xh = fq.mxfp4_resq_reconstruct(c, s, *args, residual=mode,
                                       out=gu.empty((R, H), torch.float32))
        gu.check(label + " reconstruct")
        wh = oracle.mxfp4_resq_reconstruct(want[0], want[1], *wargs, residual=mode)
        assert_same(host(xh), wh, label + " reconstruct residual=%d" % mode)


# ------------------------------------------------------------ edge suite --

def edge_rows(H, seed):
    """Rows that exercise the corner cases of the method."""
    rng = np.random.default_rng(seed)
    rows = []
    z = np.zeros(H, np.float32)
    rows.append(z)                                         # zero row
    rows.append(np.where(np.arange(H) % 2, -0.0, 0.0).astype(np.float32))  # +-0
    one = z.copy(); one[rng.integers(H)] = -3.25; rows.append(one)         # single nonzero
    rows.append(np.full(H, 1.7, np.float32))               # equal values
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, .25, .75, 1.25, 1.75, 2.5, 3.5, 5], np.float32)
    for p in (-3, 0, 7):                                   # grid points and midpoints
        r = rng.choice(grid, H) * rng.choice([-1, 1], H) * np.float32(2.0 ** p)
        r[0] = 6 * 2.0 ** p
        rows.append(r.astype(np.float32))
    rows.append(rng.standard_normal(H).astype(np.float32))
    rows.append(rng.standard_t(3, H).astype(np.float32) * 40)
    r = rng.standard_normal(H).astype(np.float32); r[rng.integers(H, size=max(1, H // 100))] *= 50
    rows.append(r)
    for sc in (2.0 ** -126, 2.0 ** -133, 2.0 ** 64, 2.0 ** 100, 2.0 ** 120):
        rows.append((rng.standard_normal(H) * sc).astype(np.float32))
    bits = [f32_to_bf16_bits(r) for r in rows]
    sub = rng.integers(1, 0x80, H).astype(np.uint16) | (rng.integers(0, 2, H).astype(np.uint16) << 15)
    bits.append(sub)                                       # BF16 subnormals only
    big = np.full(H, 0x7F7F, np.uint16); big[1::3] = 0x0001  # largest finite + tiny
    bits.append(big)
    mix = rng.integers(0, 0x7F80, H).astype(np.uint16)     # random finite patterns
    mix |= (rng.integers(0, 2, H).astype(np.uint16) << 15)
    bits.append(mix)
    return np.stack(bits, 0)


# row lengths: one block; a few; around one and several waves (2048 elements
# a wave); 10, 14 and 16 waves a row (the widest split rows, with 1024-thread
# workgroups and up to 80 KiB of LDS); past 16 waves (the long-row kernel)
HIDDEN = [16, 32, 48, 1008, 1024, 1040, 2048, 2064, 7168, 8192, 8208, 16400, 20480, 26640,
          32768, 32784]


@pytest.mark.parametrize("fos", [1, 0, 2])
@pytest.mark.parametrize("H", HIDDEN)
def test_nvfp4_edge_suite(H, fos):
    check_nvfp4(edge_rows(H, seed=H), fos, label="edge H=%d" % H)


@pytest.mark.parametrize("fos", [1, 0, 2])
@pytest.mark.parametrize("H,reps", [(2048, 1), (2048, 300), (2064, 1), (16, 1)])
def test_nvfp4_edge_suite_no_dequant(H, reps, fos):
    # without the dequant, rows of exactly 2048 elements take the persistent
    # streaming kernel (a wavefront walks many rows; with 300 copies of the
    # edge rows every wavefront of its grid gets several, tiny rows among
    # them); other lengths take the split kernel
    x = np.ascontiguousarray(np.tile(edge_rows(H, seed=H + 5), (reps, 1)))
    if reps > 1:
        x[::3] ^= 0x8000  # the copies differ
    check_nvfp4(x, fos, dequant=False, label="edge no-dequant H=%d x%d" % (H, reps))


def every_bf16_rows(H, seed):
    """Every finite BF16 pattern once (both signs, subnormals and zeros
    included), ordered by magnitude and cut into rows of H (the last padded
    with zeros), so that each row spans a few binades; the elements of every
    other row are shuffled, so its blocks mix those magnitudes."""
    pats = np.arange(1 << 16, dtype=np.uint32)
    pats = pats[(pats & 0x7F80) != 0x7F80]  # no infinities or NaNs (outside the domain)
    pats = pats[np.lexsort((pats >> 15, pats & 0x7FFF))].astype(np.uint16)
    rows = -(-pats.size // H)
    x = np.zeros(rows * H, np.uint16)
    x[:pats.size] = pats
    x = x.reshape(rows, H)
    rng = np.random.default_rng(seed)
    for r in range(1, rows, 2):
        x[r] = x[r, rng.permutation(H)]
    return x


# the split kernel's one-wave rows without dequant (the FP32 block maximum)
# and its four-wave rows with dequant (the packed one), in every mode
@pytest.mark.parametrize("fos", [1, 0, 2])
@pytest.mark.parametrize("H,dequant", [(2048, False), (2048, True), (7168, True), (7168, False)])
def test_nvfp4_every_bf16_value(H, dequant, fos):
    check_nvfp4(every_bf16_rows(H, seed=H), fos, dequant=dequant,
                label="every BF16 value H=%d dq=%d" % (H, dequant))


@pytest.mark.parametrize("H", [2048, 7168])
def test_mx_every_bf16_value(H):
    check_mx(every_bf16_rows(H, seed=H + 3), label="mx every BF16 value H=%d" % H)


@pytest.mark.parametrize("H", [32, 64, 96, 2048, 7200])
def test_mx_edge_suite(H):
    check_mx(edge_rows(H, seed=H + 1), label="mx edge H=%d" % H)


def test_golden_blocks_on_gpu():
    for name, c in load("nvfp4_worked_blocks.txt").items():
        x = to_dev(c["x"][None, :])
        codes, scales, ts, dq = fq.nvfp4_quantize(x, four_over_six=bool(c["four_over_six"]))
        torch.cuda.synchronize()
        assert host(ts).view(np.uint32)[0] == c["token_scale_bits"], name
        np.testing.assert_array_equal(host(scales)[0], c["scales"], err_msg=name)
        np.testing.assert_array_equal(host(codes)[0], c["codes"], err_msg=name)
        np.testing.assert_array_equal(bits_of(dq)[0], c["dequant"], err_msg=name)
    c = load("mxfp4_resq_worked_block.txt")["MX_first_group"]
    out = fq.mxfp4_resq_quantize(to_dev(c["x"][None, :]))
    for t, k in zip(out, ("codes", "scales", "res_codes", "res_meta", "res_scales")):
        np.testing.assert_array_equal(host(t)[0], c[k], err_msg=k)


# ------------------------------------------------------ named workloads --

@pytest.mark.parametrize("fos", [1, 0, 2])
def test_tiny_ref(fos):
    check_nvfp4(workloads.rows("tiny_ref"), fos, label="tiny_ref")


def test_moe_act_full_size_fp16_decision():
    # the FP16 fast path's 4/6 choice (four_over_six = 2) at full size
    check_nvfp4(workloads.rows("moe_act"), 2, label="moe_act fp16-decision")


def test_expert_weights_fp16_decision_rows():
    check_nvfp4(workloads.rows("expert_weights", 0, 4096), 2, label="expert_weights fp16")


def test_moe_act_full_size():
    check_nvfp4(workloads.rows("moe_act"), True, label="moe_act")


def test_expert_weights_full_size():
    check_nvfp4(workloads.rows("expert_weights"), True, label="expert_weights")


def test_ragged_routed_full_size():
    x_bits = workloads.rows("ragged_routed")
    offs = workloads.group_offsets()
    x = to_dev(x_bits)
    gu = Guards()
    codes, scales, ts, _ = fq.nvfp4_quantize(x, True, offsets=torch.from_numpy(offs).cuda(),
                                             dequant=False, out=gu.nvfp4(*x_bits.shape, False))
    gu.check("ragged")
    want = oracle_nvfp4(x_bits, True, dequant=False)
    assert_same(host(codes), want[0], "ragged codes")
    assert_same(host(scales), want[1], "ragged scales")
    assert_same(host(ts)[:, None], want[2][:, None], "ragged token_scales")


def sentinel_outputs(gu, R, H):
    """Guarded nvfp4 outputs filled with sentinels (rows outside a ragged
    range must keep them)."""
    out = gu.nvfp4(R, H)
    for t, f in zip(out, (0xAB, 0xCD, -7.0, 1.5)):
        t.fill_(f)
    return out


@pytest.mark.parametrize("H,rows,cut", [(2048, 8192, None), (32768, 50, (3, 17, 17, 40))])
def test_ragged_subrange_leaves_other_rows(H, rows, cut):
    # routed rows of 2048 (groups 2..4 of the workload), and a range inside
    # rows of 32768 (16 waves a row)
    if cut is None:
        x_bits = workloads.rows("ragged_routed", 0, rows)
        sub = workloads.group_offsets()[2:6].copy()
    else:
        x_bits = np.ascontiguousarray(np.tile(workloads.rows("ragged_routed", 0, rows),
                                              (1, H // 2048)))
        x_bits[:, ::7] ^= 0x8000  # rows differ across their 16 copies of 2048
        sub = np.array(cut, np.int64)
    x = to_dev(x_bits)
    R, H = x_bits.shape
    gu = Guards()
    out = sentinel_outputs(gu, R, H)
    fq.nvfp4_quantize(x, True, offsets=torch.from_numpy(sub).cuda(), out=out)
    gu.check("subrange H=%d" % H)
    want = oracle_nvfp4(x_bits, True)
    lo, hi = int(sub[0]), int(sub[-1])
    assert 0 < lo < hi < R
    got = [host(out[0]), host(out[1]), host(out[2]), bits_of(out[3])]
    fills = (0xAB, 0xCD, np.float32(-7.0), 0x3FC0)
    for g, w, f, n in zip(got, want, fills, ("codes", "scales", "ts", "dq")):
        w = w if w.ndim > 1 else w[:, None]
        g = g if g.ndim > 1 else g[:, None]
        assert_same(g[lo:hi], w[lo:hi], "subrange " + n)
        assert (g[:lo] == f).all() and (g[hi:] == f).all(), n


@pytest.mark.parametrize("H,rows,offs", [
    (2048, 100, (-5, 50, 200)),                 # below 0 and past the end: all rows
    (7168, 40, (30, 10)),                       # decreasing: no row
    (7168, 40, (12, 25, 1 << 40)),              # far past the end: rows 12..39
    (32784, 6, (-(1 << 40), 3, 4)),             # the long-row kernel, from far below 0
])
def test_ragged_offsets_outside_the_tensor_are_clamped(H, rows, offs):
    # offsets are not checked on the host; the kernels clamp the range to
    # [0, rows): the rows inside it are quantized, the others keep their
    # contents, and nothing is written outside the outputs
    if H % 2048 == 0:
        x_bits = np.ascontiguousarray(
            np.tile(workloads.rows("ragged_routed", 0, rows), (1, H // 2048)))
    else:
        e = edge_rows(H, seed=rows)
        x_bits = np.ascontiguousarray(np.tile(e, (-(-rows // len(e)), 1))[:rows])
    R = x_bits.shape[0]
    assert R == rows
    x = to_dev(x_bits)
    gu = Guards()
    out = sentinel_outputs(gu, R, H)
    fq.nvfp4_quantize(x, True, offsets=torch.tensor(offs, dtype=torch.int64, device="cuda"),
                      out=out)
    gu.check("clamped offsets %s" % (offs,))
    lo, hi = max(offs[0], 0), min(offs[-1], R)
    got = [host(out[0]), host(out[1]), host(out[2])[:, None], bits_of(out[3])]
    fills = (0xAB, 0xCD, np.float32(-7.0), 0x3FC0)
    if hi > lo:
        want = oracle_nvfp4(x_bits[lo:hi], True)
        for g, w, n in zip(got, want, ("codes", "scales", "ts", "dq")):
            w = w if w.ndim > 1 else w[:, None]
            assert_same(g[lo:hi], w, "clamped %s %s" % (offs, n))
    for g, f, n in zip(got, fills, ("codes", "scales", "ts", "dq")):
        assert (g[:lo] == f).all() and (g[max(hi, lo):] == f).all(), n


def test_resq_act_full_size():
    check_mx(workloads.rows("resq_act"), label="resq_act")


@pytest.mark.parametrize("offsets", [(0, 1, 0, 0, 3), (0, 0, 8, 4, 0), (0, 5, 8, 4, 9)])
def test_mx_outputs_not_16_byte_aligned(offsets):
    """Outputs that are not all 16-byte aligned are written lane by lane
    instead of as staged 16-byte pieces; the bytes are the same."""
    rng = np.random.default_rng(sum(offsets))
    x_bits = np.concatenate([edge_rows(2048, seed=7),
                             f32_to_bf16_bits(rng.standard_normal((48, 2048)).astype(np.float32))])
    R, H = x_bits.shape
    shapes = ((R, H // 2), (R, H // 32), (R, H // 4), (R, H // 8), (R, H // 32))
    gu = Guards()
    out = tuple(gu.empty(sh, torch.uint8, o) for sh, o in zip(shapes, offsets))
    got = fq.mxfp4_resq_quantize(to_dev(x_bits), out=out)
    gu.check("offsets %s" % (offsets,))
    want = oracle_mx(x_bits)
    for g, w, n in zip(got, want, ("codes", "scales", "res_codes", "res_meta", "res_scales")):
        assert_same(host(g), w, "offsets %s %s" % (offsets, n))
    dshapes = ((R, H // 2), (R, H // 32), (R, H // 2), (R, H // 32))
    dg = Guards()
    dout = tuple(dg.empty(sh, torch.uint8, o)
                 for sh, o in zip(dshapes, (0, offsets[1], 0, offsets[4])))
    gd = fq.mxfp4_resq_dense_quantize(to_dev(x_bits), out=dout)
    dg.check("dense offsets %s" % (offsets,))
    wd = oracle_mx_dense(x_bits)
    for g, w, n in zip(gd, wd, ("codes", "scales", "res_codes", "res_scales")):
        assert_same(host(g), w, "dense offsets %s %s" % (offsets, n))


# -------------------------------------------------------------- dequant --

def test_standalone_dequant_matches_fused():
    for name in ("tiny_ref", "moe_act"):
        codes, scales, ts, dq = fq.nvfp4_quantize(workloads.tensor(name, "cuda"), True)
        gu = Guards()
        out = fq.nvfp4_dequantize(codes, scales, ts, out=gu.empty(dq.shape, torch.bfloat16))
        gu.check(name)
        assert torch.equal(out.view(torch.int16), dq.view(torch.int16)), name


def test_standalone_dequant_random_bytes():
    rng = np.random.default_rng(99)
    R, H = 512, 1040
    codes = rng.integers(0, 256, (R, H // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (R, H // 16), dtype=np.uint8)
    scales |= (rng.integers(0, 2, scales.shape, dtype=np.uint8) << 7)  # signed scale bytes
    ts = (rng.standard_normal(R) * 2.0 ** rng.integers(-140, 60, R)).astype(np.float32)
    gu = Guards()
    out = fq.nvfp4_dequantize(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                              torch.from_numpy(ts).cuda(), out=gu.empty((R, H), torch.bfloat16))
    gu.check("dequant")
    assert_same(bits_of(out), oracle.nvfp4_dequantize(codes, scales, ts), "dequant")


# ------------------------------------------- determinism and invariance --

def test_determinism_streams_and_batch_invariance():
    x_bits = workloads.rows("moe_act", 0, 512)
    x = to_dev(x_bits)
    ref = fq.nvfp4_quantize(x, True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        again = fq.nvfp4_quantize(x, True)
    torch.cuda.synchronize()
    def rowbytes(t):
        return t.reshape(t.shape[0], -1).view(torch.uint8)

    for a, b in zip(ref, again):
        assert torch.equal(rowbytes(a), rowbytes(b))
    perm = torch.randperm(512, generator=torch.Generator().manual_seed(1)).cuda()
    pr = fq.nvfp4_quantize(x[perm].contiguous(), True)
    one = fq.nvfp4_quantize(x[37:38].contiguous(), True)
    torch.cuda.synchronize()
    for a, b, c in zip(ref, pr, one):
        a8, b8, c8 = rowbytes(a), rowbytes(b), rowbytes(c)
        assert torch.equal(a8[perm], b8)
        assert torch.equal(a8[37:38], c8)


def test_empty_and_rejected_calls():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    codes, scales, ts, dq = fq.nvfp4_quantize(x)
    assert codes.shape == (0, 32) and dq.shape == (0, 64)
    fq.mxfp4_resq_quantize(x)
    with pytest.raises(fq.Fp4qError):
        fq.nvfp4_quantize(torch.zeros((4, 40), dtype=torch.bfloat16, device="cuda"))
    flat = torch.zeros(16 * 5, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fq.Fp4qError):  # 2-byte offset: misaligned
        fq.nvfp4_quantize(flat[1:1 + 64].view(4, 16))


def test_binding_rejects_wrong_sized_buffers():
    # caller-supplied buffers one element short, or of the wrong type, are
    # refused before any launch (a short buffer would be written past its end)
    R, H = 4, 64
    x = torch.zeros((R, H), dtype=torch.bfloat16, device="cuda")
    u8 = lambda n: torch.zeros(n, dtype=torch.uint8, device="cuda")
    f32 = lambda n: torch.zeros(n, dtype=torch.float32, device="cuda")
    bf = lambda n: torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    good = (u8(R * H // 2), u8(R * H // 16), f32(R), bf(R * H))
    good_g = good[:2] + (f32(1),) + good[3:]  # one tensor scale
    for k in range(4):
        bad = tuple(t[:-1] if j == k else t for j, t in enumerate(good))
        with pytest.raises(fq.Fp4qError):
            fq.nvfp4_quantize(x, out=bad)
        bad_g = tuple(t[:-1] if j == k else t for j, t in enumerate(good_g))
        with pytest.raises(fq.Fp4qError):
            fq.nvfp4_quantize_global(x, out=bad_g)
    with pytest.raises(fq.Fp4qError):
        fq.nvfp4_quantize(x, out=(good[0], good[1], good[2], u8(2 * R * H)))  # wrong dtype
    with pytest.raises(fq.Fp4qError):
        fq.nvfp4_quantize_global(x, out=(good[0], good[1], f32(2), good[3]))
    with pytest.raises(fq.Fp4qError):
        fq.nvfp4_dequantize(good[0].view(R, H // 2), good[1], good[2], out=bf(R * H - 1))
    with pytest.raises(fq.Fp4qError):
        fq.nvfp4_dequantize(good[0].view(R, H // 2), u8(R * H // 16 - 1), good[2])
    with pytest.raises(fq.Fp4qError):  # codes must be [rows, hidden/2]
        fq.nvfp4_dequantize(good[0], good[1], good[2])
    mx = (u8(R * H // 2), u8(R * H // 32), u8(R * H // 4), u8(R * H // 8), u8(R * H // 32))
    for k in range(5):
        bad = tuple(u8(t.numel() - 1) if j == k else t for j, t in enumerate(mx))
        with pytest.raises(fq.Fp4qError):
            fq.mxfp4_resq_quantize(x, out=bad)
    dense = (mx[0], mx[1], u8(R * H // 2), mx[4])
    for k in range(4):
        bad = tuple(u8(t.numel() - 1) if j == k else t for j, t in enumerate(dense))
        with pytest.raises(fq.Fp4qError):
            fq.mxfp4_resq_dense_quantize(x, out=bad)
    c2 = mx[0].view(R, H // 2)
    with pytest.raises(fq.Fp4qError):  # S2:4 reconstruction needs the metadata
        fq.mxfp4_resq_reconstruct(c2, mx[1], mx[2], None, mx[4], residual=1)
    with pytest.raises(fq.Fp4qError):  # dense residual codes are [R, H/2]
        fq.mxfp4_resq_reconstruct(c2, mx[1], mx[2], None, mx[4], residual=2)
    with pytest.raises(fq.Fp4qError):
        fq.mxfp4_resq_reconstruct(c2, mx[1], out=f32(R * H - 1))
    guide = (u8(R * H // 2), u8(R * H // 16), f32(R))
    for k in range(3):
        bad = tuple(t[:-1] if j == k else t for j, t in enumerate(guide))
        with pytest.raises(fq.Fp4qError):
            fq.nvfp4_quantize_guided(x, *bad)
    with pytest.raises(fq.Fp4qError):
        fq.nvfp4_quantize_guided(x, *guide, out=(u8(R * H // 2 - 1), None))
    with pytest.raises(fq.Fp4qError):
        fq.nvfp4_quantize_guided(x, *guide, out=(u8(R * H // 2), bf(R * H - 1)))
    torch.cuda.synchronize()


# ------------------------------------------------- TRACE guided rounding --

def check_guided(x_rollout, x_train, label, guided=True):
    """The rollout's outputs from the oracle; the training side guided by
    its codes under its scales (or, guided False, rounded to nearest under
    them)."""
    codes, scales, ts, _ = oracle_nvfp4(x_rollout, 1, dequant=False)
    guide = codes if guided else None
    gu = Guards()
    got = fq.nvfp4_quantize_guided(to_dev(x_train),
                                   None if guide is None else torch.from_numpy(guide).cuda(),
                                   torch.from_numpy(scales).cuda(), torch.from_numpy(ts).cuda(),
                                   out=gu.guided(*x_train.shape))
    gu.check(label)
    want = oracle.nvfp4_quantize_guided(x_train, guide, scales, ts)
    assert_same(host(got[0]), want[0], label + " codes")
    assert_same(bits_of(got[1]), want[1], label + " dequant")


@pytest.mark.parametrize("H", [16, 2048, 7168, 7184])
def test_guided_edge_rows(H):
    x = edge_rows(H, seed=H + 7)
    check_guided(x, workloads.perturbed(x, seed=H), "guided edge H=%d" % H)
    # a guide from unrelated values, and the tensor guided by itself
    check_guided(edge_rows(H, seed=H + 99), x, "guided cross H=%d" % H)
    check_guided(x, x, "guided self H=%d" % H)
    # no guide: round to nearest under the rollout's scales
    check_guided(x, workloads.perturbed(x, seed=H), "nearest edge H=%d" % H, guided=False)
    check_guided(edge_rows(H, seed=H + 99), x, "nearest cross H=%d" % H, guided=False)


@pytest.mark.parametrize("H", [2048, 7168])
def test_guided_every_bf16_value(H):
    x = every_bf16_rows(H, seed=H + 11)
    check_guided(x, workloads.perturbed(x, seed=H + 1), "guided every BF16 value H=%d" % H)
    check_guided(x, x, "guided self every BF16 value H=%d" % H)
    check_guided(x, workloads.perturbed(x, seed=H + 1), "nearest every BF16 value H=%d" % H,
                 guided=False)


def test_guided_random_guides_and_scales():
    # arbitrary guide bytes and block scales (every branch of the rule)
    rng = np.random.default_rng(77)
    rows, H = 64, 2048
    x = workloads.rows("moe_act", 0, rows)[:, :H].copy()
    guide = rng.integers(0, 256, (rows, H // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (rows, H // 16), dtype=np.uint8)
    ts = (np.abs(rng.standard_normal(rows)) * 0.01).astype(np.float32)
    ts[::5] *= np.float32(2.0 ** -120)  # rows whose decode steps are subnormal (r = inf)
    for gd in (guide, None):
        gu = Guards()
        got = fq.nvfp4_quantize_guided(to_dev(x), None if gd is None else torch.from_numpy(gd).cuda(),
                                       torch.from_numpy(scales).cuda(),
                                       torch.from_numpy(ts).cuda(), out=gu.guided(rows, H))
        label = "guided random" if gd is not None else "nearest random"
        gu.check(label)
        want = oracle.nvfp4_quantize_guided(x, gd, scales, ts)
        assert_same(host(got[0]), want[0], label + " codes")
        assert_same(bits_of(got[1]), want[1], label + " dequant")


def test_guided_moe_act_full_size():
    x = workloads.rows("moe_act")
    check_guided(x, workloads.perturbed(x, seed=2), "guided moe_act")
    check_guided(x, workloads.perturbed(x, seed=2), "nearest moe_act", guided=False)


# ------------------------------------------------- global per-tensor scale --

def check_global(x_bits, fos, label):
    gu = Guards()
    out, ws = gu.global_(*x_bits.shape)
    got = fq.nvfp4_quantize_global(to_dev(x_bits), fos, out=out, workspace=ws)
    gu.check(label)
    want = oracle.nvfp4_quantize_global(x_bits, fos)
    assert_same(host(got[0]), want[0], label + " codes")
    assert_same(host(got[1]), want[1], label + " scales")
    assert_same(host(got[2])[None, :], want[2][None, :], label + " tensor scale")
    assert_same(bits_of(got[3]), want[3], label + " dequant")


@pytest.mark.parametrize("fos", [1, 0, 2])
@pytest.mark.parametrize("H", [16, 2048, 7168, 33024])
def test_global_scale_edge_rows(H, fos):
    check_global(edge_rows(H, seed=H + 3), fos, "global edge H=%d fos=%d" % (H, fos))


def test_global_scale_moe_act_full_size():
    check_global(workloads.rows("moe_act"), 1, "global moe_act")


@pytest.mark.parametrize("where", ["first", "last", "tail"])
def test_global_scale_max_anywhere(where):
    """The tensor max is found wherever it sits: the first element, the last
    one, or inside the part of the tensor past the last whole stride of the
    max pass (2000 x 7168 is 1,792,000 16-byte units; a 512 x 256 grid strides
    131,072 units, four at a time)."""
    rng = np.random.default_rng(11)
    R, H = 2000, 7168
    x = rng.standard_normal((R, H)).astype(np.float32)
    pos = {"first": (0, 0), "last": (R - 1, H - 1), "tail": (R - 37, 1000)}[where]
    x[pos] = -1000.0
    x_bits = f32_to_bf16_bits(x)
    check_global(x_bits, 1, "global max at %s" % where)


def test_global_scale_batch_dependency_on_gpu():
    # per-token results of a row do not depend on its batch; global ones do
    x = workloads.rows("moe_act", 0, 64)
    xs = to_dev(x)
    solo = fq.nvfp4_quantize_global(xs[5:6].contiguous())[0]
    batch = fq.nvfp4_quantize_global(xs)[0]
    torch.cuda.synchronize()
    assert not torch.equal(solo[0], batch[5])
    p_solo = fq.nvfp4_quantize(xs[5:6].contiguous())[0]
    p_batch = fq.nvfp4_quantize(xs)[0]
    torch.cuda.synchronize()
    assert torch.equal(p_solo[0], p_batch[5])
