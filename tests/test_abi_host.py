"""The C-ABI library on the host: it loads, exports every symbol include/lrq.h declares,
its descriptor layout matches the header, and every argument check fires before any
launch.  No call here reaches a kernel launch (every call with non-NULL addresses is
invalid by construction), and these tests are skipped where a GPU is visible so that a
regression in validation can never turn into a launch with made-up addresses."""
import ctypes
import os
import re
import subprocess

import pytest

from layer_rmsnorm_qkv_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lrq.h")


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:  # noqa: BLE001
        return False


pytestmark = [pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="liblrq.so not built"),
              pytest.mark.skipif(_gpu_visible(), reason="host-only checks use made-up addresses")]

FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lrq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = B.load()
    syms = declared_symbols()
    assert set(syms) == set(B.EXPORTED), syms
    for s in syms:
        assert hasattr(lib, s), s
    assert B.lrq_abi_version() == 5


def test_desc_layout_matches_header(tmp_path):
    fields = [f for f, _ in B.LrqDesc._fields_]
    src = tmp_path / "layout.c"
    body = "\n".join(f'  printf("{f} %zu\\n", offsetof(lrq_desc, {f}));' for f in fields)
    src.write_text(f'#include <stdio.h>\n#include <stddef.h>\n#include "lrq.h"\n'
                   f'int main(void) {{\n{body}\n  printf("size %zu\\n", sizeof(lrq_desc));\n  return 0;\n}}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                    "-o", str(exe)], check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                       check=True).stdout.splitlines())
    for f in fields:
        assert int(got[f]) == getattr(B.LrqDesc, f).offset, f
    assert int(got["size"]) == ctypes.sizeof(B.LrqDesc)


def test_status_strings():
    assert [B.lrq_status_string(i) for i in range(4)] == \
        ["LRQ_OK", "LRQ_ERR_INVALID_ARG", "LRQ_ERR_UNSUPPORTED", "LRQ_ERR_HIP"]
    assert B.lrq_status_string(99) == "LRQ_UNKNOWN_STATUS"


def good_desc(**kw):
    base = dict(n_tokens=8, d_model=64, n_q_heads=4, n_kv_heads=2, head_dim=16, dtype=B.LRQ_F32, eps=1e-6,
                rope_theta=1e4, lora_rank=4, lora_alpha=8.0, lora_targets=B.LRQ_TARGET_Q | B.LRQ_TARGET_V,
                has_bias=0)
    base.update(kw)
    return B.make_desc(**base)


def fwd(desc, **over):
    args = dict(x=FAKE, gamma=FAKE, w_qkv=FAKE, bias=None, lora_a=[FAKE, None, FAKE], lora_b=[FAKE, None, FAKE],
                positions=FAKE, out=FAKE, workspace=None, stream=None)
    args.update(over)
    B.lrq_forward(desc, **args)


def expect(status, fn, *a, **k):
    with pytest.raises(B.LrqError) as ei:
        fn(*a, **k)
    assert ei.value.status == status, str(ei.value)
    assert B.lrq_last_error() != ""


@pytest.mark.parametrize("field,value", [
    ("n_tokens", -1), ("d_model", 0), ("n_q_heads", 0), ("n_kv_heads", 0), ("n_q_heads", 3),
    ("head_dim", 15), ("head_dim", 0), ("dtype", 7), ("eps", -1.0), ("eps", float("nan")),
    ("rope_theta", 0.0), ("rope_theta", float("inf")), ("lora_targets", 8), ("lora_rank", 0),
    ("lora_alpha", float("nan")), ("has_bias", 2), ("variant", 9), ("lora_dropout", -0.1),
    ("lora_dropout", 1.0), ("lora_dropout", float("nan")), ("weight_format", 2), ("weight_format", -1)])
def test_invalid_descriptor(field, value):
    expect(B.LRQ_ERR_INVALID_ARG, fwd, good_desc(**{field: value}))
    assert B.lrq_workspace_size(good_desc(**{field: value})) == 0
    assert B.lrq_select_variant(good_desc(**{field: value})) == -1


@pytest.mark.parametrize("over", [dict(x=None), dict(gamma=None), dict(w_qkv=None), dict(positions=None),
                                  dict(out=None), dict(lora_a=None), dict(lora_b=[FAKE, None, None]),
                                  dict(lora_a=[None, None, FAKE])])
def test_missing_pointer(over):
    expect(B.LRQ_ERR_INVALID_ARG, fwd, good_desc(), **over)


def test_bias_required_and_alignment():
    expect(B.LRQ_ERR_INVALID_ARG, fwd, good_desc(has_bias=1), bias=None)
    expect(B.LRQ_ERR_UNSUPPORTED, fwd, good_desc(n_tokens=8, has_bias=1, eps=-1.0 + 1.0), bias=FAKE + 2,
           x=FAKE + 2)
    expect(B.LRQ_ERR_UNSUPPORTED, fwd, good_desc(lora_rank=65))


def test_forced_variant_that_cannot_run():
    # fp32 cannot use the bf16 MFMA families
    for v in (B.LRQ_VARIANT_TILED, B.LRQ_VARIANT_DECODE):
        assert B.lrq_select_variant(good_desc(variant=v)) == -1
        expect(B.LRQ_ERR_UNSUPPORTED, fwd, good_desc(variant=v))
    assert B.lrq_select_variant(good_desc()) == B.LRQ_VARIANT_GENERIC
    assert B.lrq_select_variant(good_desc(), for_backward=True) == B.LRQ_VARIANT_GENERIC


def test_dropout_workspace_and_family():
    # LoRA dropout keeps its keep bits in the workspace: [targets][T][ceil(d / 32)] uint32 for
    # the generic family (256-byte aligned); without targets the rate is ignored
    d = good_desc(n_tokens=100, d_model=80, lora_dropout=0.25)
    assert B.lrq_workspace_size(d) == (2 * 100 * 3 * 4 + 255) // 256 * 256
    assert B.lrq_workspace_size(d, for_backward=True) == B.lrq_workspace_size(d)
    assert B.lrq_workspace_size(good_desc(n_tokens=100, d_model=80, lora_dropout=0.25, lora_targets=0)) == 0
    assert B.lrq_workspace_size(good_desc(n_tokens=100, d_model=80)) == 0
    # bf16 decode-sized call: the decode family runs no dropout; AUTO picks another one and a
    # forced decode call is refused
    dec = dict(n_tokens=4, d_model=1024, n_q_heads=8, n_kv_heads=2, head_dim=128, dtype=B.LRQ_BF16)
    assert B.lrq_select_variant(good_desc(**dec)) == B.LRQ_VARIANT_DECODE
    assert B.lrq_select_variant(good_desc(**dec, lora_dropout=0.1)) == B.LRQ_VARIANT_TILED
    assert B.lrq_select_variant(good_desc(**dec, lora_dropout=0.1, variant=B.LRQ_VARIANT_DECODE)) == -1
    assert B.lrq_select_variant(good_desc(**dec, lora_dropout=0.1, lora_targets=0,
                                          variant=B.LRQ_VARIANT_DECODE)) == B.LRQ_VARIANT_DECODE
    # the tiled families add the masked adapter inputs (bf16 [targets][T][d])
    base = good_desc(**dec, variant=B.LRQ_VARIANT_TILED)
    drop = good_desc(**dec, variant=B.LRQ_VARIANT_TILED, lora_dropout=0.1)
    a256 = lambda n: (n + 255) // 256 * 256  # noqa: E731
    rows, xm = a256(2 * 4 * 32 * 4), a256(2 * 4 * 1024 * 2)
    assert B.lrq_workspace_size(drop) == a256(B.lrq_workspace_size(base)) + rows + xm
    assert B.lrq_workspace_size(drop, True) == a256(B.lrq_workspace_size(base, True)) + rows + xm


def test_nf4_sizes_and_checks():
    # NF4 buffer: codes N * d / 2 bytes rounded up to 256, then N * d / 64 float32 scales
    d = good_desc(d_model=128)                      # N = (4 + 2 * 2) * 16 = 128
    assert B.lrq_nf4_weight_size(d) == (128 * 128 // 2 + 255) // 256 * 256 + 128 * 2 * 4
    assert B.lrq_nf4_weight_size(good_desc(d_model=96)) == 0
    assert B.lrq_nf4_weight_size(good_desc(n_q_heads=0)) == 0
    expect(B.LRQ_ERR_UNSUPPORTED, fwd, good_desc(d_model=96, weight_format=B.LRQ_WEIGHT_NF4))
    expect(B.LRQ_ERR_UNSUPPORTED, B.lrq_quantize_nf4, good_desc(d_model=96), FAKE, FAKE, 1 << 20)
    expect(B.LRQ_ERR_INVALID_ARG, B.lrq_quantize_nf4, d, FAKE, FAKE, 100)
    expect(B.LRQ_ERR_INVALID_ARG, B.lrq_quantize_nf4, d, None, FAKE, 1 << 20)
    expect(B.LRQ_ERR_UNSUPPORTED, B.lrq_quantize_nf4, d, FAKE + 4, FAKE, 1 << 20)
    # every bf16 family takes NF4 weights (decode included)
    dec = dict(n_tokens=4, d_model=1024, n_q_heads=8, n_kv_heads=2, head_dim=128, dtype=B.LRQ_BF16)
    assert B.lrq_select_variant(good_desc(**dec, weight_format=B.LRQ_WEIGHT_NF4)) == B.LRQ_VARIANT_DECODE
    assert B.lrq_select_variant(good_desc(**dec, weight_format=B.LRQ_WEIGHT_NF4,
                                          variant=B.LRQ_VARIANT_TILED)) == B.LRQ_VARIANT_TILED
    # T == 0 with NF4 is still a no-op
    B.lrq_forward(good_desc(d_model=128, n_tokens=0, weight_format=B.LRQ_WEIGHT_NF4), None, None, None, None,
                  [FAKE, None, FAKE], [FAKE, None, FAKE], None, None)


def test_attn_desc_layout_matches_header(tmp_path):
    fields = [f for f, _ in B.LrqAttnDesc._fields_]
    src = tmp_path / "attn_layout.c"
    body = "\n".join(f'  printf("{f} %zu\\n", offsetof(lrq_attn_desc, {f}));' for f in fields)
    src.write_text(f'#include <stdio.h>\n#include <stddef.h>\n#include "lrq.h"\n'
                   f'int main(void) {{\n{body}\n  printf("size %zu\\n", sizeof(lrq_attn_desc));\n  return 0;\n}}\n')
    exe = tmp_path / "attn_layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                    "-o", str(exe)], check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                       check=True).stdout.splitlines())
    for f in fields:
        assert int(got[f]) == getattr(B.LrqAttnDesc, f).offset, f
    assert int(got["size"]) == ctypes.sizeof(B.LrqAttnDesc)


def attn_desc(**kw):
    base = dict(n_seqs=2, n_q_heads=8, n_kv_heads=2, head_dim=128, max_q_len=4, ld_q=1536, num_slots=64)
    base.update(kw)
    return B.make_attn_desc(**base)


def attn(desc, **over):
    args = dict(q=FAKE, k_cache=FAKE, v_cache=FAKE, q_indptr=FAKE, kv_indptr=FAKE, kv_slots=FAKE, out=FAKE)
    args.update(over)
    B.lrq_attention(desc, **args)


@pytest.mark.parametrize("over,status", [
    (dict(n_seqs=-1), B.LRQ_ERR_INVALID_ARG), (dict(n_q_heads=0), B.LRQ_ERR_INVALID_ARG),
    (dict(n_q_heads=6, n_kv_heads=4), B.LRQ_ERR_INVALID_ARG), (dict(ld_q=1000), B.LRQ_ERR_INVALID_ARG),
    (dict(scale=-1.0), B.LRQ_ERR_INVALID_ARG), (dict(scale=float("inf")), B.LRQ_ERR_INVALID_ARG),
    (dict(causal=2), B.LRQ_ERR_INVALID_ARG), (dict(max_q_len=-1), B.LRQ_ERR_INVALID_ARG),
    (dict(head_dim=64), B.LRQ_ERR_UNSUPPORTED), (dict(dtype=B.LRQ_F32), B.LRQ_ERR_UNSUPPORTED),
    (dict(ld_q=1540), B.LRQ_ERR_UNSUPPORTED), (dict(max_q_len=1 << 30), B.LRQ_ERR_UNSUPPORTED)])
def test_attention_checks(over, status):
    expect(status, attn, attn_desc(**over))


def test_attention_pointer_checks_and_noop():
    expect(B.LRQ_ERR_INVALID_ARG, attn, attn_desc(), kv_slots=None)
    expect(B.LRQ_ERR_INVALID_ARG, attn, attn_desc(), out=None)
    expect(B.LRQ_ERR_UNSUPPORTED, attn, attn_desc(), q=FAKE + 8)
    expect(B.LRQ_ERR_UNSUPPORTED, attn, attn_desc(), kv_slots=FAKE + 2)
    # nothing to do: NULL pointers are fine
    B.lrq_attention(attn_desc(n_seqs=0), None, None, None, None, None, None, None)
    B.lrq_attention(attn_desc(max_q_len=0), None, None, None, None, None, None, None)


def test_zero_tokens_is_a_noop():
    # T == 0: valid, nothing is launched, pointers may be NULL
    B.lrq_forward(good_desc(n_tokens=0), None, None, None, None, [FAKE, None, FAKE], [FAKE, None, FAKE],
                  None, None)
    B.lrq_forward(good_desc(n_tokens=0, lora_targets=0), None, None, None, None, None, None, None, None)


def fwd_kv(desc, kv_over=None, **over):
    args = dict(x=FAKE, gamma=FAKE, w_qkv=FAKE, bias=None, lora_a=[FAKE, None, FAKE], lora_b=[FAKE, None, FAKE],
                positions=FAKE, out=FAKE, k_cache=FAKE, v_cache=FAKE, slots=FAKE, num_slots=16, workspace=None,
                stream=None)
    args.update(over)
    args.update(kv_over or {})
    B.lrq_forward_kv(desc, **args)


def test_forward_kv_checks():
    # every call fails validation: the cache arguments are checked like the others
    expect(B.LRQ_ERR_INVALID_ARG, fwd_kv, good_desc(), dict(num_slots=-1))
    for missing in ("k_cache", "v_cache", "slots"):
        expect(B.LRQ_ERR_INVALID_ARG, fwd_kv, good_desc(), {missing: None})
    expect(B.LRQ_ERR_UNSUPPORTED, fwd_kv, good_desc(), dict(slots=FAKE + 4))
    expect(B.LRQ_ERR_UNSUPPORTED, fwd_kv, good_desc(), dict(k_cache=FAKE + 2))
    # the forward's own checks still apply
    expect(B.LRQ_ERR_INVALID_ARG, fwd_kv, good_desc(n_q_heads=3))
    expect(B.LRQ_ERR_INVALID_ARG, fwd_kv, good_desc(), out=None)
    # T == 0: nothing to write, NULL caches allowed
    B.lrq_forward_kv(good_desc(n_tokens=0, lora_targets=0), None, None, None, None, None, None, None, None,
                     None, None, None, 0)


def test_backward_checks():
    def bwd(desc, **over):
        args = dict(x=FAKE, gamma=FAKE, w_qkv=FAKE, bias=None, lora_a=[FAKE, None, FAKE],
                    lora_b=[FAKE, None, FAKE], positions=FAKE, y=FAKE, dy=FAKE, dx=FAKE,
                    d_lora_a=[FAKE, None, FAKE], d_lora_b=[FAKE, None, FAKE])
        args.update(over)
        B.lrq_backward(desc, **args)
    for over in (dict(y=None), dict(dy=None), dict(dx=None), dict(d_lora_a=None),
                 dict(d_lora_b=[FAKE, None, None])):
        expect(B.LRQ_ERR_INVALID_ARG, bwd, good_desc(), **over)
    expect(B.LRQ_ERR_INVALID_ARG, bwd, good_desc(head_dim=3))
    expect(B.LRQ_ERR_UNSUPPORTED, bwd, good_desc(), dy=FAKE + 4)


def test_workspace_alignment():
    # the bf16 families need a workspace; one that is not 256-byte aligned is refused
    desc = good_desc(dtype=B.LRQ_BF16, n_tokens=64, d_model=512, n_q_heads=4, n_kv_heads=4, head_dim=128)
    need = B.lrq_workspace_size(desc)
    assert need > 0
    expect(B.LRQ_ERR_UNSUPPORTED, fwd, desc, workspace=FAKE + 16, workspace_bytes=need)
    expect(B.LRQ_ERR_INVALID_ARG, fwd, desc, workspace=FAKE, workspace_bytes=need - 1)
    bdesc = good_desc(dtype=B.LRQ_BF16, n_tokens=256, d_model=512, n_q_heads=4, n_kv_heads=4, head_dim=128)
    bneed = B.lrq_workspace_size(bdesc, True)
    assert bneed > 0

    def bwd(**over):
        args = dict(x=FAKE, gamma=FAKE, w_qkv=FAKE, bias=None, lora_a=[FAKE, None, FAKE],
                    lora_b=[FAKE, None, FAKE], positions=FAKE, y=FAKE, dy=FAKE, dx=FAKE,
                    d_lora_a=[FAKE, None, FAKE], d_lora_b=[FAKE, None, FAKE], workspace=FAKE + 256 + 16,
                    workspace_bytes=bneed)
        args.update(over)
        B.lrq_backward(bdesc, **args)
    expect(B.LRQ_ERR_UNSUPPORTED, bwd)


def test_workspace_queries():
    assert B.lrq_workspace_size(good_desc()) == 0  # the generic family needs none
    assert B.lrq_workspace_size(good_desc(), True) == 0


def test_timing_hook_without_calls():
    """The measurement hook: enabling it clears the record, nothing recorded reads as 0 calls,
    and NULL outputs are rejected."""
    B.lrq_kernel_timing(True)
    assert B.lrq_kernel_time_ms(False) == (0.0, 0)
    assert B.lrq_kernel_time_ms(True) == (0.0, 0)
    lib = B.load()
    n = ctypes.c_int(-1)
    assert lib.lrq_kernel_time_ms(0, None, ctypes.byref(n)) == B.LRQ_ERR_INVALID_ARG
    ms = ctypes.c_double(-1.0)
    assert lib.lrq_kernel_time_ms(1, ctypes.byref(ms), None) == B.LRQ_ERR_INVALID_ARG
    B.lrq_kernel_timing(False)
    assert B.lrq_kernel_time_ms(False) == (0.0, 0)


def test_prepared_weight_checks():
    """Prepared frozen weights: sizes, and every argument check of the preparation and of the
    calls that take the buffer (each call below fails validation before any launch)."""
    assert B.lrq_prepared_size(good_desc()) == 0  # float32: only the generic family runs
    B.lrq_prepare_weights(good_desc(), True, FAKE, FAKE, None)  # size 0: a no-op
    desc = good_desc(dtype=B.LRQ_BF16, n_tokens=4096, d_model=512, n_q_heads=4, n_kv_heads=4, head_dim=128)
    N, d = 12 * 128, 512
    assert B.lrq_prepared_size(desc) == N * d * 2  # W' for the tiled forward
    assert B.lrq_prepared_size(desc, True) == 2 * N * d * 2  # + W^T for the tiled backward
    # independent of the token count (and of the family the call's T would pick)
    assert B.lrq_prepared_size(good_desc(dtype=B.LRQ_BF16, n_tokens=1, d_model=512, n_q_heads=4, n_kv_heads=4,
                                         head_dim=128), True) == 2 * N * d * 2
    need = B.lrq_prepared_size(desc, True)
    expect(B.LRQ_ERR_INVALID_ARG, B.lrq_prepare_weights, desc, True, None, FAKE, FAKE, need)
    expect(B.LRQ_ERR_INVALID_ARG, B.lrq_prepare_weights, desc, True, FAKE, FAKE, None, need)
    expect(B.LRQ_ERR_INVALID_ARG, B.lrq_prepare_weights, desc, True, FAKE, FAKE, FAKE, need - 1)
    expect(B.LRQ_ERR_UNSUPPORTED, B.lrq_prepare_weights, desc, True, FAKE, FAKE, FAKE + 16, need)
    # the prepared call's workspace is smaller (no per-call W' / W^T)
    assert 0 < B.lrq_workspace_size_prepared(desc) < B.lrq_workspace_size(desc)
    assert 0 < B.lrq_workspace_size_prepared(desc, True) < B.lrq_workspace_size(desc, True)
    ws = B.lrq_workspace_size_prepared(desc)

    def fwdp(**over):
        args = dict(x=FAKE, gamma=FAKE, w_qkv=FAKE, prepared=FAKE, bias=None, lora_a=[FAKE, None, FAKE],
                    lora_b=[FAKE, None, FAKE], positions=FAKE, out=FAKE, kv=None, workspace=FAKE,
                    workspace_bytes=ws, prepared_bytes=need)
        args.update(over)
        B.lrq_forward_prepared(desc, **args)
    expect(B.LRQ_ERR_INVALID_ARG, fwdp, prepared_bytes=N * d * 2 - 1)  # below the forward layout
    expect(B.LRQ_ERR_UNSUPPORTED, fwdp, prepared=FAKE + 16)
    expect(B.LRQ_ERR_INVALID_ARG, fwdp, workspace_bytes=ws - 1)
    expect(B.LRQ_ERR_INVALID_ARG, fwdp, x=None)
    bws = B.lrq_workspace_size_prepared(desc, True)

    def bwdp(**over):
        args = dict(x=FAKE, gamma=FAKE, w_qkv=FAKE, prepared=FAKE, bias=None, lora_a=[FAKE, None, FAKE],
                    lora_b=[FAKE, None, FAKE], positions=FAKE, y=FAKE, dy=FAKE, dx=FAKE,
                    d_lora_a=[FAKE, None, FAKE], d_lora_b=[FAKE, None, FAKE], workspace=FAKE,
                    workspace_bytes=bws, prepared_bytes=need)
        args.update(over)
        B.lrq_backward_prepared(desc, **args)
    # a buffer prepared for the forward only is too small for the backward
    expect(B.LRQ_ERR_INVALID_ARG, bwdp, prepared_bytes=N * d * 2)
    expect(B.LRQ_ERR_UNSUPPORTED, bwdp, prepared=FAKE + 16)
    expect(B.LRQ_ERR_INVALID_ARG, bwdp, workspace_bytes=bws - 1)


def test_noalloc_checks():
    """The no-allocation forward validates like lrq_forward_prepared and refuses a call whose
    scratch would exceed the library's array, before any HIP call."""
    assert B.NOALLOC_SCRATCH_BYTES == 16 << 20
    text = open(HEADER).read()
    assert "#define LRQ_NOALLOC_SCRATCH_BYTES (16u << 20)" in text

    def noalloc(desc, **over):
        args = dict(x=FAKE, gamma=FAKE, w_qkv=FAKE, prepared=None, bias=None, lora_a=[FAKE, None, FAKE],
                    lora_b=[FAKE, None, FAKE], positions=FAKE, out=FAKE, kv=None)
        args.update(over)
        B.lrq_forward_noalloc(desc, **args)
    expect(B.LRQ_ERR_INVALID_ARG, noalloc, good_desc(n_q_heads=3))
    expect(B.LRQ_ERR_INVALID_ARG, noalloc, good_desc(), x=None)
    # tiled family without prepared weights: W' (8192 x 1536 bf16 = 24 MiB) does not fit
    big = good_desc(dtype=B.LRQ_BF16, n_tokens=4096, d_model=8192, n_q_heads=4, n_kv_heads=4, head_dim=128)
    assert B.lrq_workspace_size(big) > B.NOALLOC_SCRATCH_BYTES
    expect(B.LRQ_ERR_UNSUPPORTED, noalloc, big)
    assert "scratch" in B.lrq_last_error()


def test_mlp_desc_layout_and_checks(tmp_path):
    """lrq_mlp_desc matches the header's layout; lrq_mlp_forward validates before any launch."""
    fields = [f for f, _ in B.LrqMlpDesc._fields_]
    src = tmp_path / "mlp_layout.c"
    body = "\n".join(f'  printf("{f} %zu\\n", offsetof(lrq_mlp_desc, {f}));' for f in fields)
    src.write_text(f'#include <stdio.h>\n#include <stddef.h>\n#include "lrq.h"\n'
                   f'int main(void) {{\n{body}\n  printf("size %zu\\n", sizeof(lrq_mlp_desc));\n  return 0;\n}}\n')
    exe = tmp_path / "mlp_layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                    "-o", str(exe)], check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                       check=True).stdout.splitlines())
    for f in fields:
        assert int(got[f]) == getattr(B.LrqMlpDesc, f).offset, f
    assert int(got["size"]) == ctypes.sizeof(B.LrqMlpDesc)

    good = dict(n_tokens=300, d_model=512, d_ff=384, dtype=B.LRQ_BF16, lora_rank=16, lora_alpha=32.0, lora_targets=7)
    desc = B.make_mlp_desc(**good)
    assert B.lrq_mlp_workspace_size(desc) == 300 * 384 * 2
    ws = B.lrq_mlp_workspace_size(desc)

    def call(d, **over):
        args = dict(h=FAKE, w_gate=FAKE, w_up=FAKE, w_down=FAKE, lora_a=[FAKE, FAKE, FAKE],
                    lora_b=[FAKE, FAKE, FAKE], out=FAKE, workspace=FAKE, workspace_bytes=ws)
        args.update(over)
        B.lrq_mlp_forward(d, **args)
    for field, value in (("n_tokens", -1), ("d_model", 0), ("dtype", 5), ("lora_targets", 8), ("lora_rank", 0)):
        expect(B.LRQ_ERR_INVALID_ARG, call, B.make_mlp_desc(**dict(good, **{field: value})))
        assert B.lrq_mlp_workspace_size(B.make_mlp_desc(**dict(good, **{field: value}))) == 0
    expect(B.LRQ_ERR_UNSUPPORTED, call, B.make_mlp_desc(**dict(good, dtype=B.LRQ_F32)))
    expect(B.LRQ_ERR_UNSUPPORTED, call, B.make_mlp_desc(**dict(good, lora_rank=33)))
    expect(B.LRQ_ERR_UNSUPPORTED, call, B.make_mlp_desc(**dict(good, d_model=500)))
    expect(B.LRQ_ERR_INVALID_ARG, call, desc, h=None)
    expect(B.LRQ_ERR_INVALID_ARG, call, desc, lora_b=[FAKE, None, FAKE])
    expect(B.LRQ_ERR_INVALID_ARG, call, desc, workspace_bytes=ws - 1)
    expect(B.LRQ_ERR_UNSUPPORTED, call, desc, out=FAKE + 2)
    # T == 0: a no-op with NULL arrays
    B.lrq_mlp_forward(B.make_mlp_desc(**dict(good, n_tokens=0)), None, None, None, None, [FAKE] * 3, [FAKE] * 3,
                      None)
