"""C-ABI checks that need no GPU (CPU only).

* libpagedattn.so loads and exports every function include/pagedattn.h
  declares.
* The ctypes mirror of pa_args has the layout a C compiler gives the header.
* Host-side validation returns the typed status codes before any device work
  (the acceptance criteria of "Add Qwen3.8 packed hybrid PagedAttention export
  for ORT GenAI Engine" ask for typed errors on unsupported combinations);
  the pointers used here are fake and are never dereferenced because every
  case fails, or has no token, before a launch.
"""
import ctypes
import os
import re
import subprocess

import pytest

import paged_kv_varlen_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedattn.h")

OK, NULL, SHAPE, UNSUP, WS, ALIGN, ABI, META, HIP = range(9)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function():
    lib = pa.library()
    names = declared_functions()
    assert set(names) == {"pa_paged_attention", "pa_workspace_bytes", "pa_status_string",
                          "pa_abi_version", "pa_merge_states", "pa_paged_attention_noalloc"}
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", pa.library_path], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (pa_\w+)", out))
    assert set(names) <= exported


@pytest.mark.parametrize("cls,cname", [(pa.PaArgs, "pa_args"), (pa.PaMergeArgs, "pa_merge_args")])
def test_struct_layout_matches_c(tmp_path, cls, cname):
    fields = [f for f, _ in cls._fields_]
    src = tmp_path / "layout.c"
    body = "\n".join(f'  printf("{f} %zu\\n", offsetof({cname}, {f}));' for f in fields)
    src.write_text(f"""#include <stdio.h>
#include <stddef.h>
#include "pagedattn.h"
int main(void) {{
  printf("sizeof %zu\\n", sizeof({cname}));
{body}
  return 0;
}}
""")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER),
                    str(src), "-o", str(exe)], check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True,
                                                         text=True, check=True).stdout.splitlines())
    assert int(got["sizeof"]) == ctypes.sizeof(cls)
    for f in fields:
        assert int(got[f]) == getattr(cls, f).offset, f


FAKE = 1 << 20  # an aligned, never-dereferenced address


def args(**kw):
    a = pa.PaArgs()
    a.struct_size = ctypes.sizeof(pa.PaArgs)
    a.dtype = 1
    for p in ("query", "key", "value", "key_cache", "value_cache", "cumulative_sequence_length",
              "past_seqlens", "block_table", "output"):
        setattr(a, p, FAKE)
    a.num_tokens, a.batch_size = 4, 2
    a.num_heads, a.kv_num_heads = 4, 2
    a.query_width = 4 * 64
    a.num_blocks, a.block_size, a.cache_kv_heads, a.cache_head_size = 8, 16, 2, 64
    a.max_blocks_per_seq = 4
    a.is_causal = 1
    a.workspace = FAKE
    a.workspace_bytes = 0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def status(a):
    return pa.library().pa_paged_attention(ctypes.byref(a) if a is not None else None, None)


def test_workspace_bytes_static_bound():
    a = args()
    need = pa.workspace_bytes(a)
    assert need > 0 and need % 256 == 0
    bigger = args(max_blocks_per_seq=400)
    assert pa.workspace_bytes(bigger) > need
    assert pa.workspace_bytes(args(num_heads=3)) == 0  # invalid shape -> 0


@pytest.mark.parametrize("case,expect", [
    (dict(), WS),                                        # workspace too small
    (dict(struct_size=8), ABI),
    (dict(num_heads=3), SHAPE),                          # H % Hkv != 0
    (dict(value=None), SHAPE),                           # key without value
    (dict(query_width=4 * 64 + 1), SHAPE),
    (dict(cache_head_size=32), SHAPE),                   # cache dims disagree with D
    (dict(cache_kv_heads=1), SHAPE),
    (dict(batch_size=0), SHAPE),                         # tokens without sequences
    (dict(num_tokens=-1), SHAPE),
    (dict(num_blocks=0), SHAPE),
    (dict(is_causal=0), UNSUP),                          # only is_causal=1 exists
    (dict(dtype=0), UNSUP),                              # T must be float16 or bfloat16
    (dict(dtype=3), UNSUP),
    (dict(dtype=2), WS),                                 # bfloat16 passes validation
    (dict(block_size=8), UNSUP),
    (dict(query_width=4 * 32, cache_head_size=32), UNSUP),  # D=32 not built
    (dict(query_width=4 * 256, cache_head_size=256), WS),   # D=256 passes validation
    (dict(query=None), NULL),
    (dict(output=None), NULL),
    (dict(query=FAKE + 2), ALIGN),
    (dict(key_cache=FAKE + 8), ALIGN),
    (dict(lse=FAKE + 2), ALIGN),                         # lse needs 4-byte alignment
    (dict(output_f32=FAKE + 4), ALIGN),                  # output_f32 needs 16
    (dict(lse=FAKE, output_f32=FAKE), WS),               # both present and aligned
    (dict(gate=FAKE + 8), ALIGN),                        # the output gate needs 16-byte alignment
    (dict(gate=FAKE), WS),                               # an aligned gate passes validation
    (dict(kv_quant=3), UNSUP),                           # only PA_KV_SAME, PA_KV_INT8, PA_KV_INT4
    (dict(kv_quant=-1), UNSUP),
    (dict(reserved=1), UNSUP),                           # reserved field must be 0
    (dict(kv_quant=2, k_scale=FAKE, v_scale=FAKE), SHAPE),  # INT4 rows are head_size / 2 bytes
    (dict(kv_quant=2, cache_head_size=32), NULL),        # INT4 caches need both scale rows
    (dict(kv_quant=2, cache_head_size=32, k_scale=FAKE, v_scale=FAKE), WS),  # INT4 passes validation
    (dict(kv_quant=2, k_scale=FAKE, v_scale=FAKE, query_width=4 * 256, cache_head_size=128,
          dtype=2), WS),                                 # INT4 with bfloat16 and D=256
    (dict(kv_quant=1), NULL),                            # INT8 caches need both scale rows
    (dict(kv_quant=1, k_scale=FAKE), NULL),
    (dict(kv_quant=1, k_scale=FAKE, v_scale=FAKE + 4), ALIGN),  # scales need 16-byte alignment
    (dict(kv_quant=1, k_scale=FAKE, v_scale=FAKE), WS),  # INT8 passes validation
    (dict(kv_quant=0, k_scale=FAKE + 4), WS),            # scales ignored for 16-bit caches
    (dict(kv_quant=1, k_scale=FAKE, v_scale=FAKE, dtype=2,
          query_width=4 * 256, cache_head_size=256), WS),  # with bfloat16 and D=256
    (dict(num_tokens=0, batch_size=2), OK),              # nothing to do: no device work
])
def test_host_validation(case, expect):
    assert status(args(**case)) == expect


def test_null_args_pointer():
    assert pa.library().pa_paged_attention(None, None) == NULL


def test_readme_example_shape_is_typed_unsupported():
    # README example: H=2, Hkv=1, D=2, block_size 2, 3 blocks, B=1, N=2.
    a = args(num_tokens=2, batch_size=1, num_heads=2, kv_num_heads=1, query_width=4,
             num_blocks=3, block_size=2, cache_kv_heads=1, cache_head_size=2,
             max_blocks_per_seq=3)
    assert status(a) == UNSUP


def test_packed_width_resolution():
    # packed [Q|K|V] width (H+2Hkv)*D with key=value=NULL resolves D=64
    a = args(key=None, value=None, query_width=(4 + 4) * 64)
    assert pa.workspace_bytes(a) > 0
    assert status(a) == WS


def test_status_strings():
    lib = pa.library()
    for s in range(9):
        assert lib.pa_status_string(s)
    assert lib.pa_abi_version() == 5


def merge_args(**kw):
    a = pa.PaMergeArgs()
    a.struct_size = ctypes.sizeof(pa.PaMergeArgs)
    a.dtype = 1
    a.num_states, a.head_size, a.num_rows = 3, 128, 10
    a.state_out = a.state_lse = a.output = FAKE
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("case,expect", [
    (dict(struct_size=8), ABI),
    (dict(num_states=0), SHAPE),
    (dict(num_rows=-1), SHAPE),
    (dict(head_size=0), SHAPE),
    (dict(head_size=6), UNSUP),                          # not a multiple of 4
    (dict(head_size=1024), UNSUP),
    (dict(dtype=0), UNSUP),
    (dict(dtype=3), UNSUP),
    (dict(dtype=2, num_rows=0), OK),                     # bfloat16 output accepted
    (dict(state_out=None), NULL),
    (dict(state_lse=None), NULL),
    (dict(state_out=FAKE + 4), ALIGN),
    (dict(output_f32=FAKE + 8), ALIGN),
    (dict(num_rows=0), OK),                              # no rows: no device work
])
def test_merge_host_validation(case, expect):
    a = merge_args(**case)
    assert pa.library().pa_merge_states(ctypes.byref(a), None) == expect


def test_merge_null_args_pointer():
    assert pa.library().pa_merge_states(None, None) == NULL


def status_noalloc(a):
    return pa.library().pa_paged_attention_noalloc(ctypes.byref(a) if a is not None else None, None)


def test_noalloc_scratch_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define PA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == pa.NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("case,expect", [
    (dict(struct_size=8), ABI),
    (dict(num_heads=3), SHAPE),
    (dict(is_causal=0), UNSUP),
    (dict(query=None), NULL),
    (dict(query=FAKE + 2), ALIGN),
    (dict(kv_quant=1), NULL),
    (dict(num_tokens=0, batch_size=2), OK),              # nothing to do: no device work
    # shapes whose workspace exceeds the scratch: rejected before any device work
    (dict(num_tokens=8_000_000, batch_size=8_000_000), WS),
])
def test_noalloc_host_validation(case, expect):
    a = args(**case)
    if expect == WS:
        assert pa.workspace_bytes(a) > pa.NOALLOC_SCRATCH_BYTES
    assert status_noalloc(a) == expect


def test_noalloc_null_args_pointer():
    assert pa.library().pa_paged_attention_noalloc(None, None) == NULL


def sections(a, b, c):
    return (ctypes.c_int32 * 3)(a, b, c)


@pytest.mark.parametrize("case,expect", [
    (dict(rotary_dim=8), UNSUP),                          # not a multiple of 16
    (dict(rotary_dim=80), UNSUP),                         # wider than the head (D=64)
    (dict(rotary_dim=-16), UNSUP),
    (dict(rope_flags=4), UNSUP),                          # unknown flag
    (dict(rotary_dim=32, rope_theta=1e6, mrope_section=sections(16, 0, 0), position_ids=FAKE), WS),
    (dict(rotary_dim=64, rope_theta=1e4, mrope_section=sections(11, 11, 10), position_ids=FAKE,
          rope_flags=3), WS),                             # full rotation, both flags
    (dict(rotary_dim=32, rope_theta=1e6, mrope_section=sections(10, 0, 0), position_ids=FAKE), SHAPE),
    (dict(rotary_dim=32, rope_theta=1e6, mrope_section=sections(17, -1, 0), position_ids=FAKE), SHAPE),
    (dict(rotary_dim=32, rope_theta=0.0, mrope_section=sections(16, 0, 0), position_ids=FAKE), SHAPE),
    (dict(rotary_dim=32, rope_theta=1e6, mrope_section=sections(16, 0, 0)), NULL),  # no positions
    (dict(rotary_dim=32, rope_theta=1e6, mrope_section=sections(16, 0, 0), position_ids=FAKE + 4), ALIGN),
    (dict(q_norm_weight=FAKE + 4), ALIGN),                # norm weights need 16-byte alignment
    (dict(k_norm_weight=FAKE + 8), ALIGN),
    (dict(q_norm_weight=FAKE, k_norm_weight=FAKE), WS),   # norms alone pass validation
    (dict(mrope_section=sections(1, 2, 3)), WS),          # sections are ignored without rotation
])
def test_prologue_host_validation(case, expect):
    assert status(args(**case)) == expect


def test_prologue_workspace_holds_the_query_rows():
    plain = pa.workspace_bytes(args())
    with_norm = pa.workspace_bytes(args(q_norm_weight=FAKE))
    # the transformed query rows: num_tokens * num_heads * head_size 16-bit values
    assert with_norm - plain >= 4 * 4 * 64 * 2
