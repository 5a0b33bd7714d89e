"""CPU oracle for TurboQuant KV compression and compressed-cache attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) imports, links or calls this package; only the tests,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` do.
It shares no code, header, table or constant generator with the HIP path.

Everything here is plain NumPy in float64, written from the method's
description on these pages:

* [A] lilting.ch, "SwiftLMはTurboQuantとSSDストリーミングをMetalシェーダーに
  統合したSwift製LLM推論サーバー" -- sections "Lloyd-Maxコードブックとは",
  "KVキャッシュ圧縮の内訳", "Walsh-Hadamard Transform（WHT）の役割".
* [B] 0h-n0 blog, "論文解説: vLLM-MLX" -- section "Paged KVキャッシュ".
* [C] SwiftLM README (nomorevibe.com mirror) -- section "TurboQuantization:
  KV Cache Compression" (K-cache steps 1-5, V-cache paragraph) and the
  ``--prefill-size`` / ``--turbo-kv`` rows of its CLI table.

Where the pages leave a step open, the reading taken is stated in the
docstring of the function that takes it.  Parity pins live in
``tests/test_oracle_*.py``.  Every public function is pinned; none is
"parity unpinned".
"""

from .codebook import lloyd_max_gaussian, codebook_fp32
from .hadamard import sylvester_hadamard, fwht
from .qjl import splitmix64_stream, gaussian_matrix, qjl_alpha
from .encode import encode_k, encode_v, quantize_codes
from .pages import (K_PAGE_BYTES, V_PAGE_BYTES, BLOCK, pack_k_page, pack_v_page,
                    unpack_k_page, unpack_v_page, write_slots, read_k_tokens,
                    read_v_tokens)
from .attention import (dequant_k, dequant_v, attention_dense, decode_paged, decode_paged_hot,
                        ring_row, decode_paged_window)

__all__ = [
    "lloyd_max_gaussian", "codebook_fp32",
    "sylvester_hadamard", "fwht",
    "splitmix64_stream", "gaussian_matrix", "qjl_alpha",
    "encode_k", "encode_v", "quantize_codes",
    "K_PAGE_BYTES", "V_PAGE_BYTES", "BLOCK", "pack_k_page", "pack_v_page",
    "unpack_k_page", "unpack_v_page", "write_slots", "read_k_tokens",
    "read_v_tokens",
    "dequant_k", "dequant_v", "attention_dense", "decode_paged", "decode_paged_hot",
    "ring_row", "decode_paged_window",
]
