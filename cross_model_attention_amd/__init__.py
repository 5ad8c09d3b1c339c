"""MapFlow cross-model attention-map reuse on MI355X: block-sparse compression of a sender
layer's causal softmax attention and the fused retrieval into a receiver layer.

The compute lives in ``lib/libmapflow.so`` (HIP kernels for gfx950, C ABI in
``include/mapflow.h``); ``mapflow`` is its Python binding.
"""
from .mapflow import (  # noqa: F401
    BlockStore,
    Context,
    PreparedV,
    PrefixCache,
    check_layer_map,
    compress,
    compress_into,
    compress_prefill_into,
    copy_probe,
    fill_probe,
    read_probe,
    write_probe,
    dense_attention,
    layer_map_uniform,
    map_layers,
    prefill_layers,
    prefill_timings,
    probs_canonical_to_store,
    prefix_hashes,
    probs_store_to_canonical,
    retrieve,
    retrieve_layers,
    retrieve_multi,
    retrieve_noalloc,
    retrieve_prepared,
    v_prepare,
    version,
)
from ._lib import MapflowError  # noqa: F401
