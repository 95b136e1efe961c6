"""The linear layers of one DiT (FLUX.2-style double-stream) block as an
NVFP4-patched model runs them, with every buffer allocated up front so the
sequence can be captured in a HIP graph and replayed.

Which layer runs in NVFP4 is decided by the exclude-pattern predicate
("英伟达B200狂飙10.2倍！AI绘图告别龟速！", nmedialink.com, section
"NVFP4量化"): the modulation linear on the timestep embedding contains
"stream" in its name and stays bf16; the attention projections and the MLP
are NVFP4 with weights quantized once at construction (quantize_weights=True)
and activations quantized dynamically on every call.  The MLP's hidden
activation is quantized with the amax the up-projection epilogue produced, so
it is read once.  Attention itself is not part of this path: the output
projection takes its input from the caller.
"""

from . import (gemm, gemm_bf16, gemm_workspace, layer_is_quantized, quantize,
               quantize_workspace, quantize_weight)

#: layer name -> (input, weight, epilogue)
LAYERS = {
    "double_stream_modulation_img.linear": ("temb", "w_mod", "none"),
    "transformer_blocks.0.attn.to_qkv": ("x_qkv", "w_qkv", "none"),
    "transformer_blocks.0.attn.to_out.0": ("x_o", "w_o", "none"),
    "transformer_blocks.0.ff.net.0.proj": ("x_mlp", "w_up", "gelu"),
    "transformer_blocks.0.ff.net.2": ("h", "w_down", "none"),
}


def gemm_flops(shapes):
    """2*M*N*K per layer for {input name: (rows, cols)} and the weights."""
    return {name: 2 * shapes[x][0] * shapes[w][0] * shapes[x][1]
            for name, (x, w, _) in LAYERS.items()}


class DitBlockLinears:
    """``weights``: bf16 device tensors w_mod, w_qkv, w_o, w_up, w_down
    ([out, in]); ``tokens``: rows of the token activations; ``cond_rows``:
    rows of the timestep embedding."""

    def __init__(self, weights, tokens, cond_rows=2):
        import torch
        dev = weights["w_qkv"].device
        self.quantized = {name: layer_is_quantized(name) for name in LAYERS}
        self.weights = {}
        for name, (_, w, _) in LAYERS.items():
            self.weights[name] = quantize_weight(weights[w]) if self.quantized[name] else weights[w]
        rows = {"temb": cond_rows, "x_qkv": tokens, "x_o": tokens, "x_mlp": tokens, "h": tokens}
        self.out = {}
        self.qbuf = {}
        self.ws = {}
        for name, (x, w, _) in LAYERS.items():
            n, k = weights[w].shape
            self.out[name] = torch.empty((rows[x], n), dtype=torch.bfloat16, device=dev)
            if self.quantized[name]:
                self.qbuf[name] = (torch.empty((rows[x], k // 2), dtype=torch.uint8, device=dev),
                                   torch.empty((rows[x], k // 16), dtype=torch.uint8, device=dev),
                                   torch.empty((1,), dtype=torch.float32, device=dev))
                self.ws[name] = gemm_workspace(rows[x], n, k, device=dev)
        self.amax = torch.empty((1,), dtype=torch.float32, device=dev)
        self.quant_ws = quantize_workspace(dev)
        names = list(LAYERS)
        # the up projection's epilogue amax feeds the down projection's quantize
        self.chain = self.quantized[names[3]] and self.quantized[names[4]]

    def _linear(self, name, x, amax_in=None, amax_out=None):
        epilogue = LAYERS[name][2]
        if not self.quantized[name]:
            return gemm_bf16(x, self.weights[name], epilogue=epilogue, out=self.out[name])
        q = quantize(x, amax=amax_in, workspace=None if amax_in is not None else self.quant_ws,
                     out=self.qbuf[name])
        return gemm(q, self.weights[name], epilogue=epilogue, y_amax=amax_out,
                    out=self.out[name], workspace=self.ws[name])

    def __call__(self, temb, x_qkv, x_o, x_mlp):
        names = list(LAYERS)
        self._linear(names[0], temb)
        self._linear(names[1], x_qkv)
        self._linear(names[2], x_o)
        amax = self.amax if self.chain else None
        h = self._linear(names[3], x_mlp, amax_out=amax)
        self._linear(names[4], h, amax_in=amax)
        return self.out
