"""Model-shaped parameter lists (forward / registration order).

Each entry is (name, numel, param_dtype, grad_dtype).  Shapes follow the
public architectures the workloads are named after; no weights are involved.
"""
from __future__ import annotations

from typing import List, NamedTuple


class ParamSpec(NamedTuple):
    name: str
    numel: int
    param_dtype: str  # "f32" | "bf16" | "f16"
    grad_dtype: str
    requires_new_bucket: int = 0
    hgroup: int = 0


def tiny() -> List[ParamSpec]:
    # [64x32, 32, 32x16, 16] = 2608 elements
    return [ParamSpec("w0", 64 * 32, "bf16", "bf16"), ParamSpec("b0", 32, "bf16", "bf16"),
            ParamSpec("w1", 32 * 16, "bf16", "bf16"), ParamSpec("b1", 16, "bf16", "bf16")]


def gpt2_small(dt: str = "bf16", gdt: str = "bf16") -> List[ParamSpec]:
    h, v, ctx, L = 768, 50257, 1024, 12
    ps = [ParamSpec("wte", v * h, dt, gdt), ParamSpec("wpe", ctx * h, dt, gdt)]
    for i in range(L):
        p = f"h{i}."
        ps += [ParamSpec(p + "ln_1.w", h, dt, gdt), ParamSpec(p + "ln_1.b", h, dt, gdt),
               ParamSpec(p + "attn.c_attn.w", h * 3 * h, dt, gdt), ParamSpec(p + "attn.c_attn.b", 3 * h, dt, gdt),
               ParamSpec(p + "attn.c_proj.w", h * h, dt, gdt), ParamSpec(p + "attn.c_proj.b", h, dt, gdt),
               ParamSpec(p + "ln_2.w", h, dt, gdt), ParamSpec(p + "ln_2.b", h, dt, gdt),
               ParamSpec(p + "mlp.c_fc.w", h * 4 * h, dt, gdt), ParamSpec(p + "mlp.c_fc.b", 4 * h, dt, gdt),
               ParamSpec(p + "mlp.c_proj.w", 4 * h * h, dt, gdt), ParamSpec(p + "mlp.c_proj.b", h, dt, gdt)]
    ps += [ParamSpec("ln_f.w", h, dt, gdt), ParamSpec("ln_f.b", h, dt, gdt)]
    return ps


def _llama(L: int, h: int, nq: int, nkv: int, hd: int, ffn: int, vocab: int, mat_dt: str, mat_gdt: str,
           norm_dt: str, norm_gdt: str) -> List[ParamSpec]:
    # Forward order inside a layer: input norm, attention, post-attention
    # norm, MLP (the order the layer runs them, which is the order a
    # Megatron-style layer registers them; its buckets fill in reverse).
    ps = [ParamSpec("embed_tokens", vocab * h, mat_dt, mat_gdt)]
    for i in range(L):
        p = f"layers.{i}."
        ps += [ParamSpec(p + "input_layernorm", h, norm_dt, norm_gdt),
               ParamSpec(p + "q_proj", h * nq * hd, mat_dt, mat_gdt),
               ParamSpec(p + "k_proj", h * nkv * hd, mat_dt, mat_gdt),
               ParamSpec(p + "v_proj", h * nkv * hd, mat_dt, mat_gdt),
               ParamSpec(p + "o_proj", nq * hd * h, mat_dt, mat_gdt),
               ParamSpec(p + "post_attention_layernorm", h, norm_dt, norm_gdt),
               ParamSpec(p + "gate_proj", h * ffn, mat_dt, mat_gdt),
               ParamSpec(p + "up_proj", h * ffn, mat_dt, mat_gdt),
               ParamSpec(p + "down_proj", ffn * h, mat_dt, mat_gdt)]
    ps += [ParamSpec("norm", h, norm_dt, norm_gdt), ParamSpec("lm_head", vocab * h, mat_dt, mat_gdt)]
    return ps


def llama3_8b() -> List[ParamSpec]:
    # bf16 matrices with fp32 main grads; RMSNorm vectors kept fp32 (fp32 grads).
    return _llama(32, 4096, 32, 8, 128, 14336, 128256, "bf16", "f32", "f32", "f32")


def dense_7b() -> List[ParamSpec]:
    # 32 layers, hidden 4096, MHA 32 heads x 128, ffn 11008, vocab 32000; all fp16.
    return _llama(32, 4096, 32, 32, 128, 11008, 32000, "f16", "f16", "f16", "f16")


def llama3_70b() -> List[ParamSpec]:
    return _llama(80, 8192, 64, 8, 128, 28672, 128256, "bf16", "bf16", "bf16", "bf16")


PARAM_LISTS = {
    "tiny": tiny,
    "gpt2-small": gpt2_small,
    "llama3-8b": llama3_8b,
    "dense-7b": dense_7b,
    "llama3-70b": llama3_70b,
}
