"""Tensor-size lists of the model shapes the workloads are built on.

Only shapes: no weights or data. Each list is the flatten (registration)
order: embedding, per-layer tensors, final norm, then the LM head when it is
not tied to the embedding. A tied weight appears once ("从 Data Parallel 到
ZeRO/FSDP" section "Shared Parameters 与 Tied Weights 为什么麻烦": ownership of a
shared parameter must be unique, so it is flattened once).
"""


def qwen25_3b():
    """Qwen2.5-3B shape: hidden 2048, 36 layers, 16 query / 2 key-value heads of
    128, biases on q/k/v, gated MLP 11008, vocabulary 151936 with the LM head
    tied to the embedding. 434 tensors, 3,085,938,688 parameters."""
    H, L, I, V, KV = 2048, 36, 11008, 151936, 2 * 128
    sizes = [V * H]
    for _ in range(L):
        sizes += [H * H, H, KV * H, KV, KV * H, KV, H * H, I * H, I * H, H * I, H, H]
    sizes.append(H)
    return sizes


def llama_7b():
    """Llama-7B shape: hidden 4096, 32 layers, 32 heads, gated MLP 11008,
    vocabulary 32000 untied, RMSNorm weights. 291 tensors, 6,738,415,616."""
    H, L, I, V = 4096, 32, 11008, 32000
    sizes = [V * H]
    for _ in range(L):
        sizes += [H * H, H * H, H * H, H * H, I * H, I * H, H * I, H, H]
    sizes += [H, V * H]
    return sizes


def llama_70b():
    """Llama-70B shape: hidden 8192, 80 layers, 64 query / 8 key-value heads of
    128, gated MLP 28672, vocabulary 128256 untied. 723 tensors,
    70,553,706,496 parameters."""
    H, L, I, V, KV = 8192, 80, 28672, 128256, 8 * 128
    sizes = [V * H]
    for _ in range(L):
        sizes += [H * H, KV * H, KV * H, H * H, I * H, I * H, H * I, H, H]
    sizes += [H, V * H]
    return sizes


def tiny():
    """One flat parameter of 1,000,003 elements (odd, so the plan must pad)."""
    return [1_000_003]
