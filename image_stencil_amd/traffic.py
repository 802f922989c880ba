"""Work and traffic counts of a convolution (host arithmetic, no device code).

Counted work follows the conventions used to report throughput:
  * flops = 2*N*K*C*R*S*H*W: one multiply and one add per filter tap for every
    output, border taps included;
  * algorithmic bytes = x + y + w + b, each moved once.
The naive traffic model is the one of "Optimizing convolution kernels - CNNs in
Vulkan Part 2/3" (section "Reducing memory traffic"): a per-pixel kernel re-reads
the whole input image once per output channel. The per-thread register and
shared-memory counts are those of "Optimizing Memory Efficiency for Convolution
Kernels on Kepler GPUs" (sections on the special-case access schedule and the
general case).
"""
MIB = float(1 << 20)


def conv_flops(n, c, h, w, k, r, s):
    return 2.0 * n * k * c * r * s * h * w


def conv_bytes(n, c, h, w, k, r, s, elem_bytes=4, bias=True, out_elem_bytes=None):
    ob = elem_bytes if out_elem_bytes is None else out_elem_bytes
    return (elem_bytes * (n * c * h * w + k * c * r * s) + ob * n * k * h * w
            + (4 * k if bias else 0))


def chain_flops(n, h, w, layers):
    """layers: (c, k, r) per layer."""
    return sum(conv_flops(n, c, h, w, k, r, r) for (c, k, r) in layers)


def chain_bytes_fused(n, h, w, layers, elem_bytes=4, bias=True):
    """Input and final output once, plus every layer's weights and bias."""
    c0, kl = layers[0][0], layers[-1][1]
    wb = sum(elem_bytes * k * c * r * r + (4 * k if bias else 0) for (c, k, r) in layers)
    return elem_bytes * n * h * w * (c0 + kl) + wb


def naive_input_reads(h, w, c_in_packed, k_out_packed, elem_bytes=4):
    """(input image bytes, total input bytes read) of the per-pixel kernel."""
    size = float(h) * w * c_in_packed * elem_bytes
    return size, size * k_out_packed


def special_case_registers(k, n):
    """Pixels one thread keeps for n contiguous outputs of a KxK filter."""
    return k * (k + n - 1)


def shared_reads(w_t, k, c, contiguous_in_thread=True):
    """Shared-memory pixel reads for W_T outputs of a KxK filter over C channels:
    (W_T+K-1)*K*C when one thread owns the W_T contiguous outputs, else W_T*K*K*C."""
    return (w_t + k - 1) * k * c if contiguous_in_thread else w_t * k * k * c
