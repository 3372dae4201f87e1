"""Device-memory plumbing around the C ABI: allocates the caller-owned buffers
with PyTorch, writes initial parameters, and forwards each step call to the
binding.  No arithmetic of the step happens here.
"""

from __future__ import annotations

import numpy as np
import torch

from . import binding as B

PARAM_NAMES = (
    "wte", "wpe", "ln1w", "ln1b", "qkvw", "qkvb", "attprojw", "attprojb",
    "ln2w", "ln2b", "fcw", "fcb", "fcprojw", "fcprojb", "lnfw", "lnfb",
)


class Config:
    """The six GPT2Config fields (train_gpt2.cu)."""

    def __init__(self, max_seq_len, vocab_size, padded_vocab_size, num_layers, num_heads, channels):
        self.max_seq_len, self.vocab_size, self.padded_vocab_size = max_seq_len, vocab_size, padded_vocab_size
        self.num_layers, self.num_heads, self.channels = num_layers, num_heads, channels


class GPT2:
    """One context over torch-allocated device buffers on the current device."""

    @classmethod
    def from_checkpoint(cls, path: str, precision: int, batch: int, seq_len: int, device="cuda"):
        """A model whose initial parameters come from a model file (read on the
        host by gpt2_checkpoint_read, then copied to the device by init)."""
        fields, _ = B.gpt2_checkpoint_header(path)
        cfg = Config(**fields)
        model = cls(cfg, precision, batch, seq_len, device)
        flat = np.empty(model.num_params, np.float32)
        B.gpt2_checkpoint_read(path, flat)
        return model.init(flat)

    def __init__(self, cfg, precision: int, batch: int, seq_len: int, device="cuda"):
        self.cfg, self.precision, self.B, self.T = cfg, precision, batch, seq_len
        self.device = torch.device(device)
        self.sizes = B.gpt2_query_sizes(cfg, precision, batch, seq_len)
        self.offsets, self.counts, self.num_params = B.gpt2_param_layout(cfg)
        self.bufs = {}
        for name, nbytes in self.sizes.items():
            if nbytes:
                self.bufs[name] = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.ctx = None

    @property
    def stream(self) -> int:
        return torch.cuda.current_stream(self.device).cuda_stream

    def _ptrs(self):
        return {k: v.data_ptr() for k, v in self.bufs.items()}

    def _flat(self, name, dtype, n):
        return self.bufs[name][: n * torch.tensor([], dtype=dtype).element_size()].view(dtype)

    def params(self):
        dt = torch.float32 if self.precision == B.GPT2_FP32 else torch.bfloat16
        return self._flat("params", dt, self.num_params)

    def master(self):
        return self._flat("master", torch.float32, self.num_params)

    def grads(self):
        return self._flat("grads", torch.float32, self.num_params)

    def adam_m(self):
        return self._flat("adam_m", torch.float32, self.num_params)

    def adam_v(self):
        return self._flat("adam_v", torch.float32, self.num_params)

    def pack(self, tensors: dict) -> np.ndarray:
        """Flat float32 vector in the library's parameter layout."""
        flat = np.zeros(self.num_params, np.float32)
        for i, name in enumerate(PARAM_NAMES):
            a = np.asarray(tensors[name], dtype=np.float32).reshape(-1)
            if a.size != self.counts[i]:
                raise ValueError(f"{name}: {a.size} elements, layout wants {self.counts[i]}")
            flat[self.offsets[i]: self.offsets[i] + self.counts[i]] = a
        return flat

    def unpack(self, flat) -> dict:
        flat = np.asarray(flat)
        return {name: flat[self.offsets[i]: self.offsets[i] + self.counts[i]]
                for i, name in enumerate(PARAM_NAMES)}

    def init(self, flat_params_f32: np.ndarray):
        """Writes the initial fp32 parameters and creates the context (which
        zeroes the AdamW state and, in bf16 mode, casts master -> params).
        Without master weights (GPT2_BF16_SR) the values are written to params
        as bf16 (exact for bf16-exact values)."""
        src = torch.from_numpy(np.ascontiguousarray(flat_params_f32, dtype=np.float32)).to(self.device)
        if self.precision == B.GPT2_BF16:
            self.master().copy_(src)
        elif self.precision == B.GPT2_BF16_SR:
            self.params().copy_(src.to(torch.bfloat16))
        else:
            self.params().copy_(src)
        self.ctx = B.gpt2_init(self.cfg, self.precision, self.B, self.T, self._ptrs(), self.stream)
        return self

    def forward(self, inputs: torch.Tensor, targets=None, losses=None, mean_loss=None):
        B.gpt2_forward(self.ctx, inputs.data_ptr(), 0 if targets is None else targets.data_ptr(),
                       0 if losses is None else losses.data_ptr(), 0 if mean_loss is None else mean_loss.data_ptr(),
                       self.stream)

    def sample(self, coins: torch.Tensor, tokens: torch.Tensor, t: int):
        B.gpt2_sample(self.ctx, coins.data_ptr(), tokens.data_ptr(), t, self.stream)

    def generate(self, tokens: torch.Tensor, coins: torch.Tensor, t_begin: int, t_end: int):
        B.gpt2_generate(self.ctx, tokens.data_ptr(), coins.data_ptr(), t_begin, t_end, self.stream)

    def zero_grad(self):
        B.gpt2_zero_grad(self.ctx, self.stream)

    def backward(self, dloss: float = 0.0):
        B.gpt2_backward(self.ctx, dloss, self.stream)

    def update(self, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, t=1):
        B.gpt2_adamw_update(self.ctx, lr, beta1, beta2, eps, weight_decay, t, self.stream)

    def check(self) -> int:
        return B.gpt2_check_device_error(self.ctx, self.stream)

    def act(self, which: int, dtype=None) -> torch.Tensor:
        """A torch view of an internal activation tensor (no copy)."""
        ptr, n = B.gpt2_act_tensor(self.ctx, which)
        if dtype is None:
            if which == B.GPT2_T_DRESIDUAL:
                dtype = torch.float32
            else:  # bf16 activations in both bf16 modes (with and without master weights)
                dtype = torch.float32 if self.precision == B.GPT2_FP32 else torch.bfloat16
        base = self.bufs["acts"]
        ofs = ptr - base.data_ptr()
        es = torch.tensor([], dtype=dtype).element_size()
        return base[ofs: ofs + n * es].view(dtype)

    def close(self):
        if self.ctx is not None:
            B.gpt2_free(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
