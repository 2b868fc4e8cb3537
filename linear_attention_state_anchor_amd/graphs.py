"""HIP graphs of the group replay, bucketed by total packed length
("SuffixReplay", System Design, Pipelined Replay Path: hits are packed into
one variable-length execution with device-side boundaries, and its graphs
are bucketed by the total packed length).

A graph fixes the host-side sizes of every launch (packed tokens, requests)
but not the device-side boundaries.  One graph per bucket of `tokens`
packed tokens and `max_requests` requests is captured once into buffers the
bucket owns; a batch with at most that many tokens and requests is copied
into those buffers with its cu_seqlens padded -- the tokens past its total
form one extra request, the requests after that are empty -- and the graph
replays the whole group (about two dozen kernel launches) as one.  Every
request is replayed independently of its neighbours, so the padding does
not touch the real requests' states, which are bit-identical to an eager
replay of the batch.
"""
from __future__ import annotations

import torch

from . import replay_group, group_workspace_bytes, SR_LAYER_GDN

__all__ = ["GroupReplayGraphs"]


class _Bucket:
    def __init__(self, tokens, max_requests, hidden, n_gdn, h_v, d, conv_dim, conv_width,
                 ws_bytes, device):
        n_pad = max_requests + 1                     # + the padding request
        self.tokens = tokens
        self.anchors = torch.zeros((tokens, hidden), dtype=torch.bfloat16, device=device)
        self.cu = torch.zeros((n_pad + 1,), dtype=torch.int32, device=device)
        self.cu[-1] = tokens
        self.states = torch.zeros((n_gdn, n_pad, h_v, d, d), dtype=torch.float32, device=device)
        self.conv = (torch.zeros((n_gdn, n_pad, conv_dim, conv_width - 1), dtype=torch.float32,
                                 device=device) if conv_dim else None)
        self.workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=device)
        self.graph = None


class GroupReplayGraphs:
    """Graph-replayed sr_replay_group for batches of up to `max_requests`
    requests, one captured graph per bucket size in `buckets` (packed
    tokens, increasing).  run() returns views of the bucket's state buffers,
    valid until the next run() that uses the same bucket."""

    def __init__(self, packed_weights, layer_kind, h_k, h_v, d, hidden, *,
                 buckets=(512, 1024, 2048, 4096, 8192), max_requests=64, conv_width=4,
                 want_conv_state=False, ffn_dim=0, device="cuda"):
        self.w = list(packed_weights)
        self.kinds = [int(x) for x in layer_kind]
        self.n_gdn = sum(1 for x in self.kinds if x == SR_LAYER_GDN)
        self.h_k, self.h_v, self.d, self.hidden = h_k, h_v, d, hidden
        self.conv_width = conv_width
        self.want_conv = want_conv_state
        self.ffn_dim = ffn_dim
        self.max_requests = max_requests
        self.sizes = sorted(int(b) for b in buckets)
        self.device = torch.device(device)
        self._b = {}

    def _bucket(self, tokens):
        for b in self.sizes:
            if tokens <= b:
                return b
        raise ValueError(f"{tokens} packed tokens exceed the largest bucket ({self.sizes[-1]})")

    def _replay(self, bk):
        replay_group(bk.anchors, self.w, bk.cu, self.kinds, self.h_k, self.h_v, self.d,
                     conv_width=self.conv_width, want_conv_state=self.want_conv,
                     states=bk.states, conv_states=bk.conv, workspace=bk.workspace,
                     ffn_dim=self.ffn_dim)

    def _capture(self, size):
        conv_dim = (2 * self.h_k + self.h_v) * self.d if self.want_conv else 0
        ws = group_workspace_bytes(size, self.hidden, self.h_k, self.h_v, self.d,
                                   self.conv_width, self.max_requests + 1, self.kinds,
                                   self.ffn_dim)
        bk = _Bucket(size, self.max_requests, self.hidden, self.n_gdn, self.h_v, self.d,
                     conv_dim, self.conv_width, ws, self.device)
        # one eager run on a side stream (loads the code objects, settles
        # the allocator), then the capture
        side = torch.cuda.Stream(device=self.device)
        side.wait_stream(torch.cuda.current_stream(self.device))
        with torch.cuda.stream(side):
            self._replay(bk)
        torch.cuda.current_stream(self.device).wait_stream(side)
        torch.cuda.synchronize(self.device)
        bk.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(bk.graph):
            self._replay(bk)
        torch.cuda.synchronize(self.device)
        return bk

    def bucket_for(self, total_tokens):
        """The bucket size a batch of total_tokens packed tokens runs in."""
        return self._bucket(int(total_tokens))

    def run(self, anchors, cu_seqlens):
        """Replay the group for the packed batch (anchors bf16 [T, hidden] and
        cu_seqlens int32 [N + 1] on the device).  Returns the states [n_gdn,
        N, h_v, d, d] (and conv windows if asked) as views of the bucket."""
        T, N = int(anchors.shape[0]), int(cu_seqlens.shape[0]) - 1
        if N > self.max_requests:
            raise ValueError(f"{N} requests exceed max_requests={self.max_requests}")
        if anchors.dtype != torch.bfloat16 or anchors.shape[1] != self.hidden:
            raise ValueError("anchors must be bf16 [T, hidden]")
        size = self._bucket(T)
        bk = self._b.get(size)
        if bk is None:
            bk = self._b[size] = self._capture(size)
        bk.anchors[:T].copy_(anchors)
        bk.cu[:N + 1].copy_(cu_seqlens)
        bk.cu[N + 1:].fill_(size)                     # padding request, then empty ones
        bk.graph.replay()
        states = bk.states[:, :N]
        if self.want_conv:
            return states, bk.conv[:, :N]
        return states
