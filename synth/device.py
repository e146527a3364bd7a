"""Device-resident synthetic inputs for a workload config (generation only).

Builds, on the GPU, exactly the tensors the host side of ``synth.synth``
defines: per-token K/V/Kr (per-token memories) or pre-pooled K-bar/V-bar and
row-major routing keys (pre-pooled memories), the routing queries Qr, the
decode queries and the local K/V, with the needle rows planted.  Nothing here
computes any part of the method; callers hand these tensors to the library.
"""
from __future__ import annotations

import numpy as np
import torch

from . import synth as S


def _i64(a, device):
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.int64)).to(device)


class DeviceInputs:
    def __init__(self, cfg: S.Config, device="cuda"):
        self.cfg = cfg
        self.mem = S.memory_config(cfg)
        self.device = device
        self.gen = S.DeviceGen(device)

    # ------------------------------------------------------------- queries
    def qr(self) -> torch.Tensor:
        """[L][B][T][8][128] bf16 (T = longest round for re-routed configs)."""
        cfg = self.cfg
        T = max(cfg.T_rounds) if cfg.T_rounds else cfg.T
        q = torch.empty((cfg.n_layers, cfg.B, T, S.H, S.D), dtype=torch.bfloat16, device=self.device)
        self.gen.fill(q, cfg.seed, S.S_QR)
        if cfg.memory_of:
            mq = DeviceInputs(self.mem, self.device).qr()
            q[:, 0, : self.mem.T] = mq[:, 0]
        return q

    def mem_qr(self) -> torch.Tensor:
        return self.qr() if self.mem is self.cfg else DeviceInputs(self.mem, self.device).qr()

    # -------------------------------------------------------- per-token memory
    def per_token(self):
        """(doc_tok_off int64 CPU, K, V, Kr [L][N_tok][8][128] bf16) with needles planted in Kr."""
        mem = self.mem
        assert mem.per_token
        tok = S.doc_tok_offsets(mem)
        n_tok = int(tok[-1])
        L = mem.n_layers
        out = []
        for stream in (S.S_K, S.S_V, S.S_KR):
            t = torch.empty((L, n_tok, S.H, S.D), dtype=torch.bfloat16, device=self.device)
            self.gen.fill(t, mem.seed, stream)
            out.append(t)
        rows, qrows = S.needle_row_table(mem, tok)
        if rows.size:
            qr = self.mem_qr()
            r_d, q_d = _i64(rows, self.device), _i64(qrows, self.device)
            for l in range(L):
                self.gen.plant(out[2][l], 0, n_tok, l, r_d, q_d, qr[l], mem.seed)
        return torch.as_tensor(tok), out[0], out[1], out[2]

    # -------------------------------------------------------- pre-pooled memory
    def prepooled_offsets(self):
        return torch.as_tensor(S.prepooled_doc_blk_offsets(self.mem))

    def prepooled_content(self):
        """K-bar, V-bar [L][N_blk][8][128] bf16."""
        mem = self.mem
        out = []
        for stream in (S.S_KBAR, S.S_VBAR):
            t = torch.empty((mem.n_layers, mem.n_blk, S.H, S.D), dtype=torch.bfloat16, device=self.device)
            self.gen.fill(t, mem.seed, stream)
            out.append(t)
        return out[0], out[1]

    def prepooled_content_host(self):
        """The same K-bar, V-bar as prepooled_content, in pinned host memory: two lists of
        per-layer [N_blk][8][128] tensors (generated on the device one layer at a time)."""
        mem = self.mem
        per = mem.n_blk * S.H * S.D
        stage = torch.empty((mem.n_blk, S.H, S.D), dtype=torch.bfloat16, device=self.device)
        out = []
        for stream in (S.S_KBAR, S.S_VBAR):
            layers = []
            for l in range(mem.n_layers):
                h = torch.empty((1, mem.n_blk, S.H, S.D), dtype=torch.bfloat16, pin_memory=True)
                self.gen.fill(stage, mem.seed, stream, l * per)
                h[0].copy_(stage)
                layers.append(h)
            out.append(layers)
        return out[0], out[1]

    def prepooled_route_rows(self, staging: torch.Tensor = None):
        """Yields (layer, rows [N_blk][8][128] bf16) of the row-major routing keys, needles
        planted, one layer at a time in a reused staging buffer."""
        mem = self.mem
        off = S.prepooled_doc_blk_offsets(mem)
        rows, qrows = S.needle_row_table(mem, off)
        if staging is None:
            staging = torch.empty((mem.n_blk, S.H, S.D), dtype=torch.bfloat16, device=self.device)
        qr = self.mem_qr() if rows.size else None
        r_d, q_d = _i64(rows, self.device), _i64(qrows, self.device)
        for l in range(mem.n_layers):
            self.gen.fill(staging, mem.seed, S.S_KRBAR, l * mem.n_blk * S.ROW)
            if rows.size:
                self.gen.plant(staging, 0, mem.n_blk, l, r_d, q_d, qr[l], mem.seed)
            yield l, staging

    def prepooled_route_rows_layer_host(self, layer: int) -> np.ndarray:
        """Row-major routing keys of one layer, needles planted, as a host array
        [N_blk][8][128] uint16 (generated on the device, then copied)."""
        mem = self.mem
        off = S.prepooled_doc_blk_offsets(mem)
        rows, qrows = S.needle_row_table(mem, off)
        staging = torch.empty((mem.n_blk, S.H, S.D), dtype=torch.bfloat16, device=self.device)
        self.gen.fill(staging, mem.seed, S.S_KRBAR, layer * mem.n_blk * S.ROW)
        if rows.size:
            qr = self.mem_qr()
            self.gen.plant(staging, 0, mem.n_blk, layer, _i64(rows, self.device), _i64(qrows, self.device),
                           qr[layer], mem.seed)
            del qr
        out = staging.view(torch.int16).cpu().numpy().view(np.uint16)
        del staging
        return out

    # ------------------------------------------------------------------ decode
    def decode_inputs(self):
        """q [L][B][Hq][128], loc_k/loc_v [L][B][L_loc][8][128] bf16, loc_len [L][B] int32."""
        cfg = self.cfg
        q = torch.empty((cfg.n_layers, cfg.B, cfg.Hq, S.D), dtype=torch.bfloat16, device=self.device)
        self.gen.fill(q, cfg.seed, S.S_DEC_Q)
        lk = torch.empty((cfg.n_layers, cfg.B, cfg.L_loc, S.H, S.D), dtype=torch.bfloat16, device=self.device)
        lv = torch.empty_like(lk)
        self.gen.fill(lk, cfg.seed, S.S_LOC_K)
        self.gen.fill(lv, cfg.seed, S.S_LOC_V)
        ll = torch.full((cfg.n_layers, cfg.B), cfg.L_loc, dtype=torch.int32, device=self.device)
        return q, lk, lv, ll

    def prefill_inputs(self, max_doc_blocks: int = None):
        """Inputs of one multi-token prefill at the longest round: q [L][B][T][Hq][128];
        a memory context [L][B][k * max_doc_blocks][8][128] whose length is the block count of
        k documents drawn (seeded) from the memory's length mix; local rows = the query
        itself [L][B][T][8][128], loc_len = T."""
        cfg, mem = self.cfg, self.mem
        T = max(cfg.T_rounds) if cfg.T_rounds else cfg.T
        L, B = cfg.n_layers, cfg.B
        counts = np.diff(S.prepooled_doc_blk_offsets(mem)) if not mem.per_token else None
        if counts is None:
            raise ValueError("prefill inputs need a pre-pooled memory")
        mdb = int(counts.max()) if max_doc_blocks is None else max_doc_blocks
        rng = np.random.default_rng(cfg.seed + S.S_PF_DOCS)
        docs = rng.choice(counts.size, size=(L, B, cfg.k), replace=True)
        ctx_len = torch.as_tensor(counts[docs].sum(axis=-1).astype(np.int32)).to(self.device)
        max_ctx = cfg.k * mdb
        q = torch.empty((L, B, T, cfg.Hq, S.D), dtype=torch.bfloat16, device=self.device)
        self.gen.fill(q, cfg.seed, S.S_PF_Q)
        ck = torch.empty((L, B, max_ctx, S.H, S.D), dtype=torch.bfloat16, device=self.device)
        cv = torch.empty_like(ck)
        self.gen.fill(ck, cfg.seed, S.S_PF_CTX_K)
        self.gen.fill(cv, cfg.seed, S.S_PF_CTX_V)
        lk = torch.empty((L, B, T, S.H, S.D), dtype=torch.bfloat16, device=self.device)
        lv = torch.empty_like(lk)
        self.gen.fill(lk, cfg.seed, S.S_LOC_K)
        self.gen.fill(lv, cfg.seed, S.S_LOC_V)
        ll = torch.full((L, B), T, dtype=torch.int32, device=self.device)
        return q, ck, cv, ctx_len, lk, lv, ll

    # ------------------------------------------------------------- encode front-end
    def encode_inputs(self, hidden: int = S.ENC_HIDDEN, n_layers: int = None):
        """Inputs of the encode front-end over this config's documents: (doc_tok_off int64 CPU,
        x [L][n_tok][hidden], W_k, W_v, W_kr [L][1024][hidden] (output-major, as a linear layer
        stores them), w_norm [L][128]), all bf16."""
        mem = self.mem
        L = mem.n_layers if n_layers is None else n_layers
        tok = S.doc_tok_offsets(mem)
        n_tok = int(tok[-1])
        seed = mem.seed
        x = torch.empty((L, n_tok, hidden), dtype=torch.bfloat16, device=self.device)
        self.gen.fill(x, seed, S.S_ENC_X)
        ws = []
        for stream in (S.S_ENC_WK, S.S_ENC_WV, S.S_ENC_WKR):
            w = torch.empty((L, S.ROW, hidden), dtype=torch.bfloat16, device=self.device)
            self.gen.fill(w, seed, stream)
            w.mul_(S.enc_weight_scale(hidden))          # a power of two: exact in bf16
            ws.append(w)
        wn = torch.from_numpy(S.enc_norm_weight_host(seed, L).view(np.int16)).to(self.device).view(torch.bfloat16)
        return torch.as_tensor(tok), x, ws[0], ws[1], ws[2], wn

