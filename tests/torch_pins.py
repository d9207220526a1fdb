"""Library-routine pins for the oracle: ``torch.nn.LSTMCell`` / ``GRUCell``
in float64 on the CPU, fed the multi-head parameters embedded into one dense
cell of hidden size H = NH*Dh.

Embedding (torch stores gates as row blocks of size H, order i,f,g,o for the
LSTM and r,z,n for the GRU, which are our i,f,z,o and r,z,n):
  weight_ih[g*H + n*Dh + j, k]        = W[k, (n*G + g)*Dh + j]
  weight_hh[g*H + n*Dh + j, n*Dh + m] = R[n, m, g*Dh + j]   (0 off the diagonal blocks)
  bias_ih[g*H + n*Dh + j]             = b[(n*G + g)*Dh + j],  bias_hh = 0
"""
import numpy as np
import torch


def embed(W, R, b, NH, Dh, G):
    Din = W.shape[0]
    H = NH * Dh
    Wt = np.asarray(W, np.float64).reshape(Din, NH, G, Dh)
    w_ih = np.transpose(Wt, (2, 1, 3, 0)).reshape(G * H, Din)          # [g][n][j] x k
    Rr = np.asarray(R, np.float64).reshape(NH, Dh, G, Dh)               # n, m, g, j
    w_hh = np.zeros((G, H, H))
    for n in range(NH):
        # rows g*H + n*Dh + j, cols n*Dh + m
        w_hh[:, n * Dh:(n + 1) * Dh, n * Dh:(n + 1) * Dh] = np.transpose(Rr[n], (1, 2, 0))
    w_hh = w_hh.reshape(G * H, H)
    bb = np.transpose(np.asarray(b, np.float64).reshape(NH, G, Dh), (1, 0, 2)).reshape(G * H)
    return w_ih, w_hh, bb


def unembed_grads(gw_ih, gw_hh, gb, NH, Dh, G):
    """Back to our layouts: dW [Din][N], dR [NH][Dh][G*Dh] (diagonal blocks
    only), db [N]."""
    H = NH * Dh
    Din = gw_ih.shape[1]
    dW = np.transpose(gw_ih.reshape(G, NH, Dh, Din), (3, 1, 0, 2)).reshape(Din, NH * G * Dh)
    ghh = gw_hh.reshape(G, H, H)
    dR = np.zeros((NH, Dh, G * Dh))
    for n in range(NH):
        blk = ghh[:, n * Dh:(n + 1) * Dh, n * Dh:(n + 1) * Dh]        # g, j, m
        dR[n] = np.transpose(blk, (2, 0, 1)).reshape(Dh, G * Dh)
    db = np.transpose(gb.reshape(G, NH, Dh), (1, 0, 2)).reshape(NH * G * Dh)
    return dW, dR, db


def run_cell(cell, x, W, R, b, h0, c0, NH, Dh, dH=None, dhT=None, dcT=None):
    """Step a float64 torch cell through x.  Returns h_seq, c_seq (LSTM) and,
    when dH is given, the gradients of L = sum dH.h_t + dhT.h_T + dcT.c_T in
    our layouts."""
    G = 4 if cell == "lstm" else 3
    T, B, Din = x.shape
    H = NH * Dh
    w_ih, w_hh, bb = embed(W, R, b, NH, Dh, G)
    mod = (torch.nn.LSTMCell if cell == "lstm" else torch.nn.GRUCell)(Din, H).double()
    with torch.no_grad():
        mod.weight_ih.copy_(torch.from_numpy(w_ih))
        mod.weight_hh.copy_(torch.from_numpy(w_hh))
        mod.bias_ih.copy_(torch.from_numpy(bb))
        mod.bias_hh.zero_()
    xt = torch.tensor(np.asarray(x, np.float64), requires_grad=True)
    h = torch.tensor(np.zeros((B, H)) if h0 is None else np.asarray(h0, np.float64),
                     requires_grad=True)
    hs, cs = [], []
    if cell == "lstm":
        c = torch.tensor(np.zeros((B, H)) if c0 is None else np.asarray(c0, np.float64),
                         requires_grad=True)
        h_in, c_in = h, c
        for t in range(T):
            h, c = mod(xt[t], (h, c))
            hs.append(h)
            cs.append(c)
    else:
        h_in, c_in = h, None
        for t in range(T):
            h = mod(xt[t], h)
            hs.append(h)
    h_seq = torch.stack(hs)
    out = {"h_seq": h_seq.detach().numpy()}
    if cell == "lstm":
        out["c_seq"] = torch.stack(cs).detach().numpy()
    if dH is None:
        return out
    loss = (h_seq * torch.from_numpy(np.asarray(dH, np.float64))).sum()
    if dhT is not None:
        loss = loss + (hs[-1] * torch.from_numpy(np.asarray(dhT, np.float64))).sum()
    if dcT is not None and cell == "lstm":
        loss = loss + (cs[-1] * torch.from_numpy(np.asarray(dcT, np.float64))).sum()
    loss.backward()
    dW, dR, db = unembed_grads(mod.weight_ih.grad.numpy(), mod.weight_hh.grad.numpy(),
                               mod.bias_ih.grad.numpy(), NH, Dh, G)
    out.update(dx=xt.grad.numpy(), dW=dW, dR=dR, db=db, dh0=h_in.grad.numpy())
    if cell == "lstm":
        out["dc0"] = c_in.grad.numpy()
    return out
